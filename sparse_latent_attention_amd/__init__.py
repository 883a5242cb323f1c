"""MI355X sparse latent attention (DeepSeek-V3.2-Exp, absorbed form).

Thin Python binding over libmla_sparse.so: every step of the computation runs
in the library's HIP kernels; this module only checks tensor shapes, converts
index lists to int32 and passes device pointers and the current HIP stream.
PyTorch serves as the device-memory and stream provider.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import MLA_BF16, MLA_F32, MLAError  # noqa: F401

N_HEADS, D_LATENT, D_ROPE, D_NOPE, D_V = 128, 512, 64, 128, 128
D_MODEL = 7168
SOFTMAX_SCALE = (D_NOPE + D_ROPE) ** -0.5
NOALLOC_SCRATCH_BYTES = 48 * 1024 * 1024   # MLA_NOALLOC_SCRATCH_BYTES in include/mla_sparse.h

__all__ = ["decode", "decode_noalloc", "prefill_chunk", "prefill_explicit", "prefill_explicit_workspace_size", "wkv_b_dequant", "output_projection_workspace_size", "cache_append", "output_projection", "decode_workspace_size", "prefill_chunk_workspace_size",
           "validate_indices", "diagnostics", "set_attention_events", "status_string",
           "abi_version",
           "MLAError", "SOFTMAX_SCALE"]


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return MLA_BF16
    if dt == torch.float32:
        return MLA_F32
    raise TypeError(f"unsupported dtype {dt}; use torch.bfloat16 or torch.float32")


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class _on_stream:
    """Run a call's preparation and launches on `stream` (default: the current stream).

    With an explicit stream, that stream first waits for the work queued so far on the
    current one (which produced the inputs), and the index conversion, the workspace and
    a library-allocated output are made while it is current, so the caching allocator
    ties them to the stream whose kernels use them.
    """

    def __init__(self, stream):
        self.stream = stream
        self.ctx = None

    def __enter__(self):
        if self.stream is not None:
            self.stream.wait_stream(torch.cuda.current_stream())
            self.ctx = torch.cuda.stream(self.stream)
            self.ctx.__enter__()
        return self

    def __exit__(self, *exc):
        if self.ctx is not None:
            self.ctx.__exit__(*exc)
        return False


def _require(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _index32(idx: torch.Tensor) -> torch.Tensor:
    if idx.dtype == torch.int32:
        return idx.contiguous()
    if idx.dtype == torch.int64:
        return idx.to(torch.int32).contiguous()
    raise TypeError(f"topk_idx has dtype {idx.dtype}, expected int32 or int64")


def status_string(status: int) -> str:
    return _lib.load().mla_status_string(status).decode()


def abi_version() -> int:
    return _lib.load().mla_abi_version()


def decode_workspace_size(B: int, T: int, k: int, dtype: torch.dtype) -> int:
    return _lib.load().mla_sparse_decode_workspace_size(B, T, k, _dtype_code(dtype))


def prefill_chunk_workspace_size(S: int, T: int, k: int, dtype: torch.dtype) -> int:
    return _lib.load().mla_sparse_prefill_chunk_workspace_size(S, T, k, _dtype_code(dtype))


def _workspace(nbytes: int, device, workspace):
    if workspace is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"needs {nbytes}")
    return workspace


def decode(q_nope, q_pe, kv_cache, pe_cache, topk_idx, w_uk, w_uv, *, T=None,
           softmax_scale=SOFTMAX_SCALE, out=None, workspace=None, stream=None):
    """Sparse latent attention decode; returns out [B, 128, 128].

    q_nope [B,128,128], q_pe [B,128,64], kv_cache [B,ld_T,512], pe_cache
    [B,ld_T,64], topk_idx [B,k] (int32/int64, <0 = empty slot), w_uk/w_uv
    [128,128,512].  T (default ld_T) is the number of valid cached positions.
    """
    with _on_stream(stream):
        lib = _lib.load()
        dt, dev = q_nope.dtype, q_nope.device
        B = q_nope.shape[0]
        ld_T = kv_cache.shape[1]
        T = ld_T if T is None else int(T)
        idx = _index32(topk_idx)
        k = idx.shape[1]
        _require(q_nope, "q_nope", (B, N_HEADS, D_NOPE), dt, dev)
        _require(q_pe, "q_pe", (B, N_HEADS, D_ROPE), dt, dev)
        _require(kv_cache, "kv_cache", (B, ld_T, D_LATENT), dt, dev)
        _require(pe_cache, "pe_cache", (B, ld_T, D_ROPE), dt, dev)
        _require(idx, "topk_idx", (B, k), torch.int32, dev)
        _require(w_uk, "w_uk", (N_HEADS, D_NOPE, D_LATENT), dt, dev)
        _require(w_uv, "w_uv", (N_HEADS, D_V, D_LATENT), dt, dev)
        if out is None:
            out = torch.empty((B, N_HEADS, D_V), dtype=dt, device=dev)
        _require(out, "out", (B, N_HEADS, D_V), dt, dev)
        code = _dtype_code(dt)
        need = lib.mla_sparse_decode_workspace_size(B, T, k, code)
        if need == 0:
            raise MLAError(2, "mla_sparse_decode_workspace_size")
        ws = _workspace(need, dev, workspace)
        st = lib.mla_sparse_decode(_ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(pe_cache),
                                   _ptr(idx), _ptr(w_uk), _ptr(w_uv), _ptr(out), B, T, ld_T, k,
                                   float(softmax_scale), code, _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream))
        _lib.check(st, "mla_sparse_decode")
        return out


def decode_noalloc(q_nope, q_pe, kv_cache, pe_cache, topk_idx, w_uk, w_uv, *, out, T=None,
                   softmax_scale=SOFTMAX_SCALE, stream=None):
    """Decode into the caller's ``out`` through the library's allocation-free entry point.

    The library takes the workspace from a fixed device array of its own
    (MLA_NOALLOC_SCRATCH_BYTES); calls that overlap on one device race.  The
    binding itself only allocates when it has to convert int64 indices.
    """
    with _on_stream(stream):
        lib = _lib.load()
        dt, dev = q_nope.dtype, q_nope.device
        B = q_nope.shape[0]
        ld_T = kv_cache.shape[1]
        T = ld_T if T is None else int(T)
        idx = _index32(topk_idx)
        k = idx.shape[1]
        _require(q_nope, "q_nope", (B, N_HEADS, D_NOPE), dt, dev)
        _require(q_pe, "q_pe", (B, N_HEADS, D_ROPE), dt, dev)
        _require(kv_cache, "kv_cache", (B, ld_T, D_LATENT), dt, dev)
        _require(pe_cache, "pe_cache", (B, ld_T, D_ROPE), dt, dev)
        _require(idx, "topk_idx", (B, k), torch.int32, dev)
        _require(w_uk, "w_uk", (N_HEADS, D_NOPE, D_LATENT), dt, dev)
        _require(w_uv, "w_uv", (N_HEADS, D_V, D_LATENT), dt, dev)
        _require(out, "out", (B, N_HEADS, D_V), dt, dev)
        st = lib.mla_sparse_decode_noalloc(_ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(pe_cache),
                                           _ptr(idx), _ptr(w_uk), _ptr(w_uv), _ptr(out), B, T, ld_T,
                                           k, float(softmax_scale), _dtype_code(dt), _stream(stream))
        _lib.check(st, "mla_sparse_decode_noalloc")
        return out


def prefill_chunk(q_nope, q_pe, kv_cache, pe_cache, topk_idx, w_uk, w_uv, *, start_pos=0,
                  softmax_scale=SOFTMAX_SCALE, out=None, workspace=None, stream=None):
    """Latent-form prefill of S queries of one sequence; returns out [S, 128, 128].

    kv_cache [T,512], pe_cache [T,64]; query s is at position start_pos + s and
    ignores listed positions beyond it; topk_idx [S,k] is -1 padded.
    """
    with _on_stream(stream):
        lib = _lib.load()
        dt, dev = q_nope.dtype, q_nope.device
        S = q_nope.shape[0]
        T = kv_cache.shape[0]
        idx = _index32(topk_idx)
        k = idx.shape[1]
        _require(q_nope, "q_nope", (S, N_HEADS, D_NOPE), dt, dev)
        _require(q_pe, "q_pe", (S, N_HEADS, D_ROPE), dt, dev)
        _require(kv_cache, "kv_cache", (T, D_LATENT), dt, dev)
        _require(pe_cache, "pe_cache", (T, D_ROPE), dt, dev)
        _require(idx, "topk_idx", (S, k), torch.int32, dev)
        _require(w_uk, "w_uk", (N_HEADS, D_NOPE, D_LATENT), dt, dev)
        _require(w_uv, "w_uv", (N_HEADS, D_V, D_LATENT), dt, dev)
        if out is None:
            out = torch.empty((S, N_HEADS, D_V), dtype=dt, device=dev)
        _require(out, "out", (S, N_HEADS, D_V), dt, dev)
        code = _dtype_code(dt)
        need = lib.mla_sparse_prefill_chunk_workspace_size(S, T, k, code)
        if need == 0:
            raise MLAError(2, "mla_sparse_prefill_chunk_workspace_size")
        ws = _workspace(need, dev, workspace)
        st = lib.mla_sparse_prefill_chunk(_ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(pe_cache),
                                          _ptr(idx), _ptr(w_uk), _ptr(w_uv), _ptr(out), S, T, k,
                                          int(start_pos), float(softmax_scale), code, _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream))
        _lib.check(st, "mla_sparse_prefill_chunk")
        return out


def output_projection_workspace_size(B: int, dtype=torch.bfloat16) -> int:
    return _lib.load().mla_output_projection_workspace_size(int(B), _dtype_code(dtype))


def output_projection(o, w_o, *, out=None, workspace=None, stream=None):
    """Delta = o W_O: o [B, 128, 128] (per-head outputs), w_o [7168, 16384]; returns out [B, 7168]."""
    with _on_stream(stream):
        lib = _lib.load()
        dt, dev = o.dtype, o.device
        B = o.shape[0]
        _require(o, "o", (B, N_HEADS, D_V), dt, dev)
        _require(w_o, "w_o", (D_MODEL, N_HEADS * D_V), dt, dev)
        if out is None:
            out = torch.empty((B, D_MODEL), dtype=dt, device=dev)
        _require(out, "out", (B, D_MODEL), dt, dev)
        code = _dtype_code(dt)
        need = lib.mla_output_projection_workspace_size(B, code)
        ws = _workspace(need, dev, workspace) if need else None
        st = lib.mla_output_projection(_ptr(o), _ptr(w_o), _ptr(out), B, code,
                                       _ptr(ws) if ws is not None else None,
                                       ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
        _lib.check(st, "mla_output_projection")
        return out


def cache_append(kv_a_out, norm_weight, cos_sin, kv_cache, pe_cache, *, start_pos, eps=1e-6,
                 stream=None):
    """Write S new positions of B sequences into the caches, in place.

    kv_a_out [B, S, 576] (latent then rotary key), norm_weight [512], cos_sin
    [S, 32, 2] float32, kv_cache [B, ld_T, 512], pe_cache [B, ld_T, 64]; rows
    start_pos .. start_pos+S-1 receive the RMS-normalised latent and the rotated
    rotary key.  Returns (kv_cache, pe_cache).
    """
    with _on_stream(stream):
        lib = _lib.load()
        dt, dev = kv_a_out.dtype, kv_a_out.device
        B, S = kv_a_out.shape[0], kv_a_out.shape[1]
        ld_T = kv_cache.shape[1]
        _require(kv_a_out, "kv_a_out", (B, S, D_LATENT + D_ROPE), dt, dev)
        _require(norm_weight, "norm_weight", (D_LATENT,), dt, dev)
        _require(cos_sin, "cos_sin", (S, D_ROPE // 2, 2), torch.float32, dev)
        _require(kv_cache, "kv_cache", (B, ld_T, D_LATENT), dt, dev)
        _require(pe_cache, "pe_cache", (B, ld_T, D_ROPE), dt, dev)
        st = lib.mla_cache_append(_ptr(kv_a_out), _ptr(norm_weight), _ptr(cos_sin), _ptr(kv_cache),
                                  _ptr(pe_cache), B, S, int(start_pos), ld_T, float(eps),
                                  _dtype_code(dt), _stream(stream))
        _lib.check(st, "mla_cache_append")
        return kv_cache, pe_cache


def prefill_explicit_workspace_size(S: int, T: int, k: int, start_pos: int, dtype=torch.bfloat16) -> int:
    return _lib.load().mla_sparse_prefill_explicit_workspace_size(S, T, k, start_pos, _dtype_code(dtype))


def prefill_explicit(q_nope, q_pe, kv_cache, pe_cache, topk_idx, w_uk, w_uv, *, start_pos=0,
                     softmax_scale=SOFTMAX_SCALE, out=None, workspace=None, stream=None):
    """Explicit-form prefill of S queries (bf16): same arguments and result as prefill_chunk."""
    with _on_stream(stream):
        lib = _lib.load()
        dt, dev = q_nope.dtype, q_nope.device
        S = q_nope.shape[0]
        T = kv_cache.shape[0]
        idx = _index32(topk_idx)
        k = idx.shape[1]
        _require(q_nope, "q_nope", (S, N_HEADS, D_NOPE), dt, dev)
        _require(q_pe, "q_pe", (S, N_HEADS, D_ROPE), dt, dev)
        _require(kv_cache, "kv_cache", (T, D_LATENT), dt, dev)
        _require(pe_cache, "pe_cache", (T, D_ROPE), dt, dev)
        _require(idx, "topk_idx", (S, k), torch.int32, dev)
        _require(w_uk, "w_uk", (N_HEADS, D_NOPE, D_LATENT), dt, dev)
        _require(w_uv, "w_uv", (N_HEADS, D_V, D_LATENT), dt, dev)
        if out is None:
            out = torch.empty((S, N_HEADS, D_V), dtype=dt, device=dev)
        _require(out, "out", (S, N_HEADS, D_V), dt, dev)
        code = _dtype_code(dt)
        need = lib.mla_sparse_prefill_explicit_workspace_size(S, T, k, int(start_pos), code)
        if need == 0:
            raise MLAError(2 if code == MLA_BF16 else 4, "mla_sparse_prefill_explicit_workspace_size")
        ws = _workspace(need, dev, workspace)
        st = lib.mla_sparse_prefill_explicit(_ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(pe_cache),
                                             _ptr(idx), _ptr(w_uk), _ptr(w_uv), _ptr(out), S, T, k,
                                             int(start_pos), float(softmax_scale), code, _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(stream))
        _lib.check(st, "mla_sparse_prefill_explicit")
        return out


def wkv_b_dequant(codes, scales, *, w_uk=None, w_uv=None, stream=None):
    """FP8 wkv_b [32768, 512] (uint8 E4M3 codes) with one float32 scale per 128 x 128 block
    ([256, 4]) to bf16 W_UK and W_UV [128, 128, 512].  Returns (w_uk, w_uv)."""
    with _on_stream(stream):
        lib = _lib.load()
        dev = codes.device
        _require(codes, "codes", (N_HEADS * (D_NOPE + D_V), D_LATENT), torch.uint8, dev)
        _require(scales, "scales", (N_HEADS * (D_NOPE + D_V) // 128, D_LATENT // 128), torch.float32, dev)
        if w_uk is None:
            w_uk = torch.empty((N_HEADS, D_NOPE, D_LATENT), dtype=torch.bfloat16, device=dev)
        if w_uv is None:
            w_uv = torch.empty((N_HEADS, D_V, D_LATENT), dtype=torch.bfloat16, device=dev)
        _require(w_uk, "w_uk", (N_HEADS, D_NOPE, D_LATENT), torch.bfloat16, dev)
        _require(w_uv, "w_uv", (N_HEADS, D_V, D_LATENT), torch.bfloat16, dev)
        st = lib.mla_wkv_b_dequant(_ptr(codes), _ptr(scales), _ptr(w_uk), _ptr(w_uv), _stream(stream))
        _lib.check(st, "mla_wkv_b_dequant")
        return w_uk, w_uv


def validate_indices(topk_idx, T: int, allow_pad: bool = False, stream=None) -> int:
    """Run the library's index check; returns 0 (valid) or a bitmask (1 range, 2 repeat)."""
    with _on_stream(stream):
        lib = _lib.load()
        idx = _index32(topk_idx)
        flag = torch.empty(1, dtype=torch.int32, device=idx.device)
        st = lib.mla_validate_indices(_ptr(idx), idx.shape[0], idx.shape[1], int(T),
                                      1 if allow_pad else 0, _ptr(flag), _stream(stream))
        _lib.check(st, "mla_validate_indices")
        return int(flag.item())


def diagnostics(workspace, rows: int, k: int, dtype: torch.dtype, stream=None) -> dict:
    """Diagnostics of the last call that used ``workspace``: index-list splits it ran twice
    (softmax reference beaten); the second word is reserved and always 0."""
    with _on_stream(stream):
        lib = _lib.load()
        buf = torch.empty(2, dtype=torch.int32, device=workspace.device)
        st = lib.mla_read_diagnostics(_ptr(workspace), int(rows), int(k), _dtype_code(dtype),
                                      _ptr(buf), _stream(stream))
        _lib.check(st, "mla_read_diagnostics")
        v = buf.cpu().tolist()
        return {"reruns": int(v[0]), "reserved": int(v[1])}


def set_attention_events(begin, end) -> None:
    """Ask the next call to record two torch.cuda.Events around its attention kernel."""
    lib = _lib.load()
    b = ctypes.c_void_p(begin.cuda_event) if begin is not None else None
    e = ctypes.c_void_p(end.cuda_event) if end is not None else None
    _lib.check(lib.mla_set_attention_events(b, e), "mla_set_attention_events")
