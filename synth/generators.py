"""Seeded synthetic inputs shaped like DeepSeek-V3.2-Exp's sparse latent attention.

Shapes come from the model pages (Key heads, Parameters: 128 heads, 512-wide
latent, 64-wide rotary key; Mix and project, in/out: one query against 1001
cached positions at p = 1000).  Distributions follow the stated recipe:

* queries ``q_nope`` [128, 128] and ``q_pe`` [128, 64]: N(0, 1);
* latent cache rows [T, 512]: N(0, 1), then each row divided by its root mean
  square (unit gain, no epsilon), standing in for the model's latent RMSNorm;
* rotary cache rows [T, 64]: N(0, 1) (they arrive already rotated);
* ``W_UK`` and ``W_UV`` [128 heads, 128, 512]: N(0, variance 1/512);
* decode indices: k-1 positions drawn uniformly without replacement from
  [0, T-1) plus the newest position T-1, sorted; when k >= T every position;
* prefill indices: query at absolute position p gets all of [0, p] when
  p + 1 <= k, else k-1 positions drawn from [0, p) plus p itself, sorted and
  padded with -1 to width k.

Every draw uses numpy's PCG64 ``default_rng`` keyed by a tuple that names the
config, batch row and tensor, so any batch row (or query row) can be regenerated
alone.  Values are drawn in float32; bf16 configs round them to bf16 with
round-to-nearest-even and hold them as uint16 bit patterns.  Nothing here
computes any part of the attention.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

DEFAULT_SEED = 20251203

N_HEADS = 128
D_LATENT = 512
D_ROPE = 64
D_NOPE = 128
D_V = 128

# Stream tags inside an rng key.
_TAG_CACHE = 0
_TAG_QUERY = 1
_TAG_INDEX = 2
_TAG_WEIGHTS = 1 << 20


@dataclass(frozen=True)
class DecodeConfig:
    cid: int
    name: str
    B: int
    T: int
    k: int
    dtype: str  # "f32" or "bf16"

    @property
    def positions(self) -> int:
        """Selected KV positions processed by one call (B * k)."""
        return self.B * self.k


@dataclass(frozen=True)
class PrefillConfig:
    cid: int
    name: str
    S: int
    T: int
    k: int
    start_pos: int
    dtype: str

    def valid_count(self, s: int) -> int:
        return min(self.start_pos + s + 1, self.k)


CONFIGS = {
    "tiny_dense_f32": DecodeConfig(0, "tiny_dense_f32", B=1, T=64, k=64, dtype="f32"),
    "page_dense_bf16": DecodeConfig(1, "page_dense_bf16", B=1, T=1001, k=1001, dtype="bf16"),
    "sparse_b32_t8k": DecodeConfig(2, "sparse_b32_t8k", B=32, T=8192, k=2048, dtype="bf16"),
    "sparse_b64_t32k": DecodeConfig(3, "sparse_b64_t32k", B=64, T=32768, k=2048, dtype="bf16"),
    "prefill_s4096": PrefillConfig(4, "prefill_s4096", S=4096, T=4096, k=2048, start_pos=0,
                                   dtype="bf16"),
}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16) with round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    rounded = ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)
    return rounded


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def _rms_rows(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.mean(np.square(x, dtype=np.float32), axis=-1, keepdims=True))


def weights(cfg, seed: int = DEFAULT_SEED):
    """W_UK, W_UV, each [128, 128, 512] in [head, d, c] order, N(0, var 1/512)."""
    rng = np.random.default_rng([seed, cfg.cid, _TAG_WEIGHTS])
    std = np.float32(1.0 / np.sqrt(512.0))
    w_uk = rng.standard_normal((N_HEADS, D_NOPE, D_LATENT), dtype=np.float32) * std
    w_uv = rng.standard_normal((N_HEADS, D_V, D_LATENT), dtype=np.float32) * std
    return _store(w_uk, cfg.dtype), _store(w_uv, cfg.dtype)


def _cache_rows(cid: int, b: int, T: int, dtype: str, seed: int):
    rng = np.random.default_rng([seed, cid, b, _TAG_CACHE])
    latent = _rms_rows(rng.standard_normal((T, D_LATENT), dtype=np.float32))
    rope = rng.standard_normal((T, D_ROPE), dtype=np.float32)
    return _store(latent, dtype), _store(rope, dtype)


def decode_batch_row(cfg: DecodeConfig, b: int, seed: int = DEFAULT_SEED):
    """Cached latent [T, 512] and rotary key [T, 64] of batch row b."""
    return _cache_rows(cfg.cid, b, cfg.T, cfg.dtype, seed)


def _decode_indices(rng, T: int, k: int) -> np.ndarray:
    if k >= T:
        return np.arange(T, dtype=np.int32)
    drawn = rng.choice(T - 1, size=k - 1, replace=False)
    return np.sort(np.append(drawn, T - 1)).astype(np.int32)


def decode_query_set(cfg: DecodeConfig, b: int, set_id: int = 0, seed: int = DEFAULT_SEED):
    """q_nope [128,128], q_pe [128,64] and topk indices [k] of batch row b in query set set_id."""
    rng = np.random.default_rng([seed, cfg.cid, b, _TAG_QUERY, set_id])
    q_nope = rng.standard_normal((N_HEADS, D_NOPE), dtype=np.float32)
    q_pe = rng.standard_normal((N_HEADS, D_ROPE), dtype=np.float32)
    irng = np.random.default_rng([seed, cfg.cid, b, _TAG_INDEX, set_id])
    idx = _decode_indices(irng, cfg.T, cfg.k)
    return _store(q_nope, cfg.dtype), _store(q_pe, cfg.dtype), idx


def _workers(n: int) -> int:
    return max(1, min(n, int(os.environ.get("SYNTH_WORKERS", "8"))))


def decode_inputs(cfg: DecodeConfig, seed: int = DEFAULT_SEED, set_id: int = 0,
                  with_cache: bool = True):
    """All tensors of a decode config, stacked over batch rows.

    Returns a dict with q_nope [B,128,128], q_pe [B,128,64], kv_cache [B,T,512],
    pe_cache [B,T,64], topk_idx [B,k] int32, w_uk, w_uv [128,128,512].
    """
    B, T = cfg.B, cfg.T
    store_dt = np.float32 if cfg.dtype == "f32" else np.uint16
    out = {}
    qs = [decode_query_set(cfg, b, set_id, seed) for b in range(B)]
    out["q_nope"] = np.stack([q[0] for q in qs])
    out["q_pe"] = np.stack([q[1] for q in qs])
    out["topk_idx"] = np.stack([q[2] for q in qs]).astype(np.int32)
    if with_cache:
        kv = np.empty((B, T, D_LATENT), dtype=store_dt)
        pe = np.empty((B, T, D_ROPE), dtype=store_dt)

        def fill(b):
            kv[b], pe[b] = decode_batch_row(cfg, b, seed)

        with ThreadPoolExecutor(_workers(B)) as ex:
            list(ex.map(fill, range(B)))
        out["kv_cache"] = kv
        out["pe_cache"] = pe
    out["w_uk"], out["w_uv"] = weights(cfg, seed)
    return out


def _prefill_indices(rng, p: int, k: int) -> np.ndarray:
    row = np.full(k, -1, dtype=np.int32)
    if p + 1 <= k:
        row[: p + 1] = np.arange(p + 1, dtype=np.int32)
    else:
        drawn = rng.choice(p, size=k - 1, replace=False)
        row[:] = np.sort(np.append(drawn, p)).astype(np.int32)
    return row


def prefill_query_rows(cfg: PrefillConfig, rows, seed: int = DEFAULT_SEED):
    """q_nope [n,128,128], q_pe [n,128,64], topk [n,k] of the listed query rows."""
    qn, qp, ix = [], [], []
    for s in rows:
        rng = np.random.default_rng([seed, cfg.cid, int(s), _TAG_QUERY])
        qn.append(rng.standard_normal((N_HEADS, D_NOPE), dtype=np.float32))
        qp.append(rng.standard_normal((N_HEADS, D_ROPE), dtype=np.float32))
        irng = np.random.default_rng([seed, cfg.cid, int(s), _TAG_INDEX])
        ix.append(_prefill_indices(irng, cfg.start_pos + int(s), cfg.k))
    return (_store(np.stack(qn), cfg.dtype), _store(np.stack(qp), cfg.dtype),
            np.stack(ix).astype(np.int32))


def prefill_inputs(cfg: PrefillConfig, seed: int = DEFAULT_SEED):
    """All tensors of a prefill chunk: one sequence (B = 1), S query rows, T cached rows."""
    kv, pe = _cache_rows(cfg.cid, 0, cfg.T, cfg.dtype, seed)
    q_nope, q_pe, idx = prefill_query_rows(cfg, range(cfg.S), seed)
    w_uk, w_uv = weights(cfg, seed)
    return {"q_nope": q_nope, "q_pe": q_pe, "kv_cache": kv, "pe_cache": pe,
            "topk_idx": idx, "w_uk": w_uk, "w_uv": w_uv}


@dataclass(frozen=True)
class AppendConfig:
    cid: int
    name: str
    B: int
    S: int
    T: int
    start_pos: int
    dtype: str


def rotary_angles(positions, dim: int = D_ROPE, base: float = 10000.0) -> np.ndarray:
    """Rotary table [len(positions), dim/2, 2] float32: (cos, sin) of t * base^(-2i/dim).

    The base frequencies follow the model's table ("Rotated shared key" page,
    the precomputation's first line); the page leaves out the long-context
    interpolation and the base value, so this input uses base 10000 and no
    interpolation.  The library takes the table as given.
    """
    freqs = 1.0 / (base ** (np.arange(0, dim, 2, dtype=np.float64) / dim))
    theta = np.outer(np.asarray(positions, dtype=np.float64), freqs)
    return np.stack([np.cos(theta), np.sin(theta)], axis=-1).astype(np.float32)


def append_inputs(cfg: AppendConfig, seed: int = DEFAULT_SEED):
    """Inputs of a cache append: down-projection output [B, S, 576] (N(0, 1)), latent gains [512]
    (N(1, 0.1^2)), the rotary table of positions start_pos .. start_pos+S-1, and existing caches
    [B, T, 512] and [B, T, 64] (N(0, 1)) whose other rows must survive."""
    rng = np.random.default_rng([seed, cfg.cid, _TAG_CACHE, 7])
    a = rng.standard_normal((cfg.B, cfg.S, D_LATENT + D_ROPE), dtype=np.float32)
    w = (1.0 + 0.1 * rng.standard_normal(D_LATENT)).astype(np.float32)
    kv = rng.standard_normal((cfg.B, cfg.T, D_LATENT), dtype=np.float32)
    pe = rng.standard_normal((cfg.B, cfg.T, D_ROPE), dtype=np.float32)
    return {"kv_a_out": _store(a, cfg.dtype), "norm_weight": _store(w, cfg.dtype),
            "cos_sin": rotary_angles(np.arange(cfg.start_pos, cfg.start_pos + cfg.S)),
            "kv_cache": _store(kv, cfg.dtype), "pe_cache": _store(pe, cfg.dtype)}


D_MODEL = 7168


def projection_inputs(B: int, dtype: str, cid: int = 70, seed: int = DEFAULT_SEED):
    """Per-head outputs o [B, 128, 128] (N(0, 1)) and an output weight w_o [7168, 16384]
    (N(0, variance 1/16384), so that outputs have unit variance)."""
    rng = np.random.default_rng([seed, cid, _TAG_WEIGHTS, 2])
    o = rng.standard_normal((B, N_HEADS, D_V), dtype=np.float32)
    w = rng.standard_normal((D_MODEL, N_HEADS * D_V), dtype=np.float32) * np.float32(1.0 / 128.0)
    return {"o": _store(o, dtype), "w_o": _store(w, dtype)}


def fp8_wkv_b_inputs(cid: int = 90, seed: int = DEFAULT_SEED, rows: int = N_HEADS * (D_NOPE + D_V)):
    """An FP8 wkv_b as the model stores it: codes [rows, 512] (uint8, uniform over the 254 codes
    that are not NaN) and one float32 scale per 128 x 128 block, log-uniform in [2^-14, 2^-4]."""
    rng = np.random.default_rng([seed, cid, _TAG_WEIGHTS, 3])
    codes = rng.integers(0, 254, size=(rows, D_LATENT), dtype=np.int64)
    codes = codes + (codes >= 0x7F)                      # skip 0x7F; 0xFF is past the range
    scales = np.exp2(rng.uniform(-14.0, -4.0, size=(-(-rows // 128), D_LATENT // 128)))
    return {"codes": codes.astype(np.uint8), "scales": scales.astype(np.float32)}
