"""Host-side checks of the C ABI: no GPU, no kernel launches.

Every call below either is a pure size query or fails a host-side argument
check before anything is launched, so it runs without a device.
"""
import ctypes
import os
import re

import pytest

from sparse_latent_attention_amd import _lib

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                   "mla_sparse.h")

FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10008)


def declared_functions():
    text = open(HDR).read()
    return re.findall(r"MLA_API\s+[\w\s\*]+?\b(mla_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_expected_entry_points():
    names = set(declared_functions())
    assert {"mla_sparse_decode", "mla_sparse_prefill_chunk", "mla_sparse_decode_workspace_size",
            "mla_sparse_prefill_chunk_workspace_size", "mla_validate_indices",
            "mla_status_string", "mla_set_attention_events", "mla_abi_version"} <= names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_status_strings(lib):
    assert lib.mla_status_string(0) == b"MLA_OK"
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.mla_status_string(code).decode().startswith(name)
    assert lib.mla_status_string(99) == b"MLA_ERR_UNKNOWN"
    assert lib.mla_abi_version() == 3


def ws_expected(rows, esize, n_split):
    """Absorbed queries, per-split mixes (bf16 or f32), per-split max and sum, diagnostics."""
    def up(x):
        return (x + 255) // 256 * 256
    q = rows * 128 * 576 * esize
    o = n_split * rows * 128 * 512 * esize
    ml = 2 * n_split * rows * 128 * 4
    return up(up(up(q) + o) + ml) + 256          # + the call's diagnostics


def test_cache_length_limit(lib):
    hdr = open(HDR).read()
    max_t = int(re.search(r"#define MLA_MAX_T (\d+)", hdr).group(1))
    # an empty slot's offset (2^31) must lie past the latent rows plus a 3 KiB prefix
    assert max_t * 1024 + 3072 <= 2 ** 31
    assert lib.mla_sparse_decode_workspace_size(1, max_t, 64, 1) > 0
    assert lib.mla_sparse_decode_workspace_size(1, max_t + 1, 64, 1) == 0
    assert lib.mla_sparse_prefill_chunk_workspace_size(4, max_t + 1, 64, 1) == 0


def test_workspace_size_plan(lib):
    # 64 rows: 4 splits of 512 slots fill the 256 compute units
    assert lib.mla_sparse_decode_workspace_size(64, 32768, 2048, 1) == ws_expected(64, 2, 4)
    # 32 rows: 8 splits of 256 slots
    assert lib.mla_sparse_decode_workspace_size(32, 8192, 2048, 1) == ws_expected(32, 2, 8)
    # one row, 1001 slots: splits capped by the 32-slot tile count
    assert lib.mla_sparse_decode_workspace_size(1, 1001, 1001, 1) == ws_expected(1, 2, 32)
    assert lib.mla_sparse_decode_workspace_size(1, 64, 64, 0) == ws_expected(1, 4, 2)
    # 4096 queries: as few splits as possible; splits never exceed 2048 slots
    assert lib.mla_sparse_prefill_chunk_workspace_size(4096, 4096, 1024, 1) == ws_expected(4096, 2, 1)
    assert lib.mla_sparse_prefill_chunk_workspace_size(4096, 4096, 2048, 1) == ws_expected(4096, 2, 1)
    assert lib.mla_sparse_prefill_chunk_workspace_size(4096, 8192, 4096, 1) == ws_expected(4096, 2, 2)
    assert lib.mla_sparse_prefill_chunk_workspace_size(4096, 8192, 4097, 1) == ws_expected(4096, 2, 3)
    # invalid arguments report zero
    assert lib.mla_sparse_decode_workspace_size(0, 10, 5, 1) == 0
    assert lib.mla_sparse_decode_workspace_size(1, 10, 11, 1) == 0
    assert lib.mla_sparse_decode_workspace_size(1, 10, 5, 7) == 0
    assert lib.mla_sparse_prefill_chunk_workspace_size(1, 10, 0, 1) == 0


def call_decode(lib, **kw):
    args = dict(q_nope=FAKE, q_pe=FAKE, kv=FAKE, pe=FAKE, idx=FAKE, w_uk=FAKE, w_uv=FAKE, out=FAKE,
                B=2, T=100, ld_T=100, k=10, scale=0.07, dtype=1, ws=FAKE, ws_bytes=0, stream=None)
    args.update(kw)
    return lib.mla_sparse_decode(args["q_nope"], args["q_pe"], args["kv"], args["pe"], args["idx"],
                                 args["w_uk"], args["w_uv"], args["out"], args["B"], args["T"],
                                 args["ld_T"], args["k"], args["scale"], args["dtype"], args["ws"],
                                 args["ws_bytes"], args["stream"])


def call_prefill(lib, **kw):
    args = dict(q_nope=FAKE, q_pe=FAKE, kv=FAKE, pe=FAKE, idx=FAKE, w_uk=FAKE, w_uv=FAKE, out=FAKE,
                S=4, T=100, k=10, start=0, scale=0.07, dtype=1, ws=FAKE, ws_bytes=0, stream=None)
    args.update(kw)
    return lib.mla_sparse_prefill_chunk(args["q_nope"], args["q_pe"], args["kv"], args["pe"],
                                        args["idx"], args["w_uk"], args["w_uv"], args["out"],
                                        args["S"], args["T"], args["k"], args["start"],
                                        args["scale"], args["dtype"], args["ws"],
                                        args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("field", ["q_nope", "q_pe", "kv", "pe", "idx", "w_uk", "w_uv", "out"])
def test_null_pointers_rejected(lib, field):
    assert call_decode(lib, **{field: None}) == 1
    assert call_prefill(lib, **{field: None}) == 1


@pytest.mark.parametrize("kw", [dict(B=0), dict(T=0), dict(k=0), dict(k=101), dict(ld_T=99),
                                dict(scale=float("nan")), dict(scale=float("inf"))])
def test_decode_shape_errors(lib, kw):
    assert call_decode(lib, **kw) == 2


@pytest.mark.parametrize("kw", [dict(S=0), dict(T=0), dict(k=0), dict(start=-1),
                                dict(start=97, S=4), dict(scale=float("nan"))])
def test_prefill_shape_errors(lib, kw):
    assert call_prefill(lib, **kw) == 2


def test_dtype_and_alignment_errors(lib):
    assert call_decode(lib, dtype=2) == 4
    assert call_prefill(lib, dtype=-1) == 4
    for field in ["q_nope", "kv", "idx", "w_uv", "out"]:
        assert call_decode(lib, **{field: MISALIGNED}) == 3
        assert call_prefill(lib, **{field: MISALIGNED}) == 3


def test_workspace_errors(lib):
    need = lib.mla_sparse_decode_workspace_size(2, 100, 10, 1)
    assert call_decode(lib, ws_bytes=need - 1) == 5
    assert call_decode(lib, ws=None, ws_bytes=need) == 5
    assert call_decode(lib, ws=ctypes.c_void_p(0x10010), ws_bytes=need) == 5   # not 256-aligned
    need_p = lib.mla_sparse_prefill_chunk_workspace_size(4, 100, 10, 1)
    assert call_prefill(lib, ws_bytes=need_p - 1) == 5


def test_validator_and_event_hook_argument_checks(lib):
    assert lib.mla_validate_indices(None, 1, 1, 1, 0, FAKE, None) == 1
    assert lib.mla_validate_indices(FAKE, 0, 1, 1, 0, FAKE, None) == 2
    assert lib.mla_validate_indices(MISALIGNED, 1, 1, 1, 0, FAKE, None) == 3
    assert lib.mla_set_attention_events(FAKE, None) == 1
    assert lib.mla_set_attention_events(None, None) == 0
    assert lib.mla_read_diagnostics(None, 1, 1, 1, FAKE, None) == 1
    assert lib.mla_read_diagnostics(FAKE, 1, 1, 1, None, None) == 1
    assert lib.mla_read_diagnostics(FAKE, 1, 1, 5, FAKE, None) == 4
    assert lib.mla_read_diagnostics(FAKE, 0, 1, 1, FAKE, None) == 2
    assert lib.mla_read_diagnostics(FAKE, 1, 1, 1, ctypes.c_void_p(0x10002), None) == 3


def call_noalloc(lib, **kw):
    args = dict(q_nope=FAKE, q_pe=FAKE, kv=FAKE, pe=FAKE, idx=FAKE, w_uk=FAKE, w_uv=FAKE, out=FAKE,
                B=2, T=100, ld_T=100, k=10, scale=0.07, dtype=1, stream=None)
    args.update(kw)
    return lib.mla_sparse_decode_noalloc(args["q_nope"], args["q_pe"], args["kv"], args["pe"],
                                         args["idx"], args["w_uk"], args["w_uv"], args["out"],
                                         args["B"], args["T"], args["ld_T"], args["k"],
                                         args["scale"], args["dtype"], args["stream"])


def test_noalloc_checks_come_before_any_device_call(lib):
    hdr = open(HDR).read()
    cap = eval(re.search(r"#define MLA_NOALLOC_SCRATCH_BYTES \(([^)]*)\)", hdr).group(1))
    from sparse_latent_attention_amd import NOALLOC_SCRATCH_BYTES
    assert cap == NOALLOC_SCRATCH_BYTES == 48 * 2 ** 20
    for field in ["q_nope", "kv", "idx", "w_uv", "out"]:
        assert call_noalloc(lib, **{field: None}) == 1
        assert call_noalloc(lib, **{field: MISALIGNED}) == 3
    assert call_noalloc(lib, B=0) == 2
    assert call_noalloc(lib, k=101) == 2
    assert call_noalloc(lib, dtype=3) == 4
    # the headline decode fits the fixed scratch; calls whose workspace does not are refused
    assert lib.mla_sparse_decode_workspace_size(64, 32768, 2048, 1) <= cap
    assert lib.mla_sparse_decode_workspace_size(128, 32768, 2048, 1) > cap
    assert call_noalloc(lib, B=128, T=32768, ld_T=32768, k=2048) == 5
    assert call_noalloc(lib, B=64, T=32768, ld_T=32768, k=2048, dtype=0) == 5


def test_cache_append_argument_checks(lib):
    def call(**kw):
        args = dict(a=FAKE, w=FAKE, cs=FAKE, kv=FAKE, pe=FAKE, B=2, S=3, start=5, ld_T=10, eps=1e-6,
                    dtype=1, stream=None)
        args.update(kw)
        return lib.mla_cache_append(args["a"], args["w"], args["cs"], args["kv"], args["pe"], args["B"],
                                    args["S"], args["start"], args["ld_T"], args["eps"], args["dtype"],
                                    args["stream"])
    for field in ["a", "w", "cs", "kv", "pe"]:
        assert call(**{field: None}) == 1
        assert call(**{field: MISALIGNED}) == 3
    for kw in [dict(B=0), dict(S=0), dict(start=-1), dict(start=8), dict(eps=-1.0),
               dict(eps=float("nan"))]:
        assert call(**kw) == 2, kw
    assert call(dtype=2) == 4


def test_output_projection_argument_checks(lib):
    def call(o=FAKE, w=FAKE, out=FAKE, B=2, dtype=1, ws=FAKE, ws_bytes=1 << 20):
        return lib.mla_output_projection(o, w, out, B, dtype, ws, ws_bytes, None)
    assert call(o=None) == 1 and call(out=None) == 1
    assert call(w=MISALIGNED) == 3
    assert call(B=0) == 2
    assert call(dtype=9) == 4
    need = lib.mla_output_projection_workspace_size(2, 1)
    assert need == 8 * 2 * 7168 * 4                       # eight float32 partial sums per output
    assert call(ws_bytes=need - 1) == 5 and call(ws=None) == 5
    assert call(ws=ctypes.c_void_p(0x10010)) == 5          # not 256-aligned
    assert lib.mla_output_projection_workspace_size(2, 0) == 0     # float32 needs none
    assert lib.mla_output_projection_workspace_size(0, 1) == 0
    hdr = open(HDR).read()
    assert int(re.search(r"#define MLA_D_MODEL (\d+)", hdr).group(1)) == 7168


def test_binding_refuses_to_run_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load(str(tmp_path / "absent.so"))


def call_explicit(lib, **kw):
    args = dict(q_nope=FAKE, q_pe=FAKE, kv=FAKE, pe=FAKE, idx=FAKE, w_uk=FAKE, w_uv=FAKE, out=FAKE,
                S=4, T=100, k=10, start=0, scale=0.07, dtype=1, ws=FAKE, ws_bytes=0, stream=None)
    args.update(kw)
    return lib.mla_sparse_prefill_explicit(args["q_nope"], args["q_pe"], args["kv"], args["pe"],
                                           args["idx"], args["w_uk"], args["w_uv"], args["out"],
                                           args["S"], args["T"], args["k"], args["start"],
                                           args["scale"], args["dtype"], args["ws"],
                                           args["ws_bytes"], args["stream"])


def test_explicit_prefill_workspace_plan(lib):
    """Up-projected keys and values of the visible positions, then one bitmap word per 32."""
    def up(x):
        return (x + 255) // 256 * 256

    def expected(S, T, start):
        tv = min(start + S, T)
        return up(tv * 128 * 256 * 2) + up(S * ((tv + 31) // 32) * 4)

    size = lib.mla_sparse_prefill_explicit_workspace_size
    assert size(4096, 4096, 2048, 0, 1) == expected(4096, 4096, 0)
    assert size(3, 100, 10, 50, 1) == expected(3, 100, 50)
    assert size(1, 1, 1, 0, 1) == expected(1, 1, 0)
    for bad in [(4, 100, 10, 0, 0), (0, 100, 10, 0, 1), (4, 100, 0, 0, 1), (4, 100, 10, -1, 1),
                (4, 100, 10, 97, 1), (4, 0, 10, 0, 1)]:
        assert size(*bad) == 0, bad


def test_explicit_prefill_argument_checks(lib):
    for field in ["q_nope", "q_pe", "kv", "pe", "idx", "w_uk", "w_uv", "out"]:
        assert call_explicit(lib, **{field: None}) == 1
        assert call_explicit(lib, **{field: MISALIGNED}) == 3
    assert call_explicit(lib, dtype=0) == 4           # float32 has no explicit form here
    for kw in [dict(S=0), dict(T=0), dict(k=0), dict(start=-1), dict(start=97),
               dict(scale=float("nan"))]:
        assert call_explicit(lib, **kw) == 2, kw
    need = lib.mla_sparse_prefill_explicit_workspace_size(4, 100, 10, 0, 1)
    assert call_explicit(lib, ws_bytes=need - 1) == 5
    assert call_explicit(lib, ws=None, ws_bytes=need) == 5
    assert call_explicit(lib, ws=ctypes.c_void_p(0x10010), ws_bytes=need) == 5


def test_wkv_b_dequant_argument_checks(lib):
    assert lib.mla_wkv_b_dequant(None, FAKE, FAKE, FAKE, None) == 1
    assert lib.mla_wkv_b_dequant(FAKE, FAKE, None, FAKE, None) == 1
    assert lib.mla_wkv_b_dequant(MISALIGNED, FAKE, FAKE, FAKE, None) == 3
    assert lib.mla_wkv_b_dequant(FAKE, ctypes.c_void_p(0x10002), FAKE, FAKE, None) == 3
    assert lib.mla_wkv_b_dequant(FAKE, FAKE, FAKE, MISALIGNED, None) == 3
