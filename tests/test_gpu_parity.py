"""GPU parity: the HIP library against the fp64 CPU oracle.

Tolerance (per tensor): max|gpu - oracle| / max|oracle| <= 1e-5 for float32
inputs and <= 2e-2 for bf16 inputs.  Decode configurations are compared on
every batch row, the headline one in the launch configuration the benchmark
times; the 4096-query prefill chunk on a strided sample that reaches every
workgroup slot, both sides of the 2048-position list limit and the last 64
queries.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
from synth.generators import DecodeConfig, PrefillConfig  # noqa: E402

from .gpu_util import TOL, log, rel_err, to_dev, to_host64  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_latent_attention_amd as m
    m._lib.load()
    return m


def upload(inp):
    return {k: to_dev(v) for k, v in inp.items()}


def run_decode(mla, dev, **kw):
    out = mla.decode(dev["q_nope"], dev["q_pe"], dev["kv_cache"], dev["pe_cache"], dev["topk_idx"],
                     dev["w_uk"], dev["w_uv"], **kw)
    torch.cuda.synchronize()
    return out


def run_prefill(mla, dev, start_pos, **kw):
    out = mla.prefill_chunk(dev["q_nope"], dev["q_pe"], dev["kv_cache"], dev["pe_cache"],
                            dev["topk_idx"], dev["w_uk"], dev["w_uv"], start_pos=start_pos, **kw)
    torch.cuda.synchronize()
    return out


def check_decode(mla, cfg, rows=None, inp=None, dev=None):
    inp = synth.decode_inputs(cfg) if inp is None else inp
    dev = upload(inp) if dev is None else dev
    assert np.array_equal(dev["topk_idx"].cpu().numpy(), inp["topk_idx"])   # indices bit-exact
    log(f"decode {cfg.name}: B={cfg.B} T={cfg.T} k={cfg.k} {cfg.dtype}")
    out = to_host64(run_decode(mla, dev))
    rows = list(range(cfg.B)) if rows is None else rows
    ref = oracle.decode(inp, rows=rows)
    err = rel_err(out[rows], ref)
    log(f"  rows {rows[:8]}{'...' if len(rows) > 8 else ''}: rel err {err:.3e} (tol {TOL[cfg.dtype]})")
    assert np.all(np.isfinite(out))
    assert err <= TOL[cfg.dtype]
    return out, inp, dev


# ------------------------------------------------------------------ configs
def test_config0_tiny_dense_f32(mla):
    check_decode(mla, synth.CONFIGS["tiny_dense_f32"])


def test_config1_page_shape_dense(mla):
    check_decode(mla, synth.CONFIGS["page_dense_bf16"])


def test_config2_sparse_b32_all_rows(mla):
    check_decode(mla, synth.CONFIGS["sparse_b32_t8k"])


def test_config3_headline_all_rows(mla):
    out, inp, dev = check_decode(mla, synth.CONFIGS["sparse_b64_t32k"])
    # unit-variance logits never beat a split's first-tile reference by ~60 (log2)
    assert rerun_count(mla, dev, inp) == 0


def _prefill_rows(S):
    """Every 16th query, offset so that the sample meets every residue mod 8 (the attention
    kernel deals query rows to workgroups, and workgroups to XCDs, by those residues), plus
    both sides of the query whose list first fills all 2048 slots, and the last 64 queries."""
    strided = [16 * i + (i % 8) for i in range(S // 16)]
    return sorted(set(strided) | set(range(2040, 2056)) | set(range(S - 64, S)))


def _oracle_prefill_parallel(inp, rows, start_pos, workers=8):
    from concurrent.futures import ThreadPoolExecutor
    chunks = [rows[i::workers] for i in range(workers)]
    with ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(lambda rr: oracle.prefill(inp, rows=rr, start_pos=start_pos), chunks))
    ref = np.empty((len(rows), 128, 128))
    pos = {r: i for i, r in enumerate(rows)}
    for rr, part in zip(chunks, parts):
        for r, o in zip(rr, part):
            ref[pos[r]] = o
    return ref


def test_config4_prefill_sampled(mla):
    cfg = synth.CONFIGS["prefill_s4096"]
    inp = synth.prefill_inputs(cfg)
    dev = upload(inp)
    assert np.array_equal(dev["topk_idx"].cpu().numpy(), inp["topk_idx"])
    log(f"prefill {cfg.name}: S={cfg.S} T={cfg.T} k={cfg.k}")
    out = to_host64(run_prefill(mla, dev, cfg.start_pos))
    assert np.all(np.isfinite(out))
    rows = _prefill_rows(cfg.S)
    assert len(rows) >= 256 and {r % 8 for r in rows} == set(range(8))
    ref = _oracle_prefill_parallel(inp, rows, cfg.start_pos)
    err = rel_err(out[rows], ref)
    log(f"  {len(rows)} queries: rel err {err:.3e}")
    assert err <= TOL["bf16"]


# ------------------------------------------------------------------ ragged and small
def test_ragged_bf16_all_rows(mla):
    check_decode(mla, DecodeConfig(10, "ragged", B=3, T=777, k=333, dtype="bf16"))


def test_sparse_f32_all_rows(mla):
    check_decode(mla, DecodeConfig(11, "f32sparse", B=2, T=300, k=100, dtype="f32"))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_small_all_rows(mla, dtype):
    cfg = PrefillConfig(12, "prefill_small", S=70, T=300, k=48, start_pos=200, dtype=dtype)
    inp = synth.prefill_inputs(cfg)
    dev = upload(inp)
    out = to_host64(run_prefill(mla, dev, cfg.start_pos))
    ref = oracle.prefill(inp, start_pos=cfg.start_pos)
    err = rel_err(out, ref)
    log(f"prefill small {dtype}: rel err {err:.3e}")
    assert err <= TOL[dtype]


def test_prefill_from_position_zero_all_rows(mla):
    cfg = PrefillConfig(13, "prefill_zero", S=150, T=150, k=100, start_pos=0, dtype="bf16")
    inp = synth.prefill_inputs(cfg)
    out = to_host64(run_prefill(mla, upload(inp), 0))
    err = rel_err(out, oracle.prefill(inp, start_pos=0))
    log(f"prefill from 0: rel err {err:.3e}")
    assert err <= TOL["bf16"]


def test_many_rows_take_row_major_queries(mla):
    """513 query rows: at 512 rows and more the absorbed queries are stored row-major
    (whole-line writes) instead of in the operand image; a strided sample of rows that
    covers every workgroup slot pattern, plus the last rows."""
    cfg = DecodeConfig(14, "many_rows", B=513, T=200, k=32, dtype="bf16")
    rows = sorted(set(range(0, cfg.B, 13)) | set(range(cfg.B - 9, cfg.B)))
    check_decode(mla, cfg, rows=rows)


def test_prefill_many_queries_all_rows(mla):
    """A 600-query chunk (row-major absorbed queries), compared on every query."""
    cfg = PrefillConfig(15, "prefill_600", S=600, T=700, k=64, start_pos=100, dtype="bf16")
    inp = synth.prefill_inputs(cfg)
    out = to_host64(run_prefill(mla, upload(inp), cfg.start_pos))
    err = rel_err(out, oracle.prefill(inp, start_pos=cfg.start_pos))
    log(f"prefill 600 queries: rel err {err:.3e}")
    assert err <= TOL["bf16"]


# ------------------------------------------------------------------ edge cases

def _bf16_decode_workspace(rows, k, n_split):
    """Workspace bytes of a bf16 decode of `rows` query rows split into n_split splits."""
    def up(x):
        return (x + 255) // 256 * 256
    q = rows * 128 * 576 * 2
    o = n_split * rows * 128 * 512 * 2
    ml = 2 * n_split * rows * 128 * 4
    return up(up(up(q) + o) + ml) + 256          # + the call's diagnostics


@pytest.mark.parametrize("B,k,n_split", [(64, 32, 1), (64, 64, 2), (64, 96, 3), (64, 128, 4),
                                         (52, 160, 5)])
def test_split_counts(mla, B, k, n_split):
    # Every split count from one to five: one split (the merge only divides by
    # the sum), the paths that stage up to four splits at once with their
    # partial-count branches, and the grouped path past four.
    assert mla.decode_workspace_size(B, 900, k, torch.bfloat16) == _bf16_decode_workspace(B, k, n_split)
    check_decode(mla, DecodeConfig(40 + n_split, f"splits{n_split}", B=B, T=900, k=k, dtype="bf16"),
                 rows=[0, 1, B // 2, B - 1])

def test_many_splits_ragged_chunk_all_rows(mla):
    # 20 rows x 2048 slots: thirteen splits of 160 slots, the last one of 128.
    # Past eight splits the merge takes its many-splits form, and 13 leaves a
    # last chunk of one split (three clamped loads with weight 0).
    B, k = 20, 2048
    assert mla.decode_workspace_size(B, 4096, k, torch.bfloat16) == _bf16_decode_workspace(B, k, 13)
    check_decode(mla, DecodeConfig(46, "splits13", B=B, T=4096, k=k, dtype="bf16"))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_selected_row(mla, dtype):
    check_decode(mla, DecodeConfig(14, "k1", B=2, T=50, k=1, dtype=dtype))


def test_empty_slots_and_empty_selection(mla):
    cfg = DecodeConfig(15, "pads", B=3, T=200, k=40, dtype="bf16")
    inp = synth.decode_inputs(cfg)
    inp["topk_idx"][0, ::3] = -1          # some empty slots
    inp["topk_idx"][1, :] = -1            # nothing selected: all-zero output
    out, _, _ = check_decode(mla, cfg, rows=[0, 2], inp=inp)
    assert np.array_equal(out[1], np.zeros((128, 128)))


def test_trailing_empty_tiles_are_skipped(mla):
    # 64 rows and k = 512: four splits of 128 slots, four tiles each.  A split runs its tiles
    # up to its last selected slot only, and a split with none selected writes an empty
    # partial; lists that end early, or hold a single slot, exercise both.
    cfg = DecodeConfig(18, "tails", B=64, T=2000, k=512, dtype="bf16")
    inp = synth.decode_inputs(cfg)
    idx = inp["topk_idx"]
    idx[0, 1:] = -1            # one slot: split 0 runs one tile, splits 1-3 are empty
    idx[1, 33:] = -1           # split 0 runs two tiles
    idx[2, 200:] = -1          # split 1 ends inside its third tile; splits 2 and 3 are empty
    idx[3, :-1] = -1           # only the last slot: split 3 runs all four tiles, the rest none
    keep = idx[4, 130]
    idx[4, :] = -1
    idx[4, 130] = keep         # one slot inside split 1's first tile
    idx[5, 64:128] = -1        # split 0 ends after two tiles; splits 1-3 are full
    check_decode(mla, cfg, rows=[0, 1, 2, 3, 4, 5, 63], inp=inp)


def test_unselected_rows_never_read(mla):
    cfg = DecodeConfig(16, "poison", B=2, T=500, k=90, dtype="bf16")
    inp = synth.decode_inputs(cfg)
    clean = to_host64(run_decode(mla, upload(inp)))
    poisoned = {k: v.copy() for k, v in inp.items()}
    for b in range(cfg.B):
        mask = np.ones(cfg.T, bool)
        mask[inp["topk_idx"][b]] = False
        poisoned["kv_cache"][b, mask] = 0x7FC0     # bf16 NaN
        poisoned["pe_cache"][b, mask] = 0x7F80     # bf16 +inf
    got = to_host64(run_decode(mla, upload(poisoned)))
    assert np.array_equal(got, clean)


def test_rows_beyond_T_never_read(mla):
    cfg = DecodeConfig(17, "ldT", B=2, T=300, k=60, dtype="bf16")
    inp = synth.decode_inputs(cfg)
    dev = upload(inp)
    ld = cfg.T + 17
    big_kv = torch.full((cfg.B, ld, 512), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    big_pe = torch.full((cfg.B, ld, 64), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    big_kv[:, :cfg.T] = dev["kv_cache"]
    big_pe[:, :cfg.T] = dev["pe_cache"]
    ref = to_host64(run_decode(mla, dev))
    dev2 = dict(dev, kv_cache=big_kv, pe_cache=big_pe)
    idx = dev["topk_idx"].clone()
    idx[:, 0] = cfg.T + 5                 # at or past T: treated as an empty slot
    dev2["topk_idx"] = idx
    got = to_host64(mla.decode(dev2["q_nope"], dev2["q_pe"], big_kv, big_pe, idx, dev2["w_uk"],
                               dev2["w_uv"], T=cfg.T))
    assert np.all(np.isfinite(got))
    idx_ref = idx.cpu().numpy()
    idx_ref[idx_ref >= cfg.T] = -1        # the library's reading: an empty slot
    inp2 = dict(inp, topk_idx=idx_ref)
    err = rel_err(got, oracle.decode(inp2))
    assert err <= TOL["bf16"]
    assert not np.array_equal(got, ref)


def test_index_order_does_not_matter(mla):
    cfg = DecodeConfig(18, "perm", B=2, T=2000, k=300, dtype="bf16")
    inp = synth.decode_inputs(cfg)
    rng = np.random.default_rng(1)
    shuffled = dict(inp, topk_idx=np.stack([rng.permutation(r) for r in inp["topk_idx"]]))
    out = to_host64(run_decode(mla, upload(shuffled)))
    assert rel_err(out, oracle.decode(inp)) <= TOL["bf16"]


def test_repeat_calls_are_bit_identical_and_workspace_contents_ignored(mla):
    cfg = DecodeConfig(19, "det", B=5, T=3000, k=700, dtype="bf16")
    dev = upload(synth.decode_inputs(cfg))
    a = run_decode(mla, dev).clone()
    need = mla.decode_workspace_size(cfg.B, cfg.T, cfg.k, torch.bfloat16)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda:0")
    b = run_decode(mla, dev, workspace=ws)
    c = run_decode(mla, dev, workspace=ws)
    assert torch.equal(a, b) and torch.equal(b, c)


def test_validate_indices(mla):
    idx = torch.tensor([[0, 5, 9, 3], [1, 2, 3, 4]], dtype=torch.int32, device="cuda:0")
    assert mla.validate_indices(idx, T=10) == 0
    dup = idx.clone()
    dup[1, 3] = 1
    assert mla.validate_indices(dup, T=10) == 2
    assert mla.validate_indices(idx, T=9) == 1
    pad = idx.clone()
    pad[0, 1] = -1
    assert mla.validate_indices(pad, T=10) == 1
    assert mla.validate_indices(pad, T=10, allow_pad=True) == 0
    inp = synth.decode_inputs(synth.CONFIGS["sparse_b32_t8k"], with_cache=False)
    assert mla.validate_indices(to_dev(inp["topk_idx"]), T=8192) == 0


def test_side_stream_with_int64_indices(mla):
    # A call on a side stream, with int64 indices the binding converts: the conversion,
    # the workspace and the output are made on that stream after it has waited for the
    # current one, so the result equals the same call on the current stream.
    cfg = DecodeConfig(24, "side_stream", B=3, T=900, k=200, dtype="bf16")
    inp = synth.decode_inputs(cfg)
    dev = upload(inp)
    ref = run_decode(mla, dev).clone()
    side = torch.cuda.Stream()
    q_nope = dev["q_nope"] * 1.0            # produced on the current stream just before the call
    idx64 = dev["topk_idx"].to(torch.int64)
    out = mla.decode(q_nope, dev["q_pe"], dev["kv_cache"], dev["pe_cache"], idx64, dev["w_uk"],
                     dev["w_uv"], stream=side)
    assert mla.validate_indices(idx64, T=cfg.T, stream=side) == 0
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_attention_event_hook(mla):
    cfg = DecodeConfig(20, "ev", B=4, T=1000, k=256, dtype="bf16")
    dev = upload(synth.decode_inputs(cfg))
    b = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    b.record()
    e.record()
    torch.cuda.synchronize()
    mla.set_attention_events(b, e)
    run_decode(mla, dev)
    ms = b.elapsed_time(e)
    assert 0.0 < ms < 1000.0


def _split_plan(rows, k):
    """(splits, slots per split) of the attention work split: about 256 workgroups, whole
    32-slot tiles, at most 2048 slots per split; confirmed against the workspace size the
    library reports for that many splits."""
    n = -(-256 // rows)
    n = max(min(n, -(-k // 32)), -(-k // 2048), 1)
    per = -(-(-(-k // n)) // 32) * 32
    n = -(-k // per)
    assert _MLA["m"].decode_workspace_size(rows, k, k, torch.bfloat16) == _bf16_decode_workspace(rows, k, n)
    return n, per


_MLA = {}


def predicted_excess(inp, scale, rows, k, causal_base=None):
    """Largest amount (log2 units) by which a scaled score beats its split's reference, the
    maximum of the split's first 32-slot tile that holds a selected position, over every
    (query, split, head); computed in float64 from the inputs (the scores' definition).
    causal_base: prefill queries see positions <= causal_base + query."""
    n, per = _split_plan(rows, k)
    qc = np.einsum("rhd,hdc->rhc", oracle.to_f64(inp["q_nope"]), oracle.to_f64(inp["w_uk"]))
    worst = -np.inf
    for r in range(rows):
        kv = inp["kv_cache"][r] if causal_base is None else inp["kv_cache"]
        pe = inp["pe_cache"][r] if causal_base is None else inp["pe_cache"]
        T = kv.shape[0]
        lim = T - 1 if causal_base is None else min(T - 1, causal_base + r)
        idx = inp["topk_idx"][r]
        for sp in range(n):
            slots = idx[sp * per:(sp + 1) * per]
            ok = (slots >= 0) & (slots <= lim)
            if not ok.any():
                continue
            pos = np.where(ok, slots, 0)
            sc = (qc[r] @ oracle.to_f64(kv[pos]).T + oracle.to_f64(inp["q_pe"][r]) @ oracle.to_f64(pe[pos]).T)
            sc = np.where(ok[None, :], sc * scale * np.log2(np.e), -np.inf)      # [128, slots]
            tiles = [sc[:, i:i + 32] for i in range(0, sc.shape[1], 32)]
            first = next(t for t in tiles if np.isfinite(t).any())
            ref = first.max(axis=1)
            worst = max(worst, float(np.max(sc.max(axis=1) - ref)))
    return worst


def rerun_count(mla, dev, inp, scale=None, prefill_start=None):
    """Run the call again with a workspace the test holds and read its rerun count."""
    rows = dev["q_nope"].shape[0]
    k = dev["topk_idx"].shape[1]
    if prefill_start is None:
        ws = torch.empty(mla.decode_workspace_size(rows, dev["kv_cache"].shape[1], k, torch.bfloat16),
                         dtype=torch.uint8, device="cuda:0")
        kw = {} if scale is None else {"softmax_scale": scale}
        run_decode(mla, dev, workspace=ws, **kw)
    else:
        ws = torch.empty(mla.prefill_chunk_workspace_size(rows, dev["kv_cache"].shape[0], k,
                                                          torch.bfloat16),
                         dtype=torch.uint8, device="cuda:0")
        run_prefill(mla, dev, prefill_start, workspace=ws, softmax_scale=scale)
    d = mla.diagnostics(ws, rows, k, torch.bfloat16)
    assert d["reserved"] == 0
    return d["reruns"]


@pytest.mark.parametrize("B,T,k", [(64, 2000, 1024), (8, 3000, 2048)])
def test_large_logits_rerun_the_split(mla, B, T, k):
    # With W_UK = 0 the scores are scale * (q_pe . k_R), computed from exact bf16 inputs,
    # so a large scale spreads them over hundreds of log2 units without amplifying any
    # rounding.  Later tiles then beat their split's first-tile reference by far more
    # than 60 (log2), and those splits run again with each head's largest score as the
    # reference.  64 rows give four splits of eight tiles; 8 rows give 32 splits of two
    # tiles, which the merge takes four at a time.
    _MLA["m"] = mla
    cfg = DecodeConfig(21, "big_logits", B=B, T=T, k=k, dtype="bf16")
    inp = synth.decode_inputs(cfg)
    inp["w_uk"] = np.zeros_like(inp["w_uk"])
    scale = 10.0
    excess = predicted_excess(inp, scale, B, k)
    log(f"large logits B={B}: largest excess over a split reference {excess:.1f} (log2)")
    assert excess > 90                       # far past the rerun threshold
    dev = upload(inp)
    out = to_host64(run_decode(mla, dev, softmax_scale=scale))
    n = rerun_count(mla, dev, inp, scale=scale)
    log(f"  splits rerun: {n}")
    assert n > 0
    ref = oracle.decode(inp, scale=scale)
    err = rel_err(out, ref)
    log(f"  all rows: rel err {err:.3e}")
    assert np.all(np.isfinite(out)) and err <= TOL["bf16"]


def test_large_logits_rerun_causal_prefill(mla):
    # The same forced case in a causal prefill chunk: 256 queries take one split each
    # (128 slots, four tiles), and each stops at its own position.
    _MLA["m"] = mla
    cfg = PrefillConfig(23, "prefill_big_logits", S=256, T=600, k=128, start_pos=300, dtype="bf16")
    inp = synth.prefill_inputs(cfg)
    inp["w_uk"] = np.zeros_like(inp["w_uk"])
    scale = 10.0
    excess = predicted_excess(inp, scale, cfg.S, cfg.k, causal_base=cfg.start_pos)
    log(f"prefill large logits: largest excess {excess:.1f} (log2)")
    assert excess > 90
    dev = upload(inp)
    out = to_host64(run_prefill(mla, dev, cfg.start_pos, softmax_scale=scale))
    assert rerun_count(mla, dev, inp, scale=scale, prefill_start=cfg.start_pos) > 0
    err = rel_err(out, oracle.prefill(inp, start_pos=cfg.start_pos, scale=scale))
    log(f"  all queries: rel err {err:.3e}")
    assert np.all(np.isfinite(out)) and err <= TOL["bf16"]


def test_moderate_scale(mla):
    cfg = DecodeConfig(22, "scale_half", B=8, T=2000, k=1024, dtype="bf16")
    inp = synth.decode_inputs(cfg)
    out = to_host64(run_decode(mla, upload(inp), softmax_scale=0.5))
    ref = oracle.decode(inp, rows=[0, 7], scale=0.5)
    assert rel_err(out[[0, 7]], ref) <= TOL["bf16"]


def _max_t() -> int:
    """MLA_MAX_T as the public header defines it."""
    import pathlib
    import re
    hdr = (pathlib.Path(__file__).resolve().parent.parent / "include" / "mla_sparse.h").read_text()
    return int(re.search(r"#define MLA_MAX_T (\d+)", hdr).group(1))


def test_largest_cache_length(mla):
    """One batch row at T = MLA_MAX_T: selected rows at both ends of the cache (byte offsets
    up to ~2^31), empty slots and an index equal to T among them, every other row NaN.
    Decode has no causal mask, so the oracle sees the same rows packed into a short cache."""
    T = _max_t()
    kv_sel = 93                                  # selected rows; + 3 empty slots = 96 (3 tiles)
    cfg = DecodeConfig(21, "maxT", B=1, T=kv_sel, k=kv_sel, dtype="bf16")
    inp = synth.decode_inputs(cfg)               # every position of the short cache selected
    rng = np.random.default_rng(7)
    pos = np.sort(np.concatenate([[0, 1, T - 2, T - 1],
                                  rng.choice(np.arange(2, T - 2), size=kv_sel - 4, replace=False)]))
    log(f"decode at T={T}: {kv_sel} rows, last at byte offset {int(pos[-1]) * 1024}")
    dev = upload({k: v for k, v in inp.items() if k not in ("kv_cache", "pe_cache", "topk_idx")})
    big_kv = torch.full((1, T, 512), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    big_pe = torch.full((1, T, 64), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    pos_t = torch.from_numpy(pos).to("cuda:0")
    big_kv[0, pos_t] = to_dev(inp["kv_cache"][0])
    big_pe[0, pos_t] = to_dev(inp["pe_cache"][0])
    idx = np.concatenate([pos, [-1, T, -1]]).astype(np.int32)   # T itself selects nothing
    idx = rng.permutation(idx)[None, :]
    got = to_host64(mla.decode(dev["q_nope"], dev["q_pe"], big_kv, big_pe,
                               torch.from_numpy(idx).to("cuda:0"), dev["w_uk"], dev["w_uv"]))
    torch.cuda.synchronize()
    del big_kv, big_pe
    assert np.all(np.isfinite(got))
    err = rel_err(got, oracle.decode(inp))
    log(f"  rel err {err:.3e}")
    assert err <= TOL["bf16"]
