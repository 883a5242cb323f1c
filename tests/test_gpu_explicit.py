"""GPU parity of the explicit-form prefill (keys and values up-projected per head,
bitmap-masked attention) against the fp64 oracle's prefill.

Same tolerance as the latent form: max|gpu - oracle| / max|oracle| <= 2e-2 for
bf16 inputs.  The 4096-query chunk is compared on the latent form's strided
sample; small chunks on every query, with ragged query blocks (128 queries per
workgroup) and ragged position tiles (32 per tile).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
from synth.generators import PrefillConfig  # noqa: E402

from .gpu_util import TOL, log, rel_err, to_host64  # noqa: E402
from .test_gpu_parity import _oracle_prefill_parallel, _prefill_rows, upload  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_latent_attention_amd as m
    m._lib.load()
    return m


def run_explicit(mla, dev, start_pos, **kw):
    out = mla.prefill_explicit(dev["q_nope"], dev["q_pe"], dev["kv_cache"], dev["pe_cache"],
                               dev["topk_idx"], dev["w_uk"], dev["w_uv"], start_pos=start_pos, **kw)
    torch.cuda.synchronize()
    return out


def test_config4_explicit_prefill_sampled(mla):
    cfg = synth.CONFIGS["prefill_s4096"]
    inp = synth.prefill_inputs(cfg)
    dev = upload(inp)
    log(f"explicit prefill {cfg.name}: S={cfg.S} T={cfg.T} k={cfg.k}")
    out = to_host64(run_explicit(mla, dev, cfg.start_pos))
    assert np.all(np.isfinite(out))
    rows = _prefill_rows(cfg.S)
    ref = _oracle_prefill_parallel(inp, rows, cfg.start_pos)
    err = rel_err(out[rows], ref)
    log(f"  {len(rows)} queries: rel err {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("S,T,k,start_pos", [(70, 300, 48, 200), (150, 150, 100, 0),
                                             (300, 1000, 256, 600), (1, 40, 8, 39),
                                             (129, 129, 129, 0)])
def test_explicit_prefill_all_rows(mla, S, T, k, start_pos):
    cfg = PrefillConfig(31, "explicit_small", S=S, T=T, k=k, start_pos=start_pos, dtype="bf16")
    inp = synth.prefill_inputs(cfg)
    out = to_host64(run_explicit(mla, upload(inp), start_pos))
    err = rel_err(out, oracle.prefill(inp, start_pos=start_pos))
    log(f"explicit S={S} T={T} k={k} start={start_pos}: rel err {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= TOL["bf16"]


def test_explicit_prefill_empty_future_and_repeated_entries(mla):
    # Empty slots, whole rows with nothing selected (all-zero output), positions after the
    # query's own (ignored) and a position listed twice (counted once: the mask is a set).
    cfg = PrefillConfig(32, "explicit_edges", S=96, T=400, k=64, start_pos=250, dtype="bf16")
    inp = synth.prefill_inputs(cfg)
    idx = inp["topk_idx"]
    idx[0, ::2] = -1
    idx[1, :] = -1
    idx[2, :5] = [399, 398, 300, 251 + 2, 260]     # > 252 are after query 2's position
    idx[3, 1] = idx[3, 0]
    idx[4, :] = -1
    idx[4, 0] = 399                                 # its only entry is in its future
    out = to_host64(run_explicit(mla, upload(inp), cfg.start_pos))
    ref = oracle.prefill(inp, start_pos=cfg.start_pos)
    assert np.array_equal(out[1], np.zeros((128, 128)))
    assert np.array_equal(out[4], np.zeros((128, 128)))
    err = rel_err(out, ref)
    log(f"explicit edge cases: rel err {err:.3e}")
    assert err <= TOL["bf16"]


def test_explicit_agrees_with_latent_form(mla):
    # The two forms are the same function of the inputs (absorbed and explicit scores agree);
    # on the GPU they round differently, so they agree to the bf16 tolerance.
    cfg = PrefillConfig(33, "explicit_vs_latent", S=256, T=700, k=200, start_pos=444, dtype="bf16")
    inp = synth.prefill_inputs(cfg)
    dev = upload(inp)
    a = to_host64(run_explicit(mla, dev, cfg.start_pos))
    b = to_host64(mla.prefill_chunk(dev["q_nope"], dev["q_pe"], dev["kv_cache"], dev["pe_cache"],
                                    dev["topk_idx"], dev["w_uk"], dev["w_uv"],
                                    start_pos=cfg.start_pos))
    assert rel_err(a, b) <= TOL["bf16"]


def test_explicit_prefill_rejects_float32(mla):
    cfg = PrefillConfig(34, "explicit_f32", S=4, T=20, k=4, start_pos=16, dtype="f32")
    dev = upload(synth.prefill_inputs(cfg))
    with pytest.raises(mla.MLAError):
        run_explicit(mla, dev, cfg.start_pos)


def reference_gaps(inp, start_pos, scale, queries, heads):
    """For sampled (query, head) pairs: the largest selected scaled score (log2 units) minus the
    first-tile reference (the largest over positions 0..31, selected or not), from the inputs in
    float64 (the scores' definition)."""
    kv, pe = oracle.to_f64(inp["kv_cache"]), oracle.to_f64(inp["pe_cache"])
    w_uk = oracle.to_f64(inp["w_uk"])
    qn, qp = oracle.to_f64(inp["q_nope"]), oracle.to_f64(inp["q_pe"])
    T = kv.shape[0]
    gaps = []
    for h in heads:
        k_nope = kv @ w_uk[h].T
        for s in queries:
            sc = (k_nope @ qn[s, h] + pe @ qp[s, h]) * scale * np.log2(np.e)
            sel = oracle.selected_rows(inp["topk_idx"][s], T, start_pos + s)
            if sel.size:
                gaps.append(float(sc[sel].max() - sc[:32].max()))
    return np.array(gaps)


def test_explicit_large_logits_restart_from_exact_reference(mla):
    # With W_UK = 0 the scores are scale * (q_pe . k_R), products of exact bf16 inputs, so a
    # large scale spreads them over hundreds of log2 units without amplifying any rounding.
    # Weights against the first tile's maximum then overflow, and every workgroup starts
    # again from its exact maximum.
    cfg = PrefillConfig(35, "explicit_big_logits", S=256, T=700, k=160, start_pos=400, dtype="bf16")
    inp = synth.prefill_inputs(cfg)
    inp["w_uk"] = np.zeros_like(inp["w_uk"])
    scale = 10.0
    gaps = reference_gaps(inp, cfg.start_pos, scale, range(0, cfg.S, 37), range(0, 128, 31))
    log(f"explicit large logits: largest gap over the first-tile reference {gaps.max():.1f} (log2)")
    assert gaps.max() > 128                         # weights against it would overflow float
    out = to_host64(run_explicit(mla, upload(inp), cfg.start_pos, softmax_scale=scale))
    err = rel_err(out, oracle.prefill(inp, start_pos=cfg.start_pos, scale=scale))
    log(f"explicit large logits: rel err {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= TOL["bf16"]


def test_explicit_reference_far_above_the_selection(mla):
    # Rotary-key rows 0..31 scaled by 60 give every query a first-tile maximum far above the
    # scores of the positions it selects (none of 0..31 for most queries), so its weights
    # against that reference would underflow; the workgroup starts again from the exact
    # maximum.  The rotary keys enter the scores unprojected, so the scaling adds no rounding.
    cfg = PrefillConfig(36, "explicit_low_sel", S=128, T=500, k=96, start_pos=372, dtype="bf16")
    inp = synth.prefill_inputs(cfg)
    rows = (inp["pe_cache"][:32].astype(np.uint32) << 16).view(np.float32) * 60.0
    inp["pe_cache"][:32] = (rows.view(np.uint32) >> 16).astype(np.uint16)
    idx = inp["topk_idx"]
    idx[4:][idx[4:] < 32] = -1                      # queries 0..3 keep theirs
    gaps = reference_gaps(inp, cfg.start_pos, oracle.SOFTMAX_SCALE, range(4, cfg.S, 13), range(0, 128, 31))
    log(f"explicit reference above selection: smallest gap {gaps.min():.1f} (log2)")
    assert gaps.min() < -60                         # weights against it would lose range
    out = to_host64(run_explicit(mla, upload(inp), cfg.start_pos))
    err = rel_err(out, oracle.prefill(inp, start_pos=cfg.start_pos))
    log(f"explicit reference above selection: rel err {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= TOL["bf16"]
