"""GPU parity of the FP8 wkv_b dequantisation against the oracle, and the decode run on the
dequantised weights against the oracle's decode on its own dequantisation.

Per element the kernel's bf16 result must be within one bf16 step of the exact value
(|gpu - ref| <= 2^-8 |ref|: the product is rounded to float32, then to bf16), NaN codes give
NaN, and zero codes give zeros of the same sign.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
from synth.generators import DecodeConfig  # noqa: E402

from .gpu_util import TOL, log, rel_err, to_dev, to_host64  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_latent_attention_amd as m
    m._lib.load()
    return m


def dequant(mla, d):
    codes = torch.from_numpy(d["codes"]).to("cuda:0")
    scales = torch.from_numpy(d["scales"]).to("cuda:0")
    w_uk, w_uv = mla.wkv_b_dequant(codes, scales)
    torch.cuda.synchronize()
    return w_uk, w_uv


def test_wkv_b_dequant_every_element(mla):
    d = synth.fp8_wkv_b_inputs()
    d["codes"][0, :4] = [0x7F, 0xFF, 0x00, 0x80]        # NaN, NaN, +0, -0
    d["codes"][1, :3] = [0x01, 0x7E, 0xFE]              # smallest subnormal, +-448
    w_uk, w_uv = dequant(mla, d)
    ref_uk, ref_uv = oracle.wkv_b_dequant(d["codes"], d["scales"])
    for got_t, ref in ((w_uk, ref_uk), (w_uv, ref_uv)):
        got = got_t.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        ok = ~np.isnan(ref)
        assert np.all(np.abs(got[ok] - ref[ok]) <= 2.0 ** -8 * np.abs(ref[ok]))
        assert np.array_equal(np.signbit(got[ok & (ref == 0)]), np.signbit(ref[ok & (ref == 0)]))
    assert np.isnan(w_uk[0, 0, 0].item()) and w_uk[0, 0, 3].item() == 0.0


def test_decode_on_dequantised_weights(mla):
    # the FP8 weight as the decode branch uses it: dequantised once, then the usual path
    cfg = DecodeConfig(91, "fp8_weights", B=4, T=700, k=256, dtype="bf16")
    inp = synth.decode_inputs(cfg)
    d = synth.fp8_wkv_b_inputs()
    # one scale for every block, so that the weights have the usual RMS 1/sqrt(512) and the
    # logits unit variance (codes are uniform over the format, so their RMS is large)
    vals = torch.from_numpy(d["codes"]).view(torch.float8_e4m3fn).to(torch.float64)
    d["scales"][:] = np.float32(512 ** -0.5 / vals.pow(2).mean().sqrt().item())
    w_uk, w_uv = dequant(mla, d)
    ref_uk, ref_uv = oracle.wkv_b_dequant(d["codes"], d["scales"])
    dev = {k: to_dev(v) for k, v in inp.items()}
    out = mla.decode(dev["q_nope"], dev["q_pe"], dev["kv_cache"], dev["pe_cache"], dev["topk_idx"], w_uk, w_uv)
    torch.cuda.synchronize()
    ref = oracle.decode(dict(inp, w_uk=ref_uk, w_uv=ref_uv))
    err = rel_err(to_host64(out), ref)
    log(f"decode on dequantised FP8 weights: rel err {err:.3e}")
    assert err <= TOL["bf16"]
