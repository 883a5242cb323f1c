"""GPU parity of the cache append against the oracle.

Written rows: max|gpu - oracle| / max|oracle| <= 1e-5 (float32) or 2e-2 (bf16),
per cache; every other row of both caches must be bit-identical to its value
before the call.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
from synth.generators import AppendConfig  # noqa: E402

from .gpu_util import TOL, log, rel_err, to_dev, to_host64  # noqa: E402

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_latent_attention_amd as m
    m._lib.load()
    return m


def check_append(mla, cfg):
    inp = synth.append_inputs(cfg)
    dev = {k: to_dev(v) for k, v in inp.items()}
    before_kv, before_pe = dev["kv_cache"].clone(), dev["pe_cache"].clone()
    log(f"append {cfg.name}: B={cfg.B} S={cfg.S} T={cfg.T} start={cfg.start_pos} {cfg.dtype}")
    mla.cache_append(dev["kv_a_out"], dev["norm_weight"], dev["cos_sin"], dev["kv_cache"], dev["pe_cache"],
                     start_pos=cfg.start_pos, eps=EPS)
    torch.cuda.synchronize()
    ref_kv, ref_pe = oracle.cache_append(inp["kv_a_out"], inp["norm_weight"], inp["cos_sin"],
                                         inp["kv_cache"], inp["pe_cache"], cfg.start_pos, EPS)
    rows = slice(cfg.start_pos, cfg.start_pos + cfg.S)
    got_kv, got_pe = to_host64(dev["kv_cache"]), to_host64(dev["pe_cache"])
    e_kv = rel_err(got_kv[:, rows], ref_kv[:, rows])
    e_pe = rel_err(got_pe[:, rows], ref_pe[:, rows])
    log(f"  written rows: latent rel err {e_kv:.3e}, rotary rel err {e_pe:.3e}")
    assert e_kv <= TOL[cfg.dtype] and e_pe <= TOL[cfg.dtype]
    keep = np.ones(cfg.T, bool)
    keep[rows] = False
    keep_t = torch.from_numpy(keep).to("cuda:0")
    assert torch.equal(dev["kv_cache"][:, keep_t], before_kv[:, keep_t])
    assert torch.equal(dev["pe_cache"][:, keep_t], before_pe[:, keep_t])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_step_append(mla, dtype):
    # one new position per sequence, at the end of a 64-row batch's caches
    check_append(mla, AppendConfig(60, "append_decode", B=64, S=1, T=1001, start_pos=1000, dtype=dtype))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_chunk_append(mla, dtype):
    # a chunk of one sequence, ragged against the four positions a workgroup takes
    check_append(mla, AppendConfig(61, "append_chunk", B=1, S=4093, T=4200, start_pos=100, dtype=dtype))


def test_ragged_batch_append(mla):
    check_append(mla, AppendConfig(62, "append_ragged", B=3, S=7, T=20, start_pos=0, dtype="bf16"))
