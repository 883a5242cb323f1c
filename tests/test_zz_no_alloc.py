"""The allocation-free decode entry point against the ordinary one.

mla_sparse_decode_noalloc runs the same kernels as mla_sparse_decode with its
workspace in the library's fixed device array, so on the same inputs the two
must give bit-identical outputs.  Two calls in a row, the second smaller,
show that the array's leftover contents from one call do not reach the next.
"""
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from synth.generators import DecodeConfig  # noqa: E402

from .gpu_util import log, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_latent_attention_amd as m
    m._lib.load()
    return m


def _both(mla, cfg):
    dev = {k: to_dev(v) for k, v in synth.decode_inputs(cfg).items()}
    args = (dev["q_nope"], dev["q_pe"], dev["kv_cache"], dev["pe_cache"], dev["topk_idx"],
            dev["w_uk"], dev["w_uv"])
    dt = dev["q_nope"].dtype
    need = mla.decode_workspace_size(cfg.B, cfg.T, cfg.k, dt)
    log(f"noalloc {cfg.name}: B={cfg.B} T={cfg.T} k={cfg.k} {cfg.dtype}, workspace {need} bytes")
    assert need <= mla.NOALLOC_SCRATCH_BYTES
    ref = mla.decode(*args)
    out = torch.full_like(ref, float("nan"))
    mla.decode_noalloc(*args, out=out)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_equals_decode_on_two_calls_in_a_row(mla):
    # a large call (four splits per row, most of the array in use), then a smaller one
    big = DecodeConfig(50, "noalloc_big", B=64, T=4096, k=2048, dtype="bf16")
    small = DecodeConfig(51, "noalloc_small", B=3, T=777, k=333, dtype="bf16")
    for cfg in (big, small):
        ref, out = _both(mla, cfg)
        assert torch.equal(out, ref), cfg.name


def test_noalloc_float32_and_refusal(mla):
    ref, out = _both(mla, DecodeConfig(52, "noalloc_f32", B=2, T=300, k=100, dtype="f32"))
    assert torch.equal(out, ref)
    # a call whose workspace exceeds the array is refused before anything runs
    cfg = DecodeConfig(53, "noalloc_too_big", B=2, T=300, k=100, dtype="bf16")
    dev = {k: to_dev(v) for k, v in synth.decode_inputs(cfg).items()}
    big_b = 128
    q = dev["q_nope"].repeat(big_b // 2, 1, 1)
    qp = dev["q_pe"].repeat(big_b // 2, 1, 1)
    kv = torch.zeros((big_b, 4096, 512), dtype=torch.bfloat16, device="cuda:0")
    pe = torch.zeros((big_b, 4096, 64), dtype=torch.bfloat16, device="cuda:0")
    idx = torch.arange(2048, dtype=torch.int32, device="cuda:0").repeat(big_b, 1)
    out = torch.empty((big_b, 128, 128), dtype=torch.bfloat16, device="cuda:0")
    assert mla.decode_workspace_size(big_b, 4096, 2048, torch.bfloat16) > mla.NOALLOC_SCRATCH_BYTES
    with pytest.raises(mla.MLAError, match="MLA_ERR_WORKSPACE"):
        mla.decode_noalloc(q, qp, kv, pe, idx, dev["w_uk"], dev["w_uv"], out=out)
