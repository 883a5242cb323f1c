"""GPU parity of the output projection Delta = o W_O against the oracle, on every output."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402

from .gpu_util import TOL, log, rel_err, to_dev, to_host64  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_latent_attention_amd as m
    m._lib.load()
    return m


@pytest.mark.parametrize("B,dtype", [(64, "bf16"), (1, "bf16"), (3, "bf16"), (97, "bf16"), (2, "f32")])
def test_output_projection(mla, B, dtype):
    # 64 rows: the decode batch (two 32-row blocks, one pass over the weight); 1, 3 and 97:
    # ragged blocks and a second pass; float32: the plain path
    inp = synth.projection_inputs(B, dtype)
    dev = {k: to_dev(v) for k, v in inp.items()}
    out = mla.output_projection(dev["o"], dev["w_o"])
    torch.cuda.synchronize()
    got = to_host64(out)
    ref = oracle.output_projection(inp["o"], inp["w_o"])
    err = rel_err(got, ref)
    log(f"projection B={B} {dtype}: rel err {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= TOL[dtype]
