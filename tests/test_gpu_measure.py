"""GPU check of the measurement helper ra_mfma_ceiling (the pure product loop
bench.py --mfma-ceiling times): with every operand element c, each product
adds 16 c^2 to each of the 16 accumulator entries a lane holds, so a lane's
output is 8 chains x 16 entries x iters x 8 products x 16 c^2."""
import pytest
import torch

pytestmark = pytest.mark.gpu

R = pytest.importorskip("context_blockwise_softmax_ra_amd")
from context_blockwise_softmax_ra_amd import _lib as L  # noqa: E402

DEV = torch.device("cuda:0")


@pytest.mark.parametrize("iters,n_wg", [(1, 1), (3, 7)])
def test_mfma_ceiling_constant_operands(iters, n_wg):
    c = 0.25
    ops = torch.full((4096, 8), c, dtype=torch.bfloat16, device=DEV)   # 64 KiB
    out = torch.full((n_wg * 256,), -1.0, dtype=torch.float32, device=DEV)
    L.ra_mfma_ceiling(ops, out, n_wg, iters)
    torch.cuda.synchronize()
    expect = 8 * 16 * iters * 8 * 16 * c * c
    assert torch.all(out == expect), (out.min().item(), out.max().item(), expect)
