"""GPU: the matrix-core rate probe (attn_mfma_probe) runs every MFMA it is asked for.

With y = 0 both operands are bf16(x) in every lane, so each of a thread's 64 accumulator values gains
16 * x^2 per MFMA and the checksum is 1024 * x^2 * iters exactly (x = 1/8: 16 * iters, exact in fp32).
The tick pairs must be positive; their ratio is the engine clock the probe reports.
"""

import pytest
import torch

import scaled_dot_product_02_amd as sd

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("blocks,iters", [(1, 1), (8, 1000), (300, 257)])
def test_probe_checksum_and_ticks(blocks, iters):
    out, ticks = sd.attn_mfma_probe(blocks, iters, x=0.125, y=0.0)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.full((blocks * 256,), 16.0 * iters))
    if iters >= 1000:  # long enough for the 100 MHz reference counter to advance
        t = ticks.cpu()
        assert (t > 0).all(), t
        # shader-clock ticks per 100 MHz tick: the engine clock, which lies between idle and boost
        ghz = 0.1 * t[:, 0].double() / t[:, 1].double()
        assert ((ghz > 0.5) & (ghz < 3.0)).all(), ghz
