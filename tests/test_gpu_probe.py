"""GPU: the measurement probes run what they are asked for.

attn_mfma_probe: the matrix-core rate probe runs every MFMA it is asked for.

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


@pytest.mark.parametrize("kind", ["b128", "b64"])
def test_lds_probe_reads_what_it_is_given(kind):
    """attn_lds_probe: the LDS array holds int32 (2k + 1) * i at element 4i + k; b128 lanes add elements
    0 and 3 of their 16 bytes, b64 lanes both elements of their 8 bytes, 8 * iters times; inactive lanes
    (negative address) write 0."""
    iters = 5
    width = 16 if kind == "b128" else 8
    addrs = [-1 if l % 7 == 3 else (width * (37 * l)) % 32768 for l in range(64)]
    out = torch.full((64,), -1, dtype=torch.int32, device="cuda:0")
    sd.attn_lds_probe(kind, addrs, iters, out)
    torch.cuda.synchronize()

    def elem(e):
        return (2 * (e % 4) + 1) * (e // 4)

    want = []
    for a in addrs:
        if a < 0:
            want.append(0)
        elif kind == "b128":
            want.append(8 * iters * (elem(a // 4) + elem(a // 4 + 3)))
        else:
            want.append(8 * iters * (elem(a // 4) + elem(a // 4 + 1)))
    assert out.cpu().tolist() == want
