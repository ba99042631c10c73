"""The measurement aids beside the kernels.  Clock probe: every workgroup reports an engine clock
within the part's range and real-time ticks covering the requested interval.  MFMA rate probe:
its sums are exact on operands whose products are small integers."""
import pytest
import torch

import exact_attention_online_amd as eao
from gpu_util import device

pytestmark = pytest.mark.gpu


def test_clock_probe_reports_a_plausible_clock():
    dev = device()
    out = torch.zeros(16, dtype=torch.int64, device=dev)
    eao.clock_probe(out, 200000)              # 2 ms
    torch.cuda.synchronize()
    c = out.view(8, 2).cpu()
    assert (c[:, 1] >= 200000).all() and (c[:, 1] < 200000 + 100000).all()
    ghz = 0.1 * c[:, 0].double() / c[:, 1].double()
    assert ((ghz > 0.05) & (ghz < 3.0)).all(), ghz.tolist()


@pytest.mark.parametrize("value, iters", [(1.0, 2), (0.0, 3), (2.0, 1)])
def test_mfma_probe_sums_are_exact(value, iters):
    """Every operand equal to x: each MFMA adds 16 x^2 to every accumulator element, 8 MFMAs
    per accumulator and iteration, and a thread sums 4 accumulators of 16 elements."""
    dev = device()
    data = torch.full((1 << 16,), value, dtype=torch.bfloat16, device=dev)
    out = torch.full((512 * 3,), -1.0, dtype=torch.float32, device=dev)
    flops = eao.mfma_probe(data, out, iters)
    torch.cuda.synchronize()
    assert flops == 3 * 8 * 32 * iters * 32768
    want = 64 * 8 * iters * 16 * value * value
    assert torch.equal(out, torch.full_like(out, want))
