"""The clock probe (a measurement aid beside the kernels): every workgroup reports an engine clock
within the part's range and real-time ticks covering the requested interval."""
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
