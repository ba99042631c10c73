"""The measurement aids beside the kernels.  Clock probe: every workgroup reports an engine clock
within the part's range and real-time ticks covering the requested interval.  MFMA rate probe:
its sums are exact on operands whose products are small integers, bf16 and fp8.  HBM read probe: the sum of
its outputs modulo 2^32 is that of every 32-bit word of the buffer (so every byte was read, once)."""
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


@pytest.mark.parametrize("code, value, iters", [(0x38, 1.0, 2), (0x00, 0.0, 1), (0x40, 2.0, 3), (0xB8, -1.0, 1)])
def test_mfma_probe_fp8_sums_are_exact(code, value, iters):
    """fp8 e4m3 operands all equal to x (0x38 = 1, 0x40 = 2, 0xB8 = -1): each MFMA adds 64 x^2 to
    every accumulator element, 8 MFMAs per accumulator and iteration, 4 x 16 elements a thread."""
    dev = device()
    data = torch.full((1 << 16,), code, dtype=torch.uint8, device=dev)
    out = torch.full((512 * 2,), -1.0, dtype=torch.float32, device=dev)
    flops = eao.mfma_probe(data, out, iters)
    torch.cuda.synchronize()
    assert flops == 2 * 8 * 32 * iters * 131072
    want = 64 * 8 * iters * 64 * value * value
    assert torch.equal(out, torch.full_like(out, want))


@pytest.mark.parametrize("stages, groups", [(1, 7), (2, 3), (3, 5), (5, 3), (16, 256)])
def test_hbm_probe_reads_every_word_once(stages, groups):
    dev = device()
    g = torch.Generator(device=dev).manual_seed(stages * 100 + groups)
    n = stages * groups * 16384 // 4
    data = torch.randint(-(1 << 31), (1 << 31) - 1, (n,), dtype=torch.int32, device=dev, generator=g)
    out = torch.full((64 * groups,), -1, dtype=torch.int32, device=dev)
    assert eao.hbm_probe(data, out) == 4 * n
    torch.cuda.synchronize()
    mask = (1 << 32) - 1
    assert (int(out.to(torch.int64).sum()) & mask) == (int(data.to(torch.int64).sum()) & mask)
    # each lane's own words: lane l of group g sums bytes 16 l .. 16 l + 15 of every 1 KB piece
    words = data.view(groups, -1, 64, 4).to(torch.int64).sum(dim=(1, 3)) & mask
    assert torch.equal(out.view(groups, 64).to(torch.int64) & mask, words)
