"""The library holds no mutable state between calls: two host threads, each driving its own
problem (forward, then backward) on its own stream at the same time, get bit for bit what the
same calls give one after another on the default stream.  ctypes releases the interpreter lock
during each call, so the threads really are inside the library together."""
import threading

import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import draw, round_to
from gpu_util import device

pytestmark = pytest.mark.gpu

PROBLEMS = [(1, 4, 2, 700, 128, "bf16", True, 40), (2, 3, 3, 333, 64, "fp16", False, 41)]
ROUNDS = 4


def _inputs(B, Hq, Hkv, N, d, dtype, seed, dev):
    _, q, k, v, do = draw(B, Hq, Hkv, N, d, seed, with_grad=True)
    return [round_to(x, dtype).to(dev) for x in (q, k, v, do)]


def _step(q, k, v, do, causal):
    o, lse = eao.fwd(q, k, v, causal=causal)
    dq, dk, dv = eao.bwd(q, k, v, o, do, lse, causal=causal)
    return o, lse, dq, dk, dv


def test_two_threads_two_streams():
    dev = device()
    inputs = [_inputs(*p[:6], p[7], dev) for p in PROBLEMS]
    serial = [_step(*x, p[6]) for x, p in zip(inputs, PROBLEMS)]
    torch.cuda.synchronize()

    results = [[None] * ROUNDS for _ in PROBLEMS]
    errors = []
    streams = [torch.cuda.Stream() for _ in PROBLEMS]

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for r in range(ROUNDS):
                    results[i][r] = _step(*inputs[i], PROBLEMS[i][6])
            streams[i].synchronize()
        except Exception as e:          # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(PROBLEMS))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(len(PROBLEMS)):
        for r in range(ROUNDS):
            for got, want in zip(results[i][r], serial[i]):
                assert torch.equal(got, want), (i, r)
