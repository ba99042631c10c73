"""Host-side behaviour without a GPU: the binding refuses to run without the built library and
rejects host tensors before any library call; bench.py refuses more than one GPU and fails
loudly (no CPU fallback) where no GPU is visible."""
import os
import subprocess
import sys

import pytest
import torch

import exact_attention_online_amd as eao

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_missing_library_raises(monkeypatch):
    monkeypatch.setattr(eao, "_lib", None)
    monkeypatch.setattr(eao, "library_path", lambda: os.path.join(ROOT, "no-such-dir", "libattn.so"))
    with pytest.raises(eao.AttnError, match="missing"):
        eao.load()


def test_host_tensors_are_rejected_before_any_call(monkeypatch):
    # a library stand-in that fails the test if anything reaches it
    class Trap:
        def __getattr__(self, name):
            raise AssertionError(f"library function {name} reached with host tensors")

    monkeypatch.setattr(eao, "_lib", Trap())
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(eao.AttnError, match="device"):
        eao.fwd(q, q, q)
    with pytest.raises(eao.AttnError):
        eao.bwd(q, q, q, q, q, torch.zeros(1, 2, 8))
    with pytest.raises(eao.AttnError):
        eao.fwd_varlen(q[0], q[0], q[0], torch.tensor([0, 8], dtype=torch.int32), 8)
    with pytest.raises(eao.AttnError):
        eao.fp8_prep(torch.zeros(1, 2, 8, 128))
    # the measurement aids: host tensors, and operand types the MFMA probe does not take
    with pytest.raises(eao.AttnError, match="device"):
        eao.mfma_probe(torch.zeros(8192, dtype=torch.bfloat16), torch.zeros(512), 1)
    with pytest.raises(eao.AttnError, match="bf16 values or uint8"):
        eao.mfma_probe(torch.zeros(8192, dtype=torch.float16), torch.zeros(512), 1)
    with pytest.raises(eao.AttnError, match="device"):
        eao.hbm_probe(torch.zeros(4096, dtype=torch.int32), torch.zeros(64, dtype=torch.int32))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, env=env, cwd=ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the behaviour where no GPU is visible")
def test_bench_fails_loudly_without_a_gpu():
    r = _bench("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode != 0
    assert "no GPU visible" in r.stderr
    assert '"value"' not in r.stdout


def test_bench_result_check_flags_a_planted_error():
    """bench.py's result check: the oracle's own outputs pass; one planted error past a bar fails."""
    import numpy as np

    sys.path.insert(0, ROOT)
    import bench
    from attn_inputs import WORKLOADS

    w = WORKLOADS["gqa_bf16"].with_(B=1, Hq=4, Hkv=2, N=8)
    rng = np.random.default_rng(0)
    G = w.Hq // w.Hkv
    outs = {1: (rng.standard_normal((1, G, 8, 128)), rng.standard_normal((1, G, 8)),
                rng.standard_normal((1, G, 8, 128)), rng.standard_normal((1, 1, 8, 128)),
                rng.standard_normal((1, 1, 8, 128)))}
    full = [torch.zeros(1, 4, 8, 128, dtype=torch.float64), torch.zeros(1, 4, 8, dtype=torch.float64),
            torch.zeros(1, 4, 8, 128, dtype=torch.float64), torch.zeros(1, 2, 8, 128, dtype=torch.float64),
            torch.zeros(1, 2, 8, 128, dtype=torch.float64)]
    for t, r, grouped in zip(full, outs[1], (True, True, True, False, False)):
        sl = slice(G, 2 * G) if grouped else slice(1, 2)
        t[:, sl] = torch.from_numpy(r)
    rep = bench.check_results(w, full, outs)
    assert rep["pass"] and all(v == 0.0 for v in rep["max_abs"].values())
    full[3][0, 1, 5, 7] += 0.05          # dK past its 3e-2 bar
    rep = bench.check_results(w, full, outs)
    assert not rep["pass"] and rep["max_abs"]["dK"] > 0.03
