#!/usr/bin/env python3
"""Benchmark: exact attention fwd+bwd on one MI355X, B=1, H=16, N=16384, d=128, bf16, causal.

One step = one forward (attn_fwd) and one backward (attn_bwd's three phases) over the same
seeded synthetic inputs, already resident in HBM.  FLOP convention: forward 4*B*H*N^2*d, halved
for causal; backward 2.5x forward (five N^2*d contractions including the recomputation of S);
fwd+bwd TFLOP/s = 3.5 * F_fwd / (time of a step).

The gradients are written in float32 (the form the contract checks read).  Prints one JSON line.
Besides the headline value it carries:
  * roofline: the dominant kernel (the backward dK/dV kernel), its algorithmic FLOPs per launch
    divided by its average launch time measured here with stream events, against the MI355X
    dense bf16 MFMA peak; `traffic` is the HBM bytes per launch from the committed rocprofv3
    counter summary, reported only while the kernel source still matches the one profiled;
  * cpu_baseline: the fp64 CPU oracle timed on a bounded sample of the same workload;
  * errors: the GPU's outputs of the sampled K/V head groups against the oracle's (max-abs,
    tolerances, pass); the run exits non-zero when a tolerance is missed;
  * clock: the mean engine clock while the timed steps run (a probe kernel beside the same steps
    repeated right after the timed region) and the fraction of the dense bf16 peak at that clock;
  * mfma_ceiling: the dense bf16 MFMA rate this machine sustains with no memory traffic at all, on
    random N(0,1) operands (the kind of data the step multiplies) and on zero operands, each
    with its clock, and the step's rates as fractions of the random-operand rate (the matrix
    cores' power, and with it the clock, depends on the bits multiplied).
The split-KV decoding legs (`--workload decode_bf16`, `decode4_bf16`) report K/V bytes per second
instead, with `hbm_ceiling`: the HBM read rate this machine sustains in the decoding kernel's own
load pattern with no compute, and the decoding rates as fractions of it.  The fp8 leg
(`--workload fp8`) carries its own `mfma_ceiling`: the fp8 MFMA rate on the workload's prepared
codes and on zero codes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6          # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
METRIC = "attention fwd / fwd+bwd TFLOPs/s (bf16, N=16k, d=128) + % of MFMA peak"
WORKLOAD = "long_bf16"
SEED = 3
# An idle GPU's engine clock ramps up over roughly the first 0.1 s of load: a workload whose step
# takes well under a millisecond needs hundreds of warm-up steps before its steady rate shows.
WARMUP_SECONDS = 0.25
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_dkdv_long_bf16_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_online_amd", "csrc", f) for f in ("bwd.hip", "common.hpp")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 3, and as many as fill %.1f s of GPU time)"
                         % WARMUP_SECONDS)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=[WORKLOAD, "gqa_bf16", "ablation_bf16", "decode_bf16", "decode4_bf16", "window_alibi_bf16",
                             "window_alibi_fwdbwd_bf16", "fp8", "varlen_bf16", "varlen_fwdbwd_bf16"],
                    help="the headline fwd+bwd workload (default); the grouped-query fwd+bwd workload; the "
                         "B=8 N=2048 forward, causal and not; split-KV decoding; the long shape with a 4096-key "
                         "sliding window and ALiBi; fp8; packed variable-length sequences")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the warmup, run one plain device-to-device copy of MIB MiB (a kernel of "
                         "known traffic that scales HBM byte counters read under a profiler)")
    return ap.parse_args()


def warm_up(step, args) -> int:
    """Run the untimed warm-up and return how many steps it took: args.warmup steps when given,
    else at least 3 and as many more as fill WARMUP_SECONDS of GPU time (batches of doubling
    size, each followed by a synchronisation)."""
    import torch

    if args.warmup is not None:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        return args.warmup
    n, batch = 0, 3
    t0 = time.perf_counter()
    while True:
        for _ in range(batch):
            step()
        n += batch
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= WARMUP_SECONDS:
            return n
        batch = min(2 * batch, 128)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter summary, or None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip().lstrip("-* ").strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _host_cores():
    try:
        import threadpoolctl

        return max(int(i.get("num_threads", 1)) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(w, q, k, v, do, target_s):
    """The fp64 oracle (as it stands) on whole K/V head groups of the workload (all their query
    heads, every batch entry) until target_s has passed.  Returns the JSON record and the oracle's
    outputs per group, {g: (O, LSE, dQ, dK, dV)}, for the result check."""
    from oracle import attention as A

    G = w.Hq // w.Hkv
    f_group = G * 4.0 * w.B * w.N * w.N * w.d / (2 if w.causal else 1)   # G query heads, every batch entry
    t0 = time.perf_counter()
    outs = {}
    for g in range(w.Hkv):
        hs = slice(g * G, (g + 1) * G)
        qg, kg, vg, dog = q[:, hs], k[:, g:g + 1], v[:, g:g + 1], do[:, hs]
        o, lse = A.forward(qg, kg, vg, w.causal, w.scale, row_block=1024)
        dq, dk, dv = A.backward(qg, kg, vg, dog, w.causal, w.scale, row_block=1024)
        outs[g] = (o, lse, dq, dk, dv)
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    rec = {
        "value": round(3.5 * f_group * len(outs) / el / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": _host_cores(),
        "kind": "oracle",
        "sample": f"fp64 forward + backward of {len(outs)} of {w.Hkv} K/V head groups ({len(outs) * G} of {w.Hq} "
                  f"query heads, all {w.B} batch entries) of the same workload, {el:.1f} s; rate counted with the "
                  f"GPU's FLOP convention",
    }
    return rec, outs


# Tolerances (max-abs over every compared element) for unit-normal bf16 inputs: O 1.5e-2, the
# float32 gradients 3e-2; LSE (float32 statistics) 1e-3.
BAR = {"O": 1.5e-2, "LSE": 1e-3, "dQ": 3e-2, "dK": 3e-2, "dV": 3e-2}


def check_results(w, gpu, outs):
    """Max-abs error of the GPU's last-step outputs against the oracle's for the groups the CPU
    leg computed; `gpu` = (O, LSE, dQ, dK, dV) device tensors."""
    import numpy as np

    G = w.Hq // w.Hkv
    err = {k: 0.0 for k in BAR}
    for g, ref in outs.items():
        hs = slice(g * G, (g + 1) * G)
        for name, t, r in zip(BAR, gpu, ref):
            part = t[:, hs] if name in ("O", "LSE", "dQ") else t[:, g:g + 1]
            e = float(np.abs(part.detach().double().cpu().numpy() - r).max())
            err[name] = max(err[name], e)
    ok = all(err[k] <= BAR[k] for k in BAR)
    return {"max_abs": {k: float(f"{v:.3e}") for k, v in err.items()}, "tolerance": BAR, "pass": ok,
            "compared": f"every output of K/V head groups {sorted(outs)} (query heads "
                        f"{sorted(h for g in outs for h in range(g * G, (g + 1) * G))}), last timed step"}


def clock_window(step, steps, ms_total):
    """Engine clock while the timed steps run: the same `steps` steps are run again (untimed)
    with attn_clock_probe on a second stream beside them, one sleeping single-wave workgroup per
    XCD for the length of the timed region.  A probe inside the timed region itself would hold a
    wave slot on 8 compute units, which kernels at 256 registers per wave cannot share."""
    import torch

    import exact_attention_online_amd as eao

    dev = torch.device("cuda", torch.cuda.current_device())
    out = torch.zeros(16, dtype=torch.int64, device=dev)
    side = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    eao.clock_probe(out, max(1, int(ms_total * 1e5)), stream=side)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    cyc = out.view(8, 2).double().cpu()
    ghz = (0.1 * cyc[:, 0] / cyc[:, 1]).tolist()
    return sum(ghz) / len(ghz), ghz


def mfma_ceiling(dev, rates):
    """Attainable dense bf16 MFMA rate on this machine (attn_mfma_probe: back-to-back MFMAs, two waves
    per SIMD, no memory traffic) on random N(0,1) operands, the values the bench feeds the
    kernels, and on zero operands; the engine clock of each (attn_clock_probe beside a second
    run); and each named rate as a fraction of the random-operand ceiling.  The matrix cores
    draw power according to the bits they multiply and the clock follows the power limit, so
    the spec peak (2.4 GHz) is out of reach on random data."""
    import torch

    import exact_attention_online_amd as eao

    gen = torch.Generator(device=dev).manual_seed(SEED)
    res = {}
    for name, data in (("random", torch.randn(1 << 23, generator=gen, device=dev).to(torch.bfloat16)),
                       ("zero", torch.zeros(1 << 23, dtype=torch.bfloat16, device=dev))):
        out = torch.empty(512 * 1024, dtype=torch.float32, device=dev)
        iters = 4000                     # about 20 ms per launch
        eao.mfma_probe(data, out, iters)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = sum(eao.mfma_probe(data, out, iters) for _ in range(3))
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        clk = torch.zeros(16, dtype=torch.int64, device=dev)
        side = torch.cuda.Stream(device=dev)
        torch.cuda.synchronize()
        eao.clock_probe(clk, max(1, int(ms * 1e5)), stream=side)
        for _ in range(3):
            eao.mfma_probe(data, out, iters)
        torch.cuda.synchronize()
        cyc = clk.view(8, 2).double().cpu()
        res[name] = (flops / (ms * 1e-3) / 1e12, float((0.1 * cyc[:, 0] / cyc[:, 1]).mean()))
    return {"random_operands_tflops": round(res["random"][0], 1), "random_operands_clock_ghz": round(res["random"][1], 3),
            "zero_operands_tflops": round(res["zero"][0], 1), "zero_operands_clock_ghz": round(res["zero"][1], 3),
            "frac_of_random_ceiling": {k: round(v / res["random"][0], 4) for k, v in rates.items()},
            "source": "attn_mfma_probe: 1024 workgroups x 8 waves x 32 x 4000 v_mfma_f32_32x32x16_bf16 on 2^23 "
                      "operand values, 3 launches timed with events"}


def clock_record(ghz, per_xcd, rates):
    """{mean GHz, per-XCD GHz, fraction of the dense bf16 peak at that clock for each named rate}."""
    peak = 256 * 4096 * ghz / 1000.0          # dense bf16 MFMA flop/clk of the chip x clock
    return {"ghz": round(ghz, 3), "per_xcd_ghz": [round(x, 3) for x in per_xcd],
            "peak_at_clock_tflops": round(peak, 1),
            "frac_of_peak_at_clock": {k: round(v / peak, 4) for k, v in rates.items()},
            "source": "attn_clock_probe (engine clocks / 100 MHz real-time ticks, one workgroup per XCD) on a "
                      "second stream while the timed steps are repeated right after the timed region"}


def cpu_baseline_decode(w, q, k, v, target_s):
    """The fp64 decoding oracle (as it stands) on whole (batch, K/V head) groups until target_s."""
    from oracle import decode as DC

    cores = _host_cores()
    G = w.Hq // w.Hkv
    t0 = time.perf_counter()
    groups = 0
    for b in range(w.B):
        for g in range(w.Hkv):
            DC.forward(q[b:b + 1, g * G:(g + 1) * G], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], w.causal, w.scale)
            groups += 1
            if time.perf_counter() - t0 >= target_s:
                break
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    kv_group = 2 * w.Nk * w.d * 2
    return {
        "value": round(kv_group * groups / el / 1e9, 6),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"fp64 forward of {groups} of {w.B * w.Hkv} (batch, K/V head) groups of the same workload "
                  f"({G * w.Nq} query rows each), {el:.1f} s; rate counted as K+V bytes of the bf16 cache",
    }


def hbm_ceiling(dev, rates):
    """Attainable HBM read rate on this machine in the decoding kernel's pattern (attn_hbm_probe:
    one-wave workgroups streaming 16 KB stages through a four-slot LDS ring with direct loads, no
    compute) over a 1 GiB buffer, with 512 and 1024 workgroups, and each named rate as a
    fraction of the better of the two.  The spec figure of 8 TB/s is not reached by reads."""
    import torch

    import exact_attention_online_amd as eao

    gen = torch.Generator(device=dev).manual_seed(SEED)
    data = torch.randint(-(1 << 31), (1 << 31) - 1, ((1 << 30) // 4,), dtype=torch.int32, device=dev, generator=gen)
    res = {}
    for groups in (512, 1024):
        out = torch.empty(64 * groups, dtype=torch.int32, device=dev)
        for _ in range(3):
            eao.hbm_probe(data, out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        nbytes = sum(eao.hbm_probe(data, out) for _ in range(10))
        e1.record()
        torch.cuda.synchronize()
        res[groups] = nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del data
    best = max(res.values())
    return {"stream_read_gbps": round(best, 1), "by_groups_gbps": {str(k): round(v, 1) for k, v in res.items()},
            "frac_of_stream_read": {k: round(v / best, 4) for k, v in rates.items()},
            "source": "attn_hbm_probe: 1 GiB read in 16 KB stages by 512 or 1024 one-wave workgroups, "
                      "10 launches timed with events"}


def bench_decode(args):
    """Split-KV decoding: K/V bytes streamed per second by attn_fwd_splitkv (split + merge kernels)."""
    import torch

    import exact_attention_online_amd as eao
    from attn_inputs import DECODE_WORKLOADS, draw_decode, round_to

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    eao.load()
    w = DECODE_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    q32, k32, v32 = draw_decode(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, SEED)
    qc, kc, vc = (round_to(x, w.dtype) for x in (q32, k32, v32))
    del q32, k32, v32
    q, k, v = (t.to(dev).contiguous() for t in (qc, kc, vc))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(eao.splitkv_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, 0), dtype=torch.uint8,
                     device=dev)
    nwarm = warm_up(lambda: eao.fwd_splitkv(q, k, v, w.causal, w.scale, 0, ws, o, lse), args)
    steps = max(args.steps, 50)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        evs[i][0].record()
        eao.fwd_splitkv(q, k, v, w.causal, w.scale, 0, ws, o, lse)
        evs[i][1].record()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    ms_call = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    if not torch.isfinite(o).all():
        print("non-finite output", file=sys.stderr)
        sys.exit(1)
    # the same call captured once in a HIP graph and replayed back to back, as a decoding loop
    # would launch it: no Python or launch gaps between the steps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        eao.fwd_splitkv(q, k, v, w.causal, w.scale, 0, ws, o, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        eao.fwd_splitkv(q, k, v, w.causal, w.scale, 0, ws, o, lse)
    graph.replay()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_graph = t0.elapsed_time(t1) / steps
    kv_bytes = 2.0 * w.B * w.Hkv * w.Nk * w.d * 2
    algo = kv_bytes + 2.0 * (2 * w.B * w.Hq * w.Nq * w.d) + 4.0 * w.B * w.Hq * w.Nq   # + Q read, O written, LSE
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    out = {
        "metric": "split-KV decoding: K/V cache GB/s streamed by attn_fwd_splitkv",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": nwarm,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d} "
                               f"causal={w.causal} fwd (split-KV)", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": w.causal, "seed": SEED, "pass": "fwd"},
        "roofline": {
            "kernel": "fwd_split_kernel<bf16, d=128> + fwd_split_merge_kernel (one attn_fwd_splitkv call)",
            "bound": "hbm",
            "achieved": round(algo / (ms_call * 1e-3) / 1e9, 1),
            "peak": 8000.0,
            "unit": "GB/s",
            "frac": round(algo / (ms_call * 1e-3) / 1e9 / 8000.0, 4),
            "traffic": None,
        },
    }
    out["graph_replay"] = {"ms_per_step": round(ms_graph, 5), "value": round(kv_bytes / (ms_graph * 1e-3) / 1e9, 1),
                           "unit": "GB/s"}
    out["hbm_ceiling"] = hbm_ceiling(dev, {"two_kernels": out["roofline"]["achieved"], "call": value,
                                           "graph_replay": out["graph_replay"]["value"]})
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w, qc, kc, vc, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def bench_window(args, with_bwd=False):
    """Forward (with_bwd: forward + backward) of the long shape (B=1, H=16, N=16384, d=128, bf16,
    causal) with a 4096-key sliding window and ALiBi slopes 2^(-8 h / H): TFLOP/s over the visible
    query-key pairs (4 d flops per pair forward, 10 d backward)."""
    import numpy as np
    import torch

    import exact_attention_online_amd as eao
    from attn_inputs import WORKLOADS, draw, round_to

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    eao.load()
    w = WORKLOADS[WORKLOAD]
    window = 4096
    dev = torch.device("cuda:0")
    _, q32, k32, v32, _ = draw(w.B, w.Hq, w.Hkv, w.N, w.d, SEED)
    q, k, v = (round_to(x, w.dtype).to(dev).contiguous() for x in (q32, k32, v32))
    del q32, k32, v32
    slopes = torch.tensor(2.0 ** (-8.0 * np.arange(1, w.Hq + 1) / w.Hq), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    if with_bwd:
        g = np.random.Generator(np.random.PCG64(SEED + 1))
        do = round_to(g.standard_normal(tuple(q.shape), dtype=np.float32), w.dtype).to(dev).contiguous()
        ws = torch.empty(eao.bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d), dtype=torch.uint8, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        eao.fwd_ext(q, k, v, True, w.scale, window, slopes, o, lse)
        if evs is not None:
            evs[1].record()
        if with_bwd:
            eao.bwd_ext(q, k, v, o, do, lse, True, w.scale, window, slopes, ws, dq, dk, dv)
            if evs is not None:
                evs[2].record()

    nwarm = warm_up(step, args)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    ms_call = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    ms_bwd = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps if with_bwd else 0.0
    if not torch.isfinite(o).all() or (with_bwd and not all(torch.isfinite(x).all() for x in (dq, dk, dv))):
        print("non-finite output", file=sys.stderr)
        sys.exit(1)
    pairs = sum(min(i + 1, window) for i in range(w.N))          # visible (query, key) pairs per head
    flops = 4.0 * w.B * w.Hq * pairs * w.d
    total = flops * (3.5 if with_bwd else 1.0)
    out = {
        "metric": (f"attention {'fwd+bwd' if with_bwd else 'fwd'} TFLOPs/s with a 4096-key sliding window and "
                   "ALiBi (visible pairs)"),
        "value": round(total / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: B={w.B} H={w.Hq} N={w.N} d={w.d} causal, window {window}, "
                               f"ALiBi slopes 2^(-8h/H), {'fwd+bwd' if with_bwd else 'fwd'}", "B": w.B, "Hq": w.Hq,
                   "N": w.N, "d": w.d, "window": window, "alibi": True, "seed": SEED,
                   "pass": "fwd+bwd" if with_bwd else "fwd"},
        "kernel_ms": {"fwd_ext": round(ms_call, 4), **({"bwd_ext": round(ms_bwd, 4)} if with_bwd else {})},
        "roofline": {
            "kernel": "attn_fwd_kernel<bf16, d=128, causal, window/ALiBi>",
            "bound": "mfma",
            "achieved": round(flops / (ms_call * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(flops / (ms_call * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
        },
    }
    print(json.dumps(out), flush=True)


def bench_ablation(args):
    """Forward of the B=8, H=16, N=2048, d=128 bf16 shape, causal and non-causal (4 d flops per
    query-key pair, halved for causal): value = both forwards' flops over both forwards' time.
    The small batch x heads setting (B=1, causal) is reported beside it as `small_batch`."""
    import torch

    import exact_attention_online_amd as eao
    from attn_inputs import WORKLOADS, draw, round_to

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    eao.load()
    w = WORKLOADS["ablation_bf16"]
    dev = torch.device("cuda:0")
    _, q32, k32, v32, _ = draw(w.B, w.Hq, w.Hkv, w.N, w.d, SEED)
    q, k, v = (round_to(x, w.dtype).to(dev).contiguous() for x in (q32, k32, v32))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    res = {}
    # a call takes about 0.2 ms, comparable with the binding's per-call checks, so the timed loop
    # calls the C ABI with the arguments marshalled once (the binding checked them in the warmup)
    import ctypes

    lib = eao.load()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nwarm = 0
    for causal in (True, False):
        nwarm += warm_up(lambda: eao.fwd(q, k, v, causal=causal, scale=w.scale, out=o, lse=lse), args)
        call_args = (P(q), P(k), P(v), P(o), P(lse), w.B, w.Hq, w.Hkv, w.N, w.d, int(causal), w.scale, eao.BF16,
                     None, None, None, stream)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            if lib.attn_fwd(*call_args) != 0:
                print("attn_fwd failed", file=sys.stderr)
                sys.exit(1)
        t1.record()
        torch.cuda.synchronize()
        if not torch.isfinite(o).all():
            print("non-finite output", file=sys.stderr)
            sys.exit(1)
        ms = t0.elapsed_time(t1) / args.steps
        flops = 4.0 * w.B * w.Hq * w.N * w.N * w.d / (2 if causal else 1)
        res["causal" if causal else "noncausal"] = (ms, flops)
    tot_ms = sum(v[0] for v in res.values())
    tot_f = sum(v[1] for v in res.values())
    tf = {kk: v[1] / (v[0] * 1e-3) / 1e12 for kk, v in res.items()}
    # the pages' second ablation setting, small batch x heads (B=1, H=16, same N, d, causal),
    # timed the same way beside the first; not part of value
    _, s32, t32, u32, _ = draw(1, w.Hq, w.Hkv, w.N, w.d, SEED)
    sq, sk, sv = (round_to(x, w.dtype).to(dev).contiguous() for x in (s32, t32, u32))
    so = torch.empty_like(sq)
    slse = torch.empty((1, w.Hq, w.N), dtype=torch.float32, device=dev)
    nwarm += warm_up(lambda: eao.fwd(sq, sk, sv, causal=True, scale=w.scale, out=so, lse=slse), args)
    small_args = (P(sq), P(sk), P(sv), P(so), P(slse), 1, w.Hq, w.Hkv, w.N, w.d, 1, w.scale, eao.BF16, None, None,
                  None, stream)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        if lib.attn_fwd(*small_args) != 0:
            print("attn_fwd failed", file=sys.stderr)
            sys.exit(1)
    t1.record()
    torch.cuda.synchronize()
    if not torch.isfinite(so).all():
        print("non-finite output", file=sys.stderr)
        sys.exit(1)
    small_ms = t0.elapsed_time(t1) / args.steps
    small_tf = 4.0 * w.Hq * w.N * w.N * w.d / 2 / (small_ms * 1e-3) / 1e12
    out = {
        "metric": "attention fwd TFLOPs/s (bf16, B=8 H=16 N=2048 d=128, causal and non-causal)",
        "value": round(tot_f / (tot_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(tot_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"ablation_bf16: B={w.B} H={w.Hq} N={w.N} d={w.d} fwd, causal and non-causal",
                   "B": w.B, "Hq": w.Hq, "N": w.N, "d": w.d, "seed": SEED, "pass": "fwd"},
        "kernel_ms": {kk: round(v[0], 4) for kk, v in res.items()},
        "kernel_tflops": {kk: round(v, 2) for kk, v in tf.items()},
        "small_batch": {"config": f"B=1 H={w.Hq} N={w.N} d={w.d} causal fwd", "ms": round(small_ms, 4),
                        "tflops": round(small_tf, 2)},
        "roofline": {
            "kernel": "attn_fwd_kernel<bf16, d=128, causal and non-causal>",
            "bound": "mfma",
            "achieved": round(tot_f / (tot_ms * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tot_f / (tot_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
        },
    }
    print(json.dumps(out), flush=True)


def bench_fp8(args):
    """FP8 forward (B=4, H=16, N=4096, d=128, non-causal, e4m3 with per-128-row scales, V's rounded
    up to powers of two): TFLOP/s of attn_fwd on prepared codes, against the dense fp8 MFMA peak;
    the preparation (Hadamard + quantisation, HBM-bound) is timed separately and not counted."""
    import torch

    import exact_attention_online_amd as eao
    from attn_inputs import WORKLOADS, draw_fp8

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    eao.load()
    w = WORKLOADS["fp8"]
    dev = torch.device("cuda:0")
    q, k, v, signs = draw_fp8(w.B, w.Hq, w.N, w.d, SEED)
    tq, tk, tv = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    ts = torch.from_numpy(signs).to(dev)

    def prep():
        return (eao.fp8_prep(tq, ts), eao.fp8_prep(tk, ts), eao.fp8_prep(tv, None, pow2_scale=True))

    (q8, qs), (k8, ks), (v8, vs) = prep()
    o = torch.empty(w.B, w.Hq, w.N, w.d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(w.B, w.Hq, w.N, dtype=torch.float32, device=dev)
    nwarm = warm_up(lambda: eao.fwd_fp8(q8, k8, v8, qs, ks, vs, w.causal, w.scale, o, lse), args)
    nwarm += warm_up(prep, args)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        evs[i][0].record()
        eao.fwd_fp8(q8, k8, v8, qs, ks, vs, w.causal, w.scale, o, lse)
        evs[i][1].record()
    t1.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        evs[i][2].record()
        prep()
        evs[i][3].record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    ms_call = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    ms_prep = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    if not torch.isfinite(o.float()).all():
        print("non-finite output", file=sys.stderr)
        sys.exit(1)
    f_fwd = 4.0 * w.B * w.Hq * w.N * w.N * w.d / (2 if w.causal else 1)
    prep_bytes = 3 * w.B * w.Hq * w.N * w.d * (4 + 1) + 3 * w.B * w.Hq * (w.N // 128) * 4
    out = {
        "metric": "fp8 attention fwd TFLOPs/s (e4m3, block scales + Hadamard)",
        "value": round(f_fwd / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": f"fp8: B={w.B} H={w.Hq} N={w.N} d={w.d} non-causal, 0.1% outliers x10, e4m3 per "
                               f"128 rows (V scales powers of two), Hadamard on Q and K", "B": w.B, "Hq": w.Hq, "N": w.N, "d": w.d,
                   "causal": w.causal, "seed": SEED, "pass": "fwd"},
        "prep_ms": round(ms_prep, 4),
        "prep_gbps": round(prep_bytes / (ms_prep * 1e-3) / 1e9, 1),
        "roofline": {
            "kernel": "fwd_fp8_kernel<non-causal>",
            "bound": "mfma",
            "achieved": round(f_fwd / (ms_call * 1e-3) / 1e12, 2),
            "peak": 5033.2,
            "unit": "TFLOP/s",
            "frac": round(f_fwd / (ms_call * 1e-3) / 1e12 / 5033.2, 4),
            "traffic": None,
        },
    }
    out["mfma_ceiling"] = fp8_mfma_ceiling(dev, k8, {"fwd_fp8": out["roofline"]["achieved"]})
    print(json.dumps(out), flush=True)


def fp8_mfma_ceiling(dev, codes, rates):
    """Attainable dense fp8 MFMA rate on this machine (attn_mfma_probe in its e4m3 mode: back-to-back
    v_mfma_scale_f32_32x32x64_f8f6f4, two waves per SIMD, no memory traffic) on the workload's own
    prepared K codes and on zero codes, and each named rate as a fraction of the first."""
    import torch

    import exact_attention_online_amd as eao

    res = {}
    flat = codes.reshape(-1)
    for name, data in (("workload_codes", flat[: (flat.numel() // 32) * 32]),
                       ("zero", torch.zeros(1 << 20, dtype=torch.uint8, device=dev))):
        out = torch.empty(512 * 1024, dtype=torch.float32, device=dev)
        iters = 2000
        eao.mfma_probe(data, out, iters)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = sum(eao.mfma_probe(data, out, iters) for _ in range(3))
        e1.record()
        torch.cuda.synchronize()
        res[name] = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    return {"workload_codes_tflops": round(res["workload_codes"], 1), "zero_codes_tflops": round(res["zero"], 1),
            "frac_of_workload_ceiling": {k: round(v / res["workload_codes"], 4) for k, v in rates.items()},
            "source": "attn_mfma_probe (e4m3): 1024 workgroups x 8 waves x 32 x 2000 "
                      "v_mfma_scale_f32_32x32x64_f8f6f4, 3 launches timed with events"}


def bench_varlen(args, with_bwd=False):
    """Forward (with_bwd: forward + backward) over 16 causal sequences packed without padding,
    lengths uniform in [128, 8192] (seed 3), H=16, d=128, bf16: TFLOP/s with 4 d flops per
    query-key pair for the forward and 10 d for the backward, halved for causal."""
    import numpy as np
    import torch

    import exact_attention_online_amd as eao
    from attn_inputs import draw_varlen, round_to, varlen_lengths

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    eao.load()
    H, d = 16, 128
    lens = varlen_lengths(16, 128, 8192, seed=SEED)
    q32, k32, v32, cu = draw_varlen(lens, H, H, d, SEED)
    dev = torch.device("cuda:0")
    q, k, v = (round_to(x, "bf16").to(dev).contiguous() for x in (q32, k32, v32))
    del q32, k32, v32
    tcu = torch.from_numpy(cu).to(dev)
    T, ms_len = int(cu[-1]), int(lens.max())
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    if with_bwd:
        g = np.random.Generator(np.random.PCG64(SEED + 1))
        do = round_to(g.standard_normal(q.shape, dtype=np.float32), "bf16").to(dev).contiguous()
        ws = torch.empty(eao.bwd_varlen_workspace_size(1 * len(lens), H, H, ms_len, d), dtype=torch.uint8,
                         device=dev)
        dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        eao.fwd_varlen(q, k, v, tcu, ms_len, True, None, o, lse)
        if evs is not None:
            evs[1].record()
        if with_bwd:
            eao.bwd_varlen(q, k, v, o, do, lse, tcu, ms_len, True, None, ws, dq, dk, dv)
            if evs is not None:
                evs[2].record()

    nwarm = warm_up(step, args)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    ms_call = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    ms_bwd = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps if with_bwd else 0.0
    if not torch.isfinite(o).all() or (with_bwd and not all(torch.isfinite(x).all() for x in (dq, dk, dv))):
        print("non-finite output", file=sys.stderr)
        sys.exit(1)
    flops = 4.0 * H * d * float((lens.astype(float) ** 2).sum()) / 2
    total = flops * (3.5 if with_bwd else 1.0)
    out = {
        "metric": ("attention fwd+bwd TFLOPs/s over packed variable-length causal sequences" if with_bwd else
                   "attention fwd TFLOPs/s over packed variable-length causal sequences"),
        "value": round(total / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: 16 sequences, lengths uniform in [128, 8192] (T={T}, longest "
                               f"{ms_len}), H={H} d={d} causal {'fwd+bwd' if with_bwd else 'fwd'}", "H": H, "d": d,
                   "T": T, "lengths": lens.tolist(), "seed": SEED, "pass": "fwd+bwd" if with_bwd else "fwd"},
        "kernel_ms": {"fwd_varlen": round(ms_call, 4), **({"bwd_varlen": round(ms_bwd, 4)} if with_bwd else {})},
        "roofline": {
            "kernel": "attn_fwd_kernel<bf16, d=128, causal, varlen>",
            "bound": "mfma",
            "achieved": round(flops / (ms_call * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(flops / (ms_call * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
        },
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the multi-GPU sharding is described in the design notes, not run.", file=sys.stderr)
        sys.exit(2)

    if args.workload in ("varlen_bf16", "varlen_fwdbwd_bf16"):
        bench_varlen(args, with_bwd=args.workload == "varlen_fwdbwd_bf16")
        return
    if args.workload == "fp8":
        bench_fp8(args)
        return
    if args.workload in ("window_alibi_bf16", "window_alibi_fwdbwd_bf16"):
        bench_window(args, with_bwd=args.workload == "window_alibi_fwdbwd_bf16")
        return
    if args.workload == "ablation_bf16":
        bench_ablation(args)
        return
    if args.workload not in (WORKLOAD, "gqa_bf16"):
        bench_decode(args)
        return

    import torch

    import exact_attention_online_amd as eao
    from attn_inputs import WORKLOADS, draw, round_to

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    eao.load()
    wname = args.workload
    w = WORKLOADS[wname]
    dev = torch.device("cuda:0")
    _, q32, k32, v32, do32 = draw(w.B, w.Hq, w.Hkv, w.N, w.d, SEED, with_grad=True)
    qc, kc, vc, doc = (round_to(x, w.dtype) for x in (q32, k32, v32, do32))
    del q32, k32, v32, do32
    q, k, v, do = (t.to(dev).contiguous() for t in (qc, kc, vc, doc))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    ws = torch.empty(eao.bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d), dtype=torch.uint8, device=dev)
    # gradients in float32, as the contract checks read them (a group sum can pass 8, where half a
    # bf16 step exceeds the 3e-2 bar)
    f32 = torch.float32
    dq, dk, dv = torch.empty_like(q, dtype=f32), torch.empty_like(k, dtype=f32), torch.empty_like(v, dtype=f32)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        eao.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
        if ev is not None:
            ev[1].record()
        hook = (lambda i: ev[1 + i].record() if i in (1, 2, 3) else None) if ev is not None else None
        eao.bwd_phases(q, k, v, o, do, lse, w.causal, w.scale, ws, dq, dk, dv, between=hook)

    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy calibration: {args.copy_calibration} MiB read + {args.copy_calibration} MiB written",
              file=sys.stderr, flush=True)
        del src, dst

    nwarm = warm_up(step, args)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    clk_ghz, clk_xcd = clock_window(step, args.steps, total_ms)
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    dkdv_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    dq_ms = sum(e[3].elapsed_time(e[4]) for e in evs) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[4]) for e in evs) / args.steps
    for t in (o, lse, dq, dk, dv):
        if not torch.isfinite(t).all():
            print("non-finite output", file=sys.stderr)
            sys.exit(1)

    f_fwd = 4.0 * w.B * w.Hq * w.N * w.N * w.d / (2 if w.causal else 1)
    ms_step = total_ms / args.steps
    value = 3.5 * f_fwd / (ms_step * 1e-3) / 1e12
    # the dK/dV kernel does four of the backward's contractions (S, dP, dV, dK): 2.0 x F_fwd;
    # the dQ kernel three (S, dP, dQ: 1.5 x F_fwd), two of them recomputations
    dkdv_tflops = 2.0 * f_fwd / (dkdv_ms * 1e-3) / 1e12
    dq_tflops = 1.5 * f_fwd / (dq_ms * 1e-3) / 1e12
    traffic = committed_traffic() if wname == WORKLOAD else None   # counters taken on the long workload
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wname}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal fwd+bwd",
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "causal": w.causal,
                   "seed": SEED, "pass": "fwd+bwd"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "grad_dtype": "fp32",
        "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
        "fwd_frac_of_peak": round(f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "bwd_tflops": round(2.5 * f_fwd / (bwd_ms * 1e-3) / 1e12, 2),
        "kernel_ms": {"attn_fwd": round(fwd_ms, 4), "bwd_dkdv": round(dkdv_ms, 4), "bwd_dq": round(dq_ms, 4),
                      "bwd_total": round(bwd_ms, 4)},
        "kernel_tflops": {"attn_fwd": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2), "bwd_dkdv": round(dkdv_tflops, 2),
                          "bwd_dq": round(dq_tflops, 2)},
        "roofline": {
            "kernel": "bwd_dkdv_kernel<bf16, d=128, causal>",
            "bound": "mfma",
            "achieved": round(dkdv_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dkdv_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    out["clock"] = clock_record(clk_ghz, clk_xcd, {"fwd+bwd": value, "fwd": f_fwd / (fwd_ms * 1e-3) / 1e12,
                                                    "bwd_dkdv": dkdv_tflops})
    out["mfma_ceiling"] = mfma_ceiling(dev, {"fwd+bwd": value, "fwd": f_fwd / (fwd_ms * 1e-3) / 1e12,
                                             "bwd_dkdv": dkdv_tflops})
    failed = False
    if not args.no_cpu_baseline:
        out["cpu_baseline"], outs = cpu_baseline(w, qc, kc, vc, doc, args.cpu_seconds)
        out["errors"] = check_results(w, (o, lse, dq, dk, dv), outs)
        failed = not out["errors"]["pass"]
    print(json.dumps(out), flush=True)
    if failed:
        print(f"result check failed: {out['errors']['max_abs']} against {BAR}", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
