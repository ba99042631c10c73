"""The C-ABI library loads without a GPU, exports what include/attn.h declares, and rejects bad
arguments on the host before enqueuing anything (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import exact_attention_online_amd as eao

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

# fake, 256-byte aligned device addresses: every call below fails validation before using them
P = ctypes.c_void_p(0x7F0000001000)
NULL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = eao.load()
    names = declared_functions()
    assert set(names) == set(eao.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = eao.load()
    for code in range(6):
        assert lib.attn_status_string(code)
    assert b"scratch" in lib.attn_status_string(5)
    assert lib.attn_status_string(99) == b"unknown status"


def fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, N=64, d=128, causal=0, scale=0.1, dtype=1,
             qd=NULL, kd=NULL, vd=NULL)
    a.update(kw)
    return eao.load().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"],
                               a["causal"], a["scale"], a["dtype"], a["qd"], a["kd"], a["vd"], NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(o=ctypes.c_void_p(0x7F0000001002)), 1), (dict(N=0), 1), (dict(B=0), 1),
    (dict(Hq=3, Hkv=2), 1), (dict(Hkv=0), 1), (dict(scale=0.0), 1), (dict(scale=float("nan")), 1),
    (dict(scale=float("inf")), 1), (dict(scale=-1.0), 1), (dict(dtype=7), 1), (dict(d=96), 2), (dict(d=256), 2),
    (dict(qd=P), 1), (dict(dtype=2), 1), (dict(dtype=2, qd=P, kd=P, vd=P, d=64), 2),
])
def test_fwd_rejects_bad_arguments(kw, code):
    assert fwd(**kw) == code


def bwd(**kw):
    a = dict(B=1, Hq=2, Hkv=1, N=64, d=128, causal=1, scale=0.1, dtype=1, gdt=None, ws=P, wsb=1 << 40)
    a.update(kw)
    gdt = a["dtype"] if a["gdt"] is None else a["gdt"]
    ptrs = [a.get(n, P) for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")]
    return eao.load().attn_bwd(*ptrs, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"], a["scale"], a["dtype"],
                               gdt, a["ws"], a["wsb"], NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(dq=NULL), 1), (dict(lse=ctypes.c_void_p(0x7F0000001004)), 1), (dict(Hq=5, Hkv=2), 1), (dict(N=-3), 1),
    (dict(scale=0.0), 1), (dict(dtype=3), 1), (dict(dtype=2), 2), (dict(d=32), 2), (dict(ws=NULL), 3),
    (dict(ws=ctypes.c_void_p(0x7F0000001010)), 3), (dict(wsb=100), 3), (dict(N=1 << 23), 2),
    # gradients in the input dtype or float32 only
    (dict(gdt=0), 1), (dict(gdt=2), 1), (dict(gdt=4), 1), (dict(dtype=0, gdt=1), 1),
    (dict(gdt=3, dq=ctypes.c_void_p(0x7F0000001008)), 1),
])
def test_bwd_rejects_bad_arguments(kw, code):
    assert bwd(**kw) == code


def test_prep_rejects_bad_arguments():
    lib = eao.load()
    assert lib.attn_fp8_prep(NULL, P, P, NULL, 1, 1, 128, 128, 0, NULL) == 1
    assert lib.attn_fp8_prep(P, P, P, ctypes.c_void_p(0x7F0000001001), 1, 1, 128, 128, 0, NULL) == 1
    assert lib.attn_fp8_prep(P, P, P, NULL, 1, 1, 0, 128, 1, NULL) == 1
    assert lib.attn_fp8_prep(P, P, P, NULL, 1, 1, 128, 48, 0, NULL) == 2


def _dkdv_splits(B, Hq, Hkv, N):
    """Splits of the dK/dV phase as documented in attn.h."""
    wg = B * Hkv * -(-N // 128)
    if Hq // Hkv < 2 or wg >= 256:
        return 1
    return min(-(-512 // wg), 2 * (Hq // Hkv))


def test_workspace_is_linear_in_n():
    ws = eao.bwd_workspace_size
    sizes = [ws(2, 8, 2, n, 128) for n in (1024, 2048, 4096, 8192, 16384)]
    # per query row: -D and LSE * log2(e) (one float each)
    # -- never an N x N buffer; with few K/V heads and keys, the float dK/dV shares of a split
    # dK/dV phase (also linear in N)
    for n, s in zip((1024, 2048, 4096, 8192, 16384), sizes):
        rows = 2 * 8 * n
        split = _dkdv_splits(2, 8, 2, n)
        part = split * 2 * 2 * 2 * n * 128 * 4 if split > 1 else 0
        assert s == 2 * rows * 4 + part   # Hkv = 2
    assert _dkdv_splits(2, 8, 2, 1024) == 8 and _dkdv_splits(2, 8, 2, 16384) == 1
    # rows are padded to whole tiles of 64 (the shares cover the N rows themselves)
    assert ws(2, 8, 2, 16383, 128) == sizes[-1]
    assert ws(1, 1, 1, 65, 64) == 2 * 512
    assert ws(3, 1, 1, 1, 64) == 2 * 3 * 64 * 4
    assert ws(2, 8, 3, 1024, 128) == 0 and ws(1, 1, 1, 1, 80) == 0
    # variable-length batches never split the phase
    assert eao.bwd_varlen_workspace_size(2, 8, 2, 1024, 128) == 2 * 2 * 8 * 1024 * 4


def splitkv(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=8, Hkv=2, Nq=1, Nk=1000, d=128, causal=1, scale=0.1, dtype=1,
             splits=0, ws=NULL, wsb=0)
    a.update(kw)
    return eao.load().attn_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                                       a["Nk"], a["d"], a["causal"], a["scale"], a["dtype"], a["splits"], a["ws"],
                                       a["wsb"], NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(Nq=0), 1), (dict(Nq=1001), 1), (dict(splits=-1), 1), (dict(scale=0.0), 1),
    (dict(dtype=2), 2), (dict(d=80), 2), (dict(Hq=8, Hkv=1, Nq=5), 3), (dict(Hq=3, Hkv=2), 1),
    (dict(), 3), (dict(ws=P, wsb=16), 3),
])
def test_splitkv_rejects_bad_arguments(kw, code):
    assert splitkv(**kw) == code


def test_splitkv_workspace_size():
    ws = eao.splitkv_workspace_size
    # one split: partial O (float) and LSE of every row, each rounded up to 256 bytes
    assert ws(1, 8, 2, 1, 100, 128, 1) == 8 * 128 * 4 + 256
    # splits are clamped to the number of 128-key tiles and never empty
    assert ws(1, 8, 2, 1, 300, 128, 64) == ws(1, 8, 2, 1, 300, 128, 3)
    # 8 heads x 5 rows per K/V head: two groups of 32 rows, the same partial rows per split
    assert ws(1, 8, 1, 5, 100, 128, 1) == 8 * 5 * 128 * 4 + 256
    assert ws(1, 8, 1, 100, 99, 128, 0) == 0    # more query rows than keys


def test_fwd_ext_rejects_bad_arguments():
    lib = eao.load()
    ok = (P, P, P, P, P, 1, 2, 2, 100, 128, 1, 0.1, 1)
    assert lib.attn_fwd_ext(*ok, -1, NULL, NULL) == 1                       # negative window
    assert lib.attn_fwd_ext(*ok, 4, ctypes.c_void_p(0x7F0000001002), NULL) == 1   # misaligned slopes
    assert lib.attn_fwd_ext(P, P, P, P, P, 1, 2, 2, 100, 128, 1, 0.1, 2, 4, NULL, NULL) == 2   # fp8
    assert lib.attn_fwd_ext(P, P, P, P, P, 1, 2, 2, 100, 96, 1, 0.1, 1, 4, NULL, NULL) == 2    # head dim


def test_fwd_varlen_rejects_bad_arguments():
    lib = eao.load()
    a = [P, P, P, P, P, P, 3, 4, 2, 1000, 500, 128, 1, 0.1, 1, NULL]
    assert lib.attn_fwd_varlen(*a[:5], NULL, *a[6:]) == 1                    # no offsets
    bad = list(a); bad[10] = 1001                                            # max_seqlen > T
    assert lib.attn_fwd_varlen(*bad) == 1
    bad = list(a); bad[10] = 0
    assert lib.attn_fwd_varlen(*bad) == 1
    bad = list(a); bad[11] = 96                                              # head dim
    assert lib.attn_fwd_varlen(*bad) == 2
    bad = list(a); bad[14] = 2                                               # fp8
    assert lib.attn_fwd_varlen(*bad) == 2


def test_bwd_varlen_rejects_bad_arguments():
    lib = eao.load()
    # q, k, v, o, dout, lse, dq, dk, dv, cu, B, Hq, Hkv, T, max_seqlen, d, causal, scale, dtype, grad dtype,
    # ws, bytes, stream
    need = lib.attn_bwd_varlen_workspace_size(3, 4, 2, 500, 128)
    assert 0 < need < lib.attn_bwd_workspace_size(3, 4, 2, 500, 128)    # the dense size adds split shares
    assert need == lib.attn_bwd_workspace_size(3, 4, 4, 500, 128)    # Hkv = 4: no split
    a = [P] * 10 + [3, 4, 2, 1000, 500, 128, 1, 0.1, 1, 1, P, need, NULL]
    bad = list(a); bad[9] = NULL                                             # no offsets
    assert lib.attn_bwd_varlen(*bad) == 1
    bad = list(a); bad[14] = 1001                                            # max_seqlen > T
    assert lib.attn_bwd_varlen(*bad) == 1
    bad = list(a); bad[15] = 96                                              # head dim
    assert lib.attn_bwd_varlen(*bad) == 2
    bad = list(a); bad[18] = 2                                               # fp8
    assert lib.attn_bwd_varlen(*bad) == 2
    bad = list(a); bad[19] = 0                                               # fp16 gradients of bf16 inputs
    assert lib.attn_bwd_varlen(*bad) == 1
    bad = list(a); bad[21] = need - 1                                        # workspace too small
    assert lib.attn_bwd_varlen(*bad) == 3
    bad = list(a); bad[20] = NULL                                            # no workspace
    assert lib.attn_bwd_varlen(*bad) == 3
    bad = list(a); bad[12] = 3                                               # Hq % Hkv != 0
    assert lib.attn_bwd_varlen(*bad) != 0
    assert lib.attn_bwd_varlen_workspace_size(3, 4, 2, 0, 128) == 0


def test_bwd_ext_rejects_bad_arguments():
    lib = eao.load()
    need = lib.attn_bwd_workspace_size(1, 2, 2, 100, 128)
    # q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, dtype, grad dtype, window, slopes, ws,
    # bytes, stream
    a = [P] * 9 + [1, 2, 2, 100, 128, 1, 0.1, 1, 3, 4, NULL, P, need, NULL]
    bad = list(a); bad[18] = -1                                              # negative window
    assert lib.attn_bwd_ext(*bad) == 1
    bad = list(a); bad[19] = ctypes.c_void_p(0x7F0000001002)                 # misaligned slopes
    assert lib.attn_bwd_ext(*bad) == 1
    bad = list(a); bad[16] = 2                                               # fp8
    assert lib.attn_bwd_ext(*bad) == 2
    bad = list(a); bad[17] = 2                                               # fp8 gradients
    assert lib.attn_bwd_ext(*bad) == 1
    bad = list(a); bad[13] = 96                                              # head dim
    assert lib.attn_bwd_ext(*bad) == 2
    bad = list(a); bad[21] = need - 1                                        # workspace too small
    assert lib.attn_bwd_ext(*bad) == 3


def test_clock_probe_rejects_bad_arguments():
    lib = eao.load()
    assert lib.attn_clock_probe(NULL, 8, 1000, NULL) == 1
    assert lib.attn_clock_probe(ctypes.c_void_p(0x7F0000001008), 8, 1000, NULL) == 1   # misaligned
    assert lib.attn_clock_probe(P, 0, 1000, NULL) == 1
    assert lib.attn_clock_probe(P, 1025, 1000, NULL) == 1
    assert lib.attn_clock_probe(P, 8, 0, NULL) == 1
    assert lib.attn_clock_probe(P, 8, 10 ** 9 + 1, NULL) == 1


def test_mfma_probe_rejects_bad_arguments():
    lib = eao.load()
    BF, F8 = 1, 2
    assert lib.attn_mfma_probe(NULL, 8192, P, 1, 1, BF, NULL) == 1
    assert lib.attn_mfma_probe(P, 8192, NULL, 1, 1, BF, NULL) == 1
    assert lib.attn_mfma_probe(ctypes.c_void_p(0x7F0000001008), 8192, P, 1, 1, BF, NULL) == 1   # misaligned
    assert lib.attn_mfma_probe(P, 8184, P, 1, 1, BF, NULL) == 1          # fewer than 8192 values
    assert lib.attn_mfma_probe(P, 8196, P, 1, 1, BF, NULL) == 1          # not a multiple of 8
    assert lib.attn_mfma_probe(P, 8192 + 16, P, 1, 1, F8, NULL) == 1     # fp8: not a multiple of 32
    assert lib.attn_mfma_probe(P, 8192, P, 0, 1, BF, NULL) == 1
    assert lib.attn_mfma_probe(P, 8192, P, 65537, 1, BF, NULL) == 1
    assert lib.attn_mfma_probe(P, 8192, P, 1, 0, F8, NULL) == 1
    assert lib.attn_mfma_probe(P, 8192, P, 1, (1 << 20) + 1, BF, NULL) == 1
    assert lib.attn_mfma_probe(P, 8192, P, 1, 1, 0, NULL) == 2           # fp16: not offered


def test_hbm_probe_rejects_bad_arguments():
    lib = eao.load()
    assert lib.attn_hbm_probe(NULL, 16384, P, 1, NULL) == 1
    assert lib.attn_hbm_probe(P, 16384, NULL, 1, NULL) == 1
    assert lib.attn_hbm_probe(ctypes.c_void_p(0x7F0000001008), 16384, P, 1, NULL) == 1   # misaligned
    assert lib.attn_hbm_probe(P, 0, P, 1, NULL) == 1
    assert lib.attn_hbm_probe(P, 16384 * 3 + 1024, P, 3, NULL) == 1      # not whole 16 KB stages
    assert lib.attn_hbm_probe(P, 16384 * 4, P, 3, NULL) == 1             # groups do not divide it
    assert lib.attn_hbm_probe(P, 16384, P, 0, NULL) == 1
    assert lib.attn_hbm_probe(P, 16384 * 65537, P, 65537, NULL) == 1
    assert lib.attn_hbm_probe(P, (1 << 32), P, 1, NULL) == 1             # share past 2^31


def test_splitkv_noalloc_rejects_on_the_host():
    """The allocation-free split-KV entry point checks its arguments, and that the problem's
    partials fit its static scratch, before any HIP call (so without a GPU too)."""
    lib = eao.load()
    ok = [P, P, P, P, P, 1, 8, 2, 1, 1000, 128, 1, 0.1, 1, 0, NULL]
    bad = list(ok); bad[0] = NULL
    assert lib.attn_fwd_splitkv_noalloc(*bad) == 1
    bad = list(ok); bad[8] = 1001                                        # Nq > Nk
    assert lib.attn_fwd_splitkv_noalloc(*bad) == 1
    bad = list(ok); bad[13] = 2                                          # fp8
    assert lib.attn_fwd_splitkv_noalloc(*bad) == 2
    # 16 x 64 heads x 64 rows, 32k keys: far more partials than 8 MiB
    big = [P, P, P, P, P, 16, 64, 64, 64, 32768, 128, 1, 0.1, 1, 0, NULL]
    assert lib.attn_fwd_splitkv_workspace_size(16, 64, 64, 64, 32768, 128, 0) > (8 << 20)
    assert lib.attn_fwd_splitkv_noalloc(*big) == 5
