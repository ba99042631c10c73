"""The hand-scheduled forward tile step (csrc/fwd_tile.inc) against its generator and the
static schedule checks (LDS results waited for before their MFMA, exp results not read by the
next instruction, ring slots not overwritten early, the tail after the last MFMA).  CPU only."""
import importlib.util
import os
import re

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "exact_attention_online_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_fwd_tile", os.path.join(CSRC, "gen_fwd_tile.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_committed_include_matches_generator():
    g = _gen()
    with open(os.path.join(CSRC, "fwd_tile.inc")) as f:
        assert f.read() == g.render()


def test_every_block_passes_the_schedule_checks():
    g = _gen()
    names = []
    for name, lines in g.blocks():
        g.check(lines)
        names.append(name)
    assert len(names) == 8


def test_block_contents():
    """Part A: 16 S MFMAs, 32 fma + 32 exp, 16 packs, 28 sum adds, 16 K reads; part B: 16 P.V
    MFMAs and 32 transposed V reads; the K reads come from the other parity's buffer."""
    g = _gen()
    blk = dict(g.blocks())
    for bf in ("bf16", "f16"):
        for par in (0, 1):
            a = blk[f"fwd_tile_a_{bf}_p{par}"]
            b = blk[f"fwd_tile_b_{bf}_p{par}"]
            count = lambda lines, pre: sum(1 for x in lines if x.startswith(pre))
            assert count(a, "v_mfma_f32_32x32x16_" + bf) == 16
            assert count(a, "v_fma_f32") == 32 and count(a, "v_exp_f32") == 32
            assert count(a, "v_cvt_pk_" + bf + "_f32") == 16 and count(a, "v_add_f32") == 28
            assert count(a, "ds_read_b128") == 16
            assert count(b, "v_mfma_f32_32x32x16_" + bf) == 16 and count(b, "ds_read_b64_tr_b16") == 32
            koffs = {int(m) for x in a for m in re.findall(r"offset:(\d+)", x)}
            assert koffs == {(1 - par) * g.TILE_BYTES, (1 - par) * g.TILE_BYTES + 32 * g.D * 2}
            voffs = {int(m) for x in b for m in re.findall(r"offset:(\d+)", x)}
            assert min(voffs) == (2 + par) * g.TILE_BYTES and max(voffs) < (3 + par) * g.TILE_BYTES
            # every probability is summed exactly once per chain term and packed exactly once
            temps = [x for x in a if x.startswith("v_fma_f32")]
            assert len({x.split(",")[2] for x in temps}) == 32


def _mutants():
    g = _gen()
    blk = dict(g.blocks())
    a, b = blk["fwd_tile_a_bf16_p0"], blk["fwd_tile_b_bf16_p0"]
    out = {}
    i = next(i for i, x in enumerate(a) if x.startswith("s_waitcnt") and i > 10)
    out["dropped wait"] = a[:i] + a[i + 1:]
    i = next(i for i, x in enumerate(b) if x.startswith("s_waitcnt lgkmcnt(") and i > 10)
    out["weaker wait"] = b[:i] + [re.sub(r"\((\d+)\)", lambda m: f"({int(m.group(1)) + 2})", b[i])] + b[i + 1:]
    j = next(i for i, x in enumerate(a) if x.startswith("v_exp_f32"))
    reg = a[j].split()[1].rstrip(",")
    out["exp read at once"] = a[:j + 1] + [f"v_add_f32 v0, {reg}, v1"] + a[j + 1:]
    out["short tail"] = [x for x in b if not x.startswith("s_nop")]
    # a ring slot reloaded before the MFMA that reads its previous contents
    k = next(i for i, x in enumerate(a) if x.startswith("v_mfma") and i > 20)
    ld = next(i for i in range(k + 1, len(a)) if a[i].startswith("ds_read"))
    out["slot overwritten early"] = a[:k - 1] + [a[ld]] + a[k - 1:ld] + a[ld + 1:]
    return g, out


@pytest.mark.parametrize("kind", ["dropped wait", "weaker wait", "exp read at once", "short tail",
                                  "slot overwritten early"])
def test_checks_catch_planted_mistakes(kind):
    g, mutants = _mutants()
    with pytest.raises(AssertionError):
        g.check(mutants[kind])
