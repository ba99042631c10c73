"""Writes fwd_tile.inc: the hand-scheduled key-tile step of the forward kernel for gfx950.

The step is the body of the online-softmax loop ("FlashAttention (NeurIPS 2022)" notes, sections
"Online Softmax" and "FlashAttention"): for one wave (32 query rows, d = 128) and one 64-key
tile it forms the probabilities of the tile against the row's running maximum, adds them to the
running denominator and accumulates O^T += V^T P^T, while the matrix cores already compute S^T
of the next tile.  It is emitted as two inline-asm blocks:

  part A  16 v_mfma_f32_32x32x16 for S^T = K Q^T of the NEXT tile (K fragments read from LDS with
          ds_read_b128), interleaved with the vector work of THIS tile: per score one fma
          (c s - m), one v_exp_f32, the row sums in four chains per lane, and v_cvt_pk to the
          16-bit B operand of part B;
  part B  16 v_mfma_f32_32x32x16 for O^T += V^T P^T (V^T fragments read with ds_read_b64_tr_b16).

The kernel decides between the two blocks whether a row's maximum has grown past the running
one (every probability of a lane is at most the lane's partial row sum, so a sum of at most 2^8
bounds them all); only then does it rescale and recompute the probabilities in C++.

Register use: the LDS operands of the MFMAs are read R MFMAs ahead into a ring of R fixed
4-register slots at the top of the register file, and the probabilities live in a pool of NP
fixed temporaries below it; both are declared clobbered, everything else is an asm operand.
Hazards that gfx950 does not interlock are respected by construction and checked by `check`:
an LDS result is waited for (s_waitcnt lgkmcnt, LDS operations complete in order) before its
MFMA; a v_exp_f32 result is read no earlier than one instruction later; a vector result read by
an MFMA is at least two instructions old; and every block ends at least TAIL wait states after
its last MFMA, so code after the block may read the MFMA results.

Run `python exact_attention_online_amd/csrc/gen_fwd_tile.py` to rewrite fwd_tile.inc; a CPU
test checks that the committed file matches this generator and passes `check`.
"""
import os
import re
import sys

D = 128                 # head dimension of the hand-scheduled step
KK = D // 16            # 16-wide k slices of S^T = K Q^T
DB = D // 32            # 32-row blocks of O^T
TILE_BYTES = 64 * D * 2  # one 64-key tile of 16-bit K or V in LDS
R = 4                   # LDS operand reads in flight ahead of their MFMA
NP = 12                 # probability temporaries
TAIL = 12               # wait states after a block's last MFMA (the distance the compiler
                        # keeps between a 32x32x16 MFMA and a vector read of its result)
RING = 256 - 4 * R      # first register of the operand ring
PT = RING - NP          # first probability temporary
# issue-cycle weights used to spread the vector work over the MFMA slots
COST = {"F": 4, "X": 8, "C": 4, "A": 4}
PRO_BUDGET = 64         # vector work placed before the first MFMA, while its operands load


def _ring(s, lo=0, n=4):
    return f"v[{RING + 4 * s + lo}:{RING + 4 * s + lo + n - 1}]"


def part_a(bf16, kpar):
    """Instruction list of part A for the K buffer of parity `kpar` (the next tile's)."""
    mf = "v_mfma_f32_32x32x16_" + ("bf16" if bf16 else "f16")
    cvt = "v_cvt_pk_bf16_f32" if bf16 else "v_cvt_pk_f16_f32"
    groups = [(kk, kb) for kk in range(KK) for kb in range(2)]   # one K fragment per MFMA

    # vector ops: F (fma) and X (exp) per score e = (kb, r), C (pack) per pair, A (sum) per term
    ops, order = {}, []

    def add(name, kind, deps, elem=None, reads=()):
        ops[name] = dict(kind=kind, deps=deps, elem=elem, reads=list(reads))
        order.append(name)

    for kb in range(2):
        for t in range(2):
            for w in range(4):
                r0 = 8 * t + 2 * w
                for r in (r0, r0 + 1):
                    add(f"F{kb}.{r}", "F", [], elem=(kb, r))
                    add(f"X{kb}.{r}", "X", [f"F{kb}.{r}"], elem=(kb, r))
                add(f"C{kb}.{t}.{w}", "C", [f"X{kb}.{r0}", f"X{kb}.{r0 + 1}"], reads=[(kb, r0), (kb, r0 + 1)])
    # chain j sums the scores r = j (mod 4): kb 0 then kb 1, r ascending (the C++ recompute path
    # adds in the same order, so both give the same bits)
    for j in range(4):
        terms = [(kb, j + 4 * q) for kb in range(2) for q in range(4)]
        prev = None
        for n in range(1, len(terms)):
            e = terms[n]
            if n == 1:
                deps, rd = [f"X{terms[0][0]}.{terms[0][1]}", f"X{e[0]}.{e[1]}"], [terms[0], e]
            else:
                deps, rd = [prev, f"X{e[0]}.{e[1]}"], [e]
            name = f"A{j}.{n}"
            add(name, "A", deps, reads=rd)
            ops[name]["chain"] = (j, n)
            prev = name
    readers = {}
    for nm in order:
        for e in ops[nm]["reads"]:
            readers.setdefault(e, []).append(nm)
    prio = {nm: i for i, nm in enumerate(order)}
    for nm in order:
        if ops[nm]["kind"] == "A":
            prio[nm] = max(prio[d] for d in ops[nm]["deps"]) + 0.5

    out, done, pos, lds = [], set(), {}, []
    free = list(range(NP))
    preg = {}

    def treg(e):
        return f"v{PT + preg[e]}"

    def text(nm):
        o = ops[nm]
        if o["kind"] == "F":
            kb, r = o["elem"]
            return f"v_fma_f32 {treg(o['elem'])}, %[c], %[s{kb}_{r}], -%[m]"
        if o["kind"] == "X":
            return f"v_exp_f32 {treg(o['elem'])}, {treg(o['elem'])}"
        if o["kind"] == "C":
            (kb, r0), e1 = o["reads"]
            return f"{cvt} %[pw{kb}{r0 // 8}{(r0 % 8) // 2}], {treg((kb, r0))}, {treg(e1)}"
        j, n = o["chain"]
        if n == 1:
            a, b = o["reads"]
            return f"v_add_f32 %[rs{j}], {treg(a)}, {treg(b)}"
        return f"v_add_f32 %[rs{j}], %[rs{j}], {treg(o['reads'][0])}"

    def ready(nm):
        o = ops[nm]
        if o["kind"] == "F" and not free:
            return False
        for d in o["deps"]:
            if d not in done or (d[0] == "X" and pos[d] == len(out) - 1):
                return False
        return True

    def place(nm):
        o = ops[nm]
        if o["kind"] == "F":
            preg[o["elem"]] = free.pop(0)
        out.append(text(nm))
        pos[nm] = len(out) - 1
        done.add(nm)
        for e in o["reads"]:
            if all(x in done for x in readers[e]):
                free.append(preg[e])

    def fill(budget):
        used = 0
        while True:
            cand = sorted((nm for nm in order if nm not in done and ready(nm)), key=lambda nm: prio[nm])
            if not cand:
                if len(done) < len(ops) and budget is None:
                    out.append("s_nop 0")       # only an exp result one instruction old blocks
                    continue
                return
            nm = cand[0]
            if budget is not None and used + COST[ops[nm]["kind"]] > budget:
                return
            place(nm)
            used += COST[ops[nm]["kind"]]

    def load(g):
        kk, kb = groups[g]
        lds.append(g)
        return f"ds_read_b128 {_ring(g % R)}, %[ka{kk}] offset:{kpar * TILE_BYTES + kb * 32 * D * 2}"

    for g in range(R):
        out.append(load(g))
    fill(PRO_BUDGET)
    per_slot = (sum(COST[ops[nm]["kind"]] for nm in order) - PRO_BUDGET) / len(groups)
    acc = 0.0
    for g, (kk, kb) in enumerate(groups):
        newer = len(lds) - 1 - max(i for i, x in enumerate(lds) if x == g)
        out.append(f"s_waitcnt lgkmcnt({newer})")
        src_c = "0" if kk == 0 else f"%[sn{kb}]"
        out.append(f"{mf} %[sn{kb}], {_ring(g % R)}, %[qf{kk}], {src_c}")
        if g + R < len(groups):
            out.append(load(g + R))
        if g + 1 < len(groups):
            acc += per_slot
            b = int(acc)
            acc -= b
            fill(b)
    fill(None)
    _pad_tail(out)
    assert len(done) == len(ops)
    return out


def part_b(bf16, vpar):
    """Instruction list of part B for the V buffer of parity `vpar` (this tile's)."""
    mf = "v_mfma_f32_32x32x16_" + ("bf16" if bf16 else "f16")
    groups = [(kb, t, db) for kb in range(2) for t in range(2) for db in range(DB)]
    out, lds = [], []

    def loads(g):
        kb, t, db = groups[g]
        off = (2 + vpar) * TILE_BYTES + (32 * kb + 16 * t) * D * 2
        lds.extend([g, g])
        return [f"ds_read_b64_tr_b16 {_ring(g % R, 0, 2)}, %[va{2 * db}] offset:{off}",
                f"ds_read_b64_tr_b16 {_ring(g % R, 2, 2)}, %[va{2 * db + 1}] offset:{off}"]

    for g in range(R):
        out.extend(loads(g))
    for g, (kb, t, db) in enumerate(groups):
        newer = len(lds) - 1 - max(i for i, x in enumerate(lds) if x == g)
        out.append(f"s_waitcnt lgkmcnt({newer})")
        out.append(f"{mf} %[o{db}], {_ring(g % R)}, %[pf{kb}{t}], %[o{db}]")
        if g + R < len(groups):
            out.extend(loads(g + R))
    _pad_tail(out)
    return out


def _pad_tail(out):
    last = max(i for i, x in enumerate(out) if x.startswith("v_mfma"))
    ws = sum(_wait_states(x) for x in out[last + 1:])
    while ws < TAIL:
        k = min(7, TAIL - ws - 1)
        out.append(f"s_nop {k}")
        ws += k + 1


def _wait_states(ins):
    m = re.match(r"s_nop (\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def check(lines):
    """Static checks of one block: the LDS read feeding each MFMA (the K or V^T fragment its
    operands name) has completed and not been overwritten (s_waitcnt lgkmcnt; LDS operations
    complete in order), exp results are not read by the next instruction, lgkmcnt stays within
    its field, nothing is left in flight, the first MFMA comes two wait states after the block
    starts (its operands may have been written by vector code just before) and the block ends
    TAIL wait states after its last MFMA.  Raises AssertionError on a violation."""
    pending = []            # (register, source) of LDS reads not yet known complete, oldest first
    done = {}               # register -> source of the completed read it holds
    for i, ins in enumerate(lines):
        srcs = ins.split(",", 1)[1] if "," in ins else ""
        if i and lines[i - 1].startswith("v_exp_f32"):
            dst = lines[i - 1].split()[1].rstrip(",")
            assert not re.search(re.escape(dst) + r"\b", srcs), f"exp result read one instruction later: {ins}"
        if ins.startswith("ds_read"):
            m = re.match(r"(ds_read\S*) (v\[\d+:\d+\]), (%\[\w+\]) offset:(\d+)", ins)
            reg, src = m.group(2), (m.group(3), int(m.group(4)))
            done.pop(reg, None)
            pending = [(r, x) for r, x in pending if r != reg] + [(reg, src)]
            assert len(pending) <= 15, "more LDS reads in flight than lgkmcnt counts"
        m = re.match(r"s_waitcnt lgkmcnt\((\d+)\)", ins)
        if m:
            k = int(m.group(1))
            assert k <= 15
            while len(pending) > k:
                r, x = pending.pop(0)
                done[r] = x
        if ins.startswith("v_mfma"):
            ops_ = [x.strip() for x in ins.split(None, 1)[1].split(",")]
            lo, hi = map(int, ops_[1][2:-1].split(":"))
            if ops_[0].startswith("%[sn"):          # S^T += K fragment (kk, kb) x Q^T slice kk
                kk, kb = int(ops_[2][4:-1]), int(ops_[0][4:-1])
                got = done.get(f"v[{lo}:{hi}]")
                assert got is not None and got[0] == f"%[ka{kk}]" and got[1] % TILE_BYTES == kb * 32 * D * 2, \
                    f"K fragment of {ins} not loaded and waited for"
            else:                                  # O^T += V^T fragment (kb, t, db) x P^T
                db = int(ops_[0][3:-1])
                kb, t = int(ops_[2][4]), int(ops_[2][5])
                for h, reg in enumerate((f"v[{lo}:{lo + 1}]", f"v[{lo + 2}:{hi}]")):
                    got = done.get(reg)
                    assert got is not None and got[0] == f"%[va{2 * db + h}]" and \
                        got[1] % TILE_BYTES == (32 * kb + 16 * t) * D * 2, f"V^T fragment of {ins} not ready"
    # a packed P^T operand written by vector code before the block is two instructions old at
    # the first MFMA at the latest
    first = min(i for i, x in enumerate(lines) if x.startswith("v_mfma"))
    assert sum(_wait_states(x) for x in lines[:first]) >= 2, "first MFMA too close to the block start"
    last = max(i for i, x in enumerate(lines) if x.startswith("v_mfma"))
    assert sum(_wait_states(x) for x in lines[last + 1:]) >= TAIL, "short tail after the last MFMA"
    assert not pending, "LDS reads left in flight at the end of the block"


def _render_a(name, bf16, kpar):
    lines = part_a(bf16, kpar)
    body = "\n".join(f'      "{x}\\n"' for x in lines)
    outs = ([f'[sn{kb}] "=&v"(sn[{kb}])' for kb in range(2)] +
            [f'[pw{kb}{t}{w}] "=&v"(pw[{kb}][{t}][{w}])' for kb in range(2) for t in range(2) for w in range(4)] +
            [f'[rs{j}] "=&v"(rs[{j}])' for j in range(4)])
    ins = ([f'[s{kb}_{r}] "v"(sc[{kb}][{r}])' for kb in range(2) for r in range(16)] +
           [f'[qf{kk}] "v"(qf[{kk}])' for kk in range(KK)] +
           [f'[ka{kk}] "v"(ka[{kk}])' for kk in range(KK)] + ['[c] "s"(c)', '[m] "v"(m)'])
    clob = ", ".join(f'"v{r}"' for r in range(PT, 256))
    return (f"__device__ __forceinline__ void {name}(const f32x16_t (&sc)[2], f32x16_t (&sn)[2], "
            f"uint32_t (&pw)[2][2][4],\n    const i16x8_t (&qf)[{KK}], const uint32_t (&ka)[{KK}], float c, float m, "
            f"float (&rs)[4]) {{\n  asm volatile(\n{body}\n      : {', '.join(outs)}\n      : {', '.join(ins)}\n"
            f"      : {clob});\n}}\n")


def _render_b(name, bf16, vpar):
    lines = part_b(bf16, vpar)
    body = "\n".join(f'      "{x}\\n"' for x in lines)
    outs = [f'[o{db}] "+v"(o[{db}])' for db in range(DB)]
    ins = ([f'[pf{kb}{t}] "v"(pf[{kb}][{t}])' for kb in range(2) for t in range(2)] +
           [f'[va{i}] "v"(va[{i}])' for i in range(2 * DB)])
    clob = ", ".join(f'"v{r}"' for r in range(RING, 256))
    return (f"__device__ __forceinline__ void {name}(f32x16_t (&o)[{DB}], const i16x8_t (&pf)[2][2], "
            f"const uint32_t (&va)[{2 * DB}]) {{\n  asm volatile(\n{body}\n      : {', '.join(outs)}\n"
            f"      : {', '.join(ins)}\n      : {clob});\n}}\n")


def blocks():
    """(name, instruction list) of every block fwd_tile.inc holds."""
    res = []
    for bf16 in (True, False):
        for par in (0, 1):
            tag = f"{'bf16' if bf16 else 'f16'}_p{par}"
            res.append((f"fwd_tile_a_{tag}", part_a(bf16, 1 - par)))
            res.append((f"fwd_tile_b_{tag}", part_b(bf16, par)))
    return res


def render():
    parts = ["// Generated by gen_fwd_tile.py (hand-scheduled key-tile step of the d = 128 forward",
             "// kernel); do not edit.  Part A of parity p computes S^T of the next tile from the K",
             "// buffer of parity 1 - p; part B accumulates O^T from the V buffer of parity p.", ""]
    for bf16 in (True, False):
        for par in (0, 1):
            tag = f"{'bf16' if bf16 else 'f16'}_p{par}"
            parts.append(_render_a(f"fwd_tile_a_{tag}", bf16, 1 - par))
            parts.append(_render_b(f"fwd_tile_b_{tag}", bf16, par))
    return "\n".join(parts)


OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fwd_tile.inc")

if __name__ == "__main__":
    for _, lines in blocks():
        check(lines)
    with open(OUT, "w") as f:
        f.write(render())
    print(OUT, file=sys.stderr)
