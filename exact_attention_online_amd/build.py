"""Build libattn.so (gfx950 HIP kernels + the C ABI) in place with hipcc.

Run ``python -m exact_attention_online_amd.build`` (or ``__graft_entry__.build()``).  Every call
recompiles: each source is compiled to an object file in parallel, then the objects are linked
into one shared library, which lands next to this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
SOURCES = ["api.hip", "fwd.hip", "bwd.hip", "fp8.hip", "splitkv.hip", "clock.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 VALU instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    "-Wno-unused-command-line-argument",
]
NOISE = "packed-fp32-ops"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(x for x in (r.stdout + r.stderr).splitlines() if NOISE not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)


def build(verbose: bool = False, extra_flags=None, out: str | None = None) -> str:
    """Compile every source and link libattn.so (or `out`); returns the library path."""
    out = out or LIB
    cc = hipcc()
    flags = [*HIPCC_FLAGS, *(extra_flags or [])]
    with tempfile.TemporaryDirectory(prefix="eao_build_") as tmpdir:
        objs = [os.path.join(tmpdir, s.replace(".hip", ".o")) for s in SOURCES]
        cmds = [[cc, *flags, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        workers = max(1, min(len(cmds), os.cpu_count() or 1))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = out + ".tmp"
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
