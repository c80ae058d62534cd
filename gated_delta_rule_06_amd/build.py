"""Build libkda.so (the HIP library behind include/kda.h) for gfx950, in-tree.

    python -m gated_delta_rule_06_amd.build

compiles every ``csrc/*.hip`` with hipcc (one object per source under
``_build/kda``, in parallel) and links them into ``gated_delta_rule_06_amd/libkda.so``.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkda.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep hipcc from forming packed fp32 instructions by itself
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the KDA library needs ROCm's hipcc to build")


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(x for x in res.stderr.splitlines() if "packed-fp32-ops" not in x)
    return res.returncode, err


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile all HIP sources into libkda.so (always recompiles): one object
    per source, compiled in parallel, then one link."""
    from concurrent.futures import ThreadPoolExecutor

    srcs = sources()
    objdir = os.path.join(ROOT, "_build", "kda")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    cflags = [f for f in HIPCC_FLAGS if f != "-shared"] + list(extra_flags or [])
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[hipcc(), *cflags, *inc, "-c", "-o", o, s] for s, o in zip(srcs, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    errs = [e for rc, e in results if rc != 0]
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    tmp = LIB + ".tmp%d" % os.getpid()
    link = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    rc, err = _run(link)
    if rc != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc link failed:\n" + err)
    for _, e in results:
        if verbose and e.strip():
            print(e, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
