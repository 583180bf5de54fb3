"""Build libnmsparse.so (all HIP sources, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libnmsparse.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["api.hip", "select.hip", "slide.hip", "gemm_dense.hip", "gemm_lds.hip", "gemm_sparse.hip",
           "gemm_lds_sp.hip", "hybrid_pack.hip", "spense.hip", "decode.hip", "pts.hip"]
# measurement helpers live in a library of their own (not exported by libnmsparse)
PROBE_SOURCES = ["probe.hip"]
PROBE_OUT = os.path.join(PKG, "libnmprobe.so")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
         # packed fp32 VALU forms stay off (code generation choice for this toolchain)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in p.stdout.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if p.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        out = _run([hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out:
            print(out)
        return obj

    psrcs = [s for s in PROBE_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, srcs + psrcs))
    for out, sel in ((OUT, objs[:len(srcs)]), (PROBE_OUT, objs[len(srcs):])):
        tmp = out + ".tmp"
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *sel])
        os.replace(tmp, out)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
