"""Build libmoe.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m dispatch_expert_gemm_amd.build

compiles every csrc/*.hip with hipcc into lib/libmoe.so.  It always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmoe.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 adds/muls/fmas.
COMMON = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]
# Per-file extras: the gather-reduce kernels keep every product and sum
# separately rounded so their results match a plain left-to-right fp32 sum.
EXTRA = {"combine.hip": ["-ffp-contract=off"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "warning: feature flag" not in l
                    and l.strip() != "1 warning generated.")
    return p.returncode, out


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.join(LIBDIR, "obj"), exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in sources():
        obj = os.path.join(LIBDIR, "obj", src.replace(".hip", ".o"))
        cmd = [cc, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((src, obj, cmd))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(lambda j: (j, _run(j[2])), jobs))
    for (src, _, cmd), (rc, out) in results:
        if verbose and out.strip():
            print(out)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{out}")
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for _, o, _ in jobs], "-o", tmp]
    rc, out = _run(cmd)
    if rc != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
