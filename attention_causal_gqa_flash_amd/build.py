"""Builds libattn.so for gfx950 in-tree with hipcc.

Each HIP source is compiled to an object in parallel, then linked into the
package directory, where the Python binding loads it.  Packed-FP32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# Sources whose MFMA accumulators the compiler may place in AGPRs: in the
# backward's d = 128 dK/dV kernel (one wave per SIMD, 512 registers) the dK and
# dV accumulators then sit in AGPRs, which frees enough VGPRs to keep eight LDS
# operand reads in flight (4096-token dK/dV kernel 321 -> 303 us); its d = 64
# kernels compile to the same code either way.
AGPR_FORM = ("attn_bwd_mfma.hip",)

# Sources compiled assuming no NaN operands (infinities are still honoured:
# masked scores are -inf): fmaxf on matrix-core results then needs no NaN
# canonicalisation, which in the forward's row maximum was 8 of its 18
# instructions per tile.  NaN inputs make NaN outputs either way.
NO_NAN = ("attn_fwd_mfma.hip",)


def compile_flags(src: str = "") -> list:
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    if os.path.basename(src) in NO_NAN:
        flags += ["-fno-honor-nans"]
    if os.path.basename(src) not in AGPR_FORM:
        # keep MFMA accumulators in VGPR form: with the AGPR form the score
        # accumulators, which the softmax reads, are copied from AGPRs to
        # VGPRs after every block, and the forward's split kernel runs slower
        flags += ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
    return flags + ["-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libattn.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    procs, objs = [], []
    for src in srcs:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [cc, *compile_flags(src), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature and says so
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append((src, "\n".join(lines)))
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        msg = "\n".join(f"--- {s}\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    # -z defs: an unresolved symbol (say a kernel launch stub the host pass did
    # not emit) fails the build here rather than the first load of the library
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
