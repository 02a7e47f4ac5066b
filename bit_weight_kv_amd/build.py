"""Build libfq.so (all HIP sources of the package) for gfx950 with hipcc.

Usage: python bit_weight_kv_amd/build.py   (or call build()).
Run as a script (not -m): importing the package loads the library itself.
The library is written next to this file so that it travels with the
source tree; nothing is installed elsewhere.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfq.so")
SOURCES = ["elementwise.hip", "quantize.hip", "gemm.hip", "attention.hip", "runtime.hip", "timing.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Packed fp32 arithmetic stays off for every kernel of this library.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division and square root (the quantiser's codes depend on it).
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-result",
]

# Per-source additions.  attention.hip: MFMA results in ordinary VGPRs -- the
# causal prefill kernel rescales and reads its accumulators with vector
# instructions every key chunk, and with the default accumulator registers
# every chunk moved them there and back (and the extra registers cost the
# second wave per SIMD).  gemm.hip keeps its inline-asm MFMAs on the
# accumulator registers.
SOURCE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source to an object (all in parallel), then link libfq.so."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = ([hipcc()] + [f for f in FLAGS if f != "-shared"] + SOURCE_FLAGS.get(src, []) + inc +
               ["-c", os.path.join(CSRC, src), "-o", obj])
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    errors = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        if p.returncode != 0:
            errors.append(f"--- {src} ---\n{out}")
        elif verbose and out.strip():
            print(out)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
