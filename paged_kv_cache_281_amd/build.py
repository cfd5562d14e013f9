"""Build libpkv.so (HIP kernels for gfx950 + the C ABI + the host block manager).

Usage: ``python -m paged_kv_cache_281_amd.build`` or ``build()``.  Every call
recompiles; object files go to ``_build/`` next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpkv.so")
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpkv")


def _flags(debug: bool):
    f = [f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
         # no packed-fp32 instructions in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA accumulators in VGPRs: the online-softmax rescale works on them with VALU ops
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         # atomics exactly as written: the plan's counting atomics on one LDS word are
         # faster issued from every lane than turned into a lane-by-lane loop
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]
    f += ["-O1", "-g", "-DPKV_DEBUG=1"] if debug else ["-O3"]
    return f


# Flags of single sources.  The prefill kernel's scores are never NaN where they count
# (masked scores are selected to -inf, pool slots past a context are zeroed bitwise):
# without NaN semantics each fmaxf is one v_max (no canonicalising of its inputs), which
# cuts the softmax's VALU work on a path that is bound by VALU and MFMA issue.
FILE_FLAGS = {"paged_prefill.hip": ["-fno-honor-nans"]}


def build(debug: bool = False, jobs: int = 8, verbose: bool = False, extra_flags=(), out: str = None) -> str:
    """Compile every source under csrc/ and link libpkv.so (or ``out``); returns its path."""
    hipcc = _hipcc()
    tag = "debug" if debug else "release"
    if extra_flags:
        tag += "-" + str(abs(hash(tuple(extra_flags))))
    out_dir = os.path.join(HERE, "_build", tag)
    os.makedirs(out_dir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    flags = _flags(debug) + list(extra_flags)

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        cmd = [hipcc] + flags + FILE_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd = [hipcc] + flags + ["-x", "hip", "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        if verbose:
            print(res.stderr)
        return obj

    with cf.ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, sources))
    lib = out or (LIB if not debug else os.path.join(HERE, "libpkv_debug.so"))
    tmp = lib + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import sys
    print(build(debug="--debug" in sys.argv, verbose="-v" in sys.argv))
