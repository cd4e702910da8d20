"""Build libfp4.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m mxfp4_block_amax_amd.build [-v] [--phase-clock]

--phase-clock builds libfp4_phase.so instead: the same library with the
one-pass NVFP4 kernel's phase clock compiled in (include/fp4_phase_clock.h),
a profiling aid read by mxfp4_block_amax_amd/phase_timeline.py.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfp4.so")
PHASE_LIB = os.path.join(HERE, "libfp4_phase.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["fp4_api.hip", "fp4_quant.hip", "fp4_gemm.hip"]

# -ffp-contract=off: no implicit fused multiply-add; the kernels spell every
# fused operation explicitly (the method's fp32 steps are separate roundings).
# fp32 division is the IEEE correctly rounded one (HIP's default, stated).
# Packed fp32 instructions are disabled (-packed-fp32-ops).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt", "-Wall", "-Xclang",
         "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, verbose: bool, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the gfx target feature; that warning is noise
    noise = ("packed-fp32-ops", "warning: feature flag", "1 warning generated", "2 warnings generated")
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    return obj


def build(verbose: bool = False, phase_clock: bool = False) -> str:
    build_dir = os.path.join(BUILD, "phase") if phase_clock else BUILD
    lib = PHASE_LIB if phase_clock else LIB
    extra = ("-DFP4_PHASE_CLOCK",) if phase_clock else ()
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phase_clock="--phase-clock" in sys.argv))
