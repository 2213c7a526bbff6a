"""Build libkvq.so (HIP, gfx950 only) in-tree with hipcc.

Usage: python -m decode_attention_int2_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "quantize.hip", "decode.hip", "decode_mfma.hip", "wo_mfma.hip", "candidate.hip", "reference_mfma.hip", "windows.hip", "fold.hip", "optr.hip"]
# -packed-fp32-ops: no v_pk_*_f32 instructions; denormals kept; IEEE fp32 division.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
         # matrix-core results and accumulators in ordinary VGPRs (no AGPR copies)
         "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form",
         # every atomic here is issued by one lane (block claims, arrivals):
         # no wave-wide rewrite, whose immediate wait on the returned value
         # would also wait for the scalar loads in flight
         "-Xarch_device", "-mllvm=-amdgpu-atomic-optimizer-strategy=None",
         # loops whose branches are all wave-uniform keep their exits: a
         # restructured exit path back to the loop head makes the wait
         # insertion assume the newest loads feed the first step (the decode
         # loop would then drain its loads in flight once per iteration)
         "-Xarch_device", "-mllvm=-structurizecfg-skip-uniform-regions=true",
         "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


PHASES_LIB = os.path.join(PKG, "libkvq_phases.so")


def build(verbose: bool = False, lib: str = LIB, build_dir: str = BUILD, host_flags=(), defines=()) -> str:
    """Compile every source and link lib.  host_flags are passed to the host
    compilation only (each behind -Xarch_host), e.g. the sanitizers of the
    host-side validation test; defines (-D...) to both compilations, e.g.
    KVQ_PHASE_TIMESTAMPS for the diagnostic phase-timestamp library."""
    os.makedirs(build_dir, exist_ok=True)
    extra = [f for fl in host_flags for f in ("-Xarch_host", fl)] + [f"-D{d}" for d in defines]
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp, *extra]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    if "--phase-timestamps" in sys.argv[1:]:
        # the diagnostic library of phase_profile.py (timestamps at the decode
        # kernel's phase boundaries); libkvq.so is not touched
        build(verbose=True, lib=PHASES_LIB, build_dir=BUILD + "_phases", defines=("KVQ_PHASE_TIMESTAMPS",))
    else:
        build(verbose=True)
    sys.exit(0)
