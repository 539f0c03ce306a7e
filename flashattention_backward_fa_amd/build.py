"""Build libfa_bwd.so in-tree for gfx950.

The host planner (csrc/fa_bwd_api.cpp) is plain C++ built with g++; the
kernels (csrc/fa_bwd_dkdv.h with csrc/fa_bwd_dkdv_kernels.hip and
csrc/fa_bwd_dkdv192_kernels.hip: the dK/dV kernel;
csrc/fa_bwd_det_kernels.hip: both dQ kernels and the partial-sum reduce;
csrc/fa_bwd_kernels.hip: preprocess and the atomic variants;
csrc/fa_bwd_fused_kernels.hip: the one-launch kernel for short key sequences;
csrc/fa_bwd_scratch.hip: the device scratch of the entry point that allocates nothing;
csrc/fa_bwd_f32_kernels.hip: the fp32 debugging form;
csrc/fa_fwd_kernels.hip: the forward that produces attn_out and
softmax_lse; csrc/fa_floyd_kernels.hip: Floyd attention, whose host side is
csrc/fa_floyd_api.cpp) are built with hipcc for gfx950 only; the objects are
linked into flashattention_backward_fa_amd/lib/libfa_bwd.so.

Usage: python -m flashattention_backward_fa_amd.build
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
BUILDDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(LIBDIR, "libfa_bwd.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of the generated code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# The default kernels are scheduled with LLVM's iterative ILP strategy:
# measured on MI355X it shortens the dK/dV kernel by 6-10 % and the D = 192
# dQ kernel by 20 % against the default occupancy-driven scheduler.
DET_FLAGS = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
# The dK/dV kernel, since its step loop holds two steps and forms its
# addresses by additions, is shorter under the iterative strategy that
# minimises register pressure (GQA -2.3 %, MHA -1.7 %, varlen -1.4 % against
# iterative ILP; the dQ GEMM is 1 % slower under it, so it keeps ILP).
DKDV_FLAGS = ["-mllvm", "-amdgpu-sched-strategy=iterative-minreg"]
# Its D = 192 instantiations (one wavefront per SIMD) under the iterative
# occupancy strategy: wide_qk -2.1 % against ILP, where minreg changes nothing.
DKDV192_FLAGS = ["-mllvm", "-amdgpu-sched-strategy=iterative-maxocc"]


def _hipcc():
    for cand in (os.path.join(ROCM, "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; set ROCM_PATH")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose=False):
    """Compile every source and link lib/libfa_bwd.so.  Always rebuilds."""
    os.makedirs(LIBDIR, exist_ok=True)
    os.makedirs(BUILDDIR, exist_ok=True)
    hipcc = _hipcc()
    api_o = os.path.join(BUILDDIR, "fa_bwd_api.o")
    ker_o = os.path.join(BUILDDIR, "fa_bwd_kernels.o")
    fwd_o = os.path.join(BUILDDIR, "fa_fwd_kernels.o")
    det_o = os.path.join(BUILDDIR, "fa_bwd_det_kernels.o")
    dkdv_o = os.path.join(BUILDDIR, "fa_bwd_dkdv_kernels.o")
    dkdv192_o = os.path.join(BUILDDIR, "fa_bwd_dkdv192_kernels.o")
    f32_o = os.path.join(BUILDDIR, "fa_bwd_f32_kernels.o")
    fus_o = os.path.join(BUILDDIR, "fa_bwd_fused_kernels.o")
    scr_o = os.path.join(BUILDDIR, "fa_bwd_scratch.o")
    fapi_o = os.path.join(BUILDDIR, "fa_floyd_api.o")
    fker_o = os.path.join(BUILDDIR, "fa_floyd_kernels.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC,
          "-c", os.path.join(CSRC, "fa_bwd_api.cpp"), "-o", api_o], verbose)
    _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "fa_bwd_kernels.hip"),
          "-o", ker_o], verbose)
    _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "fa_fwd_kernels.hip"),
          "-o", fwd_o], verbose)
    _run([hipcc, *HIP_FLAGS, *DET_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
          os.path.join(CSRC, "fa_bwd_det_kernels.hip"), "-o", det_o], verbose)
    _run([hipcc, *HIP_FLAGS, *DKDV_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
          os.path.join(CSRC, "fa_bwd_dkdv_kernels.hip"), "-o", dkdv_o], verbose)
    _run([hipcc, *HIP_FLAGS, *DKDV192_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
          os.path.join(CSRC, "fa_bwd_dkdv192_kernels.hip"), "-o", dkdv192_o], verbose)
    _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "fa_bwd_f32_kernels.hip"),
          "-o", f32_o], verbose)
    _run([hipcc, *HIP_FLAGS, *DET_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
          os.path.join(CSRC, "fa_bwd_fused_kernels.hip"), "-o", fus_o], verbose)
    _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "fa_bwd_scratch.hip"),
          "-o", scr_o], verbose)
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC,
          "-c", os.path.join(CSRC, "fa_floyd_api.cpp"), "-o", fapi_o], verbose)
    _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "fa_floyd_kernels.hip"),
          "-o", fker_o], verbose)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, api_o, ker_o, fwd_o, det_o, dkdv_o, dkdv192_o, f32_o, fus_o,
          scr_o, fapi_o, fker_o], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
