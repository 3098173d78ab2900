"""Build libbsa.so (gfx950) from csrc/*.hip with hipcc, in-tree.

Usage: python -m video_dit_block_cube_amd.build   (or call build()).
Every call recompiles; objects go to _build/ at the repository root, the shared library next to
this file so that it travels with the package.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libbsa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # never emit packed fp32 VALU ops (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]

# Per-file flags (LLVM AMDGPU options; every choice measured at the 720p-class shape, same bits):
#  * MINREG, LLVM's register-minimising scheduler: the head_dim 128 one-wave dQ then keeps its
#    score accumulators out of the AGPRs that hold dQ^T (about 2-3% faster).
#  * VGPR_MFMA, every MFMA writing architectural VGPRs.  Without it the compiler gives every MFMA
#    an AGPR destination once a kernel may use more than 256 registers, and each score element
#    then costs a v_accvgpr_read before its exponential.  The pipelined dQ (about 490 registers) loses
#    its 128 copies per tile with it (with MINREG: no spills; 2.5% faster); the head_dim 64 dQ
#    and dK/dV fit in 256 VGPRs with it (8% faster each).  The head_dim 128 dK/dV kernels already
#    use VGPRs only and compile to the same code; the head_dim 128 one-wave dQ was 2% slower with
#    it, so k_bwd_dq.hip does without.  With the option, a kernel that spills computed wrong
#    results, so it is only used where nothing spills (tests/test_build_no_spills.py): the
#    ragged-grid pipelined dQ, which would spill, has its own file built with MINREG only.
MINREG = ["-mllvm", "--amdgpu-sched-strategy=iterative-minreg"]
VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA_FLAGS = {
    "k_bwd_dq.hip": MINREG,
    "k_bwd_dq64.hip": VGPR_MFMA,
    "k_bwd_dq_pipe.hip": VGPR_MFMA + MINREG,
    "k_bwd_dq_pipe_ragged.hip": MINREG,
    "k_bwd_mfma.hip": VGPR_MFMA,
}


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build()
