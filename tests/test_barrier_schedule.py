"""Barrier schedule of the two-wave dK/dV kernel (D = 128), read from the gfx950 assembly that the
build flags produce.  The two waves of a workgroup run separate copies of the step loop (wave 0:
S, P, dV^T; wave 1: dP, dS, dK^T) over the same trip count, so each copy must execute the same
number of s_barrier per iteration, or the workgroup would wait forever.  The only barrier outside
the loops is the walk-phase broadcast, which both waves reach under one launch-uniform condition.
CPU only: hipcc cross-compiles for gfx950 without a GPU."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from video_dit_block_cube_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")


def _assembly(src: str) -> str:
    out = tempfile.mkdtemp()
    try:
        s = os.path.join(out, "k.s")
        subprocess.run([B.HIPCC, *B.FLAGS, *B.EXTRA_FLAGS.get(os.path.basename(src), []),
                        "--cuda-device-only", "-S", src, "-o", s], check=True,
                       capture_output=True, text=True)
        with open(s) as f:
            return f.read()
    finally:
        shutil.rmtree(out)


def _function(asm: str, symbol_prefix: str) -> list:
    start = asm.index("\n" + symbol_prefix)
    end = asm.index(".Lfunc_end", start)
    return asm[start:end].splitlines()


def _loops(lines: list) -> list:
    """(first, last) line of every loop: a 'Loop Header' label up to the last branch back to it."""
    loops = []
    for i, ln in enumerate(lines):
        m = re.match(r"^(\.LBB\w+):.*Loop Header", ln)
        if m:
            back = [j for j, l2 in enumerate(lines)
                    if j > i and re.search(r"\bs_c?branch\w*\s+" + re.escape(m.group(1)) + r"\b", l2)]
            if back:
                loops.append((i, max(back)))
    return loops


def _barriers(lines: list) -> int:
    return sum(1 for ln in lines if re.match(r"\s*s_barrier\b", ln))


def test_two_wave_dkdv_roles_meet_the_same_barriers():
    lines = _function(_assembly(os.path.join(B.CSRC, "k_bwd_mfma.hip")),
                      "_ZN3bsa20bwd_dkdv_pair_kernelILi128E")
    loops = _loops(lines)
    per_loop = [_barriers(lines[a:b + 1]) for a, b in loops]
    step_loops = [c for c in per_loop if c > 0]
    assert len(step_loops) == 2, per_loop                 # one step loop per role
    assert step_loops[0] == step_loops[1] >= 2, per_loop  # same barriers per iteration
    outside = _barriers(lines) - sum(step_loops)
    assert outside == 1, (outside, per_loop)              # the walk-phase broadcast only
