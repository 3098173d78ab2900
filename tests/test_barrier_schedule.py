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


def _barriers_per_loop(lines: list) -> tuple:
    """s_barrier count of each loop (innermost, keyed by its header block) and outside every
    loop, from the assembler's block comments ('Loop Header' / 'in Loop: Header=...')."""
    per, outside, cur = {}, 0, None
    for ln in lines:
        label = re.match(r"^(\.LBB\w+|; %bb\.\d+):", ln)
        if label:
            m = re.search(r"in Loop: Header=(BB\w+)", ln)
            if "Loop Header" in ln:
                cur = label.group(1).lstrip(".L")
            elif m:
                cur = m.group(1)
            else:
                cur = None
            continue
        if re.match(r"\s*s_barrier\b", ln):
            if cur is None:
                outside += 1
            else:
                per[cur] = per.get(cur, 0) + 1
    return per, outside


def _barriers(lines: list) -> int:
    return sum(1 for ln in lines if re.match(r"\s*s_barrier\b", ln))


def test_two_wave_dkdv_roles_meet_the_same_barriers():
    lines = _function(_assembly(os.path.join(B.CSRC, "k_bwd_mfma.hip")),
                      "_ZN3bsa20bwd_dkdv_pair_kernelILi128E")
    per, outside = _barriers_per_loop(lines)
    counts = sorted(per.values())
    assert len(counts) == 2, per                  # one step loop per role
    assert counts[0] == counts[1] >= 2, per       # the same barriers per iteration
    assert outside == 1, (outside, per)           # the walk-phase broadcast only


def test_key_split_dkdv_waves_share_one_loop():
    """The split-by-keys dK/dV runs one loop for both waves: one loop with barriers, the
    walk-phase broadcast outside it."""
    lines = _function(_assembly(os.path.join(B.CSRC, "k_bwd_mfma.hip")),
                      "_ZN3bsa20bwd_dkdv_keys_kernelILi128E")
    per, outside = _barriers_per_loop(lines)
    assert len(per) == 1 and min(per.values()) >= 1, per
    assert outside == 1, (outside, per)
