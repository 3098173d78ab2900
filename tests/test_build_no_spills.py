"""Every kernel of a file built with every MFMA writing architectural VGPRs (LLVM's
-amdgpu-mfma-vgpr-form, per-file flags of build.py) must run without scratch memory.  With that
option, a pipelined dQ instantiation that spilled four registers outside its loop computed wrong
gradients (half of the queries off by up to a third of the largest value, against the same
source built without the option, which matched the plain loop bit for bit), so the option is kept
only where the register allocation needs no spill slot.  Read from the gfx950 assembly the build
flags produce; CPU only: hipcc cross-compiles for gfx950 without a GPU."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from video_dit_block_cube_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")

VGPR_FORM_FILES = sorted(f for f, flags in B.EXTRA_FLAGS.items()
                         if "-amdgpu-mfma-vgpr-form" in flags)


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


def test_some_files_use_the_option():
    assert VGPR_FORM_FILES, "no file is built with -amdgpu-mfma-vgpr-form"


@pytest.mark.parametrize("name", VGPR_FORM_FILES)
def test_vgpr_form_kernels_use_no_scratch(name):
    asm = _assembly(os.path.join(B.CSRC, name))
    kernels = re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", asm, flags=re.S)
    assert kernels, name
    for kname, body in kernels:
        m = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body)
        assert m, kname
        assert int(m.group(1)) == 0, f"{kname} in {name} uses {m.group(1)} bytes of scratch"
    assert "scratch_store" not in asm, f"{name} spills"
