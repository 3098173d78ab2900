"""The allocation-free forward (bsa_sparse_attn_fwd_noalloc, workspace in the library's static
device scratch array) against the workspace-taking bsa_sparse_attn_fwd, through the C ABI: three
calls in a row, each smaller than the one before (the first with the 8-range split, whose
partials fill most of the scratch; then a ragged continuation grid; then a head-dim-64 grid), so
every call runs on scratch contents left behind by a larger one.  Both entry points run the same
kernels with the same split, so the outputs must agree bit for bit (stricter than the bf16 bar
of max-abs 2e-2 against the oracle, which the workspace forward's own tests hold).  Also: a
problem whose workspace exceeds the scratch is refused before any launch."""
import math

import numpy as np
import pytest

from tests._util import print_case
from video_dit_block_cube_amd import bsa, synth

pytestmark = pytest.mark.gpu

CASES = [
    # (workload number, overrides, r)
    (5, dict(heads=2), 62),                                             # 480p grid, 8 ranges
    (4, dict(heads=2, T=12, H=10, W=14, cond_T=4), 3),                  # ragged, condition cubes
    (2, dict(heads=3, head_dim=64, T=8, H=8, W=16), 4),                 # D = 64, single pass
]


def _run_pair(number, over, r):
    import torch
    w = synth.workload(number, **over)
    x = synth.make_inputs(w)
    p = bsa.Problem(**w.shape_dict)
    t = {k: torch.from_numpy(v).to("cuda:0").to(torch.bfloat16) for k, v in x.items()}
    ks = bsa.bsa_num_selected(p, r)
    scale = 1.0 / math.sqrt(p.head_dim)
    qm = bsa.bsa_block_pool(p, t["q"])
    km = bsa.bsa_block_pool(p, t["k"])
    idx, _ = bsa.bsa_select_topr(p, qm, km, r, with_mask=False)
    need = bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, False)
    assert 0 < need <= bsa.NOALLOC_SCRATCH_BYTES
    o_ref, l_ref = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx, ks, scale,
                                           t.get("k_cache"), t.get("v_cache"))
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    bsa.bsa_sparse_attn_fwd_noalloc(p, t["q"], t["k"], t["v"], idx, ks, scale, t.get("k_cache"),
                                    t.get("v_cache"), o=o, lse=lse)
    torch.cuda.synchronize()
    return need, o_ref, l_ref, o, lse


def test_noalloc_matches_workspace_forward():
    import torch
    sizes = []
    for number, over, r in CASES:
        print_case(f"noalloc fwd workload {number} {over} r={r}")
        need, o_ref, l_ref, o, lse = _run_pair(number, over, r)
        sizes.append(need)
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "O differs"
        assert torch.equal(lse, l_ref), "LSE differs"
        err = float((o.float() - o_ref.float()).abs().max())
        assert err <= 2e-2
    assert sizes == sorted(sizes, reverse=True) and sizes[0] > sizes[-1]


def test_noalloc_refuses_problems_beyond_the_scratch():
    import torch
    p = bsa.Problem(1, 32, 128, 24, 48, 80, 4, 4, 4)
    ks = bsa.bsa_num_selected(p, 144)
    assert bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, False) > bsa.NOALLOC_SCRATCH_BYTES
    t = torch.empty((1, 16, 1, 1), dtype=torch.bfloat16, device="cuda:0")
    shp = (p.batch, p.Nq, p.heads, p.head_dim)
    q = t.new_empty(shp)
    o = t.new_empty(shp)
    lse = torch.empty((1, 32, p.Nq), dtype=torch.float32, device="cuda:0")
    idx = torch.zeros((1, 32, p.nbq, ks), dtype=torch.int32, device="cuda:0")
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_sparse_attn_fwd_noalloc(p, q, q, q, idx, ks, o=o, lse=lse)
    assert e.value.status == 4 and "scratch" in str(e.value)
