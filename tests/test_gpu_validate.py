"""bsa_validate_idx: the selection contract of the attention calls (every entry in [0, nbk), rows
strictly ascending), checked on the GPU.  Rows of bsa_select_topr pass; rows broken on purpose
on the host (an id out of range, a repeated id, a descending pair, a negative id) are counted
exactly, one per broken row however many faults it holds."""
import numpy as np
import pytest

from tests._util import print_case
from video_dit_block_cube_amd import bsa, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("number, over, r", [
    (2, dict(heads=3, T=8, H=8, W=16), 3),
    (4, dict(heads=2, T=12, H=10, W=14, cond_T=4), 5),                 # condition cubes, ragged
    (2, dict(heads=2, T=8, H=16, W=32), 200),                           # rows longer than a wave
])
def test_validate_idx_counts_broken_rows(number, over, r):
    import torch
    w = synth.workload(number, **over)
    print_case(f"validate idx {w.name} {over} r={r}")
    x = synth.make_inputs(w)
    p = bsa.Problem(**w.shape_dict)
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    q = torch.from_numpy(x["q"]).to("cuda:0").to(dt)
    k = torch.from_numpy(x["k"]).to("cuda:0").to(dt)
    ks = bsa.bsa_num_selected(p, r)
    idx, _ = bsa.bsa_select_topr(p, bsa.bsa_block_pool(p, q), bsa.bsa_block_pool(p, k), r,
                                 with_mask=False)
    assert bsa.bsa_validate_idx(p, idx, ks) == 0
    bad = idx.cpu().numpy().copy()
    rows = bad.reshape(-1, ks)
    n = rows.shape[0]
    rng = np.random.default_rng(5)
    picks = rng.choice(n, size=min(n, 7), replace=False)
    kinds = ["high", "low", "dup", "swap", "high_last", "two_faults", "dup"]
    for row, kind in zip(picks, kinds):
        if kind == "high":
            rows[row, 0] = p.nbk
        elif kind == "low":
            rows[row, -1] = -1
        elif kind == "dup" and ks > 1:
            rows[row, 1] = rows[row, 0]
        elif kind == "swap" and ks > 1:
            rows[row, [0, 1]] = rows[row, [1, 0]]
        elif kind == "high_last":
            rows[row, -1] = p.nbk + 5
        elif kind == "two_faults" and ks > 1:
            rows[row, 0] = -3
            rows[row, -1] = 2 ** 30
        else:
            rows[row, 0] = p.nbk
    broken = sum(1 for r_ in rows if (r_.min() < 0 or r_.max() >= p.nbk or
                                      (ks > 1 and np.any(np.diff(r_) <= 0))))
    assert broken == len(picks)
    got = bsa.bsa_validate_idx(p, torch.from_numpy(bad).to("cuda:0"), ks)
    assert got == broken
