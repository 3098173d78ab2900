"""GPU parity at the size limits: the most noise cubes per (b, h) the selection supports
(39808, one key row in 160 KiB of LDS), and the largest cube (256 tokens), against the oracle."""
import numpy as np
import pytest

import oracle as orc
from tests._util import assert_close, print_case, scale_of, to_dev
from video_dit_block_cube_amd import bsa, synth

pytestmark = pytest.mark.gpu

PORTABLE, AUTO = 1, 0


@pytest.fixture(autouse=True)
def _auto_path():
    yield
    bsa.bsa_set_kernel_path(AUTO)


def test_max_noise_cubes_sampled():
    """39808 cubes (T = 4, grid 1244 x 512, 4x4x4 cubes), one head, D = 128, bf16, r = 3."""
    w = synth.workload(5, heads=1, T=4, H=4 * 311, W=4 * 128, r=3)
    print_case("limits: 39808 noise cubes")
    x = synth.make_inputs(w)
    p, op = bsa.Problem(**w.shape_dict), orc.Problem(**w.shape_dict)
    assert op.nbq == 39808
    t = {k: to_dev(v, w.dtype) for k, v in x.items()}
    qm = bsa.bsa_block_pool(p, t["q"])
    km = bsa.bsa_block_pool(p, t["k"])
    idx_d, _ = bsa.bsa_select_topr(p, qm, km, w.r, with_mask=False)
    qm_ref, km_ref = orc.block_pool(x["q"], op), orc.block_pool(x["k"], op)
    rng = np.random.default_rng(3)
    cubes = np.concatenate([[0, op.nbq - 1], rng.integers(0, op.nbq, 30)])
    np.testing.assert_allclose(qm.cpu().numpy()[:, :, cubes], qm_ref[:, :, cubes], rtol=1e-6,
                               atol=1e-7)
    np.testing.assert_allclose(km.cpu().numpy()[:, :, cubes], km_ref[:, :, cubes], rtol=1e-6,
                               atol=1e-7)
    idx = idx_d.cpu().numpy()
    S_rows = orc.block_scores(qm_ref[:, :, cubes], km_ref, op.head_dim)
    exact = 0
    for n, i in enumerate(cubes):
        ref = orc.select_row(S_rows[0, 0, n], int(i), op, w.r)
        if orc.boundary_gap(S_rows[0, 0, n], int(i), op, w.r) >= 1e-6:
            assert np.array_equal(idx[0, 0, i], ref), (i, idx[0, 0, i], ref)
            exact += 1
    assert exact >= len(cubes) - 2
    ks, scale = orc.num_selected(op, w.r), scale_of(op)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx_d, ks, scale)
    # dK/dV start as NaN: every key cube's work item (ordered longest-first inside the head) must
    # write its rows, zeros for a cube no query selected
    import torch
    nan = lambda: torch.full(t["q"].shape, float("nan"), dtype=torch.float32, device=t["q"].device)
    dq, dk, dv = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx_d, ks,
                                         scale, dk=nan(), dv=nan())
    rows = [(0, 0, int(i)) for i in cubes[:8]]
    ref = orc.attn_fwd_rows(x["q"], x["k"], x["v"], None, None, idx, op, scale, rows)
    toks = orc.noise_cube_tokens(op)
    o = o.float().cpu().numpy()
    for (b, h, i) in rows:
        assert_close(o[b, toks[i], h], ref[(b, h, i)][0], "bf16", f"O cube {i}")
    rq = orc.attn_bwd(x["q"], x["k"], x["v"], x["dO"], idx, op, scale, rows=rows[:4])[0]
    dq = dq.cpu().numpy()
    for (b, h, i) in rows[:4]:
        assert_close(dq[b, toks[i], h], rq[(b, h, i)], "bf16", f"dQ cube {i}")
    for a in (dk, dv):
        assert bool(torch_isfinite(a))
    counts = np.bincount(idx[0, 0].ravel(), minlength=op.nbk)
    cols = [(0, 0, int(j)) for j in (int(np.argmax(counts)), int(np.argmin(counts)), *cubes[2:5])]
    _, rk, rv = orc.attn_bwd(x["q"], x["k"], x["v"], x["dO"], idx, op, scale, key_cubes=cols)[:3]
    dk, dv = dk.cpu().numpy(), dv.cpu().numpy()
    for (b, h, j) in cols:
        assert_close(dk[b, toks[j], h], rk[(b, h, j)], "bf16", f"dK cube {j} ({counts[j]} queries)")
        assert_close(dv[b, toks[j], h], rv[(b, h, j)], "bf16", f"dV cube {j}")


def torch_isfinite(a):
    import torch
    return torch.isfinite(a).all().item()


@pytest.mark.parametrize("number, dtype", [(1, "f32"), (5, "bf16")])
def test_largest_cube_256_tokens(number, dtype):
    """4x8x8 cubes (c = 256) on the portable path, forward and backward in full."""
    w = synth.workload(number, heads=2, head_dim=64, T=8, H=16, W=24, cube_t=4, cube_h=8,
                       cube_w=8, r=2)
    print_case(f"limits: 256-token cubes {dtype}")
    x = synth.make_inputs(w)
    p, op = bsa.Problem(**w.shape_dict), orc.Problem(**w.shape_dict)
    assert op.c == 256
    idx = orc.select_topr(orc.block_pool(x["q"], op), orc.block_pool(x["k"], op), op, w.r)[0]
    t = {k: to_dev(v, w.dtype) for k, v in x.items()}
    dO = x.get("dO")
    if dO is None:
        dO = np.random.default_rng(9).standard_normal(x["q"].shape).astype(np.float32)
    t["dO"] = to_dev(dO, w.dtype)
    import torch
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to("cuda:0")
    ks, scale = orc.num_selected(op, w.r), scale_of(op)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx_d, ks, scale)
    # dK/dV start as NaN: every key cube's work item (ordered longest-first inside the head) must
    # write its rows, zeros for a cube no query selected
    import torch
    nan = lambda: torch.full(t["q"].shape, float("nan"), dtype=torch.float32, device=t["q"].device)
    dq, dk, dv = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx_d, ks,
                                         scale, dk=nan(), dv=nan())
    O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], None, None, idx, op, scale)
    assert_close(o.float().cpu().numpy(), O, w.dtype, "O")
    ref = orc.attn_bwd(x["q"], x["k"], x["v"], dO, idx, op, scale)
    for name, g, rf in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert_close(g.cpu().numpy(), rf, w.dtype, name)
