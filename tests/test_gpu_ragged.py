"""GPU parity on ragged latent grids (H or W not a multiple of the cube side, e.g. the real 720p
latent height 45): partial edge cubes in pool, select, prologue, forward, continuation and
backward, against the fp64 oracle through the C ABI.  Tolerances as in the other GPU tests."""
import numpy as np
import pytest

import oracle as orc
from tests._util import (assert_close, cached_inputs, check_selection, print_case, scale_of,
                         to_dev)
from video_dit_block_cube_amd import bsa, synth

pytestmark = pytest.mark.gpu

PORTABLE, AUTO = 1, 0


@pytest.fixture(autouse=True)
def _auto_path(monkeypatch):
    yield
    bsa.bsa_set_kernel_path(AUTO)


def _idx_dev(idx):
    import torch
    return torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to("cuda:0")


def _oracle_idx(x, op, r):
    return orc.select_topr(orc.block_pool(x["q"], op), orc.block_pool(x["k"], op), op, r)[0]


@pytest.mark.parametrize("number, over", [
    (2, (("heads", 2), ("T", 8), ("H", 18), ("W", 22))),
    (1, (("heads", 2), ("T", 4), ("H", 9), ("W", 10))),
])
def test_ragged_pool_and_select(number, over):
    w, x = cached_inputs(number, over)
    print_case(f"ragged pool/select {w.name} {dict(over)}")
    p, op = bsa.Problem(**w.shape_dict), orc.Problem(**w.shape_dict)
    qm = bsa.bsa_block_pool(p, to_dev(x["q"], w.dtype))
    km = bsa.bsa_block_pool(p, to_dev(x["k"], w.dtype))
    rq, rk = orc.block_pool(x["q"], op), orc.block_pool(x["k"], op)
    np.testing.assert_allclose(qm.cpu().numpy(), rq, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(km.cpu().numpy(), rk, rtol=1e-6, atol=1e-7)
    r = 3
    idx, mask = bsa.bsa_select_topr(p, qm, km, r)
    check_selection(idx.cpu().numpy(), mask.cpu().numpy(), rq, rk, op, r)


FWD = [
    # (workload, overrides, r, path)
    (2, (("heads", 2), ("T", 8), ("H", 18), ("W", 22)), 5, AUTO),
    (2, (("heads", 2), ("T", 8), ("H", 18), ("W", 22)), 5, PORTABLE),
    (2, (("heads", 2), ("head_dim", 64), ("T", 8), ("H", 9), ("W", 14)), 3, AUTO),
    (1, (("heads", 2), ("T", 4), ("H", 9), ("W", 10)), 2, AUTO),             # fp32
    (4, (("heads", 2), ("T", 12), ("H", 10), ("W", 14), ("cond_T", 4)), 3, AUTO),
    (4, (("heads", 2), ("T", 12), ("H", 10), ("W", 14), ("cond_T", 4)), 3, PORTABLE),
]


@pytest.mark.parametrize("number, over, r, path", FWD)
def test_ragged_fwd(number, over, r, path):
    w, x = cached_inputs(number, over)
    print_case(f"ragged fwd {w.name} {dict(over)} r={r} path={path}")
    bsa.bsa_set_kernel_path(path)
    p, op = bsa.Problem(**w.shape_dict), orc.Problem(**w.shape_dict)
    idx = _oracle_idx(x, op, r)
    t = {k: to_dev(v, w.dtype) for k, v in x.items()}
    ks, scale = orc.num_selected(op, r), scale_of(op)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], _idx_dev(idx), ks, scale,
                                     t.get("k_cache"), t.get("v_cache"))
    O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], x.get("k_cache"), x.get("v_cache"), idx,
                                 op, scale)
    assert_close(o.float().cpu().numpy(), O, w.dtype, "O")
    assert_close(lse.cpu().numpy(), LSE, w.dtype, "LSE",
                 max_abs=1e-4 if w.dtype == "f32" else 2e-3, rel=1e-5)


@pytest.mark.parametrize("splits", [3, 8])
def test_ragged_fwd_key_range_split(splits):
    for number, over, r in ((2, (("batch", 2), ("heads", 2), ("T", 8), ("H", 18), ("W", 22)), 5),
                            (4, (("heads", 2), ("T", 12), ("H", 10), ("W", 14), ("cond_T", 4)), 3)):
        w, x = cached_inputs(number, over)
        print_case(f"ragged fwd split={splits} {w.name} {dict(over)}")
        p, op = bsa.Problem(**w.shape_dict), orc.Problem(**w.shape_dict)
        idx = _oracle_idx(x, op, r)
        t = {k: to_dev(v, w.dtype) for k, v in x.items()}
        ks, scale = orc.num_selected(op, r), scale_of(op)
        with bsa.tuning(fwd_splits=splits):
            o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], _idx_dev(idx), ks, scale,
                                             t.get("k_cache"), t.get("v_cache"))
        O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], x.get("k_cache"), x.get("v_cache"),
                                     idx, op, scale)
        assert_close(o.float().cpu().numpy(), O, "bf16", "O")
        assert_close(lse.cpu().numpy(), LSE, "bf16", "LSE", max_abs=2e-3, rel=1e-5)


BWD = [
    (5, (("heads", 2), ("T", 8), ("H", 18), ("W", 22)), 5, AUTO),
    (5, (("heads", 2), ("T", 8), ("H", 18), ("W", 22)), 5, PORTABLE),
    (5, (("heads", 2), ("head_dim", 64), ("T", 8), ("H", 9), ("W", 14)), 3, AUTO),
    (1, (("heads", 2), ("T", 4), ("H", 9), ("W", 10)), 2, AUTO),             # fp32, portable
    (4, (("heads", 2), ("T", 12), ("H", 10), ("W", 14), ("cond_T", 4)), 3, AUTO),   # cache grads
]


@pytest.mark.parametrize("number, over, r, path", BWD)
def test_ragged_bwd(number, over, r, path):
    w, x = cached_inputs(number, over)
    print_case(f"ragged bwd {w.name} {dict(over)} r={r} path={path}")
    bsa.bsa_set_kernel_path(path)
    p, op = bsa.Problem(**w.shape_dict), orc.Problem(**w.shape_dict)
    idx = _oracle_idx(x, op, r)
    dO = x.get("dO")
    if dO is None:
        dO = np.random.default_rng(4242).standard_normal(x["q"].shape).astype(np.float32)
        if w.dtype == "bf16":
            dO = synth.round_to_bf16(dO)
    t = {k: to_dev(v, w.dtype) for k, v in x.items()}
    t["dO"] = to_dev(dO, w.dtype)
    ks, scale = orc.num_selected(op, r), scale_of(op)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], _idx_dev(idx), ks, scale,
                                     t.get("k_cache"), t.get("v_cache"))
    got = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, _idx_dev(idx), ks,
                                  scale, k_cache=t.get("k_cache"), v_cache=t.get("v_cache"))
    ref = orc.attn_bwd(x["q"], x["k"], x["v"], dO, idx, op, scale, k_cache=x.get("k_cache"),
                       v_cache=x.get("v_cache"))
    for name, g, rf in zip(("dQ", "dK", "dV", "dK_cache", "dV_cache"), got, ref):
        assert_close(g.cpu().numpy(), rf, w.dtype, name)


def test_ragged_prologue():
    import torch
    base = dict(batch=1, heads=2, head_dim=128, T=8, H=18, W=22, cube_t=4, cube_h=4, cube_w=4,
                cond_T=0)
    print_case("ragged prologue 18x22")
    p, op = bsa.Problem(**base), orc.Problem(**base)
    x = synth.round_to_bf16(
        3 * np.random.default_rng(12).standard_normal((1, p.Nq, 2, 128)).astype(np.float32))
    y, m = bsa.bsa_qk_prologue(p, to_dev(x, "bf16"))
    ref, ref_m = orc.qk_prologue(x, op)
    err = np.abs(y.float().cpu().numpy() - ref)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(err <= ulp * (1 + 1e-9) + 1e-6)
    np.testing.assert_allclose(m.cpu().numpy(), ref_m, rtol=1e-6, atol=1e-6)
    torch.cuda.synchronize()


def test_real_720p_latent_grid_sampled():
    """The real 720p latent grid 24 x 45 x 80 (45 = 11 full cube rows + one of height 1): GPU
    selection, forward and backward, checked on sampled query cubes that include partial ones."""
    w = synth.workload(5, H=45, W=80)
    print_case("ragged full size 24x45x80 fwd+bwd")
    x = synth.make_inputs(w)
    p, op = bsa.Problem(**w.shape_dict), orc.Problem(**w.shape_dict)
    t = {k: to_dev(v, w.dtype) for k, v in x.items()}
    qm = bsa.bsa_block_pool(p, t["q"])
    km = bsa.bsa_block_pool(p, t["k"])
    idx_d, _ = bsa.bsa_select_topr(p, qm, km, w.r, with_mask=False)
    ks, scale = orc.num_selected(op, w.r), scale_of(op)
    # outputs start as NaN: every token, those of the partial edge cubes included, must be written
    import torch
    nan = lambda dt=torch.float32: torch.full(t["q"].shape, float("nan"), dtype=dt,
                                              device=t["q"].device)
    l0 = torch.full((p.batch, p.heads, p.Nq), float("nan"), dtype=torch.float32,
                    device=t["q"].device)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx_d, ks, scale,
                                     o=nan(t["q"].dtype), lse=l0)
    dq, dk, dv = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx_d, ks,
                                         scale, dq=nan(), dk=nan(), dv=nan())
    for name, a in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(a).all()), f"{name}: unwritten (NaN) entries"
    idx = idx_d.cpu().numpy()
    o, dq = o.float().cpu().numpy(), dq.cpu().numpy()
    gw = 20
    # query cubes: first, a partial one in the last cube row (h index 11), the last one
    rows = [(0, 0, 0), (0, 7, 11 * gw + 3), (0, 31, op.nbq - 1), (0, 15, 5 * 12 * gw + 11 * gw)]
    ref = orc.attn_fwd_rows(x["q"], x["k"], x["v"], None, None, idx, op, scale, rows)
    toks = orc.noise_cube_tokens(op)
    for (b, h, i) in rows:
        assert_close(o[b, toks[i], h], ref[(b, h, i)][0], "bf16", f"O cube {i}")
    rq = orc.attn_bwd(x["q"], x["k"], x["v"], x["dO"], idx, op, scale, rows=rows)[0]
    for (b, h, i) in rows:
        assert_close(dq[b, toks[i], h], rq[(b, h, i)], "bf16", f"dQ cube {i}")
    assert len(toks[11 * gw + 3]) == 16
