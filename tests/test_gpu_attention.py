"""GPU parity of the sparse attention forward and backward against the fp64 oracle (through the
C ABI).  Both sides use the same selection (idx computed once and shared), so these tests check
the attention arithmetic; selection parity is covered in test_gpu_pool_select.

Tolerances: fp32 max-abs 1e-4, bf16 max-abs 2e-2, plus relative-L2 bounds (1e-5 / 1e-2)."""
import numpy as np
import pytest

import oracle as orc
from tests._util import (assert_close, cached_inputs, print_case, sample_rows, scale_of, to_dev,
                         torch_bwd_all, torch_fwd_all_rows)
from video_dit_block_cube_amd import bsa, synth

pytestmark = pytest.mark.gpu

PORTABLE, AUTO = 1, 0


@pytest.fixture(autouse=True)
def _auto_path():
    yield
    bsa.bsa_set_kernel_path(AUTO)


def _setup(w, x, r, idx=None):
    p = bsa.Problem(**w.shape_dict)
    op = orc.Problem(**w.shape_dict)
    if idx is None:
        qm, km = orc.block_pool(x["q"], op), orc.block_pool(x["k"], op)
        idx, _ = orc.select_topr(qm, km, op, r)
    t = {k: to_dev(v, w.dtype) for k, v in x.items()}
    return p, op, idx, t


def _fwd(p, t, idx, ks, scale):
    return bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], _idx_dev(idx), ks, scale,
                                   t.get("k_cache"), t.get("v_cache"))


def _idx_dev(idx):
    import torch
    return torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to("cuda:0")


SMALL = [
    # (workload, overrides, r, path)
    (1, (), 2, AUTO),                                                   # tiny fp32
    (1, (), 7, AUTO),                                                   # tiny fp32, dense
    (2, (("batch", 2), ("heads", 3), ("T", 8), ("H", 8), ("W", 16)), 3, AUTO),    # bf16 MFMA
    (2, (("batch", 2), ("heads", 3), ("T", 8), ("H", 8), ("W", 16)), 3, PORTABLE),
    (2, (("heads", 2), ("head_dim", 64), ("T", 8), ("H", 8), ("W", 16)), 4, AUTO),  # D = 64
    (2, (("heads", 2), ("T", 4), ("H", 8), ("W", 12)), 2, AUTO),        # nbq = 6 (not /8)
    (2, (("heads", 2), ("T", 8), ("H", 8), ("W", 16)), 15, AUTO),       # dense bf16
    (2, (("heads", 1), ("T", 4), ("H", 4), ("W", 4)), 3, AUTO),         # one cube, k_sel = 1
    (1, (("heads", 3), ("T", 6), ("H", 12), ("W", 10), ("cube_t", 2), ("cube_h", 3),
         ("cube_w", 5)), 3, AUTO),                                      # 30-token cubes fp32
    (2, (("heads", 2), ("head_dim", 128), ("T", 6), ("H", 12), ("W", 10), ("cube_t", 2),
         ("cube_h", 3), ("cube_w", 5)), 3, AUTO),                       # 30-token cubes bf16
    (1, (("heads", 2), ("T", 4), ("H", 8), ("W", 8), ("cube_t", 4), ("cube_h", 8),
         ("cube_w", 4)), 1, AUTO),                                      # 128-token cubes fp32
    (1, (("heads", 2), ("T", 2), ("H", 4), ("W", 4), ("cube_t", 1), ("cube_h", 1),
         ("cube_w", 1)), 5, AUTO),                                      # 1-token cubes
]


@pytest.mark.parametrize("number, over, r, path", SMALL)
def test_fwd_small(number, over, r, path):
    w, x = cached_inputs(number, over)
    print_case(f"fwd {w.name} {dict(over)} r={r} path={path}")
    bsa.bsa_set_kernel_path(path)
    p, op, idx, t = _setup(w, x, r)
    ks = orc.num_selected(op, r)
    scale = scale_of(op)
    o, lse = _fwd(p, t, idx, ks, scale)
    O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], None, None, idx, op, scale)
    assert_close(o.float().cpu().numpy(), O, w.dtype, "O")
    assert_close(lse.cpu().numpy(), LSE, w.dtype, "LSE", max_abs=1e-4 if w.dtype == "f32" else 2e-3,
                 rel=1e-5)


@pytest.mark.parametrize("path", [AUTO, PORTABLE])
def test_fwd_continuation_small(path):
    w = synth.workload(4, batch=2, heads=2, T=12, H=8, W=16, cond_T=4)
    x = synth.make_inputs(w)
    print_case(f"fwd continuation small path={path}")
    bsa.bsa_set_kernel_path(path)
    p, op, idx, t = _setup(w, x, 3)
    ks = orc.num_selected(op, 3)
    scale = scale_of(op)
    o, lse = _fwd(p, t, idx, ks, scale)
    O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], x["k_cache"], x["v_cache"], idx, op,
                                 scale)
    assert_close(o.float().cpu().numpy(), O, "bf16", "O")
    assert_close(lse.cpu().numpy(), LSE, "bf16", "LSE", max_abs=2e-3, rel=1e-5)


@pytest.mark.parametrize("splits", [2, 3, 8, 11, 16, 40])
def test_fwd_key_range_split(splits):
    """The key-range split forward (partials + merge) against the oracle, including ranges that
    hold no selected cube for some query cubes, more ranges than key cubes, and passes of fewer
    than 8 ranges (2, 3, the last 3 of 11) whose XCDs share a range."""
    for number, over, r in ((2, dict(batch=2, heads=2, T=8, H=8, W=32), 5),
                            (4, dict(heads=2, T=12, H=8, W=16, cond_T=4), 3)):
        w = synth.workload(number, **over)
        x = synth.make_inputs(w)
        print_case(f"fwd split={splits} {w.name} {over}")
        p, op, idx, t = _setup(w, x, r)
        ks = orc.num_selected(op, r)
        scale = scale_of(op)
        with bsa.tuning(fwd_splits=splits):
            o, lse = _fwd(p, t, idx, ks, scale)
        O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], x.get("k_cache"), x.get("v_cache"),
                                     idx, op, scale)
        assert_close(o.float().cpu().numpy(), O, "bf16", "O")
        assert_close(lse.cpu().numpy(), LSE, "bf16", "LSE", max_abs=2e-3, rel=1e-5)


@pytest.mark.parametrize("splits", [1, 8])
def test_fwd_peaked_softmax(splits):
    """Q scaled so that one key dominates each row: |O| then reaches max|V| (about 4) instead of
    the ~0.02 of diffuse rows, the regime where the bf16 rounding of the key-range partials
    (8 ranges) and of O itself are largest.  Max-abs 2e-2 against the oracle must still hold."""
    w = synth.workload(2, heads=2, T=8, H=16, W=32)
    x = dict(synth.make_inputs(w))
    x["q"] = synth.round_to_bf16(x["q"] * np.float32(12.0))
    print_case(f"fwd peaked softmax splits={splits} {w.name}")
    p, op, idx, t = _setup(w, x, 9)
    ks = orc.num_selected(op, 9)
    scale = scale_of(op)
    with bsa.tuning(fwd_splits=splits):
        o, lse = _fwd(p, t, idx, ks, scale)
    O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], None, None, idx, op, scale)
    assert np.abs(O).max() > 3.0            # the regime under test: outputs near max|V|
    assert_close(o.float().cpu().numpy(), O, "bf16", "O")
    assert_close(lse.cpu().numpy(), LSE, "bf16", "LSE", max_abs=2e-3, rel=1e-5)


@pytest.fixture
def fwd_splits(request):
    """Run the test with the forward key-range count of its parameter, restored afterwards."""
    saved = bsa.bsa_get_tuning(bsa.BSA_TUNE_FWD_SPLITS)
    bsa.bsa_set_tuning(bsa.BSA_TUNE_FWD_SPLITS, int(request.param))
    yield int(request.param)
    bsa.bsa_set_tuning(bsa.BSA_TUNE_FWD_SPLITS, saved)


@pytest.mark.parametrize("fwd_splits", [1, 8], indirect=True)
def test_fwd_dense_selection(fwd_splits):
    """r = all key cubes through the library's own pool and select, so the forward is dense
    3D attention; checked against the oracle and a plain masked-free softmax in fp64."""
    splits = fwd_splits
    bsa.bsa_set_kernel_path(AUTO)
    w, x = cached_inputs(2, (("heads", 2), ("T", 8), ("H", 16), ("W", 32)))
    print_case(f"fwd dense splits={splits} {w.name}")
    p = bsa.Problem(**w.shape_dict)
    op = orc.Problem(**w.shape_dict)
    t = {k: to_dev(v, w.dtype) for k, v in x.items()}
    r = op.nbq - 1
    ks = orc.num_selected(op, r)
    assert ks == op.nbq
    qm = bsa.bsa_block_pool(p, t["q"])
    km = bsa.bsa_block_pool(p, t["k"])
    idx_d, _ = bsa.bsa_select_topr(p, qm, km, r, with_mask=False)
    idx = idx_d.cpu().numpy()
    assert (idx == np.arange(op.nbq, dtype=np.int32)).all()
    scale = scale_of(op)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx_d, ks, scale)
    O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], None, None, idx, op, scale)
    assert_close(o.float().cpu().numpy(), O, "bf16", "O")
    assert_close(lse.cpu().numpy(), LSE, "bf16", "LSE", max_abs=2e-3, rel=1e-5)
    # head 1 against textbook dense attention (token order is irrelevant to dense softmax)
    q = x["q"][0, :, 1].astype(np.float64)
    k = x["k"][0, :, 1].astype(np.float64)
    v = x["v"][0, :, 1].astype(np.float64)
    s_ = scale * q[:512] @ k.T
    m = s_.max(axis=1, keepdims=True)
    e = np.exp(s_ - m)
    ref = (e @ v) / e.sum(axis=1, keepdims=True)
    assert_close(o[0, :512, 1].float().cpu().numpy(), ref, "bf16", "O dense")


def _gpu_selection(w, t, p):
    qm = bsa.bsa_block_pool(p, t["q"])
    km = bsa.bsa_block_pool(p, t["k"])
    idx, _ = bsa.bsa_select_topr(p, qm, km, w.r, with_mask=False)
    return idx


@pytest.mark.parametrize("number", [2, 3, 4])
def test_fwd_full_size_sampled(number):
    w, x = cached_inputs(number)
    print_case(f"fwd full {w.name}")
    p = bsa.Problem(**w.shape_dict)
    op = orc.Problem(**w.shape_dict)
    t = {k: to_dev(v, w.dtype) for k, v in x.items()}
    idx_d = _gpu_selection(w, t, p)
    ks = orc.num_selected(op, w.r)
    scale = scale_of(op)
    # outputs start as NaN, so "finite everywhere" below also proves every entry was written
    import torch
    o0 = torch.full_like(t["q"], float("nan"))
    l0 = torch.full((p.batch, p.heads, p.Nq), float("nan"), dtype=torch.float32,
                    device=t["q"].device)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx_d, ks, scale,
                                     t.get("k_cache"), t.get("v_cache"), o=o0, lse=l0)
    idx = idx_d.cpu().numpy()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    rows = sample_rows(op, [0, 15, 31], 4 if number == 4 else 6, seed=number)
    res = orc.attn_fwd_rows(x["q"], x["k"], x["v"], x.get("k_cache"), x.get("v_cache"), idx, op,
                            scale, rows)
    toks = orc.noise_cube_tokens(op)
    got_o = np.stack([o[b, toks[i], h] for (b, h, i) in rows])
    ref_o = np.stack([res[k][0] for k in rows])
    got_l = np.stack([lse[b, h, toks[i]] for (b, h, i) in rows])
    ref_l = np.stack([res[k][1] for k in rows])
    assert_close(got_o, ref_o, "bf16", "O")
    assert_close(got_l, ref_l, "bf16", "LSE", max_abs=2e-3, rel=1e-5)
    # at full size: finite everywhere (outputs started as NaN: every entry was written), and every
    # row against plain torch fp32 arithmetic on the device over the same selection
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    o_all, l_all = torch_fwd_all_rows(op, t, idx_d, scale)
    assert_close(o, o_all.cpu().numpy(), "bf16", "O (every row)")
    assert_close(lse, l_all.cpu().numpy(), "bf16", "LSE (every row)", max_abs=2e-3, rel=1e-5)


def test_fwd_720p_split_vs_single_pass():
    """Precision of the key-range split (8 ranges, fp16 partials with a power-of-two row scale,
    then the merge) against the single pass on the 720p-class workload, every row of every head
    against plain torch fp32 arithmetic over the same selection.  Both must meet the bf16 bar, and
    the split may not lose more than a bf16 rounding step of O over the single pass."""
    import torch
    w, x = cached_inputs(3)
    print_case(f"fwd split vs single {w.name}")
    p = bsa.Problem(**w.shape_dict)
    op = orc.Problem(**w.shape_dict)
    t = {k: to_dev(v, w.dtype) for k, v in x.items()}
    idx_d = _gpu_selection(w, t, p)
    ks = orc.num_selected(op, w.r)
    scale = scale_of(op)
    o_all, l_all = (a.cpu().numpy() for a in torch_fwd_all_rows(op, t, idx_d, scale))
    errs = {}
    for splits in (1, 8):
        with bsa.tuning(fwd_splits=splits):
            o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx_d, ks, scale)
        torch.cuda.synchronize()
        o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
        errs[splits] = (assert_close(o, o_all, "bf16", f"O splits={splits}"),
                        assert_close(lse, l_all, "bf16", f"LSE splits={splits}", max_abs=2e-3,
                                     rel=1e-5))
        print(f"  splits={splits}: O max-abs {errs[splits][0][0]:.3e} rel-L2 "
              f"{errs[splits][0][1]:.3e}; LSE max-abs {errs[splits][1][0]:.3e} rel-L2 "
              f"{errs[splits][1][1]:.3e}", flush=True)
    # one bf16 half-ulp at |O| <= 4 is 2^-7: the split's extra rounding stays inside that
    assert errs[8][0][0] <= errs[1][0][0] + 2.0 ** -7
    assert errs[8][0][1] <= 1.5 * errs[1][0][1]


BWD_SMALL = [
    (1, (), 2, AUTO),                                                   # tiny fp32 (portable)
    (5, (("batch", 2), ("heads", 2), ("T", 8), ("H", 8), ("W", 16)), 3, AUTO),   # bf16 MFMA
    (5, (("batch", 2), ("heads", 2), ("T", 8), ("H", 8), ("W", 16)), 3, PORTABLE),
    (5, (("heads", 2), ("head_dim", 64), ("T", 8), ("H", 8), ("W", 16)), 4, AUTO),   # D = 64
    (5, (("heads", 2), ("T", 4), ("H", 8), ("W", 12)), 2, AUTO),        # nbq = 6
    (5, (("heads", 1), ("T", 8), ("H", 8), ("W", 16)), 15, AUTO),       # dense
    (5, (("heads", 1), ("T", 4), ("H", 4), ("W", 4)), 0, AUTO),         # one cube
    (1, (("heads", 2), ("T", 6), ("H", 12), ("W", 10), ("cube_t", 2), ("cube_h", 3),
         ("cube_w", 5)), 3, AUTO),                                      # 30-token cubes fp32
]


def _dO(w, x):
    if "dO" in x:
        return x["dO"]
    rng = np.random.default_rng(4242)
    return rng.standard_normal(x["q"].shape).astype(np.float32)


@pytest.mark.parametrize("number, over, r, path", BWD_SMALL)
def test_bwd_small(number, over, r, path):
    w, x = cached_inputs(number, over)
    print_case(f"bwd {w.name} {dict(over)} r={r} path={path}")
    bsa.bsa_set_kernel_path(path)
    dO = _dO(w, x)
    p, op, idx, t = _setup(w, x, r)
    t["dO"] = to_dev(dO, w.dtype)
    ks = orc.num_selected(op, r)
    scale = scale_of(op)
    o, lse = _fwd(p, t, idx, ks, scale)
    dq, dk, dv = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse,
                                         _idx_dev(idx), ks, scale)
    ref = orc.attn_bwd(x["q"], x["k"], x["v"], dO, idx, op, scale)
    for name, got, rf in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert_close(got.cpu().numpy(), rf, w.dtype, name)


@pytest.mark.parametrize("period_us", [1, 37])
def test_bwd_walk_phase(period_us):
    """The backward with the real-time walk phase (each D = 128 dK/dV and pipelined dQ item
    starts its list at a clock-dependent entry and wraps): a different summation order, so
    gradients within the bf16 bar of the oracle, with and without condition cubes."""
    w, x = cached_inputs(5, (("heads", 2), ("T", 8), ("H", 16), ("W", 32)))
    print_case(f"bwd walk phase {period_us} us {w.name}")
    dO = _dO(w, x)
    p, op, idx, t = _setup(w, x, 9)
    t["dO"] = to_dev(dO, w.dtype)
    ks = orc.num_selected(op, 9)
    scale = scale_of(op)
    o, lse = _fwd(p, t, idx, ks, scale)
    with bsa.tuning(walk_phase_us=period_us):
        got = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, _idx_dev(idx),
                                      ks, scale)
    ref = orc.attn_bwd(x["q"], x["k"], x["v"], dO, idx, op, scale)
    for name, g, rf in zip(("dQ", "dK", "dV"), got, ref):
        assert_close(g.cpu().numpy(), rf, w.dtype, name)
    over = dict(heads=2, T=12, H=8, W=16, cond_T=4)
    with bsa.tuning(walk_phase_us=period_us):
        w, x, dO, op, idx, scale, got = _cached_bwd_case(over, 3)
    ref = orc.attn_bwd(x["q"], x["k"], x["v"], dO, idx, op, scale, k_cache=x["k_cache"],
                       v_cache=x["v_cache"])
    for name, g, rf in zip(("dQ", "dK", "dV", "dK_cache", "dV_cache"), got, ref):
        assert_close(g, rf, "bf16", name + " (cached)")


@pytest.mark.parametrize("case", ["plain", "cache", "ragged", "d64"])
def test_bwd_dkdv_split_by_keys(case):
    """BSA_TUNE_DKDV_SPLIT = 1 (each wave of a key cube takes half its keys and forms dS from the
    fp32 P) against the oracle: without and with condition cubes, on a ragged grid, and at
    D = 64, where the switch changes nothing (the one-wave kernel runs)."""
    print_case(f"bwd dK/dV split by keys, {case}")
    if case == "cache":
        with bsa.tuning(dkdv_split=1):
            w, x, dO, op, idx, scale, got = _cached_bwd_case(dict(heads=2, T=12, H=8, W=16,
                                                                  cond_T=4), 3)
        ref = orc.attn_bwd(x["q"], x["k"], x["v"], dO, idx, op, scale, k_cache=x["k_cache"],
                           v_cache=x["v_cache"])
        for name, g, rf in zip(("dQ", "dK", "dV", "dK_cache", "dV_cache"), got, ref):
            assert_close(g, rf, "bf16", name)
        return
    over = {"plain": (("heads", 2), ("T", 8), ("H", 16), ("W", 32)),
            "ragged": (("heads", 2), ("T", 8), ("H", 14), ("W", 27)),
            "d64": (("heads", 2), ("head_dim", 64), ("T", 8), ("H", 8), ("W", 16))}[case]
    w, x = cached_inputs(5, over)
    dO = _dO(w, x)
    p, op, idx, t = _setup(w, x, 5)
    t["dO"] = to_dev(dO, w.dtype)
    ks = orc.num_selected(op, 5)
    scale = scale_of(op)
    o, lse = _fwd(p, t, idx, ks, scale)
    with bsa.tuning(dkdv_split=1):
        got = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, _idx_dev(idx),
                                      ks, scale)
    ref = orc.attn_bwd(x["q"], x["k"], x["v"], dO, idx, op, scale)
    for name, g, rf in zip(("dQ", "dK", "dV"), got, ref):
        assert_close(g.cpu().numpy(), rf, w.dtype, name)


def test_bwd_dkdv_split_by_keys_full_size():
    """The 480p backward with the split by keys, every element against plain torch fp32
    products: dK's dS now comes from the fp32 P like dQ's, so dK's relative error drops to the
    level of dQ's and dV's; and two identical calls agree bit for bit."""
    import torch
    w, x = cached_inputs(5)
    print_case(f"bwd dK/dV split by keys, full size {w.name}")
    p = bsa.Problem(**w.shape_dict)
    op = orc.Problem(**w.shape_dict)
    t = {k: to_dev(v, w.dtype) for k, v in x.items()}
    idx_d = _gpu_selection(w, t, p)
    ks = orc.num_selected(op, w.r)
    scale = scale_of(op)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx_d, ks, scale)
    with bsa.tuning(dkdv_split=1):
        g1 = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx_d, ks, scale)
        g2 = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx_d, ks, scale)
    torch.cuda.synchronize()
    for a, b_ in zip(g1, g2):
        assert torch.equal(a, b_)
    ref = [a.cpu().numpy() for a in torch_bwd_all(op, t, idx_d, scale)]
    errs = {}
    for name, g, r in zip(("dQ", "dK", "dV"), g1, ref):
        errs[name] = assert_close(g.cpu().numpy(), r, "bf16", f"{name} (every element)")
        print(f"  {name} every element: max-abs {errs[name][0]:.3e} rel-L2 {errs[name][1]:.3e}",
              flush=True)
    assert errs["dK"][1] <= 1.2 * max(errs["dQ"][1], errs["dV"][1])


def _every_element_bwd(op, t, idx_d, scale, dq, dk, dv):
    """Every element of the three gradients against plain torch fp32 arithmetic on the device over
    the same selection (which agrees with the fp64 oracle to ~1e-6 on small grids); prints the
    measured max-abs and rel-L2 of each."""
    import torch
    ref = [a.cpu().numpy() for a in torch_bwd_all(op, t, idx_d, scale)]
    torch.cuda.synchronize()
    for name, got, r in (("dQ", dq, ref[0]), ("dK", dk, ref[1]), ("dV", dv, ref[2])):
        err, rl = assert_close(got, r, "bf16", f"{name} (every element)")
        print(f"  {name} every element: max-abs {err:.3e} rel-L2 {rl:.3e} (max |ref| "
              f"{np.abs(r).max():.3e})", flush=True)


def test_bwd_full_size_sampled():
    w, x = cached_inputs(5)
    print_case(f"bwd full {w.name}")
    p = bsa.Problem(**w.shape_dict)
    op = orc.Problem(**w.shape_dict)
    t = {k: to_dev(v, w.dtype) for k, v in x.items()}
    idx_d = _gpu_selection(w, t, p)
    ks = orc.num_selected(op, w.r)
    scale = scale_of(op)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx_d, ks, scale)
    dq, dk, dv = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx_d, ks,
                                         scale)
    idx = idx_d.cpu().numpy()
    dq, dk, dv = (a.cpu().numpy() for a in (dq, dk, dv))
    rows = sample_rows(op, [0, 31], 3, seed=11)
    cols = sample_rows(op, [0, 31], 3, seed=12)
    rq, rk, rv = orc.attn_bwd(x["q"], x["k"], x["v"], x["dO"], idx, op, scale, rows=rows,
                              key_cubes=cols)
    toks = orc.noise_cube_tokens(op)
    assert_close(np.stack([dq[b, toks[i], h] for (b, h, i) in rows]),
                 np.stack([rq[k] for k in rows]), "bf16", "dQ")
    assert_close(np.stack([dk[b, toks[j], h] for (b, h, j) in cols]),
                 np.stack([rk[k] for k in cols]), "bf16", "dK")
    assert_close(np.stack([dv[b, toks[j], h] for (b, h, j) in cols]),
                 np.stack([rv[k] for k in cols]), "bf16", "dV")
    # properties at full size: sum_k dV = sum_q dO and sum_k dK = 0 per (b, h)
    dO64 = x["dO"].astype(np.float64)
    np.testing.assert_allclose(dv.sum(axis=1), dO64.sum(axis=1), atol=0.5, rtol=1e-2)
    assert np.abs(dk.astype(np.float64).sum(axis=1)).max() < 0.5
    _every_element_bwd(op, t, idx_d, scale, dq, dk, dv)


def test_bwd_720p_full_size_sampled():
    """The backward of the headline step exactly as the benchmark runs it: 720p-class grid
    24x48x80, 32 heads, top-144, the same seeded inputs (q, k, v, dO) and the library's default
    launch configuration; sampled query cubes (dQ) and key cubes (dK, dV) against the oracle, and
    the full-size sum properties."""
    w, x = cached_inputs(3, (("with_grad", True),))
    print_case(f"bwd full {w.name} (benchmark inputs)")
    p = bsa.Problem(**w.shape_dict)
    op = orc.Problem(**w.shape_dict)
    t = {k: to_dev(v, w.dtype) for k, v in x.items()}
    idx_d = _gpu_selection(w, t, p)
    ks = orc.num_selected(op, w.r)
    scale = scale_of(op)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx_d, ks, scale)
    # gradients start as NaN: every query and key cube of every head must be written
    import torch
    nan = lambda: torch.full(t["q"].shape, float("nan"), dtype=torch.float32, device=t["q"].device)
    dq, dk, dv = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx_d, ks,
                                         scale, dq=nan(), dk=nan(), dv=nan())
    del o, lse
    idx = idx_d.cpu().numpy()
    dq, dk, dv = (a.cpu().numpy() for a in (dq, dk, dv))
    for name, a in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert np.isfinite(a).all(), f"{name}: unwritten (NaN) entries"
    _every_element_bwd(op, t, idx_d, scale, dq, dk, dv)
    del t
    rows = sample_rows(op, [0, 17, 31], 3, seed=21)
    cols = sample_rows(op, [0, 17, 31], 3, seed=22)
    rq, rk, rv = orc.attn_bwd(x["q"], x["k"], x["v"], x["dO"], idx, op, scale, rows=rows,
                              key_cubes=cols)
    toks = orc.noise_cube_tokens(op)
    assert_close(np.stack([dq[b, toks[i], h] for (b, h, i) in rows]),
                 np.stack([rq[k] for k in rows]), "bf16", "dQ")
    assert_close(np.stack([dk[b, toks[j], h] for (b, h, j) in cols]),
                 np.stack([rk[k] for k in cols]), "bf16", "dK")
    assert_close(np.stack([dv[b, toks[j], h] for (b, h, j) in cols]),
                 np.stack([rv[k] for k in cols]), "bf16", "dV")
    dO64 = x["dO"].astype(np.float64)
    np.testing.assert_allclose(dv.sum(axis=1), dO64.sum(axis=1), atol=0.5, rtol=1e-2)
    assert np.abs(dk.astype(np.float64).sum(axis=1)).max() < 0.5


# ---------------------------------------------------------------------------------------------
# Backward with the condition cache (continuation training): cache gradients included.
# ---------------------------------------------------------------------------------------------
def _cached_bwd_case(over, r, seed=4243):
    import torch
    w = synth.workload(4, **over)
    x = synth.make_inputs(w)
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal(x["q"].shape).astype(np.float32)
    dO = synth.round_to_bf16(dO)
    p, op, idx, t = _setup(w, x, r)
    t["dO"] = to_dev(dO, w.dtype)
    ks = orc.num_selected(op, r)
    scale = scale_of(op)
    o, lse = _fwd(p, t, idx, ks, scale)
    got = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, _idx_dev(idx), ks,
                                  scale, k_cache=t["k_cache"], v_cache=t["v_cache"])
    torch.cuda.synchronize()
    return w, x, dO, op, idx, scale, [a.cpu().numpy() for a in got]


@pytest.mark.parametrize("over, r", [
    (dict(batch=2, heads=2, T=12, H=8, W=16, cond_T=4), 3),
    (dict(heads=2, head_dim=64, T=12, H=8, W=16, cond_T=8), 2),
    (dict(heads=2, T=24, H=16, W=32, cond_T=12), 9),          # 96 + 96 cubes, k_sel = 106
])
def test_bwd_condition_cache(over, r):
    print_case(f"bwd cached {over} r={r}")
    w, x, dO, op, idx, scale, got = _cached_bwd_case(over, r)
    ref = orc.attn_bwd(x["q"], x["k"], x["v"], dO, idx, op, scale, k_cache=x["k_cache"],
                       v_cache=x["v_cache"])
    for name, g, rf in zip(("dQ", "dK", "dV", "dK_cache", "dV_cache"), got, ref):
        assert_close(g, rf, "bf16", name)


def test_bwd_condition_cache_full_size_sampled():
    """720p-class continuation (12 cached condition frames, top-r = 72): sampled dQ rows against
    the oracle, and every key's gradient through the full-size sums over noise and cache keys."""
    w = synth.workload(4)
    print_case("bwd cached full size 720p continuation")
    import torch
    x = synth.make_inputs(w)
    rng = np.random.default_rng(4244)
    dO = synth.round_to_bf16(rng.standard_normal(x["q"].shape).astype(np.float32))
    p = bsa.Problem(**w.shape_dict)
    op = orc.Problem(**w.shape_dict)
    t = {k: to_dev(v, w.dtype) for k, v in x.items() if k != "dO"}
    t["dO"] = to_dev(dO, w.dtype)
    idx_d = _gpu_selection(w, t, p)
    ks = orc.num_selected(op, w.r)
    scale = scale_of(op)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx_d, ks, scale, t["k_cache"],
                                     t["v_cache"])
    dq, dk, dv, dkc, dvc = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse,
                                                   idx_d, ks, scale, k_cache=t["k_cache"],
                                                   v_cache=t["v_cache"])
    idx = idx_d.cpu().numpy()
    dq, dk, dv, dkc, dvc = (a.cpu().numpy() for a in (dq, dk, dv, dkc, dvc))
    for a in (dq, dk, dv, dkc, dvc):
        assert np.all(np.isfinite(a))
    rows = [(0, 0, 0), (0, 15, 359), (0, 31, 719)]
    rq = orc.attn_bwd(x["q"], x["k"], x["v"], dO, idx, op, scale, rows=rows,
                      k_cache=x["k_cache"], v_cache=x["v_cache"])[0]
    toks = orc.noise_cube_tokens(op)
    assert_close(np.stack([dq[b, toks[i], h] for (b, h, i) in rows]),
                 np.stack([rq[k] for k in rows]), "bf16", "dQ")
    dO64 = dO.astype(np.float64)
    np.testing.assert_allclose(dv.sum(axis=1) + dvc.sum(axis=1), dO64.sum(axis=1), atol=0.5,
                               rtol=1e-2)
    assert np.abs(dk.astype(np.float64).sum(axis=1) + dkc.astype(np.float64).sum(axis=1)).max() \
        < 0.5
    # every cache row receives gradient (all noise queries attend every condition cube)
    assert np.all(np.abs(dvc).sum(axis=-1) > 0)
    # sampled condition cubes of one head against the oracle: each one's dK/dV sums over all 720
    # query cubes (the longest items of the key-stationary pass)
    cols = [(0, 9, 0), (0, 9, 361), (0, 9, op.nbc - 1)]
    rk, rv = orc.attn_bwd(x["q"], x["k"], x["v"], dO, idx, op, scale, key_cubes=cols,
                          k_cache=x["k_cache"], v_cache=x["v_cache"])[1:3]
    ctoks = orc.cond_cube_tokens(op)
    assert_close(np.stack([dkc[b, ctoks[j], h] for (b, h, j) in cols]),
                 np.stack([rk[c] for c in cols]), "bf16", "dK_cache")
    assert_close(np.stack([dvc[b, ctoks[j], h] for (b, h, j) in cols]),
                 np.stack([rv[c] for c in cols]), "bf16", "dV_cache")
