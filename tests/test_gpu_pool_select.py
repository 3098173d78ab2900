"""GPU parity of the pool and select kernels against the fp64 oracle (through the C ABI).

Pool: fp32-accumulated means against fp64 (rtol 1e-6), bit-exact on integer-valued inputs.
Select: idx and mask bit-exact, rows whose fp64 boundary gap is under 1e-6 checked for the
candidates away from the cut only."""
import numpy as np
import pytest

import oracle as orc
from tests._util import (check_selection, cached_inputs, print_case, to_dev)
from video_dit_block_cube_amd import bsa, synth

pytestmark = pytest.mark.gpu


def _pool_pair(w, x, name):
    p = bsa.Problem(**w.shape_dict)
    op = orc.Problem(**w.shape_dict)
    got = bsa.bsa_block_pool(p, to_dev(x[name], w.dtype)).cpu().numpy()
    return got, orc.block_pool(x[name], op), p, op


@pytest.mark.parametrize("number, over", [
    (1, ()),                                                   # tiny fp32
    (2, (("heads", 3), ("T", 8), ("H", 8), ("W", 12))),        # bf16, 64-token cubes
    (1, (("heads", 3), ("cube_t", 2), ("cube_h", 2), ("cube_w", 2))),   # 8-token cubes
    (1, (("heads", 3), ("T", 6), ("H", 12), ("W", 10), ("cube_t", 2), ("cube_h", 3),
         ("cube_w", 5))),                                      # 30-token cubes, 3 heads
])
def test_pool_small(number, over):
    w, x = cached_inputs(number, over)
    print_case(f"pool {w.name} {dict(over)}")
    for name in ("q", "k"):
        got, ref, _, _ = _pool_pair(w, x, name)
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7)


def test_pool_integer_inputs_bit_exact():
    import torch
    print_case("pool integer-valued bf16 and fp32")
    for dtype, over in (("bf16", dict(heads=2, T=8, H=8, W=8)), ("f32", {})):
        w = synth.workload(2 if dtype == "bf16" else 1, **over)
        rng = np.random.default_rng(99)
        x = rng.integers(-256, 257, size=(w.batch, w.n_noise_tokens, w.heads, w.head_dim))
        x = x.astype(np.float32)
        p = bsa.Problem(**w.shape_dict)
        got = bsa.bsa_block_pool(p, to_dev(x, dtype)).cpu().numpy()
        ref = orc.block_pool(x, orc.Problem(**w.shape_dict))
        assert np.array_equal(got.astype(np.float64), ref)
        torch.cuda.synchronize()


@pytest.mark.parametrize("number", [2, 3])
def test_pool_full_size(number):
    w, x = cached_inputs(number)
    print_case(f"pool full {w.name}")
    for name in ("q", "k"):
        got, ref, _, _ = _pool_pair(w, x, name)
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7)


def _select_pair(w, qm_ref, km_ref, r, heads=None):
    """GPU select on the oracle's means (rounded to fp32) against the oracle select."""
    p = bsa.Problem(**w.shape_dict)
    op = orc.Problem(**w.shape_dict)
    qm32 = qm_ref.astype(np.float32)
    km32 = km_ref.astype(np.float32)
    idx, mask = bsa.bsa_select_topr(p, to_dev(qm32, "f32"), to_dev(km32, "f32"), r)
    idx, mask = idx.cpu().numpy(), mask.cpu().numpy()
    exact, ties = check_selection(idx, mask, qm32.astype(np.float64), km32.astype(np.float64),
                                  op, r, heads)
    return idx, exact, ties


@pytest.mark.parametrize("r", [0, 1, 2, 3, 6, 7, 100])
def test_select_tiny(r):
    w, x = cached_inputs(1)
    print_case(f"select tiny r={r}")
    op = orc.Problem(**w.shape_dict)
    _, exact, _ = _select_pair(w, orc.block_pool(x["q"], op), orc.block_pool(x["k"], op), r)
    assert exact == op.nbq


def test_select_exact_ties_and_zero_rows():
    print_case("select constructed ties")
    w = synth.workload(2, heads=2, T=8, H=8, W=16)    # 16 cubes, D = 128
    op = orc.Problem(**w.shape_dict)
    rng = np.random.default_rng(5)
    km = (rng.standard_normal((1, 2, op.nbq, 128)) * 0.01).astype(np.float32)
    u = rng.standard_normal(128).astype(np.float32)
    km[:, :, 3] = u
    km[:, :, 5] = u
    qm = (u[None, None, None, :] + 0.01 * rng.standard_normal((1, 2, op.nbq, 128))).astype(np.float32)
    qm[0, 1, 7] = 0.0                                  # every score of this row is exactly 0
    p = bsa.Problem(**w.shape_dict)
    idx, mask = bsa.bsa_select_topr(p, to_dev(qm, "f32"), to_dev(km, "f32"), 1)
    idx = idx.cpu().numpy()
    for h in range(2):
        for i in range(op.nbq):
            row = [int(j) for j in idx[0, h, i]]
            if h == 1 and i == 7:
                assert row == [0, 7]                    # all-zero scores: lowest id wins
            elif i in (3, 5):
                assert row == [3, 5]
            else:
                assert row == sorted([i, 3]), (h, i, row)   # tie between 3 and 5 -> 3
    ref_idx, _ = orc.select_topr(qm.astype(np.float64), km.astype(np.float64), op, 1)
    assert np.array_equal(idx, ref_idx)


def test_select_continuation_and_single_cube():
    print_case("select continuation / single cube")
    w = synth.workload(4, heads=3, T=8, H=8, W=16, cond_T=4)
    op = orc.Problem(**w.shape_dict)
    x = synth.make_inputs(w)
    qm, km = orc.block_pool(x["q"], op), orc.block_pool(x["k"], op)
    for r in (0, 2, 5, 15):
        idx, exact, _ = _select_pair(w, qm, km, r)
        assert idx.shape[-1] == op.nbc + 1 + min(r, op.nbq - 1)
    w1 = synth.workload(2, heads=1, T=4, H=4, W=4)     # one cube: k_sel = 1
    op1 = orc.Problem(**w1.shape_dict)
    x1 = synth.make_inputs(w1)
    idx, _, _ = _select_pair(w1, orc.block_pool(x1["q"], op1), orc.block_pool(x1["k"], op1), 5)
    assert idx.shape == (1, 1, 1, 1) and idx[0, 0, 0, 0] == 0


@pytest.mark.parametrize("number", [2, 3, 4])
def test_select_full_size_sampled_heads(number):
    w, x = cached_inputs(number)
    print_case(f"select full {w.name}")
    op = orc.Problem(**w.shape_dict)
    qm = orc.block_pool(x["q"], op)
    km = orc.block_pool(x["k"], op)
    heads = [0, 15, 31]
    _, exact, ties = _select_pair(w, qm, km, w.r, heads)
    assert exact + ties == len(heads) * op.nbq
    assert ties <= 0.05 * (exact + ties)


@pytest.mark.parametrize("number", [1, 2])
def test_pool_then_select_end_to_end(number):
    w, x = cached_inputs(number)
    print_case(f"pool+select end-to-end {w.name}")
    p = bsa.Problem(**w.shape_dict)
    op = orc.Problem(**w.shape_dict)
    qm = bsa.bsa_block_pool(p, to_dev(x["q"], w.dtype))
    km = bsa.bsa_block_pool(p, to_dev(x["k"], w.dtype))
    idx, mask = bsa.bsa_select_topr(p, qm, km, w.r)
    heads = [0] if number == 1 else [0, 15, 31]
    exact, ties = check_selection(idx.cpu().numpy(), mask.cpu().numpy(),
                                  orc.block_pool(x["q"], op), orc.block_pool(x["k"], op), op,
                                  w.r, heads)
    assert ties <= 0.05 * (exact + ties)


@pytest.mark.parametrize("T, H, W, D", [
    (16, 40, 100, 128),   # 1000 cubes: 16 rows per workgroup, the last workgroup holds 8 rows
    (16, 64, 136, 128),   # 2176 cubes: the largest grid with 16 rows per workgroup at D = 128
    (16, 64, 140, 128),   # 2240 cubes: 4 rows per workgroup
    (16, 128, 128, 128),  # 4096 cubes: 2 rows per workgroup
    (16, 64, 140, 64),    # 2240 cubes at D = 64: 16 rows per workgroup
])
def test_select_rows_per_workgroup_paths(T, H, W, D):
    """The select kernel owns 16, 8, 4, 2 or 1 query rows per workgroup depending on how many
    score rows fit in LDS; every path must give the oracle's selection bit for bit."""
    w = synth.workload(2, heads=1, T=T, H=H, W=W, head_dim=D)
    op = orc.Problem(**w.shape_dict)
    print_case(f"select {op.nbq} cubes, D = {D}")
    rng = np.random.default_rng(op.nbq + D)
    qm = (rng.standard_normal((1, 1, op.nbq, D)) * 0.1).astype(np.float32)
    km = (rng.standard_normal((1, 1, op.nbq, D)) * 0.1).astype(np.float32)
    for r in (3, 144):
        _, exact, ties = _select_pair(w, qm, km, r)
        assert exact + ties == op.nbq
        assert ties <= 0.05 * op.nbq
