"""GPU parity of the fused attention prologue (QK RMS normalisation + 3D RoPE + cube means)
against the fp64 prologue oracle, through the C ABI.

bf16 outputs must lie within one bf16 unit in the last place of the fp64 value (plus 1e-6 for
results that cancel to near zero in the rotation, where the fp32 rounding of the two products
dominates); fp32 outputs within 4e-6 absolute (values are O(1) after normalisation); cube means
(of the unrounded values, fp32 sums) within 1e-6."""
import numpy as np
import pytest

import oracle as orc
from tests._util import cached_inputs, print_case, to_dev
from video_dit_block_cube_amd import bsa, synth

pytestmark = pytest.mark.gpu


def _raw(shape, seed, dtype):
    x = 3.0 * np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return synth.round_to_bf16(x) if dtype == "bf16" else x


def _check_out(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    if dtype == "bf16":
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        bad = np.abs(got - ref) > ulp * (1 + 1e-9) + 1e-6
        assert not bad.any(), f"{what}: {bad.sum()} values off by more than 1 bf16 ulp"
    else:
        err = np.abs(got - ref).max()
        assert err <= 4e-6, f"{what}: max-abs {err:.3e}"


CASES = [
    # (dtype, problem overrides, with gamma)
    ("bf16", dict(heads=3, head_dim=128, T=8, H=8, W=16), True),
    ("f32", dict(heads=2, head_dim=64, T=4, H=8, W=8, cube_t=2, cube_h=4, cube_w=4), False),
    ("bf16", dict(heads=1, head_dim=64, T=8, H=8, W=8), True),           # 8 chunks per token row
    ("f32", dict(heads=3, head_dim=128, T=6, H=12, W=10, cube_t=2, cube_h=3, cube_w=5), True),
]


@pytest.mark.parametrize("dtype, over, with_gamma", CASES)
def test_prologue_noise_segment(dtype, over, with_gamma):
    import torch
    base = dict(batch=2, heads=2, head_dim=128, T=8, H=8, W=8, cube_t=4, cube_h=4, cube_w=4,
                cond_T=0)
    base.update(over)
    print_case(f"prologue noise {dtype} {over} gamma={with_gamma}")
    p, op = bsa.Problem(**base), orc.Problem(**base)
    x = _raw((p.batch, p.Nq, p.heads, p.head_dim), 5, dtype)
    g = (np.random.default_rng(6).uniform(0.5, 1.5, p.head_dim).astype(np.float32)
         if with_gamma else None)
    y, ym = bsa.bsa_qk_prologue(p, to_dev(x, dtype),
                                None if g is None else torch.from_numpy(g).to("cuda:0"))
    ref, ref_m = orc.qk_prologue(x, op, gamma=g)
    _check_out(y.float().cpu().numpy(), ref, dtype, "y")
    np.testing.assert_allclose(ym.cpu().numpy(), ref_m, rtol=1e-6, atol=1e-6)


def test_prologue_condition_segment_and_time_offset():
    base = dict(batch=1, heads=2, head_dim=128, T=12, H=8, W=16, cube_t=4, cube_h=4, cube_w=4,
                cond_T=4)
    print_case("prologue condition + noise segments, cond_T=4")
    p, op = bsa.Problem(**base), orc.Problem(**base)
    xc = _raw((1, 4 * 8 * 16, 2, 128), 7, "bf16")
    xn = _raw((1, p.Nq, 2, 128), 8, "bf16")
    yc, mc = bsa.bsa_qk_prologue(p, to_dev(xc, "bf16"), segment=1)
    assert mc is None
    yn, mn = bsa.bsa_qk_prologue(p, to_dev(xn, "bf16"), segment=0)
    rc, _ = orc.qk_prologue(xc, op, segment="cond")
    rn, rm = orc.qk_prologue(xn, op, segment="noise")
    _check_out(yc.float().cpu().numpy(), rc, "bf16", "y cond")
    _check_out(yn.float().cpu().numpy(), rn, "bf16", "y noise")
    np.testing.assert_allclose(mn.cpu().numpy(), rm, rtol=1e-6, atol=1e-6)


def test_prologue_in_place_and_without_means():
    base = dict(batch=1, heads=4, head_dim=128, T=8, H=8, W=8, cube_t=4, cube_h=4, cube_w=4,
                cond_T=0)
    print_case("prologue in place, no means")
    p, op = bsa.Problem(**base), orc.Problem(**base)
    x = _raw((1, p.Nq, 4, 128), 9, "bf16")
    xd = to_dev(x, "bf16")
    y, m = bsa.bsa_qk_prologue(p, xd, out=xd, with_mean=False)
    assert m is None and y.data_ptr() == xd.data_ptr()
    ref, _ = orc.qk_prologue(x, op)
    _check_out(xd.float().cpu().numpy(), ref, "bf16", "y in place")


def test_prologue_full_size_sampled():
    """720p-class grid (B=1, Hh=32, D=128, 24x48x80): sampled tokens and cubes."""
    w, x = cached_inputs(3)
    print_case("prologue full size 720p, raw V as input")
    p, op = bsa.Problem(**w.shape_dict), orc.Problem(**w.shape_dict)
    y, ym = bsa.bsa_qk_prologue(p, to_dev(x["v"], "bf16"))
    y = y.float().cpu().numpy()
    ym = ym.cpu().numpy()
    rng = np.random.default_rng(10)
    toks = rng.choice(p.Nq, size=1500, replace=False)
    pos = orc.token_positions(op, "noise")[toks]
    ref = orc.rope_3d(orc.rms_norm(x["v"][:, toks]), pos)
    _check_out(y[:, toks], ref, "bf16", "y sampled")
    cube_toks = orc.noise_cube_tokens(op)
    for i in rng.choice(op.nbq, size=12, replace=False):
        t = cube_toks[i]
        r = orc.rope_3d(orc.rms_norm(x["v"][:, t]), orc.token_positions(op, "noise")[t])
        np.testing.assert_allclose(ym[:, :, i], r.mean(axis=1), rtol=1e-6, atol=1e-6)
