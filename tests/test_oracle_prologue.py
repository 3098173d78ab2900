"""Pins of the prologue oracle (QK normalisation + 3D RoPE) against closed forms and invariants.

The pages name the steps but print no values, so every pin here is mathematics: explicit
rotations of unit vectors, group properties of rotations, the relative-position property that
motivates rotary embeddings, and exact properties of RMS normalisation."""
import math

import numpy as np
import pytest

import oracle as orc


def _p(**kw):
    base = dict(batch=1, heads=2, head_dim=128, T=8, H=8, W=8, cube_t=4, cube_h=4, cube_w=4,
                cond_T=0)
    base.update(kw)
    return orc.Problem(**base)


def test_axis_widths():
    assert orc.axis_widths(128) == (44, 42, 42)
    assert orc.axis_widths(64) == (24, 20, 20)
    for d in (64, 128):
        assert sum(orc.axis_widths(d)) == d and all(a % 2 == 0 for a in orc.axis_widths(d))


def test_token_positions_segments():
    p = _p(T=12, H=4, W=8, cond_T=4)
    noise = orc.token_positions(p, "noise")
    cond = orc.token_positions(p, "cond")
    assert noise.shape == (8 * 4 * 8, 3) and cond.shape == (4 * 4 * 8, 3)
    # raster order: w fastest, then h, then t; noise frames start after the condition frames
    assert tuple(noise[0]) == (4, 0, 0) and tuple(noise[1]) == (4, 0, 1)
    assert tuple(noise[8]) == (4, 1, 0) and tuple(noise[32]) == (5, 0, 0)
    assert tuple(cond[-1]) == (3, 3, 7)


def _unit(D, ch):
    x = np.zeros((1, 1, 1, D))
    x[..., ch] = 1.0
    return x


def test_rotation_of_unit_vectors_closed_form():
    D = 128
    # first pair of the time block, frequency 1: t = 1 rotates e0 by one radian into (cos 1, sin 1)
    y = orc.rope_3d(_unit(D, 0), np.array([[1, 0, 0]]))
    assert y[0, 0, 0, 0] == pytest.approx(0.5403023058681398, abs=1e-15)
    assert y[0, 0, 0, 1] == pytest.approx(0.8414709848078965, abs=1e-15)
    assert np.abs(y[0, 0, 0, 2:]).max() == 0.0
    # the odd channel of the pair rotates to (-sin, cos)
    y = orc.rope_3d(_unit(D, 1), np.array([[1, 0, 0]]))
    assert y[0, 0, 0, 0] == pytest.approx(-0.8414709848078965, abs=1e-15)
    assert y[0, 0, 0, 1] == pytest.approx(0.5403023058681398, abs=1e-15)
    # pair 5 of the height block (channels 44 + 10, 44 + 11): frequency 10000^(-10/42), h = 7
    f = 10000.0 ** (-10.0 / 42.0)
    y = orc.rope_3d(_unit(D, 54), np.array([[0, 7, 0]]))
    assert y[0, 0, 0, 54] == pytest.approx(math.cos(7 * f), abs=1e-15)
    assert y[0, 0, 0, 55] == pytest.approx(math.sin(7 * f), abs=1e-15)
    # last pair of the width block (channels 126, 127): frequency 10000^(-40/42), w = 79
    f = 10000.0 ** (-40.0 / 42.0)
    y = orc.rope_3d(_unit(D, 126), np.array([[0, 0, 79]]))
    assert y[0, 0, 0, 126] == pytest.approx(math.cos(79 * f), abs=1e-15)
    assert y[0, 0, 0, 127] == pytest.approx(math.sin(79 * f), abs=1e-15)


def test_axis_isolation():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 1, 1, 128))
    base = orc.rope_3d(x, np.array([[3, 5, 0]]))
    moved_w = orc.rope_3d(x, np.array([[3, 5, 9]]))
    assert np.array_equal(base[..., :86], moved_w[..., :86])       # t and h blocks untouched
    assert not np.allclose(base[..., 86:], moved_w[..., 86:])
    moved_t = orc.rope_3d(x, np.array([[6, 5, 0]]))
    assert np.array_equal(base[..., 44:], moved_t[..., 44:])       # h and w blocks untouched
    zero = orc.rope_3d(x, np.array([[0, 0, 0]]))
    assert np.array_equal(zero, x)                                  # position 0 is the identity


def test_rotation_group_properties():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 5, 3, 64))
    a = rng.integers(-40, 40, size=(5, 3))
    b = rng.integers(-40, 40, size=(5, 3))
    ya = orc.rope_3d(x, a)
    # pairwise norms preserved
    np.testing.assert_allclose(ya[..., 0::2] ** 2 + ya[..., 1::2] ** 2,
                               x[..., 0::2] ** 2 + x[..., 1::2] ** 2, rtol=1e-13)
    # composition adds positions; the negative position inverts
    np.testing.assert_allclose(orc.rope_3d(ya, b), orc.rope_3d(x, a + b), atol=1e-12)
    np.testing.assert_allclose(orc.rope_3d(ya, -a), x, atol=1e-12)


def test_relative_position_property():
    """<R(p1) q, R(p2) k> depends on p1 - p2 only (per axis)."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 1, 128))
    k = rng.standard_normal((1, 1, 1, 128))
    p1, p2 = np.array([[5, 11, 30]]), np.array([[2, 17, 3]])
    s = np.array([[7, -4, 21]])
    d0 = np.sum(orc.rope_3d(q, p1) * orc.rope_3d(k, p2))
    d1 = np.sum(orc.rope_3d(q, p1 + s) * orc.rope_3d(k, p2 + s))
    assert d1 == pytest.approx(d0, abs=1e-12)


def test_rms_norm_closed_forms():
    c = 3.0
    x = np.full((1, 2, 1, 128), c)
    y = orc.rms_norm(x)
    np.testing.assert_allclose(y, c / math.sqrt(c * c + 1e-6), rtol=1e-15)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 7, 3, 64)) * 5
    g = rng.uniform(0.5, 2.0, size=64)
    y = orc.rms_norm(x, g)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    # y / g has mean square ms / (ms + eps) and the direction of x
    np.testing.assert_allclose(np.mean((y / g) ** 2, axis=-1, keepdims=True), ms / (ms + 1e-6),
                               rtol=1e-12)
    np.testing.assert_allclose((y / g) * np.sqrt(ms + 1e-6), x, rtol=1e-12)
    # scale invariance up to eps
    np.testing.assert_allclose(orc.rms_norm(1e3 * x, g), y, rtol=1e-7)


def test_prologue_composes_norm_then_rotation_and_pools():
    p = _p(T=8, H=8, W=8)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, p.Nq, 2, 128)).astype(np.float32)
    y, ym = orc.qk_prologue(x, p)
    # rotation keeps pair norms, so the normalised mean square survives it
    ms = np.mean(x.astype(np.float64) ** 2, axis=-1)
    np.testing.assert_allclose(np.mean(y ** 2, axis=-1), ms / (ms + 1e-6), rtol=1e-12)
    # norm after rotation would differ from norm before it only through eps: check the order by
    # a token whose rotation is not the identity and a gain that is not rotation-invariant
    g = np.linspace(0.5, 1.5, 128)
    y2, _ = orc.qk_prologue(x, p, gamma=g)
    alt = orc.rms_norm(orc.rope_3d(x.astype(np.float64), orc.token_positions(p, "noise")), g)
    assert np.abs(y2 - alt).max() > 1e-3
    np.testing.assert_allclose(ym, orc.block_pool(y, p), rtol=0, atol=0)
    yc, ycm = orc.qk_prologue(rng.standard_normal((1, 0, 2, 128)), _p(T=8, H=8, W=8, cond_T=0),
                              segment="cond")
    assert yc.shape == (1, 0, 2, 128) and ycm is None
