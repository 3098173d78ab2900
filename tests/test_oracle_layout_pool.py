"""Pins for the oracle's cube partition and mean-pool (CPU only).

The partition is checked against numpy's own index routines (unravel_index, reshape), and the
pool against closed forms: a coordinate field pools to the cube centre, integer inputs pool
exactly, constants stay constant."""
import numpy as np
import pytest

import oracle as orc

SHAPES = [
    # (T, H, W, ct, ch, cw, cond_T)
    (4, 8, 8, 2, 4, 4, 0),       # tiny workload grid
    (6, 12, 10, 2, 3, 5, 0),     # non-cubic cube, several cubes per axis
    (8, 8, 12, 4, 4, 4, 4),      # continuation: 4 condition frames
    (3, 5, 7, 1, 1, 1, 0),       # degenerate 1-token cubes
    (4, 4, 4, 4, 4, 4, 0),       # a single cube
]


def _problem(shape, B=1, Hh=2, D=8):
    T, H, W, ct, ch, cw, cond = shape
    return orc.Problem(B, Hh, D, T, H, W, ct, ch, cw, cond)


@pytest.mark.parametrize("shape", SHAPES)
def test_partition_is_raster_cube_order(shape):
    p = _problem(shape)
    for frames in (p.noise_T, p.cond_T):
        if frames == 0:
            continue
        toks = np.stack(orc.segment_cube_tokens(p, frames))   # divisible grids: all cubes full
        nt, nh, nw = frames // p.cube_t, p.H // p.cube_h, p.W // p.cube_w
        assert toks.shape == (nt * nh * nw, p.c)
        # every token exactly once
        assert np.array_equal(np.sort(toks.ravel()), np.arange(frames * p.H * p.W))
        # members of cube i sit at cube coordinates unravel(i) (raster over cube coordinates)
        t, h, w = np.unravel_index(toks, (frames, p.H, p.W))
        a, b, e = np.unravel_index(np.arange(toks.shape[0]), (nt, nh, nw))
        assert np.array_equal(t // p.cube_t, np.repeat(a[:, None], p.c, 1))
        assert np.array_equal(h // p.cube_h, np.repeat(b[:, None], p.c, 1))
        assert np.array_equal(w // p.cube_w, np.repeat(e[:, None], p.c, 1))
        # inside a cube, raster order over (dt, dh, dw) == ascending token index
        assert np.all(np.diff(toks, axis=1) > 0)


@pytest.mark.parametrize("shape", SHAPES)
def test_pool_of_coordinate_field_is_cube_centre(shape):
    p = _problem(shape, D=4)
    t, h, w = np.unravel_index(np.arange(p.Nq), (p.noise_T, p.H, p.W))
    x = np.zeros((1, p.Nq, p.heads, 4))
    x[0, :, :, 0] = t[:, None]
    x[0, :, :, 1] = h[:, None]
    x[0, :, :, 2] = w[:, None]
    x[0, :, :, 3] = 1.0
    pooled = orc.block_pool(x, p)
    nt, nh, nw = p.noise_T // p.cube_t, p.H // p.cube_h, p.W // p.cube_w
    a, b, e = np.unravel_index(np.arange(p.nbq), (nt, nh, nw))
    for head in range(p.heads):
        np.testing.assert_array_equal(pooled[0, head, :, 0], a * p.cube_t + (p.cube_t - 1) / 2)
        np.testing.assert_array_equal(pooled[0, head, :, 1], b * p.cube_h + (p.cube_h - 1) / 2)
        np.testing.assert_array_equal(pooled[0, head, :, 2], e * p.cube_w + (p.cube_w - 1) / 2)
        np.testing.assert_array_equal(pooled[0, head, :, 3], 1.0)


@pytest.mark.parametrize("shape", SHAPES)
def test_pool_integer_inputs_match_reshape_sum_exactly(shape):
    p = _problem(shape, B=2, Hh=3, D=5)
    rng = np.random.default_rng(7)
    x = rng.integers(-256, 257, size=(p.batch, p.Nq, p.heads, p.head_dim)).astype(np.float32)
    pooled = orc.block_pool(x, p)
    nt, nh, nw = p.noise_T // p.cube_t, p.H // p.cube_h, p.W // p.cube_w
    g = x.astype(np.int64).reshape(p.batch, nt, p.cube_t, nh, p.cube_h, nw, p.cube_w,
                                   p.heads, p.head_dim)
    sums = g.sum(axis=(2, 4, 6)).reshape(p.batch, p.nbq, p.heads, p.head_dim)
    expect = np.transpose(sums, (0, 2, 1, 3)) / p.c
    np.testing.assert_array_equal(pooled, expect)


def test_pool_constant_and_linear():
    p = _problem((4, 8, 8, 2, 4, 4, 0), B=1, Hh=2, D=6)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, p.Nq, 2, 6))
    y = rng.standard_normal((1, p.Nq, 2, 6))
    np.testing.assert_allclose(orc.block_pool(2.5 * x + y, p),
                               2.5 * orc.block_pool(x, p) + orc.block_pool(y, p), atol=1e-14)
    const = np.full((1, p.Nq, 2, 6), -3.25)
    np.testing.assert_array_equal(orc.block_pool(const, p), -3.25)
    # total mass is preserved: sum over cubes of c * mean == sum over tokens
    np.testing.assert_allclose(orc.block_pool(x, p).sum(axis=2) * p.c,
                               x.sum(axis=1), rtol=1e-12)


@pytest.mark.parametrize("bad, kind", [
    (dict(T=5), "shape"),             # noise frames not divisible by cube_t
    (dict(cond_T=1, T=5), "shape"),   # cond_T not a cube multiple
    (dict(cond_T=4), "shape"),        # cond_T == T
    (dict(heads=0), "invalid"),
])
def test_problem_rules(bad, kind):
    base = dict(batch=1, heads=1, head_dim=64, T=4, H=8, W=8, cube_t=2, cube_h=4, cube_w=4,
                cond_T=0)
    base.update(bad)
    with pytest.raises(orc.ProblemError) as ei:
        orc.check_problem(orc.Problem(**base))
    assert ei.value.kind == kind


def test_scores_are_scaled_matmul():
    rng = np.random.default_rng(11)
    qm = rng.standard_normal((2, 3, 5, 16))
    km = rng.standard_normal((2, 3, 5, 16))
    S = orc.block_scores(qm, km, 16)
    ref = np.einsum("bhid,bhjd->bhij", qm, km) * 0.25
    np.testing.assert_allclose(S, ref, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------------------------
# Ragged latent grids: partial edge cubes along H and W.
# ---------------------------------------------------------------------------------------------
RAGGED = [
    # T, H, W, ct, ch, cw, cond_T
    (4, 9, 8, 2, 4, 4, 0),       # one partial cube row of height 1
    (4, 6, 7, 2, 4, 4, 2),       # partial row and column, condition frames
    (8, 45, 10, 4, 4, 4, 4),     # the 720p-class height 45
    (2, 5, 5, 1, 2, 2, 0),
]


def test_ragged_grid_is_accepted():
    p = orc.Problem(1, 1, 64, 4, 8, 10, 2, 4, 4, 0)
    orc.check_problem(p)
    assert p.nbq == 2 * 2 * 3


@pytest.mark.parametrize("shape", RAGGED)
def test_ragged_partition(shape):
    p = _problem(shape)
    for frames in (p.noise_T, p.cond_T):
        if frames == 0:
            continue
        toks = orc.segment_cube_tokens(p, frames)
        gh, gw = -(-p.H // p.cube_h), -(-p.W // p.cube_w)
        assert len(toks) == frames // p.cube_t * gh * gw
        flat = np.concatenate(toks)
        assert np.array_equal(np.sort(flat), np.arange(frames * p.H * p.W))   # exactly once
        # the cube of every token, from its coordinates alone
        t, h, w = np.unravel_index(np.arange(frames * p.H * p.W), (frames, p.H, p.W))
        cube_of = (t // p.cube_t * gh + h // p.cube_h) * gw + w // p.cube_w
        for i, members in enumerate(toks):
            assert np.all(cube_of[members] == i)
            assert np.all(np.diff(members) > 0)
            b, e = (i // gw) % gh, i % gw
            assert len(members) == p.cube_t * min(p.cube_h, p.H - b * p.cube_h) * \
                min(p.cube_w, p.W - e * p.cube_w)


@pytest.mark.parametrize("shape", RAGGED)
def test_ragged_pool_is_clipped_box_centre(shape):
    p = _problem(shape, D=4)
    t, h, w = np.unravel_index(np.arange(p.Nq), (p.noise_T, p.H, p.W))
    x = np.stack([t, h, w, np.ones_like(t)], axis=-1).astype(np.float64)[None, :, None, :]
    x = np.repeat(x, p.heads, axis=2)
    pooled = orc.block_pool(x, p)
    gh, gw = -(-p.H // p.cube_h), -(-p.W // p.cube_w)
    for i in range(p.nbq):
        a, b, e = i // (gh * gw), (i // gw) % gh, i % gw
        he = min(p.cube_h, p.H - b * p.cube_h)
        we = min(p.cube_w, p.W - e * p.cube_w)
        np.testing.assert_allclose(pooled[0, :, i, :],
                                   np.array([[a * p.cube_t + (p.cube_t - 1) / 2,
                                              b * p.cube_h + (he - 1) / 2,
                                              e * p.cube_w + (we - 1) / 2, 1.0]] * p.heads),
                                   rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", RAGGED)
def test_ragged_pool_integer_inputs_exact(shape):
    p = _problem(shape, B=2, Hh=3, D=5)
    rng = np.random.default_rng(8)
    x = rng.integers(-256, 257, size=(p.batch, p.Nq, p.heads, p.head_dim))
    t, h, w = np.unravel_index(np.arange(p.Nq), (p.noise_T, p.H, p.W))
    gh, gw = -(-p.H // p.cube_h), -(-p.W // p.cube_w)
    cube_of = (t // p.cube_t * gh + h // p.cube_h) * gw + w // p.cube_w
    sums = np.zeros((p.batch, p.nbq, p.heads, p.head_dim), dtype=np.int64)
    np.add.at(sums, (slice(None), cube_of), x)
    counts = np.bincount(cube_of, minlength=p.nbq)
    expect = np.transpose(sums, (0, 2, 1, 3)) / counts[None, None, :, None]
    np.testing.assert_array_equal(orc.block_pool(x.astype(np.float32), p), expect)
