"""Pins for the oracle's top-r block selection (CPU only).

Brute force over every r-subset with exact rational scores, the ordering invariant (every chosen
candidate beats every unchosen one, ties to the lower id), row invariants (forced set present,
ascending, distinct), constructed exact ties and the -0.0/+0.0 tie."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc
from video_dit_block_cube_amd import synth


def _tiny():
    w = synth.workload(1)
    x = synth.make_inputs(w)
    return orc.Problem(**w.shape_dict), x, w


def test_brute_force_tiny_exact_rationals():
    p, x, w = _tiny()
    assert p.head_dim == 64  # scale 1/8 is exact in rationals
    qm = orc.block_pool(x["q"], p)
    km = orc.block_pool(x["k"], p)
    idx, _ = orc.select_topr(qm, km, p, w.r)
    toks = orc.noise_cube_tokens(p)

    def exact_mean(arr, cube):
        rows = arr[0, toks[cube], 0, :].astype(np.float64)
        return [sum(Fraction(float(v)) for v in rows[:, d]) / p.c for d in range(p.head_dim)]

    qmx = [exact_mean(x["q"], i) for i in range(p.nbq)]
    kmx = [exact_mean(x["k"], j) for j in range(p.nbq)]
    for i in range(p.nbq):
        score = {j: sum(a * b for a, b in zip(qmx[i], kmx[j])) / 8 for j in range(p.nbq) if j != i}
        best = None
        for subset in itertools.combinations(sorted(score), w.r):
            total = sum(score[j] for j in subset)
            if best is None or total > best[0] or (total == best[0] and subset < best[1]):
                best = (total, subset)
        expect = sorted([i] + list(best[1]))
        assert list(idx[0, 0, i]) == expect, (i, list(idx[0, 0, i]), expect)


def _check_rows(idx, mask, S, p, r):
    ks = orc.num_selected(p, r)
    assert idx.shape[-1] == ks
    for b in range(idx.shape[0]):
        for h in range(idx.shape[1]):
            for i in range(p.nbq):
                row = [int(j) for j in idx[b, h, i]]
                # I1: distinct, ascending, in range, forced set present
                assert row == sorted(set(row)) and 0 <= row[0] and row[-1] < p.nbk
                assert set(range(p.nbc)) | {p.nbc + i} <= set(row)
                assert list(np.nonzero(mask[b, h, i])[0]) == row
                # I2: chosen candidates beat unchosen ones (ties: lower id first)
                chosen = [j - p.nbc for j in row if j >= p.nbc and j != p.nbc + i]
                others = [j for j in range(p.nbq) if j != i and j not in chosen]
                assert len(chosen) == min(r, p.nbq - 1)
                for a in chosen:
                    for o in others:
                        sa, so = S[b, h, i, a], S[b, h, i, o]
                        assert sa > so or (sa == so and a < o)


@pytest.mark.parametrize("r", [0, 1, 2, 5, 7, 50])
def test_row_and_order_invariants_tiny(r):
    p, x, _ = _tiny()
    qm, km = orc.block_pool(x["q"], p), orc.block_pool(x["k"], p)
    idx, mask = orc.select_topr(qm, km, p, r)
    _check_rows(idx, mask, orc.block_scores(qm, km, p.head_dim), p, r)


def test_continuation_forced_condition_cubes():
    p = orc.Problem(2, 2, 16, 8, 8, 8, 2, 4, 4, cond_T=4)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, p.Nq, 2, 16))
    k = rng.standard_normal((2, p.Nq, 2, 16))
    qm, km = orc.block_pool(q, p), orc.block_pool(k, p)
    for r in (0, 2, 3, 9):
        idx, mask = orc.select_topr(qm, km, p, r)
        assert p.nbc == 8 and p.nbq == 8
        _check_rows(idx, mask, orc.block_scores(qm, km, p.head_dim), p, r)


def test_dense_special_case_selects_everything():
    p, x, _ = _tiny()
    qm, km = orc.block_pool(x["q"], p), orc.block_pool(x["k"], p)
    idx, mask = orc.select_topr(qm, km, p, 10 ** 6)
    assert np.array_equal(idx[0, 0], np.tile(np.arange(p.nbq), (p.nbq, 1)))
    assert mask.all()


def test_constructed_exact_tie_goes_to_lower_id():
    p, x, _ = _tiny()
    k = x["k"].copy()
    g = k.reshape(1, 4, 8, 8, 1, 64)
    # key cube 5 (cube coordinates (1,0,1): frames 2-3, rows 0-3, cols 4-7) becomes a copy of
    # key cube 3 (cube coordinates (0,1,1): frames 0-1, rows 4-7, cols 4-7)
    g[:, 2:4, 0:4, 4:8] = g[:, 0:2, 4:8, 4:8]
    qm, km = orc.block_pool(x["q"], p), orc.block_pool(k, p)
    assert np.array_equal(km[..., 3, :], km[..., 5, :])
    S = orc.block_scores(qm, km, p.head_dim)
    hits = 0
    for i in range(p.nbq):
        if i in (3, 5):
            continue
        assert S[0, 0, i, 3] == S[0, 0, i, 5]
        cand = [j for j in range(p.nbq) if j != i]
        order = sorted(cand, key=lambda j: (-S[0, 0, i, j], j))
        pos3 = order.index(3)
        assert order[pos3 + 1] == 5            # equal scores, adjacent, lower id first
        row = orc.select_row(S[0, 0, i], i, p, pos3 + 1)   # room for exactly one of the pair
        assert 3 in row and 5 not in row
        hits += 1
    assert hits == p.nbq - 2


def test_negative_zero_ties_positive_zero():
    p = orc.Problem(1, 1, 4, 2, 4, 4, 1, 1, 1)   # 32 one-token cubes
    row = np.full(p.nbq, -1.0)
    row[9] = -0.0
    row[4] = 0.0
    sel = orc.select_row(row, 0, p, 1)
    assert list(sel) == [0, 4]
    row[4], row[9] = -0.0, 0.0
    assert list(orc.select_row(row, 0, p, 1)) == [0, 4]


def test_boundary_gap():
    p = orc.Problem(1, 1, 4, 2, 4, 4, 1, 1, 1)
    row = np.linspace(1.0, 0.0, p.nbq)
    gap = orc.boundary_gap(row, 0, p, 3)
    assert gap == pytest.approx(row[3] - row[4])
    assert orc.boundary_gap(row, 0, p, p.nbq) == float("inf")
