"""Pins for the oracle's forward attention (CPU only).

Against torch's own scaled_dot_product_attention in float64 (a library routine): the dense
special case (every cube selected) and token-level masked attention built from the selection.
Invariants: LSE equals scipy's logsumexp of the selected scores, O lies in the hull of the
selected V rows, heads are independent, and the cached continuation mode equals the noise rows of
full-sequence block-causal attention."""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as orc
from video_dit_block_cube_amd import synth


def _tiny():
    w = synth.workload(1)
    return orc.Problem(**w.shape_dict), synth.make_inputs(w), w


def _token_mask(p, idx_bh):
    """[Nq, Nk] bool over the noise segment: query token attends key token."""
    toks = orc.noise_cube_tokens(p)
    M = np.zeros((p.Nq, p.Nq), dtype=bool)
    for i in range(p.nbq):
        for j in idx_bh[i]:
            M[np.ix_(toks[i], toks[int(j) - p.nbc])] = True
    return M


def _sdpa(q, k, v, scale, mask=None):
    qt = torch.from_numpy(np.ascontiguousarray(np.transpose(q, (0, 2, 1, 3)), dtype=np.float64))
    kt = torch.from_numpy(np.ascontiguousarray(np.transpose(k, (0, 2, 1, 3)), dtype=np.float64))
    vt = torch.from_numpy(np.ascontiguousarray(np.transpose(v, (0, 2, 1, 3)), dtype=np.float64))
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale)
    return np.transpose(o.numpy(), (0, 2, 1, 3))


def test_dense_special_case_matches_torch_sdpa():
    p, x, _ = _tiny()
    scale = 1 / math.sqrt(p.head_dim)
    qm, km = orc.block_pool(x["q"], p), orc.block_pool(x["k"], p)
    idx, _ = orc.select_topr(qm, km, p, p.nbq)
    O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], None, None, idx, p, scale)
    ref = _sdpa(x["q"], x["k"], x["v"], scale)
    np.testing.assert_allclose(O, ref, atol=1e-12, rtol=0)
    s = scale * np.einsum("nd,md->nm", x["q"][0, :, 0].astype(np.float64),
                          x["k"][0, :, 0].astype(np.float64))
    np.testing.assert_allclose(LSE[0, 0], scipy.special.logsumexp(s, axis=1), atol=1e-12)


@pytest.mark.parametrize("r", [0, 1, 2, 4])
def test_masked_matches_torch_sdpa_with_token_mask(r):
    p, x, _ = _tiny()
    scale = 1 / math.sqrt(p.head_dim)
    qm, km = orc.block_pool(x["q"], p), orc.block_pool(x["k"], p)
    idx, _ = orc.select_topr(qm, km, p, r)
    O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], None, None, idx, p, scale)
    M = _token_mask(p, idx[0, 0])
    assert M.sum() == p.Nq * orc.num_selected(p, r) * p.c
    ref = _sdpa(x["q"], x["k"], x["v"], scale, M)
    np.testing.assert_allclose(O, ref, atol=1e-12, rtol=0)
    s = scale * np.einsum("nd,md->nm", x["q"][0, :, 0].astype(np.float64),
                          x["k"][0, :, 0].astype(np.float64))
    s[~M] = -np.inf
    np.testing.assert_allclose(LSE[0, 0], scipy.special.logsumexp(s, axis=1), atol=1e-12)


def test_output_in_hull_of_selected_values_and_multi_head_batch():
    p = orc.Problem(2, 3, 16, 4, 8, 8, 2, 4, 4)
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((2, p.Nq, 3, 16)) for _ in range(3))
    scale = 0.25
    qm, km = orc.block_pool(q, p), orc.block_pool(k, p)
    idx, _ = orc.select_topr(qm, km, p, 2)
    O, _ = orc.sparse_attn_fwd(q, k, v, None, None, idx, p, scale)
    toks = orc.noise_cube_tokens(p)
    for b in range(2):
        for h in range(3):
            for i in range(p.nbq):
                vs = np.concatenate([v[b, toks[int(j)], h] for j in idx[b, h, i]])
                Oi = O[b, toks[i], h]
                assert np.all(Oi <= vs.max(axis=0) + 1e-12) and np.all(Oi >= vs.min(axis=0) - 1e-12)
    # heads and batches are independent: permuting heads permutes every output
    perm = [2, 0, 1]
    idx_p = idx[:, perm]
    O2, _ = orc.sparse_attn_fwd(q[:, :, perm], k[:, :, perm], v[:, :, perm], None, None, idx_p,
                                p, scale)
    np.testing.assert_allclose(O2, O[:, :, perm], atol=1e-14)
    # each batch alone gives the same rows
    Ob, _ = orc.sparse_attn_fwd(q[1:], k[1:], v[1:], None, None, idx[1:],
                                orc.Problem(1, 3, 16, 4, 8, 8, 2, 4, 4), scale)
    np.testing.assert_allclose(Ob[0], O[1], atol=1e-14)


def test_rows_api_matches_full():
    p, x, _ = _tiny()
    qm, km = orc.block_pool(x["q"], p), orc.block_pool(x["k"], p)
    idx, _ = orc.select_topr(qm, km, p, 2)
    O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], None, None, idx, p, 0.125)
    res = orc.attn_fwd_rows(x["q"], x["k"], x["v"], None, None, idx, p, 0.125, [(0, 0, 5)])
    toks = orc.noise_cube_tokens(p)
    np.testing.assert_array_equal(res[(0, 0, 5)][0], O[0, toks[5], 0])
    np.testing.assert_array_equal(res[(0, 0, 5)][1], LSE[0, 0, toks[5]])


def test_block_causal_cached_mode_equals_full_sequence():
    # 8 frames, the first 4 are condition frames; cube 2x4x4 -> nbc = nbq = 8
    p = orc.Problem(2, 2, 16, 8, 8, 8, 2, 4, 4, cond_T=4)
    rng = np.random.default_rng(21)
    N = p.T * p.H * p.W
    qf, kf, vf = (rng.standard_normal((2, N, 2, 16)) for _ in range(3))
    scale = 0.25
    r, r_cond = 2, 1
    Of, LSEf, sel = orc.full_block_causal_fwd(qf, kf, vf, p, r, r_cond, scale)
    # cached mode: condition K/V from the cache, queries only from the noise frames
    q, k, v = qf[:, p.Nc:], kf[:, p.Nc:], vf[:, p.Nc:]
    kc, vc = kf[:, :p.Nc], vf[:, :p.Nc]
    qm, km = orc.block_pool(q, p), orc.block_pool(k, p)
    idx, _ = orc.select_topr(qm, km, p, r)
    O, LSE = orc.sparse_attn_fwd(q, k, v, kc, vc, idx, p, scale)
    np.testing.assert_allclose(O, Of[:, p.Nc:], atol=1e-13)
    np.testing.assert_allclose(LSE, LSEf[:, :, p.Nc:], atol=1e-13)
    for (b, h, g), s in sel.items():
        if g < p.nbc:
            assert max(s) < p.nbc and g in s            # condition rows never see noise cubes
        else:
            assert set(range(p.nbc)) | {g} <= set(s)    # noise rows see every condition cube
            assert list(idx[b, h, g - p.nbc]) == s
    # the full-sequence result against torch SDPA with the token-level block-causal mask
    ctok = orc.cond_cube_tokens(p)
    ntok = [t + p.Nc for t in orc.noise_cube_tokens(p)]
    all_tok = list(ctok) + ntok
    for b in range(2):
        for h in range(2):
            M = np.zeros((N, N), dtype=bool)
            for g in range(p.nbk):
                for j in sel[(b, h, g)]:
                    M[np.ix_(all_tok[g], all_tok[j])] = True
            assert not M[:p.Nc, p.Nc:].any()
            ref = _sdpa(qf[b:b + 1, :, h:h + 1], kf[b:b + 1, :, h:h + 1], vf[b:b + 1, :, h:h + 1],
                        scale, M)
            np.testing.assert_allclose(Of[b:b + 1, :, h:h + 1], ref, atol=1e-12)


@pytest.mark.parametrize("r", [0, 2, 5])
def test_ragged_grid_matches_torch_sdpa_with_token_mask(r):
    """Partial edge cubes (H = 9, W = 6 with 4x4 cube faces): the oracle's cube-level attention
    equals dense SDPA under the token mask of the selection, and LSE is the masked logsumexp."""
    p = orc.Problem(1, 2, 64, 4, 9, 6, 2, 4, 4, 0)
    rng = np.random.default_rng(21)
    x = {n: rng.standard_normal((1, p.Nq, 2, 64)) for n in ("q", "k", "v")}
    scale = 1 / math.sqrt(p.head_dim)
    qm, km = orc.block_pool(x["q"], p), orc.block_pool(x["k"], p)
    idx, _ = orc.select_topr(qm, km, p, r)
    O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], None, None, idx, p, scale)
    for h in range(2):
        M = _token_mask(p, idx[0, h])
        sl = slice(h, h + 1)
        ref = _sdpa(x["q"][:, :, sl], x["k"][:, :, sl], x["v"][:, :, sl], scale, M)
        np.testing.assert_allclose(O[:, :, sl], ref, atol=1e-12, rtol=0)
        s = scale * x["q"][0, :, h] @ x["k"][0, :, h].T
        s[~M] = -np.inf
        np.testing.assert_allclose(LSE[0, h], scipy.special.logsumexp(s, axis=1), atol=1e-12)
