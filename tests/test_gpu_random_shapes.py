"""Seeded random sweep of problem shapes through pool, select, forward and backward against the
fp64 oracle (through the C ABI): cube shapes (64-token cubes take the MFMA path, others the
portable one), head dims, dtypes, ragged grids, condition frames, top-r and batch, in
combinations no hand-written case covers.  Sizes stay small enough for the oracle."""
import numpy as np
import pytest

import oracle as orc
from tests._util import assert_close, check_selection, print_case, scale_of, to_dev
from video_dit_block_cube_amd import bsa, synth

pytestmark = pytest.mark.gpu

CUBES = [(4, 4, 4), (2, 4, 4), (4, 2, 8), (1, 8, 8), (2, 3, 5), (4, 8, 8), (1, 1, 1), (2, 2, 2)]


def _case(seed):
    rng = np.random.default_rng(seed)
    ct, ch, cw = CUBES[seed % len(CUBES)]
    D = int(rng.choice([64, 128]))
    dtype = "bf16" if (seed % 3) else "f32"
    gt = int(rng.integers(1, 3))
    cond_t = int(rng.integers(0, 2)) if seed % 2 == 0 else 0
    gh = int(rng.integers(1, 4)) if ch > 1 else 4
    gw = int(rng.integers(2, 5)) if cw > 1 else 6
    H = gh * ch - (int(rng.integers(0, ch)) if ch > 1 and seed % 4 == 1 else 0)   # ragged
    W = gw * cw - (int(rng.integers(0, cw)) if cw > 1 and seed % 4 == 3 else 0)   # ragged
    shape = dict(batch=int(rng.integers(1, 3)), heads=int(rng.integers(1, 3)), head_dim=D,
                 T=(gt + cond_t) * ct, H=max(H, 1), W=max(W, 1), cube_t=ct, cube_h=ch,
                 cube_w=cw, cond_T=cond_t * ct)
    op = orc.Problem(**shape)
    r = int(rng.integers(0, max(op.nbq, 1) + 1))
    return shape, dtype, r


@pytest.mark.parametrize("seed", range(16))
def test_random_shape(seed):
    import torch
    shape, dtype, r = _case(seed)
    print_case(f"random shape seed={seed} {shape} {dtype} r={r}")
    p, op = bsa.Problem(**shape), orc.Problem(**shape)
    rng = np.random.default_rng(500 + seed)

    def draw(n):
        a = rng.standard_normal((op.batch, n, op.heads, op.head_dim)).astype(np.float32)
        return synth.round_to_bf16(a) if dtype == "bf16" else a
    x = {"q": draw(op.Nq), "k": draw(op.Nq), "v": draw(op.Nq), "dO": draw(op.Nq)}
    if op.cond_T:
        x["k_cache"], x["v_cache"] = draw(op.Nc), draw(op.Nc)
    t = {k: to_dev(v, dtype) for k, v in x.items()}
    # pool and select against the oracle
    qm, km = bsa.bsa_block_pool(p, t["q"]), bsa.bsa_block_pool(p, t["k"])
    rq, rk = orc.block_pool(x["q"], op), orc.block_pool(x["k"], op)
    np.testing.assert_allclose(qm.cpu().numpy(), rq, rtol=1e-6, atol=1e-6)
    idx_d, mask = bsa.bsa_select_topr(p, qm, km, r)
    check_selection(idx_d.cpu().numpy(), mask.cpu().numpy(), rq, rk, op, r)
    # attention on the oracle's selection
    idx, _ = orc.select_topr(rq, rk, op, r)
    idx_t = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to("cuda:0")
    ks, scale = orc.num_selected(op, r), scale_of(op)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx_t, ks, scale,
                                     t.get("k_cache"), t.get("v_cache"))
    O, LSE = orc.sparse_attn_fwd(x["q"], x["k"], x["v"], x.get("k_cache"), x.get("v_cache"), idx,
                                 op, scale)
    assert_close(o.float().cpu().numpy(), O, dtype, "O")
    assert_close(lse.cpu().numpy(), LSE, dtype, "LSE", max_abs=1e-4 if dtype == "f32" else 2e-3,
                 rel=1e-5)
    # backward (condition-cache gradients exist on the bf16 64-token path only)
    cache_ok = op.cond_T == 0 or (dtype == "bf16" and op.c == 64)
    if not cache_ok:
        with pytest.raises(bsa.BsaError):
            bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx_t, ks, scale,
                                    k_cache=t.get("k_cache"), v_cache=t.get("v_cache"))
        return
    got = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx_t, ks, scale,
                                  k_cache=t.get("k_cache"), v_cache=t.get("v_cache"))
    ref = orc.attn_bwd(x["q"], x["k"], x["v"], x["dO"], idx, op, scale,
                       k_cache=x.get("k_cache"), v_cache=x.get("v_cache"))
    for name, g, rf in zip(("dQ", "dK", "dV", "dK_cache", "dV_cache"), got, ref):
        assert_close(g.cpu().numpy(), rf, dtype, name)
