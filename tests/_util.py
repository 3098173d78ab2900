"""Shared helpers of the GPU parity tests: device upload, tolerance checks, near-tie aware
selection comparison, cached workload inputs."""
from __future__ import annotations

import functools
import math

import numpy as np

import oracle as orc
from video_dit_block_cube_amd import synth

# Tolerances against the fp64 oracle.  Max-abs bounds are the contract (1e-4 fp32, 2e-2 bf16);
# the relative-L2 bounds are added because outputs and gradients here are small (|O| ~ 0.02 at
# the 480p/720p sizes), where a max-abs bound alone would not catch a wrong kernel.
TOL = {"f32": dict(max_abs=1e-4, rel_l2=1e-5), "bf16": dict(max_abs=2e-2, rel_l2=1e-2)}
NEAR_TIE = 1e-6


def print_case(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


@functools.lru_cache(maxsize=4)
def inputs_for(number: int, **overrides):
    w = synth.workload(number, **dict(overrides))
    return w, synth.make_inputs(w)


def cached_inputs(number: int, overrides: tuple = ()):
    return inputs_for(number, **dict(overrides))


def to_dev(a: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    return t.to(torch.bfloat16) if dtype == "bf16" else t.float()


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got, ref, dtype: str, what: str, max_abs=None, rel=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    ma = TOL[dtype]["max_abs"] if max_abs is None else max_abs
    rl = TOL[dtype]["rel_l2"] if rel is None else rel
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    r = rel_l2(got, ref) if got.size else 0.0
    assert err <= ma, f"{what}: max-abs {err:.3e} > {ma:.1e} (rel-L2 {r:.2e})"
    assert r <= rl, f"{what}: rel-L2 {r:.3e} > {rl:.1e} (max-abs {err:.2e})"
    return err, r


def check_selection(idx_gpu: np.ndarray, mask_gpu, qm_ref, km_ref, p: orc.Problem, r: int,
                    heads=None):
    """Bit-exact comparison of the selection with the oracle's, rows whose fp64 boundary gap is
    under 1e-6 excepted; those must still agree on every candidate at least 1e-6 away from the cut
    and on the row length.  Returns (rows compared exactly, near-tie rows)."""
    S = orc.block_scores(qm_ref, km_ref, p.head_dim)
    exact = ties = 0
    heads = range(p.heads) if heads is None else heads
    for b in range(p.batch):
        for h in heads:
            for i in range(p.nbq):
                ref = orc.select_row(S[b, h, i], i, p, r)
                got = idx_gpu[b, h, i]
                assert got.shape == ref.shape
                gap = orc.boundary_gap(S[b, h, i], i, p, r)
                if gap >= NEAR_TIE:
                    assert np.array_equal(got, ref), (b, h, i, got, ref)
                    exact += 1
                else:
                    ties += 1
                    assert np.all(np.diff(got) > 0)
                    cand = np.array([j for j in range(p.nbq) if j != i])
                    sc = np.sort(S[b, h, i, cand])[::-1]
                    rr = min(r, cand.size)
                    cut = 0.5 * (sc[rr - 1] + sc[rr])
                    far = np.abs(S[b, h, i] - cut) >= NEAR_TIE
                    far[i] = False
                    got_set = set(int(j) - p.nbc for j in got if j >= p.nbc)
                    ref_set = set(int(j) - p.nbc for j in ref if j >= p.nbc)
                    for j in np.nonzero(far)[0]:
                        assert (j in got_set) == (j in ref_set), (b, h, i, j)
                if mask_gpu is not None:
                    assert np.array_equal(np.nonzero(mask_gpu[b, h, i])[0], got)
    return exact, ties


def sample_rows(p, heads, per_head, seed=0):
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(p.batch):
        for h in heads:
            picks = set([0, p.nbq - 1]) | set(rng.integers(0, p.nbq, per_head - 2).tolist())
            rows += [(b, h, int(i)) for i in sorted(picks)]
    return rows


def scale_of(p) -> float:
    return 1.0 / math.sqrt(p.head_dim)


def torch_fwd_all_rows(op, t, idx_d, scale, chunk_pairs=600_000):
    """Every output row of the sparse forward recomputed on the device with plain torch fp32 ops
    (gather the tokens of each query cube's selected key cubes, softmax, weighted sum), for a
    grid whose sides are cube multiples.  A full-size cross-check of every row of the kernels,
    beside the fp64 oracle on sampled rows; the products run in fp32 on contiguous operands.
    Returns (O [B, Nq, Hh, D] fp32, LSE [B, Hh, Nq] fp32)."""
    import torch
    dev = t["q"].device
    B, Hh, D = op.batch, op.heads, op.head_dim
    qtok = torch.from_numpy(np.asarray(orc.noise_cube_tokens(op), dtype=np.int64)).to(dev)
    ktok = qtok
    out_o = torch.empty((B, op.Nq, Hh, D), dtype=torch.float32, device=dev)
    out_l = torch.empty((B, Hh, op.Nq), dtype=torch.float32, device=dev)
    ks = idx_d.shape[-1]
    n_chunk = max(1, chunk_pairs // (ks * 64))
    for b in range(B):
        for h in range(Hh):
            kn = t["k"][b, :, h].float()[ktok]                       # [nbq, c, D]
            vn = t["v"][b, :, h].float()[ktok]
            if op.nbc:
                ctok = torch.from_numpy(np.asarray(orc.cond_cube_tokens(op),
                                                   dtype=np.int64)).to(dev)
                kall = torch.cat([t["k_cache"][b, :, h].float()[ctok], kn])
                vall = torch.cat([t["v_cache"][b, :, h].float()[ctok], vn])
            else:
                kall, vall = kn, vn
            qall = t["q"][b, :, h].float()[qtok]                     # [nbq, c, D]
            sel_all = idx_d[b, h].long()
            for i0 in range(0, op.nbq, n_chunk):
                i1 = min(op.nbq, i0 + n_chunk)
                sel = sel_all[i0:i1]
                ksel = kall[sel].reshape(i1 - i0, ks * op.c, D)
                vsel = vall[sel].reshape(i1 - i0, ks * op.c, D).contiguous()
                s = torch.bmm(qall[i0:i1].contiguous(), ksel.transpose(1, 2).contiguous()) * scale
                lse = torch.logsumexp(s, dim=-1)
                o = torch.bmm(torch.exp(s - lse[..., None]), vsel)
                rows = qtok[i0:i1].reshape(-1)
                out_o[b, rows, h] = o.reshape(-1, D)
                out_l[b, h, rows] = lse.reshape(-1)
    return out_o, out_l


def torch_bwd_all(op, t, idx_d, scale, chunk_pairs=2_000_000):
    """Every gradient of the sparse backward recomputed on the device with plain torch fp32 ops,
    for a grid whose sides are cube multiples and no condition frames: per chunk of query cubes,
    gather the selected key cubes' tokens, form P = exp(S - LSE) and dS = P o (dO V^T - Delta)
    from the recomputed forward, dQ = scale dS K, and scatter-add scale dS^T Q and P^T dO into
    the key cubes.  A full-size cross-check of every element of the kernels' gradients, beside the
    fp64 oracle on sampled cubes.  Returns (dQ, dK, dV) [B, Nq, Hh, D] fp32."""
    import torch
    assert op.nbc == 0
    dev = t["q"].device
    B, Hh, D, c = op.batch, op.heads, op.head_dim, op.c
    tok = torch.from_numpy(np.asarray(orc.noise_cube_tokens(op), dtype=np.int64)).to(dev)
    out = [torch.zeros((B, op.Nq, Hh, D), dtype=torch.float32, device=dev) for _ in range(3)]
    ks = idx_d.shape[-1]
    n_chunk = max(1, chunk_pairs // (ks * c))
    slot = torch.arange(c, device=dev)
    for b in range(B):
        for h in range(Hh):
            q = t["q"][b, :, h].float()[tok]                          # [nbq, c, D]
            k = t["k"][b, :, h].float()[tok]
            v = t["v"][b, :, h].float()[tok]
            do = t["dO"][b, :, h].float()[tok]
            dk = torch.zeros((op.nbq * c, D), dtype=torch.float32, device=dev)
            dv = torch.zeros_like(dk)
            dq = torch.empty((op.nbq, c, D), dtype=torch.float32, device=dev)
            sel_all = idx_d[b, h].long()
            for i0 in range(0, op.nbq, n_chunk):
                i1 = min(op.nbq, i0 + n_chunk)
                n = i1 - i0
                sel = sel_all[i0:i1]
                kt = k[sel].reshape(n, ks * c, D)
                vt = v[sel].reshape(n, ks * c, D)
                qi, doi = q[i0:i1].contiguous(), do[i0:i1].contiguous()
                s = torch.bmm(qi, kt.transpose(1, 2).contiguous()) * scale
                p = torch.exp(s - torch.logsumexp(s, dim=-1, keepdim=True))
                o = torch.bmm(p, vt.contiguous())
                delta = (o * doi).sum(-1, keepdim=True)
                dp = torch.bmm(doi, vt.transpose(1, 2).contiguous())
                ds = p * (dp - delta)
                dq[i0:i1] = scale * torch.bmm(ds, kt.contiguous())
                rows = (sel[:, :, None] * c + slot).reshape(-1)           # key tokens, cube order
                dk.index_add_(0, rows, (scale * torch.bmm(ds.transpose(1, 2).contiguous(), qi))
                              .reshape(-1, D))
                dv.index_add_(0, rows, torch.bmm(p.transpose(1, 2).contiguous(), doi).reshape(-1, D))
            flat = tok.reshape(-1)
            out[0][b, flat, h] = dq.reshape(-1, D)
            out[1][b, flat, h] = dk
            out[2][b, flat, h] = dv
    return tuple(out)
