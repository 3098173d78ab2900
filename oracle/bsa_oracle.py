"""Plain fp64 CPU oracle for Block Sparse Attention (BSA) over 3D video latent cubes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this module:
only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg use it.  It shares no code,
table or helper with the HIP kernels and imports nothing from them.

What it computes, step by step, in the order the LongCat-Video pages describe the method:

  1. cube partition of the latent grid: tokens are grouped into small 3D cubes
     ("LongCat-Video : Generate 1 minute long AI videos with this model", Data Science in Your
     Pocket, section "Sparse attention"; "LongCat-Video视频生成模型发布 迈出世界模型探索第一步",
     youleyou, section "块稀疏注意力（BSA）")                         -> segment_cube_tokens
  2. a relevance descriptor per cube (mean of its tokens) and a similarity score between cubes
     (Data Science in Your Pocket, "Sparse attention": cubes chosen by similarity, not distance)
                                                                      -> block_pool, block_scores
  3. each query cube keeps its own cube and its top-r key cubes (youleyou, "块稀疏注意力（BSA）";
     own cube kept: "LongCat-Video deep dive", ai-news-5min-kr, same-table analogy of the
     block-sparse attention paragraph)                                 -> select_topr
  4. attention restricted to the selected cube pairs, unselected pairs skipped entirely
     (ai-news-5min-kr deep dive, block-sparse attention paragraph)     -> attn_fwd_rows
  5. block-causal continuation with cached condition K/V ("LongCat-Video 高效長視頻生成探索世界
     模型的第壹步", meituan.com talk, section 2.1; youleyou, section "长视频生成：5分钟连贯输出，
     质量全程在线"; Data Science in Your Pocket, "The core idea: one model for all video tasks")
                                                                      -> attn_fwd_rows (cache),
                                                                         full_block_causal_fwd
  6. backward for training (meituan.com talk, section 2.2), including the gradients of the
     cached condition K/V for continuation training                   -> attn_bwd

Readings where the pages are silent (pool = arithmetic mean, score = D^-1/2 <q_mean, k_mean>,
self forced and r counted on top of it, ties to the lower cube id, raster cube order, no gradient
through the selection) are the plainest ones the rest supports; each is stated where it is used.

All arithmetic is fp64 on numpy arrays; inputs of any float dtype are upcast on read.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from functools import lru_cache

import numpy as np


class ProblemError(ValueError):
    """Raised for an invalid problem; `kind` is "invalid", "shape" or "unsupported"."""

    def __init__(self, kind: str, msg: str):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


@dataclass(frozen=True)
class Problem:
    batch: int
    heads: int
    head_dim: int
    T: int
    H: int
    W: int
    cube_t: int
    cube_h: int
    cube_w: int
    cond_T: int = 0

    # ---- derived sizes ----
    @property
    def c(self) -> int:
        return self.cube_t * self.cube_h * self.cube_w

    @property
    def noise_T(self) -> int:
        return self.T - self.cond_T

    @property
    def Nq(self) -> int:
        return self.noise_T * self.H * self.W

    @property
    def Nc(self) -> int:
        return self.cond_T * self.H * self.W

    def cubes_in(self, frames: int) -> int:
        # reading: partial edge cubes along H and W (ragged latent grids) count as cubes
        return (frames // self.cube_t) * (-(-self.H // self.cube_h)) * (-(-self.W // self.cube_w))

    @property
    def nbq(self) -> int:
        return self.cubes_in(self.noise_T)

    @property
    def nbc(self) -> int:
        return self.cubes_in(self.cond_T)

    @property
    def nbk(self) -> int:
        return self.nbc + self.nbq


def check_problem(p: Problem) -> None:
    """Shape rules of the problem (the same rules the C interface enforces)."""
    for name in ("batch", "heads", "head_dim", "T", "H", "W", "cube_t", "cube_h", "cube_w"):
        if getattr(p, name) <= 0:
            raise ProblemError("invalid", f"{name} must be positive")
    if p.cond_T < 0:
        raise ProblemError("invalid", "cond_T must be >= 0")
    if p.cond_T >= p.T:
        raise ProblemError("shape", "cond_T must be < T")
    if p.noise_T % p.cube_t or p.cond_T % p.cube_t:
        raise ProblemError("shape", "frame counts not divisible by the cube")


def num_selected(p: Problem, r: int) -> int:
    """Selected cubes per query cube: every condition cube, the own cube, and min(r, nbq-1)."""
    return p.nbc + 1 + min(r, p.nbq - 1)


# --------------------------------------------------------------------------------------------
# Step 1: cube partition (reading: raster order over cube coordinates, t slowest, then h, then w;
# inside a cube, raster order over (dt, dh, dw)).  Reading for ragged latent grids (H or W not a
# multiple of the cube side, e.g. the 45-token height of 720p): the last cube row / column keeps
# only the tokens of its box that lie inside the grid.
# --------------------------------------------------------------------------------------------
@lru_cache(maxsize=16)
def _segment_cube_tokens_cached(frames, H, W, ct, ch, cw):
    nt, nh, nw = frames // ct, -(-H // ch), -(-W // cw)
    out = []
    for a in range(nt):
        for b in range(nh):
            for e in range(nw):
                members = []
                for dt in range(ct):
                    for dh in range(ch):
                        for dw in range(cw):
                            t, h, w = a * ct + dt, b * ch + dh, e * cw + dw
                            if h < H and w < W:
                                members.append((t * H + h) * W + w)
                arr = np.array(members, dtype=np.int64)
                arr.setflags(write=False)
                out.append(arr)
    return tuple(out)


def segment_cube_tokens(p: Problem, frames: int) -> tuple:
    """Per cube of a segment of `frames` frames, the int64 array of its token indices (raster
    order inside the segment), cube by cube in raster cube order; every array has c entries
    unless the cube sits on a ragged edge."""
    return _segment_cube_tokens_cached(frames, p.H, p.W, p.cube_t, p.cube_h, p.cube_w)


def noise_cube_tokens(p: Problem) -> np.ndarray:
    return segment_cube_tokens(p, p.noise_T)


def cond_cube_tokens(p: Problem) -> np.ndarray:
    return segment_cube_tokens(p, p.cond_T)


# --------------------------------------------------------------------------------------------
# Step 2: per-cube descriptor and cube-to-cube similarity.
# Reading: the descriptor is the arithmetic mean of the cube's token vectors, per head; the score
# is the scaled dot product D^-1/2 <q_mean_i, k_mean_j>, the same similarity attention itself uses.
# --------------------------------------------------------------------------------------------
def block_pool(x: np.ndarray, p: Problem) -> np.ndarray:
    """x: [B, Nq, Hh, D] (noise segment) -> [B, Hh, nbq, D] fp64 means over each cube."""
    check_problem(p)
    toks = noise_cube_tokens(p)
    B, N, Hh, D = x.shape
    assert N == p.Nq and Hh == p.heads and D == p.head_dim
    out = np.empty((B, Hh, p.nbq, D), dtype=np.float64)
    for i in range(p.nbq):
        members = np.asarray(x[:, toks[i], :, :], dtype=np.float64)  # [B, c_i, Hh, D]
        out[:, :, i, :] = members.sum(axis=1) / len(toks[i])
    return out


def block_scores(q_mean: np.ndarray, k_mean: np.ndarray, head_dim: int) -> np.ndarray:
    """[..., nq, D] x [..., nk, D] -> [..., nq, nk] = D^-1/2 q_mean k_mean^T (fp64)."""
    qm = np.asarray(q_mean, dtype=np.float64)
    km = np.asarray(k_mean, dtype=np.float64)
    return np.matmul(qm, np.swapaxes(km, -1, -2)) / math.sqrt(head_dim)


# --------------------------------------------------------------------------------------------
# Step 3: forced set + top-r.
# Readings: the own cube is always kept and r more are chosen among the OTHER noise cubes; all
# condition cubes are always kept (continuation); ties go to the lower cube id; -0.0 == +0.0.
# Key cube ids: condition cubes 0..nbc-1, then noise cubes nbc..nbc+nbq-1.
# --------------------------------------------------------------------------------------------
def select_row(scores_row: np.ndarray, i: int, p: Problem, r: int) -> np.ndarray:
    """One query cube: ascending array of selected key cube ids (length num_selected(p, r))."""
    cand = np.array([j for j in range(p.nbq) if j != i], dtype=np.int64)
    sc = np.asarray(scores_row, dtype=np.float64)[cand] + 0.0
    order = np.lexsort((cand, -sc))                 # primary: score descending; then id asc
    chosen = cand[order[: min(r, cand.size)]]
    sel = list(range(p.nbc)) + [p.nbc + i] + [p.nbc + int(j) for j in chosen]
    return np.array(sorted(sel), dtype=np.int64)


def select_topr(q_mean: np.ndarray, k_mean: np.ndarray, p: Problem, r: int):
    """-> (idx [B, Hh, nbq, k_sel] int32 ascending, mask [B, Hh, nbq, nbk] uint8)."""
    check_problem(p)
    if r < 0:
        raise ProblemError("invalid", "r must be >= 0")
    S = block_scores(q_mean, k_mean, p.head_dim)
    ks = num_selected(p, r)
    B, Hh = S.shape[0], S.shape[1]
    idx = np.empty((B, Hh, p.nbq, ks), dtype=np.int32)
    mask = np.zeros((B, Hh, p.nbq, p.nbk), dtype=np.uint8)
    for b in range(B):
        for h in range(Hh):
            for i in range(p.nbq):
                sel = select_row(S[b, h, i], i, p, r)
                idx[b, h, i] = sel
                mask[b, h, i, sel] = 1
    return idx, mask


def boundary_gap(scores_row: np.ndarray, i: int, p: Problem, r: int) -> float:
    """Score gap between the last chosen and the first unchosen candidate of a row (inf when
    every candidate is chosen).  Rows with a gap under 1e-6 count as near-ties."""
    cand = np.array([j for j in range(p.nbq) if j != i], dtype=np.int64)
    sc = np.sort(np.asarray(scores_row, dtype=np.float64)[cand])[::-1]
    rr = min(r, cand.size)
    if rr >= cand.size or rr == 0:
        return math.inf
    return float(sc[rr - 1] - sc[rr])


# --------------------------------------------------------------------------------------------
# Step 4/5: attention over the selected cubes.  Reading: softmax scale is passed in (D^-1/2 in
# practice), no dropout, no bias; condition cubes read the cached K/V.
# --------------------------------------------------------------------------------------------
def _gather_keys(x: np.ndarray, x_cache, sel, b: int, h: int, p: Problem) -> np.ndarray:
    """Token rows of the selected key cubes, cube after cube in the order of `sel`."""
    qt, ctok = noise_cube_tokens(p), (cond_cube_tokens(p) if p.nbc else None)
    parts = []
    for j in sel:
        j = int(j)
        if j < p.nbc:
            parts.append(np.asarray(x_cache[b, ctok[j], h, :], dtype=np.float64))
        else:
            parts.append(np.asarray(x[b, qt[j - p.nbc], h, :], dtype=np.float64))
    return np.concatenate(parts, axis=0)


def attn_fwd_row(q, k, v, k_cache, v_cache, idx, p: Problem, scale: float, b: int, h: int,
                 i: int):
    """One query cube -> (O_i [c, D], LSE_i [c]) in fp64."""
    qt = noise_cube_tokens(p)
    Qi = np.asarray(q[b, qt[i], h, :], dtype=np.float64)
    sel = idx[b, h, i]
    Ks = _gather_keys(k, k_cache, sel, b, h, p)
    Vs = _gather_keys(v, v_cache, sel, b, h, p)
    s = scale * (Qi @ Ks.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    O = (e @ Vs) / l
    lse = (m + np.log(l))[:, 0]
    return O, lse


def attn_fwd_rows(q, k, v, k_cache, v_cache, idx, p: Problem, scale: float, rows):
    """{(b, h, i): (O_i, LSE_i)} for the listed query cubes."""
    check_problem(p)
    return {(b, h, i): attn_fwd_row(q, k, v, k_cache, v_cache, idx, p, scale, b, h, i)
            for (b, h, i) in rows}


def sparse_attn_fwd(q, k, v, k_cache, v_cache, idx, p: Problem, scale: float, heads=None):
    """Full forward: O [B, Nq, Hh, D] fp64 and LSE [B, Hh, Nq] fp64.  `heads` restricts the
    computed heads (the others are left NaN)."""
    check_problem(p)
    B, Hh, D = p.batch, p.heads, p.head_dim
    qt = noise_cube_tokens(p)
    O = np.full((B, p.Nq, Hh, D), np.nan)
    LSE = np.full((B, Hh, p.Nq), np.nan)
    for b in range(B):
        for h in (range(Hh) if heads is None else heads):
            for i in range(p.nbq):
                Oi, li = attn_fwd_row(q, k, v, k_cache, v_cache, idx, p, scale, b, h, i)
                O[b, qt[i], h, :] = Oi
                LSE[b, h, qt[i]] = li
    return O, LSE


# --------------------------------------------------------------------------------------------
# Step 6: backward, selection held constant (the top-r choice is discrete and gets no gradient).
# Reading: Delta is computed from the oracle's own fp64 output.
# --------------------------------------------------------------------------------------------
def attn_bwd(q, k, v, dO, idx, p: Problem, scale: float, rows=None, key_cubes=None,
             k_cache=None, v_cache=None):
    """Gradients of L = <dO, O> with respect to q, k, v and, with condition frames, the cached
    condition k_cache, v_cache (the continuation mode: the cache is read by every noise query).

    rows:      None for every query cube, else an iterable of (b, h, i) whose dQ is wanted.
    key_cubes: None for every key cube, else an iterable of (b, h, j) whose dK, dV are wanted,
               j a key cube id (condition cubes 0..nbc-1 first, then noise cubes).
    Full mode (no selector): fp64 arrays dQ, dK, dV [B, Nq, Hh, D], plus dK_cache, dV_cache
    [B, Nc, Hh, D] when cond_T > 0.  Selector mode: dicts keyed like rows / key_cubes ([c, D]
    fp64 each; condition key cubes sit in the dK, dV dicts under their ids), plus (None, None)
    when cond_T > 0."""
    check_problem(p)
    cached = p.cond_T > 0
    if cached and (k_cache is None or v_cache is None):
        raise ProblemError("invalid", "condition frames need k_cache and v_cache")
    qt = noise_cube_tokens(p)
    ct_ = cond_cube_tokens(p) if cached else ()
    D = p.head_dim
    full = rows is None and key_cubes is None
    want_rows = None if rows is None else set(map(tuple, rows))
    want_cols = None if key_cubes is None else set(map(tuple, key_cubes))
    if full:
        dQ = np.zeros((p.batch, p.Nq, p.heads, D))
        dK = np.zeros_like(dQ)
        dV = np.zeros_like(dQ)
        dKc = np.zeros((p.batch, p.Nc, p.heads, D)) if cached else None
        dVc = np.zeros_like(dKc) if cached else None
    else:
        dQ, dK, dV = {}, {}, {}
        for key in want_cols or ():
            j = key[2]
            n = len(ct_[j]) if j < p.nbc else len(qt[j - p.nbc])
            dK[key] = np.zeros((n, D))
            dV[key] = np.zeros((n, D))
    for b in range(p.batch):
        for h in range(p.heads):
            for i in range(p.nbq):
                sel = idx[b, h, i]
                need_q = full or (want_rows is not None and (b, h, i) in want_rows)
                cols_here = [] if want_cols is None else \
                    [pos for pos, j in enumerate(sel) if (b, h, int(j)) in want_cols]
                if not (full or need_q or cols_here):
                    continue
                Qi = np.asarray(q[b, qt[i], h, :], dtype=np.float64)
                dOi = np.asarray(dO[b, qt[i], h, :], dtype=np.float64)
                Ks = _gather_keys(k, k_cache, sel, b, h, p)
                Vs = _gather_keys(v, v_cache, sel, b, h, p)
                s = scale * (Qi @ Ks.T)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                P = e / l                                   # = exp(s - LSE)
                Oi = P @ Vs
                delta = np.sum(dOi * Oi, axis=1, keepdims=True)
                dP = dOi @ Vs.T
                dS = P * (dP - delta)
                dKs = scale * (dS.T @ Qi)                   # [keys, D], cube after cube
                dVs = P.T @ dOi
                ends = np.cumsum([len(ct_[int(j)] if int(j) < p.nbc else qt[int(j) - p.nbc])
                                  for j in sel])
                starts = np.concatenate([[0], ends[:-1]])
                if full:
                    dQ[b, qt[i], h, :] += scale * (dS @ Ks)
                    for pos, j in enumerate(sel):
                        j = int(j)
                        if j < p.nbc:
                            dKc[b, ct_[j], h, :] += dKs[starts[pos]:ends[pos]]
                            dVc[b, ct_[j], h, :] += dVs[starts[pos]:ends[pos]]
                        else:
                            dK[b, qt[j - p.nbc], h, :] += dKs[starts[pos]:ends[pos]]
                            dV[b, qt[j - p.nbc], h, :] += dVs[starts[pos]:ends[pos]]
                else:
                    if need_q:
                        dQ[(b, h, i)] = scale * (dS @ Ks)
                    for pos in cols_here:
                        key = (b, h, int(sel[pos]))
                        dK[key] += dKs[starts[pos]:ends[pos]]
                        dV[key] += dVs[starts[pos]:ends[pos]]
    if not cached:
        return dQ, dK, dV
    if full:
        return dQ, dK, dV, dKc, dVc
    return dQ, dK, dV, None, None


def delta_rows(o: np.ndarray, dO: np.ndarray) -> np.ndarray:
    """Delta[b, h, n] = sum_d dO[b, n, h, d] * O[b, n, h, d] (fp64), for [B, N, Hh, D] inputs."""
    return np.einsum("bnhd,bnhd->bhn", np.asarray(dO, np.float64), np.asarray(o, np.float64))


def transpose_selection(idx: np.ndarray, nbk: int):
    """CSR transpose of the selection of one (b, h): for each key cube j, the ascending list of
    query cubes whose row contains j.  -> (offsets [nbk+1], lists [sum])."""
    lists = [[] for _ in range(nbk)]
    for i, row in enumerate(idx):
        for j in row:
            lists[int(j)].append(i)
    offsets = np.zeros(nbk + 1, dtype=np.int64)
    for j in range(nbk):
        offsets[j + 1] = offsets[j] + len(lists[j])
    flat = np.array([i for j in range(nbk) for i in lists[j]], dtype=np.int64)
    return offsets, flat


# --------------------------------------------------------------------------------------------
# Full-sequence block-causal attention (used only to check the cached continuation mode).
# Reading: condition queries attend condition cubes only (own cube + top-r among the others);
# noise queries attend every condition cube, their own cube and their top-r noise cubes; there
# is no causality inside the noise segment.
# --------------------------------------------------------------------------------------------
def full_block_causal_fwd(q_full, k_full, v_full, p: Problem, r: int, r_cond: int,
                          scale: float, heads=None):
    """q_full, k_full, v_full: [B, T*H*W, Hh, D] over the whole grid (condition frames first).
    Returns (O [B, T*H*W, Hh, D], LSE [B, Hh, T*H*W], sel) where sel[(b, h, g)] is the ascending
    list of global key cube ids attended by global query cube g (ids: condition cubes, then noise
    cubes, as for the cached mode)."""
    check_problem(p)
    nbc, nbq = p.nbc, p.nbq
    ctok = cond_cube_tokens(p)
    ntok = [t + p.Nc for t in noise_cube_tokens(p)]
    all_tok = list(ctok) + ntok
    B, N, Hh, D = q_full.shape
    O = np.full((B, N, Hh, D), np.nan)
    LSE = np.full((B, Hh, N), np.nan)
    sel_out = {}
    for b in range(B):
        for h in (range(Hh) if heads is None else heads):
            qm = np.stack([np.asarray(q_full[b, all_tok[g], h, :], np.float64).mean(axis=0)
                           for g in range(nbc + nbq)])
            km = np.stack([np.asarray(k_full[b, all_tok[g], h, :], np.float64).mean(axis=0)
                           for g in range(nbc + nbq)])
            S = block_scores(qm, km, D)
            for g in range(nbc + nbq):
                if g < nbc:
                    cand = np.array([j for j in range(nbc) if j != g], dtype=np.int64)
                    rr = min(r_cond, cand.size)
                    forced = [g]
                else:
                    cand = np.array([j for j in range(nbc, nbc + nbq) if j != g], dtype=np.int64)
                    rr = min(r, cand.size)
                    forced = list(range(nbc)) + [g]
                sc = S[g, cand] + 0.0
                chosen = cand[np.lexsort((cand, -sc))[:rr]]
                sel = sorted(forced + [int(j) for j in chosen])
                sel_out[(b, h, g)] = sel
                Qg = np.asarray(q_full[b, all_tok[g], h, :], np.float64)
                Ks = np.concatenate([np.asarray(k_full[b, all_tok[j], h, :], np.float64)
                                     for j in sel])
                Vs = np.concatenate([np.asarray(v_full[b, all_tok[j], h, :], np.float64)
                                     for j in sel])
                s = scale * (Qg @ Ks.T)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                O[b, all_tok[g], h, :] = (e @ Vs) / l
                LSE[b, h, all_tok[g]] = (m + np.log(l))[:, 0]
    return O, LSE, sel_out
