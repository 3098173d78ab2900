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
