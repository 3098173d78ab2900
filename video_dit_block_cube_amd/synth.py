"""Seeded synthetic workloads for Block Sparse Attention (BSA) over 3D video latent cubes.

This module only DRAWS inputs.  It holds none of the attention method's arithmetic, and both the
HIP path and the CPU oracle consume what it returns.

Workloads (the LongCat-Video pages measure on generated 480p/720p video, which synthetic latent
grids stand in for here; sizes follow the latent compression the pages give, 4x in time and 16x16
in space per token, "美团LongCat-Video揭秘" (xugj520), section 三、模型架构):

  tiny        fp32, B=1, Hh=1,  D=64,  grid 4x8x8,   cube 2x4x4, r=2
  480p        bf16, B=1, Hh=32, D=128, grid 24x32x52, cube 4x4x4, r=62,  QKNorm on q, k
  720p        bf16, B=1, Hh=32, D=128, grid 24x48x80, cube 4x4x4, r=144, QKNorm on q, k
  continue    bf16, 720p grid, first 12 latent frames are condition frames (cached K/V), r=72,
              raw N(0,1) inputs
  480p-bwd    bf16, 480p shape, r=62, QKNorm on q, k, plus upstream gradient dO ~ N(0,1)

Recipe: numpy.random.default_rng(1000 + number) (PCG64) draws standard_normal float32 arrays in C
order, in the sequence q, k, v, k_cache, v_cache, dO, each shaped [B, N, Hh, D]; arrays a workload
does not use are not drawn.  q and k are RMS-normalised over D (x / sqrt(mean(x^2) + 1e-6), no
gain; the pages name RMSNorm + QKNorm without giving epsilon, xugj520 page, section 三、模型架构)
for the QKNorm workloads, in fp32.  bf16 workloads then round every array to bf16 with
round-to-nearest-even; the arrays returned are float32 holding those bf16 values exactly, so the
GPU receives the identical bits and the oracle upcasts them without loss.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    number: int          # 1..5, also fixes the seed 1000 + number
    name: str
    dtype: str           # "f32" or "bf16"
    batch: int
    heads: int
    head_dim: int
    T: int
    H: int
    W: int
    cube_t: int
    cube_h: int
    cube_w: int
    cond_T: int
    r: int
    qknorm: bool
    with_grad: bool      # draw dO

    @property
    def shape_dict(self) -> dict:
        return dict(batch=self.batch, heads=self.heads, head_dim=self.head_dim, T=self.T,
                    H=self.H, W=self.W, cube_t=self.cube_t, cube_h=self.cube_h,
                    cube_w=self.cube_w, cond_T=self.cond_T)

    @property
    def n_noise_tokens(self) -> int:
        return (self.T - self.cond_T) * self.H * self.W

    @property
    def n_cond_tokens(self) -> int:
        return self.cond_T * self.H * self.W


WORKLOADS = {
    1: Workload(1, "tiny-fp32", "f32", 1, 1, 64, 4, 8, 8, 2, 4, 4, 0, 2, False, False),
    2: Workload(2, "480p-bf16", "bf16", 1, 32, 128, 24, 32, 52, 4, 4, 4, 0, 62, True, False),
    3: Workload(3, "720p-bf16", "bf16", 1, 32, 128, 24, 48, 80, 4, 4, 4, 0, 144, True, False),
    4: Workload(4, "720p-continuation-bf16", "bf16", 1, 32, 128, 24, 48, 80, 4, 4, 4, 12, 72,
                False, False),
    5: Workload(5, "480p-bwd-bf16", "bf16", 1, 32, 128, 24, 32, 52, 4, 4, 4, 0, 62, True, True),
}


def workload(number: int, **overrides) -> Workload:
    """The named workload, optionally with fields replaced (e.g. fewer heads for a quick test)."""
    w = WORKLOADS[number]
    return replace(w, **overrides) if overrides else w


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even), returned as float32.

    Finite inputs only (the generators never produce NaN or Inf)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def rms_normalise(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Per-token, per-head RMS normalisation over the last axis in fp32 (input conditioning)."""
    x = np.asarray(x, dtype=np.float32)
    ms = np.mean(np.square(x, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
    return (x / np.sqrt(ms + np.float32(eps))).astype(np.float32)


def make_inputs(w: Workload) -> dict:
    """Draw the workload's arrays.  Keys: q, k, v (and k_cache, v_cache if cond_T > 0, dO if
    with_grad).  All float32 [B, N, Hh, D]; bf16 workloads hold bf16-exact values."""
    rng = np.random.default_rng(1000 + w.number)
    nq, nc = w.n_noise_tokens, w.n_cond_tokens
    shape_q = (w.batch, nq, w.heads, w.head_dim)
    shape_c = (w.batch, nc, w.heads, w.head_dim)
    out = {}
    order = [("q", shape_q), ("k", shape_q), ("v", shape_q)]
    if w.cond_T > 0:
        order += [("k_cache", shape_c), ("v_cache", shape_c)]
    if w.with_grad:
        order += [("dO", shape_q)]
    for name, shape in order:
        a = rng.standard_normal(size=shape, dtype=np.float32)
        if w.qknorm and name in ("q", "k"):
            a = rms_normalise(a)
        if w.dtype == "bf16":
            a = round_to_bf16(a)
        out[name] = a
    return out


def as_full_sequence(inputs: dict, key: str, cache_key: str) -> np.ndarray:
    """Concatenate a condition-frame array and a noise-frame array along the token axis
    (condition frames first, as in the latent grid)."""
    return np.concatenate([inputs[cache_key], inputs[key]], axis=1)
