"""Plain fp64 CPU oracle for the attention prologue that feeds BSA: QK normalisation and 3D RoPE.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this module:
only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg use it.  It shares no code,
table or helper with the HIP kernels and imports nothing from them.

What the pages fix: every 3D self-attention layer of the DiT normalises its queries and keys
(RMSNorm + QKNorm, "美团LongCat-Video揭秘：13.6B参数长视频生成模型如何终结画面漂移？",
xugj520, section "三、模型架构：Diffusion Transformer 的高维协奏") and encodes position with
rotary embeddings extended to the three axes time, height and width ("3D RoPE": same section;
"LongCat-Video deep dive", ai-news-5min-kr, the layer table row for the positional encoding;
"LongCat : Generate 1 minute long AI videos with this model", Data Science in Your Pocket, the
3D attention paragraph).  The pages give no formula, so
the readings below are the plainest ones:

  * normalisation: y = x / sqrt(mean_d x^2 + eps) * gamma over the head dimension, per (token,
    head), eps = 1e-6, gamma a per-channel gain (all ones when absent); applied before the
    rotation.
  * axes: the head dimension is cut into three contiguous blocks for (time, height, width) of
    widths D - 4*floor(D/6), 2*floor(D/6), 2*floor(D/6) (44, 42, 42 at D = 128).
  * rotation: inside a block of width d_a, channels (2i, 2i+1) are the real and imaginary parts of
    one complex number, multiplied by exp(1j * pos * theta^(-2i/d_a)), theta = 10000; pos is the
    token's integer coordinate on that axis of the full latent grid (condition frames first, so
    noise frame f sits at time position cond_T + f).

These readings are pinned by tests/test_oracle_prologue.py against mathematics, not against the
pages (which print no values): explicit rotations of unit vectors, group and relative-position
properties of rotations, and exact properties of RMS normalisation.
"""
from __future__ import annotations

import numpy as np

from .bsa_oracle import Problem, block_pool, check_problem

EPS = 1e-6
THETA = 10000.0


def axis_widths(head_dim: int) -> tuple[int, int, int]:
    """(time, height, width) channel counts of the 3D rotation."""
    s = 2 * (head_dim // 6)
    return head_dim - 2 * s, s, s


def token_positions(p: Problem, segment: str) -> np.ndarray:
    """[N, 3] integer (t, h, w) grid coordinates of the tokens of a segment, raster order.

    segment "noise": frames cond_T .. T-1 (N = Nq); "cond": frames 0 .. cond_T-1."""
    if segment == "noise":
        f0, f1 = p.cond_T, p.T
    elif segment == "cond":
        f0, f1 = 0, p.cond_T
    else:
        raise ValueError(segment)
    t, h, w = np.meshgrid(np.arange(f0, f1), np.arange(p.H), np.arange(p.W), indexing="ij")
    return np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1)


def rms_norm(x: np.ndarray, gamma=None, eps: float = EPS) -> np.ndarray:
    """x [..., D] -> x / sqrt(mean(x^2) + eps) * gamma, fp64."""
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    return y


def rope_3d(x: np.ndarray, pos: np.ndarray, theta: float = THETA) -> np.ndarray:
    """Rotate x [B, N, Hh, D] (fp64) by the 3D rotary embedding at positions pos [N, 3]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    out = np.empty_like(x)
    c0 = 0
    for axis, da in enumerate(axis_widths(D)):
        i = np.arange(da // 2)
        freq = theta ** (-2.0 * i / da)                          # [da/2]
        ang = pos[:, axis:axis + 1].astype(np.float64) * freq    # [N, da/2]
        cos = np.cos(ang)[None, :, None, :]
        sin = np.sin(ang)[None, :, None, :]
        xr = x[..., c0:c0 + da:2]
        xi = x[..., c0 + 1:c0 + da:2]
        out[..., c0:c0 + da:2] = xr * cos - xi * sin
        out[..., c0 + 1:c0 + da:2] = xr * sin + xi * cos
        c0 += da
    return out


def qk_prologue(x: np.ndarray, p: Problem, segment: str = "noise", gamma=None,
                theta: float = THETA, eps: float = EPS):
    """Normalise then rotate one segment's q or k [B, N, Hh, D]; for the noise segment also
    return the per-cube means of the result (the pool that feeds block selection), else None."""
    check_problem(p)
    y = rope_3d(rms_norm(x, gamma, eps), token_positions(p, segment), theta)
    return y, (block_pool(y, p) if segment == "noise" else None)
