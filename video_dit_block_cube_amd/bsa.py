"""Thin Python binding of libbsa.so (ctypes).  Argument marshalling only: every step of block
sparse attention runs in the library's HIP kernels.  torch supplies device memory and the stream.

The names mirror the C ABI declared in include/bsa.h: bsa_block_pool, bsa_select_topr,
bsa_sparse_attn_fwd, bsa_sparse_attn_bwd and the helpers.  Calls fail loudly (RuntimeError) when
the library is not built or cannot be loaded; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

BSA_F32, BSA_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 256 << 20     # BSA_NOALLOC_SCRATCH_BYTES of include/bsa.h
_DTYPES = {torch.float32: BSA_F32, torch.bfloat16: BSA_BF16}

STATUS = {0: "BSA_OK", 1: "BSA_ERR_INVALID_ARG", 2: "BSA_ERR_SHAPE", 3: "BSA_ERR_UNSUPPORTED",
          4: "BSA_ERR_WORKSPACE", 5: "BSA_ERR_HIP", 6: "BSA_ERR_INTERNAL"}


class BsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class bsa_problem_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads", "head_dim", "T", "H", "W", "cube_t", "cube_h", "cube_w",
                 "cond_T")]


@dataclass(frozen=True)
class Problem:
    """Problem shape (mirrors bsa_problem_t); derived sizes are for allocating outputs."""
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

    @property
    def c(self) -> int:
        return self.cube_t * self.cube_h * self.cube_w

    @property
    def Nq(self) -> int:
        return (self.T - self.cond_T) * self.H * self.W

    @property
    def Nc(self) -> int:
        return self.cond_T * self.H * self.W

    @property
    def _cubes_hw(self) -> int:
        # partial edge cubes on a ragged grid count as cubes
        return (-(-self.H // self.cube_h)) * (-(-self.W // self.cube_w))

    @property
    def nbq(self) -> int:
        return (self.T - self.cond_T) // self.cube_t * self._cubes_hw

    @property
    def nbc(self) -> int:
        return self.cond_T // self.cube_t * self._cubes_hw

    @property
    def nbk(self) -> int:
        return self.nbq + self.nbc

    def c_struct(self) -> bsa_problem_t:
        return bsa_problem_t(self.batch, self.heads, self.head_dim, self.T, self.H, self.W,
                             self.cube_t, self.cube_h, self.cube_w, self.cond_T)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libbsa.so (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m video_dit_block_cube_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(bsa_problem_t)
        vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        sigs = {
            "bsa_block_pool": (i32, [P, i32, vp, vp, vp]),
            "bsa_qk_prologue": (i32, [P, i32, i32, vp, vp, f32, f32, vp, vp, vp]),
            "bsa_select_topr": (i32, [P, vp, vp, i32, vp, vp, vp]),
            "bsa_sparse_attn_fwd": (i32, [P, i32, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp,
                                          sz, vp]),
            "bsa_sparse_attn_bwd": (i32, [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, f32,
                                          vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]),
            "bsa_num_selected": (i32, [P, i32]),
            "bsa_workspace_bytes": (sz, [P, i32, i32, i32]),
            "bsa_status_string": (ctypes.c_char_p, [i32]),
            "bsa_last_error": (ctypes.c_char_p, []),
            "bsa_set_stage_events": (None, [vp, i32]),
            "bsa_stage_count": (i32, []),
            "bsa_stage_name": (ctypes.c_char_p, [i32]),
            "bsa_set_kernel_path": (i32, [i32]),
            "bsa_set_tuning": (i32, [i32, i32]),
            "bsa_get_tuning": (i32, [i32]),
            "bsa_validate_idx": (i32, [P, vp, i32, vp, vp]),
            "bsa_sparse_attn_fwd_noalloc": (i32, [P, i32, vp, vp, vp, vp, vp, vp, i32, f32, vp,
                                                  vp, vp]),
            "bsa_probe_mfma": (i32, [vp, sz, i32, i32, vp, sz, vp]),
            "bsa_probe_mfma_shape": (i32, [vp, sz, i32, i32, i32, i32, vp, sz, vp]),
            "bsa_probe_mfma_valu": (i32, [vp, sz, i32, i32, i32, i32, i32, i32, vp, sz, vp]),
            "bsa_probe_tile_read": (i32, [vp, sz, i32, vp, sz, i32, i32, vp, sz, vp]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise BsaError(status, lib().bsa_last_error().decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t, name, shape=None, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")
    return _DTYPES[t.dtype]


def bsa_num_selected(p: Problem, r: int) -> int:
    return int(lib().bsa_num_selected(ctypes.byref(p.c_struct()), int(r)))


def bsa_workspace_bytes(p: Problem, dtype: torch.dtype, k_sel: int, bwd: bool) -> int:
    n = lib().bsa_workspace_bytes(ctypes.byref(p.c_struct()), _DTYPES[dtype], int(k_sel),
                                  1 if bwd else 0)
    if n == ctypes.c_size_t(-1).value:
        raise BsaError(1, lib().bsa_last_error().decode())
    return int(n)


def bsa_status_string(status: int) -> str:
    return lib().bsa_status_string(int(status)).decode()


def bsa_set_kernel_path(path: int) -> None:
    _check(lib().bsa_set_kernel_path(int(path)))


(BSA_TUNE_FWD_SPLITS, BSA_TUNE_DKDV_ORDER, BSA_TUNE_DQ_PIPELINE, BSA_TUNE_WALK_PHASE,
 BSA_TUNE_DKDV_SPLIT) = 0, 1, 2, 3, 4


def bsa_set_tuning(key: int, value: int) -> None:
    """Per-thread tuning switch (see include/bsa.h): forward key-range count (-1 automatic),
    longest-first dK/dV order, pipelined dQ, backward walk-phase period in microseconds (0 off;
    nondeterministic summation order when on), dK/dV split by keys (1) instead of by output."""
    _check(lib().bsa_set_tuning(int(key), int(value)))


def bsa_get_tuning(key: int) -> int:
    return int(lib().bsa_get_tuning(int(key)))


class tuning:
    """Context manager: set tuning switches on this thread, restore them on exit.
    Example: `with bsa.tuning(fwd_splits=1): ...`"""
    _KEYS = {"fwd_splits": BSA_TUNE_FWD_SPLITS, "dkdv_order": BSA_TUNE_DKDV_ORDER,
             "dq_pipeline": BSA_TUNE_DQ_PIPELINE, "walk_phase_us": BSA_TUNE_WALK_PHASE,
             "dkdv_split": BSA_TUNE_DKDV_SPLIT}

    def __init__(self, **settings):
        self.settings = {self._KEYS[k]: int(v) for k, v in settings.items()}
        self.saved = {}

    def __enter__(self):
        for key, value in self.settings.items():
            self.saved[key] = bsa_get_tuning(key)
            bsa_set_tuning(key, value)
        return self

    def __exit__(self, *exc):
        for key, value in self.saved.items():
            bsa_set_tuning(key, value)
        return False


def bsa_validate_idx(p: Problem, idx: torch.Tensor, k_sel: int) -> int:
    """Number of rows of idx that break the attention calls' contract (an entry outside
    [0, nbk) or a row not strictly ascending); synchronises the stream to read it."""
    bad = torch.empty(1, dtype=torch.int32, device=idx.device)
    _check(lib().bsa_validate_idx(ctypes.byref(p.c_struct()),
                                  _ptr(idx, "idx", (p.batch, p.heads, p.nbq, k_sel), torch.int32),
                                  int(k_sel), _ptr(bad, "bad_rows"), _stream(idx)))
    return int(bad.item())


def bsa_block_pool(p: Problem, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Per-cube mean of x [B, Nq, Hh, D] -> [B, Hh, nbq, D] fp32."""
    shape_x = (p.batch, p.Nq, p.heads, p.head_dim)
    if out is None:
        out = torch.empty((p.batch, p.heads, p.nbq, p.head_dim), dtype=torch.float32,
                          device=x.device)
    _check(lib().bsa_block_pool(ctypes.byref(p.c_struct()), _dtype_code(x),
                                _ptr(x, "x", shape_x),
                                _ptr(out, "x_mean", (p.batch, p.heads, p.nbq, p.head_dim),
                                     torch.float32),
                                _stream(x)))
    return out


def bsa_qk_prologue(p: Problem, x: torch.Tensor, gamma: torch.Tensor | None = None,
                    rope_theta: float = 10000.0, eps: float = 1e-6, segment: int = 0,
                    out: torch.Tensor | None = None, with_mean: bool = True,
                    mean: torch.Tensor | None = None):
    """RMS normalisation + 3D RoPE of one segment of q or k -> (x_out, cube means or None).

    segment 0: x [B, Nq, Hh, D] (noise frames); 1: x [B, cond_T*H*W, Hh, D] (condition frames,
    no means).  out may be x itself (in place)."""
    n = p.Nq if segment == 0 else p.cond_T * p.H * p.W
    shape_x = (p.batch, n, p.heads, p.head_dim)
    if out is None:
        out = torch.empty_like(x)
    if segment == 0 and with_mean and mean is None:
        mean = torch.empty((p.batch, p.heads, p.nbq, p.head_dim), dtype=torch.float32,
                           device=x.device)
    if segment != 0 or not with_mean:
        mean = None
    _check(lib().bsa_qk_prologue(
        ctypes.byref(p.c_struct()), _dtype_code(x), segment, _ptr(x, "x", shape_x),
        _ptr(gamma, "gamma", (p.head_dim,), torch.float32), rope_theta, eps,
        _ptr(out, "x_out", shape_x, x.dtype),
        _ptr(mean, "x_mean", (p.batch, p.heads, p.nbq, p.head_dim), torch.float32), _stream(x)))
    return out, mean


def bsa_select_topr(p: Problem, q_mean: torch.Tensor, k_mean: torch.Tensor, r: int,
                    with_mask: bool = True, idx: torch.Tensor | None = None,
                    mask: torch.Tensor | None = None):
    """-> (idx [B, Hh, nbq, k_sel] int32, mask [B, Hh, nbq, nbk] uint8 or None)."""
    ks = bsa_num_selected(p, r)
    if ks < 0:
        raise BsaError(1, lib().bsa_last_error().decode())
    shp = (p.batch, p.heads, p.nbq, p.head_dim)
    if idx is None:
        idx = torch.empty((p.batch, p.heads, p.nbq, ks), dtype=torch.int32, device=q_mean.device)
    if with_mask and mask is None:
        mask = torch.empty((p.batch, p.heads, p.nbq, p.nbk), dtype=torch.uint8,
                           device=q_mean.device)
    _check(lib().bsa_select_topr(ctypes.byref(p.c_struct()),
                                 _ptr(q_mean, "q_mean", shp, torch.float32),
                                 _ptr(k_mean, "k_mean", shp, torch.float32), int(r),
                                 _ptr(idx, "idx", (p.batch, p.heads, p.nbq, ks), torch.int32),
                                 _ptr(mask, "mask", (p.batch, p.heads, p.nbq, p.nbk), torch.uint8)
                                 if mask is not None else None,
                                 _stream(q_mean)))
    return idx, mask


def _workspace(p, dtype, k_sel, bwd, device, ws):
    need = bsa_workspace_bytes(p, dtype, k_sel, bwd)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, need


def bsa_sparse_attn_fwd(p: Problem, q, k, v, idx, k_sel: int, softmax_scale: float | None = None,
                        k_cache=None, v_cache=None, o=None, lse=None, workspace=None):
    """-> (o [B, Nq, Hh, D] input dtype, lse [B, Hh, Nq] fp32)."""
    scale = 1.0 / math.sqrt(p.head_dim) if softmax_scale is None else float(softmax_scale)
    shp = (p.batch, p.Nq, p.heads, p.head_dim)
    shc = (p.batch, p.Nc, p.heads, p.head_dim)
    dt = q.dtype
    if o is None:
        o = torch.empty(shp, dtype=dt, device=q.device)
    if lse is None:
        lse = torch.empty((p.batch, p.heads, p.Nq), dtype=torch.float32, device=q.device)
    ws, need = _workspace(p, dt, k_sel, False, q.device, workspace)
    _check(lib().bsa_sparse_attn_fwd(
        ctypes.byref(p.c_struct()), _dtype_code(q), _ptr(q, "q", shp, dt), _ptr(k, "k", shp, dt),
        _ptr(v, "v", shp, dt), _ptr(k_cache, "k_cache", shc, dt),
        _ptr(v_cache, "v_cache", shc, dt),
        _ptr(idx, "idx", (p.batch, p.heads, p.nbq, k_sel), torch.int32), int(k_sel),
        ctypes.c_float(scale), _ptr(o, "o", shp, dt),
        _ptr(lse, "lse", (p.batch, p.heads, p.Nq), torch.float32),
        _ptr(ws, "workspace") if ws is not None else None, ctypes.c_size_t(need if ws is None else ws.numel()),
        _stream(q)))
    return o, lse


def bsa_sparse_attn_fwd_noalloc(p: Problem, q, k, v, idx, k_sel: int,
                                softmax_scale: float | None = None, k_cache=None, v_cache=None,
                                o=None, lse=None):
    """bsa_sparse_attn_fwd with the library's static device scratch as workspace (no
    workspace argument, no allocation inside the call; o and lse must then be given)."""
    if o is None or lse is None:
        raise ValueError("the allocation-free forward writes into caller-provided o and lse")
    scale = 1.0 / math.sqrt(p.head_dim) if softmax_scale is None else float(softmax_scale)
    shp = (p.batch, p.Nq, p.heads, p.head_dim)
    shc = (p.batch, p.Nc, p.heads, p.head_dim)
    dt = q.dtype
    _check(lib().bsa_sparse_attn_fwd_noalloc(
        ctypes.byref(p.c_struct()), _dtype_code(q), _ptr(q, "q", shp, dt), _ptr(k, "k", shp, dt),
        _ptr(v, "v", shp, dt), _ptr(k_cache, "k_cache", shc, dt),
        _ptr(v_cache, "v_cache", shc, dt),
        _ptr(idx, "idx", (p.batch, p.heads, p.nbq, k_sel), torch.int32), int(k_sel),
        ctypes.c_float(scale), _ptr(o, "o", shp, dt),
        _ptr(lse, "lse", (p.batch, p.heads, p.Nq), torch.float32), _stream(q)))
    return o, lse


def bsa_sparse_attn_bwd(p: Problem, q, k, v, o, d_o, lse, idx, k_sel: int,
                        softmax_scale: float | None = None, dq=None, dk=None, dv=None,
                        workspace=None, k_cache=None, v_cache=None, dk_cache=None,
                        dv_cache=None, fwd_workspace=None):
    """-> (dq, dk, dv) fp32 [B, Nq, Hh, D]; with condition frames (k_cache, v_cache given)
    -> (dq, dk, dv, dk_cache, dv_cache), the last two [B, Nc, Hh, D].  fwd_workspace: the
    workspace of the forward call that produced o and lse (inputs unchanged since), whose
    gathered Q and K the backward then reuses."""
    scale = 1.0 / math.sqrt(p.head_dim) if softmax_scale is None else float(softmax_scale)
    shp = (p.batch, p.Nq, p.heads, p.head_dim)
    shc = (p.batch, p.Nc, p.heads, p.head_dim)
    dt = q.dtype
    dq = torch.empty(shp, dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty(shp, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(shp, dtype=torch.float32, device=q.device) if dv is None else dv
    cached = k_cache is not None
    if cached:
        dk_cache = torch.empty(shc, dtype=torch.float32, device=q.device) \
            if dk_cache is None else dk_cache
        dv_cache = torch.empty(shc, dtype=torch.float32, device=q.device) \
            if dv_cache is None else dv_cache
    ws, need = _workspace(p, dt, k_sel, True, q.device, workspace)
    _check(lib().bsa_sparse_attn_bwd(
        ctypes.byref(p.c_struct()), _dtype_code(q), _ptr(q, "q", shp, dt), _ptr(k, "k", shp, dt),
        _ptr(v, "v", shp, dt), _ptr(k_cache, "k_cache", shc, dt),
        _ptr(v_cache, "v_cache", shc, dt), _ptr(o, "o", shp, dt), _ptr(d_o, "d_o", shp, dt),
        _ptr(lse, "lse", (p.batch, p.heads, p.Nq), torch.float32),
        _ptr(idx, "idx", (p.batch, p.heads, p.nbq, k_sel), torch.int32), int(k_sel),
        ctypes.c_float(scale), _ptr(dq, "dq", shp, torch.float32),
        _ptr(dk, "dk", shp, torch.float32), _ptr(dv, "dv", shp, torch.float32),
        _ptr(dk_cache if cached else None, "dk_cache", shc, torch.float32),
        _ptr(dv_cache if cached else None, "dv_cache", shc, torch.float32),
        _ptr(fwd_workspace, "fwd_workspace"),
        ctypes.c_size_t(0 if fwd_workspace is None else fwd_workspace.numel()),
        _ptr(ws, "workspace"), ctypes.c_size_t(ws.numel()), _stream(q)))
    if cached:
        return dq, dk, dv, dk_cache, dv_cache
    return dq, dk, dv


# ---- stage timing with HIP events created through the HIP runtime itself ----
class StageEvents:
    """n HIP events handed to bsa_set_stage_events(); elapsed() gives per-stage milliseconds of
    the last instrumented call."""

    def __init__(self, n: int = 8):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.n = n
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = ev
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def __enter__(self):
        lib().bsa_set_stage_events(ctypes.cast(self.arr, ctypes.c_void_p), self.n)
        return self

    def __exit__(self, *exc):
        L = lib()
        L.bsa_set_stage_events(None, 0)
        count = min(L.bsa_stage_count(), self.n - 1)
        self.names = [L.bsa_stage_name(s).decode() for s in range(max(count, 0))]
        return False

    def elapsed_all(self):
        """[(stage name, ms)] for the stages of the call made inside this `with` block
        (synchronises on that call's last event)."""
        names = getattr(self, "names", [])
        if not names:
            return []
        self.hip.hipEventSynchronize(self.arr[len(names)])
        out = []
        for s, name in enumerate(names):
            ms = ctypes.c_float()
            self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[s], self.arr[s + 1])
            out.append((name, float(ms.value)))
        return out


# ---- diagnostics: microbenchmarks (see include/bsa.h) ----
def bsa_probe_mfma(operands: torch.Tensor, waves: int, iters: int, sink: torch.Tensor) -> None:
    """Back-to-back bf16 MFMA on `waves` waves, iters x 8 products each (32768 FLOP each)."""
    _check(lib().bsa_probe_mfma(_ptr(operands, "operands"), operands.numel() * operands.element_size(),
                                int(waves), int(iters), _ptr(sink, "sink"),
                                sink.numel() * sink.element_size(), _stream(operands)))


def bsa_probe_mfma_shape(operands: torch.Tensor, shape: int, chains: int, waves: int, iters: int,
                         sink: torch.Tensor) -> None:
    """Back-to-back bf16 MFMA of one shape (0: 32x32x16, 1: 16x16x32) with `chains` independent
    accumulators per wave, iters x 262144 FLOP per wave."""
    _check(lib().bsa_probe_mfma_shape(_ptr(operands, "operands"),
                                      operands.numel() * operands.element_size(), int(shape),
                                      int(chains), int(waves), int(iters), _ptr(sink, "sink"),
                                      sink.numel() * sink.element_size(), _stream(operands)))


def bsa_probe_mfma_valu(operands: torch.Tensor, mode: int, valu: int, op: int, acc: int,
                        workgroups: int, iters: int, sink: torch.Tensor) -> None:
    """bf16 MFMA beside VALU work on one SIMD (mode 0: interleaved in every wave; 1: split between
    the two waves of a SIMD; 2: products only; 3: VALU only), iters x 4 products per wave, each
    followed by `valu` VALU instructions (op 0: fma, 1: exp); accumulators in VGPRs (acc 0) or
    AGPRs (acc 1)."""
    _check(lib().bsa_probe_mfma_valu(_ptr(operands, "operands"),
                                     operands.numel() * operands.element_size(), int(mode),
                                     int(valu), int(op), int(acc), int(workgroups), int(iters),
                                     _ptr(sink, "sink"), sink.numel() * sink.element_size(),
                                     _stream(operands)))


def bsa_probe_tile_read(buf: torch.Tensor, tile_bytes: int, ids: torch.Tensor,
                        tiles_per_wave: int, sink: torch.Tensor) -> None:
    """Wave w reads tiles ids[w, :] of buf (tile_bytes each) as 1 KB wave loads."""
    waves = ids.numel() // int(tiles_per_wave)
    _check(lib().bsa_probe_tile_read(_ptr(buf, "buf"), buf.numel() * buf.element_size(),
                                     int(tile_bytes), _ptr(ids, "ids", dtype=torch.int32),
                                     ids.numel(), int(waves), int(tiles_per_wave),
                                     _ptr(sink, "sink"), sink.numel() * sink.element_size(),
                                     _stream(buf)))
