"""The C ABI library loads, exports every symbol include/bsa.h declares, and rejects bad
arguments on the host before any HIP call (CPU only: no kernel is launched here)."""
import ctypes
import os
import re

import pytest

from video_dit_block_cube_amd import bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")

OK, INVALID, SHAPE, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3, 4
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every case below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bsa.LIB_PATH):
        pytest.fail("libbsa.so is not built (run __graft_entry__.build())")
    return bsa.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), f"{n} declared in bsa.h but not exported"


def _p(**kw):
    base = dict(batch=1, heads=2, head_dim=128, T=8, H=8, W=8, cube_t=4, cube_h=4, cube_w=4,
                cond_T=0)
    base.update(kw)
    return bsa.Problem(**base).c_struct()


def test_num_selected_and_workspace(L):
    assert L.bsa_num_selected(ctypes.byref(_p()), 2) == 3
    assert L.bsa_num_selected(ctypes.byref(_p()), 100) == 8          # clamped to nbq
    assert L.bsa_num_selected(ctypes.byref(_p(T=8, cond_T=4)), 0) == 4 + 1
    assert L.bsa_num_selected(ctypes.byref(_p()), -1) == -1
    assert L.bsa_num_selected(ctypes.byref(_p(T=7)), 1) == -1
    assert L.bsa_num_selected(ctypes.byref(_p(W=10)), 100) == 2 * 2 * 3       # ragged: 3 along w
    big = bsa.Problem(1, 32, 128, 24, 48, 80, 4, 4, 4)
    assert bsa.bsa_num_selected(big, 144) == 145
    import torch
    gathers = 3 * 32 * 1440 * 64 * 128 * 2                           # Q, K rows + V^T, bf16
    fwd = bsa.bsa_workspace_bytes(big, torch.bfloat16, 145, False)
    assert fwd > gathers                                             # + key-range partials
    with bsa.tuning(fwd_splits=1):
        assert bsa.bsa_workspace_bytes(big, torch.bfloat16, 145, False) == gathers
    assert bsa.bsa_workspace_bytes(big, torch.float32, 145, False) == 0
    assert bsa.bsa_workspace_bytes(big, torch.bfloat16, 145, True) > gathers
    with pytest.raises(bsa.BsaError):
        bsa.bsa_workspace_bytes(big, torch.bfloat16, 1441, False)


@pytest.mark.parametrize("kw, status", [
    # (a W or H that is not a cube multiple is a valid ragged grid, so it is not listed here:
    # these calls carry placeholder pointers and must fail validation before any launch)
    (dict(T=7), SHAPE), (dict(cond_T=2), SHAPE), (dict(cond_T=8), SHAPE),
    (dict(head_dim=96), UNSUPPORTED), (dict(cube_t=8, cube_h=8, cube_w=8, T=8, H=8, W=8),
                                       UNSUPPORTED),
    (dict(heads=0), INVALID), (dict(cond_T=-4), INVALID),
])
def test_problem_rules(L, kw, status):
    st = L.bsa_block_pool(ctypes.byref(_p(**kw)), 1, FAKE, FAKE, None)
    assert st == status, (kw, st, L.bsa_last_error())


def test_argument_errors(L):
    p = ctypes.byref(_p())
    assert L.bsa_block_pool(None, 1, FAKE, FAKE, None) == INVALID
    assert L.bsa_block_pool(p, 7, FAKE, FAKE, None) == INVALID
    assert L.bsa_block_pool(p, 1, None, FAKE, None) == INVALID
    assert L.bsa_select_topr(p, FAKE, FAKE, -1, FAKE, None, None) == INVALID
    assert L.bsa_select_topr(p, FAKE, None, 2, FAKE, None, None) == INVALID
    fwd = L.bsa_sparse_attn_fwd
    # k_sel inconsistent with any r
    assert fwd(p, 1, FAKE, FAKE, FAKE, None, None, FAKE, 0, ctypes.c_float(0.1), FAKE, FAKE,
               FAKE, 1 << 40, None) == INVALID
    assert fwd(p, 1, FAKE, FAKE, FAKE, None, None, FAKE, 9, ctypes.c_float(0.1), FAKE, FAKE,
               FAKE, 1 << 40, None) == INVALID
    # cache given without condition frames, and missing with them
    assert fwd(p, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, ctypes.c_float(0.1), FAKE, FAKE,
               FAKE, 1 << 40, None) == INVALID
    pc = ctypes.byref(_p(T=8, cond_T=4))
    assert fwd(pc, 1, FAKE, FAKE, FAKE, None, None, FAKE, 5, ctypes.c_float(0.1), FAKE, FAKE,
               FAKE, 1 << 40, None) == INVALID
    # workspace too small for the bf16 MFMA path
    assert fwd(p, 1, FAKE, FAKE, FAKE, None, None, FAKE, 3, ctypes.c_float(0.1), FAKE, FAKE,
               FAKE, 16, None) == WORKSPACE
    assert fwd(p, 1, FAKE, FAKE, FAKE, None, None, FAKE, 3, ctypes.c_float(float("nan")), FAKE,
               FAKE, FAKE, 1 << 40, None) == INVALID
    bwd = L.bsa_sparse_attn_bwd
    sc = ctypes.c_float(0.1)
    # argument order: q, k, v, k_cache, v_cache, o, d_o, lse, idx, k_sel, scale,
    #                 dq, dk, dv, dk_cache, dv_cache, fwd_ws, fwd_ws_bytes, ws,
    #                 ws_bytes, stream
    cache4 = [FAKE, FAKE]
    # condition frames need all four cache tensors; without them none may be given
    assert bwd(pc, 1, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, 5, sc,
               FAKE, FAKE, FAKE, None, None, None, 0, FAKE, 1 << 40, None) == INVALID
    assert bwd(pc, 1, FAKE, FAKE, FAKE, *cache4, FAKE, FAKE, FAKE, FAKE, 5, sc,
               FAKE, FAKE, FAKE, FAKE, None, None, 0, FAKE, 1 << 40, None) == INVALID
    assert bwd(p, 1, FAKE, FAKE, FAKE, *cache4, FAKE, FAKE, FAKE, FAKE, 3, sc,
               FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, 1 << 40, None) == INVALID
    # cache gradients exist on the bf16 MFMA path only
    assert bwd(pc, 0, FAKE, FAKE, FAKE, *cache4, FAKE, FAKE, FAKE, FAKE, 5, sc,
               FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, 1 << 40, None) == UNSUPPORTED
    assert bwd(p, 1, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, 3, sc,
               FAKE, FAKE, FAKE, None, None, None, 0, FAKE, 8, None) == WORKSPACE
    assert bwd(p, 1, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, 3, sc,
               FAKE, FAKE, FAKE, None, None, None, 0, FAKE, 1 << 40, None) == INVALID
    # a forward workspace smaller than the forward's gathered operands is refused
    assert bwd(p, 1, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, 3, sc,
               FAKE, FAKE, FAKE, None, None, FAKE, 64, FAKE, 1 << 40, None) == WORKSPACE
    # the condition-mode workspace covers K/V gathers over every key cube
    big = bsa.Problem(1, 32, 128, 24, 48, 80, 4, 4, 4, cond_T=12)
    plain = bsa.Problem(1, 32, 128, 12, 48, 80, 4, 4, 4)
    import torch
    assert bsa.bsa_workspace_bytes(big, torch.bfloat16, 793, True) > \
        bsa.bsa_workspace_bytes(plain, torch.bfloat16, 73, True)
    assert L.bsa_last_error()  # a message is kept for the last failure


def test_status_strings_and_path_switch(L):
    for code, name in bsa.STATUS.items():
        assert bsa.bsa_status_string(code) == name
    assert L.bsa_set_kernel_path(2) == INVALID
    assert L.bsa_set_kernel_path(1) == OK
    assert L.bsa_set_kernel_path(0) == OK
    assert L.bsa_stage_name(-1) == b""


def test_prologue_argument_errors(L):
    f = L.bsa_qk_prologue
    p = ctypes.byref(_p())
    pc = ctypes.byref(_p(T=8, cond_T=4))
    one = ctypes.c_float(10000.0)
    e = ctypes.c_float(1e-6)
    assert f(p, 1, 0, None, None, one, e, FAKE, FAKE, None) == INVALID        # null x
    assert f(p, 1, 0, FAKE, None, one, e, None, FAKE, None) == INVALID        # null x_out
    assert f(p, 1, 2, FAKE, None, one, e, FAKE, FAKE, None) == INVALID        # bad segment
    assert f(p, 1, 1, FAKE, None, one, e, FAKE, None, None) == INVALID        # no condition frames
    assert f(pc, 1, 1, FAKE, None, one, e, FAKE, FAKE, None) == INVALID       # means of cond
    assert f(p, 1, 0, FAKE, None, ctypes.c_float(1.0), e, FAKE, FAKE, None) == INVALID
    assert f(p, 1, 0, FAKE, None, ctypes.c_float(float("inf")), e, FAKE, FAKE, None) == INVALID
    assert f(p, 1, 0, FAKE, None, one, ctypes.c_float(0.0), FAKE, FAKE, None) == INVALID
    assert f(p, 1, 0, FAKE, None, one, ctypes.c_float(float("nan")), FAKE, FAKE, None) == INVALID
    assert f(p, 7, 0, FAKE, None, one, e, FAKE, FAKE, None) == INVALID        # dtype
    assert f(ctypes.byref(_p(T=7)), 1, 0, FAKE, None, one, e, FAKE, FAKE, None) == SHAPE


def test_size_limits(L):
    """Largest accepted problems (selection row in LDS; CSR transpose for the backward), checked
    without launching: bsa_num_selected validates the problem, the backward fails its key-cube
    check before any launch."""
    at_limit = _p(heads=1, T=4, H=4 * 311, W=4 * 128)          # 311 * 128 = 39808 noise cubes
    over = _p(heads=1, T=4, H=4 * 311, W=4 * 128 + 1)          # ragged: 311 * 129 cubes
    assert L.bsa_num_selected(ctypes.byref(at_limit), 3) == 4
    assert L.bsa_num_selected(ctypes.byref(over), 3) == -1
    assert L.bsa_block_pool(ctypes.byref(over), 1, FAKE, FAKE, None) == UNSUPPORTED
    # 39808 condition + 39808 noise key cubes: the forward is valid, the backward is not
    pc = ctypes.byref(_p(heads=1, T=8, H=4 * 311, W=4 * 128, cond_T=4))
    sc = ctypes.c_float(0.1)
    ks = L.bsa_num_selected(pc, 1)
    assert ks == 39808 + 1 + 1
    assert L.bsa_sparse_attn_bwd(pc, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ks,
                                 sc, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, 1 << 40,
                                 None) == UNSUPPORTED
    assert b"39936" in L.bsa_last_error()


def test_tuning_switches_are_checked_and_per_thread(L):
    import threading
    import torch
    big = bsa.Problem(1, 32, 128, 24, 48, 80, 4, 4, 4)
    assert bsa.bsa_get_tuning(bsa.BSA_TUNE_FWD_SPLITS) == -1
    assert bsa.bsa_get_tuning(bsa.BSA_TUNE_DKDV_ORDER) == 1
    assert bsa.bsa_get_tuning(bsa.BSA_TUNE_DQ_PIPELINE) == 1
    assert bsa.bsa_get_tuning(bsa.BSA_TUNE_WALK_PHASE) == 0     # deterministic walk by default
    assert bsa.bsa_get_tuning(bsa.BSA_TUNE_DKDV_SPLIT) == 0     # split by output by default
    assert L.bsa_get_tuning(7) == -(2 ** 31)
    for key, bad in ((bsa.BSA_TUNE_FWD_SPLITS, 0), (bsa.BSA_TUNE_FWD_SPLITS, 65),
                     (bsa.BSA_TUNE_FWD_SPLITS, -2), (bsa.BSA_TUNE_DKDV_ORDER, 2),
                     (bsa.BSA_TUNE_DQ_PIPELINE, -1), (bsa.BSA_TUNE_WALK_PHASE, -1),
                     (bsa.BSA_TUNE_WALK_PHASE, 1000001), (bsa.BSA_TUNE_DKDV_SPLIT, 2),
                     (bsa.BSA_TUNE_DKDV_SPLIT, -1), (9, 1)):
        assert L.bsa_set_tuning(key, bad) == INVALID
    with bsa.tuning(walk_phase_us=600):
        assert bsa.bsa_get_tuning(bsa.BSA_TUNE_WALK_PHASE) == 600
    assert bsa.bsa_get_tuning(bsa.BSA_TUNE_WALK_PHASE) == 0
    assert bsa.bsa_get_tuning(bsa.BSA_TUNE_FWD_SPLITS) == -1      # a rejected value changes nothing
    auto = bsa.bsa_workspace_bytes(big, torch.bfloat16, 145, False)
    with bsa.tuning(fwd_splits=16):
        assert bsa.bsa_get_tuning(bsa.BSA_TUNE_FWD_SPLITS) == 16
        assert bsa.bsa_workspace_bytes(big, torch.bfloat16, 145, False) > auto
        seen = []
        t = threading.Thread(target=lambda: seen.append(bsa.bsa_get_tuning(bsa.BSA_TUNE_FWD_SPLITS)))
        t.start()
        t.join()
        assert seen == [-1]                                          # other threads keep their own
    assert bsa.bsa_workspace_bytes(big, torch.bfloat16, 145, False) == auto


def test_validate_idx_rejects_bad_arguments_on_host(L):
    p = _p()
    bad = ctypes.c_void_p(0x10000)
    assert L.bsa_validate_idx(ctypes.byref(p), None, 3, bad, None) == INVALID
    assert L.bsa_validate_idx(ctypes.byref(p), FAKE, 3, None, None) == INVALID
    assert L.bsa_validate_idx(ctypes.byref(p), FAKE, 0, bad, None) == INVALID   # k_sel < 1
    assert L.bsa_validate_idx(ctypes.byref(p), FAKE, 9, bad, None) == INVALID   # k_sel > nbk
    assert L.bsa_validate_idx(ctypes.byref(_p(head_dim=96)), FAKE, 1, bad, None) == UNSUPPORTED


def test_probe_arguments_are_checked_on_host(L):
    fake = ctypes.c_void_p(0x10000)
    for shape, chains in ((2, 4), (-1, 4), (0, 3), (1, 16), (0, 0)):
        assert L.bsa_probe_mfma_shape(fake, 8192, shape, chains, 1, 1, fake, 256, None) == INVALID
    assert L.bsa_probe_mfma_shape(None, 8192, 0, 4, 1, 1, fake, 256, None) == INVALID
    assert L.bsa_probe_mfma_shape(fake, 4096, 0, 4, 1, 1, fake, 256, None) == INVALID
    assert L.bsa_probe_mfma_shape(fake, 8192, 0, 4, 2, 1, fake, 256, None) == INVALID  # sink
    for mode, valu, op, acc in ((4, 4, 0, 0), (-1, 4, 0, 0), (0, 3, 0, 0), (0, 32, 0, 0),
                                (0, 8, 1, 0), (0, 0, 1, 0), (0, 4, 2, 0), (0, 4, 0, 2)):
        assert L.bsa_probe_mfma_valu(fake, 2048, mode, valu, op, acc, 1, 1, fake, 2048,
                                     None) == INVALID
    assert L.bsa_probe_mfma_valu(None, 2048, 0, 4, 0, 0, 1, 1, fake, 2048, None) == INVALID
    assert L.bsa_probe_mfma_valu(fake, 1024, 0, 4, 0, 0, 1, 1, fake, 2048, None) == INVALID
    assert L.bsa_probe_mfma_valu(fake, 2048, 0, 4, 0, 0, 2, 1, fake, 2048, None) == INVALID
    assert L.bsa_probe_mfma_valu(fake, 2048, 0, 4, 0, 0, 0, 1, fake, 2048, None) == INVALID
