"""The diagnostic probes compute what they claim, on inputs whose results are known exactly:
whole-tile reads give the XOR of the words each lane loads (ids outside the buffer skipped);
back-to-back MFMA on constant 0.5 operands adds 4 to every accumulator element per 32x32x16
product (8 per 16x16x32 product); the MFMA/VALU probe's products and VALU chains land where its
mode says, and in its split mode exactly one wave of every SIMD does the products."""
import numpy as np
import pytest

from tests._util import print_case
from video_dit_block_cube_amd import bsa

pytestmark = pytest.mark.gpu


def test_tile_read_xor():
    import torch
    print_case("probe tile read: 16 waves x 5 ids over 64 tiles of 8 KB")
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(3)
    tile, n_tiles, waves, per_wave = 8192, 64, 16, 5
    buf = torch.randint(0, 256, (n_tiles * tile,), generator=gen, device="cuda:0",
                        dtype=torch.uint8)
    ids = torch.randint(-2, n_tiles + 2, (waves, per_wave), generator=gen, device="cuda:0",
                        dtype=torch.int32)
    sink = torch.empty(waves * 64, dtype=torch.int32, device="cuda:0")
    bsa.bsa_probe_tile_read(buf.view(torch.bfloat16), tile, ids, per_wave, sink)
    torch.cuda.synchronize()
    words = buf.cpu().numpy().view(np.uint32).reshape(n_tiles, tile // 1024, 64, 4)
    lane_xor = np.bitwise_xor.reduce(np.bitwise_xor.reduce(words, axis=3), axis=1)  # [tile, lane]
    want = np.zeros((waves, 64), dtype=np.uint32)
    for w, row in enumerate(ids.cpu().numpy()):
        for t in row:
            if 0 <= t < n_tiles:
                want[w] ^= lane_xor[t]
    assert np.array_equal(sink.cpu().numpy().view(np.uint32).reshape(waves, 64), want)


@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("chains", [1, 2, 4, 8])
def test_mfma_probe_constant_operands(shape, chains):
    import torch
    print_case(f"probe mfma shape={shape} chains={chains}")
    ops = torch.full((4096,), 0.5, dtype=torch.bfloat16, device="cuda:0")
    waves, iters = 8, 10
    sink = torch.empty(waves * 64, dtype=torch.float32, device="cuda:0")
    bsa.bsa_probe_mfma_shape(ops, shape, chains, waves, iters, sink)
    torch.cuda.synchronize()
    # per iteration and lane: 8 products x 16 elements x 4.0 (32x32x16) or 16 x 4 x 8.0 (16x16x32)
    assert np.all(sink.cpu().numpy() == 512.0 * iters)


def _chains_after(lane, valu, op, updates):
    """The probe's eight fp32 chains of one lane after `updates` rounds (chains k < valu only)."""
    x = 0.001 * (lane + np.arange(8, dtype=np.float64))
    for _ in range(updates):
        for k in range(min(valu, 8)):
            x[k] = x[k] * 0.999 + 0.001 if op == 0 else 2.0 ** (-x[k])
    return x.sum()


@pytest.mark.parametrize("valu, op", [(4, 0), (2, 1)])
@pytest.mark.parametrize("acc", [0, 1])
def test_mfma_valu_probe_modes(valu, op, acc):
    import torch
    print_case(f"probe mfma/valu valu={valu} op={op} acc={acc}")
    ops = torch.full((1024,), 0.5, dtype=torch.bfloat16, device="cuda:0")
    wgs, iters = 4, 3
    sink = torch.empty(wgs * 512, dtype=torch.float32, device="cuda:0")
    lane = np.arange(512) % 64
    prod = 4 * 16 * 4.0 * iters      # 4 accumulators x 16 elements x 4.0 per product x iters
    upd = 4 * iters * (valu // min(valu, 8))   # rounds each used chain is updated
    idle = np.array([_chains_after(l, 0, op, 0) for l in range(64)])[lane]
    busy = np.array([_chains_after(l, valu, op, upd) for l in range(64)])[lane]
    got = {}
    for mode in range(4):
        bsa.bsa_probe_mfma_valu(ops, mode, valu, op, acc, wgs, iters, sink)
        torch.cuda.synchronize()
        got[mode] = sink.cpu().numpy().reshape(wgs, 512).astype(np.float64)
    np.testing.assert_allclose(got[0], np.broadcast_to(prod + busy, (wgs, 512)), rtol=1e-5)
    np.testing.assert_allclose(got[2], np.broadcast_to(prod + idle, (wgs, 512)), rtol=1e-5)
    np.testing.assert_allclose(got[3], np.broadcast_to(busy, (wgs, 512)), rtol=1e-5)
    # split: per workgroup, four waves (one per SIMD) did the products, the other four the VALU
    for g in range(wgs):
        waves = got[1][g].reshape(8, 64)
        is_prod = [np.allclose(wv, prod + idle[:64], rtol=1e-5) for wv in waves]
        is_valu = [np.allclose(wv, busy[:64], rtol=1e-5) for wv in waves]
        assert all(p != v for p, v in zip(is_prod, is_valu)), (g, is_prod, is_valu)
        assert sum(is_prod) == 4, (g, is_prod)
