"""Checks of the seeded input recipe (CPU only)."""
import numpy as np

from video_dit_block_cube_amd import synth


def test_tiny_recipe_is_seeded_fp32_normal():
    w = synth.workload(1)
    x = synth.make_inputs(w)
    assert set(x) == {"q", "k", "v"}
    rng = np.random.default_rng(1001)
    q = rng.standard_normal(size=(1, 256, 1, 64), dtype=np.float32)
    np.testing.assert_array_equal(x["q"], q)
    assert x["q"].dtype == np.float32


def test_round_to_bf16_is_rne():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0, -0.0,
                     3.0e38, 1e-40], dtype=np.float32)
    got = synth.round_to_bf16(vals)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties to even -> 1 + 2^-6
    expect = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0, -0.0], dtype=np.float32)
    np.testing.assert_array_equal(got[:7], expect)
    assert np.all(got.view(np.uint32) & 0xFFFF == 0)
    assert np.isfinite(got[7])


def test_small_bf16_workload_shapes_and_qknorm():
    w = synth.workload(2, heads=2, T=8, H=8, W=8)
    x = synth.make_inputs(w)
    assert x["q"].shape == (1, 8 * 8 * 8, 2, 128)
    for name in ("q", "k", "v"):
        assert np.all(x[name].view(np.uint32) & 0xFFFF == 0)
    rms = np.sqrt(np.mean(x["q"].astype(np.float64) ** 2, axis=-1))
    assert np.all(np.abs(rms - 1) < 1e-2)
    cont = synth.make_inputs(synth.workload(4, heads=1, T=8, H=8, W=8, cond_T=4))
    assert set(cont) == {"q", "k", "v", "k_cache", "v_cache"}
    assert cont["k_cache"].shape == (1, 4 * 64, 1, 128)
    bwd = synth.make_inputs(synth.workload(5, heads=1, T=4, H=8, W=8))
    assert "dO" in bwd
