"""The workload recipe against the figures the LongCat-Video pages print (CPU only).

The pages print no worked example of the attention's values; what they do fix is the size of the
problem: the VAE's 4x16x16 latent compression, 93-frame sequences, 480p and 720p frames and a
selection that keeps about 10% of dense attention.  tests/golden/page_figures.json holds those
figures with their citations; this test derives the workload grids and the selected fraction
from them and checks that the synthetic workloads and the oracle's selection size agree.
"""
import json
import math
import os

import pytest

from oracle import bsa_oracle as orc
from video_dit_block_cube_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


@pytest.fixture(scope="module")
def figs():
    with open(GOLDEN, encoding="utf-8") as f:
        data = json.load(f)
    return {k: v["value"] for k, v in data["figures"].items()}


def latent_grid(figs, lines, width):
    ct, ch, cw = figs["vae_compression_t_h_w"]
    frames = figs["long_sequence_frames"]
    assert (frames - 1) % ct == 0
    return 1 + (frames - 1) // ct, lines // ch, width // cw


def test_latent_grids_follow_the_printed_compression(figs):
    t720, h720, w720 = latent_grid(figs, figs["fine_resolution_lines"], 1280)
    t480, h480, w480 = latent_grid(figs, figs["coarse_resolution_lines"], 832)
    assert (t720, h720, w720) == (24, 45, 80)
    assert (t480, h480, w480) == (24, 30, 52)
    for number, (t, h, w) in ((3, (t720, h720, w720)), (4, (t720, h720, w720)),
                              (2, (t480, h480, w480)), (5, (t480, h480, w480))):
        wl = synth.workload(number)
        # the divisible workloads round the height up to the cube side; time and width match
        assert (wl.T, wl.W) == (t, w)
        assert wl.H == math.ceil(h / wl.cube_h) * wl.cube_h


def test_selected_fraction_is_the_printed_ten_percent(figs):
    keep = figs["kept_attention_fraction"]
    for number in (2, 3, 5):
        wl = synth.workload(number)
        op = orc.Problem(**wl.shape_dict)
        k_sel = orc.num_selected(op, wl.r)
        frac = k_sel / op.nbk
        # r counts on top of the always-kept own cube, so the fraction sits just above 10%
        assert keep <= frac <= keep + 0.002, (wl.name, k_sel, op.nbk, frac)
    # the real 720p latent (45 tokens high) has the same cube count as the divisible grid
    t, h, w = latent_grid(figs, figs["fine_resolution_lines"], 1280)
    wl = synth.workload(3)
    ragged = orc.Problem(batch=1, heads=1, head_dim=128, T=t, H=h, W=w, cube_t=4, cube_h=4,
                         cube_w=4)
    assert ragged.nbq == orc.Problem(**wl.shape_dict).nbq == 1440
