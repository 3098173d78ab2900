#!/usr/bin/env python3
"""Benchmark of the block sparse attention hot path on one MI355X.

One step = the whole path over one batch of the 720p-class workload (B=1, 32 heads, D=128,
latent grid 24x48x80, 4x4x4 cubes, top-r=144 plus the own cube, QKNorm'd q/k, dO ~ N(0,1)):
pool Q, pool K, select, sparse attention forward, backward (Delta + CSR transpose, gathers,
dK/dV, dQ).  Inputs are resident in HBM before the timed region.

value = effective TFLOP/s over the step, counting selected-block FLOPs only:
forward 4*B*Hh*Nq*(k_sel*c)*D, backward 2.5x forward.  Per-kernel durations come from HIP events
recorded by the library at its internal stage boundaries on the launch stream.

Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--no-cpu] [--no-continuation]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BSA fwd+bwd effective TFLOP/s & % bf16 MFMA peak; ms/call at 720p-class grid"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_CLOCK_GHZ = 2.4            # the clock the bf16 peak is quoted at


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def fwd_flops(p, k_sel: int) -> float:
    return 4.0 * p.batch * p.heads * p.Nq * (k_sel * p.c) * p.head_dim


def kernel_flops(name: str, p, k_sel: int) -> float | None:
    """Contraction FLOPs one launch of a kernel executes (2*m*n*k per GEMM over selected pairs).
    The backward recomputes S and dP in both of its passes, so it executes 7 GEMMs per pair
    where the method needs 5."""
    one_gemm = 2.0 * p.batch * p.heads * p.Nq * (k_sel * p.c) * p.head_dim
    return {"attn_fwd_mfma": 2 * one_gemm,      # S = QK^T, O = PV
            "bwd_dkdv_mfma": 4 * one_gemm,      # S, dP, dV, dK
            "bwd_dq_mfma": 3 * one_gemm}.get(name)   # S, dP (both recomputed), dQ


def credited_flops(name: str, p, k_sel: int) -> float | None:
    """The method's FLOPs a kernel is credited with: forward 2 GEMMs; backward 5 GEMMs in all
    (the FlashAttention count: S recomputed, dP, dV, dK, dQ), of which dK/dV performs 4 and dQ
    the 1 the other pass has not (its S and dP are repeats)."""
    one_gemm = 2.0 * p.batch * p.heads * p.Nq * (k_sel * p.c) * p.head_dim
    return {"attn_fwd_mfma": 2 * one_gemm, "bwd_dkdv_mfma": 4 * one_gemm,
            "bwd_dq_mfma": 1 * one_gemm}.get(name)


def compulsory_bytes(name: str, p, k_sel: int) -> float | None:
    """Bytes an MFMA kernel must move at least once at a divisible grid with no condition
    frames: its gathered bf16 operands read once, its outputs written once, its small per-row
    inputs read once."""
    tensor = p.batch * p.Nq * p.heads * p.head_dim * 2
    per_query = p.batch * p.heads * p.Nq * 4
    idx = p.batch * p.heads * p.nbq * k_sel * 4
    return {"attn_fwd_mfma": 3 * tensor + tensor + per_query + idx,     # Q, K, V^T; O; LSE; idx
            "bwd_dkdv_mfma": 4 * tensor + 2 * 2 * tensor + 2 * per_query + idx,  # Q,dO,K,V; dK,dV
            "bwd_dq_mfma": 4 * tensor + 2 * tensor + 2 * per_query + idx}.get(name)


def stage_bytes(name: str, p, k_sel: int) -> float | None:
    """Algorithmic HBM bytes of one call of a bandwidth-bound stage at a divisible grid with no
    condition frames (each tensor read or written once): bf16 token tensors, fp32 means and
    Delta/LSE, gathered cube-major copies of the same size as their source."""
    tensor = p.batch * p.Nq * p.heads * p.head_dim * 2          # one bf16 [B, Nq, Hh, D]
    means = p.batch * p.heads * p.nbq * p.head_dim * 4
    per_query = p.batch * p.heads * p.Nq * 4                    # one fp32 value per query token
    idx = p.batch * p.heads * p.nbq * k_sel * 4                  # int32 selection
    return {"pool": tensor + means,                             # x in, means out
            "gather_qkv": 3 * 2 * tensor,                       # q, k, v in; ROW/TRANS copies out
            "bwd_gather_qkv": 3 * 2 * tensor,                   # q, k, v in; ROW copies out
            "bwd_gather_v": 2 * tensor,                         # v in; ROW copy out
            # O, dO, LSE in; dO ROW copy and (LSE, Delta) pairs out; CSR transpose: idx in,
            # lists out
            "bwd_prep": 3 * tensor + 3 * per_query + 2 * idx}.get(name)


def kernel_build_flags(name: str) -> str:
    """The hipcc options build.py compiles csrc/<name> with, include paths left out."""
    from video_dit_block_cube_amd import build as B
    flags, skip = [], False
    for f in B.FLAGS:
        if skip:
            skip = False
            continue
        if f == "-I":
            skip = True
            continue
        flags.append(f)
    return " ".join(flags + list(B.EXTRA_FLAGS.get(name, [])))


def profile_record(stage: str) -> dict:
    """Counter results of a kernel (profiles/traffic_<stage>.txt: bytes fetched from beyond L2
    plus bytes written, per launch, from FETCH_SIZE and WRITE_SIZE scaled by a plain copy; shader
    clock), or {} when no measurement exists or the kernel source or its build options changed
    since it was taken.
    FETCH_SIZE counts every byte the L2 fetches, Infinity Cache hits included, so these bytes
    bound HBM traffic from above."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}.txt")
    if not os.path.exists(path):
        return {}
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    # "source" lists the kernel's files (comma separated); the hash covers their bytes in order
    srcs = [os.path.join(ROOT, f.strip()) for f in kv.get("source", "").split(",") if f.strip()]
    if not srcs or not all(os.path.exists(f) for f in srcs):
        return {}
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    if h.hexdigest() != kv.get("source_sha256"):
        return {}
    # "build_flags": the compiler options the kernel's file is built with (build.py, include
    # paths left out); a record taken under other options is not this kernel's
    if "build_flags" in kv and kv["build_flags"] != kernel_build_flags(kv.get("build_file", "")):
        return {}
    rec = {}
    for key in ("beyond_l2_bytes_per_launch", "clock_ghz"):
        try:
            rec[key] = float(kv[key])
        except (KeyError, ValueError):
            pass
    return rec


def cpu_baseline(x, op, r):
    """The fp64 oracle, as it is, on the host cores (heads are independent, so one head is an
    exact share of the work):
      - the 256-token tiny workload in full: pool, select, forward, backward;
      - its finite-difference check in full: 32 random directions over (q, k, v) and 256 single
        coordinates, central differences of the forward's loss with the selection held fixed;
      - every query cube of head 0 of the 720p-class step: pool, select, forward and the full
        backward (key gradients included).
    The head's rate is the baseline; 32 heads at that rate are the extrapolated full step."""
    import numpy as np
    import oracle as orc
    from video_dit_block_cube_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    # tiny workload in full: pool, select, forward, backward
    w1 = synth.workload(1)
    x1 = {k: v.astype(np.float64) for k, v in synth.make_inputs(w1).items()}
    p1 = orc.Problem(**w1.shape_dict)
    dO1 = np.random.default_rng(1001).standard_normal(x1["q"].shape)
    sc1 = 1 / math.sqrt(p1.head_dim)
    t0 = time.perf_counter()
    qm1, km1 = orc.block_pool(x1["q"], p1), orc.block_pool(x1["k"], p1)
    idx1, _ = orc.select_topr(qm1, km1, p1, w1.r)
    orc.sparse_attn_fwd(x1["q"], x1["k"], x1["v"], None, None, idx1, p1, sc1)
    g1 = orc.attn_bwd(x1["q"], x1["k"], x1["v"], dO1, idx1, p1, sc1)
    tiny_s = time.perf_counter() - t0

    # its finite-difference check in full
    def loss(q, k, v):
        return float(np.sum(orc.sparse_attn_fwd(q, k, v, None, None, idx1, p1, sc1)[0] * dO1))
    rng = np.random.default_rng(77)
    hstep = 1e-5
    names = ("q", "k", "v")
    worst = 0.0
    t0 = time.perf_counter()
    for _ in range(32):
        dirs = [rng.standard_normal(x1[n].shape) for n in names]
        fd = (loss(*[x1[n] + hstep * d for n, d in zip(names, dirs)]) -
              loss(*[x1[n] - hstep * d for n, d in zip(names, dirs)])) / (2 * hstep)
        an = sum(float(np.sum(g * d)) for g, d in zip(g1, dirs))
        worst = max(worst, abs(fd - an) / max(1.0, abs(an)))
    for t in range(256):
        which = t % 3
        pos = int(rng.integers(0, x1[names[which]].size))
        args = [x1[n].copy() for n in names]
        args[which].ravel()[pos] += hstep
        lp = loss(*args)
        args[which].ravel()[pos] -= 2 * hstep
        fd = (lp - loss(*args)) / (2 * hstep)
        an = float(g1[which].ravel()[pos])
        worst = max(worst, abs(fd - an) / max(1.0, abs(an)))
    fd_s = time.perf_counter() - t0

    # every query cube of head 0 of the 720p-class step
    one = {k: np.ascontiguousarray(v[:, :, 0:1]) for k, v in x.items() if k in ("q", "k", "v", "dO")}
    p_h = orc.Problem(batch=op.batch, heads=1, head_dim=op.head_dim, T=op.T, H=op.H, W=op.W,
                      cube_t=op.cube_t, cube_h=op.cube_h, cube_w=op.cube_w, cond_T=op.cond_T)
    scale = 1.0 / math.sqrt(op.head_dim)
    t0 = time.perf_counter()
    qm, km = orc.block_pool(one["q"], p_h), orc.block_pool(one["k"], p_h)
    idx, _ = orc.select_topr(qm, km, p_h, r)
    orc.sparse_attn_fwd(one["q"], one["k"], one["v"], None, None, idx, p_h, scale)
    orc.attn_bwd(one["q"], one["k"], one["v"], one["dO"], idx, p_h, scale)
    head_s = time.perf_counter() - t0
    ks = idx.shape[-1]
    head_flop = 3.5 * 4.0 * op.batch * op.Nq * (ks * op.c) * op.head_dim   # fwd + 2.5x fwd
    rate = head_flop / head_s
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle on every query cube ({op.batch * op.nbq}) of head 0 of the "
                      f"720p-class step: pool, select, forward, backward with key gradients, in "
                      f"{head_s:.1f} s; the 256-token tiny workload end to end in {tiny_s:.3f} s "
                      f"and its finite-difference check (32 directions + 256 coordinates) in "
                      f"{fd_s:.1f} s; {len(os.sched_getaffinity(0))} host cores visible, {threads} "
                      "BLAS threads",
            "head_s": round(head_s, 2),
            "tiny_workload_s": round(tiny_s, 4),
            "tiny_fd_check_s": round(fd_s, 2),
            "tiny_fd_worst_rel_err": float(f"{worst:.2e}"),
            "extrapolated_720p_step_s": round(head_s * op.heads, 1),
            "extrapolated": "extrapolated_720p_step_s = head_s x the 32 heads (heads are "
                            "independent); value, head_s and the tiny figures are measured"}


def bench_microbench(bsa, torch, dev, reps=3):
    """The limits the attention kernels run against, measured with the library's probe kernels:
    back-to-back bf16 MFMA on N(0,1) against constant operands at one and two waves per SIMD and
    by product shape and accumulator chains; MFMA beside VALU work, within a wave and across the
    two waves of a SIMD; and whole 32 KB tile reads at the working sets the kernels see per XCD
    (a forward key range, half of one, one head's K/V shared by every XCD, the whole 1.5 GB of
    K/V)."""
    import numpy as np
    res = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(31)
    ops = {"normal": torch.randn(4096, generator=gen, device=dev).to(torch.bfloat16),
           "constant": torch.full((4096,), 0.5, device=dev, dtype=torch.bfloat16)}
    n_cu_simd = 1024                          # 256 CUs x 4 SIMDs
    iters = 40000                             # ~10 ms per launch: long enough for the clock
    configs = [(name, wps) for wps in (1, 2) for name in ops]
    sinks = {wps: torch.empty(n_cu_simd * wps * 64, dtype=torch.float32, device=dev)
             for wps in (1, 2)}
    for name, wps in configs:                 # warm up every configuration
        bsa.bsa_probe_mfma(ops[name], n_cu_simd * wps, iters // 10, sinks[wps])
    torch.cuda.synchronize()
    times = {c: [] for c in configs}
    for _ in range(reps):                     # configurations interleaved, so drift hits all alike
        for name, wps in configs:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bsa.bsa_probe_mfma(ops[name], n_cu_simd * wps, iters, sinks[wps])
            e1.record()
            e1.synchronize()
            times[(name, wps)].append(e0.elapsed_time(e1))
    for (name, wps), ms in times.items():
        flops = n_cu_simd * wps * iters * 8 * 32768.0
        res[f"mfma_bf16_{name}_{wps}wave_per_simd_tflops"] = round(
            flops / (float(np.median(ms)) * 1e-3) / 1e12, 1)
    # independent accumulator chains per wave, per product shape, on N(0,1) operands: how much
    # independent MFMA work a wave must keep in flight (the kernels run 2 to 8 chains)
    chain_cfg = [(shape, ch, wps) for wps in (1, 2) for shape in (0, 1) for ch in (1, 2, 4, 8)]
    it_c = iters // 4
    for shape, ch, wps in chain_cfg:
        bsa.bsa_probe_mfma_shape(ops["normal"], shape, ch, n_cu_simd * wps, it_c // 10, sinks[wps])
    torch.cuda.synchronize()
    ctimes = {c: [] for c in chain_cfg}
    for _ in range(reps):
        for shape, ch, wps in chain_cfg:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bsa.bsa_probe_mfma_shape(ops["normal"], shape, ch, n_cu_simd * wps, it_c, sinks[wps])
            e1.record()
            e1.synchronize()
            ctimes[(shape, ch, wps)].append(e0.elapsed_time(e1))
    chains = {}
    for (shape, ch, wps), ms in ctimes.items():
        flops = n_cu_simd * wps * it_c * 262144.0
        key = f"{'32x32x16' if shape == 0 else '16x16x32'}_{wps}wave_per_simd"
        chains.setdefault(key, {})[f"chains_{ch}"] = round(
            flops / (float(np.median(ms)) * 1e-3) / 1e12, 1)
    res["mfma_bf16_normal_by_chains_tflops"] = chains
    # bf16 MFMA beside VALU work on one SIMD: interleaved in every wave (mode 0), split between
    # the two waves of a SIMD (mode 1), against products only (2) and VALU only (3).  "overlap" =
    # the share of the shorter kind's time hidden under the other: 1 = fully beside, 0 = after.
    wgs, it_x = 1024, 8000
    xsink = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    xcfg = [(op, v, acc) for acc in (0, 1) for op, vs in ((0, (4, 8, 16)), (1, (2, 4)))
            for v in vs]
    for op, v, acc in xcfg:
        for mode in range(4):
            bsa.bsa_probe_mfma_valu(ops["normal"], mode, v, op, acc, wgs, it_x // 10, xsink)
    torch.cuda.synchronize()
    xt = {(op, v, acc, m): [] for op, v, acc in xcfg for m in range(4)}
    for _ in range(reps):
        for op, v, acc in xcfg:
            for mode in range(4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                bsa.bsa_probe_mfma_valu(ops["normal"], mode, v, op, acc, wgs, it_x, xsink)
                e1.record()
                e1.synchronize()
                xt[(op, v, acc, mode)].append(e0.elapsed_time(e1))
    coexec = {}
    for op, v, acc in xcfg:
        t = [float(np.median(xt[(op, v, acc, m)])) for m in range(4)]
        both, half = t[2] + t[3], 0.5 * (t[2] + t[3])
        coexec[f"{'fma' if op == 0 else 'exp'}_x{v}_per_mfma_{'agpr' if acc else 'vgpr'}_acc"] = {
            "mfma_only_ms": round(t[2], 3), "valu_only_ms": round(t[3], 3),
            "in_wave_ms": round(t[0], 3), "across_waves_ms": round(t[1], 3),
            "overlap_in_wave": round((both - t[0]) / min(t[2], t[3]), 2),
            "overlap_across_waves": round((half - t[1]) / (0.5 * min(t[2], t[3])), 2)}
    res["mfma_valu_coexec"] = coexec
    tile = 32 * 1024
    buf = torch.empty(1536 * (1 << 20), dtype=torch.uint8, device=dev).view(torch.bfloat16)
    buf.view(torch.uint8).random_(0, 256, generator=gen)
    n_tiles = buf.numel() * 2 // tile
    waves, per_wave = 2048, 64
    sink = torch.empty(waves * 64, dtype=torch.int32, device=dev)
    scenarios = {"per_xcd_2.9MB": (int(2.9 * (1 << 20)) // tile, True),
                 "per_xcd_5.8MB": (int(5.8 * (1 << 20)) // tile, True),
                 "shared_46MB": (46 * (1 << 20) // tile, False),
                 "shared_1.5GB": (n_tiles, False)}
    for name, (span, per_xcd) in scenarios.items():
        r = torch.randint(0, span, (waves, per_wave), generator=gen, device=dev, dtype=torch.int32)
        if per_xcd:   # workgroup w runs on XCD w % 8: give each XCD its own span of tiles
            r += (torch.arange(waves, device=dev, dtype=torch.int32) % 8)[:, None] * span
        ids = r.contiguous()
        bsa.bsa_probe_tile_read(buf, tile, ids, per_wave, sink)
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bsa.bsa_probe_tile_read(buf, tile, ids, per_wave, sink)
            e1.record()
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        res[f"tile_read_{name}_TBps"] = round(waves * per_wave * tile /
                                              (float(np.median(ms)) * 1e-3) / 1e12, 2)
    del buf
    res["note"] = ("MFMA: 8 products x iters per wave on 1024 or 2048 one-wave workgroups; "
                   "MFMA beside VALU: 1024 eight-wave workgroups (one per CU at a time) x 8000 x 4 "
                   "products; tile reads: 2048 waves x 64 random 32 KB tiles, 1 KB wave loads")
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-continuation", action="store_true",
                    help="skip the continuation-mode forward measurement")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the ragged 24x45x80 (real 720p latent) fwd+bwd measurement")
    ap.add_argument("--no-prologue", action="store_true",
                    help="skip the fused QK-norm + 3D RoPE prologue measurement")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense-attention (r = all) forward comparison")
    ap.add_argument("--no-480p", action="store_true",
                    help="skip the 480p-class forward + backward step")
    ap.add_argument("--no-smooth", action="store_true",
                    help="skip the 720p-class step on spatially smooth Q/K")
    ap.add_argument("--no-d64", action="store_true",
                    help="skip the 720p-class forward + backward step at head dim 64")
    ap.add_argument("--no-microbench", action="store_true",
                    help="skip the MFMA-rate and tile-read microbenchmarks")
    ap.add_argument("--only-leg", choices=["480p", "continuation", "ragged", "d64", "smooth",
                                           "walk", "dkdv_split", "microbench"],
                    help="run only this extra measurement (no headline step), e.g. to profile it")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the block sparse "
              "attention path here runs on one GPU. Across GPUs it would shard by heads (one "
              "all-to-all before and one after, Ulysses style); that path is not built.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import oracle as orc
    from video_dit_block_cube_amd import bsa, synth

    dev = torch.device("cuda:0")
    if args.only_leg:
        legs = {"480p": lambda: bench_step(bsa, synth, torch, dev, 5, "480p-class"),
                "d64": lambda: bench_step(bsa, synth, torch, dev, 3, "720p-class", head_dim=64),
                "continuation": lambda: bench_continuation(bsa, synth, orc, torch, dev, args),
                "ragged": lambda: bench_ragged(bsa, synth, torch, dev, args),
                "smooth": lambda: bench_smooth(bsa, synth, torch, dev),
                "walk": lambda: bench_walk(bsa, synth, torch, dev),
                "dkdv_split": lambda: bench_dkdv_split(bsa, synth, torch, dev),
                "microbench": lambda: bench_microbench(bsa, torch, dev)}
        log(f"only the {args.only_leg} measurement")
        print(json.dumps({"leg": args.only_leg, "result": legs[args.only_leg]()}), flush=True)
        return 0
    w = synth.workload(3, with_grad=True)
    log(f"drawing inputs for {w.name} (seed {1000 + w.number})")
    t0 = time.perf_counter()
    x = synth.make_inputs(w)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    p = bsa.Problem(**w.shape_dict)
    op = orc.Problem(**w.shape_dict)
    t = {k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in x.items()}
    ks = bsa.bsa_num_selected(p, w.r)
    scale = 1.0 / math.sqrt(p.head_dim)

    # buffers allocated once; the step writes into them
    qm = torch.empty((p.batch, p.heads, p.nbq, p.head_dim), dtype=torch.float32, device=dev)
    km = torch.empty_like(qm)
    idx = torch.empty((p.batch, p.heads, p.nbq, ks), dtype=torch.int32, device=dev)
    o = torch.empty_like(t["q"])
    lse = torch.empty((p.batch, p.heads, p.Nq), dtype=torch.float32, device=dev)
    dq = torch.empty(t["q"].shape, dtype=torch.float32, device=dev)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    ws_f = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, False), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, True), dtype=torch.uint8,
                       device=dev)

    def step(ev=None):
        calls = [
            lambda: bsa.bsa_block_pool(p, t["q"], qm),
            lambda: bsa.bsa_block_pool(p, t["k"], km),
            lambda: bsa.bsa_select_topr(p, qm, km, w.r, with_mask=False, idx=idx),
            lambda: bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx, ks, scale, o=o,
                                            lse=lse, workspace=ws_f),
            lambda: bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx, ks,
                                            scale, dq=dq, dk=dk, dv=dv, workspace=ws_b,
                                            fwd_workspace=ws_f),
        ]
        for ci, c in enumerate(calls):
            if ev is None:
                c()
            else:
                with ev[ci]:
                    c()

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: HIP events per internal stage of every call, on the launch stream
    events = [[bsa.StageEvents(8) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    start = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - start) * 1e3 / args.steps
    stage_ms: dict[str, list] = {}
    step_ms = []
    for s in range(args.steps):
        tot = 0.0
        for ci in range(5):
            for name, ms in events[s][ci].elapsed_all():
                stage_ms.setdefault(name, []).append(ms)
                tot += ms
        step_ms.append(tot)
    ms_per_step = wall_ms
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step wall, "
        f"{np.mean(step_ms):.3f} ms/step summed over kernels")

    f_fwd = fwd_flops(p, ks)
    eff = f_fwd * 3.5
    value = eff / (ms_per_step * 1e-3) / 1e12
    avg = {k: float(np.mean(v)) for k, v in stage_ms.items()}
    # pool runs twice per step; per-launch average is what the roofline wants
    dominant = max((k for k in avg if kernel_flops(k, p, ks)), key=lambda k: avg[k])
    dom_flops = kernel_flops(dominant, p, ks)
    achieved = dom_flops / (avg[dominant] * 1e-3) / 1e12
    rec = profile_record(dominant)
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": rec.get("beyond_l2_bytes_per_launch"),
                "traffic_kind": "bytes fetched from beyond L2 (Infinity Cache hits included) + "
                                "bytes written, per launch (FETCH_SIZE, WRITE_SIZE)",
                "compulsory_bytes": compulsory_bytes(dominant, p, ks),
                "flops_per_launch": dom_flops, "avg_launch_ms": round(avg[dominant], 4)}
    if "clock_ghz" in rec:
        # the same MFMA peak at the clock the kernel actually ran at (power-limited)
        pk = PEAK_BF16_TFLOPS * rec["clock_ghz"] / PEAK_CLOCK_GHZ
        roofline.update(clock_ghz=rec["clock_ghz"], peak_at_clock=round(pk, 1),
                        frac_at_clock=round(achieved / pk, 4))
    per_kernel = {}
    for k, v in avg.items():
        kf = kernel_flops(k, p, ks)
        kc = credited_flops(k, p, ks)
        kb = stage_bytes(k, p, ks)
        per_kernel[k] = {"avg_ms": round(v, 4),
                         "median_ms": round(float(np.median(stage_ms[k])), 4),
                         "p90_ms": round(float(np.percentile(stage_ms[k], 90)), 4),
                         **({"executed_tflop": round(kf / 1e12, 3),
                             "credited_tflop": round(kc / 1e12, 3),
                             "tflops_executed": round(kf / (v * 1e-3) / 1e12, 1),
                             "tflops_credited": round(kc / (v * 1e-3) / 1e12, 1),
                             "frac_peak_executed": round(kf / (v * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                                         4)}
                            if kf else {}),
                         **({"algorithmic_GB": round(kb / 1e9, 3),
                             "achieved_GBps": round(kb / (v * 1e-3) / 1e9, 1),
                             "frac_hbm_peak": round(kb / (v * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                            if kb else {})}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "720p-class BSA fwd+bwd: B=1, Hh=32, D=128, grid 24x48x80, "
                               "cube 4x4x4, top-r=144 + own cube, QKNorm q/k, dO~N(0,1)",
                   "k_sel": ks, "selected_fraction": round(ks / p.nbq, 4),
                   "fwd_tflop": round(f_fwd / 1e12, 3),
                   "bwd_tflop_effective": round(2.5 * f_fwd / 1e12, 3),
                   "bwd_tflop_4gemm": round(2.0 * f_fwd / 1e12, 3)},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "value_4gemm_bwd": round(f_fwd * 3.0 / (ms_per_step * 1e-3) / 1e12, 2),
        "step_ms_median": round(float(np.median(step_ms)), 3),
        "step_ms_p90": round(float(np.percentile(step_ms, 90)), 3),
        "fwd_ms": round(avg.get("gather_qkv", 0) + avg.get("attn_fwd_mfma", 0), 3),
        "bwd_ms": round(sum(avg.get(k, 0) for k in ("bwd_prep", "bwd_gather_qkv",
                                                      "bwd_gather_v", "bwd_dkdv_mfma",
                                                      "bwd_dq_mfma")), 3),
        "kernels": per_kernel,
        "roofline": roofline,
    }

    if not args.no_480p:
        out["step_480p"] = bench_step(bsa, synth, torch, dev, 5, "480p-class")
    if not args.no_smooth:
        log("720p-class step on spatially smooth Q/K")
        out["smooth_qk_720p"] = bench_smooth(bsa, synth, torch, dev)
    if not args.no_d64:
        log("720p-class step at head dim 64")
        out["step_720p_d64"] = bench_step(bsa, synth, torch, dev, 3, "720p-class", head_dim=64)
    if not args.no_continuation:
        out["continuation_fwd"] = bench_continuation(bsa, synth, orc, torch, dev, args)
    if not args.no_dense:
        out["dense_vs_bsa"] = bench_dense(bsa, synth, torch, dev, t)
    if not args.no_prologue:
        out["qk_prologue"] = bench_prologue(bsa, torch, dev, p)
    if not args.no_ragged:
        out["real_latent_720p"] = bench_ragged(bsa, synth, torch, dev, args)

    if not args.no_microbench:
        log("microbenchmarks: MFMA rate, random tile reads")
        out["microbench"] = bench_microbench(bsa, torch, dev)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).normal_()
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written")

    if not args.no_cpu:
        log("CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(x, op, w.r)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def bench_continuation(bsa, synth, orc, torch, dev, args):
    """Forward of the continuation workload (12 condition frames from the cache, top-r=72)."""
    import numpy as np
    w = synth.workload(4)
    log(f"drawing inputs for {w.name}")
    x = synth.make_inputs(w)
    p = bsa.Problem(**w.shape_dict)
    t = {k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in x.items()}
    del x
    ks = bsa.bsa_num_selected(p, w.r)
    scale = 1.0 / math.sqrt(p.head_dim)
    qm = bsa.bsa_block_pool(p, t["q"])
    km = bsa.bsa_block_pool(p, t["k"])
    idx, _ = bsa.bsa_select_topr(p, qm, km, w.r, with_mask=False)
    ws = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, False), dtype=torch.uint8,
                     device=dev)
    o = torch.empty_like(t["q"])
    lse = torch.empty((p.batch, p.heads, p.Nq), dtype=torch.float32, device=dev)
    for _ in range(2):
        bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx, ks, scale, t["k_cache"],
                                t["v_cache"], o=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    evs = [bsa.StageEvents(4) for _ in range(max(3, args.steps // 2))]
    for ev in evs:
        with ev:
            bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx, ks, scale, t["k_cache"],
                                    t["v_cache"], o=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    st: dict[str, list] = {}
    for ev in evs:
        for name, ms in ev.elapsed_all():
            st.setdefault(name, []).append(ms)
    avg = {k: float(np.mean(v)) for k, v in st.items()}
    f = 4.0 * p.batch * p.heads * p.Nq * (ks * p.c) * p.head_dim
    attn = avg.get("attn_fwd_mfma", float("nan"))
    # backward with the condition-cache gradients (continuation training)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4245)
    d_o = torch.randn(t["q"].shape, generator=gen, device=dev,
                      dtype=torch.float32).to(torch.bfloat16)
    wsb = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, True), dtype=torch.uint8,
                      device=dev)
    grads = bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, d_o, lse, idx, ks, scale,
                                    workspace=wsb, k_cache=t["k_cache"], v_cache=t["v_cache"],
                                    fwd_workspace=ws)
    torch.cuda.synchronize()
    evb = [bsa.StageEvents(8) for _ in range(3)]
    for ev in evb:
        with ev:
            bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, d_o, lse, idx, ks, scale,
                                    dq=grads[0], dk=grads[1], dv=grads[2], workspace=wsb,
                                    k_cache=t["k_cache"], v_cache=t["v_cache"],
                                    dk_cache=grads[3], dv_cache=grads[4], fwd_workspace=ws)
    torch.cuda.synchronize()
    sb: dict[str, list] = {}
    for ev in evb:
        for name, ms in ev.elapsed_all():
            sb.setdefault(name, []).append(ms)
    bavg = {k: round(float(np.mean(v)), 3) for k, v in sb.items()}
    bwd_ms = sum(bavg.values())
    return {"workload": "720p-class continuation: 12 condition frames cached, top-r=72 noise "
                        "cubes + own cube + 720 condition cubes",
            "k_sel": ks, "tflop": round(f / 1e12, 3), "gather_ms": round(avg.get("gather_qkv", 0), 3),
            "attn_ms": round(attn, 3), "attn_tflops": round(f / (attn * 1e-3) / 1e12, 1),
            "frac_peak": round(f / (attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "bwd_with_cache_grads": {
                "ms": round(bwd_ms, 3), "stages_ms": bavg,
                "tflop_effective": round(2.5 * f / 1e12, 3),
                "tflops_effective": round(2.5 * f / (bwd_ms * 1e-3) / 1e12, 1)}}


def _time_fwd(bsa, torch, p, t, r, reps=3):
    """Pool, select (r), then the forward alone and (when t holds dO) the backward reusing the
    forward's gathers, each timed per stage with HIP events.  Returns (k_sel, forward ms,
    backward ms or None)."""
    import numpy as np
    ks = bsa.bsa_num_selected(p, r)
    scale = 1.0 / math.sqrt(p.head_dim)
    qm = bsa.bsa_block_pool(p, t["q"])
    km = bsa.bsa_block_pool(p, t["k"])
    idx, _ = bsa.bsa_select_topr(p, qm, km, r, with_mask=False)
    ws = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, False), dtype=torch.uint8,
                     device=t["q"].device)
    o = torch.empty_like(t["q"])
    lse = torch.empty((p.batch, p.heads, p.Nq), dtype=torch.float32, device=t["q"].device)
    bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx, ks, scale, o=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    evs = [bsa.StageEvents(4) for _ in range(reps)]
    for ev in evs:
        with ev:
            bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx, ks, scale, o=o, lse=lse,
                                    workspace=ws)
    torch.cuda.synchronize()
    fwd = float(np.median([sum(ms for _, ms in ev.elapsed_all()) for ev in evs]))
    bwd = None
    if "dO" in t:
        wsb = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, True), dtype=torch.uint8,
                          device=t["q"].device)
        dq = torch.empty(t["q"].shape, dtype=torch.float32, device=t["q"].device)
        dk, dv = torch.empty_like(dq), torch.empty_like(dq)
        evs = [bsa.StageEvents(8) for _ in range(reps + 1)]
        for ev in evs:
            with ev:
                bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx, ks,
                                        scale, dq=dq, dk=dk, dv=dv, workspace=wsb,
                                        fwd_workspace=ws)
        torch.cuda.synchronize()
        bwd = float(np.median([sum(ms for _, ms in ev.elapsed_all()) for ev in evs[1:]]))
        del wsb, dq, dk, dv
    del ws, idx
    return ks, fwd, bwd


def bench_step(bsa, synth, torch, dev, number, label, reps=5, **over):
    """The headline step (pool x2, select, forward, backward) on another seeded workload (QKNorm
    q/k, dO ~ N(0,1)): per-call ms from HIP events on the launch stream."""
    import numpy as np
    w = synth.workload(number, with_grad=True, **over)
    log(f"drawing inputs for {w.name}")
    x = synth.make_inputs(w)
    t = {k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in x.items()}
    del x
    p = bsa.Problem(**w.shape_dict)
    ks = bsa.bsa_num_selected(p, w.r)
    scale = 1.0 / math.sqrt(p.head_dim)
    ws_f = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, False), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, True), dtype=torch.uint8,
                       device=dev)
    qm = torch.empty((p.batch, p.heads, p.nbq, p.head_dim), dtype=torch.float32, device=dev)
    km = torch.empty_like(qm)
    idx = torch.empty((p.batch, p.heads, p.nbq, ks), dtype=torch.int32, device=dev)
    o = torch.empty_like(t["q"])
    lse = torch.empty((p.batch, p.heads, p.Nq), dtype=torch.float32, device=dev)
    dq = torch.empty(t["q"].shape, dtype=torch.float32, device=dev)
    dk, dv = torch.empty_like(dq), torch.empty_like(dq)

    def step(ev):
        calls = [lambda: bsa.bsa_block_pool(p, t["q"], qm),
                 lambda: bsa.bsa_block_pool(p, t["k"], km),
                 lambda: bsa.bsa_select_topr(p, qm, km, w.r, with_mask=False, idx=idx),
                 lambda: bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx, ks, scale, o=o,
                                                 lse=lse, workspace=ws_f),
                 lambda: bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx,
                                                 ks, scale, dq=dq, dk=dk, dv=dv, workspace=ws_b,
                                                 fwd_workspace=ws_f)]
        for e, c in zip(ev, calls):
            with e:
                c()

    step([bsa.StageEvents(8) for _ in range(5)])
    torch.cuda.synchronize()
    evs = [[bsa.StageEvents(8) for _ in range(5)] for _ in range(reps)]
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    stage: dict[str, list] = {}
    for ev in evs:
        per = {}
        for e in ev:
            for name, ms in e.elapsed_all():
                per[name] = per.get(name, 0.0) + ms
        for name, ms in per.items():
            stage.setdefault(name, []).append(ms)
    med = {k: float(np.median(v)) for k, v in stage.items()}
    fwd_ms = med.get("gather_qkv", 0.0) + med.get("attn_fwd_mfma", 0.0)
    bwd_ms = sum(med.get(k, 0.0) for k in ("bwd_prep", "bwd_gather_qkv", "bwd_gather_v",
                                            "bwd_dkdv_mfma", "bwd_dq_mfma"))
    step_ms = sum(med.values())
    f = fwd_flops(p, ks)
    return {"workload": f"{label} BSA fwd+bwd: B={w.batch}, Hh={w.heads}, D={w.head_dim}, grid "
                        f"{w.T}x{w.H}x{w.W}, cube {w.cube_t}x{w.cube_h}x{w.cube_w}, top-r={w.r} "
                        "+ own cube, QKNorm q/k, dO~N(0,1)",
            "k_sel": ks, "fwd_tflop": round(f / 1e12, 3),
            "step_ms": round(step_ms, 3), "fwd_ms": round(fwd_ms, 3), "bwd_ms": round(bwd_ms, 3),
            "value_tflops": round(3.5 * f / (step_ms * 1e-3) / 1e12, 1),
            "fwd_tflops": round(f / (fwd_ms * 1e-3) / 1e12, 1),
            "bwd_tflops_effective": round(2.5 * f / (bwd_ms * 1e-3) / 1e12, 1),
            "stages_ms_per_step": {k: round(v, 4) for k, v in med.items()}}


def bench_ragged(bsa, synth, torch, dev, args, reps=3):
    """One fwd+bwd step on the real 720p latent grid 24 x 45 x 80 (the last cube row is 1 token
    high: partial edge cubes), same heads, cube and top-r as the headline workload."""
    import numpy as np
    w = synth.workload(3, H=45, W=80)
    p = bsa.Problem(**w.shape_dict)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4545)
    shp = (p.batch, p.Nq, p.heads, p.head_dim)
    t = {n: torch.randn(shp, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
         for n in ("q", "k", "v", "dO")}
    ks = bsa.bsa_num_selected(p, w.r)
    scale = 1.0 / math.sqrt(p.head_dim)
    wsf = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, False), dtype=torch.uint8,
                      device=dev)
    wsb = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, True), dtype=torch.uint8,
                      device=dev)

    qm = torch.empty((p.batch, p.heads, p.nbq, p.head_dim), dtype=torch.float32, device=dev)
    km = torch.empty_like(qm)
    idx = torch.empty((p.batch, p.heads, p.nbq, ks), dtype=torch.int32, device=dev)
    o = torch.empty_like(t["q"])
    lse = torch.empty((p.batch, p.heads, p.Nq), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty(shp, dtype=torch.float32, device=dev) for _ in range(3))

    def step(ev=None):
        calls = [
            lambda: bsa.bsa_block_pool(p, t["q"], qm),
            lambda: bsa.bsa_block_pool(p, t["k"], km),
            lambda: bsa.bsa_select_topr(p, qm, km, w.r, with_mask=False, idx=idx),
            lambda: bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx, ks, scale, o=o,
                                            lse=lse, workspace=wsf),
            lambda: bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx, ks,
                                            scale, dq=dq, dk=dk, dv=dv, workspace=wsb,
                                            fwd_workspace=wsf),
        ]
        for ci, c in enumerate(calls):
            if ev is None:
                c()
            else:
                with ev[ci]:
                    c()

    step()
    torch.cuda.synchronize()
    ms = []
    stage_ms: dict = {}
    for _ in range(reps):
        ev = [bsa.StageEvents(8) for _ in range(5)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step(ev)
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
        for ci in range(5):
            for name, v in ev[ci].elapsed_all():
                stage_ms.setdefault(name, []).append(v)
    return {"grid": "24x45x80 (45 = 11 full cube rows + 1 row of height 1)", "k_sel": ks,
            "step_ms": round(float(np.median(ms)), 3),
            # per step (pool runs twice)
            "stages_ms_per_step": {k: round(float(np.sum(v)) / reps, 4) for k, v in stage_ms.items()},
            "note": "pool x2, select, fwd, bwd; partial edge cubes masked in the kernels"}


def bench_bwd_settings(bsa, synth, torch, dev, settings, reps=3):
    """The 720p-class backward under each (label, tuning) setting in turn, on the headline step's
    seeded inputs: per setting one untimed call, then reps timed calls (so a counter run over
    the leg sees the dispatches in that order)."""
    import numpy as np
    w = synth.workload(3, with_grad=True)
    log(f"drawing inputs for {w.name}")
    x = synth.make_inputs(w)
    t = {k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in x.items()}
    del x
    p = bsa.Problem(**w.shape_dict)
    ks = bsa.bsa_num_selected(p, w.r)
    scale = 1.0 / math.sqrt(p.head_dim)
    ws_f = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, False), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, True), dtype=torch.uint8,
                       device=dev)
    qm = bsa.bsa_block_pool(p, t["q"])
    km = bsa.bsa_block_pool(p, t["k"])
    idx, _ = bsa.bsa_select_topr(p, qm, km, w.r, with_mask=False)
    o, lse = bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx, ks, scale, workspace=ws_f)
    dq = torch.empty(t["q"].shape, dtype=torch.float32, device=dev)
    dk, dv = torch.empty_like(dq), torch.empty_like(dq)
    out = {}
    for label, tune in settings:
        with bsa.tuning(**tune):
            evs = [bsa.StageEvents(8) for _ in range(reps + 1)]
            for ev in evs:
                with ev:
                    bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx, ks,
                                            scale, dq=dq, dk=dk, dv=dv, workspace=ws_b,
                                            fwd_workspace=ws_f)
            torch.cuda.synchronize()
        stage: dict = {}
        for ev in evs[1:]:
            for name, ms in ev.elapsed_all():
                stage.setdefault(name, []).append(ms)
        out[label] = {k: round(float(np.median(v)), 4) for k, v in stage.items()}
    return out


def bench_walk(bsa, synth, torch, dev, period_us=600):
    """The 720p-class backward with the real-time walk phase off, then on (each D = 128 dK/dV and
    dQ item starts its list at the clock's phase within period_us, so the items running together
    read neighbouring cubes): how much the backward kernels gain from the extra L2 hits."""
    return {"workload": "720p-class backward (B=1, Hh=32, D=128, grid 24x48x80, top-r=144), "
                        f"walk phase off, then on with a {period_us} us period",
            "stages_ms": bench_bwd_settings(bsa, synth, torch, dev,
                                            [("off", {}), ("on", {"walk_phase_us": period_us})])}


def bench_dkdv_split(bsa, synth, torch, dev):
    """The 720p-class backward with the dK/dV work of each key cube split between its two waves
    by output (default; dK's dS from the bf16 P) and by keys (dS from the fp32 P)."""
    return {"workload": "720p-class backward (B=1, Hh=32, D=128, grid 24x48x80, top-r=144), "
                        "dK/dV split by output, then by keys",
            "stages_ms": bench_bwd_settings(bsa, synth, torch, dev,
                                            [("by_output", {}), ("by_keys", {"dkdv_split": 1})])}


def bench_smooth(bsa, synth, torch, dev, reps=3):
    """The headline step on spatially smooth Q/K (not one of the configs): real video tokens are
    similar to their neighbours, so neighbouring query cubes select overlapping key cubes, where
    the N(0,1) configs select uniformly at random (no K/V reuse between neighbours).  Q and K
    are trilinear upsamplings of noise drawn on a (T/2, H/8, W/8) grid, plus 0.3x white noise,
    RMS-normalised per head; V and dO stay N(0,1)."""
    import numpy as np
    import torch.nn.functional as F
    w = synth.workload(3, with_grad=True)
    p = bsa.Problem(**w.shape_dict)
    gen = torch.Generator(device=dev)
    gen.manual_seed(8080)
    C = p.heads * p.head_dim

    def smooth():
        lo = torch.randn((1, C, p.T // 2, p.H // 8, p.W // 8), generator=gen, device=dev)
        x = F.interpolate(lo, size=(p.T, p.H, p.W), mode="trilinear", align_corners=False)
        x = x.permute(0, 2, 3, 4, 1).reshape(1, p.Nq, p.heads, p.head_dim)
        x = x + 0.3 * torch.randn(x.shape, generator=gen, device=dev)
        x = x / torch.sqrt(x.square().mean(dim=-1, keepdim=True) + 1e-6)
        return x.to(torch.bfloat16).contiguous()

    t = {"q": smooth(), "k": smooth()}
    for n in ("v", "dO"):
        t[n] = torch.randn((1, p.Nq, p.heads, p.head_dim), generator=gen, device=dev).to(
            torch.bfloat16)
    ks = bsa.bsa_num_selected(p, w.r)
    scale = 1.0 / math.sqrt(p.head_dim)
    wsf = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, False), dtype=torch.uint8,
                      device=dev)
    wsb = torch.empty(bsa.bsa_workspace_bytes(p, torch.bfloat16, ks, True), dtype=torch.uint8,
                      device=dev)
    qm = torch.empty((p.batch, p.heads, p.nbq, p.head_dim), dtype=torch.float32, device=dev)
    km = torch.empty_like(qm)
    idx = torch.empty((p.batch, p.heads, p.nbq, ks), dtype=torch.int32, device=dev)
    o = torch.empty_like(t["q"])
    lse = torch.empty((p.batch, p.heads, p.Nq), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty(t["q"].shape, dtype=torch.float32, device=dev) for _ in range(3))

    def step(ev):
        calls = [lambda: bsa.bsa_block_pool(p, t["q"], qm),
                 lambda: bsa.bsa_block_pool(p, t["k"], km),
                 lambda: bsa.bsa_select_topr(p, qm, km, w.r, with_mask=False, idx=idx),
                 lambda: bsa.bsa_sparse_attn_fwd(p, t["q"], t["k"], t["v"], idx, ks, scale, o=o,
                                                 lse=lse, workspace=wsf),
                 lambda: bsa.bsa_sparse_attn_bwd(p, t["q"], t["k"], t["v"], o, t["dO"], lse, idx,
                                                 ks, scale, dq=dq, dk=dk, dv=dv, workspace=wsb,
                                                 fwd_workspace=wsf)]
        for e, c in zip(ev, calls):
            with e:
                c()

    step([bsa.StageEvents(8) for _ in range(5)])
    torch.cuda.synchronize()
    evs = [[bsa.StageEvents(8) for _ in range(5)] for _ in range(reps)]
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    stage: dict = {}
    for ev in evs:
        per = {}
        for e in ev:
            for name, ms in e.elapsed_all():
                per[name] = per.get(name, 0.0) + ms
        for name, ms in per.items():
            stage.setdefault(name, []).append(ms)
    med = {k: float(np.median(v)) for k, v in stage.items()}
    step_ms = sum(med.values())
    # locality of the selection: share of a query cube's selected key cubes that its raster
    # neighbour (next cube along w) also selected, averaged over heads 0 and 31
    sel = idx.cpu().numpy()
    share = []
    for h in (0, p.heads - 1):
        a, b = sel[0, h, :-1], sel[0, h, 1:]
        share.append(np.mean([len(np.intersect1d(x, y)) / ks for x, y in zip(a, b)]))
    f = fwd_flops(p, ks)
    return {"workload": "720p-class grid and selection size on smooth Q/K (correlated over "
                        "about 2x2 cubes in h and w), V and dO ~ N(0,1)",
            "neighbour_selection_overlap": round(float(np.mean(share)), 3),
            "step_ms": round(step_ms, 3),
            "value_tflops": round(3.5 * f / (step_ms * 1e-3) / 1e12, 1),
            "stages_ms_per_step": {k: round(v, 4) for k, v in med.items()}}


def bench_prologue(bsa, torch, dev, p, reps=5):
    """QK RMS normalisation + 3D RoPE of one raw [B, Nq, Hh, D] bf16 tensor at the 720p-class
    grid, fused with the cube means, against the same prologue followed by a separate pool."""
    import numpy as np
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    x = torch.randn((p.batch, p.Nq, p.heads, p.head_dim), generator=gen, device=dev,
                    dtype=torch.float32).to(torch.bfloat16)
    y = torch.empty_like(x)
    m = torch.empty((p.batch, p.heads, p.nbq, p.head_dim), dtype=torch.float32, device=dev)

    def timed(fn):
        # both variants launch on torch's current stream, so stream events bracket them whole
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            out.append(e0.elapsed_time(e1))
        return float(np.median(out))

    fused = timed(lambda: bsa.bsa_qk_prologue(p, x, out=y, mean=m))
    split = timed(lambda: (bsa.bsa_qk_prologue(p, x, out=y, with_mean=False),
                           bsa.bsa_block_pool(p, y, m)))
    nbytes = 2 * x.numel() * 2 + m.numel() * 4
    return {"workload": f"raw bf16 [1, {p.Nq}, {p.heads}, {p.head_dim}] -> normalised, rotated "
                        "tensor + fp32 cube means",
            "fused_ms": round(fused, 4), "prologue_then_pool_ms": round(split, 4),
            "algorithmic_bytes": nbytes,
            "achieved_GBps": round(nbytes / (fused * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (fused * 1e-3) / 1e9 / 8000.0, 4)}


def bench_dense(bsa, synth, torch, dev, t720):
    """Dense 3D attention (r = all key cubes, the same kernels) against BSA at the 480p- and
    720p-class grids: forward ms (gathers + attention), backward ms (reusing the forward's
    gathers), and the BSA speedups of the forward and of the training pair (forward + backward).
    Pool and select are not counted on either side."""
    res = {}
    for number in (2, 3):
        w = synth.workload(number, with_grad=True)
        if number == 3:
            t = t720
        else:
            log(f"drawing inputs for {w.name}")
            x = synth.make_inputs(w)
            t = {k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in x.items()
                 if k in ("q", "k", "v", "dO")}
            del x
        p = bsa.Problem(**w.shape_dict)
        ks_b, ms_b, bwd_b = _time_fwd(bsa, torch, p, t, w.r)
        ks_d, ms_d, bwd_d = _time_fwd(bsa, torch, p, t, p.nbq - 1)
        dense_f = 4.0 * p.batch * p.heads * p.Nq * p.Nq * p.head_dim
        tag = "480p" if number == 2 else "720p"
        res[tag] = {"grid": f"{p.T}x{p.H}x{p.W}", "bsa_k_sel": ks_b, "bsa_fwd_ms": round(ms_b, 3),
                    "dense_fwd_ms": round(ms_d, 3), "dense_tflop": round(dense_f / 1e12, 2),
                    "dense_tflops": round(dense_f / (ms_d * 1e-3) / 1e12, 1),
                    "dense_frac_peak": round(dense_f / (ms_d * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "bsa_speedup": round(ms_d / ms_b, 2)}
        if bwd_b is not None and bwd_d is not None:
            res[tag].update({"bsa_bwd_ms": round(bwd_b, 3), "dense_bwd_ms": round(bwd_d, 3),
                             "dense_bwd_tflops_credited": round(
                                 2.5 * dense_f / (bwd_d * 1e-3) / 1e12, 1),
                             "bsa_bwd_speedup": round(bwd_d / bwd_b, 2),
                             "bsa_fwd_bwd_speedup": round((ms_d + bwd_d) / (ms_b + bwd_b), 2)})
        log(f"dense vs BSA at {tag}: fwd {ms_d:.2f} vs {ms_b:.2f} ms, bwd "
            f"{bwd_d if bwd_d is not None else float('nan'):.2f} vs "
            f"{bwd_b if bwd_b is not None else float('nan'):.2f} ms")
    return res


if __name__ == "__main__":
    sys.exit(main())
