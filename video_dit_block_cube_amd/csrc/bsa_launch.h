// bsa_launch.h -- host-side launchers of the BSA kernels (one translation unit per kernel family).
// Every launcher enqueues asynchronously on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bsa_common.h"

namespace bsa {

// k_pool.hip: per-cube mean of a [B, Nq, Hh, D] tensor -> [B, Hh, nbq, D] fp32.
hipError_t launch_pool(const Geom& g, bool bf16, const void* x, float* out, hipStream_t s);

// k_prologue.hip: RMS normalisation + 3D RoPE of one segment (seg = its own geometry, frames
// starting at grid time t_offset) and, when y_mean is non-null, the cube means of the result.
hipError_t launch_prologue(const Geom& seg, int t_offset, bool bf16, const void* x,
                           const float* gamma, float rope_theta, float eps, void* y,
                           float* y_mean, hipStream_t s);

// k_select.hip: block scores + forced set + top-r -> idx (ascending rows) and optional mask.
hipError_t launch_select(const Geom& g, const float* qm, const float* km, int r_eff, int k_sel,
                         int32_t* idx, uint8_t* mask, hipStream_t s);

// k_attn_simt.hip: portable fp32-arithmetic attention kernels (any cube size, fp32 or bf16 I/O).
hipError_t launch_fwd_simt(const Geom& g, bool bf16, const void* q, const void* k, const void* v,
                           const void* kc, const void* vc, const int32_t* idx, int k_sel,
                           float scale, void* o, float* lse, hipStream_t s);
hipError_t launch_bwd_dq_simt(const Geom& g, bool bf16, const void* q, const void* k,
                              const void* v, const void* d_o, const float* lse_c,
                              const float* delta_c, const int32_t* idx, int k_sel, float scale,
                              float* dq, hipStream_t s);
hipError_t launch_bwd_dkdv_simt(const Geom& g, bool bf16, const void* q, const void* k,
                                const void* v, const void* d_o, const float* lse_c,
                                const float* delta_c, const int32_t* csr_off,
                                const int32_t* csr_list, float scale, float* dk, float* dv,
                                hipStream_t s);

// k_bwd_prep.hip: Delta and LSE in cube order ([B, Hh, nbq, c]) and the CSR transpose of idx;
// ld_c (may be NULL) additionally receives the interleaved (LSE * log2(e), Delta) pairs.
hipError_t launch_delta(const Geom& g, bool bf16, const void* o, const void* d_o,
                        const float* lse, float* delta_c, float* lse_c, float2* ld_c,
                        hipStream_t s);
// Delta fused with the dO gather (bf16, c == 64): ld_c pairs as above and dO in the ROW layout
// over the nbq query cubes ([B, Hh, nbq, 64*D]).
hipError_t launch_delta_gather(const Geom& g, const void* o, const void* d_o, const float* lse,
                               float2* ld_c, bf16_t* do_row, hipStream_t s);
size_t csr_bits_words(const Geom& g);
hipError_t launch_csr(const Geom& g, const int32_t* idx, int k_sel, uint32_t* bits,
                      int32_t* csr_off, int32_t* csr_list, hipStream_t s);

// k_validate.hip: counts the rows of idx ([B, Hh, nbq, k_sel]) with an entry outside [0, nbk) or
// not strictly above the entry before it; *bad_rows (device) is overwritten with the count.
hipError_t launch_validate_idx(const Geom& g, const int32_t* idx, int k_sel, int32_t* bad_rows,
                               hipStream_t s);

// k_probe.hip (diagnostics): back-to-back bf16 MFMA on `waves` one-wave workgroups (operands:
// 8 x 1 KB of bf16 at `operands`; sink: 64 floats per wave), and whole-tile reads of the tiles
// listed in ids ([waves, tiles_per_wave] tile numbers of buf; sink: 64 words per wave).
hipError_t launch_mfma_probe(const bf16_t* operands, int shape, int chains, int waves, int iters,
                             float* sink, hipStream_t s);
// mode 0-3, valu in {0, 2, 4, 8, 16} with op 0 (fma) or {1, 2, 4} with op 1 (exp), acc 0
// (VGPR accumulators) or 1 (AGPR accumulators); sink: 512 floats per workgroup
hipError_t launch_coexec_probe(const bf16_t* operands, int mode, int valu, int op, int acc,
                               int workgroups, int iters, float* sink, hipStream_t s);
hipError_t launch_tile_read(const bf16_t* buf, size_t buf_bytes, int tile_bytes,
                            const int32_t* ids, int waves, int tiles_per_wave, uint32_t* sink,
                            hipStream_t s);

// k_gather.hip: cube-major, MFMA-operand-ordered copies of a token tensor (c == 64, bf16).
//   mode bit 1: "row" layout (lane = token, 8 consecutive d per lane);
//   mode bit 2: "transposed" layout (lane = d, 8 tokens per lane, in S-accumulator key order).
// Output cube ids cover the condition cubes (from x_cache) first, then the noise cubes.
enum { GATHER_ROW = 1, GATHER_TRANS = 2 };
size_t gather_bytes(const Geom& g, bool with_cache);
hipError_t launch_gather(const Geom& g, const void* x, const void* x_cache, int mode,
                         bf16_t* out_row, bf16_t* out_trans, hipStream_t s);

// k_attn_mfma.hip: bf16 MFMA forward for c == 64, D in {64, 128}; q_row is Q in the ROW gather
// layout over the nbq query cubes ([B, Hh, nbq, 64*D]).  ns <= 1 runs one pass per
// query cube; ns > 1 splits the key cube ids into ns ranges (one XCD's L2 per range) and merges
// the partials, which need fwd_split_bytes(g, ns) bytes of split_ws.  On a ragged grid kmask
// points at fwd_kmask_bytes(g) bytes the launch fills with every key cube's slot mask (null and
// unused otherwise).
int fwd_split_ranges(const Geom& g, int k_sel, int requested);
size_t fwd_split_bytes(const Geom& g, int ns);
hipError_t launch_fwd_mfma(const Geom& g, const bf16_t* q_row, const bf16_t* k_row,
                           const bf16_t* v_trans, const int32_t* idx, int k_sel, float scale,
                           void* o, float* lse, int ns, void* split_ws, uint2* kmask,
                           hipStream_t s);
// Bytes of the per-key-cube slot-mask table the MFMA forward needs on a ragged grid (else 0).
size_t fwd_kmask_bytes(const Geom& g);

// k_bwd_mfma.hip (dK/dV), k_bwd_dq.hip (dQ): bf16 MFMA backward kernels for c == 64, D in
// {64, 128}; every operand comes from the ROW gather layout (transposed operands are read from
// LDS with ds_read_b64_tr_b16).
// k_row / v_row cover all nbk key cubes (condition cubes first), q_row / do_row the nbq query
// cubes; dK/dV of condition key cubes go to dk_cache / dv_cache ([B, Nc, Hh, D]).
// pipelined: at D = 128 run the software-pipelined variant (same bits; launch_bwd_dq_pipe).
// walk_ticks > 0 (D = 128 dK/dV and pipelined dQ only): each work item starts its walk over its
// list at the entry nearest the phase of the 100 MHz real-time clock within that period and
// wraps (locality experiment; the summation order then depends on timing).  0: from the start.
hipError_t launch_bwd_dq_mfma(const Geom& g, const bf16_t* q_row, const bf16_t* do_row,
                              const bf16_t* k_row, const bf16_t* v_row, const float2* ld_c,
                              const int32_t* idx, int k_sel, float scale, float* dq,
                              bool pipelined, int walk_ticks, hipStream_t s);
// k_bwd_dq64.hip: the one-wave dQ kernel at head_dim 64 (grid B*Hh*cpx*8 waves, cpx = query
// cubes per XCD slice); called by launch_bwd_dq_mfma.
hipError_t launch_bwd_dq64(const Geom& g, const bf16_t* q_row, const bf16_t* do_row,
                           const bf16_t* k_row, const bf16_t* v_row, const float2* ld_c,
                           const int32_t* idx, int k_sel, float scale, float c_log2, int cpx,
                           float* dq, hipStream_t s);
// k_bwd_dq_pipe_ragged.hip: the pipelined dQ at head_dim 128 on a ragged grid; called by
// launch_bwd_dq_pipe.
hipError_t launch_bwd_dq_pipe_ragged(const Geom& g, const bf16_t* q_row, const bf16_t* do_row,
                                     const bf16_t* k_row, const bf16_t* v_row,
                                     const float2* ld_c, const int32_t* idx, int k_sel,
                                     float scale, float c_log2, int cpx, int walk_ticks,
                                     float* dq, hipStream_t s);
hipError_t launch_bwd_dq_pipe(const Geom& g, const bf16_t* q_row, const bf16_t* do_row,
                              const bf16_t* k_row, const bf16_t* v_row, const float2* ld_c,
                              const int32_t* idx, int k_sel, float scale, float* dq,
                              int walk_ticks, hipStream_t s);
// order: dkdv_order_bytes(g) bytes the launch fills with the longest-first item order (null:
// the fixed XCD-balanced order).  by_keys (D = 128): the two waves of a key cube split its keys
// (dS from the fp32 P) instead of its outputs (dS from the bf16 P handed between them).
size_t dkdv_order_bytes(const Geom& g);
hipError_t launch_bwd_dkdv_mfma(const Geom& g, const bf16_t* k_row, const bf16_t* v_row,
                                const bf16_t* q_row, const bf16_t* do_row, const float2* ld_c,
                                const int32_t* csr_off, const int32_t* csr_list, int32_t* order,
                                float scale, int walk_ticks, bool by_keys, float* dk, float* dv,
                                float* dk_cache, float* dv_cache, hipStream_t s);

}  // namespace bsa
