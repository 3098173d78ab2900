/*
 * bsa.h -- C ABI of the MI355X (gfx950) Block Sparse Attention library (libbsa.so).
 *
 * Block Sparse Attention over a 3D video latent grid, as the LongCat-Video pages describe it:
 *   - the visual tokens of a (T, H, W) latent grid are cut into small 3D cubes, and each query
 *     cube attends only to the few key cubes most relevant to it, chosen by similarity rather
 *     than distance, which keeps attention compute under about a tenth of dense
 *     ["LongCat-Video : Generate 1 minute long AI videos with this model" (Data Science in Your
 *     Pocket), section "Sparse attention"; "LongCat-Video视频生成模型发布 迈出世界模型探索第一步"
 *     (youleyou), section "块稀疏注意力（BSA）"];
 *   - a query cube always keeps its own cube and skips every unselected block pair entirely
 *     ["LongCat-Video deep dive" (ai-news-5min-kr), block-sparse attention paragraph and its
 *     same-table analogy];
 *   - block-causal attention with cached condition-frame K/V serves video continuation
 *     ["LongCat-Video 高效長視頻生成探索世界模型的第壹步" (meituan.com talk), section 2.1;
 *     youleyou page, section "长视频生成：5分钟连贯输出，质量全程在线"; Data Science in Your
 *     Pocket page, section "The core idea: one model for all video tasks"];
 *   - forward and backward both exist, for inference and training (meituan.com talk, section 2.2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout.  Token tensors are [B, N, Hh, D], C-contiguous ("BNHD"), tokens in raster order of the
 *    latent grid: token n = (t*H + h)*W + w.  Query, key and value tensors (q, k, v, o, d_o and the
 *    gradients) hold only the NOISE segment, i.e. the last T - cond_T frames, so N = Nq =
 *    (T - cond_T)*H*W.  k_cache / v_cache hold the first cond_T frames: N = Nc = cond_T*H*W.
 *  Cubes.  A cube is ct x ch x cw tokens (c = ct*ch*cw).  Cube coordinates (a, b, e) =
 *    (t/ct, h/ch, w/cw) inside a segment; the cube id inside a segment is a*gh*gw + b*gw + e
 *    with gh = ceil(H/ch), gw = ceil(W/cw) cubes along h and w.
 *    Key cube ids put the nbc condition cubes first (0..nbc-1) and the nbq noise cubes after them
 *    (nbc..nbc+nbq-1); query cube i is key cube nbc+i.  nbk = nbc + nbq.
 *  Pooled tensors are [B, Hh, nbq, D] fp32.  idx is [B, Hh, nbq, k_sel] int32, each row ascending.
 *    mask is [B, Hh, nbq, nbk] uint8 (1 = key cube attended).  lse is [B, Hh, Nq] fp32 (natural log).
 *  Ownership.  The caller owns every buffer; the library never allocates, frees or synchronises.
 *    Device pointers must be device-resident (hipMalloc / torch) and 16-byte aligned.
 *  Streams.  Every launch is asynchronous on the stream passed in (NULL = the null stream).
 *  Errors.  Arguments are checked on the host before any launch and before any HIP call; a bad
 *    argument returns an error code and launches nothing.  A launch failure returns BSA_ERR_HIP.
 *    Faults inside kernels surface, as usual for HIP, at the caller's next synchronisation.
 *    No C++ exception crosses this interface.
 *  Threads.  The library keeps no state between calls other than per-thread settings
 *    (bsa_set_kernel_path, bsa_set_tuning, stage events) and the static scratch array of the
 *    allocation-free forward; concurrent calls on different streams are safe as long as their
 *    output and workspace buffers do not overlap (bsa_sparse_attn_fwd_noalloc: see there).
 */
#ifndef BSA_H_
#define BSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARG = 1, /* null required pointer, non-positive size, k_sel mismatch, bad r  */
  BSA_ERR_SHAPE = 2,       /* grid not divisible by the cube, cond_T not a cube multiple, ...   */
  BSA_ERR_UNSUPPORTED = 3, /* head_dim or cube size outside what the kernels implement          */
  BSA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than bsa_workspace_bytes()           */
  BSA_ERR_HIP = 5,         /* a HIP launch or runtime call failed                               */
  BSA_ERR_INTERNAL = 6     /* unexpected internal failure (caught exception)                    */
} bsa_status_t;

typedef enum { BSA_F32 = 0, BSA_BF16 = 1 } bsa_dtype_t;

/* Shape of one problem.  T counts all frames, condition frames included; cond_T = 0 means no
 * condition cache and plain (non-causal) block-sparse attention.
 * Requirements: all sizes > 0 except cond_T >= 0; head_dim in {64, 128}; T - cond_T and cond_T
 * divisible by cube_t, cond_T < T; cube size c = cube_t*cube_h*cube_w <= 256; at most 39808
 * cubes per segment (the selection keeps one row of keys in LDS), and for the backward at most
 * 39936 key cubes (condition + noise) in all.  H and W need not be multiples of cube_h, cube_w
 * (ragged latent grids such as the 45-token height of 720p): the last cube row / column then
 * keeps only the tokens of its box that lie inside the grid -- its mean divides by that count
 * and its missing slots are neither keys nor queries.  Cube counts are ceil(H/cube_h) *
 * ceil(W/cube_w) per cube layer. */
typedef struct {
  int32_t batch, heads, head_dim; /* B, Hh, D                                  */
  int32_t T, H, W;                /* latent grid, condition frames included    */
  int32_t cube_t, cube_h, cube_w; /* ct, ch, cw                                */
  int32_t cond_T;                 /* leading condition frames (0 = none)       */
} bsa_problem_t;

/* Mean-pool every cube of one token tensor (3D cube partition plus per-cube mean; the relevance
 * descriptor used to find the most similar cubes, Data Science in Your Pocket page, section
 * "Sparse attention").
 *   x       device, [B, Nq, Hh, D] of dtype (noise segment of Q or K)
 *   x_mean  device, [B, Hh, nbq, D] fp32, written: x_mean[b,h,i,:] = (1/c) * sum of the c token
 *           rows of cube i for head h, accumulated in fp32.
 * Errors: INVALID_ARG (null pointer, bad sizes), SHAPE, UNSUPPORTED, HIP. */
bsa_status_t bsa_block_pool(const bsa_problem_t* p, bsa_dtype_t dtype, const void* x,
                            float* x_mean, hipStream_t stream);

/* Attention prologue fused with the cube pool: QK RMS normalisation (RMSNorm + QKNorm) and 3D
 * rotary position embedding over time, height and width (xugj520 page, section "三、模型架构";
 * ai-news-5min-kr deep dive, layer table row for the positional encoding), then the per-cube
 * means of the result, in one pass over x.  The pages give no formula; per (token, head):
 *   y = x / sqrt(mean_d x^2 + eps) * gamma[d], then channel pairs (2i, 2i+1) of the time, height
 *   and width blocks (contiguous, widths D - 4*floor(D/6), 2*floor(D/6), 2*floor(D/6)) rotated by
 *   the angle pos_axis * rope_theta^(-2i / block width); pos = the token's (t, h, w) on the full
 *   latent grid, condition frames first (noise frame f has t = cond_T + f).
 *   segment  0: the noise segment, x [B, Nq, Hh, D]; 1: the condition segment (needs cond_T > 0),
 *            x [B, cond_T*H*W, Hh, D]
 *   x        device, dtype, read
 *   gamma    device, [D] fp32 per-channel gain, or NULL for all ones
 *   rope_theta  rotation base (10000 is the usual choice), finite and > 1
 *   eps      finite and > 0 (1e-6 is the usual choice)
 *   x_out    device, same shape and dtype as x, written (RNE to bf16); may equal x (in place)
 *   x_mean   device, [B, Hh, nbq, D] fp32, written with the cube means of y before rounding
 *            (segment 0 only; NULL skips it; must be NULL for segment 1)
 * Errors: INVALID_ARG (null x / x_out, bad segment, theta, eps, x_mean with segment 1), SHAPE,
 * UNSUPPORTED, HIP. */
bsa_status_t bsa_qk_prologue(const bsa_problem_t* p, bsa_dtype_t dtype, int32_t segment,
                             const void* x, const float* gamma, float rope_theta, float eps,
                             void* x_out, float* x_mean, hipStream_t stream);

/* Score every candidate key cube against each query cube and keep the top r (top-r key blocks,
 * youleyou page, section "块稀疏注意力（BSA）"; similarity-based choice, Data Science in Your Pocket
 * page, section "Sparse attention"; own block always kept, ai-news-5min-kr deep dive, same-table
 * analogy).
 *   q_mean, k_mean  device, [B, Hh, nbq, D] fp32 (from bsa_block_pool on Q and on noise K)
 *   r               >= 0; clamped to the nbq-1 candidates (r >= nbq-1 gives dense attention)
 *   idx             device, [B, Hh, nbq, k_sel] int32, written; k_sel = bsa_num_selected(p, r)
 *   mask            device, [B, Hh, nbq, nbk] uint8, written, or NULL to skip it
 * Score S[i,j] = D^-1/2 * <q_mean_i, k_mean_j> in fp32.  Row i keeps the forced set (all nbc
 * condition cubes and its own cube nbc+i) plus the first min(r, nbq-1) noise cubes j != i in order
 * of (score descending, cube id ascending); -0.0 counts as +0.0.  Rows are written ascending.
 * Scores must be finite.
 * Errors: INVALID_ARG, SHAPE, UNSUPPORTED, HIP. */
bsa_status_t bsa_select_topr(const bsa_problem_t* p, const float* q_mean, const float* k_mean,
                             int32_t r, int32_t* idx, uint8_t* mask, hipStream_t stream);

/* Gathered block-sparse flash attention, forward (skips unselected block pairs, ai-news-5min-kr
 * deep dive, block-sparse attention paragraph).  For each query cube i:
 *   O_i = softmax(softmax_scale * Q_i K_sel(i)^T) V_sel(i),  LSE_i = log sum exp(...)
 * where K_sel(i)/V_sel(i) are the tokens of the key cubes in idx[b,h,i,:]; condition cubes
 * (id < nbc) are read from k_cache / v_cache, noise cubes from k / v (block-causal continuation
 * with a condition-token cache, meituan.com talk, section 2.1).
 *   q, k, v            device, [B, Nq, Hh, D] dtype
 *   k_cache, v_cache   device, [B, Nc, Hh, D] dtype; must be NULL iff cond_T == 0
 *   idx, k_sel         as written by bsa_select_topr (every entry in [0, nbk), rows ascending)
 *   o                  device, [B, Nq, Hh, D] dtype, written (bf16 by round-to-nearest-even)
 *   lse                device, [B, Hh, Nq] fp32, written
 *   ws, ws_bytes       device workspace of at least bsa_workspace_bytes(p, dtype, k_sel, 0)
 *                      bytes (may be NULL when that is 0); contents are scratch
 * Errors: INVALID_ARG, SHAPE, UNSUPPORTED, WORKSPACE, HIP. */
bsa_status_t bsa_sparse_attn_fwd(const bsa_problem_t* p, bsa_dtype_t dtype, const void* q,
                                 const void* k, const void* v, const void* k_cache,
                                 const void* v_cache, const int32_t* idx, int32_t k_sel,
                                 float softmax_scale, void* o, float* lse, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/* Allocation-free variant of bsa_sparse_attn_fwd, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and errors as bsa_sparse_attn_fwd without ws / ws_bytes: the workspace is a
 * static device array of BSA_NOALLOC_SCRATCH_BYTES (256 MiB) that each GPU the library runs on
 * holds until the process ends.  Problems whose bsa_workspace_bytes(p, dtype, k_sel, 0) exceeds
 * it return BSA_ERR_WORKSPACE and launch nothing (a single-pass forward, BSA_TUNE_FWD_SPLITS = 1,
 * needs the least).  No call allocates or frees memory.  Every call on one GPU uses that GPU's one
 * array and leaves its contents behind (nothing in it has to start at zero): calls that overlap
 * in time on one GPU (other host threads, other streams) race and must be serialised by the
 * caller. */
#define BSA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
bsa_status_t bsa_sparse_attn_fwd_noalloc(const bsa_problem_t* p, bsa_dtype_t dtype,
                                         const void* q, const void* k, const void* v,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* idx, int32_t k_sel, float softmax_scale,
                                         void* o, float* lse, hipStream_t stream);

/* Backward of bsa_sparse_attn_fwd with the selection held constant (the forward and backward
 * both ship, meituan.com talk, section 2.2; training with a condition cache is the continuation
 * pre-training of section 2.1).  With P = exp(scale*Q_i K_j^T - LSE_i):
 *   dV_j += P^T dO_i;  dS = P o (dO_i V_j^T - Delta_i);  dQ_i += scale*dS K_j;
 *   dK_j += scale*dS^T Q_i;  Delta_i = rowsum(dO_i o O_i),  over every i and j in idx[b,h,i,:].
 * Condition key cubes (id < nbc) are read from k_cache / v_cache and their dK_j, dV_j are written
 * to dk_cache / dv_cache.
 *   q, k, v, o, d_o    device, [B, Nq, Hh, D] dtype (o, lse from the forward)
 *   k_cache, v_cache   device, [B, Nc, Hh, D] dtype; NULL iff cond_T == 0
 *   lse                device, [B, Hh, Nq] fp32
 *   dq, dk, dv         device, [B, Nq, Hh, D] fp32, overwritten
 *   dk_cache, dv_cache device, [B, Nc, Hh, D] fp32, overwritten; NULL iff cond_T == 0
 *   fwd_ws, fwd_ws_bytes  NULL / 0, or the workspace of the bsa_sparse_attn_fwd call that produced
 *                      o and lse, unchanged since, with q, k, k_cache unchanged too: the bf16 MFMA
 *                      path then reads the gathered Q and K it holds instead of gathering them
 *                      again (read only; ignored by the portable path).  WORKSPACE if it is
 *                      smaller than that forward's workspace could be.
 *   ws, ws_bytes       device workspace of at least bsa_workspace_bytes(p, dtype, k_sel, 1)
 * With cond_T > 0 only the bf16 MFMA path (64-token cubes) is implemented: UNSUPPORTED otherwise.
 * Precision (bf16): P and dS enter their products rounded to bf16, with fp32 accumulation; at
 * head_dim 128 the dS of dK/dV is formed from the bf16-rounded P.  Results are deterministic
 * (no atomics), and the same with or without fwd_ws.
 * Errors: INVALID_ARG, SHAPE, UNSUPPORTED, WORKSPACE, HIP. */
bsa_status_t bsa_sparse_attn_bwd(const bsa_problem_t* p, bsa_dtype_t dtype, const void* q,
                                 const void* k, const void* v, const void* k_cache,
                                 const void* v_cache, const void* o, const void* d_o,
                                 const float* lse, const int32_t* idx, int32_t k_sel,
                                 float softmax_scale, float* dq, float* dk, float* dv,
                                 float* dk_cache, float* dv_cache, const void* fwd_ws,
                                 size_t fwd_ws_bytes, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* ---- helpers (host only, no HIP calls) ---- */

/* k_sel = nbc + 1 + min(r, nbq - 1), or -1 if p is invalid or r < 0. */
int32_t bsa_num_selected(const bsa_problem_t* p, int32_t r);

/* Workspace bytes for the forward (bwd = 0) or backward (bwd = 1) call; (size_t)-1 if invalid. */
size_t bsa_workspace_bytes(const bsa_problem_t* p, bsa_dtype_t dtype, int32_t k_sel, int32_t bwd);

/* Human-readable name of a status code (static string). */
const char* bsa_status_string(bsa_status_t s);

/* Text of the last argument error raised on this thread (static per thread, never NULL). */
const char* bsa_last_error(void);

/* Stage timing for profiling.  When events != NULL, every entry point records HIP events (created
 * by the caller) on its stream at the boundaries of its internal kernels: events[0] before the
 * first launch and events[s + 1] after internal stage s, for slots < n.  Stage s spans
 * events[s] -> events[s + 1]; bsa_stage_count() and bsa_stage_name() describe the stages of the
 * last entry point called on this thread.  Pass NULL to disable.  The setting is per host thread. */
void bsa_set_stage_events(hipEvent_t* events, int32_t n);
int32_t bsa_stage_count(void);
const char* bsa_stage_name(int32_t s); /* "" when s is out of range */

/* Kernel path selection (testing and diagnostics), per host thread: 0 = automatic (bf16 MFMA
 * kernels for 64-token cubes, portable fp32-arithmetic kernels otherwise), 1 = always the
 * portable kernels.  Returns BSA_ERR_INVALID_ARG for other values. */
bsa_status_t bsa_set_kernel_path(int32_t path);

/* Tuning switches (testing and diagnostics), per host thread, read by every later call on that
 * thread (bsa_workspace_bytes included, so size the workspace on the thread that calls).  The
 * defaults are the measured fastest schedules.
 *   BSA_TUNE_FWD_SPLITS   -1 (default): the size rule; 1: single pass; 2..64: the bf16 MFMA
 *                         forward splits the key cubes into that many ranges, each attended
 *                         separately and merged (one XCD's L2 per range).  Changes the
 *                         summation order, so outputs change at rounding level, and the
 *                         forward workspace size.
 *   BSA_TUNE_DKDV_ORDER   1 (default): dK/dV items longest list first; 0: fixed order.  Same bits.
 *   BSA_TUNE_DQ_PIPELINE  1 (default): software-pipelined dQ where it exists; 0: plain loop.
 *                         Same bits.
 *   BSA_TUNE_WALK_PHASE   0 (default): every backward work item at D = 128 walks its list of
 *                         cubes from the first entry.  1..1000000: a period in microseconds;
 *                         each item of the D = 128 dK/dV and pipelined dQ kernels starts at the
 *                         entry nearest the phase of the GPU's real-time clock within that
 *                         period (and wraps), so the items running together read neighbouring
 *                         cubes and share L2 lines.  A locality experiment: the summation order
 *                         then depends on timing, so the gradients vary at rounding level from
 *                         run to run (not deterministic).
 *   BSA_TUNE_DKDV_SPLIT   0 (default): the bf16 MFMA dK/dV at D = 128 splits each key cube's
 *                         work between two waves by output (one accumulates dV, the other dK,
 *                         the softmax P crosses between them as bf16, so dK's dS is formed from
 *                         the bf16-rounded P).  1: by keys (each wave accumulates dK and dV of
 *                         half the keys and forms dS from its own fp32 P, as the dQ pass does):
 *                         dK closer to the exact gradient, a few percent slower.
 * Returns BSA_ERR_INVALID_ARG (setting unchanged) for an unknown key or an out-of-range value. */
typedef enum {
  BSA_TUNE_FWD_SPLITS = 0,
  BSA_TUNE_DKDV_ORDER = 1,
  BSA_TUNE_DQ_PIPELINE = 2,
  BSA_TUNE_WALK_PHASE = 3,
  BSA_TUNE_DKDV_SPLIT = 4
} bsa_tune_t;
bsa_status_t bsa_set_tuning(bsa_tune_t key, int32_t value);
int32_t bsa_get_tuning(bsa_tune_t key); /* INT32_MIN for an unknown key */

/* Check a selection against the contract of bsa_sparse_attn_fwd / _bwd (every entry in
 * [0, nbk), every row strictly ascending), asynchronously on `stream`: *bad_rows (device int32,
 * overwritten) receives the number of rows that break it, readable after the stream
 * synchronises.  The attention calls themselves do not check (a malformed row gives wrong
 * gradients, not an error); this is the debugging aid.  Rows of bsa_select_topr always pass.
 * Errors: INVALID_ARG (null pointer, k_sel), SHAPE, UNSUPPORTED, HIP. */
bsa_status_t bsa_validate_idx(const bsa_problem_t* p, const int32_t* idx, int32_t k_sel,
                              int32_t* bad_rows, hipStream_t stream);

/* ---- diagnostics: microbenchmarks of the limits the attention kernels run against ---- */

/* Back-to-back bf16 MFMA (v_mfma_f32_32x32x16_bf16, four independent accumulator chains per
 * wave) on `waves` one-wave workgroups, iters x 8 products each (32768 FLOP per product), with
 * the 8 operand fragments of every wave read from `operands` (at least 8192 bytes of bf16).  The
 * rate bf16 MFMA work reaches on that data: with N(0,1) operands the chip runs at a lower clock
 * than with constant ones.  sink: device, >= 64 floats per wave, overwritten.
 * Errors: INVALID_ARG, HIP. */
bsa_status_t bsa_probe_mfma(const void* operands, size_t operand_bytes, int32_t waves,
                            int32_t iters, float* sink, size_t sink_bytes, hipStream_t stream);

/* The same with the product shape and the chain count chosen: shape 0 = 32x32x16 (8 products of
 * 32768 FLOP per iteration), 1 = v_mfma_f32_16x16x32_bf16 (16 products of 16384 FLOP);
 * chains in {1, 2, 4, 8} independent accumulators per wave (1: every product depends on the one
 * before it).  How many independent products a wave must keep in flight for the full rate.
 * Errors: INVALID_ARG (bad shape or chains, as above), HIP. */
bsa_status_t bsa_probe_mfma_shape(const void* operands, size_t operand_bytes, int32_t shape,
                                  int32_t chains, int32_t waves, int32_t iters, float* sink,
                                  size_t sink_bytes, hipStream_t stream);

/* bf16 MFMA beside VALU work on one SIMD: `workgroups` eight-wave workgroups (two waves on every
 * SIMD of a CU), each wave iterating `iters` times over four v_mfma_f32_32x32x16_bf16 products
 * (four independent accumulators, operands from the first 2048 bytes of `operands`), each
 * product followed by `valu` VALU instructions on eight independent fp32 chains (op 0:
 * v_fma_f32; op 1: v_exp_f32).  mode 0: every wave does both, the VALU instructions scheduled
 * right after each product; 1: of the two waves on a SIMD one does the products and the other
 * the VALU instructions; 2: products only; 3: VALU instructions only.  Comparing the modes
 * shows how much VALU work (the softmax of the attention kernels) can run beside the products
 * within a wave and across the waves of a SIMD.  valu: {0, 2, 4, 8, 16} for op 0, {1, 2, 4} for
 * op 1.  acc 0: the products accumulate in VGPRs (what the compiler picks for a kernel within
 * 256 registers); 1: in AGPRs.  sink: device, >= 512 floats per workgroup, overwritten.
 * Errors: INVALID_ARG, HIP. */
bsa_status_t bsa_probe_mfma_valu(const void* operands, size_t operand_bytes, int32_t mode,
                                 int32_t valu, int32_t op, int32_t acc, int32_t workgroups,
                                 int32_t iters, float* sink, size_t sink_bytes,
                                 hipStream_t stream);

/* Whole-tile reads: wave w (workgroup w, which runs on XCD w % 8) reads tiles
 * ids[w * tiles_per_wave + t] of `buf` (tile_bytes each, a multiple of 8192 up to 1 MiB) as
 * 1 KB wave-wide 16-byte-per-lane loads -- the attention kernels' tile access pattern.  Ids
 * outside buf are skipped.  buf: device, at most 2^31 - 1 bytes; ids: device, n_ids >= waves *
 * tiles_per_wave entries; sink: device, >= 64 words per wave, overwritten.
 * Errors: INVALID_ARG, HIP. */
bsa_status_t bsa_probe_tile_read(const void* buf, size_t buf_bytes, int32_t tile_bytes,
                                 const int32_t* ids, size_t n_ids, int32_t waves,
                                 int32_t tiles_per_wave, uint32_t* sink, size_t sink_bytes,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BSA_H_ */
