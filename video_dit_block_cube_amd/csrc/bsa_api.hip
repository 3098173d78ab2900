// bsa_api.hip -- the C ABI of libbsa.so: argument checks, workspace carving, kernel dispatch.
//
// Entry points follow the statement of the method on the LongCat-Video pages: pool cubes and
// pick the top-r key cubes per query cube ("LongCat-Video视频生成模型发布 迈出世界模型探索第一步",
// youleyou, section "块稀疏注意力（BSA）"), attend only the selected cube pairs with an optional
// cached condition segment ("LongCat-Video deep dive", ai-news-5min-kr, block-sparse attention
// paragraph; "LongCat-Video 高效長視頻生成探索世界模型的第壹步", meituan.com talk, section 2.1),
// and the backward (same talk, section 2.2).  Every check runs on the host before any HIP call.
#include <cmath>
#include <cstring>
#include <exception>
#include <climits>
#include <mutex>
#include <string>

#include "bsa.h"
#include "bsa_launch.h"

using namespace bsa;

namespace {

thread_local std::string t_err;
thread_local hipEvent_t* t_events = nullptr;
thread_local int t_nevents = 0;
thread_local const char* t_stage_names[16];
thread_local int t_nstages = 0;
thread_local int t_path = 0;
// Tuning switches (bsa_set_tuning): forward key-range count (-1 = size rule), longest-first
// dK/dV dispatch, pipelined dQ.
thread_local int t_fwd_splits = -1;
thread_local int t_dkdv_order = 1;
thread_local int t_dq_pipeline = 1;
thread_local int t_walk_phase_us = 0;
thread_local int t_dkdv_split = 0;
constexpr int kMaxFwdSplits = 64;

constexpr size_t kAlign = 256;
// Cubes per segment: one selection row (a 4-byte key per noise cube), the query descriptor and a
// 1024-entry histogram share the 160 KiB of LDS -- (nbq + D + 1024) * 4 <= 160 KiB at D = 128.
constexpr int kMaxNoiseCubes = 39808;
// Key cubes (condition + noise) for the backward: the CSR transpose scans nbk counters plus a
// 1024-entry scan buffer in LDS -- (nbk + 1024) * 4 <= 160 KiB.
constexpr int kMaxBwdKeyCubes = 39936;

bsa_status_t fail(bsa_status_t st, const std::string& msg) {
  t_err = msg;
  return st;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Stage bookkeeping for the optional profiling events.
struct Stages {
  hipStream_t s;
  explicit Stages(hipStream_t st) : s(st) {
    t_nstages = 0;
    if (t_events && t_nevents > 0) hipEventRecord(t_events[0], s);
  }
  void done(const char* name) {
    if (t_nstages < 16) t_stage_names[t_nstages] = name;
    ++t_nstages;
    if (t_events && t_nstages < t_nevents) hipEventRecord(t_events[t_nstages], s);
  }
};

bsa_status_t check_problem(const bsa_problem_t* p, Geom* g) {
  if (!p) return fail(BSA_ERR_INVALID_ARG, "problem pointer is NULL");
  if (p->batch <= 0 || p->heads <= 0 || p->head_dim <= 0 || p->T <= 0 || p->H <= 0 ||
      p->W <= 0 || p->cube_t <= 0 || p->cube_h <= 0 || p->cube_w <= 0)
    return fail(BSA_ERR_INVALID_ARG, "every size must be positive");
  if (p->cond_T < 0) return fail(BSA_ERR_INVALID_ARG, "cond_T must be >= 0");
  if (p->cond_T >= p->T) return fail(BSA_ERR_SHAPE, "cond_T must be < T");
  if ((p->T - p->cond_T) % p->cube_t || p->cond_T % p->cube_t)
    return fail(BSA_ERR_SHAPE, "noise frames and cond_T must be multiples of cube_t");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(BSA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const long long c = (long long)p->cube_t * p->cube_h * p->cube_w;
  if (c > 256) return fail(BSA_ERR_UNSUPPORTED, "cube size must be <= 256 tokens");
  const long long hw = (long long)((p->H + p->cube_h - 1) / p->cube_h) *
                       ((p->W + p->cube_w - 1) / p->cube_w);  // partial edge cubes included
  const long long nbq = (long long)(p->T - p->cond_T) / p->cube_t * hw;
  const long long nbc = (long long)p->cond_T / p->cube_t * hw;
  if (nbq > kMaxNoiseCubes || nbc > kMaxNoiseCubes)
    return fail(BSA_ERR_UNSUPPORTED, "at most 39808 cubes per segment");
  const long long tokens = (long long)p->T * p->H * p->W;
  if (tokens * p->heads * p->head_dim * p->batch > (1LL << 40))
    return fail(BSA_ERR_UNSUPPORTED, "problem too large");
  *g = make_geom(p->batch, p->heads, p->head_dim, p->T, p->H, p->W, p->cube_t, p->cube_h,
                 p->cube_w, p->cond_T);
  return BSA_OK;
}

bool use_mfma(const Geom& g, bsa_dtype_t dt) { return t_path == 0 && dt == BSA_BF16 && g.c == 64; }

bsa_status_t check_dtype(bsa_dtype_t dt) {
  if (dt != BSA_F32 && dt != BSA_BF16) return fail(BSA_ERR_INVALID_ARG, "unknown dtype");
  return BSA_OK;
}

bsa_status_t check_ksel(const Geom& g, int32_t k_sel) {
  if (k_sel < g.nbc + 1 || k_sel > g.nbk)
    return fail(BSA_ERR_INVALID_ARG, "k_sel is not nbc + 1 + min(r, nbq - 1) for any r >= 0");
  // CSR positions and per-(b, h) index arithmetic stay in int32
  if ((long long)g.B * g.Hh * g.nbq * k_sel >= (1LL << 31))
    return fail(BSA_ERR_UNSUPPORTED, "selection too large for int32 positions");
  return BSA_OK;
}

bsa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BSA_OK;
  return fail(BSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Workspace layout of the backward (and of the forward for the MFMA path).
// The query-only view of a problem (no condition segment): gathers of Q cover the noise cubes.
Geom noise_only(const Geom& g) {
  return make_geom(g.B, g.Hh, g.D, g.nT, g.H, g.W, g.ct, g.ch, g.cw, 0);
}

struct BwdWs {
  size_t delta, lse, ld, bits, off, list, g_qr, g_dr, g_kr, g_vr, order, total;
};

BwdWs bwd_layout(const Geom& g, bool mfma, int k_sel) {
  BwdWs w{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at += align_up(bytes);
    return here;
  };
  const size_t per_cube = (size_t)g.B * g.Hh * g.nbq * g.c * sizeof(float);
  w.delta = take(per_cube);
  w.lse = take(per_cube);
  w.ld = take(2 * per_cube);
  w.bits = take(csr_bits_words(g) * sizeof(uint32_t));
  w.off = take((size_t)g.B * g.Hh * (g.nbk + 1) * sizeof(int32_t));
  w.list = take((size_t)g.B * g.Hh * g.nbq * (size_t)k_sel * sizeof(int32_t));
  if (mfma) {
    const size_t gq = gather_bytes(noise_only(g), true);  // Q, dO: the query cubes
    const size_t gk = gather_bytes(g, true);              // K, V: every key cube
    w.g_qr = take(gq);
    w.g_dr = take(gq);
    w.g_kr = take(gk);
    w.g_vr = take(gk);
    w.order = take(dkdv_order_bytes(g));
  }
  w.total = at;
  return w;
}

// Key-range split count of the MFMA forward: the size rule, or this thread's
// BSA_TUNE_FWD_SPLITS setting (1 disables the split).
int fwd_splits(const Geom& g, int k_sel) { return fwd_split_ranges(g, k_sel, t_fwd_splits); }

// Forward workspace (MFMA path): K rows + V^T over all nbk key cubes, Q rows over the nbq query
// cubes, the key-range partials, then (ragged grids) the key cubes' slot masks.  The gathered
// operands sit at fixed offsets whatever the split count: K rows at 0, V^T next, then Q rows.
size_t fwd_q_rows_offset(const Geom& g) { return 2 * align_up(gather_bytes(g, true)); }
size_t fwd_ws_bytes_min(const Geom& g, bool mfma) {
  return mfma ? fwd_q_rows_offset(g) + gather_bytes(noise_only(g), true) : 0;
}
size_t fwd_ws(const Geom& g, bool mfma, int k_sel) {
  if (!mfma) return 0;
  return 2 * align_up(gather_bytes(g, true)) + align_up(gather_bytes(noise_only(g), true)) +
         align_up(fwd_split_bytes(g, fwd_splits(g, k_sel))) + align_up(fwd_kmask_bytes(g));
}

template <typename F>
bsa_status_t guarded(F&& f) {
  try {
    return f();
  } catch (const std::exception& e) {
    return fail(BSA_ERR_INTERNAL, std::string("internal error: ") + e.what());
  } catch (...) {
    return fail(BSA_ERR_INTERNAL, "internal error");
  }
}

// Scratch of the allocation-free forward (bsa_sparse_attn_fwd_noalloc): one static device array
// that every GPU the library runs on holds until the process ends.  Host code never uses its name
// as an address: the device address is looked up once per device, with that device current, and
// kept per device.
constexpr size_t kScratchBytes = BSA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the device that `stream` launches to (the current device for
// the null stream).
bsa_status_t device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "device of the stream");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BSA_ERR_UNSUPPORTED, "device ordinals above 63 are not supported");
  std::call_once(g_scratch_once[dev], [dev]() {
    int cur = -1;
    hipError_t e2 = hipGetDevice(&cur);
    if (e2 == hipSuccess && cur != dev) e2 = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e2 == hipSuccess) e2 = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
    g_scratch_err[dev] = e2;
    g_scratch_ptr[dev] = e2 == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess)
    return hip_status(g_scratch_err[dev], "address of the static scratch array");
  *out = g_scratch_ptr[dev];
  return BSA_OK;
}

bsa_status_t fwd_impl(const bsa_problem_t* p, bsa_dtype_t dtype, const void* q,
                      const void* k, const void* v, const void* k_cache, const void* v_cache,
                      const int32_t* idx, int32_t k_sel, float softmax_scale, void* o, float* lse,
                      void* ws,
                      size_t ws_bytes, hipStream_t stream, const char* ws_what) {
  return guarded([&]() -> bsa_status_t {
    Geom g;
    bsa_status_t st = check_problem(p, &g);
    if (st != BSA_OK) return st;
    if ((st = check_dtype(dtype)) != BSA_OK) return st;
    if ((st = check_ksel(g, k_sel)) != BSA_OK) return st;
    if (!q || !k || !v || !idx || !o || !lse)
      return fail(BSA_ERR_INVALID_ARG, "q, k, v, idx, o and lse must be non-NULL");
    if (g.condT > 0 && (!k_cache || !v_cache))
      return fail(BSA_ERR_INVALID_ARG, "cond_T > 0 needs k_cache and v_cache");
    if (g.condT == 0 && (k_cache || v_cache))
      return fail(BSA_ERR_INVALID_ARG, "k_cache / v_cache given but cond_T == 0");
    if (!std::isfinite(softmax_scale)) return fail(BSA_ERR_INVALID_ARG, "softmax_scale not finite");
    const bool mfma = use_mfma(g, dtype);
    const size_t need = fwd_ws(g, mfma, k_sel);
    if (need > 0 && (!ws || ws_bytes < need))
      return fail(BSA_ERR_WORKSPACE, std::string(ws_what) + " holds " + std::to_string(ws_bytes) +
                                         " bytes; this problem needs " + std::to_string(need));
    Stages stages(stream);
    if (mfma) {
      char* base = static_cast<char*>(ws);
      const Geom gq = noise_only(g);
      bf16_t* krow = reinterpret_cast<bf16_t*>(base);
      bf16_t* vtr = reinterpret_cast<bf16_t*>(base + align_up(gather_bytes(g, true)));
      bf16_t* qrow = reinterpret_cast<bf16_t*>(base + 2 * align_up(gather_bytes(g, true)));
      void* split_ws = base + 2 * align_up(gather_bytes(g, true)) +
                       align_up(gather_bytes(gq, true));
      st = hip_status(launch_gather(g, k, k_cache, GATHER_ROW, krow, nullptr, stream),
                      "gather K");
      if (st != BSA_OK) return st;
      st = hip_status(launch_gather(g, v, v_cache, GATHER_TRANS, nullptr, vtr, stream),
                      "gather V");
      if (st != BSA_OK) return st;
      st = hip_status(launch_gather(gq, q, nullptr, GATHER_ROW, qrow, nullptr, stream),
                      "gather Q");
      if (st != BSA_OK) return st;
      stages.done("gather_qkv");
      const int ns = fwd_splits(g, k_sel);
      uint2* kmask = g.ragged ? reinterpret_cast<uint2*>(static_cast<char*>(split_ws) +
                                                         align_up(fwd_split_bytes(g, ns)))
                              : nullptr;
      st = hip_status(launch_fwd_mfma(g, qrow, krow, vtr, idx, k_sel, softmax_scale, o, lse, ns,
                                      split_ws, kmask, stream),
                      "attention forward launch");
      stages.done("attn_fwd_mfma");
    } else {
      st = hip_status(launch_fwd_simt(g, dtype == BSA_BF16, q, k, v, k_cache, v_cache, idx,
                                      k_sel, softmax_scale, o, lse, stream),
                      "attention forward launch");
      stages.done("attn_fwd_simt");
    }
    return st;
  });
}

}  // namespace

extern "C" {

bsa_status_t bsa_block_pool(const bsa_problem_t* p, bsa_dtype_t dtype, const void* x,
                            float* x_mean, hipStream_t stream) {
  return guarded([&]() -> bsa_status_t {
    Geom g;
    bsa_status_t st = check_problem(p, &g);
    if (st != BSA_OK) return st;
    if ((st = check_dtype(dtype)) != BSA_OK) return st;
    if (!x || !x_mean) return fail(BSA_ERR_INVALID_ARG, "x and x_mean must be non-NULL");
    Stages stages(stream);
    st = hip_status(launch_pool(g, dtype == BSA_BF16, x, x_mean, stream), "pool launch");
    stages.done("pool");
    return st;
  });
}

bsa_status_t bsa_qk_prologue(const bsa_problem_t* p, bsa_dtype_t dtype, int32_t segment,
                             const void* x, const float* gamma, float rope_theta, float eps,
                             void* x_out, float* x_mean, hipStream_t stream) {
  return guarded([&]() -> bsa_status_t {
    Geom g;
    bsa_status_t st = check_problem(p, &g);
    if (st != BSA_OK) return st;
    if ((st = check_dtype(dtype)) != BSA_OK) return st;
    if (!x || !x_out) return fail(BSA_ERR_INVALID_ARG, "x and x_out must be non-NULL");
    if (segment != 0 && segment != 1) return fail(BSA_ERR_INVALID_ARG, "segment must be 0 or 1");
    if (segment == 1 && g.condT == 0)
      return fail(BSA_ERR_INVALID_ARG, "segment 1 needs condition frames (cond_T > 0)");
    if (segment == 1 && x_mean)
      return fail(BSA_ERR_INVALID_ARG, "x_mean must be NULL for the condition segment");
    if (!(std::isfinite(rope_theta) && rope_theta > 1.0f))
      return fail(BSA_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
    if (!(std::isfinite(eps) && eps > 0.0f))
      return fail(BSA_ERR_INVALID_ARG, "eps must be finite and > 0");
    const Geom seg = segment == 0 ? noise_only(g)
                                  : make_geom(g.B, g.Hh, g.D, g.condT, g.H, g.W, g.ct, g.ch,
                                              g.cw, 0);
    Stages stages(stream);
    st = hip_status(launch_prologue(seg, segment == 0 ? g.condT : 0, dtype == BSA_BF16, x, gamma,
                                    rope_theta, eps, x_out, x_mean, stream),
                    "prologue launch");
    stages.done("qk_prologue");
    return st;
  });
}

bsa_status_t bsa_select_topr(const bsa_problem_t* p, const float* q_mean, const float* k_mean,
                             int32_t r, int32_t* idx, uint8_t* mask, hipStream_t stream) {
  return guarded([&]() -> bsa_status_t {
    Geom g;
    bsa_status_t st = check_problem(p, &g);
    if (st != BSA_OK) return st;
    if (r < 0) return fail(BSA_ERR_INVALID_ARG, "r must be >= 0");
    if (!q_mean || !k_mean || !idx)
      return fail(BSA_ERR_INVALID_ARG, "q_mean, k_mean and idx must be non-NULL");
    const int r_eff = r < g.nbq - 1 ? r : g.nbq - 1;
    const int k_sel = g.nbc + 1 + r_eff;
    if ((st = check_ksel(g, k_sel)) != BSA_OK) return st;
    Stages stages(stream);
    st = hip_status(launch_select(g, q_mean, k_mean, r_eff, k_sel, idx, mask, stream),
                    "select launch");
    stages.done("select");
    return st;
  });
}

bsa_status_t bsa_sparse_attn_fwd(const bsa_problem_t* p, bsa_dtype_t dtype, const void* q,
                                 const void* k, const void* v, const void* k_cache,
                                 const void* v_cache, const int32_t* idx, int32_t k_sel,
                                 float softmax_scale, void* o, float* lse, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  return fwd_impl(p, dtype, q, k, v, k_cache, v_cache, idx, k_sel, softmax_scale, o, lse, ws,
                  ws_bytes, stream, "workspace");
}

bsa_status_t bsa_sparse_attn_fwd_noalloc(const bsa_problem_t* p, bsa_dtype_t dtype,
                                         const void* q, const void* k, const void* v,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* idx, int32_t k_sel, float softmax_scale,
                                         void* o, float* lse, hipStream_t stream) {
  return guarded([&]() -> bsa_status_t {
    void* scratch_ptr = nullptr;
    const bsa_status_t st = device_scratch(stream, &scratch_ptr);
    if (st != BSA_OK) return st;
    return fwd_impl(p, dtype, q, k, v, k_cache, v_cache, idx, k_sel, softmax_scale, o, lse,
                    scratch_ptr, kScratchBytes, stream, "the static scratch array");
  });
}

bsa_status_t bsa_sparse_attn_bwd(const bsa_problem_t* p, bsa_dtype_t dtype, const void* q,
                                 const void* k, const void* v, const void* k_cache,
                                 const void* v_cache, const void* o, const void* d_o,
                                 const float* lse, const int32_t* idx, int32_t k_sel,
                                 float softmax_scale, float* dq, float* dk, float* dv,
                                 float* dk_cache, float* dv_cache, const void* fwd_ws,
                                 size_t fwd_ws_bytes, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  return guarded([&]() -> bsa_status_t {
    Geom g;
    bsa_status_t st = check_problem(p, &g);
    if (st != BSA_OK) return st;
    if ((st = check_dtype(dtype)) != BSA_OK) return st;
    if ((st = check_ksel(g, k_sel)) != BSA_OK) return st;
    if (!q || !k || !v || !o || !d_o || !lse || !idx || !dq || !dk || !dv)
      return fail(BSA_ERR_INVALID_ARG, "every tensor pointer must be non-NULL");
    if (g.nbk > kMaxBwdKeyCubes)
      return fail(BSA_ERR_UNSUPPORTED, "the backward supports at most 39936 key cubes");
    const bool cached = g.condT > 0;
    const bool any_cache = k_cache || v_cache || dk_cache || dv_cache;
    const bool all_cache = k_cache && v_cache && dk_cache && dv_cache;
    if (cached ? !all_cache : any_cache)
      return fail(BSA_ERR_INVALID_ARG,
                  "k_cache, v_cache, dk_cache, dv_cache are required iff cond_T > 0");
    if (!std::isfinite(softmax_scale)) return fail(BSA_ERR_INVALID_ARG, "softmax_scale not finite");
    const bool mfma = use_mfma(g, dtype);
    if (cached && !mfma)
      return fail(BSA_ERR_UNSUPPORTED,
                  "condition-cache gradients need the bf16 MFMA path (64-token cubes)");
    const BwdWs w = bwd_layout(g, mfma, k_sel);
    if (!ws || ws_bytes < w.total)
      return fail(BSA_ERR_WORKSPACE, "workspace smaller than bsa_workspace_bytes()");
    // The forward's workspace, when given, still holds the gathered K rows (every key cube) and
    // Q rows (the query cubes) of these inputs: the backward reads them instead of gathering.
    const bool reuse = mfma && fwd_ws != nullptr;
    if (fwd_ws && fwd_ws_bytes < fwd_ws_bytes_min(g, mfma))
      return fail(BSA_ERR_WORKSPACE, "fwd_ws is smaller than the forward's gathered operands");
    char* base = static_cast<char*>(ws);
    float* delta_c = reinterpret_cast<float*>(base + w.delta);
    float* lse_c = reinterpret_cast<float*>(base + w.lse);
    uint32_t* bits = reinterpret_cast<uint32_t*>(base + w.bits);
    int32_t* off = reinterpret_cast<int32_t*>(base + w.off);
    int32_t* list = reinterpret_cast<int32_t*>(base + w.list);
    const bool bf16 = dtype == BSA_BF16;
    Stages stages(stream);
    float2* ld_c = reinterpret_cast<float2*>(base + w.ld);
    auto at = [&](size_t o2) { return reinterpret_cast<bf16_t*>(base + o2); };
    if (mfma) {
      // Delta and the (LSE, Delta) pairs in one pass with the dO gather
      st = hip_status(launch_delta_gather(g, o, d_o, lse, ld_c, at(w.g_dr), stream),
                      "delta + dO gather launch");
    } else {
      st = hip_status(launch_delta(g, bf16, o, d_o, lse, delta_c, lse_c, ld_c, stream),
                      "delta launch");
    }
    if (st != BSA_OK) return st;
    st = hip_status(launch_csr(g, idx, k_sel, bits, off, list, stream), "csr launch");
    if (st != BSA_OK) return st;
    stages.done("bwd_prep");
    if (mfma) {
      const Geom gq = noise_only(g);
      const bf16_t* q_rows = reinterpret_cast<const bf16_t*>(
          reuse ? static_cast<const char*>(fwd_ws) + fwd_q_rows_offset(g) : base + w.g_qr);
      const bf16_t* k_rows = reinterpret_cast<const bf16_t*>(
          reuse ? static_cast<const char*>(fwd_ws) : base + w.g_kr);
      if (!reuse) {
        st = hip_status(launch_gather(gq, q, nullptr, GATHER_ROW, at(w.g_qr), nullptr, stream),
                        "gather Q");
        if (st != BSA_OK) return st;
        st = hip_status(launch_gather(g, k, k_cache, GATHER_ROW, at(w.g_kr), nullptr, stream),
                        "gather K");
        if (st != BSA_OK) return st;
      }
      st = hip_status(launch_gather(g, v, v_cache, GATHER_ROW, at(w.g_vr), nullptr, stream),
                      "gather V");
      if (st != BSA_OK) return st;
      stages.done(reuse ? "bwd_gather_v" : "bwd_gather_qkv");
      // longest-first dK/dV dispatch unless this thread asked for the fixed order
      int32_t* order = t_dkdv_order ? reinterpret_cast<int32_t*>(base + w.order) : nullptr;
      // the real-time walk phase (locality experiment), in ticks of the 100 MHz clock
      const int walk_ticks = t_walk_phase_us * 100;
      st = hip_status(launch_bwd_dkdv_mfma(g, k_rows, at(w.g_vr), q_rows, at(w.g_dr), ld_c,
                                           off, list, order, softmax_scale, walk_ticks,
                                           t_dkdv_split != 0, dk, dv, dk_cache, dv_cache, stream),
                      "dK/dV launch");
      if (st != BSA_OK) return st;
      stages.done("bwd_dkdv_mfma");
      // software-pipelined dQ where it is faster, unless this thread asked for the plain loop
      // (same bits)
      const bool pipelined = t_dq_pipeline != 0;
      st = hip_status(launch_bwd_dq_mfma(g, q_rows, at(w.g_dr), k_rows, at(w.g_vr), ld_c, idx,
                                         k_sel, softmax_scale, dq, pipelined, walk_ticks, stream),
                      "dQ launch");
      stages.done("bwd_dq_mfma");
    } else {
      st = hip_status(launch_bwd_dkdv_simt(g, bf16, q, k, v, d_o, lse_c, delta_c, off, list,
                                           softmax_scale, dk, dv, stream), "dK/dV launch");
      if (st != BSA_OK) return st;
      stages.done("bwd_dkdv_simt");
      st = hip_status(launch_bwd_dq_simt(g, bf16, q, k, v, d_o, lse_c, delta_c, idx, k_sel,
                                         softmax_scale, dq, stream), "dQ launch");
      stages.done("bwd_dq_simt");
    }
    return st;
  });
}

bsa_status_t bsa_validate_idx(const bsa_problem_t* p, const int32_t* idx, int32_t k_sel,
                              int32_t* bad_rows, hipStream_t stream) {
  return guarded([&]() -> bsa_status_t {
    Geom g;
    bsa_status_t st = check_problem(p, &g);
    if (st != BSA_OK) return st;
    if ((st = check_ksel(g, k_sel)) != BSA_OK) return st;
    if (!idx || !bad_rows) return fail(BSA_ERR_INVALID_ARG, "idx and bad_rows must be non-NULL");
    Stages stages(stream);
    st = hip_status(launch_validate_idx(g, idx, k_sel, bad_rows, stream), "validate launch");
    stages.done("validate_idx");
    return st;
  });
}

bsa_status_t bsa_set_tuning(bsa_tune_t key, int32_t value) {
  switch (key) {
    case BSA_TUNE_FWD_SPLITS:
      if (value != -1 && (value < 1 || value > kMaxFwdSplits))
        return fail(BSA_ERR_INVALID_ARG, "forward splits must be -1 (automatic) or 1..64");
      t_fwd_splits = value;
      return BSA_OK;
    case BSA_TUNE_DKDV_ORDER:
      if (value != 0 && value != 1) return fail(BSA_ERR_INVALID_ARG, "dK/dV order must be 0 or 1");
      t_dkdv_order = value;
      return BSA_OK;
    case BSA_TUNE_DQ_PIPELINE:
      if (value != 0 && value != 1) return fail(BSA_ERR_INVALID_ARG, "dQ pipeline must be 0 or 1");
      t_dq_pipeline = value;
      return BSA_OK;
    case BSA_TUNE_WALK_PHASE:
      if (value < 0 || value > 1000000)
        return fail(BSA_ERR_INVALID_ARG, "walk phase period must be 0 (off) or 1..1000000 us");
      t_walk_phase_us = value;
      return BSA_OK;
    case BSA_TUNE_DKDV_SPLIT:
      if (value != 0 && value != 1) return fail(BSA_ERR_INVALID_ARG, "dK/dV split must be 0 or 1");
      t_dkdv_split = value;
      return BSA_OK;
  }
  return fail(BSA_ERR_INVALID_ARG, "unknown tuning key");
}

int32_t bsa_get_tuning(bsa_tune_t key) {
  switch (key) {
    case BSA_TUNE_FWD_SPLITS: return t_fwd_splits;
    case BSA_TUNE_DKDV_ORDER: return t_dkdv_order;
    case BSA_TUNE_DQ_PIPELINE: return t_dq_pipeline;
    case BSA_TUNE_WALK_PHASE: return t_walk_phase_us;
    case BSA_TUNE_DKDV_SPLIT: return t_dkdv_split;
  }
  return INT32_MIN;
}

bsa_status_t bsa_probe_mfma_shape(const void* operands, size_t operand_bytes, int32_t shape,
                                  int32_t chains, int32_t waves, int32_t iters, float* sink,
                                  size_t sink_bytes, hipStream_t stream) {
  return guarded([&]() -> bsa_status_t {
    if (!operands || !sink) return fail(BSA_ERR_INVALID_ARG, "operands and sink must be non-NULL");
    if (operand_bytes < 8192) return fail(BSA_ERR_INVALID_ARG, "operands must hold 8192 bytes");
    if (shape != 0 && shape != 1) return fail(BSA_ERR_INVALID_ARG, "shape must be 0 or 1");
    if (chains != 1 && chains != 2 && chains != 4 && chains != 8)
      return fail(BSA_ERR_INVALID_ARG, "chains must be 1, 2, 4 or 8");
    if (waves < 1 || waves > (1 << 22) || iters < 1)
      return fail(BSA_ERR_INVALID_ARG, "waves must be in 1..2^22 and iters >= 1");
    if (sink_bytes < (size_t)waves * 64 * sizeof(float))
      return fail(BSA_ERR_INVALID_ARG, "sink must hold 64 floats per wave");
    Stages stages(stream);
    const bsa_status_t st = hip_status(launch_mfma_probe(static_cast<const bf16_t*>(operands),
                                                         shape, chains, waves, iters, sink,
                                                         stream),
                                       "MFMA probe launch");
    stages.done("probe_mfma");
    return st;
  });
}

bsa_status_t bsa_probe_mfma(const void* operands, size_t operand_bytes, int32_t waves,
                            int32_t iters, float* sink, size_t sink_bytes, hipStream_t stream) {
  return bsa_probe_mfma_shape(operands, operand_bytes, 0, 4, waves, iters, sink, sink_bytes,
                              stream);
}

bsa_status_t bsa_probe_mfma_valu(const void* operands, size_t operand_bytes, int32_t mode,
                                 int32_t valu, int32_t op, int32_t acc, int32_t workgroups,
                                 int32_t iters, float* sink, size_t sink_bytes,
                                 hipStream_t stream) {
  return guarded([&]() -> bsa_status_t {
    if (!operands || !sink) return fail(BSA_ERR_INVALID_ARG, "operands and sink must be non-NULL");
    if (operand_bytes < 2048) return fail(BSA_ERR_INVALID_ARG, "operands must hold 2048 bytes");
    if (mode < 0 || mode > 3) return fail(BSA_ERR_INVALID_ARG, "mode must be 0, 1, 2 or 3");
    const bool ok = op == 0 ? (valu == 0 || valu == 2 || valu == 4 || valu == 8 || valu == 16)
                            : op == 1 && (valu == 1 || valu == 2 || valu == 4);
    if (!ok) return fail(BSA_ERR_INVALID_ARG, "valu must be 0, 2, 4, 8 or 16 (op 0), 1, 2 or 4 (op 1)");
    if (acc != 0 && acc != 1) return fail(BSA_ERR_INVALID_ARG, "acc must be 0 or 1");
    if (workgroups < 1 || workgroups > (1 << 20) || iters < 1)
      return fail(BSA_ERR_INVALID_ARG, "workgroups must be in 1..2^20 and iters >= 1");
    if (sink_bytes < (size_t)workgroups * 512 * sizeof(float))
      return fail(BSA_ERR_INVALID_ARG, "sink must hold 512 floats per workgroup");
    Stages stages(stream);
    const bsa_status_t st = hip_status(launch_coexec_probe(static_cast<const bf16_t*>(operands),
                                                           mode, valu, op, acc, workgroups,
                                                           iters, sink, stream),
                                       "MFMA/VALU probe launch");
    stages.done("probe_mfma_valu");
    return st;
  });
}

bsa_status_t bsa_probe_tile_read(const void* buf, size_t buf_bytes, int32_t tile_bytes,
                                 const int32_t* ids, size_t n_ids, int32_t waves,
                                 int32_t tiles_per_wave, uint32_t* sink, size_t sink_bytes,
                                 hipStream_t stream) {
  return guarded([&]() -> bsa_status_t {
    if (!buf || !ids || !sink) return fail(BSA_ERR_INVALID_ARG, "buf, ids and sink must be non-NULL");
    if (tile_bytes < 8192 || tile_bytes % 8192 || tile_bytes > (1 << 20))
      return fail(BSA_ERR_INVALID_ARG, "tile_bytes must be a multiple of 8192, at most 1 MiB");
    if (buf_bytes < (size_t)tile_bytes || buf_bytes > 0x7fffffffu)
      return fail(BSA_ERR_INVALID_ARG, "buf must hold one tile and at most 2^31-1 bytes");
    if (waves < 1 || waves > (1 << 22) || tiles_per_wave < 1)
      return fail(BSA_ERR_INVALID_ARG, "waves must be in 1..2^22 and tiles_per_wave >= 1");
    if (n_ids < (size_t)waves * (size_t)tiles_per_wave)
      return fail(BSA_ERR_INVALID_ARG, "ids must hold waves * tiles_per_wave entries");
    if (sink_bytes < (size_t)waves * 64 * sizeof(uint32_t))
      return fail(BSA_ERR_INVALID_ARG, "sink must hold 64 words per wave");
    Stages stages(stream);
    const bsa_status_t st = hip_status(
        launch_tile_read(static_cast<const bf16_t*>(buf), buf_bytes, tile_bytes, ids, waves,
                         tiles_per_wave, sink, stream),
        "tile read probe launch");
    stages.done("probe_tile_read");
    return st;
  });
}

int32_t bsa_num_selected(const bsa_problem_t* p, int32_t r) {
  Geom g;
  if (r < 0 || check_problem(p, &g) != BSA_OK) return -1;
  return g.nbc + 1 + (r < g.nbq - 1 ? r : g.nbq - 1);
}

size_t bsa_workspace_bytes(const bsa_problem_t* p, bsa_dtype_t dtype, int32_t k_sel,
                           int32_t bwd) {
  Geom g;
  if (check_problem(p, &g) != BSA_OK || check_dtype(dtype) != BSA_OK ||
      check_ksel(g, k_sel) != BSA_OK)
    return (size_t)-1;
  const bool mfma = use_mfma(g, dtype);
  return bwd ? bwd_layout(g, mfma, k_sel).total : fwd_ws(g, mfma, k_sel);
}

const char* bsa_status_string(bsa_status_t s) {
  switch (s) {
    case BSA_OK: return "BSA_OK";
    case BSA_ERR_INVALID_ARG: return "BSA_ERR_INVALID_ARG";
    case BSA_ERR_SHAPE: return "BSA_ERR_SHAPE";
    case BSA_ERR_UNSUPPORTED: return "BSA_ERR_UNSUPPORTED";
    case BSA_ERR_WORKSPACE: return "BSA_ERR_WORKSPACE";
    case BSA_ERR_HIP: return "BSA_ERR_HIP";
    case BSA_ERR_INTERNAL: return "BSA_ERR_INTERNAL";
  }
  return "BSA_ERR_UNKNOWN";
}

const char* bsa_last_error(void) { return t_err.c_str(); }

void bsa_set_stage_events(hipEvent_t* events, int32_t n) {
  t_events = events;
  t_nevents = events ? n : 0;
}

int32_t bsa_stage_count(void) { return t_nstages; }

const char* bsa_stage_name(int32_t s) {
  if (s < 0 || s >= t_nstages || s >= 16) return "";
  return t_stage_names[s];
}

bsa_status_t bsa_set_kernel_path(int32_t path) {
  if (path != 0 && path != 1) return fail(BSA_ERR_INVALID_ARG, "path must be 0 or 1");
  t_path = path;
  return BSA_OK;
}

}  // extern "C"
