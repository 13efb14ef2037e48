// fgemm_api.cpp — the C ABI: handle, argument checks, plan selection and cache,
// and the classical and Strassen/Winograd schedulers that enqueue the kernels.
//
// Run-time dispatch follows the FalconGEMM summary (euno.news), Methodology 5: the
// model is queried with the actual shape, the chosen kernel runs with no further
// input from the caller; a per-shape plan cache keeps the query cost far below the
// kernels' own time (Results: model overhead under half a percent).
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <mutex>
#include <new>
#include <unordered_map>

#include "internal.h"
#include "model.h"

using namespace fgemm;

namespace fgemm {

int tile_m_of(int tile) { return kTiles[tile].bm; }
int tile_n_of(int tile) { return kTiles[tile].bn; }
int waves_n_of(int tile) { return kTiles[tile].waves_n; }

hipError_t launch_gemm(const KernelKey& k, const GemmBatch& b, hipStream_t s) {
#define FG_SEL(DT, AK, BK) \
  if (k.dtype == DT && k.a_kcontig == AK && k.b_kcontig == BK) return launch_gemm_##DT##_##AK##BK(k, b, s);
  FG_SEL(0, 0, 0) FG_SEL(0, 0, 1) FG_SEL(0, 1, 0) FG_SEL(0, 1, 1)
  FG_SEL(1, 0, 0) FG_SEL(1, 0, 1) FG_SEL(1, 1, 0) FG_SEL(1, 1, 1)
#undef FG_SEL
  return hipErrorInvalidValue;
}

}  // namespace fgemm

namespace {

struct PlanKey {
  int64_t M, N, K;
  int ta, tb, dtype, flags, vec;
  bool operator==(const PlanKey& o) const {
    return M == o.M && N == o.N && K == o.K && ta == o.ta && tb == o.tb && dtype == o.dtype &&
           flags == o.flags && vec == o.vec;
  }
};
struct PlanKeyHash {
  size_t operator()(const PlanKey& k) const {
    uint64_t h = 1469598103934665603ull;
    auto mix = [&](uint64_t v) { h = (h ^ v) * 1099511628211ull; };
    mix(k.M); mix(k.N); mix(k.K);
    mix(((uint64_t)k.ta << 1 | k.tb) << 8 | (uint64_t)k.dtype << 4 | (uint64_t)k.vec);
    mix(k.flags);
    return (size_t)h;
  }
};

}  // namespace

// A fixed, direct-mapped plan table for fgemm_gemm_noalloc (no allocation on a miss:
// the entry is overwritten).
struct NoAllocSlot {
  PlanKey key;
  fgemm_plan_t plan;
  bool valid;
};
constexpr int kNoAllocSlots = 64;

struct fgemm_handle_s {
  int device = 0;
  int cus = 0;  // compute units of the device (the model's count may be set otherwise)
  fgemm_model_t model{};
  std::unordered_map<PlanKey, fgemm_plan_t, PlanKeyHash> plans;
  NoAllocSlot noalloc_plans[kNoAllocSlots] = {};
  void* user_ws = nullptr;
  size_t user_ws_bytes = 0;
  void* own_ws = nullptr;
  size_t own_ws_bytes = 0;
  int pools = 0;  // the device supports stream-ordered allocation
  // Second stream of the overlapped Winograd schedule (the operand sums run there
  // beside the products that need none), with its fork and join events; null when
  // they could not be created (the schedule then runs on the caller's stream).
  hipStream_t aux = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

namespace {

fgemm_status_t hip_status(hipError_t e) { return e == hipSuccess ? FGEMM_OK : FGEMM_ERR_HIP; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

uint32_t epi_flags(const fgemm_epilogue_t* e) { return e ? e->flags : 0u; }

// Epilogues on gate/up column pairs of a 2N-wide op(B).
constexpr uint32_t kSwiGLUFlags = FGEMM_EPI_RMS_SWIGLU | FGEMM_EPI_SWIGLU_BWD;

// Relative error the row statistics (ROWSUMSQ) of an automatic plan are held to.
// In the CODA split (tilnote.io PingPong GEMM note, CODA section) these sums set the
// next GEMM's RMS row scale.
constexpr double kStatsRelErr = 1e-3;

// Whether the 16-byte fast path applies.
int vec_ok(fgemm_op_t ta, fgemm_op_t tb, int64_t N, const void* A, int64_t lda, const void* B,
           int64_t ldb, const void* C, int64_t ldc, const fgemm_epilogue_t* e) {
  (void)ta; (void)tb;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return 0;
  if (lda % 8 || ldb % 8 || ldc % 8) return 0;
  if ((epi_flags(e) & kSwiGLUFlags) && N % 8) return 0;
  return 1;
}

int tile_id(int tm, int tn);

fgemm_status_t check_plan_shape(const fgemm_plan_t& p, int64_t M, int64_t N, int64_t K, int vec,
                                uint32_t flags) {
  if (p.path == FGEMM_PATH_CLASSICAL) {
    if (p.split_k <= 1) return FGEMM_OK;
    // split K: fp32 slices and a finalize pass; epilogue NONE or BIAS, aligned, and
    // a whole number of pipeline phases per slice
    const int t = tile_id(p.tile_m, p.tile_n);
    if (t < 0) return FGEMM_ERR_INVALID_VALUE;
    const int64_t ktiles = ceil_div(K, kTiles[t].bk);
    if (!vec || (flags & ~(uint32_t)FGEMM_EPI_BIAS) || K == 0 || ktiles % p.split_k ||
        p.split_k > 64)
      return FGEMM_ERR_NOT_SUPPORTED;
    return FGEMM_OK;
  }
  if (p.path != FGEMM_PATH_STRASSEN) return FGEMM_ERR_INVALID_VALUE;
  if (p.depth < 1 || p.depth > 2) return FGEMM_ERR_INVALID_VALUE;
  if (const BlockScheme* s = block_scheme(p.variant)) {
    // table-driven schemes: one level, 16-element blocks, epilogues NONE and BIAS
    if (p.depth != 1) return FGEMM_ERR_INVALID_VALUE;
    if (flags & ~(uint32_t)FGEMM_EPI_BIAS) return FGEMM_ERR_NOT_SUPPORTED;
    if (M % (16 * s->mb) || K % (16 * s->kb) || N % (16 * s->nb) || M == 0 || N == 0 || K == 0)
      return FGEMM_ERR_NOT_SUPPORTED;
    if (!vec) return FGEMM_ERR_NOT_SUPPORTED;
    return FGEMM_OK;
  }
  if (p.variant != FGEMM_VARIANT_S69 && p.variant != FGEMM_VARIANT_WINOGRAD)
    return FGEMM_ERR_INVALID_VALUE;
  // the recursion runs on op(B)'s Nb columns (2N with SwiGLU: its top split is the
  // gate/up boundary); every epilogue is applied in the top-level post-add
  const int64_t q = 8ll << p.depth;
  const int64_t Nb = (flags & FGEMM_EPI_RMS_SWIGLU) ? 2 * N : N;
  if (flags & (FGEMM_EPI_SWIGLU_BWD | FGEMM_EPI_RMS_BWD))
    return FGEMM_ERR_NOT_SUPPORTED;  // classical path only
  if (M % q || Nb % q || K % q || M == 0 || N == 0 || K == 0) return FGEMM_ERR_NOT_SUPPORTED;
  if (!vec) return FGEMM_ERR_NOT_SUPPORTED;
  return FGEMM_OK;
}

// Row-sum partials of the Strassen path's top-level post-add (ROWSUMSQ only).
size_t strassen_stats_bytes(int64_t M, int64_t Nb, uint32_t flags) {
  if (!(flags & FGEMM_EPI_ROWSUMSQ)) return 0;
  return align256((size_t)postadd_ss_parts(Nb / 2) * (size_t)M * 4);
}

// Core of fgemm_select: classical tile choice, then Strassen candidates under guards.
fgemm_status_t select_plan(const fgemm_model_t& md, int64_t M, int64_t N, int64_t K,
                           fgemm_dtype_t dtype, uint32_t flags, int beta_hint, int vec,
                           size_t ws_limit, fgemm_plan_t* out, bool classical_only = false) {
  fgemm_plan_t p{};
  const int swiglu = (flags & kSwiGLUFlags) != 0;
  double tc;
  int tile = best_tile(md, M, N, K, swiglu, 1, 2.0, 2.0, beta_hint, &tc);
  p.path = FGEMM_PATH_CLASSICAL;
  p.depth = 0;
  p.variant = FGEMM_VARIANT_WINOGRAD;
  p.tile_m = tile_m_of(tile);
  p.tile_n = tile_n_of(tile);
  p.tile_k = 64;
  p.split_k = 1;
  p.workspace_bytes = 0;
  if (flags & FGEMM_EPI_ROWSUMSQ)
    p.workspace_bytes = (size_t)ceil_div(N, tile_n_of(tile)) * waves_n_of(tile) * (size_t)M * 4;
  // skinny shapes leave CUs idle: split K over extra workgroups when the model
  // says the finalize pass costs less than the idle bandwidth (tile and split
  // count are chosen together)
  if (!(flags & ~(uint32_t)FGEMM_EPI_BIAS) && vec && K > 0) {
    for (int i = 0; i < kNumTiles; ++i) {
      const TileInfo& ti = kTiles[i];
      if (ti.one_row && M > ti.bm) continue;
      const int64_t tiles = ceil_div(M, ti.bm) * ceil_div(N, ti.bn);
      const int64_t ktiles = ceil_div(K, ti.bk);
      for (int sk = 2; sk <= 16 && tiles < md.compute_units; sk *= 2) {
        if (ktiles % sk || ktiles / sk < 4) continue;
        const size_t ws = (size_t)sk * (size_t)M * (size_t)N * 4;
        if ((double)ws > md.max_workspace_bytes || ws > ws_limit) continue;
        const double t = splitk_time_us(md, ti, M, N, K, sk, beta_hint);
        if (t < tc) {
          tc = t;
          tile = ti.tile;
          p.tile_m = ti.bm;
          p.tile_n = ti.bn;
          p.split_k = sk;
          p.workspace_bytes = ws;
        }
      }
    }
  }
  {
    // fp16 MFMA work runs at a lower clock (the launch cost does not scale)
    const double launch = (p.split_k > 1 ? 2 : 1) * md.launch_us;
    tc = launch + (tc - launch) / classical_dtype_rate(dtype);
  }
  p.t_pred_us = tc;
  p.t_classical_pred_us = tc;
  p.pred_rel_err = predicted_rel_err(dtype, 0, 0);
  for (int depth = 1; depth <= (classical_only ? 0 : 2); ++depth) {
    for (int variant = FGEMM_VARIANT_S69; variant <= FGEMM_VARIANT_R223; ++variant) {
      const BlockScheme* bs = block_scheme(variant);
      if (bs && depth != 1) continue;
      fgemm_plan_t c{};
      c.path = FGEMM_PATH_STRASSEN;
      c.depth = depth;
      c.variant = variant;
      if (check_plan_shape(c, M, N, K, vec, flags) != FGEMM_OK) continue;
      // accuracy guard: the calibrated error of this variant and depth within budget
      const double err = predicted_rel_err(dtype, variant, depth);
      if (err > md.max_rel_err) continue;
      // statistics guard: a row's sum of squares of the written output moves by up
      // to about twice the output's relative error (for y' = y + d, |sum y'^2 -
      // sum y^2| / sum y^2 <= 2e + e^2 with e = ||d|| / ||y||); row statistics are
      // held to kStatsRelErr, so they stay classical unless 2e fits in it
      if ((flags & FGEMM_EPI_ROWSUMSQ) && 2.0 * err > kStatsRelErr) continue;
      // sub-problems below 512 never pay for their additions; keep them classical
      if ((M >> depth) < 512 || ((swiglu ? 2 * N : N) >> depth) < 512 || (K >> depth) < 512)
        continue;
      if (bs && (M / bs->mb < 512 || N / bs->nb < 512 || K / bs->kb < 512)) continue;
      const int64_t Nb = swiglu ? 2 * N : N;
      const size_t ws = strassen_workspace(M, Nb, K, depth, variant) +
                        strassen_stats_bytes(M, Nb, flags);
      if ((double)ws > md.max_workspace_bytes || ws > ws_limit) continue;
      int sub_tile = 0;
      const double t = strassen_time_us(md, M, Nb, K, depth, variant, beta_hint, &sub_tile);
      if (t < p.t_pred_us) {
        c.tile_m = tile_m_of(sub_tile);
        c.tile_n = tile_n_of(sub_tile);
        c.tile_k = 64;
        c.split_k = 1;
        c.workspace_bytes = ws;
        c.t_pred_us = t;
        c.t_classical_pred_us = tc;
        c.pred_rel_err = err;
        p = c;
      }
    }
  }
  *out = p;
  return FGEMM_OK;
}

int tile_id(int tm, int tn) {
  for (int i = 0; i < kNumTiles; ++i)
    if (kTiles[i].bm == tm && kTiles[i].bn == tn) return kTiles[i].tile;
  return -1;
}

// Where a call's scratch memory comes from: the handle's workspace (the caller's,
// or one the handle allocates), or a fixed device array that is never allocated.
struct WsSource {
  void* fixed = nullptr;
  size_t fixed_bytes = 0;
};

fgemm_status_t ensure_workspace(fgemm_handle_t h, const WsSource& src, size_t bytes,
                                hipStream_t stream, void** ws) {
  *ws = nullptr;
  if (bytes == 0) return FGEMM_OK;
  if (src.fixed) {
    if (bytes > src.fixed_bytes) return FGEMM_ERR_WORKSPACE;
    *ws = src.fixed;
    return FGEMM_OK;
  }
  if (h->user_ws) {
    if (h->user_ws_bytes < bytes) return FGEMM_ERR_WORKSPACE;
    *ws = h->user_ws;
    return FGEMM_OK;
  }
  if (h->own_ws_bytes < bytes) {
    // Regrowth in stream order where the device has memory pools: the old buffer is
    // released after the work already enqueued on this stream (calls that share the
    // workspace run on one stream, or the caller orders them), and the new one is
    // usable from there on; no other stream of the device waits.  Without pools,
    // the device drains first.
    if (h->own_ws) {
      hipError_t e;
      if (h->pools) {
        e = hipFreeAsync(h->own_ws, stream);
      } else {
        e = hipDeviceSynchronize();
        if (e == hipSuccess) e = hipFree(h->own_ws);
      }
      if (e != hipSuccess) return FGEMM_ERR_HIP;
      h->own_ws = nullptr;
      h->own_ws_bytes = 0;
    }
    const hipError_t e = h->pools ? hipMallocAsync(&h->own_ws, bytes, stream)
                                  : hipMalloc(&h->own_ws, bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // leave no error behind for the caller's next check
      h->own_ws = nullptr;
      return FGEMM_ERR_ALLOC;
    }
    h->own_ws_bytes = bytes;
  }
  *ws = h->own_ws;
  return FGEMM_OK;
}

struct Call {
  fgemm_op_t ta, tb;
  int64_t M, N, K;
  float alpha;
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  float beta;
  void* C; int64_t ldc;
  fgemm_dtype_t dtype;
  const fgemm_epilogue_t* epi;
  hipStream_t stream;
};

// Activation or rotary-embedding parameters of an epilogue, as the kernels take them.
void set_transform(const fgemm_epilogue_t* e, int* act, int* rope_hd, const int32_t** rope_pos,
                   int64_t* rope_off, double* rope_log2_base) {
  const uint32_t flags = epi_flags(e);
  *act = (flags & FGEMM_EPI_ACT) ? e->act : 0;
  *rope_hd = (flags & FGEMM_EPI_ROPE) ? (int)e->rope_head_dim : 0;
  *rope_pos = (flags & FGEMM_EPI_ROPE) ? e->rope_positions : nullptr;
  *rope_off = (flags & FGEMM_EPI_ROPE) ? e->rope_offset : 0;
  *rope_log2_base = (flags & FGEMM_EPI_ROPE) ? log2((double)e->rope_theta) : 0.0;
}

fgemm_status_t run_classical(fgemm_handle_t h, const fgemm_plan_t& plan, const Call& c, int vec,
                             const WsSource& wsrc) {
  const uint32_t flags = epi_flags(c.epi);
  int tile = tile_id(plan.tile_m, plan.tile_n);
  if (tile < 0) return FGEMM_ERR_INVALID_VALUE;
  const int swiglu = (flags & kSwiGLUFlags) != 0;
  const int swiglu_bwd = (flags & FGEMM_EPI_SWIGLU_BWD) != 0;
  if (swiglu && !kTiles[tile].swiglu) return FGEMM_ERR_NOT_SUPPORTED;
  GemmBatch b{};
  b.count = 1;
  b.cus = h->cus;
  GemmProblem& p = b.p[0];
  p.A = c.A; p.B = c.B; p.C = c.C; p.Cin = c.C;
  p.lda = c.lda; p.ldb = c.ldb; p.ldc = c.ldc;
  p.M = (int)c.M; p.N = (int)c.N; p.K = (int)c.K;
  p.alpha = c.alpha; p.beta = c.beta;
  p.flags = (c.beta != 0.f ? kFlagBeta : 0u);
  if (flags & FGEMM_EPI_BIAS) { p.flags |= kFlagBias; p.bias = c.epi->bias; }
  int parts = 0;
  if (flags & FGEMM_EPI_ROWSUMSQ) {
    p.flags |= kFlagRowSumSq;
    parts = (int)ceil_div(c.N, tile_n_of(tile)) * waves_n_of(tile);
    void* ws;
    fgemm_status_t st = ensure_workspace(h, wsrc, (size_t)parts * (size_t)c.M * 4, c.stream, &ws);
    if (st != FGEMM_OK) return st;
    p.ss_partial = static_cast<float*>(ws);
  }
  const int rms_bwd = (flags & FGEMM_EPI_RMS_BWD) != 0;
  if (swiglu_bwd) {
    p.dout = c.epi->swiglu_dout;
    p.ldd = c.epi->swiglu_ldd;
    if (c.epi->rms_grad) {
      // per-wave partials of the row-scale gradient, one per (output tile column, wave column)
      p.rms_grad_out = 1;
      parts = (int)ceil_div(c.N, tile_n_of(tile) / 2) * waves_n_of(tile);
      void* ws;
      fgemm_status_t st = ensure_workspace(h, wsrc, (size_t)parts * (size_t)c.M * 4, c.stream, &ws);
      if (st != FGEMM_OK) return st;
      p.ss_partial = static_cast<float*>(ws);
    }
  }
  if (rms_bwd) {
    p.rms_ss = c.epi->rms_rowsumsq;
    p.rms_inv_n = 1.0f / (float)c.epi->rms_n;
    p.rms_eps = c.epi->rms_eps;
    p.rms_grad = c.epi->rms_grad;
    p.rms_x = c.epi->rms_x;
    p.ldx = c.epi->rms_ldx;
  }
  if (swiglu) {
    p.rms_ss = c.epi->rms_rowsumsq;
    p.rms_inv_n = 1.0f / (float)c.epi->rms_n;
    p.rms_eps = c.epi->rms_eps;
  }
  const bool xform = (flags & (FGEMM_EPI_ACT | FGEMM_EPI_ROPE)) != 0;
  if (xform) set_transform(c.epi, &p.act, &p.rope_hd, &p.rope_pos, &p.rope_off, &p.rope_log2_base);
  KernelKey k{};
  k.tile = tile;
  k.a_kcontig = c.ta == FGEMM_OP_N;
  k.b_kcontig = c.tb == FGEMM_OP_T;
  k.dtype = c.dtype == FGEMM_BF16 ? kBF16 : kF16;
  k.epi = rms_bwd                       ? kEpiRmsBwd
          : swiglu_bwd                  ? kEpiSwiGLUBwd
          : swiglu                      ? kEpiSwiGLU
          : (flags & FGEMM_EPI_ACT)     ? kEpiAct
          : (flags & FGEMM_EPI_ROPE)    ? kEpiRope
                                        : kEpiStore16;
  k.vec = vec;
  if (plan.split_k > 1) {
    // fp32 K slices into the workspace, then the epilogue in the finalize pass
    void* ws;
    fgemm_status_t st =
        ensure_workspace(h, wsrc, (size_t)plan.split_k * (size_t)c.M * (size_t)c.N * 4, c.stream,
                         &ws);
    if (st != FGEMM_OK) return st;
    p.C = ws;
    p.ldc = c.N;
    b.k_splits = plan.split_k;
    k.epi = kEpiStore32;
    hipError_t e = launch_gemm(k, b, c.stream);
    if (e != hipSuccess) return FGEMM_ERR_HIP;
    e = launch_splitk_finalize(static_cast<const float*>(ws), plan.split_k, c.M, c.N, c.alpha,
                               c.beta, c.C, c.ldc,
                               (flags & FGEMM_EPI_BIAS) ? c.epi->bias : nullptr,
                               k.dtype, c.stream);
    return hip_status(e);
  }
  hipError_t e = launch_gemm(k, b, c.stream);
  if (e != hipSuccess) return FGEMM_ERR_HIP;
  if (parts) {
    e = launch_rowsumsq_reduce(p.ss_partial, parts, (int)c.M,
                               swiglu_bwd ? c.epi->rms_grad : c.epi->rowsumsq, c.stream);
    if (e != hipSuccess) return FGEMM_ERR_HIP;
  }
  return FGEMM_OK;
}

// ------------------------------------------------------------------ Strassen
struct StrassenRun {
  const Call* c;
  int cus;
  int depth, variant, sub_tile;
  int in_dtype;
  // Winograd depth 1: P1 = A11 B11 and P2 = A12 B21 read the input blocks
  // (blocks of `L0`, `R0`) on the caller's stream while the sums run on `aux`
  bool overlap;
  hipStream_t aux;
  hipEvent_t join;
  float* scale_a; float* scale_b;
  // per level l (1-based): the seven left and right product operands (fp16) and
  // the seven products (fp32)
  void* S[3][7];
  void* T[3][7];
  float* P[3][7];
  float* ss_partial;  // ROWSUMSQ: the top-level post-add's row-sum partials
};

BlockedOperand temp_op(void* p, int64_t rows, int64_t cols, int trans) {
  BlockedOperand r;
  r.ptr = p;
  r.ld = trans ? rows : cols;  // stored (cols x rows) when transposed
  r.trans = trans;
  r.dtype = kF16;
  r.scaled = 1;
  return r;
}

// One level of the recursion on the left operand L (Ml x Kl) and the right
// operand R (Kl x Nl): pre-adds, seven sub-products (batched, or recursed into the
// next level), post-add into `out32` (inner levels) or the caller's C (top level).
// Storage address of logical block (bi, bj) of a rows x cols operand split 2 x 2.
const void* block_of(const BlockedOperand& x, int64_t rows, int64_t cols, int bi, int bj) {
  const uint16_t* base = static_cast<const uint16_t*>(x.ptr);
  const int64_t hr = rows / 2, hc = cols / 2;
  return x.trans ? base + (int64_t)bj * hc * x.ld + bi * hr : base + (int64_t)bi * hr * x.ld + bj * hc;
}

// The batched sub-products [first, first + count) of one level: fp16 temporaries, or
// (overlap, products 0 and 1) the input blocks, fp32 results.
hipError_t launch_products(const StrassenRun& run, int level, const BlockedOperand& L,
                           const BlockedOperand& R, int64_t Ml, int64_t Kl, int64_t Nl,
                           int first, int count, bool inputs, int cus) {
  const int64_t m = Ml / 2, k = Kl / 2, n = Nl / 2;
  GemmBatch b{};
  b.count = count;
  b.cus = cus;
  for (int j = 0; j < count; ++j) {
    const int i = first + j;
    GemmProblem& p = b.p[j];
    if (inputs) {
      // Winograd P1 = A11 B11, P2 = A12 B21
      p.A = block_of(L, Ml, Kl, 0, i);
      p.B = block_of(R, Kl, Nl, i, 0);
      p.lda = L.ld;
      p.ldb = R.ld;
    } else {
      BlockedOperand lo = temp_op(run.S[level][i], m, k, L.trans);
      BlockedOperand ro = temp_op(run.T[level][i], k, n, R.trans);
      p.A = lo.ptr; p.lda = lo.ld;
      p.B = ro.ptr; p.ldb = ro.ld;
    }
    p.C = run.P[level][i]; p.Cin = nullptr; p.ldc = n;
    p.M = (int)m; p.N = (int)n; p.K = (int)k;
    p.alpha = 1.f; p.beta = 0.f;
  }
  KernelKey key{};
  key.tile = run.sub_tile;
  key.a_kcontig = !L.trans;
  key.b_kcontig = R.trans;
  key.dtype = inputs ? L.dtype : kF16;
  key.epi = kEpiStore32;
  key.vec = 1;
  if (inputs) {
    // the blocks keep the parent's leading dimension: whole 16-byte chunks only
    for (int j = 0; j < count; ++j)
      if (!aligned16(b.p[j].A) || !aligned16(b.p[j].B)) key.vec = 0;
    if (L.ld % 8 || R.ld % 8) key.vec = 0;
  }
  return launch_gemm(key, b, run.c->stream);
}

fgemm_status_t strassen_level(const StrassenRun& run, int level, const BlockedOperand& L,
                              const BlockedOperand& R, int64_t Ml, int64_t Kl, int64_t Nl,
                              float* out32, int64_t ld32) {
  const Call& c = *run.c;
  const int64_t m = Ml / 2, k = Kl / 2, n = Nl / 2;
  hipError_t e;
  if (run.overlap) {
    // the sums were issued on the second stream before this level: P1 and P2 take
    // the input blocks on 7/8 of the CUs meanwhile (the sums have the rest), then
    // the other five follow once the sums are done
    e = launch_products(run, level, L, R, Ml, Kl, Nl, 0, 2, true, run.cus - run.cus / 8);
    if (e == hipSuccess) e = hipStreamWaitEvent(c.stream, run.join, 0);
    if (e == hipSuccess) e = launch_products(run, level, L, R, Ml, Kl, Nl, 2, 5, false, run.cus);
    if (e != hipSuccess) return FGEMM_ERR_HIP;
  } else if (level == run.depth) {
    e = launch_preadd(L, Ml, Kl, run.variant, 0, run.scale_a, run.S[level], c.stream);
    if (e == hipSuccess) e = launch_preadd(R, Kl, Nl, run.variant, 1, run.scale_b, run.T[level], c.stream);
    if (e == hipSuccess) e = launch_products(run, level, L, R, Ml, Kl, Nl, 0, 7, false, run.cus);
    if (e != hipSuccess) return FGEMM_ERR_HIP;
  } else {
    e = launch_preadd(L, Ml, Kl, run.variant, 0, run.scale_a, run.S[level], c.stream);
    if (e == hipSuccess) e = launch_preadd(R, Kl, Nl, run.variant, 1, run.scale_b, run.T[level], c.stream);
    if (e != hipSuccess) return FGEMM_ERR_HIP;
    for (int i = 0; i < 7; ++i) {
      fgemm_status_t st = strassen_level(run, level + 1, temp_op(run.S[level][i], m, k, L.trans),
                                         temp_op(run.T[level][i], k, n, R.trans), m, k, n,
                                         run.P[level][i], n);
      if (st != FGEMM_OK) return st;
    }
  }
  PostAddArgs pa{};
  for (int i = 0; i < 7; ++i) pa.P[i] = run.P[level][i];
  pa.m = m;
  pa.n = n;
  pa.variant = run.variant;
  if (level > 1) {
    pa.out32 = out32;
    pa.ld32 = ld32;
  } else {
    pa.C = c.C;
    pa.ldc = c.ldc;
    pa.dtype = run.in_dtype;
    pa.alpha = c.alpha;
    pa.beta = c.beta;
    const uint32_t flags = epi_flags(c.epi);
    pa.bias = (flags & FGEMM_EPI_BIAS) ? c.epi->bias : nullptr;
    pa.scale_a = run.scale_a;
    pa.scale_b = run.scale_b;
    pa.unscaled = run.overlap ? 3 : 0;  // P1, P2 of the input blocks
    if (flags & FGEMM_EPI_ROWSUMSQ) {
      pa.rowsumsq = c.epi->rowsumsq;
      pa.ss_partial = run.ss_partial;
    }
    if (flags & (FGEMM_EPI_ACT | FGEMM_EPI_ROPE))
      set_transform(c.epi, &pa.act, &pa.rope_hd, &pa.rope_pos, &pa.rope_off, &pa.rope_log2_base);
    if (flags & FGEMM_EPI_RMS_SWIGLU) {
      pa.swiglu = 1;
      pa.rms_ss = c.epi->rms_rowsumsq;
      pa.rms_inv_n = 1.0f / (float)c.epi->rms_n;
      pa.rms_eps = c.epi->rms_eps;
    }
  }
  e = launch_postadd(pa, c.stream);
  return hip_status(e);
}

// A table-driven block scheme at depth 1: max|x| and the fp16 scales, one pre-add
// pass a side writing the R product operands, the products in batches of at most
// seven, one post-add pass writing C with alpha, beta*C and bias.
fgemm_status_t run_scheme(fgemm_handle_t h, const fgemm_plan_t& plan, const Call& c,
                          const BlockScheme& s) {
  const int64_t m = c.M / s.mb, k = c.K / s.kb, n = c.N / s.nb;
  // the post-add reads the bias four columns (8 bytes) at a time
  const void* bias = (epi_flags(c.epi) & FGEMM_EPI_BIAS) ? c.epi->bias : nullptr;
  if (bias && (reinterpret_cast<uintptr_t>(bias) & 7)) return FGEMM_ERR_NOT_SUPPORTED;
  const size_t need = strassen_workspace(c.M, c.N, c.K, 1, plan.variant);
  void* ws;
  fgemm_status_t st = ensure_workspace(h, WsSource{}, need, c.stream, &ws);
  if (st != FGEMM_OK) return st;
  const int in_dtype = c.dtype == FGEMM_BF16 ? kBF16 : kF16;
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* scale_a = reinterpret_cast<float*>(base + 64);
  float* scale_b = reinterpret_cast<float*>(base + 128);
  float* part_a = reinterpret_cast<float*>(base + 256);
  float* part_b = part_a + kMaxPartials;
  void* S[kLinMaxProducts];
  void* T[kLinMaxProducts];
  const float* P[kLinMaxProducts];
  size_t off = kScaleHeaderBytes;
  for (int r = 0; r < s.R; ++r) { S[r] = base + off; off += align256((size_t)(m * k * 2)); }
  for (int r = 0; r < s.R; ++r) { T[r] = base + off; off += align256((size_t)(k * n * 2)); }
  for (int r = 0; r < s.R; ++r) {
    P[r] = reinterpret_cast<float*>(base + off);
    off += align256((size_t)(m * n * 4));
  }
  const bool ta = c.ta == FGEMM_OP_T, tb = c.tb == FGEMM_OP_T;
  // power-of-two scales keeping every fp16 sum in range (sums of at most four blocks)
  int na = 0, nb = 0;
  hipError_t e = launch_maxabs(c.A, c.lda, ta ? c.K : c.M, ta ? c.M : c.K, in_dtype, part_a, &na,
                               c.stream);
  if (e == hipSuccess)
    e = launch_maxabs(c.B, c.ldb, tb ? c.N : c.K, tb ? c.K : c.N, in_dtype, part_b, &nb, c.stream);
  if (e == hipSuccess) e = launch_scale_from_max(part_a, na, 8192.f, scale_a, c.stream);
  if (e == hipSuccess) e = launch_scale_from_max(part_b, nb, 8192.f, scale_b, c.stream);
  BlockedOperand L{c.A, c.lda, ta, in_dtype, 0};
  BlockedOperand R{c.B, c.ldb, tb, in_dtype, 0};
  if (e == hipSuccess)
    e = launch_lin_pre(L, c.M, c.K, s.mb, s.kb, s.R, s.U, scale_a, S, c.stream);
  if (e == hipSuccess)
    e = launch_lin_pre(R, c.K, c.N, s.kb, s.nb, s.R, s.V, scale_b, T, c.stream);
  int sub_tile = tile_id(plan.tile_m, plan.tile_n);
  if (sub_tile != 0 && sub_tile != 1) sub_tile = 0;
  for (int r0 = 0; e == hipSuccess && r0 < s.R; r0 += 7) {
    GemmBatch b{};
    b.count = s.R - r0 < 7 ? s.R - r0 : 7;
    b.cus = h->cus;
    for (int j = 0; j < b.count; ++j) {
      BlockedOperand lo = temp_op(S[r0 + j], m, k, ta);
      BlockedOperand ro = temp_op(T[r0 + j], k, n, tb);
      GemmProblem& p = b.p[j];
      p.A = lo.ptr; p.lda = lo.ld;
      p.B = ro.ptr; p.ldb = ro.ld;
      p.C = const_cast<float*>(P[r0 + j]); p.Cin = nullptr; p.ldc = n;
      p.M = (int)m; p.N = (int)n; p.K = (int)k;
      p.alpha = 1.f; p.beta = 0.f;
    }
    KernelKey key{};
    key.tile = sub_tile;
    key.a_kcontig = !ta;
    key.b_kcontig = tb;
    key.dtype = kF16;
    key.epi = kEpiStore32;
    key.vec = 1;
    e = launch_gemm(key, b, c.stream);
  }
  if (e == hipSuccess) {
    LinPostArgs pa{};
    for (int r = 0; r < s.R; ++r) pa.P[r] = P[r];
    pa.np = s.R;
    pa.m = m;
    pa.n = n;
    pa.mbc = s.mb;
    pa.nbc = s.nb;
    pa.coef = s.W;
    pa.C = c.C;
    pa.ldc = c.ldc;
    pa.dtype = in_dtype;
    pa.alpha = c.alpha;
    pa.beta = c.beta;
    pa.bias = bias;
    pa.scale_a = scale_a;
    pa.scale_b = scale_b;
    e = launch_lin_post(pa, c.stream);
  }
  return hip_status(e);
}

fgemm_status_t run_strassen(fgemm_handle_t h, const fgemm_plan_t& plan, const Call& c) {
  if (const BlockScheme* bs = block_scheme(plan.variant)) return run_scheme(h, plan, c, *bs);
  const uint32_t flags = epi_flags(c.epi);
  const int64_t Nb = (flags & FGEMM_EPI_RMS_SWIGLU) ? 2 * c.N : c.N;  // columns of op(B)
  const size_t body = strassen_workspace(c.M, Nb, c.K, plan.depth, plan.variant);
  const size_t need = body + strassen_stats_bytes(c.M, Nb, flags);
  void* ws;
  fgemm_status_t st = ensure_workspace(h, WsSource{}, need, c.stream, &ws);
  if (st != FGEMM_OK) return st;
  StrassenRun run{};
  run.c = &c;
  run.cus = h->cus;
  run.depth = plan.depth;
  run.variant = plan.variant;
  run.sub_tile = tile_id(plan.tile_m, plan.tile_n);
  if (run.sub_tile != 0 && run.sub_tile != 1) run.sub_tile = 0;
  run.in_dtype = c.dtype == FGEMM_BF16 ? kBF16 : kF16;
  uint8_t* base = static_cast<uint8_t*>(ws);
  run.ss_partial = (flags & FGEMM_EPI_ROWSUMSQ) ? reinterpret_cast<float*>(base + body) : nullptr;
  static_assert(kScaleHeaderBytes >= 256 + 2 * kMaxPartials * sizeof(float), "header");
  run.scale_a = reinterpret_cast<float*>(base + 64);
  run.scale_b = reinterpret_cast<float*>(base + 128);
  float* part_a = reinterpret_cast<float*>(base + 256);
  float* part_b = part_a + kMaxPartials;
  size_t off = kScaleHeaderBytes;
  for (int l = 1; l <= plan.depth; ++l) {
    const int64_t m = c.M >> l, k = c.K >> l, n = Nb >> l;
    for (int q = 0; q < 7; ++q) { run.S[l][q] = base + off; off += align256((size_t)(m * k * 2)); }
    for (int q = 0; q < 7; ++q) { run.T[l][q] = base + off; off += align256((size_t)(k * n * 2)); }
    for (int q = 0; q < 7; ++q) {
      run.P[l][q] = reinterpret_cast<float*>(base + off);
      off += align256((size_t)(m * n * 4));
    }
  }
  BlockedOperand L{c.A, c.lda, c.ta == FGEMM_OP_T, run.in_dtype, 0};
  BlockedOperand R{c.B, c.ldb, c.tb == FGEMM_OP_T, run.in_dtype, 0};
  // Winograd depth 1 overlapped: P1 and P2 need no operand sums (FalconGEMM page,
  // group-parallel optimizations: additions overlapped with products), so max|x|,
  // the scales and the sums of the other five run on the second stream while P1
  // and P2 run on the caller's; their plain-block temporaries are not written.
  // (the input blocks feed the 16-byte loads directly: whole 8-element block
  // offsets, leading dimensions and base addresses)
  const bool blocks16 = c.M % 16 == 0 && c.K % 16 == 0 && Nb % 16 == 0 && c.lda % 8 == 0 &&
                        c.ldb % 8 == 0 && aligned16(c.A) && aligned16(c.B);
  run.overlap = plan.variant == FGEMM_VARIANT_WINOGRAD && plan.depth == 1 && h->aux && blocks16;
  run.aux = h->aux;
  run.join = h->join;
  const hipStream_t as = run.overlap ? h->aux : c.stream;
  hipError_t e = hipSuccess;
  if (run.overlap) {
    e = hipEventRecord(h->fork, c.stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(as, h->fork, 0);
    if (e != hipSuccess) return FGEMM_ERR_HIP;
  }
  // power-of-two scales keeping every fp16 sum in range: at most 4^depth terms
  const float target = plan.depth == 1 ? 8192.f : 2048.f;
  int na = 0, nb = 0;
  e = launch_maxabs(c.A, c.lda, c.ta == FGEMM_OP_T ? c.K : c.M, c.ta == FGEMM_OP_T ? c.M : c.K,
                    run.in_dtype, part_a, &na, as);
  if (e == hipSuccess)
    e = launch_maxabs(c.B, c.ldb, c.tb == FGEMM_OP_T ? Nb : c.K, c.tb == FGEMM_OP_T ? c.K : Nb,
                      run.in_dtype, part_b, &nb, as);
  if (e == hipSuccess) e = launch_scale_from_max(part_a, na, target, run.scale_a, as);
  if (e == hipSuccess) e = launch_scale_from_max(part_b, nb, target, run.scale_b, as);
  if (run.overlap) {
    void* S[7];
    void* T[7];
    for (int q = 0; q < 7; ++q) {
      S[q] = q < 2 ? nullptr : run.S[1][q];
      T[q] = q < 2 ? nullptr : run.T[1][q];
    }
    if (e == hipSuccess) e = launch_preadd(L, c.M, c.K, run.variant, 0, run.scale_a, S, as);
    if (e == hipSuccess) e = launch_preadd(R, c.K, Nb, run.variant, 1, run.scale_b, T, as);
    if (e == hipSuccess) e = hipEventRecord(h->join, as);
  }
  if (e != hipSuccess) return FGEMM_ERR_HIP;
  return strassen_level(run, 1, L, R, c.M, c.K, Nb, nullptr, 0);
}

// Makes the handle's device current for the scope of a call and restores the
// caller's afterwards.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int device) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != device && hipSetDevice(device) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

fgemm_status_t execute(fgemm_handle_t h, const fgemm_plan_t& plan, const Call& c,
                       const WsSource& wsrc = WsSource{}) {
  DeviceGuard guard(h->device);
  if (!guard.ok) return FGEMM_ERR_HIP;
  const int vec = vec_ok(c.ta, c.tb, c.N, c.A, c.lda, c.B, c.ldb, c.C, c.ldc, c.epi);
  const uint32_t flags = epi_flags(c.epi);
  fgemm_status_t st = check_plan_shape(plan, c.M, c.N, c.K, vec, flags);
  if (st != FGEMM_OK) return st;
  if (plan.path == FGEMM_PATH_STRASSEN) {
    if (wsrc.fixed) return FGEMM_ERR_NOT_SUPPORTED;  // its workspace is not fixed-size
    return run_strassen(h, plan, c);
  }
  return run_classical(h, plan, c, vec, wsrc);
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

const char* fgemm_status_string(fgemm_status_t s) {
  switch (s) {
    case FGEMM_OK: return "FGEMM_OK";
    case FGEMM_ERR_INVALID_VALUE: return "FGEMM_ERR_INVALID_VALUE";
    case FGEMM_ERR_NOT_SUPPORTED: return "FGEMM_ERR_NOT_SUPPORTED";
    case FGEMM_ERR_WORKSPACE: return "FGEMM_ERR_WORKSPACE";
    case FGEMM_ERR_ALLOC: return "FGEMM_ERR_ALLOC";
    case FGEMM_ERR_HIP: return "FGEMM_ERR_HIP";
  }
  return "FGEMM_UNKNOWN_STATUS";
}

fgemm_status_t fgemm_check_args(fgemm_op_t ta, fgemm_op_t tb, int64_t M, int64_t N, int64_t K,
                                const void* A, int64_t lda, const void* B, int64_t ldb,
                                float beta, const void* C, int64_t ldc, fgemm_dtype_t dtype,
                                const fgemm_epilogue_t* epi) {
  if (ta != FGEMM_OP_N && ta != FGEMM_OP_T) return FGEMM_ERR_INVALID_VALUE;
  if (tb != FGEMM_OP_N && tb != FGEMM_OP_T) return FGEMM_ERR_INVALID_VALUE;
  if (dtype != FGEMM_F16 && dtype != FGEMM_BF16) return FGEMM_ERR_INVALID_VALUE;
  if (M < 0 || N < 0 || K < 0) return FGEMM_ERR_INVALID_VALUE;
  if (M > INT32_MAX || N > INT32_MAX / 2 || K > INT32_MAX) return FGEMM_ERR_NOT_SUPPORTED;
  const uint32_t flags = epi_flags(epi);
  if (flags & ~(uint32_t)(FGEMM_EPI_BIAS | FGEMM_EPI_ROWSUMSQ | FGEMM_EPI_RMS_SWIGLU |
                          FGEMM_EPI_ACT | FGEMM_EPI_ROPE | FGEMM_EPI_SWIGLU_BWD |
                          FGEMM_EPI_RMS_BWD))
    return FGEMM_ERR_INVALID_VALUE;
  // the RMS backward epilogue runs alone, without beta
  const int rms_bwd = (flags & FGEMM_EPI_RMS_BWD) != 0;
  if (rms_bwd && (flags != (uint32_t)FGEMM_EPI_RMS_BWD || beta != 0.f))
    return FGEMM_ERR_NOT_SUPPORTED;
  const int swiglu = (flags & kSwiGLUFlags) != 0;
  const int swiglu_bwd = (flags & FGEMM_EPI_SWIGLU_BWD) != 0;
  if (swiglu && (flags & ~kSwiGLUFlags)) return FGEMM_ERR_NOT_SUPPORTED;
  if ((flags & kSwiGLUFlags) == kSwiGLUFlags) return FGEMM_ERR_NOT_SUPPORTED;
  if (swiglu_bwd && beta != 0.f) return FGEMM_ERR_NOT_SUPPORTED;
  // one transform before the rounding: an activation or the rotary embedding
  if ((flags & FGEMM_EPI_ACT) && (flags & FGEMM_EPI_ROPE)) return FGEMM_ERR_NOT_SUPPORTED;
  if ((flags & FGEMM_EPI_ACT) &&
      (epi->act != FGEMM_ACT_RELU && epi->act != FGEMM_ACT_SILU && epi->act != FGEMM_ACT_GELU_TANH))
    return FGEMM_ERR_INVALID_VALUE;
  if (flags & FGEMM_EPI_ROPE) {
    const int64_t hd = epi->rope_head_dim;
    if (hd <= 0 || hd % 2 || hd > INT32_MAX || N % hd || !(epi->rope_theta > 0.f))
      return FGEMM_ERR_INVALID_VALUE;
    // the kernels rotate runs of 4 or 8 columns inside one head, and keep the pair
    // frequencies of one head in a table
    if (hd % 8 || hd > 1024) return FGEMM_ERR_NOT_SUPPORTED;
  }
  const int64_t Nb = swiglu ? 2 * N : N;
  const int64_t a_cols = ta == FGEMM_OP_N ? K : M;   // stored row width of A
  const int64_t b_cols = tb == FGEMM_OP_N ? Nb : K;  // stored row width of B
  if (lda < (a_cols > 1 ? a_cols : 1)) return FGEMM_ERR_INVALID_VALUE;
  if (ldb < (b_cols > 1 ? b_cols : 1)) return FGEMM_ERR_INVALID_VALUE;
  const int64_t Nc = swiglu_bwd ? 2 * N : N;  // output width
  if (ldc < (Nc > 1 ? Nc : 1)) return FGEMM_ERR_INVALID_VALUE;
  const bool any_out = M > 0 && N > 0;
  if (any_out && K > 0 && (A == nullptr || B == nullptr)) return FGEMM_ERR_INVALID_VALUE;
  if (any_out && C == nullptr) return FGEMM_ERR_INVALID_VALUE;
  if (swiglu_bwd && ((any_out && epi->swiglu_dout == nullptr) || epi->swiglu_ldd < (N > 1 ? N : 1)))
    return FGEMM_ERR_INVALID_VALUE;
  if (rms_bwd) {
    if (any_out && (epi->rms_x == nullptr || epi->rms_grad == nullptr ||
                    epi->rms_rowsumsq == nullptr))
      return FGEMM_ERR_INVALID_VALUE;
    if (epi->rms_ldx < (N > 1 ? N : 1) || epi->rms_n <= 0 || !(epi->rms_eps >= 0.f))
      return FGEMM_ERR_INVALID_VALUE;
  }
  if ((flags & FGEMM_EPI_BIAS) && any_out && epi->bias == nullptr) return FGEMM_ERR_INVALID_VALUE;
  if ((flags & FGEMM_EPI_ROWSUMSQ) && any_out && epi->rowsumsq == nullptr)
    return FGEMM_ERR_INVALID_VALUE;
  if (swiglu) {
    if (any_out && epi->rms_rowsumsq == nullptr) return FGEMM_ERR_INVALID_VALUE;
    if (epi->rms_n <= 0 || !(epi->rms_eps >= 0.f)) return FGEMM_ERR_INVALID_VALUE;
  }
  return FGEMM_OK;
}

fgemm_status_t fgemm_create(fgemm_handle_t* handle, int device) {
  if (!handle) return FGEMM_ERR_INVALID_VALUE;
  *handle = nullptr;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return FGEMM_ERR_HIP;
  if (device < 0 || device >= count) return FGEMM_ERR_INVALID_VALUE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return FGEMM_ERR_HIP;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return FGEMM_ERR_NOT_SUPPORTED;
  {
    // the fixed scratch of fgemm_gemm_noalloc: its device address on this device,
    // asked once, with the device current
    DeviceGuard guard(device);
    if (!guard.ok || noalloc_scratch_init(device) != hipSuccess) return FGEMM_ERR_HIP;
  }
  fgemm_handle_s* h = new (std::nothrow) fgemm_handle_s();
  if (!h) return FGEMM_ERR_ALLOC;
  h->device = device;
  h->cus = prop.multiProcessorCount;
  if (hipDeviceGetAttribute(&h->pools, hipDeviceAttributeMemoryPoolsSupported, device) !=
      hipSuccess) {
    (void)hipGetLastError();
    h->pools = 0;
  }
  {
    // the overlapped Winograd schedule's second stream (default priority) and
    // events; without them that schedule runs on the caller's stream alone
    DeviceGuard guard(device);
    if (!guard.ok || hipStreamCreateWithFlags(&h->aux, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&h->fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&h->join, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      if (h->join) (void)hipEventDestroy(h->join);
      if (h->fork) (void)hipEventDestroy(h->fork);
      if (h->aux) (void)hipStreamDestroy(h->aux);
      h->aux = nullptr;
      h->fork = h->join = nullptr;
    }
  }
  double ghz = prop.clockRate > 0 ? prop.clockRate / 1e6 : 2.4;
  model_defaults(&h->model, prop.multiProcessorCount, ghz, (double)prop.totalGlobalMem);
  *handle = h;
  return FGEMM_OK;
}

fgemm_status_t fgemm_destroy(fgemm_handle_t h) {
  if (!h) return FGEMM_ERR_INVALID_VALUE;
  if (h->aux) {
    DeviceGuard guard(h->device);
    (void)hipStreamSynchronize(h->aux);
    (void)hipEventDestroy(h->join);
    (void)hipEventDestroy(h->fork);
    (void)hipStreamDestroy(h->aux);
  }
  if (h->own_ws) {
    DeviceGuard guard(h->device);
    (void)hipDeviceSynchronize();
    if (h->pools) {
      (void)hipFreeAsync(h->own_ws, nullptr);
      (void)hipStreamSynchronize(nullptr);
    } else {
      (void)hipFree(h->own_ws);
    }
  }
  delete h;
  return FGEMM_OK;
}

fgemm_status_t fgemm_set_workspace(fgemm_handle_t h, void* dptr, size_t bytes) {
  if (!h) return FGEMM_ERR_INVALID_VALUE;
  if (dptr == nullptr && bytes != 0) return FGEMM_ERR_INVALID_VALUE;
  if (dptr && !aligned16(dptr)) return FGEMM_ERR_INVALID_VALUE;
  h->user_ws = dptr;
  h->user_ws_bytes = dptr ? bytes : 0;
  h->plans.clear();  // workspace guards depend on it
  return FGEMM_OK;
}

fgemm_status_t fgemm_get_model(fgemm_handle_t h, fgemm_model_t* m) {
  if (!h || !m) return FGEMM_ERR_INVALID_VALUE;
  *m = h->model;
  return FGEMM_OK;
}

fgemm_status_t fgemm_set_model(fgemm_handle_t h, const fgemm_model_t* m) {
  if (!h || !m) return FGEMM_ERR_INVALID_VALUE;
  if (m->compute_units <= 0 || !(m->peak_tflops > 0) || !(m->hbm_gbps > 0) ||
      !(m->eta_mfma > 0) || !(m->eta_hbm > 0) || !(m->launch_us >= 0) || !(m->max_rel_err > 0))
    return FGEMM_ERR_INVALID_VALUE;
  h->model = *m;
  h->plans.clear();
  return FGEMM_OK;
}

fgemm_status_t fgemm_select_model(const fgemm_model_t* md, fgemm_op_t ta, fgemm_op_t tb,
                                  int64_t M, int64_t N, int64_t K, fgemm_dtype_t dtype,
                                  const fgemm_epilogue_t* epi, fgemm_plan_t* plan) {
  if (!md || !plan) return FGEMM_ERR_INVALID_VALUE;
  if (ta != FGEMM_OP_N && ta != FGEMM_OP_T) return FGEMM_ERR_INVALID_VALUE;
  if (tb != FGEMM_OP_N && tb != FGEMM_OP_T) return FGEMM_ERR_INVALID_VALUE;
  if (dtype != FGEMM_F16 && dtype != FGEMM_BF16) return FGEMM_ERR_INVALID_VALUE;
  if (M < 0 || N < 0 || K < 0) return FGEMM_ERR_INVALID_VALUE;
  if (md->compute_units <= 0 || !(md->peak_tflops > 0) || !(md->hbm_gbps > 0) ||
      !(md->max_rel_err > 0))
    return FGEMM_ERR_INVALID_VALUE;
  // shapes only: assume the aligned fast path, no beta traffic, no workspace cap
  // beyond the model's own
  return select_plan(*md, M, N, K, dtype, epi_flags(epi), 0, 1, (size_t)-1, plan);
}

fgemm_status_t fgemm_select(fgemm_handle_t h, fgemm_op_t ta, fgemm_op_t tb, int64_t M, int64_t N,
                            int64_t K, fgemm_dtype_t dtype, const fgemm_epilogue_t* epi,
                            fgemm_plan_t* plan) {
  if (!h) return FGEMM_ERR_INVALID_VALUE;
  return fgemm_select_model(&h->model, ta, tb, M, N, K, dtype, epi, plan);
}

fgemm_status_t fgemm_gemm_plan(fgemm_handle_t h, const fgemm_plan_t* plan, fgemm_op_t ta,
                               fgemm_op_t tb, int64_t M, int64_t N, int64_t K, float alpha,
                               const void* A, int64_t lda, const void* B, int64_t ldb, float beta,
                               void* C, int64_t ldc, fgemm_dtype_t dtype,
                               const fgemm_epilogue_t* epi, void* stream) {
  if (!h || !plan) return FGEMM_ERR_INVALID_VALUE;
  fgemm_status_t st = fgemm_check_args(ta, tb, M, N, K, A, lda, B, ldb, beta, C, ldc, dtype, epi);
  if (st != FGEMM_OK) return st;
  if (M == 0 || N == 0) return FGEMM_OK;
  Call c{ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, epi,
         static_cast<hipStream_t>(stream)};
  fgemm_plan_t p = *plan;
  if (p.path == FGEMM_PATH_CLASSICAL && (p.tile_m == 0 || p.tile_n == 0)) {
    const int swiglu = (epi_flags(epi) & kSwiGLUFlags) != 0;
    int t = best_tile(h->model, M, N, K, swiglu, 1, 2.0, 2.0, beta != 0.f, nullptr);
    p.tile_m = tile_m_of(t);
    p.tile_n = tile_n_of(t);
  } else if (p.path == FGEMM_PATH_STRASSEN && (p.tile_m == 0 || p.tile_n == 0)) {
    if (p.depth >= 1 && p.depth <= 2) {
      int t = best_tile(h->model, M >> p.depth, N >> p.depth, K >> p.depth, 0, 7, 2.0, 4.0, 0,
                        nullptr);
      if (t > 1) t = 1;
      p.tile_m = tile_m_of(t);
      p.tile_n = tile_n_of(t);
    }
  }
  if (p.path == FGEMM_PATH_STRASSEN && tile_id(p.tile_m, p.tile_n) > 1)
    return FGEMM_ERR_NOT_SUPPORTED;
  if (tile_id(p.tile_m, p.tile_n) < 0 && p.path == FGEMM_PATH_CLASSICAL)
    return FGEMM_ERR_INVALID_VALUE;
  return execute(h, p, c);
}

fgemm_status_t fgemm_gemm(fgemm_handle_t h, fgemm_op_t ta, fgemm_op_t tb, int64_t M, int64_t N,
                          int64_t K, float alpha, const void* A, int64_t lda, const void* B,
                          int64_t ldb, float beta, void* C, int64_t ldc, fgemm_dtype_t dtype,
                          const fgemm_epilogue_t* epi, void* stream) {
  if (!h) return FGEMM_ERR_INVALID_VALUE;
  fgemm_status_t st = fgemm_check_args(ta, tb, M, N, K, A, lda, B, ldb, beta, C, ldc, dtype, epi);
  if (st != FGEMM_OK) return st;
  if (M == 0 || N == 0) return FGEMM_OK;
  const int vec = vec_ok(ta, tb, N, A, lda, B, ldb, C, ldc, epi);
  // beta != 0 sits above every epilogue flag bit
  PlanKey key{M, N, K, (int)ta, (int)tb, (int)dtype,
              (int)epi_flags(epi) | (beta != 0.f ? 1 << 30 : 0), vec};
  auto it = h->plans.find(key);
  fgemm_plan_t plan;
  if (it != h->plans.end()) {
    plan = it->second;
  } else {
    size_t limit = h->user_ws ? h->user_ws_bytes : (size_t)-1;
    st = select_plan(h->model, M, N, K, dtype, epi_flags(epi), beta != 0.f, vec, limit, &plan);
    if (st != FGEMM_OK) return st;
    h->plans.emplace(key, plan);
  }
  Call c{ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, epi,
         static_cast<hipStream_t>(stream)};
  st = execute(h, plan, c);
  if (st == FGEMM_ERR_ALLOC && !h->user_ws && plan.workspace_bytes > 0) {
    // the device could not hold the planned workspace (nothing was launched): plan
    // again within what the handle holds now, which at worst is the classical path
    fgemm_plan_t alt;
    if (select_plan(h->model, M, N, K, dtype, epi_flags(epi), beta != 0.f, vec,
                    h->own_ws_bytes, &alt) == FGEMM_OK &&
        alt.workspace_bytes < plan.workspace_bytes) {
      h->plans[key] = alt;
      st = execute(h, alt, c);
    }
  }
  return st;
}

fgemm_status_t fgemm_gemm_noalloc(fgemm_handle_t h, fgemm_op_t ta, fgemm_op_t tb, int64_t M,
                                  int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                                  const void* B, int64_t ldb, float beta, void* C, int64_t ldc,
                                  fgemm_dtype_t dtype, const fgemm_epilogue_t* epi,
                                  void* stream) {
  if (!h) return FGEMM_ERR_INVALID_VALUE;
  fgemm_status_t st = fgemm_check_args(ta, tb, M, N, K, A, lda, B, ldb, beta, C, ldc, dtype, epi);
  if (st != FGEMM_OK) return st;
  if (M == 0 || N == 0) return FGEMM_OK;
  WsSource wsrc;
  wsrc.fixed = noalloc_scratch(h->device);
  wsrc.fixed_bytes = kNoAllocScratchBytes;
  if (!wsrc.fixed) return FGEMM_ERR_HIP;  // fgemm_create sets it up on the handle's device
  const int vec = vec_ok(ta, tb, N, A, lda, B, ldb, C, ldc, epi);
  PlanKey key{M, N, K, (int)ta, (int)tb, (int)dtype,
              (int)epi_flags(epi) | (beta != 0.f ? 1 << 30 : 0), vec};
  NoAllocSlot& slot = h->noalloc_plans[PlanKeyHash()(key) % kNoAllocSlots];
  if (!slot.valid || !(slot.key == key)) {
    fgemm_plan_t plan;
    st = select_plan(h->model, M, N, K, dtype, epi_flags(epi), beta != 0.f, vec,
                     kNoAllocScratchBytes, &plan, /*classical_only=*/true);
    if (st != FGEMM_OK) return st;
    slot.key = key;
    slot.plan = plan;
    slot.valid = true;
  }
  Call c{ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, epi,
         static_cast<hipStream_t>(stream)};
  return execute(h, slot.plan, c, wsrc);
}

}  // extern "C"

namespace {

// The 8-bit GEMM with per-tensor scales (mx_a == mx_b == null) or E8M0 block scales;
// with f4, the MXFP4 GEMM (E2M1 values two a byte, block scales required, formats
// unused, lda/ldb in bytes).
fgemm_status_t gemm_f8(fgemm_handle_t h, int64_t M, int64_t N, int64_t K, float alpha,
                       const void* A, int64_t lda, fgemm_f8_format_t a_format, float scale_a,
                       const uint8_t* mx_a, int64_t ld_mxa, const void* B, int64_t ldb,
                       fgemm_f8_format_t b_format, float scale_b, const uint8_t* mx_b,
                       int64_t ld_mxb, float beta, void* C, int64_t ldc, fgemm_dtype_t dtype,
                       const fgemm_epilogue_t* epi, void* stream, bool f4 = false) {
  if (!h) return FGEMM_ERR_INVALID_VALUE;
  const bool mx = mx_a != nullptr || mx_b != nullptr;
  if (mx) {
    // whole 16-byte groups of 16 block scales per row (the kernel loads a group of
    // 4 phases at a time), 16-byte aligned rows
    const int64_t groups = (K / 32 + 15) / 16 * 16;
    if (K > 0 && (mx_a == nullptr || mx_b == nullptr)) return FGEMM_ERR_INVALID_VALUE;
    if (ld_mxa < (K / 32 > 1 ? K / 32 : 1) || ld_mxb < (K / 32 > 1 ? K / 32 : 1))
      return FGEMM_ERR_INVALID_VALUE;
    if (ld_mxa % 16 || ld_mxb % 16 || ld_mxa < groups || ld_mxb < groups || !aligned16(mx_a) ||
        !aligned16(mx_b))
      return FGEMM_ERR_NOT_SUPPORTED;
  }
  if (!f4 && ((a_format != FGEMM_E4M3 && a_format != FGEMM_E5M2) ||
              (b_format != FGEMM_E4M3 && b_format != FGEMM_E5M2)))
    return FGEMM_ERR_INVALID_VALUE;
  if (dtype != FGEMM_F16 && dtype != FGEMM_BF16) return FGEMM_ERR_INVALID_VALUE;
  if (M < 0 || N < 0 || K < 0) return FGEMM_ERR_INVALID_VALUE;
  if (M > INT32_MAX || N > INT32_MAX / 2 || K > INT32_MAX) return FGEMM_ERR_NOT_SUPPORTED;
  const uint32_t flags = epi_flags(epi);
  if (flags & ~(uint32_t)(FGEMM_EPI_BIAS | FGEMM_EPI_ROWSUMSQ | FGEMM_EPI_RMS_SWIGLU |
                          FGEMM_EPI_ACT | FGEMM_EPI_ROPE | FGEMM_EPI_SWIGLU_BWD |
                          FGEMM_EPI_RMS_BWD))
    return FGEMM_ERR_INVALID_VALUE;
  if (flags & ~(uint32_t)(FGEMM_EPI_BIAS | FGEMM_EPI_ROWSUMSQ)) return FGEMM_ERR_NOT_SUPPORTED;
  const int64_t row_bytes = f4 ? (K + 1) / 2 : K;  // bytes of one operand row
  if (lda < (row_bytes > 1 ? row_bytes : 1) || ldb < (row_bytes > 1 ? row_bytes : 1) ||
      ldc < (N > 1 ? N : 1))
    return FGEMM_ERR_INVALID_VALUE;
  const bool any_out = M > 0 && N > 0;
  if (any_out && K > 0 && (A == nullptr || B == nullptr)) return FGEMM_ERR_INVALID_VALUE;
  if (any_out && C == nullptr) return FGEMM_ERR_INVALID_VALUE;
  if ((flags & FGEMM_EPI_BIAS) && any_out && epi->bias == nullptr) return FGEMM_ERR_INVALID_VALUE;
  if ((flags & FGEMM_EPI_ROWSUMSQ) && any_out && epi->rowsumsq == nullptr)
    return FGEMM_ERR_INVALID_VALUE;
  if (!isfinite(scale_a) || !isfinite(scale_b) || !isfinite(alpha)) return FGEMM_ERR_INVALID_VALUE;
  // whole phases (128 bytes a row: 128 values, 256 at 4 bits), 16-byte rows and
  // pointers: the kernel has no K tail path
  if (K % (f4 ? 256 : 128) || lda % 16 || ldb % 16 || ldc % 8 || !aligned16(A) ||
      !aligned16(B) || !aligned16(C))
    return FGEMM_ERR_NOT_SUPPORTED;
  // the tensor scales enter through alpha, formed in fp32: it must stay a normal value
  const double f = (double)alpha * (double)scale_a * (double)scale_b;
  if (f != 0.0 && (fabs(f) < 1.1754943508222875e-38 || fabs(f) > 3.4028234663852886e38))
    return FGEMM_ERR_NOT_SUPPORTED;
  if (!any_out) return FGEMM_OK;
  DeviceGuard guard(h->device);
  if (!guard.ok) return FGEMM_ERR_HIP;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  GemmBatch b{};
  b.count = 1;
  b.cus = h->cus;
  GemmProblem& p = b.p[0];
  // byte pairs: the kernel addresses both operands in 16-bit units (2 values at 8
  // bits, 4 at 4 bits)
  p.A = A; p.B = B; p.C = C; p.Cin = C;
  p.lda = lda / 2; p.ldb = ldb / 2; p.ldc = ldc;
  p.M = (int)M; p.N = (int)N; p.K = (int)(f4 ? K / 4 : K / 2);
  p.alpha = (float)f;
  p.beta = beta;
  p.flags = beta != 0.f ? kFlagBeta : 0u;
  if (flags & FGEMM_EPI_BIAS) { p.flags |= kFlagBias; p.bias = epi->bias; }
  int parts = 0;
  if (flags & FGEMM_EPI_ROWSUMSQ) {
    // one partial per (tile column, wave column) and row
    parts = (int)ceil_div(N, kF8TileN) * kF8WavesN;
    void* ws;
    fgemm_status_t s = ensure_workspace(h, WsSource{}, (size_t)parts * (size_t)M * 4, st, &ws);
    if (s != FGEMM_OK) return s;
    p.flags |= kFlagRowSumSq;
    p.ss_partial = static_cast<float*>(ws);
  }
  if (mx) {
    p.mx_a = mx_a; p.mx_b = mx_b;
    p.ld_mxa = ld_mxa; p.ld_mxb = ld_mxb;
  }
  KernelKey k{};
  k.a_kcontig = 1;
  k.b_kcontig = 1;
  k.dtype = f4 ? kF4MX : f8_code((int)a_format, (int)b_format, mx ? 1 : 0);
  k.epi = kEpiStore16;
  k.vec = 1;
  k.odt = dtype == FGEMM_BF16 ? kBF16 : kF16;
  if (launch_gemm_f8(k, b, st) != hipSuccess) return FGEMM_ERR_HIP;
  if (parts && launch_rowsumsq_reduce(p.ss_partial, parts, (int)M, epi->rowsumsq, st) != hipSuccess)
    return FGEMM_ERR_HIP;
  return FGEMM_OK;
}

}  // namespace

extern "C" {

fgemm_status_t fgemm_gemm_f8(fgemm_handle_t h, int64_t M, int64_t N, int64_t K, float alpha,
                             const void* A, int64_t lda, fgemm_f8_format_t a_format,
                             float scale_a, const void* B, int64_t ldb,
                             fgemm_f8_format_t b_format, float scale_b, float beta, void* C,
                             int64_t ldc, fgemm_dtype_t dtype, const fgemm_epilogue_t* epi,
                             void* stream) {
  return gemm_f8(h, M, N, K, alpha, A, lda, a_format, scale_a, nullptr, 0, B, ldb, b_format,
                 scale_b, nullptr, 0, beta, C, ldc, dtype, epi, stream);
}

fgemm_status_t fgemm_gemm_mxf8(fgemm_handle_t h, int64_t M, int64_t N, int64_t K, float alpha,
                               const void* A, int64_t lda, fgemm_f8_format_t a_format,
                               const void* a_scales, int64_t ld_a_scales, const void* B,
                               int64_t ldb, fgemm_f8_format_t b_format, const void* b_scales,
                               int64_t ld_b_scales, float beta, void* C, int64_t ldc,
                               fgemm_dtype_t dtype, const fgemm_epilogue_t* epi, void* stream) {
  if (K > 0 && (a_scales == nullptr || b_scales == nullptr)) return FGEMM_ERR_INVALID_VALUE;
  // K = 0 reads no scale (C = beta*C + bias): the unscaled kernel does the same
  const uint8_t* sa = K > 0 ? static_cast<const uint8_t*>(a_scales) : nullptr;
  const uint8_t* sb = K > 0 ? static_cast<const uint8_t*>(b_scales) : nullptr;
  return gemm_f8(h, M, N, K, alpha, A, lda, a_format, 1.f, sa, ld_a_scales, B, ldb, b_format,
                 1.f, sb, ld_b_scales, beta, C, ldc, dtype, epi, stream);
}

fgemm_status_t fgemm_quantize_mx(const void* X, int64_t rows, int64_t cols, int64_t ldx,
                                 fgemm_dtype_t x_dtype, int transpose, fgemm_f8_format_t format,
                                 void* Q, int64_t ldq, void* scales, int64_t ld_scales,
                                 void* stream) {
  if (rows < 0 || cols < 0 || ldx < (cols > 1 ? cols : 1)) return FGEMM_ERR_INVALID_VALUE;
  if (x_dtype != FGEMM_F16 && x_dtype != FGEMM_BF16) return FGEMM_ERR_INVALID_VALUE;
  if (format != FGEMM_E4M3 && format != FGEMM_E5M2 && format != FGEMM_E2M1)
    return FGEMM_ERR_INVALID_VALUE;
  const int64_t orows = transpose ? cols : rows, olen = transpose ? rows : cols;
  if (olen % 32) return FGEMM_ERR_INVALID_VALUE;
  const int64_t row_bytes = format == FGEMM_E2M1 ? olen / 2 : olen;
  if (ldq < (row_bytes > 1 ? row_bytes : 1) || ld_scales < (olen / 32 > 1 ? olen / 32 : 1))
    return FGEMM_ERR_INVALID_VALUE;
  if (orows == 0 || olen == 0) return FGEMM_OK;
  if (!X || !Q || !scales) return FGEMM_ERR_INVALID_VALUE;
  if (!aligned16(X) || !aligned16(Q) || ldx % 8 || ldq % 16) return FGEMM_ERR_NOT_SUPPORTED;
  // 32-bit grid limits of the two kernels
  if ((!transpose && rows * (cols / 32) * 4 / 256 >= INT32_MAX) ||
      (transpose && (rows + 127) / 128 > 65535))
    return FGEMM_ERR_NOT_SUPPORTED;
  const hipError_t e = launch_quantize_mx(X, rows, cols, ldx,
                                          x_dtype == FGEMM_BF16 ? kBF16 : kF16, transpose != 0,
                                          (int)format, Q, ldq, scales, ld_scales,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FGEMM_OK : FGEMM_ERR_HIP;
}

fgemm_status_t fgemm_gemm_mxf4(fgemm_handle_t h, int64_t M, int64_t N, int64_t K, float alpha,
                               const void* A, int64_t lda, const void* a_scales,
                               int64_t ld_a_scales, const void* B, int64_t ldb,
                               const void* b_scales, int64_t ld_b_scales, float beta, void* C,
                               int64_t ldc, fgemm_dtype_t dtype, const fgemm_epilogue_t* epi,
                               void* stream) {
  if (K > 0 && (a_scales == nullptr || b_scales == nullptr)) return FGEMM_ERR_INVALID_VALUE;
  if (K == 0) {
    // no value and no scale is read (C = beta*C + bias): the 8-bit kernel does that
    return gemm_f8(h, M, N, 0, alpha, A, lda, FGEMM_E4M3, 1.f, nullptr, 0, B, ldb, FGEMM_E4M3,
                   1.f, nullptr, 0, beta, C, ldc, dtype, epi, stream);
  }
  return gemm_f8(h, M, N, K, alpha, A, lda, FGEMM_E4M3, 1.f,
                 static_cast<const uint8_t*>(a_scales), ld_a_scales, B, ldb, FGEMM_E4M3, 1.f,
                 static_cast<const uint8_t*>(b_scales), ld_b_scales, beta, C, ldc, dtype, epi,
                 stream, true);
}

}  // extern "C"
