// model.cpp — the analytic decision model (pure host code, no device calls).
//
// FalconGEMM summary (euno.news), Methodology 4: the decision module estimates the
// run time of every candidate from compute throughput, memory bandwidth and the
// extra cost of each recursion level, and picks the algorithm and tiling of least
// predicted time; Methodology 5: it is queried at run time with the actual sizes.
// The time terms come from CS336 Lecture 05 notes:
//   Page 21 (roofline): a kernel's time is about max(FLOPs / P_peak, bytes / B_mem);
//   Page 43 (tile quantization): ceil-divided tile grids compute padded tiles;
//   Page 48 (wave quantization): tiles run in waves of one tile per compute unit,
//     the last wave possibly partly empty.
// Strassen candidates add the traffic of their block additions per level and run
// 7^d sub-products of (M/2^d, N/2^d, K/2^d) in batches of seven.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "model.h"

namespace fgemm {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute and memory time of one kernel: they overlap, but not perfectly; the
// shorter one still shows a little (this also breaks ties toward less padding).
double overlap(double a, double b) {
  const double hi = a > b ? a : b, lo = a > b ? b : a;
  return hi + 0.05 * lo;
}

// Bandwidth `blocks` workgroups can pull: each keeps a few tile phases in flight,
// measured at ~50 GB/s per workgroup (112 workgroups of the 32x128 tile stream
// 5.6 TB/s), capped by HBM.
double stream_bw(const fgemm_model_t& md, int64_t blocks) {
  constexpr double kWgBytesPerSec = 50e9;
  const double hbm = md.hbm_gbps * 1e9 * md.eta_hbm;
  // an empty grid (M or N = 0) still gets one workgroup's rate: its time stays finite
  const double wg = (double)(blocks > 0 ? blocks : 1) * kWgBytesPerSec;
  return wg < hbm ? wg : hbm;
}

// Macro-tiles of the classical kernel and the share of the per-CU MFMA rate each
// reaches at steady state relative to the 256x256 tile (smaller tiles re-read
// operands more often per FLOP and hide less latency).
const TileInfo kTiles[kNumTiles] = {
    {0, 256, 256, 64, 1.00, 2, 1, 0},
    {1, 128, 128, 32, 0.70, 2, 1, 0},
    {2, 64, 128, 32, 0.45, 2, 1, 0},
    {3, 32, 128, 64, 0.30, 4, 0, 0},
    // twice the workgroups of the 32x128 tile on one-row (decode) shapes: 7 % more
    // bandwidth at M = 1 and 16 on N = 14336, K = 4096 and 3 % at M = 64 (where the
    // 32x128 tile reads B twice); with more rows it would re-read B, hence one row
    {4, 64, 64, 64, 0.30, 2, 0, 1},
};

void model_defaults(fgemm_model_t* m, int cus, double clock_ghz, double device_bytes) {
  m->compute_units = cus;
  // dense 16-bit MFMA: 4 SIMDs x 1024 FLOP per clock per CU on gfx950
  m->peak_tflops = cus * 4096.0 * clock_ghz * 1e9 / 1e12;
  m->hbm_gbps = 8000.0;
  // measured on MI355X (bf16 8192^3 and LLM shapes, 256x256 tile): ~1.27-1.33
  // PFLOP/s against 2.5 at the nominal clock (the chip holds ~1.3-1.5 GHz under
  // this load); the streaming add kernels move ~5.2-5.3 TB/s
  m->eta_mfma = 0.52;
  m->eta_hbm = 0.66;
  m->launch_us = 4.0;
  // a third of device memory (96 GB on a 288 GB MI355X): Strassen workspace grows as
  // (M*K + K*N + M*N) * (2/4 + ...) bytes, and its crossover on this chip sits near
  // 49152^3, whose two-level plan needs 42 GB (75 GB at 65536^3)
  m->max_workspace_bytes = device_bytes > 0 ? device_bytes / 3.0 : 16.0 * (1ull << 30);
  m->max_rel_err = 5e-3;
}

// Normwise error ||C - RNE(D)||_F / ||RNE(D)||_F of each path, measured on MI355X for
// i.i.d. U[-1,1] and N(0,1) inputs at 1024^3 and 4096^3 (the two sizes and the two
// distributions agreed to within 15 %), rounded up by about 5 %.  It is set by the
// fp16 temporaries of the Strassen sums (unit roundoff 2^-11) and by how many of them
// each output combines: Strassen's products of fewer sums beat Winograd's chained ones,
// and a second level roughly doubles the first.  Not a worst-case bound: inputs of
// widely different magnitudes can do worse.
double predicted_rel_err(int dtype, int variant, int depth) {
  if (depth <= 0) return 1e-4;  // fp32 accumulation and one rounding (measured <= 6.4e-5)
  const bool bf = dtype == FGEMM_BF16;
  // <2,2,3;11>: S69's seven products on two thirds of C, fp16-scaled plain blocks on
  // the last third; measured 5.6-6.7e-4 (bf16) and 5.05e-4 (fp16) at 1024 x 1536 x 1024
  if (variant == FGEMM_VARIANT_R223) return bf ? 7.3e-4 : 5.5e-4;
  const bool s69 = variant == FGEMM_VARIANT_S69;
  if (depth == 1) return s69 ? (bf ? 8.6e-4 : 6.5e-4) : (bf ? 1.17e-3 : 8.4e-4);
  return s69 ? (bf ? 1.64e-3 : 1.33e-3) : (bf ? 2.6e-3 : 2.26e-3);
}

// Rate of the classical kernel on fp16 inputs relative to bf16 ones: the chip holds a
// lower clock on fp16 MFMA work under its power limit.  Measured fp16/bf16 time ratios
// at 16384^3, 32768x8192x8192, 40960^3, 49152^3 and 65536^3 were 0.99-1.09, 1.03 on
// average.
double classical_dtype_rate(int dtype) { return dtype == FGEMM_F16 ? 0.97 : 1.0; }

// Time of one classical launch of `count` same-shape problems on one tile config.
double classical_time_us(const fgemm_model_t& md, const TileInfo& t, int64_t M, int64_t N,
                         int64_t K, int64_t Nb, int64_t out_bn, int count, double in_bytes,
                         double out_bytes, int beta) {
  const int64_t tiles = ceil_div(M, t.bm) * ceil_div(N, out_bn) * count;
  const int64_t waves = ceil_div(tiles, md.compute_units);
  const double per_cu = md.peak_tflops * 1e12 / md.compute_units;  // FLOP/s per CU
  const double tile_flops = 2.0 * t.bm * t.bn * (double)(K > 0 ? K : 1);
  const double t_compute = waves * tile_flops / (per_cu * md.eta_mfma * t.rel_eta);
  const double bytes = count * ((double)M * K * in_bytes + (double)K * Nb * in_bytes +
                                (double)M * N * out_bytes * (beta ? 2.0 : 1.0));
  const double t_mem = bytes / stream_bw(md, tiles);
  return overlap(t_compute, t_mem) * 1e6 + md.launch_us;
}

int best_tile(const fgemm_model_t& md, int64_t M, int64_t N, int64_t K, int swiglu, int count,
              double in_bytes, double out_bytes, int beta, double* t_us, int max_tile) {
  int best = -1;
  double bt = 0;
  for (int i = 0; i < kNumTiles && kTiles[i].tile <= max_tile; ++i) {
    const TileInfo& t = kTiles[i];
    if (swiglu && !t.swiglu) continue;  // the SwiGLU epilogue needs two column halves
    if (t.one_row && M > t.bm) continue;
    const int64_t out_bn = swiglu ? t.bn / 2 : t.bn;
    const int64_t Nb = swiglu ? 2 * N : N;
    double tt = classical_time_us(md, t, M, N, K, Nb, out_bn, count, in_bytes, out_bytes, beta);
    // on a tie prefer fewer tile rows (every tile row reads B again, from L2 at
    // best), then more tiles (more workgroups keep more loads in flight)
    const TileInfo* b = best < 0 ? nullptr : &kTiles[best];
    const int64_t rows = ceil_div(M, t.bm), brows = b ? ceil_div(M, b->bm) : 0;
    const int64_t cols = ceil_div(N, out_bn);
    const int64_t bcols = b ? ceil_div(N, swiglu ? b->bn / 2 : b->bn) : 0;
    if (!b || tt < bt ||
        (tt == bt && (rows < brows || (rows == brows && cols > bcols)))) {
      best = t.tile;
      bt = tt;
    }
  }
  if (t_us) *t_us = bt;
  return best;
}

double splitk_time_us(const fgemm_model_t& md, const TileInfo& t, int64_t M, int64_t N,
                      int64_t K, int splits, int beta) {
  // `splits` slices of K/splits each, fp32 partials out, then one finalize pass
  const int64_t tiles = ceil_div(M, t.bm) * ceil_div(N, t.bn);
  const int64_t blocks = tiles * splits;
  const int64_t waves = ceil_div(blocks, md.compute_units);
  const double per_cu = md.peak_tflops * 1e12 / md.compute_units;
  const double t_compute =
      waves * 2.0 * t.bm * t.bn * (double)(K / splits) / (per_cu * md.eta_mfma * t.rel_eta);
  const double bytes = (double)M * K * 2 + (double)K * N * 2 + (double)splits * M * N * 4;
  const double bw = md.hbm_gbps * 1e9 * md.eta_hbm;
  const double t_mem = bytes / stream_bw(md, blocks);
  const double fin = ((double)splits * M * N * 4 + (double)M * N * 2 * (beta ? 2.0 : 1.0)) / bw;
  return (overlap(t_compute, t_mem) + fin) * 1e6 + 2 * md.launch_us;
}

// <2,2,3;11>: Strassen (1969) on op(B) and C's first two column blocks, then the four
// block products of the third (C13 = A11 B13 + A12 B23, C23 = A21 B13 + A22 B23).
// Blocks of op(A): A11 A12 A21 A22; of op(B): B11 B12 B13 B21 B22 B23; of C: C11 C12
// C13 C21 C22 C23.
namespace {
const signed char kR223U[11 * 4] = {
    1, 0, 0, 1,    // M1: A11 + A22
    0, 0, 1, 1,    // M2: A21 + A22
    1, 0, 0, 0,    // M3: A11
    0, 0, 0, 1,    // M4: A22
    1, 1, 0, 0,    // M5: A11 + A12
    -1, 0, 1, 0,   // M6: A21 - A11
    0, 1, 0, -1,   // M7: A12 - A22
    1, 0, 0, 0,    // M8: A11
    0, 1, 0, 0,    // M9: A12
    0, 0, 1, 0,    // M10: A21
    0, 0, 0, 1,    // M11: A22
};
const signed char kR223V[11 * 6] = {
    1, 0, 0, 0, 1, 0,    // M1: B11 + B22
    1, 0, 0, 0, 0, 0,    // M2: B11
    0, 1, 0, 0, -1, 0,   // M3: B12 - B22
    -1, 0, 0, 1, 0, 0,   // M4: B21 - B11
    0, 0, 0, 0, 1, 0,    // M5: B22
    1, 1, 0, 0, 0, 0,    // M6: B11 + B12
    0, 0, 0, 1, 1, 0,    // M7: B21 + B22
    0, 0, 1, 0, 0, 0,    // M8: B13
    0, 0, 0, 0, 0, 1,    // M9: B23
    0, 0, 1, 0, 0, 0,    // M10: B13
    0, 0, 0, 0, 0, 1,    // M11: B23
};
const signed char kR223W[6 * 11] = {
    1, 0, 0, 1, -1, 0, 1, 0, 0, 0, 0,    // C11 = M1 + M4 - M5 + M7
    0, 0, 1, 0, 1, 0, 0, 0, 0, 0, 0,     // C12 = M3 + M5
    0, 0, 0, 0, 0, 0, 0, 1, 1, 0, 0,     // C13 = M8 + M9
    0, 1, 0, 1, 0, 0, 0, 0, 0, 0, 0,     // C21 = M2 + M4
    1, -1, 1, 0, 0, 1, 0, 0, 0, 0, 0,    // C22 = M1 - M2 + M3 + M6
    0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 1,     // C23 = M10 + M11
};
const BlockScheme kR223{2, 2, 3, 11, kR223U, kR223V, kR223W};
}  // namespace

const BlockScheme* block_scheme(int variant) {
  return variant == FGEMM_VARIANT_R223 ? &kR223 : nullptr;
}

// Time of a table-driven scheme at depth 1: max|x| passes, one pre-add pass a side
// (its blocks read, R fp16 operands written), R products of the block size, the
// post-add (R fp32 products read, C written, beta*C read).
double scheme_time_us(const fgemm_model_t& md, const BlockScheme& s, int64_t M, int64_t N,
                      int64_t K, int beta, int* sub_tile) {
  const double bw = md.hbm_gbps * 1e9 * md.eta_hbm;
  const double m = (double)(M / s.mb), k = (double)(K / s.kb), n = (double)(N / s.nb);
  const double R = s.R;
  double bytes = ((double)M * K + (double)K * N) * 2.0;                // max|x|
  bytes += s.mb * s.kb * m * k * 2 + R * m * k * 2;                     // pre-add, A side
  bytes += s.kb * s.nb * k * n * 2 + R * k * n * 2;                     // pre-add, B side
  bytes += R * m * n * 4 + (double)M * N * 2 * (beta ? 2.0 : 1.0);     // post-add
  double tp;  // a batch of seven products (the batches hold at most seven)
  const int tile = best_tile(md, M / s.mb, N / s.nb, K / s.kb, 0, 7, 2.0, 4.0, 0, &tp, 1);
  if (sub_tile) *sub_tile = tile;
  constexpr double kProductRate = 0.93;  // fp16 operands, fp32 outputs (as for Strassen)
  const double one = (tp - md.launch_us) * 1e-6 / kProductRate / 7.0;
  const int launches = 4 + 2 + (s.R + 6) / 7 + 1;
  return (bytes / bw + R * one) * 1e6 + launches * md.launch_us;
}

size_t strassen_workspace(int64_t M, int64_t N, int64_t K, int depth, int variant) {
  if (const BlockScheme* s = block_scheme(variant)) {
    if (depth != 1) return 0;
    const int64_t m = M / s->mb, k = K / s->kb, n = N / s->nb;
    return kScaleHeaderBytes + (align256((size_t)(m * k * 2)) + align256((size_t)(k * n * 2)) +
                                align256((size_t)(m * n * 4))) * (size_t)s->R;
  }
  const int64_t ns = 7;  // the seven fp16 operands of each side's products
  size_t total = kScaleHeaderBytes;
  for (int l = 1; l <= depth; ++l) {
    const int64_t m = M >> l, k = K >> l, n = N >> l;
    total += align256((size_t)(m * k * 2)) * ns;
    total += align256((size_t)(k * n * 2)) * ns;
    total += align256((size_t)(m * n * 4)) * 7;
  }
  return total;
}

// Winograd at depth 1 runs overlapped: max|x|, the scales and the sums of P3..P7 on
// a second stream beside P1 = A11 B11 and P2 = A12 B21 (no sums, the input blocks)
// on 7/8 of the CUs; then P3..P7 on the whole chip and the post-add.  Measured on
// the 16384^3 and 32768 x 8192^2 bf16 shapes: the sums reach about a quarter of the
// chip's HBM rate on their eighth of the CUs, P1/P2 take 13 % longer beside them
// than their CU share alone gives, and whatever sum traffic is left when P1/P2 end
// runs at the full rate.
double winograd_overlapped_us(const fgemm_model_t& md, int64_t M, int64_t N, int64_t K, int beta,
                              int* sub_tile) {
  constexpr double kAuxBwShare = 0.25, kContention = 1.13, kProductRate = 0.93;
  const double bw = md.hbm_gbps * 1e9 * md.eta_hbm;
  const double m = (double)(M / 2), k = (double)(K / 2), n = (double)(N / 2);
  // max passes, then sums: four blocks read and five fp16 operands written a side
  const double aux = ((double)M * K + (double)K * N) * 2.0 + 9 * m * k * 2 + 9 * k * n * 2;
  const double post = 7 * m * n * 4 + 4 * m * n * 2.0 + (beta ? 4 * m * n * 2.0 : 0.0);
  double tp;  // a batch of seven products on the whole chip
  const int tile = best_tile(md, M / 2, N / 2, K / 2, 0, 7, 2.0, 4.0, 0, &tp, 1);
  if (sub_tile) *sub_tile = tile;
  const double one = (tp - md.launch_us) * 1e-6 / kProductRate / 7.0;  // one product, s
  const double t12 = 2 * one * 8.0 / 7.0 * kContention;
  const double aux_slow = aux / (bw * kAuxBwShare);
  const double t_aux = aux_slow <= t12 ? aux_slow : t12 + (aux - t12 * bw * kAuxBwShare) / bw;
  const double t = (t12 > t_aux ? t12 : t_aux) + 5 * one + post / bw;
  return t * 1e6 + 9 * md.launch_us;  // 4 max/scale, 2 sums, 2 product batches, post-add
}

double strassen_time_us(const fgemm_model_t& md, int64_t M, int64_t N, int64_t K, int depth,
                        int variant, int beta, int* sub_tile) {
  const double bw = md.hbm_gbps * 1e9 * md.eta_hbm;
  if (variant == FGEMM_VARIANT_WINOGRAD && depth == 1)
    return winograd_overlapped_us(md, M, N, K, beta, sub_tile);
  if (const BlockScheme* s = block_scheme(variant)) return scheme_time_us(md, *s, M, N, K, beta, sub_tile);
  const double ns = 7;  // fp16 operands written per side (sums and plain blocks)
  double t = 0, launches = 0;
  // max|A|, max|B| for the fp16 scales
  t += ((double)M * K + (double)K * N) * 2.0 / bw;
  launches += 4;  // two max passes, two scale kernels
  double instances = 1;  // how many problems of this level run
  for (int l = 1; l <= depth; ++l) {
    const double m = (double)(M >> l), k = (double)(K >> l), n = (double)(N >> l);
    const double pre = 4 * m * k * 2 + ns * m * k * 2 + 4 * k * n * 2 + ns * k * n * 2;
    // (the fp32 products are written by the MFMA-bound sub-product kernels, under
    // their compute time)
    const double post = 7 * m * n * 4 + 4 * m * n * (l == 1 ? 2.0 : 4.0) +
                        (l == 1 && beta ? 4 * m * n * 2.0 : 0.0);
    t += instances * (pre + post) / bw;
    launches += instances * 3;
    instances *= 7;
  }
  // sub-products: 7^d problems of the deepest size, seven per launch.  They run on
  // fp16 operands with fp32 outputs, measured at ~0.93 of the bf16 rate of the
  // same kernel (the chip clocks lower on fp16 MFMA work under its power limit).
  constexpr double kProductRate = 0.93;
  const int64_t m = M >> depth, n = N >> depth, k = K >> depth;
  double tp;
  int tile = best_tile(md, m, n, k, 0, 7, 2.0, 4.0, 0, &tp, 1);
  if (sub_tile) *sub_tile = tile;
  const double batches = instances / 7;
  t += batches * (tp - md.launch_us) / kProductRate * 1e-6;
  launches += batches;
  return t * 1e6 + launches * md.launch_us;
}

}  // namespace fgemm

using namespace fgemm;

extern "C" int64_t fgemm_tile_count(int64_t M, int64_t N, int64_t tile_m, int64_t tile_n) {
  if (M < 0 || N < 0 || tile_m <= 0 || tile_n <= 0) return -1;
  return ceil_div(M, tile_m) * ceil_div(N, tile_n);
}

extern "C" double fgemm_plan_rel_err(fgemm_dtype_t dtype, const fgemm_plan_t* plan) {
  if (!plan || (dtype != FGEMM_F16 && dtype != FGEMM_BF16)) return -1.0;
  if (plan->path == FGEMM_PATH_CLASSICAL) return predicted_rel_err(dtype, 0, 0);
  if (plan->path != FGEMM_PATH_STRASSEN || plan->depth < 1 || plan->depth > 2 ||
      (plan->variant != FGEMM_VARIANT_S69 && plan->variant != FGEMM_VARIANT_WINOGRAD &&
       plan->variant != FGEMM_VARIANT_R223) ||
      (plan->variant == FGEMM_VARIANT_R223 && plan->depth != 1))
    return -1.0;
  return predicted_rel_err(dtype, plan->variant, plan->depth);
}

extern "C" int64_t fgemm_wave_count(int64_t tiles, int64_t units, double* tail_fraction) {
  if (tiles < 0 || units <= 0) return -1;
  const int64_t waves = ceil_div(tiles, units);
  if (tail_fraction) {
    const int64_t last = tiles - (waves > 0 ? (waves - 1) * units : 0);
    *tail_fraction = waves > 0 ? (double)last / (double)units : 0.0;
  }
  return waves;
}
