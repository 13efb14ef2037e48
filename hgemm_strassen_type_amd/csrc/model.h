// model.h — the analytic time model shared by selection and dispatch (host only).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fgemm.h"

namespace fgemm {

struct TileInfo {
  int tile;        // kernel tile id (its index in kTiles)
  int bm, bn;      // macro-tile (bn MFMA columns; SwiGLU writes bn/2 outputs)
  int bk;          // K depth of one pipeline phase
  double rel_eta;  // steady-state MFMA efficiency relative to the 256x256 tile
  int waves_n;     // waves across the tile's columns (row-sum partials per tile)
  int swiglu;      // the SwiGLU epilogue runs on it (each wave holds both halves)
  int one_row;     // offered only when M fits one tile row (decode shapes)
};

constexpr int kNumTiles = 5;
extern const TileInfo kTiles[kNumTiles];
// Strassen workspace header: the two scales, then the partial maxima of A and B.
constexpr size_t kScaleHeaderBytes = 256 + 2 * 4096 * 4;

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
int64_t ceil_div(int64_t a, int64_t b);
double overlap(double a, double b);
// HBM bandwidth (bytes/s) that `blocks` concurrently streaming workgroups reach.
double stream_bw(const fgemm_model_t& md, int64_t blocks);

void model_defaults(fgemm_model_t* m, int cus, double clock_ghz, double device_bytes);

double classical_time_us(const fgemm_model_t& md, const TileInfo& t, int64_t M, int64_t N,
                         int64_t K, int64_t Nb, int64_t out_bn, int count, double in_bytes,
                         double out_bytes, int beta);
// Tile of least predicted time among tile ids 0..max_tile.
int best_tile(const fgemm_model_t& md, int64_t M, int64_t N, int64_t K, int swiglu, int count,
              double in_bytes, double out_bytes, int beta, double* t_us,
              int max_tile = kNumTiles - 1);
// Split-K plan of `splits` K slices with an fp32 finalize pass.
double splitk_time_us(const fgemm_model_t& md, const TileInfo& t, int64_t M, int64_t N,
                      int64_t K, int splits, int beta);
// Table-driven block schemes: op(A) in mb x kb blocks, op(B) in kb x nb, C in mb x nb;
// R products P_r = (sum_a U[r*mb*kb + a] A_a)(sum_b V[r*kb*nb + b] B_b) and output
// blocks C_c = sum_r W[c*R + r] P_r (blocks numbered row by row).  Null for the 2 x 2
// recursive variants, which have their own chained kernels.
struct BlockScheme {
  int mb, kb, nb, R;
  const signed char* U;
  const signed char* V;
  const signed char* W;
};
const BlockScheme* block_scheme(int variant);
size_t strassen_workspace(int64_t M, int64_t N, int64_t K, int depth, int variant);
// Predicted normwise error against the exactly rounded result (depth 0: classical).
double predicted_rel_err(int dtype, int variant, int depth);
double classical_dtype_rate(int dtype);
double strassen_time_us(const fgemm_model_t& md, int64_t M, int64_t N, int64_t K, int depth,
                        int variant, int beta, int* sub_tile);

}  // namespace fgemm
