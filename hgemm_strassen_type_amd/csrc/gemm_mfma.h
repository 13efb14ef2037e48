// gemm_mfma.hip — classical tiled MFMA GEMM for gfx950 with fused epilogues.
//
// Method (CS336 Lecture 05 notes, Pages 40-42 "tiling"): every workgroup owns one
// BM x BN output tile and walks K in BK = 64 phases, staging an A and a B tile in
// LDS per phase, so each input element is fetched from HBM about N/BN (M/BM) times
// instead of N times.  The epilogue (tilnote.io PingPong GEMM note, mainloop +
// epilogue; CODA section for the RMSNorm statistics and SwiGLU) runs on the fp32
// accumulators in registers before the only store of the tile.
//
// gfx950 mapping:
//   - 256 threads = 4 wave64s in a WAVES_M x WAVES_N grid; each wave owns a
//     (BM/WAVES_M) x (BN/WAVES_N) sub-tile of 32x32 MFMA blocks;
//   - v_mfma_f32_32x32x16_{bf16,f16}: every lane feeds 8 consecutive k of one row
//     of each operand, so both operands sit in LDS with K contiguous (128 bytes per
//     row for BK = 64) and a fragment is one 16-byte LDS read;
//   - the B fragment is passed as the MFMA's first operand and the A fragment as
//     its second, so the accumulator layout gives each lane 4 consecutive output
//     columns of one row (8-byte stores, in-lane row statistics);
//   - operands that are M- or N-contiguous in memory (A transposed, B not) are
//     loaded as 8 x KB blocks and transposed in registers before the LDS store;
//   - LDS rows are XOR-swizzled on 16-byte chunks so fragment reads and both kinds
//     of LDS stores spread over the banks;
//   - two LDS buffers: the global loads of phase k+1 are in flight while phase k
//     runs on the MFMA units, one barrier per phase;
//   - workgroup ids are remapped so that each XCD (ids are dealt round-robin over
//     the 8 XCDs) works on a contiguous, L2-friendly group of tiles.
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace fgemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kRowBytes = kBK * 2;  // one LDS row: 64 16-bit values

// ------------------------------------------------------------------ scalar codecs
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32, RNE
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);    // RNE
}
template <int DT>
__device__ __forceinline__ float to_f32(uint32_t h) {
  return DT == kBF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
}
template <int DT>
__device__ __forceinline__ uint32_t from_f32(float f) {
  return DT == kBF16 ? f32_to_bf16_bits(f) : f32_to_f16_bits(f);
}

// LDS chunk swizzle: 16-byte chunk c of row r lives at chunk c ^ swz(r).
// Consecutive rows (fragment reads) and rows 8 apart (transposed stores) both land
// on distinct chunk positions.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 4)) & 7; }

// --------------------------------------------------------------- configuration
template <int BM_, int BN_, int WAVES_M_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = 4 / WAVES_M_;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int VA = BM / 32;  // 16-byte vectors per thread for the A tile
  static constexpr int VB = BN / 32;  // ... and for the B tile
  static constexpr int LDS_A = BM * kRowBytes, LDS_B = BN * kRowBytes;
  static constexpr int LDS_STAGE = LDS_A + LDS_B;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 block");
};

// ------------------------------------------------------------ operand loading
// Converts 8 packed 16-bit values of type IN to fp16 times `scale` (Strassen
// operands kept as fp16 temporaries).
template <int IN>
__device__ __forceinline__ uint4 convert8(uint4 v, float scale) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float lo = to_f32<IN>(w[p] & 0xffffu) * scale;
    float hi = to_f32<IN>(w[p] >> 16) * scale;
    o[p] = f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Load 8 consecutive 16-bit values starting at p, of which the first `n` exist.
template <bool VEC>
__device__ __forceinline__ uint4 load8(const uint16_t* p, int n) {
  if (VEC && n >= 8) return *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < n) w[j >> 1] |= (uint32_t)p[j] << (16 * (j & 1));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Column map of the B tile.  Plain GEMM: tile column c is global column n0 + c.
// SwiGLU: each wave column of WN tile columns holds WN/2 gate columns followed by
// the WN/2 up columns of the same outputs; `out` is the output column, `g` the
// column of op(B).  Returns the number of valid columns from c on (<= 8 needed).
template <bool SWIGLU, int WN>
__device__ __forceinline__ int bcol_map(int c, int n0, int N, int* g) {
  if (!SWIGLU) {
    *g = n0 + c;
    return N - (n0 + c);
  }
  constexpr int half = WN / 2;
  int wn = c / WN, cc = c % WN;
  int out = n0 + wn * half + (cc % half);
  *g = cc < half ? out : N + out;
  return N - out;
}

template <class CFG, int DT, bool AK, bool BKC, int EPI, bool VEC, bool STR, int INDT>
struct GemmTile {
  static constexpr int BM = CFG::BM, BN = CFG::BN;
  static constexpr bool SWIGLU = EPI == kEpiSwiGLU;

  // ---- A: op(A) is M x K.  AK: stored M x K (K contiguous); else stored K x M.
  __device__ __forceinline__ static void load_a(const GemmProblem& P, int m0, int k0, int tid,
                                                float sa, uint4 (&r)[CFG::VA]) {
    const uint16_t* A = static_cast<const uint16_t*>(P.A);
    if (AK) {
#pragma unroll
      for (int i = 0; i < CFG::VA; ++i) {
        int idx = tid + i * kThreads, row = idx >> 3, c = idx & 7;
        int gm = m0 + row, gk = k0 + c * 8;
        int n = (gm < P.M) ? P.K - gk : 0;
        r[i] = n > 0 ? load8<VEC>(A + (int64_t)gm * P.lda + gk, n) : make_uint4(0, 0, 0, 0);
        if (STR && P.cvt_a) r[i] = convert8<INDT>(r[i], sa);
      }
    } else {
      constexpr int KB = CFG::VA, CHUNKS = BM / 8;
      int cm = tid % CHUNKS, kg = tid / CHUNKS;
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        int gk = k0 + kg * KB + j, gm = m0 + cm * 8;
        int n = (gk < P.K) ? P.M - gm : 0;
        r[j] = n > 0 ? load8<VEC>(A + (int64_t)gk * P.lda + gm, n) : make_uint4(0, 0, 0, 0);
        if (STR && P.cvt_a) r[j] = convert8<INDT>(r[j], sa);
      }
    }
  }

  // ---- B: op(B) is K x Nb.  BKC: stored Nb x K (K contiguous); else stored K x Nb.
  __device__ __forceinline__ static void load_b(const GemmProblem& P, int n0, int k0, int tid,
                                                float sb, uint4 (&r)[CFG::VB]) {
    const uint16_t* B = static_cast<const uint16_t*>(P.B);
    if (BKC) {
#pragma unroll
      for (int i = 0; i < CFG::VB; ++i) {
        int idx = tid + i * kThreads, row = idx >> 3, c = idx & 7;
        int g;
        int valid = bcol_map<SWIGLU, CFG::WN>(row, n0, P.N, &g);
        int gk = k0 + c * 8;
        int n = valid > 0 ? P.K - gk : 0;
        r[i] = n > 0 ? load8<VEC>(B + (int64_t)g * P.ldb + gk, n) : make_uint4(0, 0, 0, 0);
        if (STR && P.cvt_b) r[i] = convert8<INDT>(r[i], sb);
      }
    } else {
      constexpr int KB = CFG::VB, CHUNKS = BN / 8;
      int cn = tid % CHUNKS, kg = tid / CHUNKS;
      int g;
      int valid = bcol_map<SWIGLU, CFG::WN>(cn * 8, n0, P.N, &g);
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        int gk = k0 + kg * KB + j;
        int n = (gk < P.K) ? valid : 0;
        r[j] = n > 0 ? load8<VEC>(B + (int64_t)gk * P.ldb + g, n) : make_uint4(0, 0, 0, 0);
        if (STR && P.cvt_b) r[j] = convert8<INDT>(r[j], sb);
      }
    }
  }

  // ---- LDS stores.  K-contiguous operand: one 16-byte chunk per vector.
  template <int ROWS, int V>
  __device__ __forceinline__ static void store_kcontig(uint8_t* lds, int tid, const uint4 (&r)[V]) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      int idx = tid + i * kThreads, row = idx >> 3, c = idx & 7;
      *reinterpret_cast<uint4*>(lds + row * kRowBytes + ((c ^ swz(row)) << 4)) = r[i];
    }
  }

  // MN-contiguous operand: KB rows of 8 values -> 8 LDS rows of KB values.
  template <int ROWS, int KB>
  __device__ __forceinline__ static void store_transposed(uint8_t* lds, int tid,
                                                          const uint4 (&r)[KB]) {
    constexpr int CHUNKS = ROWS / 8;
    int cm = tid % CHUNKS, kg = tid / CHUNKS;
    int kel = kg * KB;                 // first k (element) this thread holds
    int chunk = kel >> 3, within = (kel & 7) * 2;
    uint32_t w[KB][4];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      w[j][0] = r[j].x; w[j][1] = r[j].y; w[j][2] = r[j].z; w[j][3] = r[j].w;
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      int row = cm * 8 + n;
      uint8_t* dst = lds + row * kRowBytes + ((chunk ^ swz(row)) << 4) + within;
      const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
      if constexpr (KB == 1) {
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(w[0][n >> 1] >> (16 * (n & 1)));
      } else {
        uint32_t o[KB / 2];
#pragma unroll
        for (int q = 0; q < KB / 2; ++q)
          o[q] = __builtin_amdgcn_perm(w[2 * q + 1][n >> 1], w[2 * q][n >> 1], sel);
        if constexpr (KB == 2) {
          *reinterpret_cast<uint32_t*>(dst) = o[0];
        } else if constexpr (KB == 4) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
        } else {
          *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  }

  __device__ __forceinline__ static void store_a(uint8_t* lds, int tid, const uint4 (&r)[CFG::VA]) {
    if (AK) store_kcontig<BM, CFG::VA>(lds, tid, r);
    else store_transposed<BM, CFG::VA>(lds, tid, r);
  }
  __device__ __forceinline__ static void store_b(uint8_t* lds, int tid, const uint4 (&r)[CFG::VB]) {
    if (BKC) store_kcontig<BN, CFG::VB>(lds, tid, r);
    else store_transposed<BN, CFG::VB>(lds, tid, r);
  }

  // ---- one BK = 64 phase on the MFMA units
  __device__ __forceinline__ static void compute(const uint8_t* la, const uint8_t* lb, int wm,
                                                 int wn, int lane,
                                                 f32x16_t (&acc)[CFG::FM][CFG::FN]) {
    const int lr = lane & 31, hk = lane >> 5;
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int chunk = 2 * s + hk;
      uint4 af[CFG::FM], bfr[CFG::FN];
#pragma unroll
      for (int f = 0; f < CFG::FM; ++f) {
        int row = wm * CFG::WM + f * 32 + lr;
        af[f] = *reinterpret_cast<const uint4*>(la + row * kRowBytes + ((chunk ^ swz(row)) << 4));
      }
#pragma unroll
      for (int f = 0; f < CFG::FN; ++f) {
        int row = wn * CFG::WN + f * 32 + lr;
        bfr[f] = *reinterpret_cast<const uint4*>(lb + row * kRowBytes + ((chunk ^ swz(row)) << 4));
      }
#pragma unroll
      for (int i = 0; i < CFG::FM; ++i)
#pragma unroll
        for (int j = 0; j < CFG::FN; ++j) {
          if constexpr (DT == kBF16) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, bfr[j]), __builtin_bit_cast(bf16x8_t, af[i]),
                acc[i][j], 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8_t, bfr[j]), __builtin_bit_cast(f16x8_t, af[i]),
                acc[i][j], 0, 0, 0);
          }
        }
    }
  }

  // ---- epilogues.  Lane layout of acc[i][j][4q+s]: row = wave row base + 32i +
  // (lane & 31), column = wave column base + 32j + 8q + 4*(lane >> 5) + s.
  __device__ __forceinline__ static void epilogue(const GemmProblem& P, int m0, int n0, int tn,
                                                  int wm, int wn, int lane,
                                                  f32x16_t (&acc)[CFG::FM][CFG::FN]) {
    const int lr = lane & 31, h = lane >> 5;
    if constexpr (EPI == kEpiStore32) {
      float* C = static_cast<float*>(P.C);
#pragma unroll
      for (int i = 0; i < CFG::FM; ++i) {
        int row = m0 + wm * CFG::WM + i * 32 + lr;
        if (row >= P.M) continue;
#pragma unroll
        for (int j = 0; j < CFG::FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            int col = n0 + wn * CFG::WN + j * 32 + 8 * q + 4 * h;
            float* dst = C + (int64_t)row * P.ldc + col;
            if (VEC && col + 4 <= P.N) {
              *reinterpret_cast<float4*>(dst) = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                            acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            } else {
#pragma unroll
              for (int s = 0; s < 4; ++s)
                if (col + s < P.N) dst[s] = acc[i][j][4 * q + s];
            }
          }
      }
      return;
    }
    uint16_t* C = static_cast<uint16_t*>(P.C);
    const uint16_t* Cin = static_cast<const uint16_t*>(P.Cin);
    const bool use_beta = (P.flags & kFlagBeta) != 0;
    if constexpr (EPI == kEpiStore16) {
      const bool use_bias = (P.flags & kFlagBias) != 0;
      const bool use_ss = (P.flags & kFlagRowSumSq) != 0;
      const uint16_t* bias = static_cast<const uint16_t*>(P.bias);
#pragma unroll
      for (int i = 0; i < CFG::FM; ++i) {
        int row = m0 + wm * CFG::WM + i * 32 + lr;
        bool rv = row < P.M;
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < CFG::FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            int col = n0 + wn * CFG::WN + j * 32 + 8 * q + 4 * h;
            int nv = P.N - col;
            if (!rv || nv <= 0) continue;
            float v[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) v[s] = P.alpha * acc[i][j][4 * q + s];
            const int64_t off = (int64_t)row * P.ldc + col;
            if (use_beta) {
              uint32_t c[4];
              if (VEC && nv >= 4) {
                uint2 cv = *reinterpret_cast<const uint2*>(Cin + off);
                c[0] = cv.x & 0xffff; c[1] = cv.x >> 16; c[2] = cv.y & 0xffff; c[3] = cv.y >> 16;
              } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) c[s] = s < nv ? Cin[off + s] : 0;
              }
#pragma unroll
              for (int s = 0; s < 4; ++s) v[s] += P.beta * to_f32<DT>(c[s]);
            }
            if (use_bias) {
#pragma unroll
              for (int s = 0; s < 4; ++s) v[s] += s < nv ? to_f32<DT>(bias[col + s]) : 0.f;
            }
            uint32_t o[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              o[s] = from_f32<DT>(v[s]);
              float r = to_f32<DT>(o[s]);
              if (s < nv) ss += r * r;
            }
            if (VEC && nv >= 4) {
              *reinterpret_cast<uint2*>(C + off) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
            } else {
#pragma unroll
              for (int s = 0; s < 4; ++s)
                if (s < nv) C[off + s] = (uint16_t)o[s];
            }
          }
        if (use_ss) {
          ss += __shfl_xor(ss, 32);
          if (h == 0 && rv) P.ss_partial[(int64_t)(tn * CFG::WAVES_N + wn) * P.M + row] = ss;
        }
      }
    } else {  // kEpiSwiGLU: output tile is BM x BN/2
      constexpr int HF = CFG::FN / 2;
      const int out0 = n0 + wn * (CFG::WN / 2);
#pragma unroll
      for (int i = 0; i < CFG::FM; ++i) {
        int row = m0 + wm * CFG::WM + i * 32 + lr;
        if (row >= P.M) continue;
        float r = rsqrtf(P.rms_ss[row] * P.rms_inv_n + P.rms_eps) * P.alpha;
#pragma unroll
        for (int j = 0; j < HF; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            int col = out0 + j * 32 + 8 * q + 4 * h;
            int nv = P.N - col;
            if (nv <= 0) continue;
            float v[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              float g = r * acc[i][j][4 * q + s];
              float u = r * acc[i][j + HF][4 * q + s];
              v[s] = g / (1.f + __expf(-g)) * u;
            }
            const int64_t off = (int64_t)row * P.ldc + col;
            if (use_beta) {
#pragma unroll
              for (int s = 0; s < 4; ++s) v[s] += s < nv ? P.beta * to_f32<DT>(Cin[off + s]) : 0.f;
            }
            uint32_t o[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) o[s] = from_f32<DT>(v[s]);
            if (VEC && nv >= 4) {
              *reinterpret_cast<uint2*>(C + off) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
            } else {
#pragma unroll
              for (int s = 0; s < 4; ++s)
                if (s < nv) C[off + s] = (uint16_t)o[s];
            }
          }
      }
    }
  }
};

// Workgroup id -> tile.  Ids are dealt round-robin over the 8 XCDs; renumber so
// each XCD gets a contiguous range, then walk tiles in groups of 8 tile-rows so
// that tiles running together share A rows and B columns in L2.
__device__ __forceinline__ void tile_of(int bid, int nblk, int tiles_m, int tiles_n, int* tm,
                                        int* tn) {
  int xcd = bid & 7, idx = bid >> 3;
  int base = nblk >> 3, rem = nblk & 7;
  int pid = xcd * base + (xcd < rem ? xcd : rem) + idx;
  constexpr int G = 8;
  int per_group = G * tiles_n;
  int group = pid / per_group;
  int first = group * G;
  int gsz = tiles_m - first < G ? tiles_m - first : G;
  int in = pid - group * per_group;
  *tm = first + in % gsz;
  *tn = in / gsz;
}

template <class CFG, int DT, bool AK, bool BKC, int EPI, bool VEC, bool STR, int INDT>
__global__ __launch_bounds__(kThreads) void gemm_mfma_kernel(GemmBatch batch) {
  using T = GemmTile<CFG, DT, AK, BKC, EPI, VEC, STR, INDT>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * CFG::LDS_STAGE];
  const GemmProblem& P = batch.p[blockIdx.z];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / CFG::WAVES_N, wn = wave % CFG::WAVES_N;
  const int out_bn = EPI == kEpiSwiGLU ? CFG::BN / 2 : CFG::BN;
  const int tiles_m = (P.M + CFG::BM - 1) / CFG::BM;
  const int tiles_n = (P.N + out_bn - 1) / out_bn;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, &tm, &tn);
  if (tm >= tiles_m || tn >= tiles_n) return;
  const int m0 = tm * CFG::BM, n0 = tn * out_bn;
  const float sa = (STR && P.cvt_a) ? *P.scale_a : 1.f;
  const float sb = (STR && P.cvt_b) ? *P.scale_b : 1.f;

  f32x16_t acc[CFG::FM][CFG::FN];
#pragma unroll
  for (int i = 0; i < CFG::FM; ++i)
#pragma unroll
    for (int j = 0; j < CFG::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int ktiles = (P.K + kBK - 1) / kBK;
  if (ktiles > 0) {
    uint4 ra[CFG::VA], rb[CFG::VB];
    T::load_a(P, m0, 0, tid, sa, ra);
    T::load_b(P, n0, 0, tid, sb, rb);
    T::store_a(smem, tid, ra);
    T::store_b(smem + CFG::LDS_A, tid, rb);
    __syncthreads();
    for (int kt = 0; kt < ktiles; ++kt) {
      uint8_t* cur = smem + (kt & 1) * CFG::LDS_STAGE;
      uint8_t* nxt = smem + ((kt + 1) & 1) * CFG::LDS_STAGE;
      const bool more = kt + 1 < ktiles;
      if (more) {
        T::load_a(P, m0, (kt + 1) * kBK, tid, sa, ra);
        T::load_b(P, n0, (kt + 1) * kBK, tid, sb, rb);
      }
      T::compute(cur, cur + CFG::LDS_A, wm, wn, lane, acc);
      if (more) {
        T::store_a(nxt, tid, ra);
        T::store_b(nxt + CFG::LDS_A, tid, rb);
      }
      __syncthreads();
    }
  }
  T::epilogue(P, m0, n0, tn, wm, wn, lane, acc);
}

// ------------------------------------------------------------------ launching
using Cfg256 = TileCfg<256, 256, 2>;
using Cfg128 = TileCfg<128, 128, 2>;
using Cfg64 = TileCfg<64, 128, 2>;
using Cfg32 = TileCfg<32, 128, 1>;

template <class CFG, int DT, bool AK, bool BKC, int EPI, bool VEC, bool STR, int INDT>
static hipError_t launch_t(const GemmBatch& b, hipStream_t s) {
  int maxtiles = 0;
  for (int i = 0; i < b.count; ++i) {
    int out_bn = EPI == kEpiSwiGLU ? CFG::BN / 2 : CFG::BN;
    int t = ((b.p[i].M + CFG::BM - 1) / CFG::BM) * ((b.p[i].N + out_bn - 1) / out_bn);
    if (t > maxtiles) maxtiles = t;
  }
  if (maxtiles == 0) return hipSuccess;
  dim3 grid(maxtiles, 1, b.count);
  hipLaunchKernelGGL((gemm_mfma_kernel<CFG, DT, AK, BKC, EPI, VEC, STR, INDT>), grid,
                     dim3(kThreads), 0, s, b);
  return hipGetLastError();
}

}  // namespace fgemm
