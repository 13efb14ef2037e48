// gemm_mfma.h — classical tiled MFMA GEMM for gfx950 with fused epilogues.
//
// Method (CS336 Lecture 05 notes, Pages 40-42 "tiling"): every workgroup owns one
// BM x BN output tile and walks K in BK-deep phases, staging an A and a B tile in
// LDS per phase, so each input element is fetched from HBM about N/BN (M/BM) times
// instead of N times.  The epilogue (tilnote.io PingPong GEMM note, mainloop +
// epilogue; CODA section for the RMSNorm statistics and SwiGLU) runs on the fp32
// accumulators in registers before the only store of the tile.
//
// gfx950 mapping:
//   - NT = 64 * WAVES_M * WAVES_N threads; each wave64 owns a (BM/WAVES_M) x
//     (BN/WAVES_N) sub-tile of MI x MI blocks of v_mfma_f32_32x32x16 (MI = 32) or
//     v_mfma_f32_16x16x32 (MI = 16), bf16 or f16;
//   - the B fragment is passed as the MFMA's first operand and the A fragment as
//     its second, so the accumulator layout gives each lane groups of 4
//     consecutive output columns of one row (in-lane row statistics);
//   - tiles reach LDS through global_load_lds_dwordx4 (16 bytes per lane straight
//     into LDS, no registers, asynchronous): a ring of STAGES phase buffers keeps
//     the loads of STAGES-1 phases in flight while one phase feeds the MFMAs; the
//     loads into a stage are issued as soon as the barrier that frees it has
//     passed, one after each MFMA of the last k-step of the phase that read it;
//   - LDS keeps each operand in its memory layout.  K-contiguous operands (A not
//     transposed, B transposed) are rows of BK values read as one 16-byte fragment
//     per lane; M/N-contiguous operands (A transposed, B not) are BK rows of BM or
//     BN values read with ds_read_b64_tr_b16, whose 16-lane groups hand every lane
//     one column of four consecutive rows, i.e. four consecutive k;
//   - 16-byte chunks are XOR-swizzled per row so that the fragment reads of both
//     kinds hit 64 distinct banks; the direct loads fetch each lane's chunk from
//     the swizzled source position, so LDS is written densely in 1 KB blocks;
//   - edge tiles (partial M, N or K) load the same slots through registers with
//     bounds tests and zero fill, and store them to the same LDS positions;
//   - the grid is persistent (as many workgroups as the device holds), each
//     looping over tiles; workgroups of one XCD (ids are dealt round-robin over
//     the 8 XCDs) take a contiguous, L2-friendly run of tiles per round, and a
//     tile's first loads are issued by its predecessor before that one's epilogue;
//   - with aligned operands the epilogues (plain, fp32 slices, SwiGLU, activation or
//     rotary embedding) stage their results through LDS so that every lane stores
//     (and reads beta*C as) 8 consecutive columns: whole 128-byte lines.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "epilogue_ops.h"
#include "internal.h"

namespace fgemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
// Native vectors, not HIP's uint4/uint2 structs: struct copies are lowered through
// private memory and lose their place in the schedule.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

#define FGEMM_LDS __attribute__((address_space(3)))
#define FGEMM_GLOBAL __attribute__((address_space(1)))

// Phase boundary: neither the IR optimizer (memory clobber) nor the machine
// scheduler (sched_barrier) moves instructions across it.
#define FGEMM_PHASE_FENCE()            \
  do {                                 \
    asm volatile("" ::: "memory");     \
    __builtin_amdgcn_sched_barrier(0); \
  } while (0)

// ------------------------------------------------------------------ scalar codecs
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);  // RNE
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
// Two values rounded (RNE) and packed low | high << 16: one v_cvt_pk_{bf16,f16}_f32.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  if constexpr (DT == kBF16) {
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, h2));
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, h2));
  }
}

// s_waitcnt immediate for "vector memory count <= n", other counters unconstrained
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// --------------------------------------------------------------- configuration
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int STAGES_, int OCC_ = 1,
          int MI_ = 32>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int OCC = OCC_;  // workgroups per CU the register budget is sized for
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  // MFMA shape: MI x MI output blocks, KSTEP-deep (v_mfma_f32_32x32x16 or _16x16x32);
  // either way a lane feeds 8 consecutive k of one row/column per operand and holds
  // ACC accumulators, in groups of 4 consecutive output columns of one row.
  static constexpr int MI = MI_;
  static constexpr int KSTEP = MI == 32 ? 16 : 32;
  static constexpr int ACC = MI * MI / 64;
  using AccT = typename std::conditional<MI == 32, f32x16_t, f32x4_t>::type;
  static constexpr int FM = WM / MI, FN = WN / MI;
  static constexpr int STEPS = BK / KSTEP;  // MFMA k-steps per phase
  static_assert(MI == 32 || MI == 16, "MFMA shape");
  static_assert(STEPS == 2 || STEPS == 4, "k-steps per phase");
  static constexpr int LDS_A = BM * BK * 2, LDS_B = BN * BK * 2;
  static constexpr int LDS_STAGE = LDS_A + LDS_B;
  static constexpr int QA = LDS_A / 1024, QB = LDS_B / 1024;  // 1 KB load slots per phase
  static constexpr int QAW = (QA + NW - 1) / NW, QBW = (QB + NW - 1) / NW;  // per wave
  static_assert(FM >= 1 && FN >= 1 && WM % 32 == 0, "wave tile: whole MFMA blocks, 32-row bands");
  static_assert(BK == 32 || BK == 64, "phase depth");
  static_assert(LDS_A % 1024 == 0 && LDS_B % 1024 == 0, "1 KB load slots");
  // Epilogue staging: each wave transposes 32 x EPI_CW fp32 blocks through its own
  // EPI_CW*128-byte region of the last stage (free at the end of a tile; the first
  // STAGES-1 stages may already hold the next tile's first phases).
  static constexpr int EPI_CW = (WN % 64 == 0 && NW * 32 * 64 * 4 <= LDS_STAGE) ? 64 : 32;
  static constexpr int EPI_WAVE_BYTES = 32 * EPI_CW * 4;
  static constexpr int EPI_OFF = (STAGES - 1) * LDS_STAGE;
  static constexpr int SMEM = STAGES * LDS_STAGE > EPI_OFF + NW * EPI_WAVE_BYTES
                                  ? STAGES * LDS_STAGE
                                  : EPI_OFF + NW * EPI_WAVE_BYTES;
  static_assert(STAGES >= 2 && SMEM <= 160 * 1024, "LDS budget");
  static_assert(WN % EPI_CW == 0, "epilogue blocks");
};

// ------------------------------------------------------------------ LDS layout
// K-contiguous operand: R rows of BK values (BK*2 bytes), chunk c of row r at
// chunk c ^ swz_k(r).  Fragment reads take 16 consecutive rows per bank cycle; the
// swizzle depends on r mod 16 only, so fragments 16 or 32 rows apart share it and
// their addresses differ by a constant (one base register per operand).
template <int BK>
__device__ __forceinline__ int swz_k(int r) {
  return BK == 32 ? ((r >> 2) & 3) : ((r >> 1) & 7);
}
// M/N-contiguous operand: BK rows of R values (R*2 bytes), chunk c of row k at
// chunk c ^ swz_mn(k); a transposed read takes rows k..k+3 (k % 4 == 0) of two
// consecutive chunks per 16 lanes, and the 32 lanes served together read either
// 4 more chunks of the same rows (32x32 blocks) or the same 2 chunks of rows
// k+8..k+11 (16x16 blocks): bit 3 of k moves those by 2 chunks.
template <int R>
__device__ __forceinline__ int swz_mn(int k) {
  return (4 * (k & 3) + 2 * ((k >> 3) & 1)) & (R / 8 - 1);
}

// Column map of the B tile.  Plain GEMM: tile column c is global column n0 + c.
// SwiGLU: each wave column of WN tile columns holds WN/2 gate columns followed by
// the WN/2 up columns of the same outputs; `*g` is the column of op(B).  Returns
// the number of valid columns from c on.
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

// Load 8 consecutive 16-bit values starting at p, of which the first `n` exist.
__device__ __forceinline__ v4u load8_checked(const uint16_t* p, int n, bool vec) {
  if (vec && n >= 8) return *reinterpret_cast<const v4u*>(p);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < n) w[j >> 1] |= (uint32_t)p[j] << (16 * (j & 1));
  return v4u{w[0], w[1], w[2], w[3]};
}

// DT is the MFMA input type: kF16 or kBF16, or an 8-bit pair code f8_code(fa, fb)
// (operands stored as bytes and addressed here as pairs of bytes, i.e. in 16-bit
// units: BK = 64 units is 128 8-bit values).  ODT is the 16-bit output type.
template <class CFG, int DT, bool AK, bool BKC, int EPI, bool VEC, int ODT = DT>
struct GemmTile {
  static constexpr int BM = CFG::BM, BN = CFG::BN, BK = CFG::BK, NT = CFG::NT;
  // 8-bit inputs: v_mfma_scale_f32_32x32x64_f8f6f4 (64 k a step) or _16x16x128
  // (128 k), fed with two 16-byte chunks of one row per lane (FC).  The instruction
  // takes its k as two halves: lane group g (lane / MI) holds k 16g..16g+15 of the
  // first half in its first chunk and the same k of the second half in its second,
  // so a lane reads chunks g and g + 2 (32x32) or g and g + 4 (16x16) of the step,
  // CHUNK2 bytes apart, and the hardware's k order is the memory order (which the MX
  // block scales need: block b is k 32b..32b+31, its scale in lane group b)
  static constexpr bool F8 = DT >= kF8Base;
  // 4-bit inputs (E2M1, two values a byte) through the same instruction: a lane's
  // operand is 16 bytes, 32 values, and lane group g holds k 32g..32g+31 of the
  // step, one whole E8M0 block, in memory order.  That is the 16-bit 32x32x16
  // fragment geometry (lane group g reads the step's 16-byte chunk g), so the
  // K-contiguous fragment addressing serves unchanged, with 128 bytes (256 values,
  // 8 blocks, 4 steps) a row a phase.
  static constexpr bool F4 = DT == kF4MX;
  // MX: one E8M0 scale per 32 values along K for every row of A and B (the 8-bit
  // code's third bit), fed to the MFMA per lane: the lane's 32 bytes are one block
  static constexpr bool MX = DT >= kF8Base + 4;
  static constexpr int FC = F8 && !F4 ? 2 : 1;
  static constexpr int CHUNK2 = CFG::MI == 32 ? 32 : 64;  // F8: XOR offset of the second chunk
  // MX scales in LDS after the stages: per group of 4 phases (16 blocks) the tile's
  // BM + BN rows of 16 scale bytes, two groups (one read while the next arrives)
  static constexpr int MX_OFF = CFG::SMEM;
  static constexpr int MX_BUF = (CFG::BM + CFG::BN) * 16;
  static constexpr int MX_SLOTS_A = CFG::BM / 64, MX_SLOTS_B = CFG::BN / 64;
  // 1 KB scale slots (64 rows of 16 bytes) a wave loads: slot q = wave + NW*i
  static constexpr int MX_SW = (MX_SLOTS_A + MX_SLOTS_B + CFG::NW - 1) / CFG::NW;
  // k per MFMA step in 16-bit units (8-bit: 64 or 128 values) and steps per phase
  static constexpr int KSTEP = F4 ? 16 : F8 ? (CFG::MI == 32 ? 32 : 64) : CFG::KSTEP;
  static constexpr int STEPS = CFG::BK / KSTEP;
  // MX: E8M0 blocks of 32 values a step covers (a 16-bit unit is 4 values at 4 bits)
  static constexpr int BPS = F4 ? KSTEP / 8 : KSTEP / 16;
  // MX: blocks a phase covers, and phases a 16-block scale group covers
  static constexpr int BPP = STEPS * BPS;
  static constexpr int PPG = MX ? 16 / BPP : 1;
  static_assert(!F8 || (AK && BKC && CFG::BK == 64 && EPI == kEpiStore16),
                "8/4-bit inputs: K-contiguous operands, 128 bytes a row a phase, the 16-bit "
                "store epilogue");
  static_assert(!MX || BPP * PPG == 16, "whole phases a scale group");
  static_assert(!F4 || (CFG::MI == 32 && MX), "4-bit inputs: 32x32x64 MFMAs with block scales");
  // gate/up column pairs: the SwiGLU epilogue and its backward
  static constexpr bool SWIGLU = EPI == kEpiSwiGLU || EPI == kEpiSwiGLUBwd;
  using Acc = typename CFG::AccT;
  static constexpr int OUT_BN = SWIGLU ? BN / 2 : BN;

  // ============================================================ load slots
  // Slot q of an operand is the 1 KB block [q*1024, q*1024 + 1024) of its LDS region;
  // lane l of the wave that owns it moves the 16 bytes at q*1024 + 16*l.  slot_src
  // gives the source of that chunk: `row` (operand row for K-contiguous, k for
  // M/N-contiguous) and the logical 16-byte chunk `c` inside the row.
  template <bool KCONTIG, int R>
  __device__ __forceinline__ static void slot_src(int q, int lane, int* row, int* c) {
    constexpr int CPR = KCONTIG ? BK / 8 : R / 8;  // chunks per LDS row
    const int e = q * 64 + lane;
    const int r = e / CPR, p = e % CPR;
    *row = r;
    *c = p ^ (KCONTIG ? swz_k<BK>(r) : swz_mn<R>(r));
  }

  // Per-lane byte offsets of the fast path (relative to a per-phase uniform base).
  struct LoadAddr {
    uint32_t a[CFG::QAW];
    uint32_t b[CFG::QBW];
    uint32_t mx[MX ? MX_SW : 1];  // MX: the wave's scale slots (row of A or B times its ld)
  };

  // Rows and columns beyond M or N (edge tiles) are clamped onto the last valid
  // ones: they load real memory, feed MFMA rows/columns the epilogue never stores,
  // and keep the fast path open for partial tiles whose K is a whole number of phases.
  // For M/N-contiguous operands the caller guarantees that the edge dimension is a
  // multiple of 8 on such tiles, so a chunk is either wholly valid (never moved) or
  // wholly past the edge (moved onto the last 8 valid values, never stored).
  __device__ __forceinline__ static void load_addr(const GemmProblem& P, int m0, int n0,
                                                   int wave, int lane_in, LoadAddr& la) {
    // recomputed per tile: an opaque lane id keeps the lane-only parts from being
    // hoisted out of the tile loop and held in registers across the main loop
    int lane = lane_in;
    asm volatile("" : "+v"(lane));
    if constexpr (MX) {
      // slot q < MX_SLOTS_A: rows 64q.. of A's tile; then rows of B's (clamped)
#pragma unroll
      for (int i = 0; i < MX_SW; ++i) {
        const int q = wave + CFG::NW * i;
        la.mx[i] = 0;
        if (q < MX_SLOTS_A) {
          const int r = m0 + 64 * q + lane;
          la.mx[i] = (uint32_t)((int64_t)(r < P.M ? r : P.M - 1) * P.ld_mxa);
        } else if (q < MX_SLOTS_A + MX_SLOTS_B) {
          const int r = n0 + 64 * (q - MX_SLOTS_A) + lane;
          la.mx[i] = (uint32_t)((int64_t)(r < P.N ? r : P.N - 1) * P.ld_mxb);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CFG::QAW; ++i) {
      int q = wave + CFG::NW * i, row, c;
      slot_src<AK, BM>(q < CFG::QA ? q : 0, lane, &row, &c);
      if (AK) {  // base = A + m0 rows + k0; row = m - m0
        int r = m0 + row < P.M ? row : P.M - 1 - m0;
        la.a[i] = (uint32_t)((int64_t)r * P.lda * 2 + c * 16);
      } else {   // base = A + k0 rows + m0; row = k, columns m0 + 8c .. +7
        int mc = m0 + 8 * c + 8 <= P.M ? 8 * c : P.M - 8 - m0;
        la.a[i] = (uint32_t)((int64_t)row * P.lda * 2 + (int64_t)mc * 2);
      }
    }
#pragma unroll
    for (int i = 0; i < CFG::QBW; ++i) {
      int q = wave + CFG::NW * i, row, c;
      slot_src<BKC, BN>(q < CFG::QB ? q : 0, lane, &row, &c);
      int g;
      if (BKC) {  // row = tile column n: global row g of B (stored Nb x K)
        int valid = bcol_map<SWIGLU, CFG::WN>(row, n0, P.N, &g);
        if (valid <= 0) g = SWIGLU ? 0 : P.N - 1;
        la.b[i] = (uint32_t)((int64_t)g * P.ldb * 2 + c * 16);
      } else {    // row = k, chunk c = tile columns 8c..8c+7
        int valid = bcol_map<SWIGLU, CFG::WN>(c * 8, n0, P.N, &g);
        if (valid < 8) g -= 8 - valid;  // shift the chunk back inside its column block
        la.b[i] = (uint32_t)((int64_t)row * P.ldb * 2 + (int64_t)g * 2);
      }
    }
  }

  // The operand pointers and leading dimensions the direct loads use, read once per
  // tile into (scalar) registers: the phase fences would otherwise make the
  // compiler fetch them from the argument block again in every phase.
  struct Src {
    const char* A;
    const char* B;
    int64_t lda, ldb;
    const char* mxa;  // MX scale arrays
    const char* mxb;
  };
  __device__ __forceinline__ static Src src_of(const GemmProblem& P) {
    Src r;
    r.A = static_cast<const char*>(P.A);
    r.B = static_cast<const char*>(P.B);
    r.lda = P.lda;
    r.ldb = P.ldb;
    r.mxa = static_cast<const char*>(P.mx_a);
    r.mxb = static_cast<const char*>(P.mx_b);
    return r;
  }

  // MX: scale group g (blocks 16g..16g+15, phases PPG*g..PPG*g+PPG-1) of this wave's
  // slot into buffer g % 2.
  __device__ __forceinline__ static void issue_scales(const Src& S, int g, int wave,
                                                      const LoadAddr& la, uint8_t* smem) {
    if constexpr (MX) {
#pragma unroll
      for (int i = 0; i < MX_SW; ++i) {
        const int q = wave + CFG::NW * i;
        if (q >= MX_SLOTS_A + MX_SLOTS_B) break;
        const char* base = uniform_ptr((q < MX_SLOTS_A ? S.mxa : S.mxb) + 16 * g);
        lds_dma(base, la.mx[i], lds_addr(smem + MX_OFF + (g & 1) * MX_BUF + q * 1024));
      }
    }
  }

  // Uniform byte base of phase kt.
  __device__ __forceinline__ static const char* a_base(const Src& S, int m0, int kt) {
    return AK ? S.A + ((int64_t)m0 * S.lda + (int64_t)kt * BK) * 2
              : S.A + ((int64_t)kt * BK * S.lda + m0) * 2;
  }
  __device__ __forceinline__ static const char* b_base(const Src& S, int kt) {
    return BKC ? S.B + (int64_t)kt * BK * 2 : S.B + (int64_t)kt * BK * S.ldb * 2;
  }

  // One global_load_lds_dwordx4: 64 lanes x 16 bytes from gbase + voff (per lane)
  // to LDS [lds, lds + 1 KB).  Written as assembly so that the compiler does not see
  // an LDS write it cannot disambiguate from the fragment reads (it would wait for
  // every load in flight before each of them); the ring's own vmcnt waits order
  // them instead.  M0 carries the LDS address; one wait state after writing it.
  __device__ __forceinline__ static void lds_dma(const char* gbase, uint32_t voff, uint32_t lds) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(gbase)
                 : "memory", "m0");
#pragma clang diagnostic pop
  }

  __device__ __forceinline__ static uint32_t lds_addr(const uint8_t* p) {
    return (uint32_t)(uintptr_t)(const FGEMM_LDS uint8_t*)p;
  }

  // A wave-uniform pointer, held in scalar registers (the load's base operand).
  __device__ __forceinline__ static const char* uniform_ptr(const char* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
  }

  // Fast path: issue this wave's direct-to-LDS loads of phase kt into `stage`.
  __device__ __forceinline__ static void issue_loads(const Src& S, int m0, int kt, int wave,
                                                     const LoadAddr& la, uint8_t* stage) {
    const char* ab = uniform_ptr(a_base(S, m0, kt));
    const char* bb = uniform_ptr(b_base(S, kt));
    const uint32_t ls = lds_addr(stage);
#pragma unroll
    for (int i = 0; i < CFG::QAW; ++i) {
      const int q = wave + CFG::NW * i;
      if (CFG::QA % CFG::NW == 0 || q < CFG::QA) lds_dma(ab, la.a[i], ls + q * 1024);
    }
#pragma unroll
    for (int i = 0; i < CFG::QBW; ++i) {
      const int q = wave + CFG::NW * i;
      if (CFG::QB % CFG::NW == 0 || q < CFG::QB) lds_dma(bb, la.b[i], ls + CFG::LDS_A + q * 1024);
    }
  }

  // Edge path: the same slots through registers, bounds-tested, zero-filled.
  __device__ __forceinline__ static void load_checked(const GemmProblem& P, int m0, int n0,
                                                      int kt, int wave, int lane,
                                                      v4u (&ra)[CFG::QAW], v4u (&rb)[CFG::QBW]) {
    const uint16_t* A = static_cast<const uint16_t*>(P.A);
    const uint16_t* B = static_cast<const uint16_t*>(P.B);
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < CFG::QAW; ++i) {
      int q = wave + CFG::NW * i, row, c;
      ra[i] = v4u{0u, 0u, 0u, 0u};
      if (q >= CFG::QA) continue;
      slot_src<AK, BM>(q, lane, &row, &c);
      if (AK) {
        int gm = m0 + row, gk = k0 + c * 8;
        int n = gm < P.M ? P.K - gk : 0;
        if (n > 0) ra[i] = load8_checked(A + (int64_t)gm * P.lda + gk, n, VEC);
      } else {
        int gk = k0 + row, gm = m0 + c * 8;
        int n = gk < P.K ? P.M - gm : 0;
        if (n > 0) ra[i] = load8_checked(A + (int64_t)gk * P.lda + gm, n, VEC);
      }
    }
#pragma unroll
    for (int i = 0; i < CFG::QBW; ++i) {
      int q = wave + CFG::NW * i, row, c;
      rb[i] = v4u{0u, 0u, 0u, 0u};
      if (q >= CFG::QB) continue;
      slot_src<BKC, BN>(q, lane, &row, &c);
      int g;
      if (BKC) {
        int valid = bcol_map<SWIGLU, CFG::WN>(row, n0, P.N, &g);
        int gk = k0 + c * 8;
        int n = valid > 0 ? P.K - gk : 0;
        if (n > 0) rb[i] = load8_checked(B + (int64_t)g * P.ldb + gk, n, VEC);
      } else {
        int valid = bcol_map<SWIGLU, CFG::WN>(c * 8, n0, P.N, &g);
        int gk = k0 + row;
        int n = gk < P.K ? valid : 0;
        if (n > 0) rb[i] = load8_checked(B + (int64_t)gk * P.ldb + g, n, VEC);
      }
    }
  }

  __device__ __forceinline__ static void store_checked(uint8_t* stage, int wave, int lane,
                                                       const v4u (&ra)[CFG::QAW],
                                                       const v4u (&rb)[CFG::QBW]) {
#pragma unroll
    for (int i = 0; i < CFG::QAW; ++i) {
      int q = wave + CFG::NW * i;
      if (q < CFG::QA) *reinterpret_cast<v4u*>(stage + q * 1024 + lane * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CFG::QBW; ++i) {
      int q = wave + CFG::NW * i;
      if (q < CFG::QB)
        *reinterpret_cast<v4u*>(stage + CFG::LDS_A + q * 1024 + lane * 16) = rb[i];
    }
  }

  // ============================================================ fragments
  struct Frags {
    v4u a[CFG::FM][FC];
    v4u b[CFG::FN][FC];
  };
  // MX: the E8M0 scales of the lane's blocks for every pair of steps and fragment of
  // a phase: steps 2q and 2q+1 use blocks 4q+g and 4q+2+g of the phase (lane group g,
  // two blocks a step), one aligned dword of the row's scale bytes shifted right by
  // 8g, so they sit in bytes 0 and 2, which the MFMA's op_sel picks (one VGPR and
  // one LDS read for two steps)
  static_assert(!MX || BPS == 2, "block scales: two blocks a step (32x32x64)");
  struct Scales {
    uint32_t a[MX ? (STEPS + 1) / 2 : 1][MX ? CFG::FM : 1];
    uint32_t b[MX ? (STEPS + 1) / 2 : 1][MX ? CFG::FN : 1];
  };

  // Per-lane LDS byte offsets of the fragments at MFMA step 0 (stage-relative).
  // A lane feeds row (lane % MI) of its fragment with k slot lane / MI (8 k each).
  //   K-contiguous: row r = base + MI*f + (lane % MI), chunk (KSTEP/8)*s + lane/MI.
  //   M/N-contiguous: two transposed 8-byte reads per fragment (k 0-3 and 4-7 of
  //   the lane's 8-k slot); in a 16-lane group, lane j reads row kb + j/4 at the
  //   four columns from 4*(j%4) of the group's 16 columns.
  struct FragAddr {
    int a[CFG::FM];
    int b[CFG::FN];
    int sc;    // MX: the lane's row's first scale byte within a group buffer, minus the
               // fragment's rows
    int scsh;  // MX: 8 * lane group: the shift that brings the lane's block to byte 0
  };

  template <bool KCONTIG, int R, int F>
  __device__ __forceinline__ static void frag_base(int wbase, int lane, int base_off,
                                                   int (&out)[F]) {
#pragma unroll
    for (int f = 0; f < F; ++f) {
      constexpr int MI = CFG::MI;
      if (KCONTIG) {
        int r = wbase + f * MI + lane % MI;
        const int c = lane / MI;  // F8: chunk g; chunk g + 4 is CHUNK2 bytes away
        out[f] = base_off + r * (BK * 2) + ((c ^ swz_k<BK>(r)) << 4);
      } else {
        // 16-lane group g: k slot g / (MI/16), columns 16 * (g % (MI/16)) ..
        int g = lane >> 4, j = lane & 15;
        int kr = 8 * (g / (MI / 16)) + (j >> 2);  // row within the k-step
        int col = wbase + f * MI + 16 * (g % (MI / 16)) + 4 * (j & 3);
        out[f] = base_off + kr * (R * 2) + (((col >> 3) ^ swz_mn<R>(kr)) << 4) + (col & 7) * 2;
      }
    }
  }

  __device__ __forceinline__ static void frag_addr(int wm, int wn, int lane, FragAddr& fa) {
    frag_base<AK, BM, CFG::FM>(wm * CFG::WM, lane, 0, fa.a);
    frag_base<BKC, BN, CFG::FN>(wn * CFG::WN, lane, CFG::LDS_A, fa.b);
    fa.sc = (lane % CFG::MI) * 16;
    fa.scsh = 8 * (lane / CFG::MI);
  }

  // Offset of step s from step 0.  K-contiguous: chunk (KSTEP/8)*s + slot, and the
  // step only flips chunk bits above the slot's, so it is an XOR of 2*KSTEP*s bytes.
  // M/N-contiguous: KSTEP rows further down (the swizzle depends on k mod 16 only).
  template <bool KCONTIG, int R>
  __device__ __forceinline__ static int step_addr(int base, int s) {
    if constexpr (KCONTIG) {
      if (s == 0) return base;
      int b = base;  // opaque: the XORed address is formed at its use, not held
      asm volatile("" : "+v"(b));
      return b ^ (2 * KSTEP * s);
    }
    return base + s * KSTEP * (R * 2);
  }

  template <bool KCONTIG, int R>
  __device__ __forceinline__ static v4u read_frag(const uint8_t* stage, int addr) {
    if constexpr (KCONTIG) {
      return *reinterpret_cast<const v4u*>(stage + addr);
    } else {
      const uint8_t* p = stage + addr;
      v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s FGEMM_LDS*)(p));
      v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s FGEMM_LDS*)(p + 4 * (R * 2)));
      v2u l2 = __builtin_bit_cast(v2u, lo), h2 = __builtin_bit_cast(v2u, hi);
      return v4u{l2.x, l2.y, h2.x, h2.y};
    }
  }

  __device__ __forceinline__ static void read_frags(const uint8_t* stage, const FragAddr& fa,
                                                    int s, Frags& fr) {
#pragma unroll
    for (int f = 0; f < CFG::FM; ++f)
#pragma unroll
      for (int p = 0; p < FC; ++p)
        fr.a[f][p] = read_frag<AK, BM>(stage, step_addr<AK, BM>(fa.a[f], s) ^ (CHUNK2 * p));
#pragma unroll
    for (int f = 0; f < CFG::FN; ++f)
#pragma unroll
      for (int p = 0; p < FC; ++p)
        fr.b[f][p] = read_frag<BKC, BN>(stage, step_addr<BKC, BN>(fa.b[f], s) ^ (CHUNK2 * p));
  }

  // MX: the scales of phase p (kt within the tile) for every step and fragment: the
  // lane's row and block (phase p's BPP blocks follow each other in the group's 16
  // bytes, BPS of them a step).
  __device__ __forceinline__ static void read_scales(const uint8_t* smem, const FragAddr& fa,
                                                     int wm, int wn, int p, Scales& sc) {
    if constexpr (MX) {
      const uint8_t* buf = smem + MX_OFF + ((p / PPG) & 1) * MX_BUF + (p % PPG) * BPP + fa.sc;
#pragma unroll
      for (int q = 0; q < (STEPS + 1) / 2; ++q) {
#pragma unroll
        for (int i = 0; i < CFG::FM; ++i)
          sc.a[q][i] = *reinterpret_cast<const uint32_t*>(
                           buf + 4 * q + (wm * CFG::WM + i * CFG::MI) * 16) >> fa.scsh;
#pragma unroll
        for (int j = 0; j < CFG::FN; ++j)
          sc.b[q][j] = *reinterpret_cast<const uint32_t*>(
                           buf + 4 * q + (CFG::BM + wn * CFG::WN + j * CFG::MI) * 16) >> fa.scsh;
      }
    }
  }

  // One MFMA: the B fragment first, so that a lane's accumulators are consecutive
  // columns of one output row.  OPS: the byte of the scale registers the 8/4-bit
  // MFMA applies (its op_sel).
  template <int OPS = 0>
  __device__ __forceinline__ static Acc mfma(const v4u (&bf)[FC], const v4u (&af)[FC],
                                             const Acc& c, uint32_t scb = 127,
                                             uint32_t sca = 127) {
    const v4u& b = bf[0];
    const v4u& a = af[0];
    if constexpr (F8) {
      // 8-bit codes with E8M0 block scales (127 = 2^0 without MX: the tensor scales
      // are applied in the epilogue through alpha)
      // format numbers: 0 E4M3, 1 E5M2, 4 E2M1 (whose operand is the low 4 registers)
      constexpr int FA = F4 ? 4 : ((DT - kF8Base) >> 1) & 1;
      constexpr int FB = F4 ? 4 : (DT - kF8Base) & 1;
      const v8i bv = F4 ? v8i{(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0}
                        : v8i{(int)bf[0].x, (int)bf[0].y, (int)bf[0].z, (int)bf[0].w,
                              (int)bf[FC - 1].x, (int)bf[FC - 1].y, (int)bf[FC - 1].z,
                              (int)bf[FC - 1].w};
      const v8i av = F4 ? v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0}
                        : v8i{(int)af[0].x, (int)af[0].y, (int)af[0].z, (int)af[0].w,
                              (int)af[FC - 1].x, (int)af[FC - 1].y, (int)af[FC - 1].z,
                              (int)af[FC - 1].w};
      if constexpr (CFG::MI == 32)
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, c, FB, FA, OPS, (int)scb,
                                                              OPS, (int)sca);
      else
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv, av, c, FB, FA, OPS,
                                                               (int)scb, OPS, (int)sca);
    } else if constexpr (CFG::MI == 32) {
      if constexpr (DT == kBF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b),
                                                       __builtin_bit_cast(bf16x8_t, a), c, 0, 0, 0);
      else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, b),
                                                      __builtin_bit_cast(f16x8_t, a), c, 0, 0, 0);
    } else {
      if constexpr (DT == kBF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b),
                                                       __builtin_bit_cast(bf16x8_t, a), c, 0, 0, 0);
      else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, b),
                                                      __builtin_bit_cast(f16x8_t, a), c, 0, 0, 0);
    }
  }

  // The MFMA of step s on fragments i of A and j of B: with MX, the scale registers
  // of s's pair of steps and the byte for s (0 or 2; s is a constant at every call,
  // so the choice folds away); else unit scales (127 = 2^0).
  __device__ __forceinline__ static Acc mfma_s(const v4u (&bf)[FC], const v4u (&af)[FC],
                                               const Acc& c, const Scales& sc, int s, int i,
                                               int j) {
    if constexpr (MX) {
      if (s & 1) return mfma<2>(bf, af, c, sc.b[s >> 1][j], sc.a[s >> 1][i]);
      return mfma<0>(bf, af, c, sc.b[s >> 1][j], sc.a[s >> 1][i]);
    }
    return mfma(bf, af, c);
  }

  // An empty asm that reads every accumulator block in its AGPRs: the MFMAs that
  // produce them must issue before it (it is volatile, so it stays in program order
  // with the barrier that follows it).
  __device__ __forceinline__ static void pin_acc(Acc (&acc)[CFG::FM][CFG::FN]) {
#pragma unroll
    for (int i = 0; i < CFG::FM; ++i)
#pragma unroll
      for (int j = 0; j < CFG::FN; ++j) asm volatile("" : : "a"(acc[i][j]));
  }

  __device__ __forceinline__ static void mfma_step(const Frags& fr, const Scales& sc, int s,
                                                   Acc (&acc)[CFG::FM][CFG::FN]) {
#pragma unroll
    for (int i = 0; i < CFG::FM; ++i)
#pragma unroll
      for (int j = 0; j < CFG::FN; ++j)
        acc[i][j] = mfma_s(fr.b[j], fr.a[i], acc[i][j], sc, s, i, j);
  }

  // one MFMA, then one instruction of OTHER_MASK, while both last (I counts MFMAs)
  template <int I, int MFMA, int OTHER_MASK, int OTHERS>
  __device__ __forceinline__ static void interleave() {
    if constexpr (I < MFMA) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (I < OTHERS) __builtin_amdgcn_sched_group_barrier(OTHER_MASK, 1, 0);
      interleave<I + 1, MFMA, OTHER_MASK, OTHERS>();
    }
  }
  static constexpr int kMfmaPerStep = CFG::FM * CFG::FN;
  static constexpr int kReadsPerStep = CFG::FM * (AK ? FC : 2) + CFG::FN * (BKC ? FC : 2);

  // ---- step 0 with the phase's direct loads slotted between its MFMAs
  static constexpr int kRA = AK ? FC : 2, kRB = BKC ? FC : 2;  // read instructions a fragment
  static constexpr int kLoadsPerPhase = CFG::QAW + CFG::QBW;

  // Read instruction r of step s into `next`: A fragments first, then B.
  template <int R>
  __device__ __forceinline__ static void read_job(const uint8_t* cur, const FragAddr& fa, int s,
                                                  Frags& next) {
    if constexpr (R < CFG::FM * kRA) {
      constexpr int f = R / kRA, part = R % kRA;
      const int addr = step_addr<AK, BM>(fa.a[f], s);
      if constexpr (AK) {
        next.a[f][part] = *reinterpret_cast<const v4u*>(cur + (addr ^ (CHUNK2 * part)));
      } else {
        v4s t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (v4s FGEMM_LDS*)(cur + addr + part * 4 * (BM * 2)));
        v2u t2 = __builtin_bit_cast(v2u, t);
        if (part == 0) { next.a[f][0].x = t2.x; next.a[f][0].y = t2.y; }
        else { next.a[f][0].z = t2.x; next.a[f][0].w = t2.y; }
      }
    } else {
      constexpr int r = R - CFG::FM * kRA;
      constexpr int f = r / kRB, part = r % kRB;
      const int addr = step_addr<BKC, BN>(fa.b[f], s);
      if constexpr (BKC) {
        next.b[f][part] = *reinterpret_cast<const v4u*>(cur + (addr ^ (CHUNK2 * part)));
      } else {
        v4s t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (v4s FGEMM_LDS*)(cur + addr + part * 4 * (BN * 2)));
        v2u t2 = __builtin_bit_cast(v2u, t);
        if (part == 0) { next.b[f][0].x = t2.x; next.b[f][0].y = t2.y; }
        else { next.b[f][0].z = t2.x; next.b[f][0].w = t2.y; }
      }
    }
  }

  // Direct load L of this wave's share of a phase (A slots, then B slots).
  template <int L>
  __device__ __forceinline__ static void load_job(const char* ab, const char* bb,
                                                  const LoadAddr& la, int wave, uint32_t ls) {
    if constexpr (L < CFG::QAW) {
      const int q = wave + CFG::NW * L;
      if (CFG::QA % CFG::NW == 0 || q < CFG::QA) lds_dma(ab, la.a[L], ls + q * 1024);
    } else {
      constexpr int i = L - CFG::QAW;
      const int q = wave + CFG::NW * i;
      if (CFG::QB % CFG::NW == 0 || q < CFG::QB) lds_dma(bb, la.b[i], ls + CFG::LDS_A + q * 1024);
    }
  }

  // MFMA M of the step on `now`, then read instruction M of step `rs` of stage `rd`
  // into `next`, then load M (when LD); a scheduling fence after each group keeps
  // the order.  Leftover reads and loads follow the last MFMA.
  template <int M, bool LD>
  __device__ __forceinline__ static void emit0(const uint8_t* rd, int rs, const FragAddr& fa,
                                               const Frags& now, const Scales& sc, Frags& next,
                                               Acc (&acc)[CFG::FM][CFG::FN],
                                               const char* ab, const char* bb,
                                               const LoadAddr& la, int wave, uint32_t ls) {
    constexpr int NM = kMfmaPerStep, NR = kReadsPerStep, NL = LD ? kLoadsPerPhase : 0;
    if constexpr (M < NM) {
      constexpr int i = M / CFG::FN, j = M % CFG::FN;
      acc[i][j] = mfma_s(now.b[j], now.a[i], acc[i][j], sc, STEPS - 1, i, j);
      if constexpr (M < NR) read_job<M>(rd, fa, rs, next);
      if constexpr (M < NL) load_job<M>(ab, bb, la, wave, ls);
      __builtin_amdgcn_sched_barrier(0);
      emit0<M + 1, LD>(rd, rs, fa, now, sc, next, acc, ab, bb, la, wave, ls);
    } else {
      emit0_rest<NM, LD>(rd, rs, fa, next, ab, bb, la, wave, ls);
    }
  }
  template <int X, bool LD>
  __device__ __forceinline__ static void emit0_rest(const uint8_t* rd, int rs, const FragAddr& fa,
                                                    Frags& next, const char* ab, const char* bb,
                                                    const LoadAddr& la, int wave, uint32_t ls) {
    constexpr int NR = kReadsPerStep, NL = LD ? kLoadsPerPhase : 0;
    if constexpr (X < NR || X < NL) {
      if constexpr (X < NR) read_job<X>(rd, fa, rs, next);
      if constexpr (X < NL) load_job<X>(ab, bb, la, wave, ls);
      emit0_rest<X + 1, LD>(rd, rs, fa, next, ab, bb, la, wave, ls);
    }
  }

  // MFMA step s of the phase in `cur` on fragments `now`, reading step s+1 into `next`.
  __device__ __forceinline__ static void step(const uint8_t* cur, const FragAddr& fa, int s,
                                              const Frags& now, const Scales& sc, Frags& next,
                                              Acc (&acc)[CFG::FM][CFG::FN]) {
    read_frags(cur, fa, s + 1, next);
    mfma_step(now, sc, s, acc);
    interleave<0, kMfmaPerStep, 0x100, kReadsPerStep>();
    FGEMM_PHASE_FENCE();
  }

  // ============================================================ main loops
  // Interior tiles: STAGES-deep ring of direct-to-LDS phases.  Per phase kt: run
  // the MFMA steps but the last while reading the next step's fragments, wait for
  // phase kt+1's loads, barrier, then run the last step while reading phase kt+1's
  // first fragments and issuing the loads of phase kt+STAGES into the stage that
  // the barrier has just freed (so a phase's loads have a whole phase to land).
  template <int VMC>
  __device__ __forceinline__ static void wait_phase(bool steady) {
    if (steady) wait_vmcnt<VMC>();
    else wait_vmcnt<0>();
  }

  // Next tile's first phases, issued by the last phase of the current tile (after
  // its final barrier every stage is free) so that they fly during the epilogue.
  struct Next {
    int m0, n0, kt0, ktiles;
  };

  __device__ __forceinline__ static void issue_prologue(const Src& S, int m0, int kt0,
                                                        int ktiles, int wave, const LoadAddr& la,
                                                        uint8_t* smem) {
    if constexpr (MX) issue_scales(S, 0, wave, la, smem);  // phases 0..PPG-1 (kt0 is 0)
#pragma unroll
    for (int t = 0; t < CFG::STAGES - 1; ++t)
      if (t < ktiles) issue_loads(S, m0, kt0 + t, wave, la, smem + t * CFG::LDS_STAGE);
  }

  // `pre`: this tile's prologue was issued by the previous tile (before its
  // epilogue stores, which share the wait counter).  `chain`: issue the prologue of
  // `nx` (a tile of problem `Pn`) at the end.
  __device__ __forceinline__ static void loop_fast(const GemmProblem& P, int m0, int n0,
                                                   uint8_t* smem, int wave, int wm, int wn,
                                                   int lane, int kt0, int ktiles, bool pre,
                                                   bool chain, const GemmProblem& Pn,
                                                   const Next& nx,
                                                   Acc (&acc)[CFG::FM][CFG::FN]) {
    constexpr int S = CFG::STAGES;
    // every wave issues the same number of loads per phase, so one vmcnt bound fits all
    static_assert(CFG::QA % CFG::NW == 0 && CFG::QB % CFG::NW == 0, "even load slots");
    constexpr int QW = CFG::QAW + CFG::QBW;  // loads this wave issues per phase
    const Src src = src_of(P);
    LoadAddr la;
    load_addr(P, m0, n0, wave, lane, la);
    int flane = lane;  // opaque: fragment offsets are rebuilt per tile, not held across it
    asm volatile("" : "+v"(flane));
    FragAddr fa;
    frag_addr(wm, wn, flane, fa);
    if (!pre) issue_prologue(src, m0, kt0, ktiles, wave, la, smem);
    // phase 0 ready: at most the later prologue phases still in flight (all of
    // them when stores were issued after them)
    wait_phase<(S - 2) * QW>(!pre && ktiles >= S - 1);
    __syncthreads();
    // the last stage is free now (it held the previous tile's epilogue staging)
    if (S - 1 < ktiles)
      issue_loads(src, m0, kt0 + S - 1, wave, la, smem + (S - 1) * CFG::LDS_STAGE);
    Frags f0, f1;
    read_frags(smem, fa, 0, f0);
    Scales sc;  // MX: the scales of phase kt (read a phase ahead, with its first fragments)
    if constexpr (MX) read_scales(smem, fa, wm, wn, 0, sc);
    int st = 0;  // stage of phase kt
    // phases that still load a later phase, then the last S that do not: two
    // straight loop bodies
    int kt = 0;
#define FGEMM_PHASE(LD, K, X, Y) \
  phase<LD>(src, m0, smem, wave, wm, wn, lane, fa, la, kt0, K, ktiles, st, chain, Pn, nx, X, Y, \
            sc, acc)
    if constexpr (STEPS == 1) {
      // the two fragment sets swap roles every phase: two phases an iteration, and
      // one copy where a loop leaves an odd phase over (a selection of sets at run
      // time would put them in private memory)
      for (; kt + 1 + S < ktiles; kt += 2) {
        FGEMM_PHASE(true, kt, f0, f1);
        FGEMM_PHASE(true, kt + 1, f1, f0);
      }
      if (kt + S < ktiles) {
        FGEMM_PHASE(true, kt, f0, f1);
        ++kt;
        f0 = f1;
      }
      for (; kt + 1 < ktiles; kt += 2) {
        FGEMM_PHASE(false, kt, f0, f1);
        FGEMM_PHASE(false, kt + 1, f1, f0);
      }
      if (kt < ktiles) FGEMM_PHASE(false, kt, f0, f1);
    } else {
      for (; kt + S < ktiles; ++kt) FGEMM_PHASE(true, kt, f0, f1);
      for (; kt < ktiles; ++kt) FGEMM_PHASE(false, kt, f0, f1);
    }
#undef FGEMM_PHASE
    FGEMM_PHASE_FENCE();
  }

  // Phase kt of the ring (stage st): the steps but the last, the wait for phase kt+1
  // and the barrier, then the last step under the first reads of phase kt+1 and,
  // when LD, the loads of phase kt+S into stage st (after the last phase: the next
  // tile's first loads instead).
  template <bool LD>
  __device__ __forceinline__ static void phase(const Src& src, int m0, uint8_t* smem, int wave,
                                               int wm, int wn,
                                               int lane, const FragAddr& fa, const LoadAddr& la,
                                               int kt0, int kt, int ktiles, int& st, bool chain,
                                               const GemmProblem& Pn, const Next& nx, Frags& f0,
                                               Frags& f1, Scales& sc,
                                               Acc (&acc)[CFG::FM][CFG::FN]) {
    constexpr int S = CFG::STAGES;
    constexpr int QW = CFG::QAW + CFG::QBW;
    FGEMM_PHASE_FENCE();
    uint8_t* cur = smem + st * CFG::LDS_STAGE;
    const int kl = kt0 + kt + S;
    const char* ab = LD ? uniform_ptr(a_base(src, m0, kl)) : nullptr;
    const char* bb = LD ? uniform_ptr(b_base(src, kl)) : nullptr;
    // every step but the last; the last step's fragments end up in f1 (in f0 for
    // one-step phases, whose caller swaps the two sets every phase)
    if constexpr (STEPS >= 2) step(cur, fa, 0, f0, sc, f1, acc);
    if constexpr (STEPS == 4) {
      step(cur, fa, 1, f1, sc, f0, acc);
      step(cur, fa, 2, f0, sc, f1, acc);
    }
    Frags& fl = STEPS == 1 ? f0 : f1;  // the last step's fragments
    Frags& fn = STEPS == 1 ? f1 : f0;  // receives the next phase's first
    // MX: the accumulators of the steps above, read in place by an empty asm ahead of
    // the barrier.  The scale-group branch after the barrier otherwise lets the
    // compiler sink those MFMAs below it, and the phase then runs its fragment reads,
    // wait and barrier with the MFMA pipe idle.
    if constexpr (MX && STEPS >= 2) pin_acc(acc);
    // phase kt+1 must have landed; the S-2 phases after it may still fly when
    // they have all been issued
    wait_phase<(S - 2) * QW>(kt + S - 1 < ktiles);
    __syncthreads();
    // raised issue priority for the last step: a wave still in it is served ahead of
    // its SIMD partner that has moved on, so the pair reaches the next barrier
    // together (measured 0.5-1 % faster)
    __builtin_amdgcn_s_setprio(1);
    const int st_next = st + 1 == S ? 0 : st + 1;
    const uint8_t* nxt = smem + st_next * CFG::LDS_STAGE;
    // MX scale groups of 16 blocks (P = PPG phases: 4 at 8 bits, 2 at 4 bits)
    // alternate between two buffers.  Group g is issued at phase Pg-P after the
    // barrier, ahead of that phase's loads of phase Pg-P+S, so it has landed by the
    // wait of phase Pg-P+S-1 (loads complete in issue order), and it is read from the
    // barrier of phase Pg-1 on (phase Pg's scales are read with its first fragments):
    // hence S <= P.  Its buffer is refilled at phase Pg+P, after the barriers that
    // follow the last read of it, at phase Pg+P-2.  The last phase of a tile reads no
    // scales after its barrier, so the next tile's first group may go to buffer 0.
    static_assert(!MX || S <= PPG, "block scales must land before their first read");
    if constexpr (MX)
      if (kt % PPG == 0 && kt + PPG < ktiles) issue_scales(src, kt / PPG + 1, wave, la, smem);
    Scales scn;  // MX: phase kt+1's scales
    if (kt + 1 < ktiles) {
      if constexpr (MX) read_scales(smem, fa, wm, wn, kt + 1, scn);
      if constexpr (LD) {
        // stage st is free once every wave has passed the barrier: phase kt+S goes
        // there, its loads slotted between the last step's MFMAs
        emit0<0, true>(nxt, 0, fa, fl, sc, fn, acc, ab, bb, la, wave, lds_addr(cur));
        __builtin_amdgcn_s_setprio(0);
        if constexpr (MX) sc = scn;
        FGEMM_PHASE_FENCE();
        st = st_next;
        return;
      }
      read_frags(nxt, fa, 0, fn);
    } else if (chain) {
      LoadAddr ln;  // computed here, where the next fragments are dead
      load_addr(Pn, nx.m0, nx.n0, wave, lane, ln);
      issue_prologue(src_of(Pn), nx.m0, nx.kt0, nx.ktiles, wave, ln, smem);
    }
    mfma_step(fl, sc, STEPS - 1, acc);
    interleave<0, kMfmaPerStep, 0x100, kReadsPerStep>();
    __builtin_amdgcn_s_setprio(0);
    if constexpr (MX)
      if (kt + 1 < ktiles) sc = scn;
    st = st_next;
  }

  // Edge tiles: bounds-tested register loads into two stages, one barrier a phase.
  __device__ __forceinline__ static void loop_checked(const GemmProblem& P, int m0, int n0,
                                                      uint8_t* smem, int wave, int wm, int wn,
                                                      int lane_in, int kt0, int ktiles,
                                                      Acc (&acc)[CFG::FM][CFG::FN]) {
    int lane = lane_in;  // opaque: per-tile recomputation instead of hoisted registers
    asm volatile("" : "+v"(lane));
    FragAddr fa;
    frag_addr(wm, wn, lane, fa);
    v4u ra[CFG::QAW], rb[CFG::QBW];
    load_checked(P, m0, n0, kt0, wave, lane, ra, rb);
    store_checked(smem, wave, lane, ra, rb);
    __syncthreads();
    for (int kt = 0; kt < ktiles; ++kt) {
      const uint8_t* cur = smem + (kt & 1) * CFG::LDS_STAGE;
      uint8_t* nxt = smem + ((kt + 1) & 1) * CFG::LDS_STAGE;
      const bool more = kt + 1 < ktiles;
      if (more) load_checked(P, m0, n0, kt0 + kt + 1, wave, lane, ra, rb);
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        Frags fr;
        read_frags(cur, fa, s, fr);
        mfma_step(fr, Scales{}, s, acc);  // 16-bit inputs only: no block scales
      }
      if (more) store_checked(nxt, wave, lane, ra, rb);
      __syncthreads();
    }
  }

  // ============================================================ epilogues
  // One lane's 8 consecutive outputs of a whole block (row < M, 8 columns < N):
  // alpha is applied already; + beta*C (prefetched), + bias, the activation, one
  // rounding of each pair into a packed word, the row's sum of squares of the
  // rounded values, one non-temporal 16-byte store.  Same arithmetic, in the same
  // order, as the general path of epilogue_rows.
  __device__ __forceinline__ static void store_whole(const GemmProblem& P, void* Cout, int row,
                                                     int col, const v4u* cpre, bool use_bias,
                                                     bool use_ss, v4f lo, v4f hi, float& ss) {
    float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    if (cpre) {
      const v4u cv = *cpre;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] += P.beta * to_f32<ODT>(cv[e] & 0xffff);
        v[2 * e + 1] += P.beta * to_f32<ODT>(cv[e] >> 16);
      }
    }
    if (use_bias) {
      const uint16_t* bias = static_cast<const uint16_t*>(P.bias) + col;
      if ((reinterpret_cast<uintptr_t>(bias) & 15) == 0) {
        const v4u b4 = *reinterpret_cast<const v4u*>(bias);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] += to_f32<ODT>(b4[e] & 0xffff);
          v[2 * e + 1] += to_f32<ODT>(b4[e] >> 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += to_f32<ODT>(bias[e]);
      }
    }
    if constexpr (EPI == kEpiAct) apply_act_run<8>(P.act, v);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack2<ODT>(v[2 * e], v[2 * e + 1]);
    if (use_ss) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = to_f32<ODT>(w[e] & 0xffff), b = to_f32<ODT>(w[e] >> 16);
        ss += a * a;
        ss += b * b;
      }
    }
    uint16_t* C = static_cast<uint16_t*>(Cout);
    __builtin_nontemporal_store(v4u{w[0], w[1], w[2], w[3]},
                                reinterpret_cast<v4u*>(C + (int64_t)row * P.ldc + col));
  }

  // Row-contiguous epilogue (16-byte aligned operands): every 32-row, EPI_CW-column
  // block of the wave's results goes to LDS in the MFMA layout and comes back as 8
  // consecutive columns of one row per lane, so that beta*C is read and the result
  // written in whole 128-byte lines.  The arithmetic per element is that of the
  // register epilogue below: alpha*acc (SwiGLU: silu(g)*u of the row-scaled gate and
  // up accumulators), + beta*C, + bias, one rounding.  The 16-bit C traffic is
  // non-temporal: each line is read once and written once, and in L2 it would only
  // evict the A and B panels the XCD's next tiles reuse (1.5-2 % at 8192^3).
  __device__ __forceinline__ static void epilogue_rows(const GemmProblem& P, void* Cout, int m0,
                                                       int n0, int tn, int wave, int wm, int wn,
                                                       int lane_in, uint8_t* smem,
                                                       Acc (&acc)[CFG::FM][CFG::FN]) {
    int lane = lane_in;  // opaque: recomputed per tile rather than held across the loop
    asm volatile("" : "+v"(lane));
    constexpr int CW = CFG::EPI_CW;
    constexpr int NCH = CW / 4;          // 16-byte chunks per staged row
    constexpr int LPR = NCH / 2;         // lanes per row on the way out (8 columns each)
    constexpr int RPT = 64 / LPR;        // rows per pass
    constexpr int MI = CFG::MI;
    constexpr int JC = CW / MI;          // accumulator block columns per staged block
    constexpr int BPB = 32 / MI;         // accumulator block rows per 32-row band
    constexpr int NB = CFG::WM / 32;     // 32-row bands of the wave tile
    constexpr int G4 = CFG::ACC / 4;     // groups of 4 columns a lane holds per block
    uint8_t* region = smem + CFG::EPI_OFF + wave * CFG::EPI_WAVE_BYTES;
    // chunk swizzle: 16 consecutive rows of one logical chunk hit distinct banks
    auto swz = [](int r) { return NCH == 16 ? (r & 15) : ((r >> 1) & 7); };
    const int lr = lane % MI, lc = lane / MI;  // lane's row and column slot in a block
    const int orow = lane / LPR, oc = lane % LPR;
    const bool use_beta = EPI != kEpiStore32 && (P.flags & kFlagBeta) != 0;
    constexpr bool STORE16 = EPI == kEpiStore16 || EPI == kEpiAct || EPI == kEpiRope;
    const bool use_bias = STORE16 && (P.flags & kFlagBias) != 0;
    const bool use_ss = STORE16 && (P.flags & kFlagRowSumSq) != 0;
    const uint16_t* bias = static_cast<const uint16_t*>(P.bias);
    const uint16_t* Cin = static_cast<const uint16_t*>(P.Cin);
    // beta*C: every whole 8-column piece of the wave's tile is requested up front so
    // that the reads overlap the staging instead of waiting once per piece
    constexpr int WO = SWIGLU ? CFG::WN / 2 : CFG::WN;  // output columns of the wave
    constexpr int HF = CFG::FN / 2;                       // SwiGLU: up blocks follow gate ones
    static_assert(WO % CW == 0, "epilogue blocks");
    constexpr int NPASS = 32 / RPT, NJC = WO / CW;
    constexpr bool HAS_C = EPI != kEpiStore32;
    v4u cpre[HAS_C ? NB : 1][HAS_C ? NJC : 1][HAS_C ? NPASS : 1];
    if constexpr (HAS_C) {
      if (use_beta) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int jc = 0; jc < NJC; ++jc)
#pragma unroll
            for (int t = 0; t < NPASS; ++t) {
              const int row = m0 + wm * CFG::WM + i * 32 + t * RPT + orow;
              const int col = n0 + wn * WO + jc * CW + 8 * oc;
              cpre[i][jc][t] = v4u{0u, 0u, 0u, 0u};
              if (row < P.M && P.N - col >= 8)
                cpre[i][jc][t] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4u*>(Cin + (int64_t)row * P.ldc + col));
            }
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int row_base = m0 + wm * CFG::WM + i * 32;
      float ss[32 / RPT];
#pragma unroll
      for (int t = 0; t < 32 / RPT; ++t) ss[t] = 0.f;
#pragma unroll
      for (int jc = 0; jc < NJC; ++jc) {
#pragma unroll
        for (int ib = 0; ib < BPB; ++ib) {
          // SwiGLU row scale of this lane's row (alpha folded in)
          float rs = 0.f;
          if constexpr (SWIGLU) {
            const int row = row_base + ib * MI + lr;
            if (row < P.M) rs = rsqrtf(P.rms_ss[row] * P.rms_inv_n + P.rms_eps) * P.alpha;
          }
#pragma unroll
          for (int jj = 0; jj < JC; ++jj)
#pragma unroll
            for (int g = 0; g < G4; ++g) {
              const Acc& a = acc[i * BPB + ib][jc * JC + jj];
              v4f v;
              if constexpr (SWIGLU) {
                const Acc& ua = acc[i * BPB + ib][jc * JC + jj + HF];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float gg = rs * a[4 * g + e];
                  const float uu = rs * ua[4 * g + e];
                  v[e] = gg / (1.f + __expf(-gg)) * uu;
                }
              } else {
                v = v4f{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
                if (STORE16) v = v * P.alpha;
              }
              // row ib*MI + lr of the band; 16-byte chunk of columns
              // jj*MI + g*(256/MI) + 4*lc
              const int r = ib * MI + lr;
              const int c = jj * (MI / 4) + g * (64 / MI) + lc;
              *reinterpret_cast<v4f*>(region + r * (CW * 4) + ((c ^ swz(r)) << 4)) = v;
            }
        }
        const int col = n0 + wn * WO + jc * CW + 8 * oc;
        const int nv = P.N - col;
        // the wave's 32 rows and CW columns all inside the matrix (wave-uniform): the
        // passes store whole 16-byte pieces with no per-element tests
        const bool whole = row_base + 32 <= P.M && P.N - (n0 + wn * WO + jc * CW) >= CW;
#pragma unroll
        for (int t = 0; t < 32 / RPT; ++t) {
          const int r = t * RPT + orow;
          const uint8_t* src = region + r * (CW * 4);
          v4f lo = *reinterpret_cast<const v4f*>(src + (((2 * oc) ^ swz(r)) << 4));
          v4f hi = *reinterpret_cast<const v4f*>(src + (((2 * oc + 1) ^ swz(r)) << 4));
          const int row = row_base + r;
          // (16-bit inputs only: in the 4-wave 8-bit tiles this path measured 4-8 % slower
          // and spilled with fp16 outputs)
          if constexpr (STORE16 && EPI != kEpiRope && !F8) {
            if (whole) {
              store_whole(P, Cout, row, col, use_beta ? &cpre[i][jc][t] : nullptr, use_bias,
                          use_ss, lo, hi, ss[t]);
              continue;
            }
          }
          if (row >= P.M || nv <= 0) continue;
          float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          const int64_t off = (int64_t)row * P.ldc + col;
          if constexpr (EPI == kEpiStore32) {
            float* C = static_cast<float*>(Cout);
            if (nv >= 8) {
              *reinterpret_cast<v4f*>(C + off) = lo;
              *reinterpret_cast<v4f*>(C + off + 4) = hi;
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (e < nv) C[off + e] = v[e];
            }
          } else {
            uint16_t* C = static_cast<uint16_t*>(Cout);
            if (use_beta) {
              uint32_t cb[8];
              if (nv >= 8) {
                const v4u cv = cpre[i][jc][t];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  cb[2 * e] = cv[e] & 0xffff;
                  cb[2 * e + 1] = cv[e] >> 16;
                }
              } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) cb[e] = e < nv ? Cin[off + e] : 0;
              }
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] += P.beta * to_f32<ODT>(cb[e]);
            }
            if (use_bias) {
              // one 16-byte load where the bias vector is aligned
              if (nv >= 8 && (reinterpret_cast<uintptr_t>(bias + col) & 15) == 0) {
                const v4u b4 = *reinterpret_cast<const v4u*>(bias + col);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  v[2 * e] += to_f32<ODT>(b4[e] & 0xffff);
                  v[2 * e + 1] += to_f32<ODT>(b4[e] >> 16);
                }
              } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] += e < nv ? to_f32<ODT>(bias[col + e]) : 0.f;
              }
            }
            if constexpr (EPI == kEpiAct) apply_act_run<8>(P.act, v);
            if constexpr (EPI == kEpiRope) {
              // pair rates of this run from the table after the stages
              const double* ft = reinterpret_cast<const double*>(smem + CFG::SMEM) +
                                 ((col % P.rope_hd) >> 1);
              rope_run<8>(rope_pos_of(P.rope_pos, P.rope_off, row),
                          [&](int q) { return ft[q]; }, v);
            }
            uint32_t o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              o[e] = from_f32<ODT>(v[e]);
              if (use_ss) {
                const float rr = to_f32<ODT>(o[e]);
                if (e < nv) ss[t] += rr * rr;
              }
            }
            if (nv >= 8) {
              __builtin_nontemporal_store(
                  v4u{o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16),
                      o[6] | (o[7] << 16)},
                  reinterpret_cast<v4u*>(C + off));
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (e < nv) C[off + e] = (uint16_t)o[e];
            }
          }
        }
      }
      if (use_ss) {
#pragma unroll
        for (int t = 0; t < 32 / RPT; ++t) {
          float x = ss[t];
#pragma unroll
          for (int d = 1; d < LPR; d <<= 1) x += __shfl_xor(x, d);
          const int row = row_base + t * RPT + orow;
          if (oc == 0 && row < P.M)
            P.ss_partial[(int64_t)(tn * CFG::WAVES_N + wn) * P.M + row] = x;
        }
      }
    }
  }


  // Lane layout of acc[i][j][4g+s]: row = wave row base + MI*i + lane % MI,
  // column = wave column base + MI*j + g*(256/MI) + 4*(lane / MI) + s.
  __device__ __forceinline__ static void epilogue(const GemmProblem& P, void* Cout, int m0,
                                                  int n0, int tn, int wm, int wn, int lane,
                                                  const uint8_t* smem,
                                                  Acc (&acc)[CFG::FM][CFG::FN]) {
    constexpr int MI = CFG::MI, G4 = CFG::ACC / 4;
    const int lr = lane % MI, lc = lane / MI;
    if constexpr (EPI == kEpiStore32) {
      float* C = static_cast<float*>(Cout);
#pragma unroll
      for (int i = 0; i < CFG::FM; ++i) {
        int row = m0 + wm * CFG::WM + i * MI + lr;
        if (row >= P.M) continue;
#pragma unroll
        for (int j = 0; j < CFG::FN; ++j)
#pragma unroll
          for (int q = 0; q < G4; ++q) {
            int col = n0 + wn * CFG::WN + j * MI + q * (256 / MI) + 4 * lc;
            float* dst = C + (int64_t)row * P.ldc + col;
            if (VEC && col + 4 <= P.N) {
              *reinterpret_cast<v4f*>(dst) = v4f{acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                 acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            } else {
#pragma unroll
              for (int s = 0; s < 4; ++s)
                if (col + s < P.N) dst[s] = acc[i][j][4 * q + s];
            }
          }
      }
      return;
    }
    uint16_t* C = static_cast<uint16_t*>(Cout);
    const uint16_t* Cin = static_cast<const uint16_t*>(P.Cin);
    const bool use_beta = (P.flags & kFlagBeta) != 0;
    if constexpr (EPI == kEpiStore16 || EPI == kEpiAct || EPI == kEpiRope) {
      const bool use_bias = (P.flags & kFlagBias) != 0;
      const bool use_ss = (P.flags & kFlagRowSumSq) != 0;
      const uint16_t* bias = static_cast<const uint16_t*>(P.bias);
#pragma unroll
      for (int i = 0; i < CFG::FM; ++i) {
        int row = m0 + wm * CFG::WM + i * MI + lr;
        bool rv = row < P.M;
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < CFG::FN; ++j)
#pragma unroll
          for (int q = 0; q < G4; ++q) {
            int col = n0 + wn * CFG::WN + j * MI + q * (256 / MI) + 4 * lc;
            int nv = P.N - col;
            if (!rv || nv <= 0) continue;
            float v[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) v[s] = P.alpha * acc[i][j][4 * q + s];
            const int64_t off = (int64_t)row * P.ldc + col;
            if (use_beta) {
              uint32_t c[4];
              if (VEC && nv >= 4) {
                v2u cv = *reinterpret_cast<const v2u*>(Cin + off);
                c[0] = cv.x & 0xffff; c[1] = cv.x >> 16; c[2] = cv.y & 0xffff; c[3] = cv.y >> 16;
              } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) c[s] = s < nv ? Cin[off + s] : 0;
              }
#pragma unroll
              for (int s = 0; s < 4; ++s) v[s] += P.beta * to_f32<ODT>(c[s]);
            }
            if (use_bias) {
#pragma unroll
              for (int s = 0; s < 4; ++s) v[s] += s < nv ? to_f32<ODT>(bias[col + s]) : 0.f;
            }
            if constexpr (EPI == kEpiAct) apply_act_run<4>(P.act, v);
            if constexpr (EPI == kEpiRope) {
              const double* ft = reinterpret_cast<const double*>(smem + CFG::SMEM) +
                                 ((col % P.rope_hd) >> 1);
              rope_run<4>(rope_pos_of(P.rope_pos, P.rope_off, row),
                          [&](int q) { return ft[q]; }, v);
            }
            uint32_t o[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              o[s] = from_f32<ODT>(v[s]);
              float r = to_f32<ODT>(o[s]);
              if (s < nv) ss += r * r;
            }
            if (VEC && nv >= 4) {
              *reinterpret_cast<v2u*>(C + off) = v2u{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
            } else {
#pragma unroll
              for (int s = 0; s < 4; ++s)
                if (s < nv) C[off + s] = (uint16_t)o[s];
            }
          }
        if (use_ss) {
#pragma unroll
          for (int d = MI; d < 64; d <<= 1) ss += __shfl_xor(ss, d);
          if (lc == 0 && rv) P.ss_partial[(int64_t)(tn * CFG::WAVES_N + wn) * P.M + row] = ss;
        }
      }
    } else if constexpr (EPI == kEpiSwiGLUBwd) {
      // gradient of silu(g)*u with respect to the gate and up accumulators (row scale
      // fixed): columns out and N + out of a 2N-wide output
      constexpr int HF = CFG::FN / 2;
      const int out0 = n0 + wn * (CFG::WN / 2);
      const uint16_t* dO = static_cast<const uint16_t*>(P.dout);
#pragma unroll
      for (int i = 0; i < CFG::FM; ++i) {
        int row = m0 + wm * CFG::WM + i * MI + lr;
        const bool rv = row < P.M;
        const float r = rv ? rsqrtf(P.rms_ss[row] * P.rms_inv_n + P.rms_eps) * P.alpha : 0.f;
        float rsum = 0.f;  // this lane's share of the row-scale gradient (times r)
#pragma unroll
        for (int j = 0; j < HF; ++j)
#pragma unroll
          for (int q = 0; q < G4; ++q) {
            const int col = out0 + j * MI + q * (256 / MI) + 4 * lc;
            const int nv = P.N - col;
            if (!rv || nv <= 0) continue;
            uint32_t og[4], ou[4], dv[4];
            const int64_t doff = (int64_t)row * P.ldd + col;
            if (VEC && nv >= 4 && P.ldd % 4 == 0 &&
                (reinterpret_cast<uintptr_t>(dO) & 7) == 0) {  // 8-byte aligned group of 4
              const v2u w = *reinterpret_cast<const v2u*>(dO + doff);
              dv[0] = w.x & 0xffff; dv[1] = w.x >> 16; dv[2] = w.y & 0xffff; dv[3] = w.y >> 16;
            } else {
#pragma unroll
              for (int s = 0; s < 4; ++s) dv[s] = s < nv ? dO[doff + s] : 0u;
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const float d = to_f32<ODT>(dv[s]);
              const float g = r * acc[i][j][4 * q + s];
              const float u = r * acc[i][j + HF][4 * q + s];
              const float sg = 1.f / (1.f + __expf(-g));
              const float dsilu = sg * (1.f + g * (1.f - sg));
              og[s] = from_f32<ODT>(d * u * dsilu * r);
              ou[s] = from_f32<ODT>(d * g * sg * r);
              rsum += d * (dsilu * g * u + g * sg * u);
            }
            const int64_t off = (int64_t)row * P.ldc + col;
            if (VEC && nv >= 4 && P.N % 4 == 0) {
              *reinterpret_cast<v2u*>(C + off) = v2u{og[0] | (og[1] << 16), og[2] | (og[3] << 16)};
              *reinterpret_cast<v2u*>(C + off + P.N) =
                  v2u{ou[0] | (ou[1] << 16), ou[2] | (ou[3] << 16)};
            } else {
#pragma unroll
              for (int s = 0; s < 4; ++s)
                if (s < nv) {
                  C[off + s] = (uint16_t)og[s];
                  C[off + P.N + s] = (uint16_t)ou[s];
                }
            }
          }
        if (P.rms_grad_out) {
          // lanes of one row in a fixed butterfly; the partial carries alpha/r so the
          // partials of a row sum to the row-scale gradient
#pragma unroll
          for (int d = MI; d < 64; d <<= 1) rsum += __shfl_xor(rsum, d);
          if (lc == 0 && rv)
            P.ss_partial[(int64_t)(tn * CFG::WAVES_N + wn) * P.M + row] = rsum * P.alpha / r;
        }
      }
    } else if constexpr (EPI == kEpiRmsBwd) {
      // alpha*acc + c_i*X with c_i = -r_i^3 * grad_i / n (beta is 0)
      const uint16_t* X = static_cast<const uint16_t*>(P.rms_x);
#pragma unroll
      for (int i = 0; i < CFG::FM; ++i) {
        const int row = m0 + wm * CFG::WM + i * MI + lr;
        if (row >= P.M) continue;
        const float rr = rsqrtf(P.rms_ss[row] * P.rms_inv_n + P.rms_eps);
        const float c = -rr * rr * rr * P.rms_grad[row] * P.rms_inv_n;
#pragma unroll
        for (int j = 0; j < CFG::FN; ++j)
#pragma unroll
          for (int q = 0; q < G4; ++q) {
            const int col = n0 + wn * CFG::WN + j * MI + q * (256 / MI) + 4 * lc;
            const int nv = P.N - col;
            if (nv <= 0) continue;
            const int64_t off = (int64_t)row * P.ldc + col;
            const int64_t xo = (int64_t)row * P.ldx + col;
            uint32_t xv[4], o[4];
            const bool v4 = VEC && nv >= 4 && P.ldx % 4 == 0 &&
                            (reinterpret_cast<uintptr_t>(X) & 7) == 0;  // 8-byte aligned groups
            if (v4) {
              const v2u w = *reinterpret_cast<const v2u*>(X + xo);
              xv[0] = w.x & 0xffff; xv[1] = w.x >> 16; xv[2] = w.y & 0xffff; xv[3] = w.y >> 16;
            } else {
#pragma unroll
              for (int s = 0; s < 4; ++s) xv[s] = s < nv ? X[xo + s] : 0u;
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
              o[s] = from_f32<ODT>(P.alpha * acc[i][j][4 * q + s] + c * to_f32<ODT>(xv[s]));
            if (v4) {
              *reinterpret_cast<v2u*>(C + off) = v2u{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
            } else {
#pragma unroll
              for (int s = 0; s < 4; ++s)
                if (s < nv) C[off + s] = (uint16_t)o[s];
            }
          }
      }
    } else {  // kEpiSwiGLU: output tile is BM x BN/2
      constexpr int HF = CFG::FN / 2;
      const int out0 = n0 + wn * (CFG::WN / 2);
#pragma unroll
      for (int i = 0; i < CFG::FM; ++i) {
        int row = m0 + wm * CFG::WM + i * MI + lr;
        if (row >= P.M) continue;
        float r = rsqrtf(P.rms_ss[row] * P.rms_inv_n + P.rms_eps) * P.alpha;
#pragma unroll
        for (int j = 0; j < HF; ++j)
#pragma unroll
          for (int q = 0; q < G4; ++q) {
            int col = out0 + j * MI + q * (256 / MI) + 4 * lc;
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
              for (int s = 0; s < 4; ++s) v[s] += s < nv ? P.beta * to_f32<ODT>(Cin[off + s]) : 0.f;
            }
            uint32_t o[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) o[s] = from_f32<ODT>(v[s]);
            if (VEC && nv >= 4) {
              *reinterpret_cast<v2u*>(C + off) = v2u{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
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

// Position of a workgroup inside one round of `G` items.  Ids are dealt
// round-robin over the 8 XCDs; renumber so that the workgroups of one XCD take a
// contiguous range of the round.
__device__ __forceinline__ int xcd_slot(int bid, int G) {
  int xcd = bid & 7, idx = bid >> 3;
  int base = G >> 3, rem = G & 7;
  return xcd * base + (xcd < rem ? xcd : rem) + idx;
}

// Tile index -> (tile row, tile column), walking groups of 8 tile rows column by
// column, so that the tiles of one XCD share A rows and B columns in L2.
__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int* tm, int* tn) {
  constexpr int G = 8;
  int per_group = G * tiles_n;
  int group = t / per_group;
  int first = group * G;
  int gsz = tiles_m - first < G ? tiles_m - first : G;
  int in = t - group * per_group;
  *tm = first + in % gsz;
  *tn = in / gsz;
}

// One work item: problem z, K slice y, tile (tm, tn).
struct Work {
  int z, y, tm, tn, m0, n0, kt0, ktiles;
  bool fast;
};

template <class T, class CFG, int EPI, bool VEC, bool AK, bool BKC>
__device__ __forceinline__ bool work_of(const GemmBatch& b, int item, int splits, Work* w) {
  const int t = item % b.tiles;
  const int zy = item / b.tiles;
  w->z = zy % b.count;
  w->y = zy / b.count;
  const GemmProblem& P = b.p[w->z];
  const int tiles_m = (P.M + CFG::BM - 1) / CFG::BM;
  const int tiles_n = (P.N + T::OUT_BN - 1) / T::OUT_BN;
  if (t >= tiles_m * tiles_n) return false;
  raster(t, tiles_m, tiles_n, &w->tm, &w->tn);
  w->m0 = w->tm * CFG::BM;
  w->n0 = w->tn * T::OUT_BN;
  // split K: the host makes the phase count a multiple of the split count
  const int ktiles_all = (P.K + CFG::BK - 1) / CFG::BK;
  w->ktiles = ktiles_all / splits;
  w->kt0 = w->y * w->ktiles;
  // Phases with no K tail take the direct-load ring, also on M/N edge tiles
  // (rows and columns past the edge are clamped onto valid memory).  An operand
  // stored M- or N-contiguous moves 8 consecutive rows/columns per 16-byte chunk,
  // and a clamped chunk is moved whole: on an edge tile every chunk must be either
  // wholly inside the matrix or wholly outside, i.e. that edge dimension must be a
  // multiple of 8 (a chunk straddling the edge would land its valid values in the
  // wrong tile positions).  Other edge tiles take the bounds-checked path.
  // Per-lane offsets are 32-bit, which bounds the leading dimensions there.
  const int64_t b_rows = BKC ? (T::SWIGLU ? 2 * (int64_t)P.N : P.N) : CFG::BK;
  w->fast = VEC && (P.K % CFG::BK == 0) &&
            (AK || P.M % 8 == 0 || P.M - w->m0 >= CFG::BM) &&
            (BKC || P.N % 8 == 0 || P.N - w->n0 >= T::OUT_BN) &&
            (int64_t)(AK ? CFG::BM : CFG::BK + 1) * P.lda < (1ll << 31) &&
            (b_rows + 1) * P.ldb < (1ll << 31);
  return true;
}

// Persistent: gridDim.x workgroups (at most what the device holds at once) take
// items in rounds of gridDim.x.  A tile that follows a direct-load tile has its
// first phases loaded during that tile's epilogue.
template <class CFG, int DT, bool AK, bool BKC, int EPI, bool VEC, int ODT = DT>
__global__ __launch_bounds__(CFG::NT, CFG::OCC) void gemm_mfma_kernel(GemmBatch batch) {
  using T = GemmTile<CFG, DT, AK, BKC, EPI, VEC, ODT>;
  // the rotary embedding keeps its pair rates in a table after the stages
  __shared__ __attribute__((aligned(1024)))
  uint8_t smem[CFG::SMEM + (EPI == kEpiRope ? kRopeMaxPairs * sizeof(double) : 0) +
               (T::MX ? 2 * T::MX_BUF : 0)];
  const int tid = threadIdx.x, lane = tid & 63;
  if constexpr (EPI == kEpiRope) {
    double* ft = reinterpret_cast<double*>(smem + CFG::SMEM);
    const GemmProblem& P0 = batch.p[0];
    for (int t = tid; t < P0.rope_hd / 2; t += CFG::NT)
      ft[t] = rope_turns(t, P0.rope_hd, P0.rope_log2_base);
    __syncthreads();
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / CFG::WAVES_N, wn = wave % CFG::WAVES_N;
  const int G = gridDim.x;
  const int splits = EPI == kEpiStore32 && batch.k_splits > 1 ? batch.k_splits : 1;
  const int items = batch.count * splits * batch.tiles;

  int item = xcd_slot(blockIdx.x, G);
  Work cur;
  bool have = false;
  for (; item < items && !have; item += G)
    have = work_of<T, CFG, EPI, VEC, AK, BKC>(batch, item, splits, &cur);
  bool pre = false;
  while (have) {
    Work nxt;
    bool have_next = false;
    for (; item < items && !have_next; item += G)
      have_next = work_of<T, CFG, EPI, VEC, AK, BKC>(batch, item, splits, &nxt);
    const GemmProblem& P = batch.p[cur.z];

    typename T::Acc acc[CFG::FM][CFG::FN];
#pragma unroll
    for (int i = 0; i < CFG::FM; ++i)
#pragma unroll
      for (int j = 0; j < CFG::FN; ++j)
#pragma unroll
        for (int e = 0; e < CFG::ACC; ++e) acc[i][j][e] = 0.f;

    bool issued = false;
    if (cur.ktiles > 0) {
      if (cur.fast) {
        typename T::Next nx{};
        const bool chain = have_next && nxt.fast && nxt.ktiles > 0;
        const GemmProblem& Pn = batch.p[chain ? nxt.z : cur.z];
        if (chain) {
          nx.m0 = nxt.m0;
          nx.n0 = nxt.n0;
          nx.kt0 = nxt.kt0;
          nx.ktiles = nxt.ktiles;
        }
        T::loop_fast(P, cur.m0, cur.n0, smem, wave, wm, wn, lane, cur.kt0, cur.ktiles, pre,
                     chain, Pn, nx, acc);
        issued = chain;
      } else if constexpr (!T::F8) {  // 8-bit calls are whole phases by contract
        T::loop_checked(P, cur.m0, cur.n0, smem, wave, wm, wn, lane, cur.kt0, cur.ktiles, acc);
      }
    }
    void* Cout = P.C;
    if (EPI == kEpiStore32 && splits > 1)
      Cout = static_cast<float*>(P.C) + (int64_t)cur.y * P.M * P.ldc;
    // the SwiGLU backward writes both halves from registers
    if constexpr (VEC && EPI != kEpiSwiGLUBwd && EPI != kEpiRmsBwd)
      T::epilogue_rows(P, Cout, cur.m0, cur.n0, cur.tn, wave, wm, wn, lane, smem, acc);
    else
      T::epilogue(P, Cout, cur.m0, cur.n0, cur.tn, wm, wn, lane, smem, acc);
    pre = issued;
    cur = nxt;
    have = have_next;
  }
}

// ------------------------------------------------------------------ launching
// 256x256: 8 waves (two per SIMD) of 64x128, BK = 64, two stages; measured on the
// 8192^3 bf16 shapes against 4-wave 128x128 waves, 2x4 waves of 128x64, BK = 32
// with 3-5 stages, and 256x128 / 128x256 tiles at two workgroups per CU.  The
// 16x16x32 MFMAs are 1-5 % faster than 32x32x16 (the chip holds a higher clock on
// them).
using Cfg256 = TileCfg<256, 256, 4, 2, 64, 2, 1, 16>;
using Cfg128 = TileCfg<128, 128, 2, 2, 32, 4>;
using Cfg64 = TileCfg<64, 128, 2, 2, 32, 4>;
using Cfg32 = TileCfg<32, 128, 1, 4, 64, 4>;
using Cfg64n = TileCfg<64, 64, 2, 2, 64, 4>;
// 8-bit inputs: 256 x 256 in 4 waves of 128 x 128 (one per SIMD, 256 accumulators in
// AGPRs) in 32x32x64 MFMA blocks, phases of 128 k (64 KB), two stages.  Per phase a
// CU reads half the LDS bytes per MFMA of 8 waves of 64 x 64 on 256 x 128 (which read
// as much LDS as their MFMAs take cycles): 8-13 % faster at 8192^3 and the LLM shapes.
using CfgF8 = TileCfg<256, kF8TileN, 2, kF8WavesN, 64, 2, 1, 32>;
// 4-bit inputs: the same tile and ring (128 bytes a row a phase, now 256 values in
// 4 MFMA steps; two 64 KB stages).  Measured against 64-byte phases in four stages:
// those carry half the MFMA work a phase for the same barrier, waits and scale reads.
using CfgF4 = TileCfg<256, kF8TileN, 2, kF8WavesN, 64, 2, 1, 32>;

template <class CFG, int DT, bool AK, bool BKC, int EPI, bool VEC, int ODT = DT>
static hipError_t launch_t(const GemmBatch& b0, hipStream_t s) {
  GemmBatch b = b0;
  int maxtiles = 0;
  for (int i = 0; i < b.count; ++i) {
    int out_bn = (EPI == kEpiSwiGLU || EPI == kEpiSwiGLUBwd) ? CFG::BN / 2 : CFG::BN;
    int t = ((b.p[i].M + CFG::BM - 1) / CFG::BM) * ((b.p[i].N + out_bn - 1) / out_bn);
    if (t > maxtiles) maxtiles = t;
  }
  if (maxtiles == 0) return hipSuccess;
  b.tiles = maxtiles;
  const int splits = EPI == kEpiStore32 && b.k_splits > 1 ? b.k_splits : 1;
  const int64_t items = (int64_t)maxtiles * splits * b.count;
  if (items > 0x7fffffff) return hipErrorInvalidValue;
  // workgroups resident per CU, asked of the runtime once per instantiation (the
  // kernel's resources are the same on every gfx950 device); racing first calls
  // from several threads ask twice and store the same value
  static std::atomic<int> occ{0};
  int o = occ.load(std::memory_order_relaxed);
  if (o <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &o, gemm_mfma_kernel<CFG, DT, AK, BKC, EPI, VEC, ODT>, CFG::NT, 0) != hipSuccess ||
        o < 1) {
      (void)hipGetLastError();
      o = 1;
    }
    occ.store(o, std::memory_order_relaxed);
  }
  int64_t groups = items;
  if (b.cus > 0 && (int64_t)b.cus * o < groups) groups = (int64_t)b.cus * o;
  hipLaunchKernelGGL((gemm_mfma_kernel<CFG, DT, AK, BKC, EPI, VEC, ODT>), dim3((unsigned)groups),
                     dim3(CFG::NT), 0, s, b);
  return hipGetLastError();
}

}  // namespace fgemm
