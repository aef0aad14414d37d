// gfx950 (CDNA4) kernels of the whole-tensor Muon step.
//
// Kernels in one step, in launch order:
//   momentum  fused M' = beta*M + G, U = G + beta*M' (Nesterov), U stored as
//             X0 (transposed for a tall matrix), per-tile sums of squares (HBM-bound)
//   norm      fixed-order reduction of those sums to s = 1/(||U||_F + eps)
//   T times:
//     gram    A = X X^T          symmetric: upper tiles only, each mirrored
//     square  B = b*A + c*A*A    A symmetric, so A*A is too: upper tiles, mirrored
//     update  X' = a*X + B X     on the last iteration, W -= lr*scale*O instead
//   apply     W -= lr*scale*s*U  only when T = 0
//
// Muon orthogonalises the whole matrix with Newton-Schulz iterations (Canzona
// analysis page, section 2). Those are the repeated products that mix every row
// and column of the gradient (section 3.4, the Atomicity Constraint). The three
// GEMM phases are dense contractions and run on MFMA:
// - bf16 path: v_mfma_f32_32x32x16_bf16, fp32 accumulation;
// - fp32 path: v_mfma_f32_32x32x2f32.
// Each phase is one persistent launch over the tiles of every matrix in the
// batch. Workgroups pull tiles from an atomic queue whose order is longest
// first: the LPT rule the pages use to assign work to ranks (section 3.4,
// "Why LPT ordering matters"), applied here across CUs.
//
// Operands:
// - X X^T and A*A = A A^T (A is symmetric) read both operands along
//   contiguous rows: each MFMA operand is a 16-byte LDS read.
// - B X reads rows of B (symmetric) and X with K as its row index, through the
//   transposing LDS load ds_read_b64_tr_b16. So X is kept in one orientation
//   only.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "muon_internal.h"

namespace muon {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------ element access
//
// Every global access goes through an address_space(1) pointer, so it
// compiles to global_load / global_store. Generic (flat) accesses would also
// count against the LDS wait counter and serialise the GEMM pipeline.

#define MUON_INLINE __device__ __forceinline__ __attribute__((always_inline))

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef u32x4 __attribute__((address_space(1))) g_u32x4;
typedef u32x2 __attribute__((address_space(1))) g_u32x2;
typedef f32x4 __attribute__((address_space(1))) g_f32x4;
typedef u16 __attribute__((address_space(1))) g_u16;
typedef float __attribute__((address_space(1))) g_f32;

MUON_INLINE u32x4 gload16(const void* p) { return *((const g_u32x4*)(p)); }

MUON_INLINE float bf16_to_f32(u16 v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16 with gfx950's v_cvt_pk_bf16_f32: rounds to nearest even under
// the default rounding mode, and a NaN stays a quiet NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
MUON_INLINE u16 f32_to_bf16(float f) { return __builtin_bit_cast(u16, (__bf16)f); }
MUON_INLINE uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <class T> struct Elem;
template <> struct Elem<float> {
  static MUON_INLINE float load(const float* p) { return *((const g_f32*)(p)); }
  static MUON_INLINE void store(float* p, float v) { *((g_f32*)(p)) = v; }
  static MUON_INLINE float lds_load(const float* p) { return *p; }
  static MUON_INLINE float round(float v) { return v; }
  static MUON_INLINE float to_storage(float v) { return v; }
};
template <> struct Elem<u16> {
  static MUON_INLINE float load(const u16* p) { return bf16_to_f32(*((const g_u16*)(p))); }
  static MUON_INLINE void store(u16* p, float v) { *((g_u16*)(p)) = f32_to_bf16(v); }
  static MUON_INLINE float lds_load(const u16* p) { return bf16_to_f32(*p); }
  static MUON_INLINE float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
  static MUON_INLINE u16 to_storage(float v) { return f32_to_bf16(v); }
};

// Four consecutive elements, as one 8-byte (bf16) or 16-byte (fp32) access.
template <class T> struct Vec4;
template <> struct Vec4<float> {
  static MUON_INLINE void load(const float* p, float v[4]) {
    f32x4 t = *((const g_f32x4*)(p));
    v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
  }
  static MUON_INLINE void store(float* p, const float v[4]) {
    f32x4 t = {v[0], v[1], v[2], v[3]};
    *((g_f32x4*)(p)) = t;
  }
};
template <> struct Vec4<u16> {
  static MUON_INLINE void load(const u16* p, float v[4]) {
    u32x2 t = *((const g_u32x2*)(p));
    v[0] = __uint_as_float(t[0] << 16); v[1] = __uint_as_float(t[0] & 0xffff0000u);
    v[2] = __uint_as_float(t[1] << 16); v[3] = __uint_as_float(t[1] & 0xffff0000u);
  }
  static MUON_INLINE void store(u16* p, const float v[4]) {
    u32x2 t;
    t[0] = pack_bf16x2(v[0], v[1]);
    t[1] = pack_bf16x2(v[2], v[3]);
    *((g_u32x2*)(p)) = t;
  }
};

// ------------------------------------------------------------ GEMM engines
//
// Each engine computes one BM x BN output tile, C[i][j] = sum_k P[i][k] Q[j][k]
// (P, Q row-major, K a multiple of BK), and leaves it in MFMA accumulators.
// A 32 x 32 MFMA block D = A B^T puts A's rows in its registers and B's rows
// on its lanes: element r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l % 32].
// The fp32 engine passes (P, Q): lane l holds output column l % 32 and four
// runs of 4 consecutive rows. The bf16 engine passes (Q, P): lane l holds
// output row l % 32 and four runs of 4 consecutive columns, which its
// epilogue writes as 8-byte units. WAVES_M x WAVES_N waves each own a WM x WN
// sub-tile; fewer, larger wave tiles read less LDS per flop.

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4).
// Lane l's bytes land at LDS address lds + 16*l, so one wave instruction
// fills 1 KB of LDS. It is issued from inline asm, with M0 saved and restored
// around it. The compiler then does not track these loads, and would not put a
// conservative vmcnt(0) in front of every LDS read. The engine waits for them
// itself, with the exact counts of its ring of stages. Untracked loads can
// only make the compiler's own vmcnt waits stricter, never looser.
MUON_INLINE void dma16(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds)
      : "memory");
}

template <int N>
MUON_INLINE void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS rows hold BK bf16: S = BK/8 16-byte slots. The slot of chunk c of row
// r is c ^ swz(r). With these swizzles, the rows read by any 8 (32-bank model)
// or 16 (64-bank model) consecutive lanes of an MFMA fragment read hit
// distinct banks. Both depend only on r % 32, so every 32-row fragment block
// shares one set of offsets.
template <int S>
MUON_INLINE int lds_swizzle(int r) {
  if (S == 4) return ((r >> 1) ^ (r >> 3)) & 3;
  return (r & 7) ^ ((r >> 3) & 1);
}

// Q operand stored K-major (QK engines): LDS rows are K indices of 256 bf16
// (512 bytes, 32 slots). The slot of chunk c of row k is c ^ swzk(k), which
// keeps the transposing fragment reads below free of bank conflicts for 32-
// and 64-bank LDS. It depends only on k % 4.
MUON_INLINE int lds_swizzle_k(int k) { return ((k & 1) ? 4 : 0) ^ ((k & 2) ? 10 : 0); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 4 x 16-bit values at the address of lane 4e + i/4, for
// e = 0..3. If lane j of the group points at row k0 + j/4, columns
// n0 + 4(j%4) .. +3 of a K-major tile, lane i gets column n0 + i at rows
// k0 .. k0+3: the B-operand fragment layout of the MFMA.
MUON_INLINE v4i16 lds_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<unsigned char*>(p)));
}

// QK = false: both operands are row-major with K contiguous (C = P Q^T).
// QK = true: Q is row-major with K as its row index (C = P Q), read through
// transposing LDS loads, so no transposed copy of Q is needed.
template <int WAVES_M, int WAVES_N, int BK_, int STAGES_, bool QK>
struct EngineBF16 {
  typedef u16 T;
  static constexpr int BM = 256, BN = 256, BK = BK_;
  static constexpr int STAGES = STAGES_;  // loads run STAGES - 1 K steps ahead
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int NW = NT / 64;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int S = BK / 8;                  // 16-byte slots per P row
  static constexpr int ROW = BK * 2;                // P row bytes
  static constexpr int RPI = 1024 / ROW;            // P rows per DMA wave instruction
  static constexpr int OP_BYTES = BM * ROW;         // one operand tile of one stage (P or Q)
  static constexpr int STAGE_BYTES = 2 * OP_BYTES;
  static constexpr int DPW = OP_BYTES / 1024 / NW;  // DMA instructions per wave per operand
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr bool kStageTile = true;          // epilogue operand tiles go through LDS
  static constexpr bool kQK = QK;
  static MUON_INLINE int wave_m(int w) { return w / WAVES_N; }
  static MUON_INLINE int wave_n(int w) { return w % WAVES_N; }

  // diag_kt0 >= 0 adds diag_coef times a tile of the operands to the
  // product, read while it is in LDS anyway. Update (QK): Q is the X panel of
  // the output tile's columns, and its K steps diag_kt0 .. +BM/BK-1 hold X over
  // the tile's own rows, so the a*X term of X' = a*X + B*X needs no separate
  // read of X. Square: P is the A panel of the tile's rows, and its K steps
  // diag_kt0 .. +BN/BK-1 hold A over the tile's own columns, for the b*A term.
  static MUON_INLINE void run(const u16* __restrict__ P, int64_t ldp, const u16* __restrict__ Q,
                              int64_t ldq, int K, u16* smem, f32x16 (&acc)[FM][FN],
                              int diag_kt0 = -1, float diag_coef = 0.f) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave_m(wave), wn = wave_n(wave);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // DMA plan. P (and Q unless QK): instruction (wave, p) fills rows
    // RPI*(wave*DPW + p) .. +RPI of the stage; lane l carries row + l/S, slot
    // l%S, i.e. the global chunk slot ^ swz(row). QK: instruction (wave, p)
    // fills K rows 2*(wave*DPW + p) .. +1 of 512 bytes; lane l carries row
    // + l/32, slot l%32, i.e. the global chunk slot ^ swzk(row).
    const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
    const u16* gp[DPW];
    const u16* gq[DPW];
#pragma unroll
    for (int p = 0; p < DPW; ++p) {
      const int row = (wave * DPW + p) * RPI + lane / S;
      const int ch = (lane % S) ^ lds_swizzle<S>(row);
      gp[p] = P + row * ldp + ch * 8;
      if (QK) {
        const int kr = (wave * DPW + p) * 2 + (lane >> 5);
        gq[p] = Q + kr * ldq + ((lane & 31) ^ lds_swizzle_k(kr)) * 8;
      } else {
        gq[p] = Q + row * ldq + ch * 8;
      }
    }
    const int64_t qstep = QK ? (int64_t)BK * ldq : BK;  // Q elements per K step
    // The K loop starts at the diagonal window (if any) and wraps around:
    // loop step kt reads operand K step (kt + kt0) mod KT. The window is then
    // the first BM/BK steps, and the steady-state loop carries no diagonal
    // code.
    const int KT = K / BK;
    const int kt0 = diag_kt0 >= 0 ? diag_kt0 : 0;
    auto issue = [&](int kt) __attribute__((always_inline)) {
      const uint32_t st = lds_base + (kt % STAGES) * STAGE_BYTES;
      int ks = kt + kt0;
      if (ks >= KT) ks -= KT;
#pragma unroll
      for (int p = 0; p < DPW; ++p) {
        const uint32_t off = (wave * DPW + p) * 1024;
        dma16(gp[p] + ks * BK, __builtin_amdgcn_readfirstlane(st + off));
        dma16(gq[p] + ks * qstep, __builtin_amdgcn_readfirstlane(st + OP_BYTES + off));
      }
    };
    // P fragment reads: lane l reads row l % 32 of each 32-row block, 16-byte
    // chunk 2*kk + l/32, at slot chunk ^ swz(row).
    const int r32 = lane & 31, h = lane >> 5, sw = lds_swizzle<S>(r32);
    const unsigned char* sb = reinterpret_cast<const unsigned char*>(smem);
    const uint32_t rowp = (wm * WM + r32) * ROW, rowq = OP_BYTES + (wn * WN + r32) * ROW;
    // QK fragment reads: in lane group G = l/16, lane i16 = l%16 points at K
    // row 8*(G/2) + i16/4 (+16 kk, +4 for the upper half) and columns
    // wn*WN + 32j + 16*(G%2) + 4*(i16%4) .. +3.
    const int G = lane >> 4, i16 = lane & 15;
    const uint32_t qrow = OP_BYTES + (8 * (G >> 1) + (i16 >> 2)) * 512;
    uint32_t qcol[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int chunk = (wn * WN + 32 * j + 16 * (G & 1) + 4 * (i16 & 3)) >> 3;
      qcol[j] = ((chunk ^ lds_swizzle_k(i16 >> 2)) << 4) + 8 * (i16 & 1);
    }

    // Register fragments are double-buffered: the reads of sub-step kk+1 are
    // in flight while the MFMAs of sub-step kk run.
    constexpr int KK = BK / 16;
    bf16x8 fp[2][FM], fq[2][FN];
    auto read_frags = [&](int buf, int kt, int kk) __attribute__((always_inline)) {
      const unsigned char* st = sb + (kt % STAGES) * STAGE_BYTES;
      const int fo = (((2 * kk) | h) ^ sw) * 16;
#pragma unroll
      for (int i = 0; i < FM; ++i) fp[buf][i] = *reinterpret_cast<const bf16x8*>(st + rowp + i * 32 * ROW + fo);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (QK) {
          const unsigned char* q = st + qrow + kk * 16 * 512 + qcol[j];
          const v4i16 lo = lds_read_tr(q), hi = lds_read_tr(q + 4 * 512);
          fq[buf][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          fq[buf][j] = *reinterpret_cast<const bf16x8*>(st + rowq + j * 32 * ROW + fo);
        }
      }
    };
    auto mfmas = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[buf][j], fp[buf][i], acc[i][j], 0, 0, 0);
    };
    // Diagonal window: loop steps slab = 0 .. BM/BK - 1 (operand K steps
    // diag_kt0 + slab) hold the output tile's own rows (QK: Q's K rows) or
    // columns (otherwise: P's K columns) slab*BK .. +BK. Accumulator group
    // (i, j, g) of lane l holds row R = wm*WM + 32i + l%32, columns
    // C .. C+3 with C = wn*WN + 32j + 8g + 4(l/32): one 8-byte read of the
    // operand row R - slab*BK (QK) or of P row R at K column C - slab*BK.
    auto diag_add = [&](int kt) __attribute__((always_inline)) {
      const int slab = kt;
      const unsigned char* st = sb + (kt % STAGES) * STAGE_BYTES;
      const int h8 = 8 * h;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (QK) {
            const int k0 = wm * WM + i * 32 - slab * BK;  // K row of the block's first row
            if (k0 < 0 || k0 + 32 > BK) continue;         // block outside this slab
            const int kr = k0 + r32;
            const unsigned char* row = st + OP_BYTES + kr * 512 + h8;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int chunk = (wn * WN + 32 * j + 8 * g) >> 3;
              const u32x2 v = *reinterpret_cast<const u32x2*>(row + ((chunk ^ lds_swizzle_k(kr)) << 4));
              acc[i][j][4 * g + 0] += diag_coef * __uint_as_float(v[0] << 16);
              acc[i][j][4 * g + 1] += diag_coef * __uint_as_float(v[0] & 0xffff0000u);
              acc[i][j][4 * g + 2] += diag_coef * __uint_as_float(v[1] << 16);
              acc[i][j][4 * g + 3] += diag_coef * __uint_as_float(v[1] & 0xffff0000u);
            }
          } else {
            const int kc0 = wn * WN + j * 32 - slab * BK;  // K column of the block's first column
            if (kc0 < 0 || kc0 + 32 > BK) continue;
            const unsigned char* row = st + rowp + i * 32 * ROW + h8;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int chunk = (kc0 + 8 * g) >> 3;
              const u32x2 v = *reinterpret_cast<const u32x2*>(row + ((chunk ^ sw) << 4));
              acc[i][j][4 * g + 0] += diag_coef * __uint_as_float(v[0] << 16);
              acc[i][j][4 * g + 1] += diag_coef * __uint_as_float(v[0] & 0xffff0000u);
              acc[i][j][4 * g + 2] += diag_coef * __uint_as_float(v[1] << 16);
              acc[i][j][4 * g + 3] += diag_coef * __uint_as_float(v[1] & 0xffff0000u);
            }
          }
        }
    };
    constexpr int PS = 2 * DPW;  // DMA instructions per wave per stage
    // Waits until this wave's loads of stage j are done: at most the loads of
    // the later stages already issued, min(STAGES - 2, KT - 1 - j) of them,
    // may still be outstanding.
    auto wait_stage = [&](int j) __attribute__((always_inline)) {
      const int later = KT - 1 - j;
      if (STAGES >= 4 && later >= 2) wait_vmcnt<2 * PS>();
      else if (STAGES >= 3 && later >= 1) wait_vmcnt<PS>();
      else wait_vmcnt<0>();
    };

#pragma unroll
    for (int k = 0; k < STAGES - 1; ++k)
      if (k < KT) issue(k);
    wait_stage(0);
    __syncthreads();
    if (STAGES - 1 < KT) issue(STAGES - 1);
    read_frags(0, 0, 0);
    auto step = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < KK - 1; ++kk) {
        read_frags((kk + 1) & 1, kt, kk + 1);
        mfmas(kk & 1);
      }
      // The last sub-step's MFMAs are issued before the wait and the barrier,
      // so they keep the matrix pipe busy across both, the next DMA issue and
      // the first fragment reads of stage kt+1.
      mfmas((KK - 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      wait_stage(kt + 1);
      // After the barrier, every wave's stage kt+1 is in LDS, and every wave
      // is done reading stage kt, which the next issue overwrites.
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      if (kt + STAGES < KT) issue(kt + STAGES);
      read_frags(0, kt + 1, 0);
    };
    const int window = diag_kt0 >= 0 ? BM / BK : 0;
    int kt = 0;
    for (; kt < window && kt < KT - 1; ++kt) {
      diag_add(kt);
      step(kt);
    }
    for (; kt < KT - 1; ++kt) step(kt);
    if (KT - 1 < window) diag_add(KT - 1);
#pragma unroll
    for (int kk = 0; kk < KK - 1; ++kk) {
      read_frags((kk + 1) & 1, KT - 1, kk + 1);
      mfmas(kk & 1);
    }
    mfmas((KK - 1) & 1);
    // Every wave is done with the ring before the next tile's first loads.
    __syncthreads();
  }
};

// Direct global -> LDS copy of 16 bytes per lane, addressed as a uniform
// 64-bit base plus a per-lane 32-bit byte offset (the saddr form of
// global_load_lds_dwordx4). Same M0 handling as dma16.
MUON_INLINE void dma16s(const void* base_, uint32_t voff, uint32_t lds) {
  // The base must live in SGPRs; read it from the first lane (it is
  // uniform). readfirstlane returns int: each half goes through uint32_t so
  // that the low half is zero-extended, not sign-extended, into 64 bits.
  const uint64_t b = (uint64_t)(uintptr_t)base_;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}

// threadIdx.x behind an empty asm: address arithmetic derived from it stays
// where it is written. Without this the compiler hoists per-lane offsets (of
// the engines' fragment reads and DMA, and of the epilogues) out of the
// persistent tile loop as loop invariants, keeps dozens of them live across
// the GEMM, spills them, and reloads them one by one.
MUON_INLINE int fresh_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Operands of one output tile for Engine4: C = P Q^T over K, or P Q for QK
// engines, with K steps taken from step kt0 on (mod K/BK). diag: the first
// BM/BK loop steps form the diagonal window (see Engine4).
struct Opnd {
  const u16* P;
  int64_t ldp;
  const u16* Q;
  int64_t ldq;
  int K;
  int kt0;
  int diag;
};

// A read-only kernel table viewed through the constant address space: the
// compiler then loads from it with scalar loads, into scalar registers, even
// after the kernel's own stores (through a generic pointer it has to assume
// they may alias, and falls back to vector loads that also wait for every
// store in flight).
template <class T>
MUON_INLINE const __attribute__((address_space(4))) T* kconst(const T* p) {
  return (const __attribute__((address_space(4))) T*)p;
}

MUON_INLINE Tile load_tile(const Tile* tiles, int i) {
  const auto& t = kconst(tiles)[i];
  return Tile{t.mat, t.ij, t.kr, t.slot};
}

MUON_INLINE int64_t uniform64(int64_t v) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  return (int64_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// The same operands, every field read from the first lane. They are uniform
// anyway, but the compiler cannot always prove it (for a tile claimed inside
// the K loop, say), and then it keeps them and all DMA address arithmetic in
// vector registers.
MUON_INLINE Opnd uniform(const Opnd& o) {
  Opnd u;
  u.P = reinterpret_cast<const u16*>(uniform64((int64_t)(uintptr_t)o.P));
  u.ldp = uniform64(o.ldp);
  u.Q = reinterpret_cast<const u16*>(uniform64((int64_t)(uintptr_t)o.Q));
  u.ldq = uniform64(o.ldq);
  u.K = __builtin_amdgcn_readfirstlane(o.K);
  u.kt0 = __builtin_amdgcn_readfirstlane(o.kt0);
  u.diag = __builtin_amdgcn_readfirstlane(o.diag);
  return u;
}

// Four-wave bf16 engine: 2 x 2 waves of 128 x 128 each (accumulators in the
// AGPR half of the register file), K step BK, a ring of STAGES LDS stages.
//
// With one wave per SIMD nothing else hides a stalled instruction stream, so
// the loop issues MFMAs one at a time with the rest of the work between
// them: while MFMA n of a sub-step runs, the wave reads fragment n - 8 of the
// next sub-step (n >= 8), and the DMA instructions of the step STAGES - 1
// ahead are spread over the first MFMAs of the step. Larger wave tiles read a third less LDS per flop
// than the eight-wave layout; on a power-capped chip that is worth more than
// the latency the second wave per SIMD would hide.
//
// The loads are latency-bound, not bandwidth-bound: a CU only streams as many
// bytes per K step as it keeps in flight. With a ring of 2 stages that is one
// K step, and steps then last about one memory round trip whatever the MFMA
// work. K step 32 with 4 stages of 32 KB keeps three steps (96 KB) in flight
// in the same 128 KB of LDS.
//
// Every step issues the loads of one stage, so the vmcnt accounting is the
// same in every step: waiting for step kt+1 leaves STAGES - 2 later stages in
// flight. Steps past the end re-load the last K step (L2-hot) into a stage
// nobody reads; run() drains them before it returns.
//
// The operand layouts, the swizzles, the accumulator layout, the diagonal
// window and the rotated K order are those of EngineBF16.
template <bool QK, int BK_, int STAGES_>
struct Engine4 {
  typedef u16 T;
  static constexpr int BM = 256, BN = 256, BK = BK_, STAGES = STAGES_;
  static constexpr int NT = 256, NW = 4;
  static constexpr int WM = 128, WN = 128, FM = 4, FN = 4;
  static constexpr int S = BK / 8, ROW = BK * 2;     // P rows: S 16-byte slots
  static constexpr int RPI = 1024 / ROW;             // P rows per DMA instruction
  static constexpr int OP_BYTES = BM * ROW;          // per operand and stage
  static constexpr int STAGE_BYTES = 2 * OP_BYTES;
  static constexpr int DPW = OP_BYTES / 1024 / NW;   // DMA instructions per wave and operand
  static constexpr int PS = 2 * DPW;                 // per wave and stage
  static constexpr int KK = BK / 16;                 // sub-steps per K step
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr bool kStageTile = true;
  static constexpr bool kQK = QK;
  static_assert(DPW % 2 == 0 && 16 % PS == 0 && KK % 2 == 0 && (STAGES & (STAGES - 1)) == 0,
                "schedule assumptions");
  // DMA issue slots. A 2-stage ring must have step kt+1's loads issued before
  // the wait in step kt. Load d goes with MFMA 7d/4 (the first 27 MFMAs of
  // the step): issued closer together they compete with the same sub-steps'
  // fragment reads for LDS and the CU's memory path, issued later they arrive
  // late. Measured on the update: one per MFMA is 2.5% slower, one per 2 MFMAs
  // 0.4% slower, one per 2.5 or 3 MFMAs slower again, and two per MFMA right
  // after the barrier 3% slower. A deeper ring loads step kt + STAGES - 1 in
  // step kt, needed steps later, so the loads are spread over the whole step
  // (one per SPREAD MFMAs).
  static constexpr bool SPREAD_ALL = STAGES >= 3;
  static constexpr int SPREAD = SPREAD_ALL ? 16 * KK / PS : 1;
  static constexpr int SLOT_NUM = 7, SLOT_DEN = 4;  // 2-stage ring: load d at MFMA d * 7 / 4
  // The wait for step kt+1 and the barrier come after SPLIT of the last
  // sub-step's 16 MFMAs; the other 16 - SPLIT MFMAs cover the first fragment
  // reads of step kt+1. Measured (step time, same GPU): SPLIT 8 and 10 cost
  // 0.4% and 0.5% more than 12 to 15; the update does best at 12, gram at 14.
  static constexpr int SPLIT = QK ? 12 : 14;
  static constexpr int WAIT_AT = (KK - 1) * 16 + SPLIT;  // MFMAs of a step issued before its wait
  static constexpr int DMA_BEFORE_WAIT = SPREAD_ALL ? (WAIT_AT + SPREAD - 1) / SPREAD : PS;
  // Loads that may still be in flight at the wait for step kt+1: those of
  // steps kt+2 .. kt+STAGES-2 and the ones of step kt+STAGES-1 already issued.
  static constexpr int WAIT_N = (STAGES - 3) * PS + DMA_BEFORE_WAIT;
  static_assert(!SPREAD_ALL || SPREAD * PS == 16 * KK, "spread covers the step");
  static_assert(SPREAD_ALL || (PS - 1) * SLOT_NUM / SLOT_DEN < WAIT_AT, "every load issued before the wait");
  static MUON_INLINE int wave_m(int w) { return w >> 1; }
  static MUON_INLINE int wave_n(int w) { return w & 1; }

  // Computes tile c into acc. A tile long enough for it claims its successor
  // while it runs: claim(0), claim(1) and claim(2, n) are called at three
  // consecutive step boundaries before the last STAGES - 1 steps (claim(2, n)
  // returns whether there is a successor and then sets n). Those last steps
  // load n's first STAGES - 1 steps into the ring, so n starts without
  // waiting for memory; pre: c's own first steps were loaded that way by the
  // previous call. Without a successor, those steps re-load c's last step into
  // stages nobody reads, and run() drains them before returning. K is a
  // multiple of BM, so the step count is a multiple of STAGES and a step past
  // the end maps to n's step of the same ring stage. Returns whether n was
  // set. On return every wave is done with the ring's last stage (n's first
  // steps occupy the others), which the epilogue may use until the next
  // call's first barrier.
  template <class Claim>
  static MUON_INLINE bool run(const Opnd& c, Claim&& claim, Opnd& n, bool pre, u16* smem,
                              f32x16 (&acc)[FM][FN]) {
    const int tid = fresh_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave_m(wave), wn = wave_n(wave);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int KT = c.K / BK;
    bool has_next = false;
    // DMA plan. Instruction p of this wave fills 1 KB of each operand: P rows
    // RPI*(wave*DPW + p) .. +RPI-1 (lane l: row + l/S, slot l%S, global chunk
    // slot ^ swz(row)), Q likewise, or for QK the K rows 2(wave*DPW + p) .. +1
    // (lane l: row + l/32, slot l%32, global chunk slot ^ swzk(row)). With DPW
    // even, swz(row) and swzk(row) depend on p only through p%2: the per-lane
    // part of the address takes two values per operand (and per tile, since
    // the row strides differ).
    auto lane_offsets = [&](int64_t ldp, int64_t ldq, uint32_t (&vp)[2], uint32_t (&vq)[2])
        __attribute__((always_inline)) {
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int prow = (wave * DPW + par) * RPI + lane / S;
        vp[par] = (uint32_t)((lane / S) * ldp * 2) + (((lane % S) ^ lds_swizzle<S>(prow)) << 4);
        if (QK)
          vq[par] = (uint32_t)((lane >> 5) * ldq * 2) +
                    (((lane & 31) ^ lds_swizzle_k(2 * (wave * DPW + par) + (lane >> 5))) << 4);
        else
          vq[par] = (uint32_t)((lane / S) * ldq * 2) + (((lane % S) ^ lds_swizzle<S>(prow)) << 4);
      }
    };
    uint32_t vp[2], vq[2], vpn[2] = {0u, 0u}, vqn[2] = {0u, 0u};
    lane_offsets(c.ldp, c.ldq, vp, vq);
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
    // DMA instruction d (0 .. PS-1) of loop step kt of tile c (kt < KT):
    // even d loads P, odd d loads Q, both for p = d/2.
    auto dma_cur = [&](int kt, int d) __attribute__((always_inline)) {
      int ks = kt;
      if constexpr (!QK) {  // QK tiles run K in order (no window to put first)
        ks += c.kt0;
        if (ks >= KT) ks -= KT;
      }
      const int p = d >> 1, row = wave * DPW + p;
      const uint32_t st = lds_base + (kt & (STAGES - 1)) * STAGE_BYTES + row * 1024;
      if (d & 1) {
        const u16* qb = QK ? c.Q + ((int64_t)ks * BK + 2 * row) * c.ldq : c.Q + (int64_t)(RPI * row) * c.ldq + ks * BK;
        dma16s(qb, vq[p & 1], st + OP_BYTES);
      } else {
        dma16s(c.P + (int64_t)(RPI * row) * c.ldp + ks * BK, vp[p & 1], st);
      }
    };
    // The same for any loop step, including those past the end of c.
    auto dma_any = [&](int kt, int d) __attribute__((always_inline)) {
      const bool past = kt >= KT, nx = past && has_next;
      int ks;
      if (nx) {
        const int KTn = n.K / BK;
        ks = kt - KT;
        if constexpr (!QK) {
          ks += n.kt0;
          if (ks >= KTn) ks -= KTn;
        }
      } else {
        ks = past ? KT - 1 : kt;
        if constexpr (!QK) {
          ks += c.kt0;
          if (ks >= KT) ks -= KT;
        }
      }
      const int p = d >> 1, row = wave * DPW + p;
      const uint32_t st = lds_base + (kt & (STAGES - 1)) * STAGE_BYTES + row * 1024;
      if (d & 1) {
        const u16* Q = nx ? n.Q : c.Q;
        const int64_t ldq = nx ? n.ldq : c.ldq;
        const u16* qb = QK ? Q + ((int64_t)ks * BK + 2 * row) * ldq : Q + (int64_t)(RPI * row) * ldq + ks * BK;
        dma16s(qb, nx ? vqn[p & 1] : vq[p & 1], st + OP_BYTES);
      } else {
        const u16* P = nx ? n.P : c.P;
        const int64_t ldp = nx ? n.ldp : c.ldp;
        dma16s(P + (int64_t)(RPI * row) * ldp + ks * BK, nx ? vpn[p & 1] : vp[p & 1], st);
      }
    };

    // Fragment reads. P: lane l reads row l%32 of each 32-row block, 16-byte
    // chunk 2*kk + l/32 at slot chunk ^ swz(row). Q (not QK): the same on Q
    // rows. QK: two transposing reads per fragment, as in EngineBF16.
    const int r32 = lane & 31, h = lane >> 5, sw = lds_swizzle<S>(r32);
    const unsigned char* sb = reinterpret_cast<const unsigned char*>(smem);
    const uint32_t rowp = (wm * WM + r32) * ROW, rowq = OP_BYTES + (wn * WN + r32) * ROW;
    const int G = lane >> 4, i16 = lane & 15;
    const uint32_t qrow = OP_BYTES + (8 * (G >> 1) + (i16 >> 2)) * 512;
    uint32_t qcol[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int chunk = (wn * WN + 32 * j + 16 * (G & 1) + 4 * (i16 & 3)) >> 3;
      qcol[j] = ((chunk ^ lds_swizzle_k(i16 >> 2)) << 4) + 8 * (i16 & 1);
    }
    bf16x8 fp[2][FM], fq[2][FN];
    // Read item f (0..3: P block f, 4..7: Q block f-4) of sub-step kk of loop
    // step kt into buffer buf.
    auto rd = [&](int buf, int kt, int kk, int f) __attribute__((always_inline)) {
      const unsigned char* st = sb + (kt & (STAGES - 1)) * STAGE_BYTES;
      const int fo = (((2 * kk) | h) ^ sw) * 16;
      if (f < FM) {
        fp[buf][f] = *reinterpret_cast<const bf16x8*>(st + rowp + f * 32 * ROW + fo);
      } else if (QK) {
        const unsigned char* q = st + qrow + kk * 16 * 512 + qcol[f - FM];
        const v4i16 lo = lds_read_tr(q), hi = lds_read_tr(q + 4 * 512);
        fq[buf][f - FM] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        fq[buf][f - FM] = *reinterpret_cast<const bf16x8*>(st + rowq + (f - FM) * 32 * ROW + fo);
      }
    };
    // MFMA n (block i = n/4, j = n%4) on buffer buf: Q fragment first, so
    // lane l%32 indexes output rows (the accumulator layout of EngineBF16).
    auto mf = [&](int buf, int n) __attribute__((always_inline)) {
      const int i = n >> 2, j = n & 3;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[buf][j], fp[buf][i], acc[i][j], 0, 0, 0);
    };

    // Diagonal window (loop steps 0 .. BM/BK - 1, when c.diag): the
    // term added is 1 * (the operand tile at the output tile's own rows or
    // columns), added by MFMAs against 0/1 selection fragments
    // I_t[c][k] = (c == 16t + k) over the 16 K values of a sub-step. Step s
    // holds output rows (QK) or columns s*BK .. +BK-1, owned by the waves with
    // wm (QK) or wn equal to s*BK/128, in accumulator block
    // (s*BK % 128)/32 + kk/2; sub-step kk covers half t = kk%2 of it. The
    // fragments the sub-step already holds are the operand values:
    //  - QK (update, X' = X + B X): fq[j] holds X[row][col] with the column
    //    on lanes, so D += fq[j] * I_t^T adds X to block (blk, j);
    //  - otherwise (square, A' A' + A'): fp[i] holds P[row][k] with the row
    //    on lanes, so D += I_t * fp[i] adds A' to block (i, blk).
    // The diagonal coefficient is 1.
    bf16x8 sel[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sel[t][e] = (__bf16)(r32 == 16 * t + 8 * h + e ? 1.f : 0.f);

#define MUON_SB() __builtin_amdgcn_sched_barrier(0)
    // One loop step kt. Fragments of sub-step 0 are in buffer 0 on entry; on
    // exit those of step kt+1 are (after the last step, reads of a stage
    // nobody uses). WIN >= 0: a diagonal-window step whose first accumulator
    // block is WIN; the waves that do not own the step's slab add 0 (their
    // selection fragments are zero), so every wave runs the same code.
    // TAIL: the step may load past the end of c (the last STAGES - 1 steps,
    // and the window steps, which may be among them).
    auto kstep = [&](int kt, auto WIN_, auto TAIL_) __attribute__((always_inline)) {
      constexpr int WIN = decltype(WIN_)::value;
      constexpr bool TAIL = decltype(TAIL_)::value;
      bf16x8 ds[2];
      if constexpr (WIN >= 0) {
        const bool own = ((kt * BK) >> 7) == (QK ? wm : wn);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          ds[t] = own ? sel[t] : __builtin_bit_cast(bf16x8, z);
        }
      }
      auto diag = [&](int buf, int kk) __attribute__((always_inline)) {
        if constexpr (WIN >= 0) {
          const int blk = WIN + (kk >> 1);
#pragma unroll
          for (int o = 0; o < 4; ++o) {
            if (QK) acc[blk][o] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[buf][o], ds[kk & 1], acc[blk][o], 0, 0, 0);
            else acc[o][blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ds[kk & 1], fp[buf][o], acc[o][blk], 0, 0, 0);
          }
        }
      };
      // DMA slot of MFMA g (0 .. 16*KK - 1) of the step.
      auto dma_slot = [&](int g) __attribute__((always_inline)) {
        if constexpr (SPREAD_ALL) {
          if (g % SPREAD == 0) {
            if constexpr (TAIL) dma_any(kt + STAGES - 1, g / SPREAD);
            else dma_cur(kt + STAGES - 1, g / SPREAD);
          }
        } else {
#pragma unroll
          for (int d = 0; d < PS; ++d)
            if (g == d * SLOT_NUM / SLOT_DEN) {
              if constexpr (TAIL) dma_any(kt + STAGES - 1, d);
              else dma_cur(kt + STAGES - 1, d);
            }
        }
      };
#pragma unroll
      for (int kk = 0; kk < KK - 1; ++kk) {
        const int b = kk & 1;
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          mf(b, n);
          // The next sub-step's 8 fragments are read under this sub-step's
          // second half: away from the DMA issue, which falls mostly in the
          // first half (0.4% faster than reading under the first half; one
          // read per 7/4 or 2 MFMAs is 1-2% slower).
#pragma unroll
          for (int f = 0; f < 8; ++f)
            if (f + 8 == n) rd(b ^ 1, kt, kk + 1, f);
          dma_slot(16 * kk + n);
          MUON_SB();
        }
        diag(b, kk);
        MUON_SB();
      }
      // Last sub-step (buffer 1): SPLIT MFMAs, then wait for this wave's
      // loads of step kt+1 and the barrier (after it every wave's loads of
      // that step are in LDS and every wave is done with this step's stage,
      // which the next step's DMA overwrites), then the other MFMAs under the
      // 8 first reads of the next step.
#pragma unroll
      for (int n = 0; n < SPLIT; ++n) {
        mf(1, n);
        dma_slot(16 * (KK - 1) + n);
        MUON_SB();
      }
      wait_vmcnt<WAIT_N>();
      __syncthreads();
      MUON_SB();
#pragma unroll
      for (int n = SPLIT; n < 16; ++n) {
        mf(1, n);
#pragma unroll
        for (int f = 0; f < 8; ++f)
          if (f * (16 - SPLIT) / 8 == n - SPLIT) rd(0, kt + 1, 0, f);
        dma_slot(16 * (KK - 1) + n);
        MUON_SB();
      }
      diag(1, KK - 1);  // buffer 1 is intact: the reads above fill buffer 0
      MUON_SB();
    };
#undef MUON_SB
    using NOWIN = std::integral_constant<int, -1>;

    if (pre) {
      // Step 0 was issued before the previous tile's epilogue, whose stores
      // came after it: wait for everything (those stores are nearly done).
      wait_vmcnt<0>();
    } else {
#pragma unroll
      for (int k = 0; k < STAGES - 1; ++k)
#pragma unroll
        for (int d = 0; d < PS; ++d) dma_cur(k, d);
      wait_vmcnt<(STAGES - 2) * PS>();
    }
    __syncthreads();
#pragma unroll
    for (int f = 0; f < 8; ++f) rd(0, 0, 0, f);
    // K >= BM, so the window's BM/BK steps all exist. A tile claims its
    // successor only if the claim steps come after the window.
    using F_ = std::false_type;
    using T_ = std::true_type;
    constexpr int WSTEPS = BM / BK;
    const int CL = KT - (STAGES - 1) - 3;  // first claim step
    const bool win = !QK && c.diag;        // QK tiles (the update) have no diagonal window
    const bool late = CL >= (win ? WSTEPS : 0);
    int kt = 0;
    auto window = [&](auto TAIL_) __attribute__((always_inline)) {
      if constexpr (QK) return;
      for (int g = 0; g < BM / 128; ++g) {
        if constexpr (BK == 64) {
          kstep(kt, std::integral_constant<int, 0>{}, TAIL_);
          kstep(kt + 1, std::integral_constant<int, 2>{}, TAIL_);
          kt += 2;
        } else {
          kstep(kt, std::integral_constant<int, 0>{}, TAIL_);
          kstep(kt + 1, std::integral_constant<int, 1>{}, TAIL_);
          kstep(kt + 2, std::integral_constant<int, 2>{}, TAIL_);
          kstep(kt + 3, std::integral_constant<int, 3>{}, TAIL_);
          kt += 4;
        }
      }
    };
    if (late) {
      if (win) window(F_{});
      for (; kt < CL; ++kt) kstep(kt, NOWIN{}, F_{});
      kstep(kt, NOWIN{}, F_{});
      claim(0, n);
      kstep(kt + 1, NOWIN{}, F_{});
      claim(1, n);
      kstep(kt + 2, NOWIN{}, F_{});
      has_next = claim(2, n);
      if (has_next) lane_offsets(n.ldp, n.ldq, vpn, vqn);
      kt += 3;
    } else {
      // Short tile (only the window and a few steps): no successor.
      if (win) window(T_{});
      for (; kt < KT - (STAGES - 1); ++kt) kstep(kt, NOWIN{}, F_{});
    }
    for (; kt < KT; ++kt) kstep(kt, NOWIN{}, T_{});
    if (!has_next) wait_vmcnt<0>();
    return has_next;
  }
};

template <bool QK>
struct EngineF32 {
  typedef float T;
  static constexpr int BM = 128, BN = 128, BK = 32, NT = 256;
  static constexpr int WM = 64, WN = 64;     // wave tile: 4 waves as 2 x 2
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int LDS_STRIDE = BK + 1;  // floats; odd stride spreads rows over banks
  static constexpr int QK_STRIDE = BN + 4;   // floats per K row of a K-major Q tile
  static constexpr int PART = BM * LDS_STRIDE;  // = BK * QK_STRIDE: P and Q parts are the same size
  static constexpr int STAGE = 2 * PART;
  static constexpr int LDS_BYTES = 2 * STAGE * 4;
  static constexpr bool kStageTile = false;
  static constexpr bool kQK = QK;
  static MUON_INLINE int wave_m(int w) { return w >> 1; }
  static MUON_INLINE int wave_n(int w) { return w & 1; }
  static_assert(BM * LDS_STRIDE == BK * QK_STRIDE, "P and Q parts of a stage differ in size");

  static MUON_INLINE void run(const float* __restrict__ P, int64_t ldp, const float* __restrict__ Q,
                              int64_t ldq, int K, float* smem, f32x16 (&acc)[FM][FN], int = -1, float = 0.f) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave_m(wave), wn = wave_n(wave);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // P: 128 rows x 32 floats (8 chunks per row). Q, QK: 32 K rows x 128
    // floats (32 chunks per row); otherwise like P.
    u32x4 rp[4], rq[4];
    auto gload = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int q = tid + p * NT;
        rp[p] = gload16(P + (q >> 3) * ldp + k0 + (q & 7) * 4);
        if (QK) rq[p] = gload16(Q + (int64_t)(k0 + (q >> 5)) * ldq + (q & 31) * 4);
        else rq[p] = gload16(Q + (q >> 3) * ldq + k0 + (q & 7) * 4);
      }
    };
    auto sstore = [&](int s) __attribute__((always_inline)) {
      float* sp = smem + s * STAGE;
      float* sq = sp + PART;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int q = tid + p * NT;
        float* dp = sp + (q >> 3) * LDS_STRIDE + (q & 7) * 4;
        float* dq = QK ? sq + (q >> 5) * QK_STRIDE + (q & 31) * 4 : sq + (q >> 3) * LDS_STRIDE + (q & 7) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dp[e] = __uint_as_float(rp[p][e]);
          dq[e] = __uint_as_float(rq[p][e]);
        }
      }
    };

    const int KT = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int s = kt & 1;
      if (kt + 1 < KT) gload((kt + 1) * BK);
      const float* sp = smem + s * STAGE + (wm * WM + (lane & 31)) * LDS_STRIDE + (lane >> 5);
      const float* sq = QK ? smem + s * STAGE + PART + (lane >> 5) * QK_STRIDE + wn * WN + (lane & 31)
                           : smem + s * STAGE + PART + (wn * WN + (lane & 31)) * LDS_STRIDE + (lane >> 5);
#pragma unroll
      for (int kk = 0; kk < BK / 2; ++kk) {
        float fp[FM], fq[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) fp[i] = sp[i * 32 * LDS_STRIDE + kk * 2];
#pragma unroll
        for (int j = 0; j < FN; ++j) fq[j] = QK ? sq[kk * 2 * QK_STRIDE + j * 32] : sq[j * 32 * LDS_STRIDE + kk * 2];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fp[i], fq[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < KT) sstore(s ^ 1);
      __syncthreads();
    }
  }
};

// ------------------------------------------------------------ phase epilogues
//
// fp32 engine: the epilogue walks the accumulators in groups of four
// consecutive rows of one column and stores straight from them.
//
// bf16 engines: a lane's accumulator group holds four consecutive columns of
// one row. The epilogue writes the scaled tile to an LDS staging tile as bf16
// (one 8-byte write per group), and then copies
// the staging tile to global memory in coalesced 16-byte stores, once per
// output orientation. Entries outside the matrix are zeroed in LDS; only tiles
// on the matrix edge need that pass.

template <class E>
struct TileWalk {
  // fp32 engine layout. Calls f(row0, col, v[4]) for every 4-row group of the
  // tile at (tile_r, tile_c).
  template <class F>
  static MUON_INLINE void each(int64_t tile_r, int64_t tile_c, f32x16 (&acc)[E::FM][E::FN], F&& f) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t wr = tile_r + E::wave_m(wave) * E::WM + 4 * (lane >> 5);
    const int64_t wc = tile_c + E::wave_n(wave) * E::WN + (lane & 31);
#pragma unroll
    for (int i = 0; i < E::FM; ++i)
#pragma unroll
      for (int j = 0; j < E::FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                        acc[i][j][4 * g + 3]};
          f(wr + i * 32 + 8 * g, wc + j * 32, v);
        }
  }
};

// Valid extent of a tile at (tr, tc) of an m x n matrix, in tile-local rows
// and columns (at most BM x BN).
template <class E>
MUON_INLINE int tile_rows(int64_t tr, int m) { return (int)(m - tr < E::BM ? m - tr : E::BM); }
template <class E>
MUON_INLINE int tile_cols(int64_t tc, int n) { return (int)(n - tc < E::BN ? n - tc : E::BN); }

// Stores a symmetric m x m result tile straight from the accumulators:
// C[row][col] and the mirror C[col][row] (off-diagonal tiles only). Entries
// outside the valid m x m block are 0.
template <class T>
MUON_INLINE void store_sym(T* C, int64_t ld, int m, bool mirror, int64_t row0, int64_t col, float v[4]) {
  const bool cok = col < m;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (!(cok && row0 + q < m)) v[q] = 0.f;
    Elem<T>::store(C + (row0 + q) * ld + col, v[q]);
  }
  if (mirror) Vec4<T>::store(C + col * ld + row0, v);
}

// Output staging tile: 256 rows of 256 bf16 (512 bytes each), in 8-byte units
// of four columns. Unit u of row r is stored at unit u ^ stage_swz(r) of that
// row. stage_swz is a bijection of r % 32 chosen so that the three access
// patterns below hit distinct banks, for 32- and for 64-bank LDS:
//  - the accumulator writes: 32 consecutive rows, one unit;
//  - row reads: one row, 16 bytes per lane;
//  - transposing reads: 4 consecutive rows by 4 consecutive units per 16
//    lanes, two such groups 8 rows apart per 32 lanes.
constexpr int kOutStride = 512;
constexpr int kOutBytes = 256 * kOutStride;

MUON_INLINE int stage_swz(int r) {
  return ((r >> 2) & 1) | (((r >> 3) & 1) << 1) | ((r & 3) << 2) | ((((r >> 3) ^ (r >> 4)) & 1) << 4);
}
MUON_INLINE int stage_off(int r, int u) { return r * kOutStride + ((u ^ stage_swz(r)) << 3); }


MUON_INLINE u32x4 bf16x8_bits(v4i16 lo, v4i16 hi) {
  return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Columns 8ch .. 8ch+7 of staging row r. The two units of the chunk sit in one
// 16-byte slot, swapped when stage_swz(r) is odd.
MUON_INLINE u32x4 stage_read_row8(const unsigned char* smem, int r, int ch) {
  const int sw = stage_swz(r);
  const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * kOutStride + ((ch ^ (sw >> 1)) << 4));
  if (sw & 1) return u32x4{v[2], v[3], v[0], v[1]};
  return v;
}

// Transposing read. In each group of 16 lanes, lane i receives rows
// r0 .. r0+7 of column c0 + i, where c0 is a multiple of 16 and r0 a multiple
// of 8 (both uniform over the group). Lane i addresses row r0 + i/4 (and
// r0 + 4 + i/4), unit c0/4 + i%4.
MUON_INLINE u32x4 stage_read_col8(const unsigned char* smem, int r0, int c0, int tid) {
  const int i = tid & 15;
  const int u = (c0 >> 2) + (i & 3);
  const v4i16 lo = lds_read_tr(smem + stage_off(r0 + (i >> 2), u));
  const v4i16 hi = lds_read_tr(smem + stage_off(r0 + 4 + (i >> 2), u));
  return bf16x8_bits(lo, hi);
}

// bf16 accumulator tile, times scale, -> staging tile. Lane l's group
// (i, j, g) holds row wm*WM + 32i + l%32, columns wn*WN + 32j + 8g + 4(l/32)
// .. +3: one unit. The scale is applied here, where every accumulator is read
// once anyway, rather than in a pass of its own.
template <class E>
MUON_INLINE void acc_to_lds(f32x16 (&acc)[E::FM][E::FN], unsigned char* smem, float scale) {
  // Row wr + 32i has stage_swz(lane % 32); unit wu + 8j + 2g, where wu's set
  // bits and those of 8j + 2g are disjoint, sits at (wu ^ swz) ^ (8j + 2g).
  const int tid = fresh_tid(), lane = tid & 63, wave = tid >> 6;
  const int wr = E::wave_m(wave) * E::WM + (lane & 31);
  const int wu = E::wave_n(wave) * (E::WN / 4) + (lane >> 5);
  static_assert(E::WN / 4 >= 8 * E::FN, "unit bits of wu and 8j + 2g must not overlap");
  unsigned char* row = smem + wr * kOutStride;
  const int ux = (wu ^ stage_swz(lane & 31)) << 3;
#pragma unroll
  for (int j = 0; j < E::FN; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      unsigned char* p = row + (ux ^ ((8 * j + 2 * g) << 3));
#pragma unroll
      for (int i = 0; i < E::FM; ++i) {
        u32x2 t;
        t[0] = pack_bf16x2(scale * acc[i][j][4 * g], scale * acc[i][j][4 * g + 1]);
        t[1] = pack_bf16x2(scale * acc[i][j][4 * g + 2], scale * acc[i][j][4 * g + 3]);
        *reinterpret_cast<u32x2*>(p + i * 32 * kOutStride) = t;
      }
    }
}

// Zeroes the staging entries at rows >= rl or columns >= cl. Called between
// two barriers, for edge tiles only.
template <int NT>
MUON_INLINE void mask_lds(unsigned char* smem, int rl, int cl) {
  const int tid = fresh_tid();
#pragma unroll 1
  for (int p = 0; p < 256 * 64 / NT; ++p) {
    const int idx = tid + p * NT, r = idx >> 6, u = idx & 63;
    const int keep = r < rl ? cl - 4 * u : 0;  // valid columns in this unit
    if (keep >= 4) continue;
    u32x2* q = reinterpret_cast<u32x2*>(smem + stage_off(r, u));
    u32x2 v = *q;
    if (keep <= 0) { v[0] = 0u; v[1] = 0u; }
    else if (keep == 1) { v[0] &= 0xffffu; v[1] = 0u; }
    else if (keep == 2) { v[1] = 0u; }
    else { v[1] &= 0xffffu; }
    *q = v;
  }
}

// Staging tile -> the 256 x 256 tile at dst (row stride ld): 32 lanes per row.
template <int NT>
MUON_INLINE void lds_to_global(const unsigned char* smem, u16* dst, int64_t ld) {
  const int tid = fresh_tid();
#pragma unroll 2
  for (int p = 0; p < 256 * 32 / NT; ++p) {
    const int idx = tid + p * NT, row = idx >> 5, ch = idx & 31;
    *((g_u32x4*)(dst + row * ld + ch * 8)) = stage_read_row8(smem, row, ch);
  }
}

// Staging tile -> the transpose of the tile at dst_t: row c of dst_t gets
// column c of the staging tile. Wave task t covers columns 16(t%16) .. +15 and
// rows 32(t/16) .. +31; its 4 lane groups take 8 rows each, so every dst_t row
// receives 64 contiguous bytes per store instruction.
template <int NT>
MUON_INLINE void lds_to_global_t(const unsigned char* smem, u16* dst_t, int64_t ld_t) {
  constexpr int NW = NT / 64;
  const int tid = fresh_tid();
  const int wave = tid >> 6, G = (tid >> 4) & 3, i = tid & 15;
#pragma unroll 2
  for (int p = 0; p < 128 / NW; ++p) {
    const int t = wave + p * NW;
    const int c0 = 16 * (t & 15), r0 = 32 * (t >> 4) + 8 * G;
    *((g_u32x4*)(dst_t + (c0 + i) * ld_t + r0)) = stage_read_col8(smem, r0, c0, tid);
  }
}

// Writes scale times the accumulator tile to dst and, if dst_t is set, its
// transpose to dst_t, through one staging pass. Entries outside the first rl
// rows and cl columns are written as 0. LDS must be free on entry; it is free
// again on exit.
template <class E>
MUON_INLINE void store_tile_staged(f32x16 (&acc)[E::FM][E::FN], unsigned char* smem, float scale, int rl,
                                   int cl, u16* dst, int64_t ld, u16* dst_t, int64_t ld_t) {
  acc_to_lds<E>(acc, smem, scale);
  __syncthreads();
  if (rl < E::BM || cl < E::BN) {
    mask_lds<E::NT>(smem, rl, cl);
    __syncthreads();
  }
  lds_to_global<E::NT>(smem, dst, ld);
  if (dst_t) lds_to_global_t<E::NT>(smem, dst_t, ld_t);
  __syncthreads();
}

// bf16 path: the polynomial is folded so that both diagonal terms have
// coefficient 1, which the engines add exactly (Engine4 with MFMAs against 0/1
// fragments). With a' = a (1 if a = 0) and, when b, c != 0, g = c/b:
//   gram stores    A' = g * A
//   square stores  B' = B / a' = (b^2 / (c a')) * (A' A' + A')
//   update forms   X_next = a X + B X = a' * (X + B' X)      (a != 0)
//                         = B' X                              (a = 0)
// b = 0 or c = 0 keep g = 1: B' = (c/a') A A, or the elementwise (b/a') A.
// The four-wave kernels fold the update's identity term into the square's
// output instead: it stores B'' = B' + I (a != 0), with the 1 added in fp32
// before the one rounding to bf16, and the update forms a' * B'' X. Late in
// the iteration X X^T is close to I and B' close to -0.8 I, so rounding
// 1 + B'_ii once loses less than rounding B'_ii and adding 1 exactly; and the
// update tiles need no diagonal window, so all of them run K in one order.
struct Fold {
  float g;      // gram output scale (times s^2 on the first iteration)
  float sq;     // square output scale
  int sq_mode;  // 0: elementwise B' = sq * A; 1: product only; 2: product + diagonal
  float up;     // update output scale (times s on the first iteration)
  bool up_diag;
};
MUON_INLINE Fold fold_coeffs(const StepCoeffs& co) {
  Fold f;
  const float ap = co.a != 0.f ? co.a : 1.f;
  if (co.b != 0.f && co.c != 0.f) {
    f.g = co.c / co.b; f.sq = co.b * co.b / co.c / ap; f.sq_mode = 2;
  } else if (co.c == 0.f) {
    f.g = 1.f; f.sq = co.b / ap; f.sq_mode = 0;
  } else {
    f.g = 1.f; f.sq = co.c / ap; f.sq_mode = 1;
  }
  f.up = ap;
  f.up_diag = co.a != 0.f;
  return f;
}

template <class E>
MUON_INLINE void gram_tile(const PhaseArgs& args, const MatDev& d, int ti, int tj, void* smem) {
  typedef typename E::T T;
  const T* X = static_cast<const T*>(d.x[args.src]);
  f32x16 acc[E::FM][E::FN];
  E::run(X + (int64_t)ti * E::BM * d.ldx, d.ldx, X + (int64_t)tj * E::BN * d.ldx, d.ldx, d.np,
         static_cast<T*>(smem), acc);
  // First iteration: X holds the unscaled U, so A = s^2 U U^T.
  float alpha = 1.f;
  if (args.first) {
    const float s = args.scale[&d - args.mats];
    alpha = s * s;
  }
  T* A = static_cast<T*>(d.a);
  const bool mirror = ti != tj;
  const int64_t tr = (int64_t)ti * E::BM, tc = (int64_t)tj * E::BN;
  const int m = d.m;
  if constexpr (E::kStageTile) {
    alpha *= fold_coeffs(args.co).g;
    store_tile_staged<E>(acc, static_cast<unsigned char*>(smem), alpha, tile_rows<E>(tr, m), tile_cols<E>(tc, m),
                         A + tr * d.lda + tc, d.lda, mirror ? A + tc * d.lda + tr : nullptr, d.lda);
  } else {
    TileWalk<E>::each(tr, tc, acc, [&](int64_t row0, int64_t col, float v[4]) __attribute__((always_inline)) {
      for (int q = 0; q < 4; ++q) v[q] *= alpha;
      store_sym<T>(A, d.lda, m, mirror, row0, col, v);
    });
  }
}

// B' = f * A when c = 0: no product, the tile and its mirror are scaled
// elementwise, 16 bytes per lane. On a diagonal tile, 1 is added to the first
// diag_rows diagonal entries (0: none).
template <int NT>
MUON_INLINE void scale_tile_pair(const u16* A, u16* B, int64_t ld, int64_t tr, int64_t tc, bool mirror,
                                 float cb, int diag_rows = 0) {
#pragma unroll 1
  for (int p = 0; p < 256 * 32 / NT; ++p) {
    const int idx = threadIdx.x + p * NT, row = idx >> 5, ch = idx & 31;
    const int dcol = row < diag_rows ? row - 8 * ch : -1;  // the diagonal entry's place in the run
#pragma unroll 1
    for (int s = 0; s < (mirror ? 2 : 1); ++s) {
      const int64_t o = (s ? (tc + row) * ld + tr : (tr + row) * ld + tc) + ch * 8;
      u32x4 v = *((const g_u32x4*)(A + o));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = pack_bf16x2(cb * __uint_as_float(v[e] << 16) + (dcol == 2 * e ? 1.f : 0.f),
                           cb * __uint_as_float(v[e] & 0xffff0000u) + (dcol == 2 * e + 1 ? 1.f : 0.f));
      *((g_u32x4*)(B + o)) = v;
    }
  }
}

template <class E>
MUON_INLINE void square_tile(const PhaseArgs& args, const MatDev& d, int ti, int tj, void* smem) {
  typedef typename E::T T;
  const T* A = static_cast<const T*>(d.a);
  T* B = static_cast<T*>(d.b);
  const float cb = args.co.b, cc = args.co.c;
  const bool mirror = ti != tj;
  const int64_t tr = (int64_t)ti * E::BM, tc = (int64_t)tj * E::BN;
  const int m = d.m;
  if constexpr (E::kStageTile) {
    const Fold f = fold_coeffs(args.co);
    if (f.sq_mode == 0) {
      scale_tile_pair<E::NT>(A, B, d.lda, tr, tc, mirror, f.sq);
      return;
    }
    // B' = sq * (A' A' + A') (or sq * A' A'). The engine adds A'[i][j] while
    // the K steps over the tile's columns, which hold it, are in LDS.
    f32x16 acc[E::FM][E::FN];
    E::run(A + tr * d.lda, d.lda, A + tc * d.lda, d.lda, d.mp, static_cast<T*>(smem), acc,
           f.sq_mode == 2 ? tj * (E::BN / E::BK) : -1, 1.f);
    store_tile_staged<E>(acc, static_cast<unsigned char*>(smem), f.sq, tile_rows<E>(tr, m), tile_cols<E>(tc, m),
                         B + tr * d.lda + tc, d.lda, mirror ? B + tc * d.lda + tr : nullptr, d.lda);
  } else {
    f32x16 acc[E::FM][E::FN];
    E::run(A + tr * d.lda, d.lda, A + tc * d.lda, d.lda, d.mp, static_cast<T*>(smem), acc);
    TileWalk<E>::each(tr, tc, acc, [&](int64_t row0, int64_t col, float v[4]) __attribute__((always_inline)) {
      for (int q = 0; q < 4; ++q) v[q] = cb * Elem<T>::load(A + (row0 + q) * d.lda + col) + cc * v[q];
      store_sym<T>(B, d.lda, m, mirror, row0, col, v);
    });
  }
}

// Last-iteration weight update of 8 consecutive W elements (row gr, columns
// gc .. gc+7, clipped to the matrix) from the bf16 O values in o:
// W' = W - lr*scale*O and delta = -lr*scale*O, each rounded once. A full,
// 16-byte aligned group uses vector accesses; a ragged or unaligned one goes
// element by element.
MUON_INLINE void apply8(const MatDev& d, int64_t gr, int64_t gc, u32x4 ov) {
  u16* W = static_cast<u16*>(d.w);
  u16* D = static_cast<u16*>(d.delta);
  const float ls = d.lr_scale;
  const int64_t C = d.cols;
  float o[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[2 * e] = __uint_as_float(ov[e] << 16);
    o[2 * e + 1] = __uint_as_float(ov[e] & 0xffff0000u);
  }
  const int64_t base = gr * C + gc;
  if (gc + 8 <= C && (base & 7) == 0) {
    if (W) {
      u32x4 wv = *((const g_u32x4*)(W + base));
      u32x4 nv;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        nv[e] = pack_bf16x2(__uint_as_float(wv[e] << 16) - ls * o[2 * e],
                            __uint_as_float(wv[e] & 0xffff0000u) - ls * o[2 * e + 1]);
      *((g_u32x4*)(W + base)) = nv;
    }
    if (D) {
      u32x4 dv;
#pragma unroll
      for (int e = 0; e < 4; ++e) dv[e] = pack_bf16x2(-ls * o[2 * e], -ls * o[2 * e + 1]);
      *((g_u32x4*)(D + base)) = dv;
    }
  } else {
    for (int e = 0; e < 8 && gc + e < C; ++e) {
      if (W) Elem<u16>::store(W + base + e, Elem<u16>::load(W + base + e) - ls * o[e]);
      if (D) Elem<u16>::store(D + base + e, -ls * o[e]);
    }
  }
}

// Last iteration: the staging tile holds the X tile at (tr, tc). O = X for a
// wide matrix (W tile at (tr, tc), read by rows), O = X^T for a tall one (W
// tile at (tc, tr), read by columns).
template <int NT>
MUON_INLINE void apply_from_lds(const unsigned char* smem, const MatDev& d, int64_t tr, int64_t tc) {
  const int64_t R = d.rows, C = d.cols;
  const int tid = fresh_tid();
  if (!d.tall) {
#pragma unroll 1
    for (int p = 0; p < 256 * 32 / NT; ++p) {
      const int idx = tid + p * NT, row = idx >> 5, ch = idx & 31;
      const int64_t gr = tr + row, gc = tc + ch * 8;
      if (gr < R && gc < C) apply8(d, gr, gc, stage_read_row8(smem, row, ch));
    }
  } else {
    constexpr int NW = NT / 64;
    const int wave = tid >> 6, G = (tid >> 4) & 3, i = tid & 15;
#pragma unroll 1
    for (int p = 0; p < 128 / NW; ++p) {
      const int t = wave + p * NW;
      const int c0 = 16 * (t & 15), r0 = 32 * (t >> 4) + 8 * G;
      const u32x4 v = stage_read_col8(smem, r0, c0, tid);  // every lane takes part
      const int64_t gr = tc + c0 + i, gc = tr + r0;
      if (gr < R && gc < C) apply8(d, gr, gc, v);
    }
  }
}

template <class E, bool LAST>
MUON_INLINE void update_tile(const PhaseArgs& args, const MatDev& d, int ti, int tj, void* smem) {
  static_assert(E::kQK, "the update reads X as a K-major operand");
  typedef typename E::T T;
  const int src = args.src, dst = src ^ 1;
  const T* B = static_cast<const T*>(d.b);
  const T* X = static_cast<const T*>(d.x[src]);
  const int64_t tr = (int64_t)ti * E::BM, tc = (int64_t)tj * E::BN;
  f32x16 acc[E::FM][E::FN];
  // (B X)[i][j] = sum_k B[i][k] X[k][j]. The bf16 engine also adds X[i][j]
  // while its K steps over this tile's rows are in LDS (B holds B/a there).
  const Fold f = fold_coeffs(args.co);
  E::run(B + tr * d.lda, d.lda, X + tc, d.ldx, d.mp, static_cast<T*>(smem), acc,
         E::kStageTile && f.up_diag ? ti * (E::BM / E::BK) : -1, 1.f);
  const float ca = args.co.a;
  // First iteration: X holds the unscaled U, and B was built from s*U, so
  // X1 = s * (a U + B U).
  const float xs = args.first ? args.scale[&d - args.mats] : 1.f;
  const int m = d.m, n = d.n;
  if constexpr (E::kStageTile) {
    // acc holds X + B' X (or B' X when a = 0).
    const float us = xs * f.up;
    unsigned char* sm = static_cast<unsigned char*>(smem);
    if constexpr (!LAST) {
      store_tile_staged<E>(acc, sm, us, tile_rows<E>(tr, m), tile_cols<E>(tc, n),
                           static_cast<T*>(d.x[dst]) + tr * d.ldx + tc, d.ldx, nullptr, 0);
    } else {
      acc_to_lds<E>(acc, sm, us);
      __syncthreads();
      apply_from_lds<E::NT>(sm, d, tr, tc);
      __syncthreads();
    }
    return;
  }
  if constexpr (!LAST) {
    T* Xo = static_cast<T*>(d.x[dst]);
    TileWalk<E>::each(tr, tc, acc, [&](int64_t row0, int64_t col, float v[4]) __attribute__((always_inline)) {
      const bool cok = col < n;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t o = (row0 + q) * d.ldx + col;
        Elem<T>::store(Xo + o, (cok && row0 + q < m) ? xs * (ca * Elem<T>::load(X + o) + v[q]) : 0.f);
      }
    });
  } else {
    // Last iteration: O = X_T (or X_T^T for a tall matrix).
    // W -= lr*scale*O, delta = -lr*scale*O.
    T* W = static_cast<T*>(d.w);
    T* D = static_cast<T*>(d.delta);
    const float ls = d.lr_scale;
    const int64_t ldw = d.cols;
    TileWalk<E>::each(tr, tc, acc, [&](int64_t row0, int64_t col, float v[4]) __attribute__((always_inline)) {
      if (col >= n) return;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t r = row0 + q;
        if (r >= m) break;
        const float o = xs * (ca * Elem<T>::load(X + r * d.ldx + col) + v[q]);
        const int64_t wo = d.tall ? col * ldw + r : r * ldw + col;
        if (W) Elem<T>::store(W + wo, Elem<T>::load(W + wo) - ls * o);
        if (D) Elem<T>::store(D + wo, -ls * o);
      }
    });
  }
}

// ------------------------------------------------------------ persistent phase kernel

template <class E, int PH>
__global__ void __launch_bounds__(E::NT) phase_kernel(PhaseArgs args) {
  constexpr int SMEM = E::kStageTile && kOutBytes > E::LDS_BYTES ? kOutBytes : E::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  __shared__ int s_tile;
  const int home = blockIdx.x % kQueues;
  for (int qq = 0; qq < kQueues; ++qq) {
    const int q = (home + qq) % kQueues;
    const int base = args.qoff[q], len = args.qoff[q + 1] - base;
    while (true) {
      if (threadIdx.x == 0) s_tile = atomicAdd(args.counter + q, 1);
      __syncthreads();
      const int t = __builtin_amdgcn_readfirstlane(s_tile);  // uniform: tile state stays scalar
      __syncthreads();  // every thread has read s_tile before thread 0 writes it again
      if (t >= len) break;
      const Tile tile = args.tiles[base + t];
      const MatDev& d = args.mats[tile.mat];
      const int ti = tile.ij >> 16, tj = tile.ij & 0xffff;
      if constexpr (PH == kGram) gram_tile<E>(args, d, ti, tj, smem);
      else if constexpr (PH == kSquare) square_tile<E>(args, d, ti, tj, smem);
      else if constexpr (PH == kUpdate) update_tile<E, false>(args, d, ti, tj, smem);
      else update_tile<E, true>(args, d, ti, tj, smem);
    }
  }
}

// ------------------------------------------------------------ four-wave persistent kernel
//
// The four-wave engine pipelines across tiles: while a tile's last K steps
// run, the ring already receives the next tile's first steps, so a tile starts
// without waiting for memory. The epilogue therefore only has the LDS those
// steps leave free: the ring's last stage and the 32 KB after the ring, 64 KB
// in all, which hold one half of the output tile (128 rows of the staging
// layout) at a time. Each half is written from the accumulators of the two
// waves that hold it, then read back by all four waves: by rows for the tile
// itself (16 bytes per lane, whole 512-byte rows per wave instruction), by
// columns with ds_read_b64_tr_b16 for the transposed copies.

constexpr int kEpiRows = 128;
constexpr int kEpiBytes = kEpiRows * kOutStride;  // 64 KB
constexpr int kEpiExtra = 32 * 1024;              // LDS past the ring

// Half H of the output tile: accumulator blocks 2H and 2H+1 of every wave,
// i.e. tile rows 64H .. +63 and 128 + 64H .. +63, times scale, into the 128
// staging rows of epi (staged row r holds tile row half_row(r, H)). All four
// waves convert in both halves. Entries outside the matrix are masked when the
// half is read out.
MUON_INLINE int half_row(int r, int H) { return (r & 63) + ((r >> 6) << 7) + 64 * H; }

// EYE: add 1 on the tile's diagonal after scaling (a diagonal tile). Element
// (R, C) of a wave tile is lane l's register 4g + q of block (i, j), with
// R = 32i + l%32 and C = 32j + 8g + 4(l/32) + q: on the diagonal iff the wave
// sits on the tile's diagonal (wm = wn), i = j and l%32 = 8g + 4(l/32) + q.
template <class E, int H, bool EYE = false>
MUON_INLINE void stage_half(f32x16 (&acc)[E::FM][E::FN], unsigned char* epi, float scale) {
  static_assert(E::WM == 128 && E::FM == 4 && E::BM == 256, "halves are blocks {0,1} and {2,3} of 128-row waves");
  static_assert(E::WN / 4 >= 8 * E::FN, "unit bits of wu and 8j + 2g must not overlap");
  const int tid = fresh_tid(), lane = tid & 63, wave = tid >> 6;
  const int wu = E::wave_n(wave) * (E::WN / 4) + (lane >> 5);
  const int ux = (wu ^ stage_swz(lane & 31)) << 3;
  const int l = lane & 31;
  const bool eye = EYE && E::wave_m(wave) == E::wave_n(wave) && ((l >> 2) & 1) == (lane >> 5);
  const int er = 4 * (l >> 3) + (l & 3);  // the register holding the diagonal element
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) {
    const int i = 2 * H + ii;
    unsigned char* row = epi + (64 * E::wave_m(wave) + 32 * ii + (lane & 31)) * kOutStride;
#pragma unroll
    for (int j = 0; j < E::FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = scale * acc[i][j][4 * g + q];
          if (EYE && i == j) v[q] += (eye && 4 * g + q == er) ? 1.f : 0.f;
        }
        u32x2 t;
        t[0] = pack_bf16x2(v[0], v[1]);
        t[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(row + (ux ^ ((8 * j + 2 * g) << 3))) = t;
      }
  }
}

// Eight bf16 of one run (element e in half e%2 of word e/2) with the
// elements at positions p0 + e >= lim zeroed, all of them unless ok.
MUON_INLINE u32x4 mask_run(u32x4 v, bool ok, int p0, int lim) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t m = (p0 + 2 * e < lim ? 0xffffu : 0u) | (p0 + 2 * e + 1 < lim ? 0xffff0000u : 0u);
    v[e] &= ok ? m : 0u;
  }
  return v;
}

// Staged half H -> its 128 rows of dst (dst: the tile's first element, row
// stride ld, 16-byte aligned rows), entries at tile rows >= rl or columns >= cl
// as zero. The padding of the operand buffers stays zero that way. U is the
// unroll count of this loop and of mirror_out's: in full (16), a thread's LDS
// reads are all in flight before its first store waits for one, 0.1-0.3% less
// step time than 4 at a time on the Qwen3 configs; the split-K Gram instance
// keeps 4, with which its K loop does not spill.
template <int NT, int U = 16>
MUON_INLINE void rows_out(const unsigned char* epi, u16* dst, int64_t ld, int H, int rl, int cl) {
  const int tid = fresh_tid();
  if (rl >= 256 && cl >= 256) {
#pragma unroll U
    for (int p = 0; p < kEpiRows * 32 / NT; ++p) {
      const int idx = tid + p * NT, row = idx >> 5, ch = idx & 31;
      *((g_u32x4*)(dst + (int64_t)half_row(row, H) * ld + 8 * ch)) = stage_read_row8(epi, row, ch);
    }
  } else {
#pragma unroll U
    for (int p = 0; p < kEpiRows * 32 / NT; ++p) {
      const int idx = tid + p * NT, row = idx >> 5, ch = idx & 31;
      const int tr = half_row(row, H);
      const u32x4 v = mask_run(stage_read_row8(epi, row, ch), tr < rl, 8 * ch, cl);
      *((g_u32x4*)(dst + (int64_t)tr * ld + 8 * ch)) = v;
    }
  }
}

// Staged half H -> the transpose: row c of dst_t (c = 0 .. 255) gets, at the
// half's 128 tile rows, column c of the staged rows (masked as in rows_out). Wave
// task t: columns 16(t%16) .. +15, rows 32(t/16) .. +31, lane group G taking 8
// of those rows, so one wave instruction writes 64 contiguous bytes of each of
// 16 rows.
template <int NT, int U = 16>
MUON_INLINE void mirror_out(const unsigned char* epi, u16* dst_t, int64_t ld_t, int H, int rl, int cl) {
  constexpr int NW = NT / 64;
  const int tid = fresh_tid();
  const int wave = tid >> 6, G = (tid >> 4) & 3, i = tid & 15;
  const bool edge = rl < 256 || cl < 256;
#pragma unroll U
  for (int p = 0; p < 64 / NW; ++p) {
    const int t = wave + p * NW;
    const int c0 = 16 * (t & 15), r0 = 32 * (t >> 4) + 8 * G;
    const int tr0 = half_row(r0, H);  // 8 staged rows, 8 consecutive tile rows
    u32x4 v = stage_read_col8(epi, r0, c0, tid);
    if (edge) v = mask_run(v, c0 + i < cl, tr0, rl);
    *((g_u32x4*)(dst_t + (int64_t)(c0 + i) * ld_t + tr0)) = v;
  }
}

// What the last iteration's apply needs of a matrix, as scalars.
struct ApplyDev {
  void* w;      // W, of the apply's storage type (bf16 or fp32), or null
  void* delta;  // delta, of the same type, or null
  float ls;
  int64_t rows, cols;
  int tall;
};

// Element e (0..7) of an 8-element W run loaded as NV 16-byte vectors.
template <class TW>
MUON_INLINE float w_elem(const u32x4 (&v)[sizeof(TW) / 2], int e) {
  if constexpr (sizeof(TW) == 2) return __uint_as_float(e & 1 ? v[0][e >> 1] & 0xffff0000u : v[0][e >> 1] << 16);
  else return __uint_as_float(v[e >> 2][e & 3]);
}

// Stores 8 values as one 8-element run of TW (16 bytes of bf16, 32 of fp32).
template <class TW>
MUON_INLINE void w_store8(TW* p, const float (&x)[8]) {
  if constexpr (sizeof(TW) == 2) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    *((g_u32x4*)(p)) = v;
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      f32x4 v = {x[4 * k], x[4 * k + 1], x[4 * k + 2], x[4 * k + 3]};
      *((g_f32x4*)(p + 4 * k)) = v;
    }
  }
}

// Last iteration, staged half H of the X tile (tile rows half_row(r, H)).
// Wide matrix: W rows tr + half_row(r, H), read by rows; tall matrix (X = the
// transposed update): those W columns of W rows tc + c, read by columns. A
// thread's 16 runs of 8 are applied in batches whose W loads are all in flight
// together, so a batch costs one memory round trip, not one per run: one batch
// for bf16 W, two for fp32 W.
template <int NT, class TW>
MUON_INLINE void apply_half(const unsigned char* epi, const ApplyDev& d, int64_t tr, int64_t tc, int H) {
  constexpr int N = kEpiRows * 32 / NT;
  constexpr int NW = NT / 64;
  static_assert(N == 64 / NW, "row and column item counts agree");
  // W runs of 8 elements: one 16-byte vector for bf16, two for fp32, which
  // take twice the registers per run, hence the second batch.
  constexpr int NV = sizeof(TW) / 2;
  constexpr int B = N / NV;
  const int64_t R = d.rows, C = d.cols;
  TW* W = static_cast<TW*>(d.w);
  TW* D = static_cast<TW*>(d.delta);
  const float ls = d.ls;
  const int tid = fresh_tid();
  const int wave = tid >> 6, G = (tid >> 4) & 3, i = tid & 15;
  u32x4 ov[N];
  int64_t gr[N], gc[N];
#pragma unroll
  for (int p = 0; p < N; ++p) {
    if (!d.tall) {
      const int idx = tid + p * NT, row = idx >> 5, ch = idx & 31;
      gr[p] = tr + half_row(row, H);
      gc[p] = tc + ch * 8;
      ov[p] = stage_read_row8(epi, row, ch);
    } else {
      const int t = wave + p * NW;
      const int c0 = 16 * (t & 15), r0 = 32 * (t >> 4) + 8 * G;
      gr[p] = tc + c0 + i;
      gc[p] = tr + half_row(r0, H);
      ov[p] = stage_read_col8(epi, r0, c0, tid);  // every lane takes part
    }
  }
#pragma unroll
  for (int b0 = 0; b0 < N; b0 += B) {
    // Whole aligned runs: W loaded for all items of the batch first.
    u32x4 wv[B][NV];
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int p = b0 + q;
      const int64_t base = gr[p] * C + gc[p];
      const bool fast = gr[p] < R && gc[p] + 8 <= C && (base & 7) == 0;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        wv[q][k] = u32x4{0u, 0u, 0u, 0u};
        if (W && fast) wv[q][k] = *((const g_u32x4*)(W + base) + k);
      }
    }
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int p = b0 + q;
      if (gr[p] >= R || gc[p] >= C) continue;
      const int64_t base = gr[p] * C + gc[p];
      if (gc[p] + 8 <= C && (base & 7) == 0) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[2 * e] = __uint_as_float(ov[p][e] << 16);
          o[2 * e + 1] = __uint_as_float(ov[p][e] & 0xffff0000u);
        }
        if (W) {
          float nw[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) nw[e] = w_elem<TW>(wv[q], e) - ls * o[e];
          w_store8(W + base, nw);
        }
        if (D) {
          float nd[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) nd[e] = -ls * o[e];
          w_store8(D + base, nd);
        }
      } else {  // ragged edge or unaligned row: element by element
        for (int e = 0; e < 8 && gc[p] + e < C; ++e) {
          const float o = __uint_as_float(e & 1 ? ov[p][e >> 1] & 0xffff0000u : ov[p][e >> 1] << 16);
          if (W) Elem<TW>::store(W + base + e, Elem<TW>::load(W + base + e) - ls * o);
          if (D) Elem<TW>::store(D + base + e, -ls * o);
        }
      }
    }
  }
}

// WF32: W and delta are fp32 (fp32 master weights; the last update only).
// KSPLIT: the launch's Gram tiles include split-K pieces (a separate
// instance, so that the code of launches without pieces stays as it is).
template <class E, int PH, bool WF32 = false, bool KSPLIT = false>
__global__ void __launch_bounds__(E::NT) phase_kernel4(PhaseArgs args) {
  static_assert(E::LDS_BYTES + kEpiExtra <= 160 * 1024, "ring + staging exceed LDS");
  static_assert(E::STAGE_BYTES >= kEpiBytes - kEpiExtra, "the staging half must not reach the preloaded stages");
  __shared__ __attribute__((aligned(16))) unsigned char smem[E::LDS_BYTES + kEpiExtra];
  unsigned char* epi = smem + E::LDS_BYTES + kEpiExtra - kEpiBytes;
  // Tile claims go through one word past the ring: free while a tile runs
  // (the epilogue is the only other user of that LDS).
  int* s_tile = reinterpret_cast<int*>(smem + E::LDS_BYTES);
  const Fold f = fold_coeffs(args.co);
  const int home = blockIdx.x % kQueues;
  int qq = 0;  // queues home + 0 .. qq-1 are known to be empty
  // Next tile of this workgroup (index into args.tiles), or -1: its home
  // queue first, then the others. Every thread calls it (it has barriers).
  auto fetch = [&]() -> int {
    while (qq < kQueues) {
      const int q = __builtin_amdgcn_readfirstlane((home + qq) % kQueues);
      if (threadIdx.x == 0) *s_tile = atomicAdd(args.counter + q, 1);
      __syncthreads();
      const int t = __builtin_amdgcn_readfirstlane(*s_tile);
      __syncthreads();  // every thread has read s_tile before it is written again
      const int base = kconst(args.qoff)[q];
      if (t < kconst(args.qoff)[q + 1] - base) return base + t;
      ++qq;
    }
    return -1;
  };
  if constexpr (PH == kSquare) {
    if (f.sq_mode == 0) {  // B' = sq * A elementwise: no product
      for (int t = fetch(); t >= 0; t = fetch()) {
        const Tile tile = args.tiles[t];
        const MatDev& d = args.mats[tile.mat];
        const int64_t tr = (int64_t)(tile.ij >> 16) * E::BM, tc = (int64_t)(tile.ij & 0xffff) * E::BN;
        const bool dt = (tile.ij >> 16) == (tile.ij & 0xffff);
        scale_tile_pair<E::NT>(static_cast<const u16*>(d.a), static_cast<u16*>(d.b), d.lda, tr, tc, !dt, f.sq,
                               f.up_diag && dt ? tile_rows<E>(tr, d.m) : 0);
      }
      return;
    }
  }
  auto operands = [&](int t) __attribute__((always_inline)) {
    const Tile tile = load_tile(args.tiles, __builtin_amdgcn_readfirstlane(t));
    const auto& d = kconst(args.mats)[tile.mat];
    const int ti = tile.ij >> 16, tj = tile.ij & 0xffff;
    const int64_t tr = (int64_t)ti * E::BM, tc = (int64_t)tj * E::BN;
    Opnd o;
    if constexpr (PH == kGram) {
      // A split-K piece covers K chunks kr >> 16 .. + (kr & 0xffff) of 256.
      const u16* X = static_cast<const u16*>(d.x[args.src]);
      const int64_t k0 = (int64_t)(tile.kr >> 16) * 256;
      const int K = tile.kr ? (tile.kr & 0xffff) * 256 : d.np;
      o = Opnd{X + tr * d.ldx + k0, d.ldx, X + tc * d.ldx + k0, d.ldx, K, 0, 0};
    } else if constexpr (PH == kSquare) {
      const u16* A = static_cast<const u16*>(d.a);
      const int dg = f.sq_mode == 2;
      o = Opnd{A + tr * d.lda, d.lda, A + tc * d.lda, d.lda, d.mp, dg ? tj * (E::BN / E::BK) : 0, dg};
    } else {
      const u16* B = static_cast<const u16*>(d.b);
      const u16* X = static_cast<const u16*>(d.x[args.src]);
      o = Opnd{B + tr * d.lda, d.lda, X + tc, d.ldx, d.mp, 0, 0};  // B'' holds the identity term
    }
    return uniform(o);
  };
  // In-loop claim of the successor from the current queue (see Engine4::run):
  // thread 0 takes a ticket, parks it in s_tile after a step's barrier has
  // passed, and every thread reads it after the next step's barrier. An empty
  // queue moves qq on and leaves the successor to fetch().
  int ticket = 0, nxt = -1;
  auto claim = [&](int st, Opnd& n) __attribute__((always_inline)) -> bool {
    if (qq >= kQueues) return false;
    const int q = __builtin_amdgcn_readfirstlane((home + qq) % kQueues);
    if (st == 0) {
      if (threadIdx.x == 0) ticket = atomicAdd(args.counter + q, 1);
      return false;
    }
    if (st == 1) {
      if (threadIdx.x == 0) *s_tile = ticket;
      return false;
    }
    const int t = __builtin_amdgcn_readfirstlane(*s_tile);
    const int base = kconst(args.qoff)[q];
    if (t >= kconst(args.qoff)[q + 1] - base) {
      ++qq;
      return false;
    }
    nxt = __builtin_amdgcn_readfirstlane(base + t);
    n = operands(nxt);
    return true;
  };
  int cur = fetch();
  if (cur < 0) return;
  Opnd oc = operands(cur);
  bool pre = false;
  while (true) {
    f32x16 acc[E::FM][E::FN];
    Opnd on;
    nxt = -1;
    const bool has_next = E::run(oc, claim, on, pre, reinterpret_cast<u16*>(smem), acc);

    const Tile tile = load_tile(args.tiles, __builtin_amdgcn_readfirstlane(cur));
    const auto& d = kconst(args.mats)[tile.mat];
    const int ti = tile.ij >> 16, tj = tile.ij & 0xffff;
    const int64_t tr = (int64_t)ti * E::BM, tc = (int64_t)tj * E::BN;
    const float s = kconst(args.scale)[tile.mat];
    // Each half: stage, barrier, read out, barrier (the second half's closing
    // barrier is the next tile's first one when it was preloaded).
    if (KSPLIT && PH == kGram && tile.slot >= 0) {
      // A split-K piece: its partial sums go to its slot in accumulator
      // order (thread t's 16 values of block (i, j) at 16 * (256 (4i + j) +
      // t)), so every wave stores 4 KB contiguous per block and the reduce
      // launch reads them back in the same layout. No LDS is touched.
      float* dst = args.kpart + (int64_t)tile.slot * kPartFloats + 16 * (int)threadIdx.x;
#pragma unroll
      for (int i = 0; i < E::FM; ++i)
#pragma unroll
        for (int j = 0; j < E::FN; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const f32x4 x = {acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2], acc[i][j][4 * v + 3]};
            *((g_f32x4*)(dst + 4096 * (i * E::FN + j) + 4 * v)) = x;
          }
    } else if constexpr (PH == kGram || PH == kSquare) {
      // gram: A' = g s^2 U U^T on the first iteration (X holds U), else g X X^T.
      // square: B'' = sq * (A' A' + A') + I (the update's identity term; only
      //   when the update has it, and only a diagonal tile has a diagonal).
      const float sc = PH == kGram ? (args.first ? s * s : 1.f) * f.g : f.sq;
      u16* O = static_cast<u16*>(PH == kGram ? d.a : d.b);
      const int rl = tile_rows<E>(tr, d.m), cl = tile_cols<E>(tc, d.m);
      auto half = [&](auto H_, auto EYE_) __attribute__((always_inline)) {
        constexpr int H = decltype(H_)::value;
        stage_half<E, H, decltype(EYE_)::value>(acc, epi, sc);
        __syncthreads();
        constexpr int U = KSPLIT ? 4 : 16;
        rows_out<E::NT, U>(epi, O + tr * d.lda + tc, d.lda, H, rl, cl);
        if (ti != tj) mirror_out<E::NT, U>(epi, O + tc * d.lda + tr, d.lda, H, rl, cl);
      };
      using H0 = std::integral_constant<int, 0>;
      using H1 = std::integral_constant<int, 1>;
      if (PH == kSquare && f.up_diag && ti == tj) {
        half(H0{}, std::true_type{});
        __syncthreads();
        half(H1{}, std::true_type{});
      } else {
        half(H0{}, std::false_type{});
        __syncthreads();
        half(H1{}, std::false_type{});
      }
    } else {
      // X_next = s' * a' * B'' X, s' = s on the first iteration.
      const float us = (args.first ? s : 1.f) * f.up;
      auto half = [&](auto H_) __attribute__((always_inline)) {
        constexpr int H = decltype(H_)::value;
        if constexpr (PH == kUpdate) {
          stage_half<E, H>(acc, epi, us);
          __syncthreads();
          rows_out<E::NT>(epi, static_cast<u16*>(d.x[args.src ^ 1]) + tr * d.ldx + tc, d.ldx, H,
                          tile_rows<E>(tr, d.m), tile_cols<E>(tc, d.n));
        } else {
          stage_half<E, H>(acc, epi, us);
          __syncthreads();
          const ApplyDev ad{d.w, d.delta, d.lr_scale, d.rows, d.cols, d.tall};
          if constexpr (WF32) apply_half<E::NT, float>(epi, ad, tr, tc, H);
          else apply_half<E::NT, u16>(epi, ad, tr, tc, H);
        }
      };
      half(std::integral_constant<int, 0>{});
      __syncthreads();
      half(std::integral_constant<int, 1>{});
    }
    if (has_next) {
      cur = nxt;
      oc = on;
      pre = true;
    } else {
      __syncthreads();  // the staging half is read out before fetch() writes s_tile
      cur = fetch();
      if (cur < 0) break;
      oc = operands(cur);
      pre = false;
    }
  }
}

// Sum of a split Gram tile's pieces, then the Gram epilogue: A' = g (s^2)
// X X^T for the tile and its mirror. Four workgroups per tile, one per
// 128 x 128 quadrant (the sub-tile one wave of the four-wave engine held).
// In the pieces' layout, quadrant w's 16 accumulator blocks (i, j) are 4 KB
// each: lane l's 16 values at 16 (256 (4i + j) + 64 w + l). Here wave v takes
// block row i = v: lane l holds quadrant row 32v + l % 32 and, for each j, the
// 16 columns 32j + 8g + 4(l / 32) + q (g, q < 4) of it. The sums (in piece
// order), scaled, go to a bf16 staging tile of 128 rows (pitch 136 elements,
// so that 8 consecutive rows of one column fall in 8 different banks), which
// is written out by rows (16 bytes per lane) and, for an off-diagonal tile,
// by columns to the mirror (8 rows gathered per 16-byte store). Entries
// outside the matrix are written as 0, as the Gram kernel's are.
__global__ void __launch_bounds__(256) gram_reduce_kernel(PhaseArgs args, const Tile* list) {
  constexpr int QP = 136;  // staging pitch in bf16 elements
  __shared__ __attribute__((aligned(16))) u16 stage[128 * QP];
  const Tile tile = load_tile(list, blockIdx.x >> 2);
  const int w = blockIdx.x & 3, wm = w >> 1, wn = w & 1;
  const auto& d = kconst(args.mats)[tile.mat];
  const int ti = tile.ij >> 16, tj = tile.ij & 0xffff, pieces = tile.kr;
  const int tid = threadIdx.x, lane = tid & 63, v = tid >> 6;
  const float s = kconst(args.scale)[tile.mat];
  const float sc = (args.first ? s * s : 1.f) * fold_coeffs(args.co).g;
  // Valid rows and columns of this quadrant (the tile is m x m at most).
  const int64_t qr = (int64_t)ti * 256 + wm * 128, qc = (int64_t)tj * 256 + wn * 128;
  const int rl = (int)(d.m - qr < 128 ? (d.m - qr > 0 ? d.m - qr : 0) : 128);
  const int cl = (int)(d.m - qc < 128 ? (d.m - qc > 0 ? d.m - qc : 0) : 128);
  const int row = 32 * v + (lane & 31);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float* src = args.kpart + (int64_t)tile.slot * kPartFloats + 16 * (256 * (4 * v + j) + 64 * w + lane);
    f32x4 x[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) x[g] = *((const g_f32x4*)(src + 4 * g));
    for (int pc = 1; pc < pieces; ++pc) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 y = *((const g_f32x4*)(src + (int64_t)pc * kPartFloats + 4 * g));
        x[g][0] += y[0]; x[g][1] += y[1]; x[g][2] += y[2]; x[g][3] += y[3];
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * j + 8 * g + 4 * (lane >> 5);
      float o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = (row < rl && col + q < cl) ? sc * x[g][q] : 0.f;
      *reinterpret_cast<u32x2*>(&stage[row * QP + col]) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
  }
  __syncthreads();
  u16* A = static_cast<u16*>(d.a);
  // Rows: 128 rows x 256 bytes, 16 lanes per row.
#pragma unroll 4
  for (int p = 0; p < 8; ++p) {
    const int idx = tid + 256 * p, r = idx >> 4, c8 = (idx & 15) * 8;
    *((g_u32x4*)(A + (qr + r) * d.lda + qc + c8)) = *reinterpret_cast<const u32x4*>(&stage[r * QP + c8]);
  }
  if (ti == tj) return;
  // Mirror: row c of the mirror quadrant gets column c of the staging tile;
  // a lane gathers 8 consecutive staged rows of one column.
#pragma unroll 4
  for (int p = 0; p < 8; ++p) {
    const int idx = tid + 256 * p, c = idx & 127, r8 = (idx >> 7) * 8;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)stage[(r8 + 2 * e) * QP + c] | ((uint32_t)stage[(r8 + 2 * e + 1) * QP + c] << 16);
    *((g_u32x4*)(A + (qc + c) * d.lda + qr + r8)) = o;
  }
}

// ------------------------------------------------------------ elementwise kernels

// Matrix of elementwise block b: the last i with prefix[i] <= b.
MUON_INLINE int find_mat(const int32_t* prefix, int n, int b) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= b) lo = mid; else hi = mid - 1;
  }
  return lo;
}

MUON_INLINE float block_sum_256(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Fused momentum. One 64 x 64 tile of one matrix per workgroup of 256 threads.
// Nothing here mixes elements of a tile, except the sum of squares. TG, TM
// and TX are the storage types of G, of M and of the X buffer (all bf16, all
// fp32, or bf16 G and X with an fp32 M).
//
// A tall matrix's tile goes to X transposed, through LDS. bf16: element
// (r, c) of the tile is half c % 2 of 4-byte word
// r * 32 + ((c / 2) ^ (2 * ((r / 4) % 16))). A thread writes its 4 columns as
// one 8-byte store (the swizzle is even, so the pair of words stays adjacent),
// and the half-waves of a store cover 2 rows x 32 distinct words; the
// transposing reads take column c of rows 4k + e, k = 0..15, whose words
// (c / 2) ^ 2k are 16 distinct even numbers: with the adjacent column's word
// (the odd one, or the same word read twice) no two lanes meet in one bank
// at different addresses, for 32- or 64-bank LDS. fp32: rows of 65 floats, so
// bank (r + c) mod 64 differs across the lanes of both access patterns.
template <class TG, class TM, class TX>
__global__ void __launch_bounds__(256) momentum_kernel(EwArgs args) {
  constexpr int TS = kEwTile;
  constexpr bool kHalf = sizeof(TX) == 2;
  __shared__ uint32_t tileW[kHalf ? TS * TS / 2 : 1];
  __shared__ float tileF[kHalf ? 1 : TS][TS + 1];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0)
    for (int i = tid; i < args.n_counters; i += 256) args.counters[i] = 0;

  const int mi = find_mat(args.prefix, args.n_mats, blockIdx.x);
  const MatDev& d = args.mats[mi];
  const int local = blockIdx.x - args.prefix[mi];
  const int64_t r0 = (int64_t)(local / d.ew_tiles_c) * TS;
  const int64_t c0 = (int64_t)(local % d.ew_tiles_c) * TS;
  const int rows = d.rows, cols = d.cols;
  const TG* G = static_cast<const TG*>(d.g);
  TM* Mo = static_cast<TM*>(d.mom);
  // X0 = U (rows <= cols) or U^T (tall), in the X buffer: a wide matrix is
  // stored directly, a tall one through the LDS tile, transposed.
  TX* Xb = static_cast<TX*>(d.x[0]);
  const int64_t ldx = d.ldx;
  const bool tall = d.tall != 0;
  const float beta = args.co.beta;
  const bool nesterov = args.co.nesterov != 0;
  const bool vec_ok = (cols & 3) == 0;

  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int lr = p * 16 + (tid >> 4), lc = (tid & 15) * 4;
    const int64_t gr = r0 + lr, gc = c0 + lc;
    float u[4] = {0.f, 0.f, 0.f, 0.f};
    if (gr < rows) {
      const int64_t o = gr * cols + gc;
      if (vec_ok && gc + 3 < cols) {
        float g[4], mm[4], mn[4];
        Vec4<TG>::load(G + o, g);
        Vec4<TM>::load(Mo + o, mm);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mn[e] = beta * mm[e] + g[e];
          u[e] = nesterov ? g[e] + beta * mn[e] : mn[e];
        }
        Vec4<TM>::store(Mo + o, mn);
        if (!tall) Vec4<TX>::store(Xb + gr * ldx + gc, u);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (gc + e < cols) {
            const float g = Elem<TG>::load(G + o + e);
            const float mn = beta * Elem<TM>::load(Mo + o + e) + g;
            u[e] = nesterov ? g + beta * mn : mn;
            Elem<TM>::store(Mo + o + e, mn);
            if (!tall) Elem<TX>::store(Xb + gr * ldx + gc + e, u[e]);
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += u[e] * u[e];
    if (tall) {
      if constexpr (kHalf) {
        const int w = (lc >> 1) ^ (2 * ((lr >> 2) & 15));
        *reinterpret_cast<u32x2*>(&tileW[lr * 32 + w]) = u32x2{pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3])};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) tileF[lr][lc + e] = u[e];
      }
    }
  }
  const float tot = block_sum_256(ss, red);  // contains a barrier: tileU is complete
  if (tid == 0) args.partials[d.part_off + local] = tot;

  if (!tall) return;
  // Tall matrix: row gc of X = U^T holds column gc of U.
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int lc = p * 16 + (tid >> 4), lr = (tid & 15) * 4;
    const int64_t gc = c0 + lc, gr = r0 + lr;
    if (gc >= cols) continue;
    TX* dst = Xb + gc * ldx + gr;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (kHalf) {
        const uint32_t word = tileW[(lr + e) * 32 + ((lc >> 1) ^ (2 * ((lr >> 2) & 15)))];
        v[e] = __uint_as_float((lc & 1) ? word & 0xffff0000u : word << 16);
      } else {
        v[e] = tileF[lr + e][lc];
      }
    }
    if (gr + 3 < rows) {
      Vec4<TX>::store(dst, v);
    } else {
      for (int e = 0; e < 4 && gr + e < rows; ++e) Elem<TX>::store(dst + e, v[e]);
    }
  }
}

// s = 1 / (||U||_F + eps) for one matrix per workgroup. The partials are summed
// in fp64 in a fixed order, so the result does not depend on scheduling.
__global__ void __launch_bounds__(256) norm_kernel(const MatDev* mats, const float* partials,
                                                   float* scale, float eps) {
  __shared__ double red[256];
  const MatDev& d = mats[blockIdx.x];
  double s = 0.0;
  for (int i = threadIdx.x; i < d.n_parts; i += 256) s += (double)partials[d.part_off + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) scale[blockIdx.x] = (float)(1.0 / (sqrt(red[0]) + (double)eps));
}

// T = 0: O = s*U, so W -= lr*scale*s*U and delta = -lr*scale*s*U. TX is the
// X buffer's storage type, TW that of W and delta.
template <class TX, class TW>
__global__ void __launch_bounds__(256) apply_kernel(EwArgs args) {
  const int mi = find_mat(args.prefix, args.n_mats, blockIdx.x);
  const MatDev& d = args.mats[mi];
  const int local = blockIdx.x - args.prefix[mi];
  const int64_t r0 = (int64_t)(local / d.ew_tiles_c) * kEwTile;
  const int64_t c0 = (int64_t)(local % d.ew_tiles_c) * kEwTile;
  const TX* Xb = static_cast<const TX*>(d.x[0]);  // U, or U^T for a tall matrix
  TW* W = static_cast<TW*>(d.w);
  TW* D = static_cast<TW*>(d.delta);
  const float f = d.lr_scale * args.scale[mi];
  for (int e = threadIdx.x; e < kEwTile * kEwTile; e += 256) {
    const int64_t gr = r0 + e / kEwTile, gc = c0 + e % kEwTile;
    if (gr >= d.rows || gc >= d.cols) continue;
    const float o = f * Elem<TX>::load(Xb + (d.tall ? gc * d.ldx + gr : gr * d.ldx + gc));
    const int64_t wo = gr * d.cols + gc;
    if (W) Elem<TW>::store(W + wo, Elem<TW>::load(W + wo) - o);
    if (D) Elem<TW>::store(D + wo, -o);
  }
}

// TP local update: P += D over strided views. A workgroup of 4 waves takes
// kApplyRows rows x 1 KB of one shard: lane l a 16-byte vector of each of the
// rows wave, wave + 4, ... (8 bf16 or 4 fp32), so every wave instruction
// moves one contiguous kilobyte of a row. A thread issues all of its P and D
// loads before its first store. Each sum is formed in fp32 and stored once;
// for two bf16 (or fp32) values that is their exactly rounded sum.
template <class T>
__global__ void __launch_bounds__(256) shard_apply_kernel(const ShardDev* shards, const int32_t* prefix,
                                                          int n) {
  constexpr int VE = 16 / sizeof(T);  // elements per 16-byte vector
  constexpr int TC = 64 * VE;         // tile columns
  constexpr int RQ = kApplyRows / 4;  // rows per thread
  const int si = find_mat(prefix, n, blockIdx.x);
  const auto& s = kconst(shards)[si];
  const int local = blockIdx.x - prefix[si];
  const int64_t r0 = (int64_t)(local / s.tiles_c) * kApplyRows;
  const int64_t gc = (int64_t)(local % s.tiles_c) * TC + (threadIdx.x & 63) * VE;
  const int wave = threadIdx.x >> 6;
  T* P = static_cast<T*>(s.p);
  const T* D = static_cast<const T*>(s.d);
  const int64_t rows = s.rows, cols = s.cols, ldp = s.ldp, ldd = s.ldd;
  if (gc >= cols) return;
  if (s.vec && gc + VE <= cols) {
    u32x4 pv[RQ], dv[RQ];
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int64_t gr = r0 + wave + 4 * q;
      if (gr < rows) {
        pv[q] = gload16(P + gr * ldp + gc);
        dv[q] = gload16(D + gr * ldd + gc);
      }
    }
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int64_t gr = r0 + wave + 4 * q;
      if (gr >= rows) continue;
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(T) == 2) {
          o[e] = pack_bf16x2(__uint_as_float(pv[q][e] << 16) + __uint_as_float(dv[q][e] << 16),
                             __uint_as_float(pv[q][e] & 0xffff0000u) + __uint_as_float(dv[q][e] & 0xffff0000u));
        } else {
          o[e] = __float_as_uint(__uint_as_float(pv[q][e]) + __uint_as_float(dv[q][e]));
        }
      }
      *((g_u32x4*)(P + gr * ldp + gc)) = o;
    }
  } else {
    for (int q = 0; q < RQ; ++q) {
      const int64_t gr = r0 + wave + 4 * q;
      if (gr >= rows) continue;
      T* pp = P + gr * ldp + gc;
      const T* dd = D + gr * ldd + gc;
      for (int e = 0; e < VE && gc + e < cols; ++e) Elem<T>::store(pp + e, Elem<T>::load(pp + e) + Elem<T>::load(dd + e));
    }
  }
}

// MFMA throughput probe (measurement only): v_mfma_f32_32x32x16_bf16 back to
// back on register operands holding random bf16 values (xorshift of the lane
// and workgroup), 8 independent accumulators per wave so that no MFMA waits
// for another's result, and a different operand pair for consecutive MFMAs so
// that the inputs toggle as they do in a GEMM. It measures what the chip
// sustains on random data under its power limit: the ceiling the GEMM kernels
// run against. The sums are stored so that nothing is optimised away.
__global__ void __launch_bounds__(256) mfma_probe_kernel(float* out, int iters) {
  const int tid = threadIdx.x;
  uint32_t h = (blockIdx.x * 256u + (uint32_t)tid) * 2654435761u + 12345u;
  auto rnd = [&]() {
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    return h;
  };
  bf16x8 a[4], b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[k][e] = (__bf16)((float)((int)(rnd() & 0xffffu) - 32768) * (1.f / 32768.f));
      b[k][e] = (__bf16)((float)((int)(rnd() & 0xffffu) - 32768) * (1.f / 32768.f));
    }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j + (j >> 2)) & 3], acc[j], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[j][e];
  out[(size_t)blockIdx.x * 256 + tid] = sum;
}

// ------------------------------------------------------------ static scratch
//
// The workspace of muon_step_noalloc: one array per GPU, held by the library
// from its first use on that GPU until the process ends. Host code never uses
// the array's name as an address (on the host it names a stand-in, not device
// memory): scratch_address() looks up the device address once per device,
// with that device current, and every later use goes through that pointer.

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

// dst[0 .. n16) = 0 in 16-byte words (grid-stride).
__global__ void __launch_bounds__(256) zero_kernel(u32x4* dst, int64_t n16) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    *((g_u32x4*)(dst + i)) = z;
}

// A table copy whose bytes travel in the kernel arguments, so the host
// buffer they came from may be freed as soon as the launch returns.
constexpr int kUploadWords = 120;  // 16-byte words per launch
struct UploadArgs {
  u32x4* dst;
  int32_t n16;
  u32x4 words[kUploadWords];
};
__global__ void __launch_bounds__(128) upload_kernel(UploadArgs a) {
  if ((int)threadIdx.x < a.n16) *((g_u32x4*)(a.dst + threadIdx.x)) = a.words[threadIdx.x];
}

hipError_t launch_zero(void* dst, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n16 + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const unsigned char* in = static_cast<const unsigned char*>(src);
  unsigned char* out = static_cast<unsigned char*>(dst);
  for (size_t done = 0; done < bytes; done += 16 * kUploadWords) {
    const size_t len = std::min<size_t>(bytes - done, 16 * kUploadWords);
    UploadArgs a;
    std::memset(&a, 0, sizeof(a));
    a.dst = reinterpret_cast<u32x4*>(out + done);
    a.n16 = (int32_t)((len + 15) / 16);
    std::memcpy(a.words, in + done, len);
    hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(128), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ------------------------------------------------------------ launchers

hipError_t launch_momentum(int dtype, const EwArgs& args, int32_t n_blocks, hipStream_t s) {
  if (dtype == 1) hipLaunchKernelGGL((momentum_kernel<u16, u16, u16>), dim3(n_blocks), dim3(256), 0, s, args);
  else if (dtype == 2) hipLaunchKernelGGL((momentum_kernel<u16, float, u16>), dim3(n_blocks), dim3(256), 0, s, args);
  else hipLaunchKernelGGL((momentum_kernel<float, float, float>), dim3(n_blocks), dim3(256), 0, s, args);
  return hipGetLastError();
}

hipError_t launch_norm(const MatDev* mats, const float* partials, float* scale, int32_t n_mats,
                       float eps, hipStream_t s) {
  hipLaunchKernelGGL(norm_kernel, dim3(n_mats), dim3(256), 0, s, mats, partials, scale, eps);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(float* out, int32_t blocks, int32_t iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, s, out, iters);
  return hipGetLastError();
}

hipError_t launch_shard_apply(int dtype, const ShardDev* shards, const int32_t* prefix, int32_t n,
                              int32_t n_blocks, hipStream_t s) {
  if (dtype == 1) hipLaunchKernelGGL(shard_apply_kernel<u16>, dim3(n_blocks), dim3(256), 0, s, shards, prefix, n);
  else hipLaunchKernelGGL(shard_apply_kernel<float>, dim3(n_blocks), dim3(256), 0, s, shards, prefix, n);
  return hipGetLastError();
}

hipError_t launch_apply(int dtype, const EwArgs& args, int32_t n_blocks, hipStream_t s) {
  if (dtype == 1) hipLaunchKernelGGL((apply_kernel<u16, u16>), dim3(n_blocks), dim3(256), 0, s, args);
  else if (dtype == 2) hipLaunchKernelGGL((apply_kernel<u16, float>), dim3(n_blocks), dim3(256), 0, s, args);
  else hipLaunchKernelGGL((apply_kernel<float, float>), dim3(n_blocks), dim3(256), 0, s, args);
  return hipGetLastError();
}

// E reads both operands along K (gram, square); EQ reads Q as a K-major
// operand (update).
template <class E, class EQ>
static hipError_t launch_phase_e(Phase ph, const PhaseArgs& args, int32_t grid, hipStream_t s) {
  switch (ph) {
    case kGram: hipLaunchKernelGGL((phase_kernel<E, kGram>), dim3(grid), dim3(E::NT), 0, s, args); break;
    case kSquare: hipLaunchKernelGGL((phase_kernel<E, kSquare>), dim3(grid), dim3(E::NT), 0, s, args); break;
    default:
      if (args.last) hipLaunchKernelGGL((phase_kernel<EQ, kUpdateLast>), dim3(grid), dim3(EQ::NT), 0, s, args);
      else hipLaunchKernelGGL((phase_kernel<EQ, kUpdate>), dim3(grid), dim3(EQ::NT), 0, s, args);
      break;
  }
  return hipGetLastError();
}

// The four-wave engine's kernels (tile pipelining, epilogues off the ring).
template <class E, class EQ>
static hipError_t launch_phase_e4(Phase ph, const PhaseArgs& args, int32_t grid, hipStream_t s) {
  switch (ph) {
    case kGram:
      if (args.kpart) hipLaunchKernelGGL((phase_kernel4<E, kGram, false, true>), dim3(grid), dim3(E::NT), 0, s, args);
      else hipLaunchKernelGGL((phase_kernel4<E, kGram>), dim3(grid), dim3(E::NT), 0, s, args);
      break;
    case kSquare: hipLaunchKernelGGL((phase_kernel4<E, kSquare>), dim3(grid), dim3(E::NT), 0, s, args); break;
    default:
      if (args.last && args.wf32)
        hipLaunchKernelGGL((phase_kernel4<EQ, kUpdateLast, true>), dim3(grid), dim3(EQ::NT), 0, s, args);
      else if (args.last) hipLaunchKernelGGL((phase_kernel4<EQ, kUpdateLast>), dim3(grid), dim3(EQ::NT), 0, s, args);
      else hipLaunchKernelGGL((phase_kernel4<EQ, kUpdate>), dim3(grid), dim3(EQ::NT), 0, s, args);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_phase(int dtype, int variant, Phase ph, const PhaseArgs& args, int32_t grid,
                        hipStream_t s) {
  if (dtype != 1) return launch_phase_e<EngineF32<false>, EngineF32<true>>(ph, args, grid, s);
  if (variant == kGemmBK32)
    return launch_phase_e<EngineBF16<2, 4, 32, 4, false>, EngineBF16<2, 4, 32, 4, true>>(ph, args, grid, s);
  if (variant == kGemm4W) return launch_phase_e4<Engine4<false, 64, 2>, Engine4<true, 64, 2>>(ph, args, grid, s);
  if (variant == kGemm4WDeep) return launch_phase_e4<Engine4<false, 32, 4>, Engine4<true, 32, 4>>(ph, args, grid, s);
  return launch_phase_e<EngineBF16<2, 4, 64, 2, false>, EngineBF16<2, 4, 64, 2, true>>(ph, args, grid, s);
}

hipError_t launch_gram_reduce(const PhaseArgs& args, const Tile* list, int32_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gram_reduce_kernel, dim3(4 * n), dim3(256), 0, s, args, list);
  return hipGetLastError();
}

int gemm_blocks_per_cu(int dtype, int variant) {
  // Each bf16 workgroup (either engine) holds 128 KB of LDS: one per CU. The
  // fp32 engine uses 66 KB and 256 threads: two per CU.
  (void)variant;
  return dtype == 1 ? 1 : 2;
}

}  // namespace muon
