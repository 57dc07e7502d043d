// tile_core.hpp -- the MFMA tile engine shared by every GEMM phase of the
// blocked vocabulary-projection cross-entropy on gfx950 (CDNA4).
//
// A workgroup computes one 256 x 256 fp32 tile C = A . B^T where A [M x K]
// and B [Nc x K] are both row-major with K contiguous ("NT" form). Its waves
// split the tile as Layout<WM, WN> says (4 x 2 waves of 64 x 128 by default,
// two waves per SIMD); each wave holds its sub-tile as R x C accumulators of
// the 32x32 MFMA layout:
//   element r (0..15) of accumulator (i, j) on lane l is
//   row = i*32 + 8*(r/4) + 4*(l/32) + (r%4),  col = j*32 + (l%32)
// within the wave's sub-tile.
//
// Operands stream through a ring of NST LDS stages of RB bytes of K per row
// (128 B x 2 stages by default), copied global -> LDS by buffer loads that
// write LDS directly, NST - 1 stages ahead of the MFMAs. Within a row the
// 16-byte chunk index is XOR-swizzled by row bits, so the MFMA fragment reads
// (consecutive rows, same chunk) hit distinct banks whether the LDS serves 8
// or 16 lanes of a 128-bit read per cycle; the copies write 1 KiB contiguous
// blocks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vpce {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kTile = 256;                          // BM = BN
constexpr int kGemmLds = 128 * 1024;                // LDS of the operand ring

// Elements of T per 16-byte chunk.
template <typename T> struct Chunk;
template <> struct Chunk<__bf16> { static constexpr int E = 8; };
template <> struct Chunk<float> { static constexpr int E = 4; };

// How the waves of a workgroup split the 256 x 256 tile: WM x WN waves, each
// owning a (256/WM) x (256/WN) sub-tile held as R x C accumulators of the
// 32x32 MFMA layout. Wave w sits at (w / WN, w % WN). With 8 waves two of
// them share each SIMD, so one wave's MFMAs keep the matrix unit busy while
// the other waits to issue a copy or an LDS read.
template <int WM_, int WN_>
struct Layout {
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kWaveRows = kTile / WM;
  static constexpr int kWaveCols = kTile / WN;
  static constexpr int R = kWaveRows / 32;  // accumulator row blocks
  static constexpr int C = kWaveCols / 32;  // accumulator column blocks
};

// Shape of the operand ring: RB bytes of K per row per stage, NST stages.
// A stage holds both 256-row operand tiles; copies run NST - 1 stages ahead.
//   RB = 64:  chunk slot = chunk ^ ((row >> 1) ^ (row >> 2)) & 3
//   RB = 128: chunk slot = chunk ^ (row & 7) ^ ((row >> 3) & 1)
// Either way, 8 consecutive rows read at one chunk fill a 128-byte bank
// window exactly once and 16 consecutive rows fill a 256-byte window once.
template <int RB, int NST, int WAVES>
struct Ring {
  static_assert(RB == 64 || RB == 128, "row bytes per stage");
  static constexpr int kChunks = RB / 16;              // chunks per row
  static constexpr int kSteps = RB / 32;               // MFMA K-steps
  static constexpr int kBlockRows = 1024 / RB;         // rows per 1 KiB copy
  static constexpr int kBlocks = kTile / kBlockRows / WAVES;  // per wave/op
  static constexpr int kOperandBytes = kTile * RB;
  static constexpr int kStageBytes = 2 * kOperandBytes;
  static constexpr int kCopies = 2 * kBlocks;          // per wave per stage
  static_assert(kBlocks >= 1, "every wave copies at least one block");
  static_assert(RB == 64 || kBlocks % 2 == 0, "block parity fixes the swizzle");
  static_assert(NST * kStageBytes <= kGemmLds, "ring exceeds LDS budget");
  __device__ static constexpr int swz(int row) {
    return RB == 64 ? ((row >> 1) ^ (row >> 2)) & 3
                    : (row & 7) ^ ((row >> 3) & 1);
  }
};

// One K-step of one accumulator row block (C accumulators sharing the A
// fragment): each lane supplies 16 bytes of A and 16 bytes of B per block.
//   bf16: one v_mfma_f32_32x32x16_bf16 per accumulator (lane half h carries
//         k = 8h..8h+7 of the step's 16).
//   fp32: four v_mfma_f32_32x32x2_f32 per accumulator; instruction e pairs
//         element e of the two halves' chunks. Any pairing of k between A and
//         B that is the same on both operands gives the same sum.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int C>
__device__ __forceinline__ void mma_row(f32x16_t (&acc)[C], u32x4_t a,
                                        const u32x4_t (&b)[C],
                                        const __bf16*) {
#pragma unroll
  for (int j = 0; j < C; ++j)
    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b[j]),
        acc[j], 0, 0, 0);
}
template <int C>
__device__ __forceinline__ void mma_row(f32x16_t (&acc)[C], u32x4_t a,
                                        const u32x4_t (&b)[C], const float*) {
  const f32x4_t af = __builtin_bit_cast(f32x4_t, a);
  f32x4_t bf[C];
#pragma unroll
  for (int j = 0; j < C; ++j) bf[j] = __builtin_bit_cast(f32x4_t, b[j]);
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int j = 0; j < C; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[e], bf[j][e], acc[j],
                                                    0, 0, 0);
}

typedef __attribute__((address_space(3))) char lds_char_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// A raw buffer resource (as four dwords) over the valid rows of one operand
// tile: loads past its end return zero, which masks ragged row tails.
template <typename T>
__device__ __forceinline__ i32x4_t tile_rsrc_dw(const T* base, int64_t ld,
                                                int rows) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t bytes = (uint32_t)((int64_t)rows * ld * (int64_t)sizeof(T));
  return i32x4_t{(int)(uint32_t)a, (int)((a >> 32) & 0xffff), (int)bytes,
                 0x00020000};
}

// 16 bytes per lane from global memory (resource rs, byte offset voff) into
// LDS at lds_addr + 16 * lane. Written as one asm statement so that the
// compiler's wait insertion does not track it as an LDS store: it would
// otherwise wait for every outstanding copy before unrelated LDS reads. The
// caller orders copies and reads with explicit s_waitcnt and s_barrier.
__device__ __forceinline__ void copy16_to_lds(uint32_t lds_addr,
                                              uint32_t voff, i32x4_t rs) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rs)
      : "memory", "m0");
#pragma clang diagnostic pop
}

// A byte offset that every buffer resource here rejects (loads read zero).
// Resources span less than 2^31 bytes and a block offset (fewer than 32
// blocks of at most 16 rows, rows below 2^23 bytes) added to it stays below
// 2^32, so it stays rejected.
constexpr uint32_t kOutOfRange = 0x80000000u;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14]); unnamed counters left at their maximum.
constexpr int waitcnt_vm_lgkm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14);
}

// acc = A[0:256, 0:K] . B[0:256, 0:K]^T for the workgroup's tile; this wave's
// sub-tile lands in acc (layout L). A, B point at the tile's first row;
// a_rows / b_rows are the valid rows (clamped by the caller to [0, 256]);
// 256 * ld * sizeof(T) must stay below 2^31 bytes and K must be a multiple of
// 16 bytes' worth of T (checked on the host). smem must hold kGemmLds bytes.
// Ends with every copy landed and a workgroup barrier, so smem may be reused
// right after.
//
// Global memory is copied straight into LDS by the buffer-load-to-LDS path
// (no register staging): each wave copies kBlocks 1 KiB blocks of each
// operand per stage; lane l of a block copies row l / kChunks into slot
// l % kChunks of that row, which holds the global chunk slot ^ swz(row).
// Per stage kt (ring buffer kt % NST), each of its S K-steps runs R row
// groups of C MFMAs, with the next step's fragments read at the step's
// start; the last step starts with the workgroup barrier, after which the
// wave reads stage kt + 1's first fragments and issues its copies of stage
// kt + NST into the buffer stage kt leaves (see the loop for why that order
// is safe).
template <typename T, typename L, int RB, int NST>
__device__ __forceinline__ void tile_mainloop_ring(
    f32x16_t (&acc)[L::R][L::C], const T* __restrict__ A, int64_t lda,
    int a_rows, const T* __restrict__ B, int64_t ldb, int b_rows, int64_t K,
    char* smem) {
  using P = Ring<RB, NST, L::kWaves>;
  constexpr int R = L::R, C = L::C;
  constexpr int E = Chunk<T>::E;           // elements per 16-byte chunk
  constexpr int BK = RB / (int)sizeof(T);  // elements of K per stage
  constexpr int S = P::kSteps;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int swave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform
  const int wm = wave / L::WN, wn = wave % L::WN;
  const int p = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < C; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = (int)((K + BK - 1) / BK);
  if (KT <= 0) return;
  const i32x4_t rsa = tile_rsrc_dw<T>(A, lda, a_rows);
  const i32x4_t rsb = tile_rsrc_dw<T>(B, ldb, b_rows);
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_char_t*)smem;

  // copy side: blocks kBlocks*w .. kBlocks*w + kBlocks-1 of both operands.
  // The swizzle of a row depends on its bits 0..3; block starts are
  // multiples of kBlockRows, so the lane's chunk depends on the block only
  // through bit 3 of its first row (RB = 128: blocks of 8 rows, an even
  // number per wave, so that bit is the parity of u).
  const int crow = lane / P::kChunks;
  const int slot = lane % P::kChunks;
  const int ch0 = slot ^ P::swz(crow);
  const int ch1 = slot ^ P::swz(crow + 8);
  const uint32_t pa = (uint32_t)(lda * (int64_t)sizeof(T));
  const uint32_t pb = (uint32_t)(ldb * (int64_t)sizeof(T));
  const uint32_t row0 = (uint32_t)(swave * P::kBlocks * P::kBlockRows + crow);
  const uint32_t cdst = lds + (uint32_t)(swave * P::kBlocks * 1024);
  // stages whose chunk (for even/odd blocks) lies inside K:
  // s * BK + ch * E < K  <=>  s < klim
  const int Ki = (int)K;  // K < 2^31 (checked on the host)
  const int klim0 = Ki > ch0 * E ? (Ki - ch0 * E + BK - 1) / BK : 0;
  const int klim1 = Ki > ch1 * E ? (Ki - ch1 * E + BK - 1) / BK : 0;
  const uint32_t ra0 = row0 * pa + (uint32_t)(ch0 * 16);
  const uint32_t ra1 = row0 * pa + (uint32_t)(ch1 * 16);
  const uint32_t rb0 = row0 * pb + (uint32_t)(ch0 * 16);
  const uint32_t rb1 = row0 * pb + (uint32_t)(ch1 * 16);
  uint32_t va[2], vb[2];
  // lane offsets of stage s for even/odd blocks (past K -> out of range)
  auto stage_offsets = [&](int s) {
    const uint32_t ko = (uint32_t)s * (uint32_t)RB;
    va[0] = s < klim0 ? ra0 + ko : kOutOfRange;
    vb[0] = s < klim0 ? rb0 + ko : kOutOfRange;
    if (RB == 128) {
      va[1] = s < klim1 ? ra1 + ko : kOutOfRange;
      vb[1] = s < klim1 ? rb1 + ko : kOutOfRange;
    }
  };
  // copy c of a stage: even c -> A block c/2, odd c -> B block c/2
  auto copy_one = [&](int s, int c) {
    const int u = c >> 1;
    const uint32_t dst =
        cdst + (uint32_t)((s % NST) * P::kStageBytes + u * 1024);
    const int e = (RB == 128) ? (u & 1) : 0;
    const uint32_t rows = (uint32_t)(u * P::kBlockRows);
    if ((c & 1) == 0)
      copy16_to_lds(dst, va[e] + rows * pa, rsa);
    else
      copy16_to_lds(dst + P::kOperandBytes, vb[e] + rows * pb, rsb);
  };

  // fragment side: lane (p, h) reads row (base + 32*i + p) at chunk 2s + h;
  // rows differ from p by multiples of 32, so the swizzle is swz(p).
  const int g = P::swz(p);
  const int fa = (wm * L::kWaveRows + p) * RB;
  const int fb = P::kOperandBytes + (wn * L::kWaveCols + p) * RB;
  int fo[S];
#pragma unroll
  for (int st = 0; st < S; ++st) fo[st] = ((2 * st + h) ^ g) << 4;
  u32x4_t af[2][R], bfr[2][C];
  // read number n of a step's R + C fragment reads: A0, B0..B(C-1),
  // A1..A(R-1)
  constexpr int kReads = R + C;
  auto read_one = [&](int stage_off, int st, int buf, int n) {
    if (n == 0 || n > C) {
      const int i = n == 0 ? 0 : n - C;
      af[buf][i] = *reinterpret_cast<const u32x4_t*>(
          smem + stage_off + fa + fo[st] + i * 32 * RB);
    } else {
      const int j = n - 1;
      bfr[buf][j] = *reinterpret_cast<const u32x4_t*>(
          smem + stage_off + fb + fo[st] + j * 32 * RB);
    }
  };
  // reads [n0, n1) of a step
  auto reads = [&](int stage_off, int st, int buf, int n0, int n1) {
#pragma unroll
    for (int n = 0; n < kReads; ++n)
      if (n >= n0 && n < n1) read_one(stage_off, st, buf, n);
  };

  for (int st = 0; st < NST; ++st) {
    stage_offsets(st);
#pragma unroll
    for (int c = 0; c < P::kCopies; ++c) copy_one(st, c);
  }
  // stage 0 landed (the copies of stages 1 .. NST-1 may stay outstanding)
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm((NST - 1) * P::kCopies, 15));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  reads(0, 0, 0, 0, kReads);
  const T* tag = nullptr;

  // Each step's fragment reads are spread over the previous step's row
  // groups (A0 and the B fragments first). The last step of stage kt opens
  // with the barrier, which waits until this wave's copies of stage kt + 1
  // have landed and its own LDS reads have completed: after it every wave
  // holds stage kt's fragments in registers, so buffer kt % NST is free and
  // the wave issues its copies of stage kt + NST into it while reading stage
  // kt + 1's first fragments. Copies of stages kt + 2 .. kt + NST - 1 may
  // stay outstanding at the barrier.
  constexpr int kVmAllowed = (NST - 2) * P::kCopies;
  static_assert((NST - 1) * P::kCopies <= 63, "vmcnt range");
  auto copies_at = [&](int s, int grp) {
#pragma unroll
    for (int c = 0; c < P::kCopies; ++c)
      if (c * R / P::kCopies == grp) copy_one(s, c);
  };

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = (kt % NST) * P::kStageBytes;
    const int nxt = ((kt + 1) % NST) * P::kStageBytes;
#pragma unroll
    for (int st = 0; st < S - 1; ++st) {
#pragma unroll
      for (int q = 0; q < R; ++q) {
        reads(cur, st + 1, (st + 1) & 1, q * kReads / R,
              (q + 1) * kReads / R);
        mma_row<C>(acc[q], af[st & 1][q], bfr[st & 1], tag);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    constexpr int LB = (S - 1) & 1;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(kVmAllowed, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    stage_offsets(kt + NST);
#pragma unroll
    for (int q = 0; q < R; ++q) {
      reads(nxt, 0, 0, q * kReads / R, (q + 1) * kReads / R);
      copies_at(kt + NST, q);
      mma_row<C>(acc[q], af[LB][q], bfr[LB], tag);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // drain the copies issued past K before smem is reused
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(0, 0));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Build-time shape of the engine (measured on the 1M-context slice: 4 x 2
// waves with a 2-deep ring of 128-byte slabs is the fastest of the shapes
// tried, 4% ahead of a 4-deep ring of 64-byte slabs over a full step: whole
// 128-byte lines per request, a barrier every four K-steps instead of two;
// 2 x 2 waves also work, and 3-, 4- or 5-deep 64-byte rings time the same).
#ifndef VPCE_WAVES_M
#define VPCE_WAVES_M 4
#endif
#ifndef VPCE_RING_RB
#define VPCE_RING_RB 128
#endif
#ifndef VPCE_RING_NST
#define VPCE_RING_NST 2
#endif

// The configuration every GEMM phase uses.
using TileLayout = Layout<VPCE_WAVES_M, 2>;
constexpr int kThreads = TileLayout::kThreads;

// smem must hold kGemmLds bytes.
template <typename T>
__device__ __forceinline__ void tile_mainloop(
    f32x16_t (&acc)[TileLayout::R][TileLayout::C], const T* __restrict__ A,
    int64_t lda, int a_rows, const T* __restrict__ B, int64_t ldb,
    int b_rows, int64_t K, char* smem) {
  tile_mainloop_ring<T, TileLayout, VPCE_RING_RB, VPCE_RING_NST>(
      acc, A, lda, a_rows, B, ldb, b_rows, K, smem);
}

// Workgroup L is dispatched to XCD (L mod 8). Renumber so that the workgroups
// of one XCD form one contiguous range of tile indices: neighbouring tiles,
// which share operand rows, then meet in the same XCD's L2.
__device__ __forceinline__ int xcd_remap(int L, int total) {
  const int q = total >> 3, rr = total & 7;
  const int x = L & 7, k = L >> 3;
  return x < rr ? x * (q + 1) + k : rr * (q + 1) + (x - rr) * q + k;
}

// Grouped raster: `group` consecutive M-tiles sweep all N-tiles together.
__device__ __forceinline__ void grouped_tile(int idx, int tiles_m, int tiles_n,
                                             int group, int& tm, int& tn) {
  const int per = group * tiles_n;
  const int g = idx / per;
  const int first = g * group;
  const int gs = min(group, tiles_m - first);
  const int off = idx - g * per;
  tm = first + off % gs;
  tn = off / gs;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// XOR shuffle inside each 32-lane half of the wave (ds_swizzle bitmask mode).
template <int MASK>
__device__ __forceinline__ float half_xor(float v) {
  constexpr int pattern = 0x1F | (MASK << 10);
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), pattern));
}

// Combine two (max, sum-exp) states kept in base-2 units: the result
// describes the union of both sets. Empty states are (-inf, 0).
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2,
                                         float s2) {
  const float hi = fmaxf(m, m2), lo = fminf(m, m2);
  const bool first_hi = m >= m2;
  const float s_hi = first_hi ? s : s2;
  const float s_lo = first_hi ? s2 : s;
  const float e = (hi == -INFINITY) ? 0.f : fast_exp2(lo - hi);
  m = hi;
  s = s_hi + s_lo * e;
}

}  // namespace vpce
