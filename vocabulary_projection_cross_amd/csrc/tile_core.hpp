// tile_core.hpp -- the MFMA tile engine shared by every GEMM phase of the
// blocked vocabulary-projection cross-entropy on gfx950 (CDNA4).
//
// A workgroup computes one TM x TN fp32 tile C = A . B^T where A [M x K] and
// B [Nc x K] are both row-major with K contiguous ("NT" form). Its waves split
// the tile as Layout<TM, TN, WM, WN> says (4 x 2 waves, two per SIMD, of
// 64 x 128 on a 256 x 256 tile or 64 x 160 on a 256 x 320 tile); each wave
// holds its sub-tile as R x C accumulators of MB x MB MFMA blocks (MB = 16 by
// default, 32 as a build option):
//   element r of accumulator (i, j) on lane l is
//   row = i*MB + 8*(r/4) + 4*(l/MB) + (r%4),  col = j*MB + (l%MB)
// within the wave's sub-tile (MB = 16: r = 0..3; MB = 32: r = 0..15).
//
// Operands stream through a ring of NST LDS stages of RB bytes of K per row
// (128 B x 2 stages by default), copied global -> LDS by buffer loads that
// write LDS directly, NST - 1 stages ahead of the MFMAs. Within a row the
// 16-byte chunk index is XOR-swizzled by row bits, so the MFMA fragment reads
// hit 64 distinct banks in every LDS cycle (see Ring); the copies write 1 KiB
// contiguous blocks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace vpce {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kLdsBytes = 160 * 1024;  // LDS of one workgroup on gfx950

// Build-time shape of the engine. Measured on the 1M-context slice: a 2-deep
// ring of 128-byte slabs is 4% ahead of a 4-deep ring of 64-byte slabs over a
// full step (whole 128-byte lines per request, a barrier every four K-steps
// of 32 x 32 blocks instead of two), and 4 x 2 waves ahead of 2 x 2. 64-byte
// slabs copy 16-row blocks, which a 320-row operand does not split into over
// 8 waves, so they build only with VPCE_WIDE_COLS=256. These options shape
// the forward and the logit recompute; the products are fixed (see
// TileLayout). For the products, a 3-, 4- or 5-deep ring of 64-byte slabs
// was measured 4% slower than the two-stage ring of 128-byte slabs.
#ifndef VPCE_WAVES_M
#define VPCE_WAVES_M 4
#endif
#ifndef VPCE_RING_RB
#define VPCE_RING_RB 128
#endif
#ifndef VPCE_RING_NST
#define VPCE_RING_NST 2
#endif
#ifndef VPCE_WIDE_COLS
#define VPCE_WIDE_COLS 320
#endif
// Side of the MFMA output block: 16 (v_mfma_f32_16x16x32_bf16) or 32
// (v_mfma_f32_32x32x16_bf16). Both have the same nominal rate, but the 16 x 16
// form reads and writes half the accumulator bytes per flop, and on random
// bf16 operands the chip, which lowers its clock under MFMA load, holds about
// 2.0 GHz with it against 1.8 GHz with 32 x 32 blocks. Measured on the
// 1M-context slice: forward 12% and logit recompute 7% faster with 16 x 16.
#ifndef VPCE_MFMA_BLOCK
#define VPCE_MFMA_BLOCK 16
#endif


// Elements of T per 16-byte chunk.
template <typename T> struct Chunk;
template <> struct Chunk<__bf16> { static constexpr int E = 8; };
template <> struct Chunk<float> { static constexpr int E = 4; };

// How the waves of a workgroup split a TM x TN tile: WM x WN waves, each
// owning a (TM/WM) x (TN/WN) sub-tile held as R x C accumulators of MB x MB
// MFMA blocks. Wave w sits at (w / WN, w % WN). With 8 waves two of them share
// each SIMD, so one wave's MFMAs keep the matrix unit busy while the other
// waits to issue a copy or an LDS read.
//
// Accumulator layout (element r of accumulator (i, j) on lane l), within the
// wave's sub-tile, for either block side:
//   row = i*MB + 8*(r/4) + 4*(l/MB) + (r%4),  col = j*MB + (l%MB)
// (MB = 32: 16 elements, 4 groups of 4 consecutive rows; MB = 16: 4 elements,
// one group). row_base(i, g, l) is the first of group g's 4 rows.
//
// Per K-step a wave runs its R x C MFMAs in NG groups along its longer side
// (column groups when C > R: group j pairs B fragment j with every A
// fragment), and spreads the next step's fragment reads and, after the
// barrier, the stage's copies over those groups. Many small groups issue the
// copies in small bunches between MFMAs: on a 64 x 160 sub-tile five column
// groups of two MFMAs take 7% less time than two row groups of five.
template <int MB> struct AccOf;
template <> struct AccOf<32> { typedef f32x16_t type; };
template <> struct AccOf<16> {
  typedef float type __attribute__((ext_vector_type(4)));
};

template <int TM_, int TN_, int WM_, int WN_, int MB_ = VPCE_MFMA_BLOCK,
          int RB_ = VPCE_RING_RB, int NST_ = VPCE_RING_NST>
struct Layout {
  static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_, MB = MB_;
  static constexpr int RB = RB_, NST = NST_;  // operand ring (see Ring)
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kWaveRows = TM / WM;
  static constexpr int kWaveCols = TN / WN;
  static constexpr int R = kWaveRows / MB;  // accumulator row blocks
  static constexpr int C = kWaveCols / MB;  // accumulator column blocks
  static constexpr int kAccRegs = MB * MB / 64;  // fp32 elements per lane
  static constexpr int kRowGroups = kAccRegs / 4;
  typedef typename AccOf<MB>::type Acc;
  static constexpr bool kColGroups = C > R;
  static constexpr int NG = kColGroups ? C : R;  // MFMA groups per K-step
  static_assert(MB == 16 || MB == 32, "MFMA block side");
  static_assert(kWaveRows * WM == TM && kWaveCols * WN == TN &&
                    kWaveRows % MB == 0 && kWaveCols % MB == 0,
                "whole MFMA blocks per wave");
  __device__ static constexpr int row_base(int i, int g, int lane) {
    return i * MB + 8 * g + 4 * (lane / MB);
  }
  __device__ static constexpr int col(int j, int lane) {
    return j * MB + lane % MB;
  }
};

// Shape of the operand ring: RB bytes of K per row per stage, NST stages.
// A stage holds the TM-row A tile and the TN-row B tile; copies run NST - 1
// stages ahead.
//   RB = 64:  chunk slot = chunk ^ ((row >> 1) ^ (row >> 2)) & 3
//   RB = 128: chunk slot = chunk ^ (row & 7) ^ ((row >> 4) & 1)
// The LDS (64 banks of 4 bytes) serves a 16-byte read 16 lanes per cycle:
// the 8-lane groups g and g ^ 3 (lanes 0-7 with 24-31, 8-15 with 16-23, and
// likewise in the upper half), as timed on gfx950 with probe patterns. Two
// such groups read rows r..r+7 and r+24..r+31 at one chunk (32 x 32
// fragments) or rows r..r+7 and r+8..r+15 at chunks c and c ^ 1 (16 x 16
// fragments); the swizzle sends either set to 64 distinct banks. (With row
// bit 3 in place of bit 4, 16 x 16 fragment reads collide two ways and cost
// twice the LDS cycles.)
// Stage layout of a K-outer operand: in memory each row is one k (the
// tile's TX entries of the M or N side are contiguous in it), so a stage holds
// BK k-rows of TX entries, row k at k * kRowBytes (two rows per 1 KiB copy
// block for bf16 tiles of 256, one for fp32). In a bf16 row k the logical
// 32-byte segment s sits at segment s ^ f(k), f(k) = (k & 3) | ((k >> 3) & 1)
// << 2. A transposing read (see tile_mainloop_ring) touches k-rows
// {8h + 4e + j : j < 4} of one logical segment in each 16-lane group h; the
// groups h = 0, 1 (and 2, 3) thus see f = j + 4 (h & 1), eight distinct
// segments, 64 distinct banks. Measured on gfx950 with probe patterns: 306
// bytes per clock per compute unit for such reads, against 289 for the
// swizzled 16-byte fragment reads of K-contiguous operands (and 72 for the
// same transposing reads without the XOR). fp32 rows are not swizzled.
template <typename T, int TX, int RB>
struct KOuter {
  static constexpr int kRowBytes = TX * (int)sizeof(T);
  // (defined for every tile width so that K-contiguous uses of Ring can name
  // it; only kSupported shapes are ever read K-outer)
  static constexpr int kRows = kRowBytes <= 1024 ? 1024 / kRowBytes : 1;
  static constexpr int BK = RB / (int)sizeof(T);
  static constexpr int kBlocks = BK / kRows;
  static constexpr int kBytes = BK * kRowBytes;
  static constexpr int kChunksPerRow = kRowBytes / 16;
  // rows of 512 (bf16) or 1024 bytes (fp32): tiles of 256 entries
  static constexpr bool kSupported = kRows * kRowBytes == 1024 &&
                                     kBlocks * kRows == BK &&
                                     (kRows == 1 || kRows == 2);
  __device__ static constexpr int swz(int k) {
    return sizeof(T) == 2 ? (k & 3) | (((k >> 3) & 1) << 2) : 0;
  }
};

template <int RB, int NST, int TM, int TN, int WAVES, typename T = __bf16,
          bool TA = false, bool TB = false>
struct Ring {
  static_assert(RB == 64 || RB == 128, "row bytes per stage");
  static constexpr int kChunks = RB / 16;              // chunks per row
  static constexpr int kBlockRows = 1024 / RB;         // rows per 1 KiB copy
  using KA = KOuter<T, TM, RB>;
  using KB = KOuter<T, TN, RB>;
  static constexpr int kBlocksA =
      (TA ? KA::kBlocks : TM / kBlockRows) / WAVES;  // per wave
  static constexpr int kBlocksB = (TB ? KB::kBlocks : TN / kBlockRows) / WAVES;
  static constexpr int kOperandBytesA = TA ? KA::kBytes : TM * RB;
  static constexpr int kOperandBytesB = TB ? KB::kBytes : TN * RB;
  static constexpr int kStageBytes = kOperandBytesA + kOperandBytesB;
  static constexpr int kBytes = NST * kStageBytes;
  static constexpr int kCopies = kBlocksA + kBlocksB;  // per wave per stage
  static_assert((TA ? kBlocksA * WAVES == KA::kBlocks
                    : kBlocksA * kBlockRows * WAVES == TM) &&
                    (TB ? kBlocksB * WAVES == KB::kBlocks
                        : kBlocksB * kBlockRows * WAVES == TN) &&
                    kBlocksA >= 1 && kBlocksB >= 1,
                "every wave copies whole blocks of both operands");
  static_assert(kBytes <= kLdsBytes, "ring exceeds the LDS");
  __device__ static constexpr int swz(int row) {
    return RB == 64 ? ((row >> 1) ^ (row >> 2)) & 3
                    : (row & 7) ^ ((row >> 4) & 1);
  }
};

// One K-step of MFMA group q (see Layout): row group q updates accumulators
// (q, 0..C-1), column group q updates (0..R-1, q). Each lane supplies 16
// bytes of A and 16 bytes of B per MFMA block; lane l serves row l % MB of
// the block and K-chunk l / MB of the step's 64 / MB chunks.
//   bf16, MB = 32: one v_mfma_f32_32x32x16_bf16 per accumulator (K = 16).
//   bf16, MB = 16: one v_mfma_f32_16x16x32_bf16 per accumulator (K = 32).
//   fp32: four v_mfma_f32_32x32x2_f32 (16x16x4_f32) per accumulator;
//         instruction e pairs element e of every lane's chunk. Any pairing of
//         k between A and B that is the same on both operands gives the same
//         sum.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename L>
__device__ __forceinline__ typename L::Acc mfma_block(const u32x4_t& a,
                                                      const u32x4_t& b,
                                                      typename L::Acc c,
                                                      const __bf16*) {
  if constexpr (L::MB == 32)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
        0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
        0, 0, 0);
}
// fp32: element e of both chunks (one step of four; see mma_group).
template <typename L>
__device__ __forceinline__ typename L::Acc mfma_block_f32(float a, float b,
                                                          typename L::Acc c) {
  if constexpr (L::MB == 32)
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename L, typename T>
__device__ __forceinline__ void mma_group(typename L::Acc (&acc)[L::R][L::C],
                                          const u32x4_t (&a)[L::R],
                                          const u32x4_t (&b)[L::C], int q,
                                          const T* tag) {
  constexpr int GS = L::kColGroups ? L::R : L::C;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      const int i = L::kColGroups ? g : q, j = L::kColGroups ? q : g;
      acc[i][j] = mfma_block<L>(a[i], b[j], acc[i][j], tag);
    }
  } else {
    // the four instructions of one accumulator are interleaved with the
    // group's other accumulators, so consecutive MFMAs are independent
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        const int i = L::kColGroups ? g : q, j = L::kColGroups ? q : g;
        acc[i][j] = mfma_block_f32<L>(__builtin_bit_cast(f32x4_t, a[i])[e],
                                      __builtin_bit_cast(f32x4_t, b[j])[e],
                                      acc[i][j]);
      }
  }
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
// Resources span less than 2^31 bytes, and a block offset added to it (at
// most 256 rows of a K-contiguous operand's pitch, a row of fp32 H or W:
// 4 d bytes) leaves it below 2^32, so it stays rejected. The library checks
// that bound against its largest d at compile time. K-outer operands never
// take this offset: their stages past K get an empty resource instead.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int64_t kMaxBlockOffsetRows = 256;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14]); unnamed counters left at their maximum.
constexpr int waitcnt_vm_lgkm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14);
}

// acc = A[0:TM, 0:K] . B[0:TN, 0:K]^T for the workgroup's tile; this wave's
// sub-tile lands in acc (layout L).
//
// Each operand is K-contiguous (the default: rows of memory are rows of the
// tile, K runs along them) or K-outer (TA / TB: rows of memory are k, the
// tile's entries run along them, as for the token-major G, H and W read by
// the backward products).
//  * K-contiguous X: X points at the tile's first row, ldx is the row pitch,
//    x_rows the valid rows (clamped by the caller to [0, TM] or [0, TN]);
//    TM * ldx * sizeof(T) stays below 2^31 bytes; chunks past K read zero.
//  * K-outer X: X points at row k = 0 of the whole matrix, x_col0 is the
//    tile's first entry in a row, ldx the row pitch (a multiple of 16 bytes),
//    x_rows the valid k-rows: rows past it read zero. Entries past the end of
//    a row are the next row's (they only reach outputs the caller discards);
//    the matrix ends at row x_rows. BK * ldx * sizeof(T) stays below 2^31.
// K must be a multiple of 16 bytes' worth of T (checked on the host). smem
// must hold the ring's kBytes. Ends with every copy landed and a workgroup
// barrier, so smem may be reused right after.
//
// Global memory is copied straight into LDS by the buffer-load-to-LDS path
// (no register staging): per stage each wave copies kBlocksA 1 KiB blocks of
// A and kBlocksB of B (every W-th block, W waves). K-contiguous: lane l of a
// block copies row l / kChunks into slot l % kChunks of that row, which holds
// the global chunk slot ^ swz(row). K-outer: lane l copies row l / 32 of the
// block (bf16; fp32 blocks are one row) into slot l % 32 of it, which holds
// the row's chunk with the segment XOR of KOuter; the stage's buffer
// resource starts at its first k-row, so the 32-bit offsets stay small
// however long K is.
// Per stage kt (ring buffer kt % NST), each of its S K-steps runs the NG MFMA
// groups, with the next step's fragments read at the step's start; the last
// step starts with the workgroup barrier, after which the wave reads stage
// kt + 1's first fragments and issues its copies of stage kt + NST into the
// buffer stage kt leaves (see the loop for why that order is safe).
//
// A K-outer bf16 fragment is two transposing reads (ds_read_b64_tr_b16):
// within each 16-lane group, lane 4a + b receives element b of the 8-byte
// pieces addressed by lanes a, a + 4, a + 8 and a + 12. Lane a + 4j (group h)
// addresses k-row 32 st + 8h + 4e + j, entries 4a .. 4a + 3 of the 16-entry
// block, so lane p of the group receives k-rows 8h + 4e .. 8h + 4e + 3 of
// entry p: read e = 0 and e = 1 together give the same 8 values of K that the
// K-contiguous fragment holds, and the MFMAs see the same operands either
// way. fp32 K-outer fragments are four 4-byte reads down a column.
template <typename T, typename L, int RB, int NST, bool TA = false,
          bool TB = false>
__device__ __forceinline__ void tile_mainloop_ring(
    typename L::Acc (&acc)[L::R][L::C], const T* __restrict__ A, int64_t lda,
    int a_rows, const T* __restrict__ B, int64_t ldb, int b_rows, int64_t K,
    char* smem, int a_col0 = 0, int b_col0 = 0) {
  using P = Ring<RB, NST, L::TM, L::TN, L::kWaves, T, TA, TB>;
  constexpr int R = L::R, C = L::C, NG = L::NG, MB = L::MB;
  constexpr int E = Chunk<T>::E;           // elements per 16-byte chunk
  constexpr int BK = RB / (int)sizeof(T);  // elements of K per stage
  constexpr int CPS = 64 / MB;             // 16-byte chunks per K-step
  constexpr int S = P::kChunks / CPS;      // K-steps per stage
  static_assert(S >= 1 && S * CPS == P::kChunks, "whole K-steps per stage");
  static_assert(!(TA || TB) || (MB == 16 && RB == 128),
                "K-outer operands: 16 x 16 blocks, 128-byte stages");
  constexpr int KA = P::kBlocksA, KB = P::kBlocksB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int swave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform
  const int wm = wave / L::WN, wn = wave % L::WN;
  const int p = lane % MB, h = lane / MB;
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < C; ++j)
#pragma unroll
      for (int r = 0; r < L::kAccRegs; ++r) acc[i][j][r] = 0.f;

  const int KT = (int)((K + BK - 1) / BK);
  if (KT <= 0) return;
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_char_t*)smem;
  constexpr int W = L::kWaves;
  const uint32_t pa = (uint32_t)(lda * (int64_t)sizeof(T));
  const uint32_t pb = (uint32_t)(ldb * (int64_t)sizeof(T));
  const uint32_t dsta = lds + (uint32_t)(swave * 1024);
  const uint32_t dstb = lds + (uint32_t)(P::kOperandBytesA + swave * 1024);

  // K-contiguous copy side: wave w copies blocks w, w + W, w + 2W, ... (W
  // waves) of each operand; lane l copies row crow = l / kChunks of a block
  // into slot l % kChunks. The swizzle depends on row bits 0..4 only and W
  // blocks span a multiple of 32 rows, so every block of a wave has the same
  // swizzle pattern, that of the wave's first block: one chunk per lane.
  static_assert((L::kWaves * P::kBlockRows) % 32 == 0 &&
                    (P::kBlocksA - 1) * L::kWaves * P::kBlockRows <=
                        kMaxBlockOffsetRows &&
                    (P::kBlocksB - 1) * L::kWaves * P::kBlockRows <=
                        kMaxBlockOffsetRows,
                "a wave's blocks share their swizzle; block offsets stay "
                "within kMaxBlockOffsetRows rows (see kOutOfRange)");
  const int crow = lane / P::kChunks;
  const int slot = lane % P::kChunks;
  const int ch = slot ^ P::swz(swave * P::kBlockRows + crow);
  const uint32_t row0 = (uint32_t)(swave * P::kBlockRows + crow);
  // stages whose chunk lies inside K: s * BK + ch * E < K  <=>  s < klim
  const int Ki = (int)K;  // K < 2^31 (checked on the host)
  const int kl = Ki > ch * E ? (Ki - ch * E + BK - 1) / BK : 0;
  const uint32_t ra = row0 * pa + (uint32_t)(ch * 16);
  const uint32_t rb = row0 * pb + (uint32_t)(ch * 16);

  // K-outer copy side: lane l copies k-row k = w kRows + l / kChunksPerRow
  // of its wave's block into slot l % kChunksPerRow, which holds the row's
  // chunk slot ^ (2 swz(k)) (the segment XOR). The wave's later blocks are
  // W kRows = 16 rows further on, which leaves k's bits 0, 1 and 3, and so
  // the XOR, unchanged: one chunk per lane.
  static_assert((!TA || P::KA::kSupported) && (!TB || P::KB::kSupported),
                "K-outer tiles of 256 entries (bf16 or fp32)");
  static_assert(sizeof(T) == 4 ||
                    ((!TA || (W * P::KA::kRows) % 16 == 0) &&
                     (!TB || (W * P::KB::kRows) % 16 == 0)),
                "a wave's K-outer blocks share their XOR pattern");
  auto kouter_lane = [&](auto ko, uint32_t pitch) -> uint32_t {
    using KO = decltype(ko);
    const int k = swave * KO::kRows + lane / KO::kChunksPerRow;
    const int c = (lane % KO::kChunksPerRow) ^ (2 * KO::swz(k));
    return (uint32_t)k * pitch + (uint32_t)(c * 16);
  };
  const uint32_t ta_lane = TA ? kouter_lane(typename P::KA{}, pa) : 0u;
  const uint32_t tb_lane = TB ? kouter_lane(typename P::KB{}, pb) : 0u;
  // bytes of a K-outer operand readable from its tile start (k-row 0, entry
  // x_col0): the valid k-rows, less the part of the last row before x_col0
  const int64_t a_valid = (int64_t)a_rows * pa - (int64_t)a_col0 * sizeof(T);
  const int64_t b_valid = (int64_t)b_rows * pb - (int64_t)b_col0 * sizeof(T);
  // a K-outer operand's resource for stage s: its BK k-rows, clipped to the
  // valid bytes (rows past them read zero)
  auto kouter_rsrc = [&](const T* X, int col0, uint32_t pitch, int64_t valid,
                         int s) -> i32x4_t {
    const int64_t stage = (int64_t)BK * pitch;
    const int64_t off = (int64_t)s * stage;
    int64_t rem = valid - off;
    rem = rem < 0 ? 0 : (rem > stage ? stage : rem);
    const uint64_t a = (uint64_t)(uintptr_t)(X + col0) + (uint64_t)off;
    return i32x4_t{(int)(uint32_t)a, (int)((a >> 32) & 0xffff), (int)(uint32_t)rem,
                   0x00020000};
  };
  i32x4_t rsa = TA ? i32x4_t{0, 0, 0, 0} : tile_rsrc_dw<T>(A, lda, a_rows);
  i32x4_t rsb = TB ? i32x4_t{0, 0, 0, 0} : tile_rsrc_dw<T>(B, ldb, b_rows);
  uint32_t va = 0, vb = 0;
  // stage s: lane offsets (K-contiguous, past K -> out of range) or the
  // stage's resource (K-outer)
  auto stage_offsets = [&](int s) {
    const uint32_t ko = (uint32_t)s * (uint32_t)RB;
    if constexpr (TA) rsa = kouter_rsrc(A, a_col0, pa, a_valid, s);
    else va = s < kl ? ra + ko : kOutOfRange;
    if constexpr (TB) rsb = kouter_rsrc(B, b_col0, pb, b_valid, s);
    else vb = s < kl ? rb + ko : kOutOfRange;
  };
  // copy c of a stage: A and B blocks alternate while both last, then the
  // rest of the larger operand
  constexpr int MinAB = KA < KB ? KA : KB;
  auto copy_one = [&](int s, int c) {
    const bool is_a = c < 2 * MinAB ? (c & 1) == 0 : KA > KB;
    const int u = c < 2 * MinAB ? c >> 1 : MinAB + (c - 2 * MinAB);
    if (is_a) {
      if constexpr (TA)
        copy16_to_lds(dsta + (uint32_t)((s % NST) * P::kStageBytes +
                                        u * W * 1024),
                      ta_lane + (uint32_t)(u * W * P::KA::kRows) * pa, rsa);
      else
        copy16_to_lds(dsta + (uint32_t)((s % NST) * P::kStageBytes +
                                        u * W * 1024),
                      va + (uint32_t)(u * W * P::kBlockRows) * pa, rsa);
    } else {
      if constexpr (TB)
        copy16_to_lds(dstb + (uint32_t)((s % NST) * P::kStageBytes +
                                        u * W * 1024),
                      tb_lane + (uint32_t)(u * W * P::KB::kRows) * pb, rsb);
      else
        copy16_to_lds(dstb + (uint32_t)((s % NST) * P::kStageBytes +
                                        u * W * 1024),
                      vb + (uint32_t)(u * W * P::kBlockRows) * pb, rsb);
    }
  };

  // fragment side, K-contiguous: lane (p, h) reads row (base + MB*x + p) at
  // chunk CPS*s + h. The wave's first rows are multiples of 32, so the row's
  // bits 0..2 are p's and its bit 4 is p's (MB = 32) or x's bit 0 (MB = 16):
  // the swizzle is swz(p), flipped for odd x when MB = 16 and RB = 128.
  static_assert(L::kWaveRows % 32 == 0 && L::kWaveCols % 32 == 0,
                "wave sub-tiles start at multiples of 32 rows");
  const int g = P::swz(p);
  const int fa = (wm * L::kWaveRows + p) * RB;
  const int fb = P::kOperandBytesA + (wn * L::kWaveCols + p) * RB;
  int fo[S];
#pragma unroll
  for (int st = 0; st < S; ++st) fo[st] = ((CPS * st + h) ^ g) << 4;
  auto xflip = [](int x) { return MB == 16 && RB == 128 ? (x & 1) << 4 : 0; };

  // fragment side, K-outer bf16 (see the transposing read above): lane
  // (a = lane % 4, j = lane / 4 % 4, group h) of read e of K-step st
  // addresses k-row 32 st + 8h + 4e + j, entries 4a .. 4a + 3 of 16-entry
  // block x of the wave's blocks, whose first is segment seg0 (a multiple of
  // 4 for A, of 8 for B, so seg0 + x = seg0 ^ x). That k-row's XOR is
  // f = j | (h & 1) << 2 for every st and e, so the byte offset is
  // (base ^ (x << 5)) + 512 (32 st + 4e) with base = (8h + j) 512 + 8a +
  // ((seg0 ^ f) << 5): bits 5..8 of base hold the segment, and the terms
  // added after the XOR have none of those bits.
  const int tj = (lane >> 2) & 3;
  const int t_f = tj | ((h & 1) << 2);
  const int t_lane = (8 * h + tj) * 512 + 8 * (lane & 3);
  const int ta_base = TA ? t_lane + (((wm * L::kWaveRows / 16) ^ t_f) << 5) : 0;
  const int tb_base = TB ? t_lane + (((wn * L::kWaveCols / 16) ^ t_f) << 5) : 0;
  static_assert(!TA || (L::kWaveRows / 16) % 4 == 0 && R <= 4,
                "A's wave blocks: seg0 a multiple of 4, at most 4 blocks");
  static_assert(!TB || (L::kWaveCols / 16) % 8 == 0 && C <= 8,
                "B's wave blocks: seg0 a multiple of 8, at most 8 blocks");
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
  // the two transposing reads of a fragment: k-rows 8h + j and 8h + 4 + j
  // (2 KiB further on) from byte offset o
  auto tr_pair = [&](int o) {
    const s16x4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(lds_char_t*)(smem + o));
    const s16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(lds_char_t*)(smem + o + 4 * 512));
    const u32x2_t q0 = __builtin_bit_cast(u32x2_t, r0);
    const u32x2_t q1 = __builtin_bit_cast(u32x2_t, r1);
    return u32x4_t{q0[0], q0[1], q1[0], q1[1]};
  };
  // fp32 K-outer: lane (p, h) gathers k-rows 16 st + 4h + i (i < 4) of entry
  // wbase + 16x + p, 1 KiB apart
  auto f32_col = [&](int o) {
    const float* q = reinterpret_cast<const float*>(smem + o);
    return u32x4_t{__builtin_bit_cast(uint32_t, q[0]),
                   __builtin_bit_cast(uint32_t, q[256]),
                   __builtin_bit_cast(uint32_t, q[512]),
                   __builtin_bit_cast(uint32_t, q[768])};
  };
  auto frag_a = [&](int stage_off, int st, int x) {
    if constexpr (TA) {
      if constexpr (sizeof(T) == 2)
        return tr_pair((ta_base ^ (x << 5)) + stage_off + 32 * st * 512);
      else
        return f32_col(stage_off + (16 * st + 4 * h) * 1024 +
                       (wm * L::kWaveRows + 16 * x + p) * 4);
    } else {
      return *reinterpret_cast<const u32x4_t*>(
          smem + stage_off + fa + (fo[st] ^ xflip(x)) + x * MB * RB);
    }
  };
  auto frag_b = [&](int stage_off, int st, int x) {
    if constexpr (TB) {
      if constexpr (sizeof(T) == 2)
        return tr_pair((tb_base ^ (x << 5)) + stage_off + P::kOperandBytesA +
                       32 * st * 512);
      else
        return f32_col(stage_off + P::kOperandBytesA +
                       (16 * st + 4 * h) * 1024 +
                       (wn * L::kWaveCols + 16 * x + p) * 4);
    } else {
      return *reinterpret_cast<const u32x4_t*>(
          smem + stage_off + fb + (fo[st] ^ xflip(x)) + x * MB * RB);
    }
  };
  const T* tag = nullptr;

  // The last step of stage kt opens with the barrier, which waits until this
  // wave's copies of stage kt + 1 have landed and its own LDS reads have
  // completed: after it every wave holds stage kt's last fragments in
  // registers, so buffer kt % NST is free and the wave issues its copies of
  // stage kt + NST into it while reading stage kt + 1's first fragments.
  // Copies of stages kt + 2 .. kt + NST - 1 may stay outstanding at the
  // barrier.
  constexpr int kVmAllowed = (NST - 2) * P::kCopies;
  static_assert((NST - 1) * P::kCopies <= 63, "vmcnt range");
  auto copies_at = [&](int s, int grp) {
#pragma unroll
    for (int c = 0; c < P::kCopies; ++c)
      if (c * NG / P::kCopies == grp) copy_one(s, c);
  };
  auto prologue = [&]() {
    for (int st = 0; st < NST; ++st) {
      stage_offsets(st);
#pragma unroll
      for (int c = 0; c < P::kCopies; ++c) copy_one(st, c);
    }
    // stage 0 landed (the copies of stages 1 .. NST-1 may stay outstanding)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm((NST - 1) * P::kCopies, 15));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  if constexpr (MB == 32) {
    // Two fragment sets by step parity: each step's R + C reads are spread
    // over the previous step's groups (the first group's fragments first).
    u32x4_t af[2][R], bfr[2][C];
    // read number n of a step's R + C fragment reads, in the order the
    // groups need them: row groups A0, B0..B(C-1), A1..A(R-1); column groups
    // B0, A0..A(R-1), B1..B(C-1)
    constexpr int kReads = R + C;
    auto read_one = [&](int stage_off, int st, int buf, int n) {
      bool is_a;
      int x;
      if (!L::kColGroups) {
        is_a = n == 0 || n > C;
        x = n == 0 ? 0 : (n > C ? n - C : n - 1);
      } else {
        is_a = n >= 1 && n <= R;
        x = n == 0 ? 0 : (n <= R ? n - 1 : n - R);
      }
      if (is_a)
        af[buf][x] = frag_a(stage_off, st, x);
      else
        bfr[buf][x] = frag_b(stage_off, st, x);
    };
    // reads [n0, n1) of a step
    auto reads = [&](int stage_off, int st, int buf, int n0, int n1) {
#pragma unroll
      for (int n = 0; n < kReads; ++n)
        if (n >= n0 && n < n1) read_one(stage_off, st, buf, n);
    };
    prologue();
    reads(0, 0, 0, 0, kReads);
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = (kt % NST) * P::kStageBytes;
      const int nxt = ((kt + 1) % NST) * P::kStageBytes;
#pragma unroll
      for (int st = 0; st < S - 1; ++st) {
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          reads(cur, st + 1, (st + 1) & 1, q * kReads / NG,
                (q + 1) * kReads / NG);
          mma_group<L>(acc, af[st & 1], bfr[st & 1], q, tag);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      constexpr int LB = (S - 1) & 1;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(kVmAllowed, 0));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      stage_offsets(kt + NST);
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        reads(nxt, 0, 0, q * kReads / NG, (q + 1) * kReads / NG);
        copies_at(kt + NST, q);
        mma_group<L>(acc, af[LB], bfr[LB], q, tag);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    // MB = 16, column groups: every group uses all R A-fragments, group q
    // B-fragment q. A has two sets by step parity (the next step's A is read
    // during the current step, in its first R groups); B has one set,
    // refilled in place: right after group q's MFMAs the wave reads the next
    // step's B fragment q into it, so a step holds R + C fragments of its own
    // plus R of the next (a second B set would not fit beside 160
    // accumulator registers). With an odd number of steps per stage the
    // stages alternate in which A set they start with, so the stage loop runs
    // two stages per iteration.
    static_assert(L::kColGroups, "16 x 16 blocks: column groups");
    u32x4_t af[2][R], bfr[C];
    prologue();
#pragma unroll
    for (int x = 0; x < C; ++x) bfr[x] = frag_b(0, 0, x);
#pragma unroll
    for (int x = 0; x < R; ++x) af[0][x] = frag_a(0, 0, x);
    // stage kt, whose first step uses A set A0
    auto run_stage = [&](int kt, auto a0) {
      constexpr int A0 = decltype(a0)::value;
      const int cur = (kt % NST) * P::kStageBytes;
      const int nxt = ((kt + 1) % NST) * P::kStageBytes;
#pragma unroll
      for (int st = 0; st < S - 1; ++st) {
        const int as = (A0 + st) & 1;
#pragma unroll
        for (int q = 0; q < C; ++q) {
          mma_group<L>(acc, af[as], bfr, q, tag);
          __builtin_amdgcn_sched_barrier(0);
          bfr[q] = frag_b(cur, st + 1, q);
          if (q < R) af[as ^ 1][q] = frag_a(cur, st + 1, q);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      constexpr int LB = (A0 + S - 1) & 1;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(kVmAllowed, 0));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      stage_offsets(kt + NST);
#pragma unroll
      for (int q = 0; q < C; ++q) {
        mma_group<L>(acc, af[LB], bfr, q, tag);
        __builtin_amdgcn_sched_barrier(0);
        bfr[q] = frag_b(nxt, 0, q);
        if (q < R) af[LB ^ 1][q] = frag_a(nxt, 0, q);
        copies_at(kt + NST, q);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (S % 2 == 0) {
      for (int kt = 0; kt < KT; ++kt)
        run_stage(kt, std::integral_constant<int, 0>{});
    } else {
      for (int kt = 0; kt < KT; kt += 2) {
        run_stage(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < KT) run_stage(kt + 1, std::integral_constant<int, 1>{});
      }
    }
  }
  // drain the copies issued past K before smem is reused
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(0, 0));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// The two configurations: 256 x 256 tiles for the dW and dH products (whose
// output dimensions are multiples of 256 in the usual shapes), 256 x 320 tiles
// (vocabulary on the 320 side) for the forward and the logit recompute.
// The products read K-outer operands, which take 16 x 16 blocks and a
// two-stage ring of 128-byte K-slabs (the build options below apply to the
// forward and the logit recompute only).
using TileLayout = Layout<256, 256, VPCE_WAVES_M, 2, 16, 128, 2>;
// 128 x 256 tiles (32 x 128 per wave) for products whose 256 x 256 grid would
// leave compute units idle: twice the tiles, at 50% more copied bytes per
// flop.
using HalfTileLayout = Layout<128, 256, 4, 2, 16, 128, 2>;
using WideLayout = Layout<256, VPCE_WIDE_COLS, 4, 2>;
template <typename L, typename T = __bf16, bool TA = false, bool TB = false>
using RingOf = Ring<L::RB, L::NST, L::TM, L::TN, L::kWaves, T, TA, TB>;

// smem must hold RingOf<L, T, TA, TB>::kBytes.
template <typename T, typename L, bool TA = false, bool TB = false>
__device__ __forceinline__ void tile_mainloop(
    typename L::Acc (&acc)[L::R][L::C], const T* __restrict__ A, int64_t lda,
    int a_rows, const T* __restrict__ B, int64_t ldb, int b_rows, int64_t K,
    char* smem, int a_col0 = 0, int b_col0 = 0) {
  tile_mainloop_ring<T, L, L::RB, L::NST, TA, TB>(
      acc, A, lda, a_rows, B, ldb, b_rows, K, smem, a_col0, b_col0);
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

// Workgroup barrier that orders LDS accesses only (s_waitcnt lgkmcnt(0);
// s_barrier): unlike __syncthreads it does not wait for the wave's global
// stores, which stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

// Exchange within each 16-lane DPP row with a partner whose lane index differs
// from this lane's in bit log2(MASK): p ^ 1 and p ^ 2 (quad permutations),
// the half-row mirror 7 - p (bit 2) and the row mirror 15 - p (bit 3).
template <int MASK>
__device__ __forceinline__ float row_partner(float v) {
  constexpr int ctrl = MASK == 1   ? 0xB1    // quad_perm [1, 0, 3, 2]
                       : MASK == 2 ? 0x4E    // quad_perm [2, 3, 0, 1]
                       : MASK == 4 ? 0x141   // row_half_mirror
                                   : 0x140;  // row_mirror
  static_assert(MASK == 1 || MASK == 2 || MASK == 4 || MASK == 8,
                "partner bit");
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF,
                                      0xF, false));
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
