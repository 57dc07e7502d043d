// tile_core.hpp -- the MFMA tile engine shared by every GEMM phase of the
// blocked vocabulary-projection cross-entropy on gfx950 (CDNA4).
//
// One workgroup of 256 threads (4 wave64s in a 2x2 arrangement) computes a
// 256 x 256 fp32 tile C = A . B^T where A [M x K] and B [Nc x K] are both
// row-major with K contiguous ("NT" form). Each wave owns a 128 x 128 sub-tile
// held as 4 x 4 accumulators of the 32x32 MFMA layout:
//   element r (0..15) of accumulator (i, j) on lane l is
//   row = i*32 + 8*(r/4) + 4*(l/32) + (r%4),  col = j*32 + (l%32)
// within the wave's sub-tile.
//
// K is consumed in stages of 128 bytes per row (64 bf16 or 32 fp32): the two
// operand tiles of a stage are 256 rows x 128 B each, double-buffered in LDS
// (4 x 32 KiB). Rows are stored with the 16-byte chunk index XOR-swizzled by
// the row, so that both the coalesced stage writes and the MFMA fragment reads
// (16 consecutive rows, same chunk) touch distinct banks whether the LDS
// services 8 or 16 lanes of a 128-bit access per cycle.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vpce {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kTile = 256;          // BM = BN
constexpr int kRowBytes = 128;      // bytes of K per row per stage
constexpr int kStageBytes = kTile * kRowBytes;   // 32 KiB
constexpr int kGemmLds = 4 * kStageBytes;        // A,B x 2 stages = 128 KiB

// Elements of T per 16-byte chunk.
template <typename T> struct Chunk;
template <> struct Chunk<__bf16> { static constexpr int E = 8; };
template <> struct Chunk<float> { static constexpr int E = 4; };

__device__ __forceinline__ int swz(int row) {
  return (row & 7) ^ ((row >> 3) & 1);
}
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

// One "chunk pair" step of the wave's 4 x 4 accumulators: each lane supplies
// 16 bytes of A for each of its 4 row blocks and 16 bytes of B for each of
// its 4 column blocks.
//   bf16: one v_mfma_f32_32x32x16_bf16 per accumulator (lane half h carries
//         k = 8h..8h+7 of the chunk pair).
//   fp32: four v_mfma_f32_32x32x2_f32 per accumulator; instruction e pairs
//         element e of the two halves' chunks. Any pairing of k between A and
//         B that is the same on both operands gives the same sum. The e loop
//         is outermost so that dependent instructions are 16 apart.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void mma_block(f32x16_t (&acc)[4][4],
                                          const u32x4_t (&a)[4],
                                          const u32x4_t (&b)[4],
                                          const __bf16*) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, a[i]), __builtin_bit_cast(bf16x8_t, b[j]),
          acc[i][j], 0, 0, 0);
}
__device__ __forceinline__ void mma_block(f32x16_t (&acc)[4][4],
                                          const u32x4_t (&a)[4],
                                          const u32x4_t (&b)[4],
                                          const float*) {
  f32x4_t af[4], bf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    af[i] = __builtin_bit_cast(f32x4_t, a[i]);
    bf[i] = __builtin_bit_cast(f32x4_t, b[i]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][e], bf[j][e],
                                                         acc[i][j], 0, 0, 0);
}

// One accumulator row block (4 accumulators sharing the A fragment).
__device__ __forceinline__ void mma_row(f32x16_t (&acc)[4], u32x4_t a,
                                        const u32x4_t (&b)[4],
                                        const __bf16*) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b[j]),
        acc[j], 0, 0, 0);
}
__device__ __forceinline__ void mma_row(f32x16_t (&acc)[4], u32x4_t a,
                                        const u32x4_t (&b)[4], const float*) {
  const f32x4_t af = __builtin_bit_cast(f32x4_t, a);
  f32x4_t bf[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bf[j] = __builtin_bit_cast(f32x4_t, b[j]);
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[e], bf[j][e], acc[j],
                                                    0, 0, 0);
}

// A buffer resource over the valid rows of one operand tile: loads past its
// end return zero, which masks ragged row tails without branches.
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const T* base,
                                                            int64_t ld,
                                                            int rows) {
  const uint32_t bytes = (uint32_t)((int64_t)rows * ld * (int64_t)sizeof(T));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0,
                                           (int)bytes, 0x00020000);
}

// Global -> registers for one 256-row x 128-byte stage of an operand.
// Thread t loads chunks q = u*256 + t (u = 0..7): row q/8, chunk q%8, so each
// group of 8 threads reads one row's 128 contiguous bytes. Rows past the
// resource and chunks at or beyond K read as zero.
template <typename T>
__device__ __forceinline__ void stage_load(u32x4_t (&r)[8],
                                           __amdgpu_buffer_rsrc_t rs,
                                           int64_t ld, int64_t k0,
                                           int64_t K) {
  constexpr int E = Chunk<T>::E;
  const int t = threadIdx.x;
  const int row0 = t >> 3, c = t & 7;
  const int64_t k = k0 + c * E;
  const uint32_t rowb = (uint32_t)(ld * (int64_t)sizeof(T));
  const uint32_t off = k < K ? (uint32_t)row0 * rowb + (uint32_t)(k * (int64_t)sizeof(T))
                             : 0x80000000u;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    r[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + u * 32 * rowb), 0, 0);
}

__device__ __forceinline__ void stage_store(char* stage,
                                            const u32x4_t (&r)[8]) {
  const int t = threadIdx.x;
  const int row0 = t >> 3, c = t & 7;
  char* p = stage + lds_off(row0, c);
#pragma unroll
  for (int u = 0; u < 8; ++u)
    *reinterpret_cast<u32x4_t*>(p + u * 32 * kRowBytes) = r[u];
}

__device__ __forceinline__ u32x4_t frag(const char* stage, int row,
                                        int chunk) {
  return *reinterpret_cast<const u32x4_t*>(stage + lds_off(row, chunk));
}

// acc = A[0:256, 0:K] . B[0:256, 0:K]^T for the workgroup's tile.
// A, B point at the tile's first row; a_rows / b_rows are the valid rows
// (clamped by the caller to [0, 256]); 256 * ld * sizeof(T) must stay below
// 2^31 bytes (checked on the host). smem must hold kGemmLds bytes.
// Ends with a workgroup barrier, so smem may be rewritten right after.
template <typename T>
__device__ __forceinline__ void tile_mainloop(f32x16_t (&acc)[4][4],
                                              const T* __restrict__ A,
                                              int64_t lda, int a_rows,
                                              const T* __restrict__ B,
                                              int64_t ldb, int b_rows,
                                              int64_t K, char* smem) {
  constexpr int BK = 8 * Chunk<T>::E;  // elements of K per stage
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int p = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = (int)((K + BK - 1) / BK);
  if (KT <= 0) return;
  u32x4_t ra[8], rb[8];
  const __amdgpu_buffer_rsrc_t rsa = tile_rsrc<T>(A, lda, a_rows);
  const __amdgpu_buffer_rsrc_t rsb = tile_rsrc<T>(B, ldb, b_rows);
  stage_load<T>(ra, rsa, lda, 0, K);
  stage_load<T>(rb, rsb, ldb, 0, K);
  stage_store(smem, ra);
  stage_store(smem + 2 * kStageBytes, rb);
  __syncthreads();
  const T* tag = nullptr;
  // Software pipeline, per stage of 4 chunk-pair steps:
  //   step 0: issue the next stage's global loads; read step 1's fragments
  //   steps 1, 2: read the following step's fragments
  //   step 3: write the next stage into the other LDS buffer
  // each while the MFMAs of the current step run; then one barrier and the
  // next stage's step-0 fragments. Past the last stage the loads fall
  // outside the resource (zeros) and land in the idle buffer.
  u32x4_t fa[2][4], fb[2][4];
  const int arow = wm * 128 + p, brow = wn * 128 + p;
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[0][i] = frag(smem, arow + i * 32, h);
#pragma unroll
  for (int j = 0; j < 4; ++j) fb[0][j] = frag(smem + 2 * kStageBytes, brow + j * 32, h);
  constexpr int E = Chunk<T>::E;
  const int t = threadIdx.x;
  const uint32_t rowa = (uint32_t)(lda * (int64_t)sizeof(T));
  const uint32_t rowbb = (uint32_t)(ldb * (int64_t)sizeof(T));
  const uint32_t base_a = (uint32_t)(t >> 3) * rowa + (uint32_t)((t & 7) * E * sizeof(T));
  const uint32_t base_b = (uint32_t)(t >> 3) * rowbb + (uint32_t)((t & 7) * E * sizeof(T));
  const int st_off = lds_off(t >> 3, t & 7);
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const char* sa = smem + cur * kStageBytes;
    const char* sb = smem + (2 + cur) * kStageBytes;
    char* wa = smem + (cur ^ 1) * kStageBytes + st_off;
    char* wb = smem + (2 + (cur ^ 1)) * kStageBytes + st_off;
    // next stage's global offsets (past K: outside the resource -> zeros)
    const int64_t kn = (int64_t)(kt + 1) * BK + (t & 7) * E;
    const bool kin = kn < K;
    const uint32_t ga = kin ? base_a + (uint32_t)((kt + 1) * BK * sizeof(T)) : 0x80000000u;
    const uint32_t gb = kin ? base_b + (uint32_t)((kt + 1) * BK * sizeof(T)) : 0x80000000u;
    // The stage is issued as 16 groups of 4 MFMAs; sched_barrier keeps
    // each group's memory operations next to its MFMAs:
    //   steps 0-2, group q: read fragments A[q], B[q] of the next step
    //                       (+ in step 0 and 1: four global loads)
    //   step 3,    group q: write four chunks of the next stage to LDS
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (s < 3) {
          fa[(s + 1) & 1][q] = frag(sa, arow + q * 32, 2 * (s + 1) + h);
          fb[(s + 1) & 1][q] = frag(sb, brow + q * 32, 2 * (s + 1) + h);
        }
        if (s < 2) {
          const int g = s * 4 + q;  // 0..7: two A and two B chunks
          if (g < 4) {
            ra[2 * g] = __builtin_amdgcn_raw_buffer_load_b128(rsa, (int)(ga + (2 * g) * 32 * rowa), 0, 0);
            ra[2 * g + 1] = __builtin_amdgcn_raw_buffer_load_b128(rsa, (int)(ga + (2 * g + 1) * 32 * rowa), 0, 0);
          } else {
            const int gg = g - 4;
            rb[2 * gg] = __builtin_amdgcn_raw_buffer_load_b128(rsb, (int)(gb + (2 * gg) * 32 * rowbb), 0, 0);
            rb[2 * gg + 1] = __builtin_amdgcn_raw_buffer_load_b128(rsb, (int)(gb + (2 * gg + 1) * 32 * rowbb), 0, 0);
          }
        }
        if (s == 3) {
          *reinterpret_cast<u32x4_t*>(wa + (2 * q) * 32 * kRowBytes) = ra[2 * q];
          *reinterpret_cast<u32x4_t*>(wa + (2 * q + 1) * 32 * kRowBytes) = ra[2 * q + 1];
          *reinterpret_cast<u32x4_t*>(wb + (2 * q) * 32 * kRowBytes) = rb[2 * q];
          *reinterpret_cast<u32x4_t*>(wb + (2 * q + 1) * 32 * kRowBytes) = rb[2 * q + 1];
        }
        mma_row(acc[q], fa[s & 1][q], fb[s & 1], tag);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    const char* na = smem + (cur ^ 1) * kStageBytes;
    const char* nb = smem + (2 + (cur ^ 1)) * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[0][i] = frag(na, arow + i * 32, h);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[0][j] = frag(nb, brow + j * 32, h);
  }
  __syncthreads();
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
