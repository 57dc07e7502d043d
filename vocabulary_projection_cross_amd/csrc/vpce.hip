// vpce.hip -- kernels and C ABI of the blocked vocabulary-projection
// cross-entropy for gfx950 ("Flattening Every Memory Peak in Long-Context
// Mixture-of-Experts Training", section 3.2 "Ring-DTP", Figure 3).
//
// Forward: the R vocabulary shards are the rounds of the ring. A workgroup
// owns one 256-token tile, one shard and one contiguous split of that shard's
// 320-column vocabulary tiles. For each vocabulary tile it forms the logit
// tile with MFMA (never leaving registers), folds it into a per-token running
// (max, sum-exp) state with the online-softmax update, and picks up the target
// logit if the tile owns the label. At the end of the split the state is
// written as one partial per token. A merge kernel folds the partials of all
// shards in ring order, giving the per-token log-sum-exp, the per-token NLL and
// the mean loss (fp64 accumulation, fixed order).
//
// Backward: the shards are replayed in the same order, each in fixed-width
// chunks of C columns. Per chunk: recompute the logit tile, form
// G = dloss/n * (exp(z - lse) - onehot) in registers and store it (bf16 or
// fp32) token-major; then dW_chunk = G^T H and dH += G W_chunk, both on the
// same MFMA tile engine, which reads G, H and the W chunk as they are stored
// (the products take them as K-outer operands where their K runs down the
// rows). Device working set: partials R x S x N and one G chunk N x C --
// fixed by N, R, S and C, never by V.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "tile_core.hpp"
#include "vpce.h"

using namespace vpce;

// Device memory of vpce_forward_noalloc: its per-token partial states, target
// logits and block sums live here instead of in a caller's workspace. Every
// GPU the library runs on holds its own copy until the process ends. In host
// code this name is only a stand-in for the symbol; the device address comes
// from hipGetSymbolAddress (scratch_on_current_device).
static __device__ __align__(256) char scratch[VPCE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Backward chunk width C: at most 32 column tiles of the dW product. Measured
// on the workloads of 16384 to 131072 tokens, 8192 columns are as fast as
// 16384 (the 1M-context slice) or faster (2% on the stress workload, whose
// 21706-column shards then split 8192 + 8192 + 5322) at half the workspace;
// 4096 is 2% slower on the 1M-context slice (twice the fp32 read-modify-write
// passes of dH). A smaller workspace gets the widest multiple of kChunkStep
// that fits.
constexpr int kChunkCols = 8192;
constexpr int kChunkStep = 256;
constexpr int kMaxSplits = 16;
constexpr int64_t kMaxTokens = 2000000;
constexpr int64_t kMaxHidden = 1000000;  // 320 rows of d fp32 stay below 2^31 B
// 32-bit buffer offsets (tile_core.hpp). K-contiguous operand tiles (rows of
// H, W or G, at most 320 of them) have resources spanning under 2^31 bytes,
// and the rejected offset kOutOfRange plus a block offset of up to
// kMaxBlockOffsetRows rows stays below 2^32; their longest pitch is a row of
// H or W (d elements) at fp32, G rows being at most kChunkCols elements.
// K-outer operands (H, G and W read by the backward products) get one
// resource per stage, spanning its BK k-rows: 32 fp32 or 64 bf16 rows of at
// most d elements.
static_assert(kMaxHidden * 4 * kMaxBlockOffsetRows + (int64_t)kOutOfRange <
                  ((int64_t)1 << 32),
              "out-of-range offsets stay rejected");
static_assert(kMaxHidden * 4 * 320 < ((int64_t)1 << 31) &&
                  (int64_t)kChunkCols * 4 * 256 < ((int64_t)1 << 31) &&
                  kMaxHidden * 128 < ((int64_t)1 << 31),
              "operand tile and stage resources span under 2^31 bytes");
// Grouped raster (consecutive workgroups of an XCD share operand rows): how
// many token / output-row tiles sweep the column tiles together. Measured on
// the 1M-context slice: 2 suits the forward, 8 the dW product, 4 the dH
// product (2% ahead of 8 there), 4 the logit recompute.
constexpr int kGroupFwd = 2;
constexpr int kGroupDW = 8;  // the backward's dW product
constexpr int kGroupDH = 4;  // the backward's dH product
constexpr int kGroupRec = 4;  // the backward's logit recompute
constexpr int kLabIgnored = -2;   // label slot codes in LDS
constexpr int kLabInvalid = -1;
using TL = TileLayout;  // dW and dH products
using HL = HalfTileLayout;  // the products where 256 x 256 tiles are few
using FL = WideLayout;  // forward and logit recompute: 256 tokens x FL::TN
constexpr int kTile = 256;  // token tile of every kernel; product tile side
static_assert(FL::TM == kTile && TL::TM == kTile && TL::TN == kTile &&
                  HL::TN == kTile,
              "token tiles and product tiles are 256 rows");
static_assert(FL::WN == 2, "forward row merge pairs two waves per row");
constexpr int kFwdWaves = FL::kWaves / 4;  // waves per SIMD

struct Shards {
  int64_t V;
  int R;
  __host__ __device__ int64_t begin(int r) const {
    const int64_t base = V / R, extra = V % R;
    return r * base + (r < extra ? r : extra);
  }
  __host__ __device__ int64_t width(int r) const {
    const int64_t base = V / R, extra = V % R;
    return base + (r < extra ? 1 : 0);
  }
};

__device__ __forceinline__ int label_code(int64_t y, int64_t ignore_index,
                                          int64_t V) {
  if (y == ignore_index) return kLabIgnored;
  if (y < 0 || y >= V) return kLabInvalid;
  return (int)y;
}

__device__ __forceinline__ int clamp_rows(int64_t remaining, int cap) {
  return remaining <= 0 ? 0 : (remaining >= cap ? cap : (int)remaining);
}

// ---------------------------------------------------------------------------
// Forward tile kernel
// ---------------------------------------------------------------------------
struct FwdParams {
  const void* H;
  const void* W;        // rows of vocabulary entries v_base .. v_base + V - 1
  const int64_t* labels;
  int64_t N, d, V, ignore_index;
  int R, S, T;  // shards of W's rows, splits per shard, token tiles
  float* part_m;  // [R*S][N], base-2 running max
  float* part_s;  // [R*S][N], running sum of 2^(y - m)
  float* tgt;     // [N] target logit (natural units)
  int64_t v_base;  // vocabulary index of W's first row
  int64_t V_lab;   // labels outside [0, V_lab) (and not ignored) are invalid
};

// Row reduction of the forward epilogue. A lane holds 16 row values of a
// "unit" of accumulator row blocks (one 32-row block for MB = 32, four 16-row
// blocks for MB = 16); the lanes that share those rows (the MB lanes of a
// lane group) reduce-scatter them, after which lane l holds fully reduced
// value k(l) of the unit (MB = 32: k = (l % 32) / 2, lanes l and l ^ 1 alike;
// MB = 16: k = l % 16). Value k is element k % kAccRegs of row block
// k / kAccRegs of the unit.
constexpr int kUnitBlocks = FL::MB == 32 ? 1 : 16 / FL::kAccRegs;
constexpr int kUnits = FL::R / kUnitBlocks;  // units per wave
static_assert(kUnitBlocks * FL::kAccRegs == 16 && kUnits * kUnitBlocks == FL::R,
              "16 row values per unit");

template <typename T>
__global__ __launch_bounds__(FL::kThreads) __attribute__((amdgpu_waves_per_eu(kFwdWaves, kFwdWaves)))
void fwd_lse_kernel(FwdParams a) {
  __shared__ __attribute__((aligned(16))) char smem[RingOf<FL>::kBytes];
  __shared__ __attribute__((aligned(16))) int lab_s[kTile];
  __shared__ float xm[FL::WM][kUnits * 64], xs[FL::WM][kUnits * 64];
  constexpr int MB = FL::MB;

  const int total = a.T * a.R * a.S;
  const int idx = xcd_remap(blockIdx.x, total);
  int it, g;
  grouped_tile(idx, a.T, a.R * a.S, kGroupFwd, it, g);
  const int r = g / a.S, j = g % a.S;
  const Shards sh{a.V, a.R};
  const int64_t v0 = a.v_base + sh.begin(r), vw = sh.width(r);
  const int64_t vend = v0 + vw;
  const int Q = (int)((vw + FL::TN - 1) / FL::TN);
  const int q0 = (int)((int64_t)Q * j / a.S), q1 = (int)((int64_t)Q * (j + 1) / a.S);

  const int tid = threadIdx.x;
  const int64_t tok0 = (int64_t)it * kTile;
  if (tid < kTile) {
    const int64_t tok = tok0 + tid;
    lab_s[tid] = tok < a.N ? label_code(a.labels[tok], a.ignore_index, a.V_lab)
                           : kLabIgnored;
  }
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / FL::WN, wn = wave % FL::WN;
  const int p = lane % MB;

  const T* Hb = reinterpret_cast<const T*>(a.H) + tok0 * a.d;
  const int a_rows = clamp_rows(a.N - tok0, kTile);

  // running (max, sum) in base-2 units of this lane's reduced value k(lane)
  // of each unit
  float run_m[kUnits], run_s[kUnits];
#pragma unroll
  for (int u = 0; u < kUnits; ++u) { run_m[u] = -INFINITY; run_s[u] = 0.f; }
  typename FL::Acc acc[FL::R][FL::C];

  for (int q = q0; q < q1; ++q) {
    const int64_t col0 = v0 + (int64_t)q * FL::TN;
    const T* Wb = reinterpret_cast<const T*>(a.W) + (col0 - a.v_base) * a.d;
    tile_mainloop<T, FL>(acc, Hb, a.d, a_rows, Wb, a.d,
                         clamp_rows(vend - col0, FL::TN), a.d, smem);
    // columns of this lane: lc + MB*jj, jj = 0..C-1 (global vocabulary
    // index; V < 2^31)
    const int lc = (int)col0 + wn * FL::kWaveCols + FL::col(0, lane);
    const int vend32 = (int)vend;
    bool cv[FL::C];
#pragma unroll
    for (int jj = 0; jj < FL::C; ++jj) cv[jj] = lc + jj * MB < vend32;

#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      float ml[16], sl[16];
#pragma unroll
      for (int ib = 0; ib < kUnitBlocks; ++ib) {
        const int i = u * kUnitBlocks + ib;
#pragma unroll
        for (int rg = 0; rg < FL::kRowGroups; ++rg) {
          // 4 consecutive rows of this lane
          const int rowb = wm * FL::kWaveRows + FL::row_base(i, rg, lane);
          const int4 labs = *reinterpret_cast<const int4*>(&lab_s[rowb]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int rr = rg * 4 + e;              // element of acc[i][.]
            const int k = ib * FL::kAccRegs + rr;   // value of the unit
            float y[FL::C];
#pragma unroll
            for (int jj = 0; jj < FL::C; ++jj)
              y[jj] = cv[jj] ? acc[i][jj][rr] * kLog2e : -INFINITY;
            float m = y[0];
#pragma unroll
            for (int jj = 1; jj < FL::C; ++jj) m = fmaxf(m, y[jj]);
            float s = 0.f;
            if (cv[0]) {
#pragma unroll
              for (int jj = 0; jj < FL::C; ++jj) s += fast_exp2(y[jj] - m);
            }
            ml[k] = m;
            sl[k] = s;
            // target logit: the label's column is lc + MB*jj for some jj
            // (label codes of ignored or invalid tokens are negative)
            const int lab = e == 0 ? labs.x : e == 1 ? labs.y : e == 2 ? labs.z : labs.w;
            const int off = lab - lc;
            if (lab >= 0 && (unsigned)off < (unsigned)FL::kWaveCols &&
                (off % MB) == 0 && lab < vend32) {
              const int jsel = off / MB;
              float z = acc[i][0][rr];
#pragma unroll
              for (int jj = 1; jj < FL::C; ++jj)
                if (jsel == jj) z = acc[i][jj][rr];
              a.tgt[tok0 + rowb + e] = z;
            }
          }
        }
      }
      // reduce-scatter the 16 row values across the lanes that share them:
      // at each step a lane keeps the half of its values selected by one bit
      // of its lane index and merges in its partner's copy of that half (the
      // partner differs in that bit; MB = 32: XOR partner in the 32-lane
      // half, ds_swizzle; MB = 16: a DPP partner in the 16-lane row)
#define VPCE_RS_STEP(XCHG, MASK, HALF)                                  \
      {                                                                 \
        const bool upper = (p & (MASK)) != 0;                           \
        _Pragma("unroll") for (int k = 0; k < (HALF); ++k) {            \
          const float mk = upper ? ml[k + (HALF)] : ml[k];              \
          const float sk = upper ? sl[k + (HALF)] : sl[k];              \
          const float mo = XCHG<MASK>(upper ? ml[k] : ml[k + (HALF)]);  \
          const float so = XCHG<MASK>(upper ? sl[k] : sl[k + (HALF)]);  \
          float m = mk, s = sk;                                         \
          ms_merge(m, s, mo, so);                                       \
          ml[k] = m;                                                    \
          sl[k] = s;                                                    \
        }                                                               \
      }
      if constexpr (MB == 32) {
        VPCE_RS_STEP(half_xor, 16, 8)
        VPCE_RS_STEP(half_xor, 8, 4)
        VPCE_RS_STEP(half_xor, 4, 2)
        VPCE_RS_STEP(half_xor, 2, 1)
        const float mo = half_xor<1>(ml[0]);
        const float so = half_xor<1>(sl[0]);
        ms_merge(ml[0], sl[0], mo, so);
      } else {
        VPCE_RS_STEP(row_partner, 8, 8)
        VPCE_RS_STEP(row_partner, 4, 4)
        VPCE_RS_STEP(row_partner, 2, 2)
        VPCE_RS_STEP(row_partner, 1, 1)
      }
#undef VPCE_RS_STEP
      ms_merge(run_m[u], run_s[u], ml[0], sl[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // the two waves sharing rows (wn = 0, 1) combine through LDS
  if (wn == 1) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      xm[wm][u * 64 + lane] = run_m[u];
      xs[wm][u * 64 + lane] = run_s[u];
    }
  }
  __syncthreads();
  const int kred = MB == 32 ? (p >> 1) : p;  // reduced value of this lane
  if (wn == 0 && (MB == 16 || (p & 1) == 0)) {
    const int ib = kred / FL::kAccRegs, rr = kred % FL::kAccRegs;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      float m = run_m[u], s = run_s[u];
      ms_merge(m, s, xm[wm][u * 64 + lane], xs[wm][u * 64 + lane]);
      const int row = wm * FL::kWaveRows +
                      FL::row_base(u * kUnitBlocks + ib, rr / 4, lane) + rr % 4;
      const int64_t tok = tok0 + row;
      if (tok < a.N) {
        const int64_t o = (int64_t)(r * a.S + j) * a.N + tok;
        a.part_m[o] = m;
        a.part_s[o] = s;
      }
    }
  }
}

__global__ void fill_kernel(float* x, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = v;
}

// Fold the partials of every shard (ring order) and split; write lse and the
// per-block sums of the token losses (fp64) and valid counts.
__global__ __launch_bounds__(256) void merge_kernel(
    const float* part_m, const float* part_s, const float* tgt,
    const int64_t* labels, int64_t N, int G, int64_t ignore_index,
    float* lse, double* bsum, int* bcnt) {
  __shared__ double ssum[256];
  __shared__ int scnt[256];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  double nll = 0.0;
  int cnt = 0;
  if (i < N) {
    float m = -INFINITY, s = 0.f;
    for (int gg = 0; gg < G; ++gg)
      ms_merge(m, s, part_m[(int64_t)gg * N + i], part_s[(int64_t)gg * N + i]);
    const float l = (m + __builtin_amdgcn_logf(s)) * kLn2;
    lse[i] = l;
    if (labels[i] != ignore_index) {
      nll = (double)l - (double)tgt[i];
      cnt = 1;
    }
  }
  ssum[threadIdx.x] = nll;
  scnt[threadIdx.x] = cnt;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      ssum[threadIdx.x] += ssum[threadIdx.x + w];
      scnt[threadIdx.x] += scnt[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    bsum[blockIdx.x] = ssum[0];
    bcnt[blockIdx.x] = scnt[0];
  }
}

// Mean of the token losses from the per-block sums. With totals (fp64
// [sum of token losses, count]) the sums are added to it first and loss is
// the mean over everything accumulated there so far (loss may then be NULL).
__global__ __launch_bounds__(256) void loss_kernel(const double* bsum,
                                                   const int* bcnt, int nb,
                                                   float* loss,
                                                   double* totals) {
  __shared__ double ssum[256];
  __shared__ long long scnt[256];
  double s = 0.0;
  long long c = 0;
  for (int b = threadIdx.x; b < nb; b += 256) {
    s += bsum[b];
    c += bcnt[b];
  }
  ssum[threadIdx.x] = s;
  scnt[threadIdx.x] = c;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      ssum[threadIdx.x] += ssum[threadIdx.x + w];
      scnt[threadIdx.x] += scnt[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double sum = ssum[0], cnt = (double)scnt[0];
    if (totals) {
      sum += totals[0];
      cnt += totals[1];
      totals[0] = sum;
      totals[1] = cnt;
    }
    if (loss) loss[0] = cnt > 0.0 ? (float)(sum / cnt) : 0.f;
  }
}

// Fold the G split partials of one shard, in split order, into each token's
// running base-2 state (m, s).
__global__ __launch_bounds__(256) void fold_state_kernel(
    const float* part_m, const float* part_s, int64_t N, int G,
    float* state_m, float* state_s) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  float m = state_m[i], s = state_s[i];
  for (int g = 0; g < G; ++g)
    ms_merge(m, s, part_m[(int64_t)g * N + i], part_s[(int64_t)g * N + i]);
  state_m[i] = m;
  state_s[i] = s;
}

// ---------------------------------------------------------------------------
// Backward kernels
// ---------------------------------------------------------------------------

// scale = dloss / n_valid (0 when no token counts)
__global__ __launch_bounds__(1024) void scale_kernel(const int64_t* labels,
                                                     int64_t N,
                                                     int64_t ignore_index,
                                                     const float* dloss,
                                                     float* scale) {
  __shared__ long long sc[1024];
  long long c = 0;
  for (int64_t i = threadIdx.x; i < N; i += 1024) c += labels[i] != ignore_index;
  sc[threadIdx.x] = c;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) sc[threadIdx.x] += sc[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float up = dloss ? dloss[0] : 1.f;
    scale[0] = sc[0] > 0 ? (float)((double)up / (double)sc[0]) : 0.f;
  }
}

// scale = dloss / n, n the token count accumulated in totals[1]
__global__ void scale_from_totals_kernel(const double* totals,
                                         const float* dloss, float* scale) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const double n = totals[1];
    const float up = dloss ? dloss[0] : 1.f;
    scale[0] = n > 0.0 ? (float)((double)up / n) : 0.f;
  }
}

// The bf16 G tile leaves through LDS one wave column (L::kWaveCols chunk
// columns, the waves with one wn) at a time: each token row holds the
// L::kWaveCols columns, padded by 16 bytes so that the lanes writing 32
// different columns spread over the banks.
template <typename L>
struct RecStage {
  static constexpr int kGRowBytes = L::kWaveCols * 2 + 16;
  static constexpr int kGLds = kTile * kGRowBytes;
  static constexpr int kLds =
      RingOf<L>::kBytes > kGLds ? RingOf<L>::kBytes : kGLds;
  static_assert(L::kWaveCols % 8 == 0, "16-byte row chunks");
};
// The logit recompute runs on FL tiles (256 x 320), or on RL tiles
// (256 x 256) where those leave fewer compute units idle in the last wave.
using RL = Layout<256, 256, 4, 2>;

struct GParams {
  const void* H;
  const void* Wc;        // first row of the chunk in W
  const int64_t* labels;
  const float* lse;
  const float* scale;
  int64_t N, d, V, ignore_index;
  int64_t cv0;           // global vocabulary index of chunk column 0
  int64_t C_eff, C_pad;  // valid / padded chunk width
  int T, CT;             // token tiles, chunk column tiles
  void* G;               // [N][C_pad], token-major
};

// two floats as bf16 (round to nearest even), lo in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }

template <typename T, typename L>
__global__ __launch_bounds__(L::kThreads) __attribute__((amdgpu_waves_per_eu(L::kWaves / 4, L::kWaves / 4)))
void recompute_g_kernel(GParams a) {
  constexpr int kGRowBytes = RecStage<L>::kGRowBytes;
  // The operand ring, reused after the mainloop to stage the bf16 G tile.
  __shared__ __attribute__((aligned(16))) char smem[RecStage<L>::kLds];
  __shared__ __attribute__((aligned(16))) int lab_s[kTile];
  __shared__ __attribute__((aligned(16))) float lse_s[kTile];

  const int total = a.T * a.CT;
  const int idx = xcd_remap(blockIdx.x, total);
  int it, ct;
  grouped_tile(idx, a.T, a.CT, kGroupRec, it, ct);
  const int tid = threadIdx.x;
  const int64_t tok0 = (int64_t)it * kTile;
  const int64_t c0 = (int64_t)ct * L::TN;
  if (tid < kTile) {
    const int64_t tok = tok0 + tid;
    lab_s[tid] = tok < a.N ? label_code(a.labels[tok], a.ignore_index, a.V)
                           : kLabIgnored;
    lse_s[tid] = tok < a.N ? a.lse[tok] * kLog2e : 0.f;
  }
  typename L::Acc acc[L::R][L::C];
  tile_mainloop<T, L>(acc, reinterpret_cast<const T*>(a.H) + tok0 * a.d, a.d,
                       clamp_rows(a.N - tok0, kTile),
                       reinterpret_cast<const T*>(a.Wc) + c0 * a.d, a.d,
                       clamp_rows(a.C_eff - c0, L::TN), a.d, smem);
  const float scale = a.scale[0];
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / L::WN, wn = wave % L::WN;
  T* G = reinterpret_cast<T*>(a.G);
  // G packed to bf16 pairs (rows 2k, 2k + 1 of row group rq of accumulator
  // (i, jj) in gpk[i][jj][2rq + k]), or stored at once (fp32). Chunk columns
  // of this lane: ccol[jj] = c0 + wn * kWaveCols + col(jj) (< 2^31).
  uint32_t gpk[L::R][L::C][L::kAccRegs / 2];
  int ccol[L::C];
#pragma unroll
  for (int jj = 0; jj < L::C; ++jj)
    ccol[jj] = (int)c0 + wn * L::kWaveCols + L::col(jj, lane);
#pragma unroll
  for (int i = 0; i < L::R; ++i) {
#pragma unroll
    for (int rq = 0; rq < L::kRowGroups; ++rq) {
      const int rowb = wm * L::kWaveRows + L::row_base(i, rq, lane);
      const int4 labs = *reinterpret_cast<const int4*>(&lab_s[rowb]);
      const float4 l2 = *reinterpret_cast<const float4*>(&lse_s[rowb]);
#pragma unroll
      for (int jj = 0; jj < L::C; ++jj) {
        const int c = ccol[jj];
        const bool cvalid = c < a.C_eff;
        const int v = (int)a.cv0 + c;
        float gv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int lab = e == 0 ? labs.x : e == 1 ? labs.y : e == 2 ? labs.z : labs.w;
          const float ls = e == 0 ? l2.x : e == 1 ? l2.y : e == 2 ? l2.z : l2.w;
          const float z = acc[i][jj][rq * 4 + e];
          // computed everywhere and selected (no per-element branch); a
          // discarded value may be NaN, the selected one never is
          const float pr = fast_exp2(fmaf(z, kLog2e, -ls));
          const float gg = (cvalid && lab != kLabIgnored)
                               ? scale * (pr - (lab == v ? 1.f : 0.f))
                               : 0.f;
          gv[e] = gg;
          if constexpr (sizeof(T) != 2) {
            const int64_t tok = tok0 + rowb + e;
            if (c < a.C_pad && tok < a.N) store_elem(G + tok * a.C_pad + c, gg);
          }
        }
        if constexpr (sizeof(T) == 2) {
          gpk[i][jj][2 * rq] = pack_bf16x2(gv[0], gv[1]);
          gpk[i][jj][2 * rq + 1] = pack_bf16x2(gv[2], gv[3]);
          // opaque from here on: the compiler would otherwise keep every
          // unpacked bf16 value alive for the row-major stores and spill
          asm volatile("" : "+v"(gpk[i][jj][2 * rq]), "+v"(gpk[i][jj][2 * rq + 1]));
        }
      }
    }
  }
  if constexpr (sizeof(T) == 2) {
    // The barriers order the LDS staging only; the G stores stay in flight
    // across them and past the end of the workgroup.
    constexpr int kRowChunks = L::kWaveCols * 2 / 16;  // per G row (one pass)
#pragma unroll 1
    for (int pass = 0; pass < L::WN; ++pass) {
      const int64_t cp0 = c0 + pass * L::kWaveCols;  // first column of the pass
      // G rows: the waves of this column write their columns row-major, then
      // every lane stores 16-byte chunks of the rows, coalesced.
      if (wn == pass) {
#pragma unroll
        for (int jj = 0; jj < L::C; ++jj) {
          const int cl = L::col(jj, lane);
#pragma unroll
          for (int i = 0; i < L::R; ++i)
#pragma unroll
            for (int rr = 0; rr < L::kAccRegs; ++rr) {
              const int row = wm * L::kWaveRows +
                              L::row_base(i, rr >> 2, lane) + (rr & 3);
              *reinterpret_cast<uint16_t*>(smem + row * kGRowBytes + cl * 2) =
                  (uint16_t)(gpk[i][jj][rr >> 1] >> (16 * (rr & 1)));
            }
        }
      }
      lds_barrier();
#pragma unroll 4
      for (int id = tid; id < kTile * kRowChunks; id += L::kThreads) {
        const int row = id / kRowChunks, u = id % kRowChunks;
        const int64_t tok = tok0 + row;
        const int64_t cc = cp0 + 8 * u;
        if (tok < a.N && cc < a.C_pad) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
              smem + row * kGRowBytes + u * 16);
          // non-temporal: the chunk (1 GB on the 65536-token batch) is
          // re-read only by the next launch, and keeping it out of the
          // caches measured 0.4-0.9% faster per step than plain stores
          __builtin_nontemporal_store(
              v, reinterpret_cast<u32x4_t*>(G + tok * a.C_pad + cc));
        }
      }
      lds_barrier();
    }
  }
}

// Output staging of the products: a band of one row of waves' tile rows in
// fp32, rows padded by 16 bytes (the lanes of one accumulator write hit 64
// distinct banks).
template <typename L>
struct ProdStage {
  static constexpr int kBandRows = L::kWaveRows;
  static constexpr int kPitch = L::TN * 4 + 16;
  static_assert(kBandRows * kPitch <= RingOf<L>::kBytes,
                "a band fits the operand ring");
};

// out[M x Nc] (row stride ldo) = A . B^T over K, stored or accumulated (fp32).
// A K-contiguous operand is [M x K] (or [Nc x K]) with row pitch lda (ldb);
// a K-outer one is [K x M] (or [K x Nc]): its row k holds the M (Nc) entries
// at row pitch lda (ldb), and only its first a_krows (b_krows) rows are read.
struct ProdParams {
  const void* A;
  int64_t lda;
  int64_t M;
  const void* B;
  int64_t ldb;
  int64_t Nc;
  int64_t K;
  float* out;
  int64_t ldo;
  int TM, TN;
  int accumulate;
  int group;  // grouped raster: output-row tiles per group
  int a_krows, b_krows;  // valid k-rows of K-outer operands
};

// One output tile of a product: tile idx (row-major in the grouped raster of
// a.group output-row tiles) of out (+)= A . B^T. smem holds
// RingOf<PL, T, TA, TB>::kBytes.
template <typename T, typename PL, bool TA, bool TB>
__device__ __forceinline__ void prod_tile(const ProdParams& a, int idx,
                                          char* smem) {
  constexpr int kProdBandRows = ProdStage<PL>::kBandRows;
  constexpr int kProdPitch = ProdStage<PL>::kPitch;
  int tm, tn;
  grouped_tile(idx, a.TM, a.TN, a.group, tm, tn);
  const int64_t m0 = (int64_t)tm * PL::TM, n0 = (int64_t)tn * PL::TN;
  typename PL::Acc acc[PL::R][PL::C];
  const T* Ab = reinterpret_cast<const T*>(a.A);
  const T* Bb = reinterpret_cast<const T*>(a.B);
  tile_mainloop<T, PL, TA, TB>(
      acc, TA ? Ab : Ab + m0 * a.lda, a.lda,
      TA ? a.a_krows : clamp_rows(a.M - m0, PL::TM), TB ? Bb : Bb + n0 * a.ldb,
      a.ldb, TB ? a.b_krows : clamp_rows(a.Nc - n0, PL::TN), a.K, smem,
      (int)m0, (int)n0);
  // The tile leaves through LDS one band of 64 rows (one row of waves) at a
  // time: those waves write their accumulators into the band, then every
  // thread moves 16-byte pieces of whole rows (1 KiB per wave instruction),
  // reading all its old values (accumulate) before its first store.
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / PL::WN, wn = wave % PL::WN;
  constexpr int kRowF4 = PL::TN / 4;                     // float4 per tile row
  static_assert(kRowF4 == 64, "one tile row per wave instruction");
  constexpr int kPerThread = kProdBandRows * kRowF4 / PL::kThreads;
  static_assert(kPerThread * PL::kThreads == kProdBandRows * kRowF4,
                "whole float4 pieces per thread");
#pragma unroll 1
  for (int band = 0; band < PL::WM; ++band) {
    if (wm == band) {
#pragma unroll
      for (int i = 0; i < PL::R; ++i)
#pragma unroll
        for (int jj = 0; jj < PL::C; ++jj) {
          const int col = wn * PL::kWaveCols + PL::col(jj, lane);
#pragma unroll
          for (int rr = 0; rr < PL::kAccRegs; ++rr) {
            const int row = PL::row_base(i, rr >> 2, lane) + (rr & 3);
            *reinterpret_cast<float*>(smem + row * kProdPitch + col * 4) =
                acc[i][jj][rr];
          }
        }
    }
    lds_barrier();
    f32x4_t v[kPerThread];
    bool ok[kPerThread];
    int64_t at[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int id = tid + k * PL::kThreads;
      // lanes 32..63 take the row's 16-byte pieces with 128-byte halves
      // swapped, so lanes l and l + 32 (served in one LDS cycle) read
      // different banks; the wave still covers one whole row
      const int row = id / kRowF4, c4 = (id % kRowF4) ^ (((id >> 5) & 1) << 3);
      const int64_t grow = m0 + band * kProdBandRows + row;
      const int64_t gcol = n0 + c4 * 4;
      // Nc is a multiple of 4, so a piece is wholly inside or outside
      ok[k] = grow < a.M && gcol < a.Nc;
      at[k] = grow * a.ldo + gcol;
      v[k] = *reinterpret_cast<const f32x4_t*>(smem + row * kProdPitch + c4 * 16);
    }
    if (a.accumulate) {
      f32x4_t old[kPerThread];
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        old[k] = ok[k] ? __builtin_nontemporal_load(
                             reinterpret_cast<const f32x4_t*>(a.out + at[k]))
                       : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) v[k] += old[k];
    }
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
      if (ok[k])
        __builtin_nontemporal_store(v[k], reinterpret_cast<f32x4_t*>(a.out + at[k]));
    lds_barrier();
  }
}


// The dW and dH products of one backward chunk in one launch: the workgroups
// of each XCD (workgroup L runs on XCD L mod 8) take that XCD's share of the
// dW tiles first and then its share of the dH tiles, each share a contiguous
// range of its product's grouped raster. dW tiles (K = the batch's tokens)
// are long; dH tiles (K = the chunk's columns) fill the compute units around
// them, so a dW grid that is not a whole number of waves leaves no units
// idle. dW: A = G and B = H, both K-outer; dH: A = G K-contiguous, B = the W
// chunk K-outer, on DHL tiles.
struct PairParams {
  ProdParams dw, dh;
  int n_dw, n_dh;  // tiles of each product
};

template <typename T, typename DHL>
__global__ __launch_bounds__(TL::kThreads) __attribute__((amdgpu_waves_per_eu(TL::kWaves / 4, TL::kWaves / 4)))
void prod_pair_kernel(PairParams a) {
  static_assert(DHL::kThreads == TL::kThreads, "one block size");
  constexpr int kDw = RingOf<TL, T, true, true>::kBytes;
  constexpr int kDh = RingOf<DHL, T, false, true>::kBytes;
  __shared__ __attribute__((aligned(16))) char smem[kDw > kDh ? kDw : kDh];
  const int total = a.n_dw + a.n_dh;
  const int L = blockIdx.x, x = L & 7, k = L >> 3;
  const int q = total >> 3, r = total & 7;
  const int qw = a.n_dw >> 3, rw = a.n_dw & 7;
  const int n_dw_x = qw + (x < rw ? 1 : 0);         // dW tiles of XCD x
  const int dw0 = x * qw + (x < rw ? x : rw);       // its first dW tile
  const int before = x * q + (x < r ? x : r);       // workgroups of XCDs < x
  if (k < n_dw_x)
    prod_tile<T, TL, true, true>(a.dw, dw0 + k, smem);
  else
    prod_tile<T, DHL, false, true>(a.dh, (before - dw0) + (k - n_dw_x), smem);
}

// ---------------------------------------------------------------------------
// Host side: validation, plan, launches
// ---------------------------------------------------------------------------

constexpr size_t kAlign = 256;
inline size_t up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

struct Plan {
  int64_t N, d, V;
  int R, dt, esz;
  int T, S, nb;
  int64_t C;
  // forward layout
  size_t o_pm, o_ps, o_tgt, o_bsum, o_bcnt, fwd_bytes;
  // backward layout
  size_t o_scale, o_G, bwd_bytes;
  size_t bytes;
};

// The most vocabulary splits per shard a forward may use: enough workgroups
// to cover 256 compute units twice, at most kMaxSplits. It sizes the
// per-token partial states in the workspace, so it never depends on V.
int splits_for(int64_t T, int R) {
  const int64_t want = 512;
  int64_t s = (want + T * R - 1) / (T * R);
  if (s < 1) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  return (int)s;
}

// The splits a forward runs with, at most s_cap: the fewest whose makespan --
// waves of T x R x S workgroups (one per compute unit) times the most
// vocabulary tiles one split of the widest shard holds -- is the smallest.
int run_splits(int64_t T, int R, int s_cap, int64_t widest, int cus) {
  const int64_t units = cus > 0 ? cus : 256;
  const int64_t Q = (widest + FL::TN - 1) / FL::TN;
  int best = 1;
  int64_t best_span = -1;
  for (int s = 1; s <= s_cap; ++s) {
    const int64_t waves = (T * R * s + units - 1) / units;
    const int64_t span = waves * ((Q + s - 1) / s);
    if (best_span < 0 || span < best_span) {
      best_span = span;
      best = s;
    }
  }
  return best;
}

int32_t check_shape(int64_t N, int64_t d, int64_t V, int32_t R, int32_t dt) {
  if (dt != VPCE_BF16 && dt != VPCE_F32) return VPCE_ERR_UNSUPPORTED;
  if (N < 0 || d < 1 || V < 1 || R < 1 || (int64_t)R > V) return VPCE_ERR_SHAPE;
  // 32-bit buffer offsets stay in range (see the static checks above)
  if (V >= ((int64_t)1 << 31) || N > kMaxTokens || d > kMaxHidden)
    return VPCE_ERR_SHAPE;
  if (d % (dt == VPCE_BF16 ? 8 : 4) != 0) return VPCE_ERR_SHAPE;
  // tile indices are int: keep the grids in range
  if ((N + kTile - 1) / kTile * (int64_t)R * kMaxSplits >= ((int64_t)1 << 31))
    return VPCE_ERR_SHAPE;
  return VPCE_OK;
}

Plan make_plan(int64_t N, int64_t d, int64_t V, int R, int dt,
               int64_t C = kChunkCols) {
  Plan p{};
  p.N = N; p.d = d; p.V = V; p.R = R; p.dt = dt;
  p.esz = dt == VPCE_BF16 ? 2 : 4;
  p.T = (int)((N + kTile - 1) / kTile);
  p.S = splits_for(p.T > 0 ? p.T : 1, R);
  p.nb = (int)((N + 255) / 256);
  p.C = C;
  size_t o = 0;
  const size_t part = (size_t)R * p.S * (size_t)N * 4;
  p.o_pm = o; o = up(o + part);
  p.o_ps = o; o = up(o + part);
  p.o_tgt = o; o = up(o + (size_t)N * 4);
  p.o_bsum = o; o = up(o + (size_t)(p.nb > 0 ? p.nb : 1) * 8);
  p.o_bcnt = o; o = up(o + (size_t)(p.nb > 0 ? p.nb : 1) * 4);
  p.fwd_bytes = o;
  o = 0;
  p.o_scale = o; o = up(o + 16);
  p.o_G = o; o = up(o + (size_t)N * p.C * p.esz);
  p.bwd_bytes = o;
  p.bytes = p.fwd_bytes > p.bwd_bytes ? p.fwd_bytes : p.bwd_bytes;
  return p;
}

bool valid_chunk(int64_t C) {
  return C >= kChunkStep && C <= kChunkCols && C % kChunkStep == 0;
}

// The widest backward chunk whose workspace fits in `bytes` (0 if even the
// narrowest does not): the backward's own part, or (shared) the buffer that
// serves the forward and the backward. Both grow with C, so the first width
// that fits, scanning down, is the widest.
int64_t widest_chunk(int64_t N, int64_t d, int64_t V, int R, int dt,
                     size_t bytes, bool shared) {
  for (int64_t C = kChunkCols; C >= kChunkStep; C -= kChunkStep) {
    const Plan p = make_plan(N, d, V, R, dt, C);
    if ((shared ? p.bytes : p.bwd_bytes) <= bytes) return C;
  }
  return 0;
}

// Device bytes of the caller's own buffers around one forward + backward:
// inputs H, W, labels; outputs lse, loss, dH, dW.
size_t caller_bytes(int64_t N, int64_t d, int64_t V, int dt) {
  const size_t esz = dt == VPCE_BF16 ? 2 : 4;
  return (size_t)N * d * esz + (size_t)V * d * esz + (size_t)N * 8 +
         (size_t)N * 4 + 4 + (size_t)N * d * 4 + (size_t)V * d * 4;
}

inline bool aligned(const void* p, size_t a) {
  return ((uintptr_t)p % a) == 0;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept for the life of the process.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int32_t scratch_on_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return VPCE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess ||
        ptr == nullptr)
      return VPCE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = reinterpret_cast<char*>(g_scratch_ptr[dev]);
  return VPCE_OK;
}

#define VPCE_LAUNCH_CHECK()                              \
  do {                                                   \
    if (hipGetLastError() != hipSuccess) return VPCE_ERR_HIP; \
  } while (0)

// Optional timing of the launches of one call (the *_traced entry points):
// event pair i brackets the i-th kernel launch on the call's stream, and
// kinds[i] says which kernel it was. Launches past `cap` are counted only.
struct Trace {
  const hipEvent_t* ev;  // 2 * cap events
  int32_t* kinds;        // cap entries
  int cap;
  int n;
};

inline int32_t trace_begin(Trace* t, hipStream_t st) {
  if (t && t->n < t->cap && hipEventRecord(t->ev[2 * t->n], st) != hipSuccess)
    return VPCE_ERR_HIP;
  return VPCE_OK;
}

inline int32_t trace_end(Trace* t, int32_t kind, hipStream_t st) {
  if (!t) return VPCE_OK;
  if (t->n < t->cap) {
    if (hipEventRecord(t->ev[2 * t->n + 1], st) != hipSuccess)
      return VPCE_ERR_HIP;
    t->kinds[t->n] = kind;
  }
  ++t->n;
  return VPCE_OK;
}

// Launch a kernel, check the launch, and bracket it for the trace (if any).
#define VPCE_LAUNCH(KIND, KERNEL, GRID, BLOCK, ...)                       \
  do {                                                                   \
    if (trace_begin(tr, st) != VPCE_OK) return VPCE_ERR_HIP;             \
    hipLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, st, __VA_ARGS__);         \
    if (hipGetLastError() != hipSuccess) return VPCE_ERR_HIP;            \
    if (trace_end(tr, KIND, st) != VPCE_OK) return VPCE_ERR_HIP;         \
  } while (0)

// Compute units of the current device (0 if the runtime cannot say).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                            dev) != hipSuccess)
    return 0;
  return cus;
}

template <typename T>
int32_t run_forward(const Plan& p, const void* H, const void* W,
                    const int64_t* labels, int64_t ignore_index, float* loss,
                    float* lse, char* ws, hipStream_t st,
                    Trace* tr = nullptr) {
  float* pm = reinterpret_cast<float*>(ws + p.o_pm);
  float* ps = reinterpret_cast<float*>(ws + p.o_ps);
  float* tgt = reinterpret_cast<float*>(ws + p.o_tgt);
  double* bsum = reinterpret_cast<double*>(ws + p.o_bsum);
  int* bcnt = reinterpret_cast<int*>(ws + p.o_bcnt);
  if (p.N > 0) {
    VPCE_LAUNCH(VPCE_KERNEL_OTHER, fill_kernel,
                dim3((unsigned)((p.N + 255) / 256)), dim3(256), tgt, p.N, NAN);
    const int S = run_splits(p.T, p.R, p.S, Shards{p.V, p.R}.width(0),
                             device_cus());
    FwdParams fp{H, W, labels, p.N, p.d, p.V, ignore_index, p.R, S, p.T,
                 pm, ps, tgt, 0, p.V};
    const unsigned grid = (unsigned)((int64_t)p.T * p.R * S);
    VPCE_LAUNCH(VPCE_KERNEL_FORWARD_TILE, fwd_lse_kernel<T>, dim3(grid),
                dim3(FL::kThreads), fp);
    VPCE_LAUNCH(VPCE_KERNEL_MERGE, merge_kernel, dim3((unsigned)p.nb),
                dim3(256), pm, ps, tgt, labels, p.N, p.R * S, ignore_index,
                lse, bsum, bcnt);
  }
  VPCE_LAUNCH(VPCE_KERNEL_OTHER, loss_kernel, dim3(1), dim3(256), bsum, bcnt,
              p.nb, loss, static_cast<double*>(nullptr));
  return VPCE_OK;
}


// dW rows = G^T H and dH (+)= G W_chunk of one chunk in one launch (see
// prod_pair_kernel). dH runs on 256 x 256 tiles, or on 128 x 256 tiles where
// the former would give fewer tiles than the device has compute units. Sets
// TM in both parameter sets.
template <typename T>
int32_t launch_products(ProdParams dw, ProdParams dh, bool with_dh, int cus,
                        hipStream_t st, Trace* tr) {
  dw.TM = (int)((dw.M + TL::TM - 1) / TL::TM);
  PairParams pp{dw, dh, dw.TM * dw.TN, 0};
  const int64_t dh_tiles = (dh.M + TL::TM - 1) / TL::TM * dh.TN;
  const bool half = with_dh && cus > 0 && dh_tiles < cus;
  if (with_dh) {
    pp.dh.TM = (int)(half ? (dh.M + HL::TM - 1) / HL::TM
                          : (dh.M + TL::TM - 1) / TL::TM);
    pp.n_dh = pp.dh.TM * pp.dh.TN;
  }
  const dim3 grid((unsigned)(pp.n_dw + pp.n_dh));
  if (half)
    VPCE_LAUNCH(VPCE_KERNEL_PRODUCTS, (prod_pair_kernel<T, HL>), grid,
                dim3(TL::kThreads), pp);
  else
    VPCE_LAUNCH(VPCE_KERNEL_PRODUCTS, (prod_pair_kernel<T, TL>), grid,
                dim3(TL::kThreads), pp);
  return VPCE_OK;
}

// Backward over the vocabulary entries [v_first, v_first + v_count), whose
// rows of W start at Wspan and whose rows of dW start at dWspan, in chunks of
// p.C columns: recompute G for the chunk (token-major, [N x C_pad]), then
// dW rows = G^T H and dH += G W_chunk. G, H and W are all read as they are
// stored: the dW product takes G and H as K-outer operands (K = tokens), the
// dH product G as a K-contiguous one and the W chunk as a K-outer one
// (K = vocabulary entries). The first chunk overwrites dH unless dH_acc; dW
// rows are overwritten unless dW_acc. *scale must be on the device.
template <typename T>
int32_t backward_span(const Plan& p, const void* H, const void* Wspan,
                      int64_t v_first, int64_t v_count, int64_t V_lab,
                      const int64_t* labels, const float* lse,
                      const float* scale, int64_t ignore_index, float* dH,
                      bool dH_acc, float* dWspan, bool dW_acc, char* ws,
                      hipStream_t st, Trace* tr) {
  void* G = ws + p.o_G;
  const int TD = (int)((p.d + kTile - 1) / kTile);
  bool acc_h = dH_acc;
  const int cus = device_cus();
  for (int64_t c0 = 0; c0 < v_count; c0 += p.C) {
    const int64_t ceff = (v_count - c0) < p.C ? (v_count - c0) : p.C;
    const int64_t cpad = (ceff + 63) / 64 * 64;
    const int64_t cv0 = v_first + c0;
    const T* Wc = reinterpret_cast<const T*>(Wspan) + c0 * p.d;
    if (p.N > 0) {
      // 256 x 256 recompute tiles where their last wave leaves clearly fewer
      // compute units idle: the makespan in column-units (waves of one
      // workgroup per unit, times the tile width) at least 10% below that
      // of 256 x 320 tiles, which move fewer operand bytes per flop
      const int64_t units = cus > 0 ? cus : 256;
      const int64_t ct_w = (cpad + FL::TN - 1) / FL::TN;
      const int64_t ct_n = (cpad + RL::TN - 1) / RL::TN;
      const int64_t span_w = (p.T * ct_w + units - 1) / units * FL::TN;
      const int64_t span_n = (p.T * ct_n + units - 1) / units * RL::TN;
      const bool narrow = 10 * span_n < 9 * span_w;
      const int CT = (int)(narrow ? ct_n : ct_w);
      GParams gp{H, Wc, labels, lse, scale, p.N, p.d, V_lab,
                 ignore_index, cv0, ceff, cpad, p.T, CT, G};
      if (narrow)
        VPCE_LAUNCH(VPCE_KERNEL_RECOMPUTE, (recompute_g_kernel<T, RL>),
                    dim3((unsigned)(p.T * CT)), dim3(RL::kThreads), gp);
      else
        VPCE_LAUNCH(VPCE_KERNEL_RECOMPUTE, (recompute_g_kernel<T, FL>),
                    dim3((unsigned)(p.T * CT)), dim3(FL::kThreads), gp);
    }
    // dW rows of the chunk = G^T H: A = G (K-outer: row k = token, C_pad
    // entries), B = H (K-outer: row k = token, d entries), K = N; and
    // dH (+)= G W_chunk: A = G [N x C_pad] (K-contiguous), B = W chunk
    // (K-outer: row k = vocabulary entry, d entries; rows past ceff read 0)
    const ProdParams pw{G, cpad, ceff, H, p.d, p.d, p.N,
                        dWspan + c0 * p.d, p.d, 0, TD, dW_acc ? 1 : 0,
                        kGroupDW, (int)p.N, (int)p.N};
    const ProdParams ph{G, cpad, p.N, Wc, p.d, p.d, cpad, dH, p.d, 0, TD,
                        acc_h ? 1 : 0, kGroupDH, 0, (int)ceff};
    const int32_t rc = launch_products<T>(pw, ph, p.N > 0, cus, st, tr);
    if (rc != VPCE_OK) return rc;
    acc_h = true;
  }
  return VPCE_OK;
}

template <typename T>
int32_t run_backward(const Plan& p, const void* H, const void* W,
                     const int64_t* labels, const float* lse,
                     const float* dloss, int64_t ignore_index, float* dH,
                     float* dW, char* ws, hipStream_t st,
                     Trace* tr = nullptr) {
  float* scale = reinterpret_cast<float*>(ws + p.o_scale);
  VPCE_LAUNCH(VPCE_KERNEL_OTHER, scale_kernel, dim3(1), dim3(1024), labels,
              p.N, ignore_index, dloss, scale);
  const Shards sh{p.V, p.R};
  for (int r = 0; r < p.R; ++r) {
    const int64_t v0 = sh.begin(r), vw = sh.width(r);
    const int32_t rc = backward_span<T>(
        p, H, reinterpret_cast<const T*>(W) + v0 * p.d, v0, vw, p.V, labels,
        lse, scale, ignore_index, dH, r > 0, dW + v0 * p.d, false, ws, st, tr);
    if (rc != VPCE_OK) return rc;
  }
  return VPCE_OK;
}

// One batch meets one vocabulary shard: fold the shard's logits into the
// batch's running state [m | s | t] (3 x N floats).
template <typename T>
int32_t run_shard_fold(const Plan& p, const void* H, const void* Wshard,
                       int64_t v_begin, int64_t V_lab, const int64_t* labels,
                       int64_t ignore_index, float* state, char* ws,
                       hipStream_t st) {
  if (p.N == 0) return VPCE_OK;
  float* pm = reinterpret_cast<float*>(ws + p.o_pm);
  float* ps = reinterpret_cast<float*>(ws + p.o_ps);
  const int S = run_splits(p.T, 1, p.S, p.V, device_cus());
  FwdParams fp{H, Wshard, labels, p.N, p.d, p.V, ignore_index, 1, S, p.T,
               pm, ps, state + 2 * p.N, v_begin, V_lab};
  hipLaunchKernelGGL(fwd_lse_kernel<T>, dim3((unsigned)((int64_t)p.T * S)),
                     dim3(FL::kThreads), 0, st, fp);
  VPCE_LAUNCH_CHECK();
  hipLaunchKernelGGL(fold_state_kernel, dim3((unsigned)((p.N + 255) / 256)),
                     dim3(256), 0, st, pm, ps, p.N, S, state, state + p.N);
  VPCE_LAUNCH_CHECK();
  return VPCE_OK;
}
}  // namespace

extern "C" {

size_t vpce_workspace_bytes(int64_t N, int64_t d, int64_t V, int32_t R,
                            int32_t dtype) {
  if (check_shape(N, d, V, R, dtype) != VPCE_OK) return 0;
  return make_plan(N, d, V, R, dtype).bytes;
}

size_t vpce_workspace_bytes_chunk(int64_t N, int64_t d, int64_t V, int32_t R,
                                  int32_t dtype, int64_t chunk_cols) {
  if (check_shape(N, d, V, R, dtype) != VPCE_OK || !valid_chunk(chunk_cols))
    return 0;
  return make_plan(N, d, V, R, dtype, chunk_cols).bytes;
}

int32_t vpce_plan(int64_t N, int64_t d, int64_t V, int32_t R, int32_t dtype,
                  size_t budget_bytes, int64_t* chunk_cols,
                  size_t* workspace_bytes, size_t* peak_bytes) {
  const int32_t s = check_shape(N, d, V, R, dtype);
  if (s != VPCE_OK) return s;
  if (!chunk_cols || !workspace_bytes || !peak_bytes) return VPCE_ERR_NULL;
  const size_t fixed = caller_bytes(N, d, V, dtype);
  const int64_t C =
      budget_bytes > fixed
          ? widest_chunk(N, d, V, R, dtype, budget_bytes - fixed, true)
          : 0;
  if (C == 0) return VPCE_ERR_WORKSPACE;
  const size_t ws = make_plan(N, d, V, R, dtype, C).bytes;
  *chunk_cols = C;
  *workspace_bytes = ws;
  *peak_bytes = fixed + ws;
  return VPCE_OK;
}

namespace {
int32_t forward_entry(const void* H, const void* W, const int64_t* labels,
                      int64_t N, int64_t d, int64_t V, int32_t R,
                      int64_t ignore_index, int32_t dtype, float* loss,
                      float* lse, void* workspace, size_t workspace_bytes,
                      void* stream, Trace* tr) {
  const int32_t s = check_shape(N, d, V, R, dtype);
  if (s != VPCE_OK) return s;
  if (!W || !loss || !workspace) return VPCE_ERR_NULL;
  if (N > 0 && (!H || !labels || !lse)) return VPCE_ERR_NULL;
  if ((H && !aligned(H, 16)) || !aligned(W, 16) || (labels && !aligned(labels, 8)) ||
      !aligned(loss, 4) || (lse && !aligned(lse, 4)) || !aligned(workspace, kAlign))
    return VPCE_ERR_ALIGN;
  const Plan p = make_plan(N, d, V, R, dtype);
  if (workspace_bytes < p.fwd_bytes) return VPCE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == VPCE_BF16)
    return run_forward<__bf16>(p, H, W, labels, ignore_index, loss, lse, ws, st, tr);
  return run_forward<float>(p, H, W, labels, ignore_index, loss, lse, ws, st, tr);
}

int32_t backward_entry(const void* H, const void* W, const int64_t* labels,
                       const float* lse, const float* dloss, int64_t N,
                       int64_t d, int64_t V, int32_t R, int64_t ignore_index,
                       int32_t dtype, float* dH, float* dW, void* workspace,
                       size_t workspace_bytes, void* stream, Trace* tr) {
  const int32_t s = check_shape(N, d, V, R, dtype);
  if (s != VPCE_OK) return s;
  if (!W || !dW || !workspace) return VPCE_ERR_NULL;
  if (N > 0 && (!H || !labels || !lse || !dH)) return VPCE_ERR_NULL;
  if ((H && !aligned(H, 16)) || !aligned(W, 16) || (labels && !aligned(labels, 8)) ||
      (lse && !aligned(lse, 4)) || (dloss && !aligned(dloss, 4)) ||
      (dH && !aligned(dH, 16)) || !aligned(dW, 16) || !aligned(workspace, kAlign))
    return VPCE_ERR_ALIGN;
  const int64_t C = widest_chunk(N, d, V, R, dtype, workspace_bytes, false);
  if (C == 0) return VPCE_ERR_WORKSPACE;
  const Plan p = make_plan(N, d, V, R, dtype, C);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == VPCE_BF16)
    return run_backward<__bf16>(p, H, W, labels, lse, dloss, ignore_index, dH,
                                dW, ws, st, tr);
  return run_backward<float>(p, H, W, labels, lse, dloss, ignore_index, dH,
                             dW, ws, st, tr);
}

// Validates the trace arguments of the *_traced calls and sets up *t.
int32_t make_trace(void* const* events, int32_t max_launches, int32_t* kinds,
                   int32_t* n_launches, Trace* t) {
  if (max_launches < 0) return VPCE_ERR_SHAPE;
  if (!n_launches || (max_launches > 0 && (!events || !kinds)))
    return VPCE_ERR_NULL;
  for (int32_t i = 0; i < 2 * max_launches; ++i)
    if (!events[i]) return VPCE_ERR_NULL;
  t->ev = reinterpret_cast<const hipEvent_t*>(events);
  t->kinds = kinds;
  t->cap = max_launches;
  t->n = 0;
  return VPCE_OK;
}
}  // namespace

int32_t vpce_forward(const void* H, const void* W, const int64_t* labels,
                     int64_t N, int64_t d, int64_t V, int32_t R,
                     int64_t ignore_index, int32_t dtype, float* loss,
                     float* lse, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return forward_entry(H, W, labels, N, d, V, R, ignore_index, dtype, loss,
                       lse, workspace, workspace_bytes, stream, nullptr);
}

int32_t vpce_forward_traced(const void* H, const void* W,
                            const int64_t* labels, int64_t N, int64_t d,
                            int64_t V, int32_t R, int64_t ignore_index,
                            int32_t dtype, float* loss, float* lse,
                            void* workspace, size_t workspace_bytes,
                            void* stream, void* const* events,
                            int32_t max_launches, int32_t* kinds,
                            int32_t* n_launches) {
  Trace t;
  const int32_t s = make_trace(events, max_launches, kinds, n_launches, &t);
  if (s != VPCE_OK) return s;
  const int32_t rc = forward_entry(H, W, labels, N, d, V, R, ignore_index,
                                   dtype, loss, lse, workspace,
                                   workspace_bytes, stream, &t);
  *n_launches = t.n;
  return rc;
}

int32_t vpce_forward_noalloc(const void* H, const void* W,
                             const int64_t* labels, int64_t N, int64_t d,
                             int64_t V, int32_t R, int64_t ignore_index,
                             int32_t dtype, float* loss, float* lse,
                             void* stream) {
  const int32_t s = check_shape(N, d, V, R, dtype);
  if (s != VPCE_OK) return s;
  if (!W || !loss) return VPCE_ERR_NULL;
  if (N > 0 && (!H || !labels || !lse)) return VPCE_ERR_NULL;
  if ((H && !aligned(H, 16)) || !aligned(W, 16) || (labels && !aligned(labels, 8)) ||
      !aligned(loss, 4) || (lse && !aligned(lse, 4)))
    return VPCE_ERR_ALIGN;
  const Plan p = make_plan(N, d, V, R, dtype);
  if (p.fwd_bytes > (size_t)VPCE_NOALLOC_SCRATCH_BYTES) return VPCE_ERR_SCRATCH;
  char* ws = nullptr;
  const int32_t rc = scratch_on_current_device(&ws);
  if (rc != VPCE_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == VPCE_BF16)
    return run_forward<__bf16>(p, H, W, labels, ignore_index, loss, lse, ws, st);
  return run_forward<float>(p, H, W, labels, ignore_index, loss, lse, ws, st);
}

size_t vpce_forward_noalloc_bytes(int64_t N, int64_t d, int64_t V, int32_t R,
                                  int32_t dtype) {
  if (check_shape(N, d, V, R, dtype) != VPCE_OK) return 0;
  return make_plan(N, d, V, R, dtype).fwd_bytes;
}

int32_t vpce_backward(const void* H, const void* W, const int64_t* labels,
                      const float* lse, const float* dloss, int64_t N,
                      int64_t d, int64_t V, int32_t R, int64_t ignore_index,
                      int32_t dtype, float* dH, float* dW, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return backward_entry(H, W, labels, lse, dloss, N, d, V, R, ignore_index,
                        dtype, dH, dW, workspace, workspace_bytes, stream,
                        nullptr);
}

int32_t vpce_backward_traced(const void* H, const void* W,
                             const int64_t* labels, const float* lse,
                             const float* dloss, int64_t N, int64_t d,
                             int64_t V, int32_t R, int64_t ignore_index,
                             int32_t dtype, float* dH, float* dW,
                             void* workspace, size_t workspace_bytes,
                             void* stream, void* const* events,
                             int32_t max_launches, int32_t* kinds,
                             int32_t* n_launches) {
  Trace t;
  const int32_t s = make_trace(events, max_launches, kinds, n_launches, &t);
  if (s != VPCE_OK) return s;
  const int32_t rc = backward_entry(H, W, labels, lse, dloss, N, d, V, R,
                                    ignore_index, dtype, dH, dW, workspace,
                                    workspace_bytes, stream, &t);
  *n_launches = t.n;
  return rc;
}

int32_t vpce_state_init(float* state, int64_t N, void* stream) {
  if (N < 0 || N > kMaxTokens) return VPCE_ERR_SHAPE;
  if (N == 0) return VPCE_OK;
  if (!state) return VPCE_ERR_NULL;
  if (!aligned(state, 4)) return VPCE_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 g((unsigned)((N + 255) / 256));
  hipLaunchKernelGGL(fill_kernel, g, dim3(256), 0, st, state, N, -INFINITY);
  VPCE_LAUNCH_CHECK();
  hipLaunchKernelGGL(fill_kernel, g, dim3(256), 0, st, state + N, N, 0.f);
  VPCE_LAUNCH_CHECK();
  hipLaunchKernelGGL(fill_kernel, g, dim3(256), 0, st, state + 2 * N, N, NAN);
  VPCE_LAUNCH_CHECK();
  return VPCE_OK;
}

int32_t vpce_shard_fold(const void* H, const void* W_shard,
                        const int64_t* labels, int64_t N, int64_t d, int64_t V,
                        int64_t v_begin, int64_t v_count,
                        int64_t ignore_index, int32_t dtype, float* state,
                        void* workspace, size_t workspace_bytes,
                        void* stream) {
  const int32_t s = check_shape(N, d, V, 1, dtype);
  if (s != VPCE_OK) return s;
  if (v_begin < 0 || v_count < 1 || v_begin > V - v_count)
    return VPCE_ERR_SHAPE;
  if (!W_shard || !workspace) return VPCE_ERR_NULL;
  if (N > 0 && (!H || !labels || !state)) return VPCE_ERR_NULL;
  if ((H && !aligned(H, 16)) || !aligned(W_shard, 16) ||
      (labels && !aligned(labels, 8)) || (state && !aligned(state, 4)) ||
      !aligned(workspace, kAlign))
    return VPCE_ERR_ALIGN;
  const Plan p = make_plan(N, d, v_count, 1, dtype);
  if (workspace_bytes < p.fwd_bytes) return VPCE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == VPCE_BF16)
    return run_shard_fold<__bf16>(p, H, W_shard, v_begin, V, labels,
                                  ignore_index, state, ws, st);
  return run_shard_fold<float>(p, H, W_shard, v_begin, V, labels,
                               ignore_index, state, ws, st);
}

int32_t vpce_state_finish(const float* state, const int64_t* labels,
                          int64_t N, int64_t ignore_index, float* lse,
                          double* totals, float* loss, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (N < 0 || N > kMaxTokens) return VPCE_ERR_SHAPE;
  if (!totals || !workspace) return VPCE_ERR_NULL;
  if (N > 0 && (!state || !labels || !lse)) return VPCE_ERR_NULL;
  if ((state && !aligned(state, 4)) || (labels && !aligned(labels, 8)) ||
      (lse && !aligned(lse, 4)) || !aligned(totals, 8) ||
      (loss && !aligned(loss, 4)) || !aligned(workspace, kAlign))
    return VPCE_ERR_ALIGN;
  const int nb = (int)((N + 255) / 256);
  const size_t o_bcnt = up((size_t)(nb > 0 ? nb : 1) * 8);
  if (workspace_bytes < o_bcnt + up((size_t)(nb > 0 ? nb : 1) * 4))
    return VPCE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  double* bsum = reinterpret_cast<double*>(workspace);
  int* bcnt = reinterpret_cast<int*>(reinterpret_cast<char*>(workspace) + o_bcnt);
  if (N > 0) {
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)nb), dim3(256), 0, st,
                       state, state + N, state + 2 * N, labels, N, 1,
                       ignore_index, lse, bsum, bcnt);
    VPCE_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(256), 0, st, bsum, bcnt, nb,
                     loss, totals);
  VPCE_LAUNCH_CHECK();
  return VPCE_OK;
}

int32_t vpce_shard_backward(const void* H, const void* W_shard,
                            const int64_t* labels, const float* lse,
                            const double* totals, const float* dloss,
                            int64_t N, int64_t d, int64_t V, int64_t v_begin,
                            int64_t v_count, int64_t ignore_index,
                            int32_t dtype, float* dH, float* dW_shard,
                            void* workspace, size_t workspace_bytes,
                            void* stream) {
  const int32_t s = check_shape(N, d, V, 1, dtype);
  if (s != VPCE_OK) return s;
  if (v_begin < 0 || v_count < 1 || v_begin > V - v_count)
    return VPCE_ERR_SHAPE;
  if (!W_shard || !dW_shard || !totals || !workspace) return VPCE_ERR_NULL;
  if (N > 0 && (!H || !labels || !lse || !dH)) return VPCE_ERR_NULL;
  if ((H && !aligned(H, 16)) || !aligned(W_shard, 16) ||
      (labels && !aligned(labels, 8)) || (lse && !aligned(lse, 4)) ||
      !aligned(totals, 8) || (dloss && !aligned(dloss, 4)) ||
      (dH && !aligned(dH, 16)) || !aligned(dW_shard, 16) ||
      !aligned(workspace, kAlign))
    return VPCE_ERR_ALIGN;
  const int64_t C =
      widest_chunk(N, d, v_count, 1, dtype, workspace_bytes, false);
  if (C == 0) return VPCE_ERR_WORKSPACE;
  const Plan p = make_plan(N, d, v_count, 1, dtype, C);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  float* scale = reinterpret_cast<float*>(ws + p.o_scale);
  hipLaunchKernelGGL(scale_from_totals_kernel, dim3(1), dim3(64), 0, st,
                     totals, dloss, scale);
  VPCE_LAUNCH_CHECK();
  if (dtype == VPCE_BF16)
    return backward_span<__bf16>(p, H, W_shard, v_begin, v_count, V, labels,
                                 lse, scale, ignore_index, dH, true, dW_shard,
                                 true, ws, st, nullptr);
  return backward_span<float>(p, H, W_shard, v_begin, v_count, V, labels, lse,
                              scale, ignore_index, dH, true, dW_shard, true,
                              ws, st, nullptr);
}

int32_t vpce_ring_mode(int64_t N, int64_t d, int64_t V, int32_t R,
                       int32_t dtype, int32_t* mode, size_t* activation_bytes,
                       size_t* weight_bytes) {
  const int32_t s = check_shape(N, d, V, R, dtype);
  if (s != VPCE_OK) return s;
  if (!mode || !activation_bytes || !weight_bytes) return VPCE_ERR_NULL;
  const size_t esz = dtype == VPCE_BF16 ? 2 : 4;
  const int64_t widest = (V + R - 1) / R;
  *activation_bytes = (size_t)N * d * esz;
  *weight_bytes = (size_t)widest * d * esz;
  *mode = widest < N ? VPCE_RING_MOVE_WEIGHTS : VPCE_RING_MOVE_ACTIVATIONS;
  return VPCE_OK;
}

const char* vpce_status_string(int32_t status) {
  switch (status) {
    case VPCE_OK: return "ok";
    case VPCE_ERR_NULL: return "a required pointer is NULL";
    case VPCE_ERR_SHAPE: return "invalid shape (N, d, V or R)";
    case VPCE_ERR_UNSUPPORTED: return "unsupported dtype";
    case VPCE_ERR_ALIGN: return "misaligned pointer";
    case VPCE_ERR_WORKSPACE: return "workspace too small";
    case VPCE_ERR_HIP: return "HIP kernel launch failed";
    case VPCE_ERR_SCRATCH:
      return "shape needs more than the static scratch of the "
             "allocation-free forward (VPCE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
