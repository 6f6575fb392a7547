// The linear layers on either side of the decode-attention block (nodes
// attn.qkv_proj and attn.o_proj of the "Qwen3-0.6B" Model Spec page,
// "Compute-graph nodes": y[t,n] = sum_k x[t,k] w[n,k]) on the matrix cores
// of MI355X (gfx950).
//
// x is float32 [T][K], w bfloat16 [N][K] (the checkpoints' dtype), y float32.
// Both operands are K-contiguous, which is the layout v_mfma_f32_16x16x32_bf16
// reads: lane l = 16 r + c supplies row c and the 8 contiguous k values
// 8r .. 8r+7 of a 32-wide k step, for A (x) and B (w) alike.  x enters as two
// bfloat16 terms, hi = RNE(x) and lo = RNE(x - hi), so the product carries x
// to 2^-18 relative; w is exact.  Accumulation is float32.
//
// For decode's few rows (T < 32) the product is a few microseconds of data
// movement, so what matters is latency: few dependent round trips to memory
// per wave and enough workgroups.  linear_splitk_kernel gives each of a
// workgroup's 8 waves an eighth of k with operands loaded straight into
// registers (four k steps in flight), sums the partial tiles in LDS, and
// picks the tile width so that the grid has at least 256 workgroups.  From a
// few dozen rows on, every weight tile is shared by several row tiles, and
// linear_lds_kernel stages coalesced x and w tiles in LDS so that each is
// read from L2 once per tile instead of once per wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dah.h"
#include "dah_host.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Two floats -> two bfloat16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ float lo_half(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_half(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 floats -> hi and lo bfloat16 terms (4 words each).
__device__ __forceinline__ void split8(const float4& a, const float4& b, u32x4& hi, u32x4& lo) {
  hi[0] = pack2(a.x, a.y);
  hi[1] = pack2(a.z, a.w);
  hi[2] = pack2(b.x, b.y);
  hi[3] = pack2(b.z, b.w);
  lo[0] = pack2(a.x - lo_half(hi[0]), a.y - hi_half(hi[0]));
  lo[1] = pack2(a.z - lo_half(hi[1]), a.w - hi_half(hi[1]));
  lo[2] = pack2(b.x - lo_half(hi[2]), b.y - hi_half(hi[2]));
  lo[3] = pack2(b.z - lo_half(hi[3]), b.w - hi_half(hi[3]));
}

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Output columns [begin, begin + width) go to y[t * width + (n - begin)],
// plus res at the same place when res is set (res may be y).
struct Segment {
  float* y;
  int begin;
  int width;
  const float* res;
};

struct LinearArgs {
  const float* x;
  const uint16_t* w;
  int T, N, K;
  int nseg;
  Segment seg[3];
  int x_stride;         // floats per row of x
  const float* x_gain;  // kNorm: the norm's gain [K]
  float eps;            // kNorm
  // k slices (linear_lds_kernel): workgroup blockIdx.x takes output tile
  // blockIdx.x mod (the number of tiles) over k slice blockIdx.x / (the
  // number of tiles), an equal 1 / ksplit of k.  With ksplit > 1 (kPlain,
  // one segment only) each slice's products go to part[slice][T][N] and
  // linear_reduce_kernel adds them, in slice order, and the segment's
  // residual.
  int ksplit;
  float* part;
  // gated > 0 (mlp.act folded in): w has 2 gated rows, the gate rows
  // [0, gated) then the up rows [gated, 2 gated).  The product's columns
  // come in groups of 32: the first 16 read gate rows j .. j+15, the next
  // 16 up rows j .. j+15 (weight_row), so the lane that holds gate[t][j]
  // in one 16 x 16 accumulator block holds up[t][j] in the next, and the
  // store writes act[t][j] = silu(gate) * up to seg[0] (width gated).
  int gated;
};

// The weight row of product column n (n itself unless gated).
__device__ __forceinline__ int weight_row(const LinearArgs& a, int n) {
  if (a.gated == 0) return n;
  const int j = ((n >> 5) << 4) | (n & 15);
  return (n & 16) ? a.gated + j : j;
}

// What the products read as their input row x[t] (the kernels' kXMode):
//   kPlain  x as stored;
//   kNorm   the row RMS-normed, x[t][k] / sqrt(sum_j x[t][j]^2 / K + eps) *
//           gain[k] (the rmsnorm rows input_norm and post_attn_norm): x * gain
//           enters the product and each output row is scaled by the inverse
//           RMS, whose sum of squares is accumulated while the row streams
//           through (every workgroup reads all of k for its rows).  Each
//           column tile redoes this per element work, which stays cheap (a
//           multiply and a multiply-add); the SwiGLU activation, an exp and a
//           division per element, cost more redone per tile than a launch of
//           its own (measured) and stays a separate kernel.
enum XMode { kPlain = 0, kNorm = 1 };

__device__ __forceinline__ float4 mul4(const float4& a, const float4& b) {
  return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}
__device__ __forceinline__ float sumsq4(const float4& v, float acc) {
  return fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, acc))));
}
// The inverse RMS of a row from its sum of squares over K.
__device__ __forceinline__ float inv_rms(float ss, int K, float eps) {
  return 1.0f / sqrtf(ss / (float)K + eps);
}

__device__ __forceinline__ Segment segment_of(const LinearArgs& a, int n0) {
  Segment s = a.seg[0];
  if (a.nseg > 1 && n0 >= a.seg[1].begin) s = a.seg[1];
  if (a.nseg > 2 && n0 >= a.seg[2].begin) s = a.seg[2];
  return s;
}

// Stores one 16 x 16 accumulator block (D layout: lane (r, c) holds rows
// 4r + v, column c) whose top-left output is (m, n), row 4r + v scaled by
// scale[v].
__device__ __forceinline__ void store_block(const LinearArgs& a, const Segment& s, int m, int n,
                                            const f32x4& acc, int lane,
                                            const float (&scale)[4] = {1.f, 1.f, 1.f, 1.f}) {
  const int r = lane >> 4, c = lane & 15;
  float* col = s.y + (n - s.begin) + c;
  const float* rcol = s.res != nullptr ? s.res + (n - s.begin) + c : nullptr;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t = m + 4 * r + v;
    if (t < a.T) {
      const size_t at = (size_t)t * s.width;
      const float y = acc[v] * scale[v];
      col[at] = rcol != nullptr ? y + rcol[at] : y;
    }
  }
}

// Stores the SwiGLU activation of a (gate, up) pair of 16 x 16 accumulator
// blocks whose top-left output is (m, j0) of act: act[t][j] = silu(g) * u
// with g and u the row-scaled products, silu(z) = z / (1 + e^-z) (the
// mlp.act row, siluMul).
__device__ __forceinline__ void store_gated(const LinearArgs& a, int m, int j0, const f32x4& g,
                                            const f32x4& u, int lane,
                                            const float (&scale)[4] = {1.f, 1.f, 1.f, 1.f}) {
  const int r = lane >> 4, c = lane & 15;
  float* col = a.seg[0].y + j0 + c;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t = m + 4 * r + v;
    if (t < a.T) {
      const float gz = g[v] * scale[v], uz = u[v] * scale[v];
      col[(size_t)t * a.gated] = gz / (1.0f + expf(-gz)) * uz;
    }
  }
}

// ---------------------------------------------------------------- split-k

// One 32-wide k step of the split-k kernel's operands, per input mode (the
// norm's gain for kNorm).
template <int kMB, int kNB, int kXMode>
struct LinStep {
  float4 x[kMB][2];
  u32x4 w[kNB];
};
template <int kMB, int kNB>
struct LinStep<kMB, kNB, kNorm> {
  float4 x[kMB][2];
  float4 g[2];
  u32x4 w[kNB];
};

constexpr int kLinWaves = 8;        // waves per workgroup, each an eighth of k
constexpr int kLinMinGroups = 256;  // aim: one workgroup per compute unit or more

// One workgroup computes a (16 kMB kMW) x (16 kNB) output tile with 8 waves:
// wave w takes row group w mod kMW (16 kMB rows) and k slice w / kMW of
// kKS = 8 / kMW equal slices, with operands loaded straight into registers
// (up to four 32-wide k steps in flight); the kKS partial tiles of each row
// group are added in LDS.  The weight tile is read once per row tile (by the
// kMW row groups together, from L1/L2 after the first).
template <int kMB, int kNB, int kMW, int kXMode>
__global__ __launch_bounds__(kWave * kLinWaves) void linear_splitk_kernel(LinearArgs a) {
  constexpr int kKS = kLinWaves / kMW;
  static_assert(kLinWaves % kMW == 0, "row groups must divide the waves");
  __shared__ f32x4 part[kLinWaves][kMB * kNB][kWave];
  __shared__ float rowss[kLinWaves][kMB][16];  // kNorm: sums of squares per wave and row
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mw = wave % kMW, ks = wave / kMW;
  const int r = lane >> 4, c = lane & 15;
  const int n_tiles = a.N / (16 * kNB);
  const int n_tile = blockIdx.x % n_tiles;
  const int m_tile = blockIdx.x / n_tiles;
  const int m0 = m_tile * 16 * kMB * kMW + 16 * kMB * mw, n0 = n_tile * 16 * kNB;
  const int kw = a.K / kKS;
  const int k_begin = ks * kw;
  const int steps = kw / 32;

  // Lane (r, c): row c of each 16-row block of x and of each 16-column block
  // of w, k values 8r .. 8r+7 of every 32-wide step.
  const float* xp[kMB];
  bool ok[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    const int t = m0 + 16 * mb + c;
    ok[mb] = t < a.T;
    xp[mb] = a.x + (size_t)(ok[mb] ? t : 0) * a.x_stride + k_begin + 8 * r;
  }
  const float* gp = a.x_gain + k_begin + 8 * r;  // kNorm
  const uint16_t* wp[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
    wp[nb] = a.w + (size_t)weight_row(a, n0 + 16 * nb + c) * a.K + k_begin + 8 * r;

  using Step = LinStep<kMB, kNB, kXMode>;
  // Ordinary (cacheable) loads: row tiles that share a weight tile find it
  // in L2.
  auto load = [&](Step& st, int s) {
    const int k = 32 * s;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) st.w[nb] = *reinterpret_cast<const u32x4*>(wp[nb] + k);
    // (Zeros as prvalues: a named zero would make the selects pick between
    // addresses and put the zero in scratch memory.)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const float4* q = reinterpret_cast<const float4*>(xp[mb] + k);
      st.x[mb][0] = ok[mb] ? q[0] : make_float4(0.f, 0.f, 0.f, 0.f);
      st.x[mb][1] = ok[mb] ? q[1] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if constexpr (kXMode == kNorm) {
      st.g[0] = *reinterpret_cast<const float4*>(gp + k);
      st.g[1] = *reinterpret_cast<const float4*>(gp + k + 4);
    }
  };
  float ss[kMB];  // kNorm: this lane's share of its rows' sums of squares
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) ss[mb] = 0.0f;
  f32x4 acc[kMB][kNB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const Step& st) {
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      float4 x0 = st.x[mb][0], x1 = st.x[mb][1];
      if constexpr (kXMode == kNorm) {
        ss[mb] = sumsq4(x1, sumsq4(x0, ss[mb]));
        x0 = mul4(x0, st.g[0]);
        x1 = mul4(x1, st.g[1]);
      }
      u32x4 hi, lo;
      split8(x0, x1, hi, lo);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = mfma(hi, st.w[nb], acc[mb][nb]);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = mfma(lo, st.w[nb], acc[mb][nb]);
    }
  };

  // A multiple of 4 steps: four in flight per wave, each buffer refilled as
  // soon as it is consumed.  Otherwise two at a time.
  Step b0, b1, b2, b3;
  if ((steps & 3) == 0) {
    load(b0, 0);
    load(b1, 1);
    load(b2, 2);
    load(b3, 3);
    for (int s = 0; s + 4 < steps; s += 4) {
      __builtin_amdgcn_sched_barrier(0);
      consume(b0);
      load(b0, s + 4);
      __builtin_amdgcn_sched_barrier(0);
      consume(b1);
      load(b1, s + 5);
      __builtin_amdgcn_sched_barrier(0);
      consume(b2);
      load(b2, s + 6);
      __builtin_amdgcn_sched_barrier(0);
      consume(b3);
      load(b3, s + 7);
    }
    __builtin_amdgcn_sched_barrier(0);
    consume(b0);
    consume(b1);
    consume(b2);
    consume(b3);
  } else {
    for (int s = 0; s < steps; s += 2) {
      load(b0, s);
      if (s + 1 < steps) load(b1, s + 1);
      consume(b0);
      if (s + 1 < steps) consume(b1);
    }
  }

#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) part[wave][mb * kNB + nb][lane] = acc[mb][nb];
  if constexpr (kXMode == kNorm) {
    // Lanes c, c+16, c+32, c+48 hold row c's k values 8r..8r+7 of each step.
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      float v = ss[mb];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (r == 0) rowss[wave][mb][c] = v;
    }
  }
  __syncthreads();
  // (row group g, block blk) pairs spread over the waves; slice q of row
  // group g is wave g + kMW q.
  const Segment sg = segment_of(a, n0);
  const int m_base = m_tile * 16 * kMB * kMW;
  auto row_scale = [&](int g, int mb, float (&scale)[4]) {
    if constexpr (kXMode == kNorm) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < kKS; ++q) sum += rowss[g + kMW * q][mb][4 * r + v];
        scale[v] = inv_rms(sum, a.K, a.eps);
      }
    }
  };
  if constexpr (kNB % 2 == 0) {
   if (a.gated) {
    // (gate, up) block pairs
    constexpr int kPairs = kNB / 2;
    for (int job = wave; job < kMW * kMB * kPairs; job += kLinWaves) {
      const int g = job / (kMB * kPairs), pr = job % (kMB * kPairs);
      const int mb = pr / kPairs, nb = 2 * (pr % kPairs);
      f32x4 tg = part[g][mb * kNB + nb][lane], tu = part[g][mb * kNB + nb + 1][lane];
#pragma unroll
      for (int q = 1; q < kKS; ++q) {
        tg += part[g + kMW * q][mb * kNB + nb][lane];
        tu += part[g + kMW * q][mb * kNB + nb + 1][lane];
      }
      float scale[4] = {1.f, 1.f, 1.f, 1.f};
      row_scale(g, mb, scale);
      store_gated(a, m_base + 16 * kMB * g + 16 * mb, ((n0 + 16 * nb) >> 5) << 4, tg, tu, lane,
                  scale);
    }
    return;
   }
  }
  for (int job = wave; job < kMW * kMB * kNB; job += kLinWaves) {
    const int g = job / (kMB * kNB), blk = job % (kMB * kNB);
    f32x4 t = part[g][blk][lane];
#pragma unroll
    for (int q = 1; q < kKS; ++q) t += part[g + kMW * q][blk][lane];
    float scale[4] = {1.f, 1.f, 1.f, 1.f};
    row_scale(g, blk / kNB, scale);
    store_block(a, sg, m_base + 16 * kMB * g + 16 * (blk / kNB), n0 + 16 * (blk % kNB), t, lane,
                scale);
  }
}

// ---------------------------------------------------------------- LDS tiles

constexpr int kLdsThreads = 256;   // 4 waves

// For larger T, where every weight tile is shared by several row tiles and
// every x row by many column tiles, a workgroup of 4 waves computes a
// kBM x kBN output tile and walks k in chunks of kBK = 32 kKS kWK.  Per
// chunk the 256 threads load the x and w tiles with coalesced 16-byte loads
// (kDepth chunks ahead: the loads of the next kDepth chunks are in flight
// while this one is multiplied, since one chunk's round trip to L2 takes
// longer than its products), split x into its two bfloat16 terms once, and
// write hi, lo and w to LDS in
// the operand layout; wave (wm, wn, wk) then multiplies its
// (kBM / kWM) x (kBN / kWN) sub-tile over kKS 32-wide k steps of the chunk.
// With kWK > 1 the waves of a sub-tile take different k steps and their
// partial tiles are added in LDS, in a fixed order, at the end.
template <int kBM, int kBN, int kWM, int kWN, int kWK, int kKS, int kDepth, int kXMode>
__global__ __launch_bounds__(kLdsThreads) void linear_lds_kernel(LinearArgs a) {
  static_assert(kWM * kWN * kWK == kLdsThreads / kWave, "4 waves");
  constexpr int kBK = 32 * kKS * kWK;
  constexpr int kSM = kBM / kWM / 16, kSN = kBN / kWN / 16;   // 16 x 16 blocks per wave
  static_assert(kSM * kWM * 16 == kBM && kSN * kWN * 16 == kBN, "tile split");
  // bfloat16 per LDS row: 32 bytes of padding.  With 16, the operand reads
  // (16 bytes of rows c = 0..15 at one k offset) put rows c and c + 8 on the
  // same banks (about 1.9 conflict cycles per LDS instruction); with 32 none
  // do, and every row stays 16-byte aligned.
  constexpr int kRow = kBK + 16;
  constexpr int kX4 = kBM * kBK / 4 / kLdsThreads;   // float4 loads of x per thread
  constexpr int kW8 = kBN * kBK / 8 / kLdsThreads;   // 16-byte loads of w per thread
  static_assert(kX4 * 4 * kLdsThreads == kBM * kBK && kW8 * 8 * kLdsThreads == kBN * kBK,
                "whole loads");
  __shared__ __attribute__((aligned(16))) uint16_t xh[kBM][kRow];
  __shared__ __attribute__((aligned(16))) uint16_t xl[kBM][kRow];
  __shared__ __attribute__((aligned(16))) uint16_t ws[kBN][kRow];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWM, wn = (wave / kWM) % kWN, wk = wave / (kWM * kWN);
  const int r = lane >> 4, c = lane & 15;
  const int n_tiles = a.N / kBN;
  const int tiles = ((a.T + kBM - 1) / kBM) * n_tiles;
  const int tile = blockIdx.x % tiles, slice = blockIdx.x / tiles;
  const int n0 = (tile % n_tiles) * kBN;
  const int m0 = (tile / n_tiles) * kBM;
  const int chunks = a.K / kBK / a.ksplit;
  const int k_base = slice * chunks * kBK;

  // Coalesced tile loads: consecutive threads take consecutive 16 bytes of
  // a row.  Rows of x past T read as zero.
  const float* xsrc[kX4];
  bool xok[kX4];
#pragma unroll
  for (int i = 0; i < kX4; ++i) {
    const int idx = tid + kLdsThreads * i;
    const int row = idx / (kBK / 4), t = m0 + row;
    xok[i] = t < a.T;
    xsrc[i] = a.x + (size_t)(xok[i] ? t : 0) * a.x_stride + k_base + 4 * (idx % (kBK / 4));
  }
  const uint16_t* wsrc[kW8];
#pragma unroll
  for (int i = 0; i < kW8; ++i) {
    const int idx = tid + kLdsThreads * i;
    wsrc[i] = a.w + (size_t)weight_row(a, n0 + idx / (kBK / 8)) * a.K + k_base +
              8 * (idx % (kBK / 8));
  }
  struct Chunk {
    float4 x[kX4];
    float4 g[kXMode == kNorm ? kX4 : 1];  // kNorm: the gain
    u32x4 w[kW8];
  };
  auto load = [&](Chunk& b, int chunk) {
    const int k = chunk * kBK;
#pragma unroll
    for (int i = 0; i < kX4; ++i) {
      b.x[i] = xok[i] ? *reinterpret_cast<const float4*>(xsrc[i] + k) : make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (kXMode == kNorm)
        b.g[i] = *reinterpret_cast<const float4*>(a.x_gain + k_base + k +
                                                  4 * ((tid + kLdsThreads * i) % (kBK / 4)));
    }
#pragma unroll
    for (int i = 0; i < kW8; ++i) b.w[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + k);
  };
  float ss[kX4];  // kNorm: this thread's share of its rows' sums of squares
#pragma unroll
  for (int i = 0; i < kX4; ++i) ss[i] = 0.0f;
  auto stage = [&](const Chunk& b) {
#pragma unroll
    for (int i = 0; i < kX4; ++i) {
      const int idx = tid + kLdsThreads * i;
      const int row = idx / (kBK / 4), col = 4 * (idx % (kBK / 4));
      float4 v = b.x[i];
      if constexpr (kXMode == kNorm) {
        ss[i] = sumsq4(v, ss[i]);
        v = mul4(v, b.g[i]);
      }
      const uint32_t h0 = pack2(v.x, v.y), h1 = pack2(v.z, v.w);
      const uint32_t l0 = pack2(v.x - lo_half(h0), v.y - hi_half(h0));
      const uint32_t l1 = pack2(v.z - lo_half(h1), v.w - hi_half(h1));
      *reinterpret_cast<uint2*>(&xh[row][col]) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(&xl[row][col]) = make_uint2(l0, l1);
    }
#pragma unroll
    for (int i = 0; i < kW8; ++i) {
      const int idx = tid + kLdsThreads * i;
      *reinterpret_cast<u32x4*>(&ws[idx / (kBK / 8)][8 * (idx % (kBK / 8))]) = b.w[i];
    }
  };

  f32x4 acc[kSM][kSN];
#pragma unroll
  for (int mb = 0; mb < kSM; ++mb)
#pragma unroll
    for (int nb = 0; nb < kSN; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int arow = wm * (kBM / kWM) + c, brow = wn * (kBN / kWN) + c;

  auto multiply = [&]() {
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
      const int kk = 32 * (wk * kKS + s) + 8 * r;
      u32x4 b[kSN];
#pragma unroll
      for (int nb = 0; nb < kSN; ++nb) b[nb] = *reinterpret_cast<const u32x4*>(&ws[brow + 16 * nb][kk]);
#pragma unroll
      for (int mb = 0; mb < kSM; ++mb) {
        const u32x4 hi = *reinterpret_cast<const u32x4*>(&xh[arow + 16 * mb][kk]);
        const u32x4 lo = *reinterpret_cast<const u32x4*>(&xl[arow + 16 * mb][kk]);
#pragma unroll
        for (int nb = 0; nb < kSN; ++nb) acc[mb][nb] = mfma(hi, b[nb], acc[mb][nb]);
#pragma unroll
        for (int nb = 0; nb < kSN; ++nb) acc[mb][nb] = mfma(lo, b[nb], acc[mb][nb]);
      }
    }
  };

  // A ring of kDepth register buffers; buffer i always holds chunks
  // congruent to i mod kDepth, so every index is a compile-time constant.
  Chunk buf[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth; ++i)
    if (i < chunks) load(buf[i], i);
  for (int c0 = 0; c0 < chunks; c0 += kDepth) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      const int chunk = c0 + i;
      if (chunk < chunks) {
        __syncthreads();   // the previous chunk's products are done with LDS
        stage(buf[i]);
        __syncthreads();
        if (chunk + kDepth < chunks) load(buf[i], chunk + kDepth);
        multiply();
      }
    }
  }

  const Segment sg = a.ksplit > 1 ? Segment{a.part + (size_t)slice * a.T * a.N, 0, a.N, nullptr}
                                  : segment_of(a, n0);
  // kNorm: the rows' inverse RMS.  The kBK / 4 consecutive threads that stage
  // one row's chunk hold its sum of squares between them.
  __shared__ float row_scale[kXMode == kNorm ? kBM : 1];
  if constexpr (kXMode == kNorm) {
#pragma unroll
    for (int i = 0; i < kX4; ++i) {
      float v = ss[i];
#pragma unroll
      for (int off = 1; off < kBK / 4; off <<= 1) v += __shfl_xor(v, off);
      const int idx = tid + kLdsThreads * i;
      if (idx % (kBK / 4) == 0) row_scale[idx / (kBK / 4)] = inv_rms(v, a.K, a.eps);
    }
    __syncthreads();
  }
  auto scales = [&](int mrow) {  // scales of rows mrow + 4r + v (local rows)
    f32x4 sc = {1.f, 1.f, 1.f, 1.f};
    if constexpr (kXMode == kNorm) {
#pragma unroll
      for (int v = 0; v < 4; ++v) sc[v] = row_scale[mrow + 4 * r + v];
    }
    return sc;
  };
  static_assert(kSN % 2 == 0, "gate and up blocks pair up within a wave");
  if constexpr (kWK == 1) {
    if (a.gated) {
#pragma unroll
      for (int mb = 0; mb < kSM; ++mb)
#pragma unroll
        for (int nb = 0; nb < kSN; nb += 2) {
          const int mrow = wm * (kBM / kWM) + 16 * mb;
          float sc[4];
          const auto s4 = scales(mrow);
#pragma unroll
          for (int v = 0; v < 4; ++v) sc[v] = s4[v];
          store_gated(a, m0 + mrow, ((n0 + wn * (kBN / kWN) + 16 * nb) >> 5) << 4, acc[mb][nb],
                      acc[mb][nb + 1], lane, sc);
        }
      return;
    }
#pragma unroll
    for (int mb = 0; mb < kSM; ++mb)
#pragma unroll
      for (int nb = 0; nb < kSN; ++nb) {
        const int mrow = wm * (kBM / kWM) + 16 * mb;
        float sc[4];
        const auto s4 = scales(mrow);
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[v] = s4[v];
        store_block(a, sg, m0 + mrow, n0 + wn * (kBN / kWN) + 16 * nb, acc[mb][nb], lane, sc);
      }
  } else {
    __shared__ f32x4 part[kWK][kWM * kWN * kSM * kSN][kWave];
    const int sub = wm + kWM * wn;
#pragma unroll
    for (int mb = 0; mb < kSM; ++mb)
#pragma unroll
      for (int nb = 0; nb < kSN; ++nb) part[wk][(sub * kSM + mb) * kSN + nb][lane] = acc[mb][nb];
    __syncthreads();
    if (a.gated) {
      for (int job = wave; job < kWM * kWN * kSM * (kSN / 2); job += kLdsThreads / kWave) {
        const int js = job / (kSM * (kSN / 2)), mb = (job / (kSN / 2)) % kSM;
        const int nb = 2 * (job % (kSN / 2));
        const int base = (js * kSM + mb) * kSN + nb;
        f32x4 tg = part[0][base][lane], tu = part[0][base + 1][lane];
#pragma unroll
        for (int q = 1; q < kWK; ++q) {
          tg += part[q][base][lane];
          tu += part[q][base + 1][lane];
        }
        const int mrow = (js % kWM) * (kBM / kWM) + 16 * mb;
        float sc[4];
        const auto s4 = scales(mrow);
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[v] = s4[v];
        store_gated(a, m0 + mrow, ((n0 + (js / kWM) * (kBN / kWN) + 16 * nb) >> 5) << 4, tg, tu,
                    lane, sc);
      }
      return;
    }
    for (int job = wave; job < kWM * kWN * kSM * kSN; job += kLdsThreads / kWave) {
      f32x4 t = part[0][job][lane];
#pragma unroll
      for (int q = 1; q < kWK; ++q) t += part[q][job][lane];
      const int js = job / (kSM * kSN), mb = (job / kSN) % kSM, nb = job % kSN;
      const int mrow = (js % kWM) * (kBM / kWM) + 16 * mb;
      float sc[4];
      const auto s4 = scales(mrow);
#pragma unroll
      for (int v = 0; v < 4; ++v) sc[v] = s4[v];
      store_block(a, sg, m0 + mrow, n0 + (js / kWM) * (kBN / kWN) + 16 * nb, t, lane, sc);
    }
  }
}

// ---------------------------------------------------------------- k slices

// y = part[0] + ... + part[kS - 1] (+ res), added in slice order; one float4
// per thread, every slice's load in flight at once.  part [kS][n4] float4,
// y and res [n4] float4 (res may be y: each thread reads its own element
// before it writes it).
template <int kS>
__global__ __launch_bounds__(256) void linear_reduce_kernel(const float4* part, size_t n4,
                                                            const float4* res, float4* y) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  float4 v[kS];
#pragma unroll
  for (int q = 0; q < kS; ++q) v[q] = part[q * n4 + i];
  float4 sum = v[0];
#pragma unroll
  for (int q = 1; q < kS; ++q) {
    sum.x += v[q].x;
    sum.y += v[q].y;
    sum.z += v[q].z;
    sum.w += v[q].w;
  }
  if (res != nullptr) {
    const float4 r = res[i];
    sum.x += r.x;
    sum.y += r.y;
    sum.z += r.z;
    sum.w += r.w;
  }
  y[i] = sum;
}

struct LinearConfig {
  int lds;          // 0: linear_splitk_kernel<mb, nb, mw>; else an LDS tile shape, by id
  int mb, nb, mw;
  int ksplit = 1;   // k slices
};

// An LDS tile shape needs N, and every output segment's first column, to be
// multiples of its width, and k to be a multiple of its chunk.
bool lds_fits(const LinearArgs& a, int bn, int bk) {
  if (a.N % bn != 0 || a.K % bk != 0) return false;
  for (int i = 0; i < a.nseg; ++i)
    if (a.seg[i].begin % bn != 0) return false;
  return true;
}

// The instantiated LDS tile shapes (launch_lds_shape):
//   1: 64 x 128, 2 x 2 waves, k chunks of 64     2: 64 x 64, 2 x 2 waves, chunks of 64
//   3: 32 x 64, 1 x 2 waves x 2 k slices, 64     4: 32 x 32, 4 k slices, chunks of 128
//   5: 32 x 32, 4 k slices, chunks of 256, two chunks in flight
//
// Tile choice: the largest tile that still gives 512 workgroups (two per
// compute unit), else 32 x 32 with the k steps split over the waves (the
// deep-chunk form for long k at up to 256 rows) while that gives 128
// workgroups, else the split-k kernel; T < 32 always takes the split-k
// kernel, which is built for decode's few rows.  Swept on MI355X over
// T = 32 .. 4096 and (N, K) = (4096, 1024), (1024, 2048), (6144, 1024),
// (1024, 3072), (10240, 1024), (1024, 8192) (graph-replayed launch times):
// this rule picks the fastest or one within 5% of it in every case.
int pick_lds(const LinearArgs& a) {
  if (a.T < 32) return 0;
  auto groups = [&](int bm, int bn) { return (long long)((a.T + bm - 1) / bm) * (a.N / bn); };
  if (lds_fits(a, 128, 64) && groups(64, 128) >= 512) return 1;
  if (lds_fits(a, 64, 64) && groups(64, 64) >= 512) return 2;
  if (lds_fits(a, 64, 64) && groups(32, 64) >= 512) return 3;
  if (lds_fits(a, 32, 128) && groups(32, 32) >= 128)
    return (a.K >= 2048 && a.T <= 256 && lds_fits(a, 32, 256)) ? 5 : 4;
  return 0;
}

// Split-k tile shape (T < 32, or too few LDS tiles): the widest of 64, 32,
// 16 columns (32 rows per tile) that still gives kLinMinGroups workgroups,
// else 16 x 16 tiles.  Swept on MI355X over 12 shapes (rows per wave 1-2,
// columns 1-4 blocks, 1-4 row groups) at T = 2 .. 256 and N x K =
// 4096 x 1024, 1024 x 2048 (graph-replayed launch times): this rule picks
// the fastest shape or one within 3% of it in every case.
// With the norm folded in (kNorm) the split-k tiles stop at 32 columns: the
// gain in flight leaves no registers for 64.
// A gated product (mlp.act folded in) needs its gate and up blocks side by
// side in every wave: 2 or 4 column blocks per wave.
LinearConfig pick_config(const LinearArgs& a, int x_mode = kPlain) {
  const int lds = pick_lds(a);
  if (lds != 0) return {lds, 0, 0, 0};
  const int min_nb = a.gated ? 2 : 1;
  if (a.T > 16) {
    const int m_tiles = (a.T + 31) / 32;
    for (int nb = x_mode == kPlain ? 4 : 2; nb >= min_nb; nb /= 2)
      if (m_tiles * (a.N / (16 * nb)) >= kLinMinGroups) return {0, 2, nb, 1};
  }
  return {0, 1, min_nb, 1};
}

// With a workspace for k slices (plain products into one segment), products
// with K >= 2048 also consider splitting k: the largest LDS tile (64 x 128,
// 64 x 64, 32 x 64, 32 x 32) whose tiles times 1, 4 or 8 slices (the
// fewest) reach 512 workgroups with slices of 384 k or more; failing that,
// 32 x 32 tiles over 8 slices (or 4) of 256 k or more.  (Two slices would
// only pay for T < 32 with N >= 32768.)
// Shorter k keeps pick_config's choice.  Swept on MI355X over T = 16 .. 512
// and (N, K) = (1024, 2048 .. 8192), (4096 .. 10240, 1024), slices 1-8 on
// every tile shape (back-to-back launch times, the reduce included): this
// rule is within 4% of the fastest configuration wherever it splits, and up
// to 2.4x faster than the unsplit choice (T = 16, N = 1024, K = 5120).
constexpr int kSplitMinK = 2048;
LinearConfig pick_split_config(const LinearArgs& a) {
  if (a.K >= kSplitMinK) {
    static const int kShapeBM[5] = {64, 64, 32, 32, 32}, kShapeBN[5] = {128, 64, 64, 32, 32};
    static const int kShapeBK[5] = {64, 64, 64, 128, 256};
    auto tiles = [&](int id) {
      return (long long)((a.T + kShapeBM[id - 1] - 1) / kShapeBM[id - 1]) * (a.N / kShapeBN[id - 1]);
    };
    if (a.T >= 32)
      for (int id = 1; id <= 3; ++id)
        if (lds_fits(a, kShapeBN[id - 1], kShapeBK[id - 1]) && tiles(id) >= 512) return {id, 0, 0, 0, 1};
    for (int id = 1; id <= 4; ++id)
      for (int ks = 4; ks <= 8; ks *= 2)
        if (a.K / ks >= 384 && lds_fits(a, kShapeBN[id - 1], kShapeBK[id - 1] * ks) &&
            tiles(id) * ks >= 512)
          return {id, 0, 0, 0, ks};
    for (int ks = 8; ks >= 4; ks /= 2)
      if (a.K / ks >= 256 && lds_fits(a, 32, 128 * ks)) return {(a.K / ks) % 512 == 0 ? 5 : 4, 0, 0, 0, ks};
  }
  return pick_config(a);
}

// Bytes of k-slice partial products a configuration needs.
size_t split_bytes(const LinearArgs& a, const LinearConfig& c) {
  return c.ksplit > 1 ? (size_t)c.ksplit * a.T * a.N * sizeof(float) : 0;
}

template <int kBM, int kBN, int kWM, int kWN, int kWK, int kKS, int kDepth, int kXMode>
int launch_lds(const LinearArgs& a, hipStream_t stream) {
  if (!lds_fits(a, kBN, 32 * kKS * kWK * a.ksplit))
    return dah::set_error(DAH_ERR_SHAPE, "linear: tile %dx%d does not divide N=%d, K=%d", kBM,
                          kBN, a.N, a.K);
  const long long groups = (long long)((a.T + kBM - 1) / kBM) * (a.N / kBN) * a.ksplit;
  if (groups > INT32_MAX) return dah::set_error(DAH_ERR_SHAPE, "linear: grid too large");
  linear_lds_kernel<kBM, kBN, kWM, kWN, kWK, kKS, kDepth, kXMode>
      <<<dim3((unsigned)groups), kLdsThreads, 0, stream>>>(a);
  return DAH_OK;
}

template <int kXMode>
int launch_lds_shape(int id, const LinearArgs& a, hipStream_t stream) {
  switch (id) {
    case 1: return launch_lds<64, 128, 2, 2, 1, 2, 1, kXMode>(a, stream);
    case 2: return launch_lds<64, 64, 2, 2, 1, 2, 1, kXMode>(a, stream);
    case 3: return launch_lds<32, 64, 1, 2, 2, 1, 1, kXMode>(a, stream);
    case 4: return launch_lds<32, 32, 1, 1, 4, 1, 1, kXMode>(a, stream);
    case 5: return launch_lds<32, 32, 1, 1, 4, 2, 2, kXMode>(a, stream);
    default: return dah::set_error(DAH_ERR_HIP, "linear: no LDS tile shape %d", id);
  }
}

template <int kMB, int kNB, int kMW, int kXMode>
int launch_cfg(const LinearArgs& a, hipStream_t stream) {
  const int rows = 16 * kMB * kMW;
  const long long groups = (long long)((a.T + rows - 1) / rows) * (a.N / (16 * kNB));
  if (groups > INT32_MAX) return dah::set_error(DAH_ERR_SHAPE, "linear: grid too large");
  linear_splitk_kernel<kMB, kNB, kMW, kXMode>
      <<<dim3((unsigned)groups), kWave * kLinWaves, 0, stream>>>(a);
  return DAH_OK;
}

template <int kXMode>
int launch_mode(const LinearArgs& a, const LinearConfig& c, hipStream_t stream) {
  if (c.lds != 0) return launch_lds_shape<kXMode>(c.lds, a, stream);
  // The instantiated shapes; N is a multiple of 64, so every column tiling divides it.
#define DAH_LIN_CASE(MB, NB, MW) \
  if (c.mb == MB && c.nb == NB && c.mw == MW) return launch_cfg<MB, NB, MW, kXMode>(a, stream);
  DAH_LIN_CASE(1, 1, 1)
  DAH_LIN_CASE(1, 2, 1)
  DAH_LIN_CASE(2, 1, 1)
  DAH_LIN_CASE(2, 2, 1)
  if constexpr (kXMode == kPlain) {
    DAH_LIN_CASE(2, 4, 1)
  }
#undef DAH_LIN_CASE
  return dah::set_error(DAH_ERR_HIP, "linear: no kernel for tile %d/%d/%d", c.mb, c.nb, c.mw);
}

// The product under configuration c; with c.ksplit > 1 (kPlain, one
// segment starting at column 0) the slices' partial products go to part
// [ksplit][T][N] float32 and linear_reduce_kernel writes the segment.
// Sets a.x_stride, a.ksplit and a.part.
int launch_config(LinearArgs& a, const LinearConfig& c, int x_mode, float* part,
                  hipStream_t stream) {
  a.x_stride = a.K;
  a.ksplit = c.ksplit;
  a.part = part;
  if (c.ksplit > 1) {
    if (x_mode != kPlain || a.nseg != 1 || a.seg[0].begin != 0 || a.seg[0].width != a.N)
      return dah::set_error(DAH_ERR_HIP, "linear: k slices need a plain single-segment product");
    if (c.lds == 0 || (c.ksplit != 4 && c.ksplit != 8))
      return dah::set_error(DAH_ERR_HIP, "linear: k slices need an LDS tile and 4 or 8 slices");
    if (part == nullptr || reinterpret_cast<uintptr_t>(part) % 16 != 0)
      return dah::set_error(DAH_ERR_HIP, "linear: k slices need a 16-byte aligned workspace");
  }
  int st = x_mode == kNorm ? launch_mode<kNorm>(a, c, stream) : launch_mode<kPlain>(a, c, stream);
  if (st != DAH_OK) return st;
  if (c.ksplit > 1) {
    const size_t n4 = (size_t)a.T * a.N / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256));
    const float4* p4 = reinterpret_cast<const float4*>(part);
    const float4* r4 = reinterpret_cast<const float4*>(a.seg[0].res);
    float4* y4 = reinterpret_cast<float4*>(a.seg[0].y);
    if (c.ksplit == 4) linear_reduce_kernel<4><<<grid, 256, 0, stream>>>(p4, n4, r4, y4);
    if (c.ksplit == 8) linear_reduce_kernel<8><<<grid, 256, 0, stream>>>(p4, n4, r4, y4);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dah::set_error(DAH_ERR_HIP, "linear kernel launch failed: %s", hipGetErrorString(e));
  return DAH_OK;
}

// x_mode: kPlain or kNorm (a.x_gain, a.eps set).
int launch_linear(LinearArgs& a, hipStream_t stream, int x_mode = kPlain) {
  return launch_config(a, pick_config(a, x_mode), x_mode, nullptr, stream);
}

int check_norm(const float* gain, float eps, const char* who) {
  if (!gain) return dah::set_error(DAH_ERR_NULL, "%s: the norm gain is NULL", who);
  if (reinterpret_cast<uintptr_t>(gain) % 16 != 0)
    return dah::set_error(DAH_ERR_ALIGN, "%s: the norm gain needs 16-byte alignment", who);
  if (!(eps >= 0.0f)) return dah::set_error(DAH_ERR_SHAPE, "%s: eps must be >= 0", who);
  return DAH_OK;
}

}  // namespace

namespace dah {

int qkv_proj(const float* x, const float* x_gain, float eps, const void* w_qkv, int T, int hidden,
             int num_heads, float* q, float* k, float* v, void* stream) {
  if (!q || !k || !v) return set_error(DAH_ERR_NULL, "attn_qkv_proj: an output is NULL");
  if (!valid_heads(num_heads))
    return set_error(DAH_ERR_SHAPE, "num_heads = %d, need 16, 32, 40 or 64", num_heads);
  const int nq = num_heads * kHeadDim, nkv = kKvHeads * kHeadDim;
  int st = x_gain ? check_norm(x_gain, eps, "attn_qkv_proj") : DAH_OK;
  if (st == DAH_OK) st = validate_linear(x, w_qkv, T, nq + 2 * nkv, hidden, q);
  if (st != DAH_OK) return st;
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) % 16 != 0)
    return set_error(DAH_ERR_ALIGN, "attn_qkv_proj: k and v need 16-byte alignment");
  LinearArgs a = {};
  a.x = x;
  a.w = static_cast<const uint16_t*>(w_qkv);
  a.T = T;
  a.N = nq + 2 * nkv;
  a.K = hidden;
  a.nseg = 3;
  a.seg[0] = Segment{q, 0, nq, nullptr};
  a.seg[1] = Segment{k, nq, nkv, nullptr};
  a.seg[2] = Segment{v, nq + nkv, nkv, nullptr};
  a.x_gain = x_gain;
  a.eps = eps;
  return launch_linear(a, static_cast<hipStream_t>(stream), x_gain ? kNorm : kPlain);
}

}  // namespace dah

extern "C" {

int dah_linear_kernel(int T, int N, int K) {
  if (T < 1 || N < 64 || N % 64 != 0 || K < 256 || K % 256 != 0) return -1;
  LinearArgs a = {};
  a.T = T;
  a.N = N;
  a.K = K;
  a.nseg = 1;
  return pick_config(a).lds;
}

int dah_linear(const float* x, const void* w, int T, int N, int K, float* y, void* stream) {
  int st = dah::validate_linear(x, w, T, N, K, y);
  if (st != DAH_OK) return st;
  LinearArgs a = {};
  a.x = x;
  a.w = static_cast<const uint16_t*>(w);
  a.T = T;
  a.N = N;
  a.K = K;
  a.nseg = 1;
  a.seg[0] = Segment{y, 0, N, nullptr};
  return launch_linear(a, static_cast<hipStream_t>(stream));
}

int dah_linear_residual(const float* x, const void* w, const float* residual, int T, int N,
                        int K, float* y, void* stream) {
  if (!residual) return dah::set_error(DAH_ERR_NULL, "dah_linear_residual: residual is NULL");
  if (reinterpret_cast<uintptr_t>(residual) % 16 != 0)
    return dah::set_error(DAH_ERR_ALIGN, "dah_linear_residual: residual needs 16-byte alignment");
  int st = dah::validate_linear(x, w, T, N, K, y);
  if (st != DAH_OK) return st;
  LinearArgs a = {};
  a.x = x;
  a.w = static_cast<const uint16_t*>(w);
  a.T = T;
  a.N = N;
  a.K = K;
  a.nseg = 1;
  a.seg[0] = Segment{y, 0, N, residual};
  return launch_linear(a, static_cast<hipStream_t>(stream));
}

size_t dah_linear_workspace_bytes(int T, int N, int K) {
  if (T < 1 || N < 64 || N % 64 != 0 || K < 256 || K % 256 != 0) return 0;
  LinearArgs a = {};
  a.T = T;
  a.N = N;
  a.K = K;
  a.nseg = 1;
  return split_bytes(a, pick_split_config(a));
}

int dah_linear_ws_kernel(int T, int N, int K, int* k_slices) {
  if (T < 1 || N < 64 || N % 64 != 0 || K < 256 || K % 256 != 0) return -1;
  LinearArgs a = {};
  a.T = T;
  a.N = N;
  a.K = K;
  a.nseg = 1;
  const LinearConfig c = pick_split_config(a);
  if (k_slices) *k_slices = c.ksplit;
  return c.lds;
}

int dah_linear_ws(const float* x, const void* w, const float* residual, int T, int N, int K,
                  float* y, void* workspace, size_t workspace_bytes, void* stream) {
  if (reinterpret_cast<uintptr_t>(residual) % 16 != 0)
    return dah::set_error(DAH_ERR_ALIGN, "dah_linear_ws: residual needs 16-byte alignment");
  int st = dah::validate_linear(x, w, T, N, K, y);
  if (st != DAH_OK) return st;
  LinearArgs a = {};
  a.x = x;
  a.w = static_cast<const uint16_t*>(w);
  a.T = T;
  a.N = N;
  a.K = K;
  a.nseg = 1;
  a.seg[0] = Segment{y, 0, N, residual};
  const LinearConfig c = pick_split_config(a);
  const size_t need = split_bytes(a, c);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return dah::set_error(DAH_ERR_WORKSPACE, "dah_linear_ws: workspace of %zu bytes, need %zu",
                          workspace ? workspace_bytes : (size_t)0, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return dah::set_error(DAH_ERR_ALIGN, "dah_linear_ws: workspace needs 256-byte alignment");
  return launch_config(a, c, kPlain, static_cast<float*>(workspace), static_cast<hipStream_t>(stream));
}

int attn_qkv_proj(const float* x, const void* w_qkv, int T, int hidden, int num_heads, float* q,
                  float* k, float* v, void* stream) {
  return dah::qkv_proj(x, nullptr, 0.0f, w_qkv, T, hidden, num_heads, q, k, v, stream);
}

int dah_rmsnorm_linear(const float* x, const float* x_gain, float eps, const void* w, int T,
                       int N, int K, float* y, void* stream) {
  int st = check_norm(x_gain, eps, "dah_rmsnorm_linear");
  if (st == DAH_OK) st = dah::validate_linear(x, w, T, N, K, y);
  if (st != DAH_OK) return st;
  LinearArgs a = {};
  a.x = x;
  a.w = static_cast<const uint16_t*>(w);
  a.T = T;
  a.N = N;
  a.K = K;
  a.nseg = 1;
  a.seg[0] = Segment{y, 0, N, nullptr};
  a.x_gain = x_gain;
  a.eps = eps;
  return launch_linear(a, static_cast<hipStream_t>(stream), kNorm);
}

int dah_rmsnorm_swiglu(const float* x, const float* x_gain, float eps, const void* w_gate_up,
                       int T, int inter, int K, float* act, void* stream) {
  int st = x_gain ? check_norm(x_gain, eps, "dah_rmsnorm_swiglu") : DAH_OK;
  if (st == DAH_OK && (inter < 32 || inter % 32 != 0))
    st = dah::set_error(DAH_ERR_SHAPE, "dah_rmsnorm_swiglu: inter = %d, need a positive "
                        "multiple of 32", inter);
  if (st == DAH_OK) st = dah::validate_linear(x, w_gate_up, T, 2 * inter, K, act);
  if (st != DAH_OK) return st;
  LinearArgs a = {};
  a.x = x;
  a.w = static_cast<const uint16_t*>(w_gate_up);
  a.T = T;
  a.N = 2 * inter;
  a.K = K;
  a.nseg = 1;
  a.seg[0] = Segment{act, 0, inter, nullptr};
  a.x_gain = x_gain;
  a.eps = eps;
  a.gated = inter;
  return launch_linear(a, static_cast<hipStream_t>(stream), x_gain ? kNorm : kPlain);
}

int attn_o_proj(const float* o, const void* w_o, int T, int num_heads, int hidden, float* y,
                void* stream) {
  if (!dah::valid_heads(num_heads))
    return dah::set_error(DAH_ERR_SHAPE, "num_heads = %d, need 16, 32, 40 or 64", num_heads);
  return dah_linear(o, w_o, T, hidden, num_heads * dah::kHeadDim, y, stream);
}

int attn_o_proj_ws(const float* o, const void* w_o, int T, int num_heads, int hidden, float* y,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!dah::valid_heads(num_heads))
    return dah::set_error(DAH_ERR_SHAPE, "num_heads = %d, need 16, 32, 40 or 64", num_heads);
  return dah_linear_ws(o, w_o, nullptr, T, hidden, num_heads * dah::kHeadDim, y, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"
