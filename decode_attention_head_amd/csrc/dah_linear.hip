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
// At decode sizes (T <= a few hundred tokens, K and N ~ 1-10 thousand) the
// product is a few microseconds of data movement, so what matters is
// latency: few dependent round trips to memory per wave and enough
// workgroups.  linear_splitk_kernel gives each of a workgroup's 8 waves an
// eighth of k with operands loaded straight into registers (four k steps in
// flight), sums the partial tiles in LDS, and picks the tile width so that
// the grid has at least 256 workgroups.
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
};

__device__ __forceinline__ Segment segment_of(const LinearArgs& a, int n0) {
  Segment s = a.seg[0];
  if (a.nseg > 1 && n0 >= a.seg[1].begin) s = a.seg[1];
  if (a.nseg > 2 && n0 >= a.seg[2].begin) s = a.seg[2];
  return s;
}

// Stores one 16 x 16 accumulator block (D layout: lane (r, c) holds rows
// 4r + v, column c) whose top-left output is (m, n).
__device__ __forceinline__ void store_block(const LinearArgs& a, const Segment& s, int m, int n,
                                            const f32x4& acc, int lane) {
  const int r = lane >> 4, c = lane & 15;
  float* col = s.y + (n - s.begin) + c;
  const float* rcol = s.res != nullptr ? s.res + (n - s.begin) + c : nullptr;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t = m + 4 * r + v;
    if (t < a.T) {
      const size_t at = (size_t)t * s.width;
      col[at] = rcol != nullptr ? acc[v] + rcol[at] : acc[v];
    }
  }
}

// ---------------------------------------------------------------- split-k

constexpr int kLinWaves = 8;        // waves per workgroup, each an eighth of k
constexpr int kLinMinGroups = 256;  // aim: one workgroup per compute unit or more

// One workgroup computes a (16 kMB kMW) x (16 kNB) output tile with 8 waves:
// wave w takes row group w mod kMW (16 kMB rows) and k slice w / kMW of
// kKS = 8 / kMW equal slices, with operands loaded straight into registers
// (up to four 32-wide k steps in flight); the kKS partial tiles of each row
// group are added in LDS.  The weight tile is read once per row tile (by the
// kMW row groups together, from L1/L2 after the first).
template <int kMB, int kNB, int kMW>
__global__ __launch_bounds__(kWave * kLinWaves) void linear_splitk_kernel(LinearArgs a) {
  constexpr int kKS = kLinWaves / kMW;
  static_assert(kLinWaves % kMW == 0, "row groups must divide the waves");
  __shared__ f32x4 part[kLinWaves][kMB * kNB][kWave];
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
    xp[mb] = a.x + (size_t)(ok[mb] ? t : 0) * a.K + k_begin + 8 * r;
  }
  const uint16_t* wp[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) wp[nb] = a.w + (size_t)(n0 + 16 * nb + c) * a.K + k_begin + 8 * r;

  struct Step {
    float4 x[kMB][2];
    u32x4 w[kNB];
  };
  // Ordinary (cacheable) loads: row tiles that share a weight tile find it
  // in L2.
  auto load = [&](Step& st, int s) {
    const int k = 32 * s;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) st.w[nb] = *reinterpret_cast<const u32x4*>(wp[nb] + k);
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const float4* q = reinterpret_cast<const float4*>(xp[mb] + k);
      st.x[mb][0] = ok[mb] ? q[0] : make_float4(0.f, 0.f, 0.f, 0.f);
      st.x[mb][1] = ok[mb] ? q[1] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  f32x4 acc[kMB][kNB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const Step& st) {
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      u32x4 hi, lo;
      split8(st.x[mb][0], st.x[mb][1], hi, lo);
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
  __syncthreads();
  // (row group g, block blk) pairs spread over the waves; slice q of row
  // group g is wave g + kMW q.
  const Segment sg = segment_of(a, n0);
  const int m_base = m_tile * 16 * kMB * kMW;
  for (int job = wave; job < kMW * kMB * kNB; job += kLinWaves) {
    const int g = job / (kMB * kNB), blk = job % (kMB * kNB);
    f32x4 t = part[g][blk][lane];
#pragma unroll
    for (int q = 1; q < kKS; ++q) t += part[g + kMW * q][blk][lane];
    store_block(a, sg, m_base + 16 * kMB * g + 16 * (blk / kNB), n0 + 16 * (blk % kNB), t, lane);
  }
}

struct LinearConfig {
  int mb, nb, mw;
};

// Tile shape: the widest of 64, 32, 16 columns (32 rows per tile) that
// still gives kLinMinGroups workgroups, else 16 x 16 tiles.  Swept on MI355X
// over 12 shapes (rows per wave 1-2, columns 1-4 blocks, 1-4 row groups) at
// T = 2 .. 256 and N x K = 4096 x 1024, 1024 x 2048 (graph-replayed launch
// times): this rule picks the fastest shape or one within 3% of it in every
// case.  What the time follows is the traffic from L2: x is read once per
// column tile and w once per row tile, at ~6 TB/s.
LinearConfig pick_config(int T, int N) {
#ifdef DAH_LINEAR_CONFIG
  (void)T; (void)N;
  return LinearConfig{DAH_LINEAR_CONFIG};
#else
  if (T > 16) {
    const int m_tiles = (T + 31) / 32;
    for (int nb = 4; nb >= 1; nb /= 2)
      if (m_tiles * (N / (16 * nb)) >= kLinMinGroups) return {2, nb, 1};
  }
  return {1, 1, 1};
#endif
}

template <int kMB, int kNB, int kMW>
void launch_cfg(const LinearArgs& a, hipStream_t stream) {
  const int rows = 16 * kMB * kMW;
  const dim3 grid(((a.T + rows - 1) / rows) * (a.N / (16 * kNB)));
  linear_splitk_kernel<kMB, kNB, kMW><<<grid, kWave * kLinWaves, 0, stream>>>(a);
}

int launch_linear(LinearArgs& a, hipStream_t stream) {
  const LinearConfig c = pick_config(a.T, a.N);
  // The instantiated shapes; N is a multiple of 64, so every column tiling divides it.
#define DAH_LIN_CASE(MB, NB, MW) \
  if (c.mb == MB && c.nb == NB && c.mw == MW) launch_cfg<MB, NB, MW>(a, stream); else
  DAH_LIN_CASE(1, 1, 1)
  DAH_LIN_CASE(2, 1, 1)
  DAH_LIN_CASE(2, 2, 1)
  DAH_LIN_CASE(2, 4, 1)
#ifdef DAH_LINEAR_CONFIG
  DAH_LIN_CASE(1, 1, 2)
  DAH_LIN_CASE(1, 2, 2)
  DAH_LIN_CASE(1, 4, 2)
  DAH_LIN_CASE(2, 1, 2)
  DAH_LIN_CASE(2, 2, 2)
  DAH_LIN_CASE(2, 4, 2)
  DAH_LIN_CASE(2, 2, 4)
  DAH_LIN_CASE(1, 4, 4)
#endif
  return dah::set_error(DAH_ERR_HIP, "linear: no kernel for tile %d/%d/%d", c.mb, c.nb, c.mw);
#undef DAH_LIN_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dah::set_error(DAH_ERR_HIP, "linear kernel launch failed: %s", hipGetErrorString(e));
  return DAH_OK;
}

}  // namespace

extern "C" {

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

int attn_qkv_proj(const float* x, const void* w_qkv, int T, int hidden, int num_heads, float* q,
                  float* k, float* v, void* stream) {
  if (!q || !k || !v) return dah::set_error(DAH_ERR_NULL, "attn_qkv_proj: an output is NULL");
  if (!dah::valid_heads(num_heads))
    return dah::set_error(DAH_ERR_SHAPE, "num_heads = %d, need 16, 32, 40 or 64", num_heads);
  const int nq = num_heads * dah::kHeadDim, nkv = dah::kKvHeads * dah::kHeadDim;
  int st = dah::validate_linear(x, w_qkv, T, nq + 2 * nkv, hidden, q);
  if (st != DAH_OK) return st;
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) % 16 != 0)
    return dah::set_error(DAH_ERR_ALIGN, "attn_qkv_proj: k and v need 16-byte alignment");
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
  return launch_linear(a, static_cast<hipStream_t>(stream));
}

int attn_o_proj(const float* o, const void* w_o, int T, int num_heads, int hidden, float* y,
                void* stream) {
  if (!dah::valid_heads(num_heads))
    return dah::set_error(DAH_ERR_SHAPE, "num_heads = %d, need 16, 32, 40 or 64", num_heads);
  return dah_linear(o, w_o, T, hidden, num_heads * dah::kHeadDim, y, stream);
}

}  // extern "C"
