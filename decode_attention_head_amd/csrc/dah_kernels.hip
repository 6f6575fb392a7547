// HIP kernels and C entry points of the Qwen3-0.6B decode-attention block
// for MI355X (gfx950, CDNA4, wave64).
//
// Nodes implemented (the "Qwen3-0.6B" Model Spec page, "Compute-graph nodes"):
//   attn.qk_norm + attn.rope + cache store   -> norm_rope_append_kernel
//   attn.core (decodeGQA), split-S           -> decode_split_kernel
//   log-sum-exp merge of the splits          -> combine_splits_kernel
// The split/merge form is exact in real arithmetic by the theorems
// flashAttn_eq and softmax_shift ("Supported models" page, "Facts proved about
// the specs").
//
// Decode design.  The work is HBM-bound: every cached position costs 4 KiB of
// K and V (bf16) and ~1 flop per byte.  One wavefront owns one
// (sequence, KV head, split) and both query heads 2g, 2g+1 of that KV head.
// A (page, KV head) tile is 16 positions x 128 dims, contiguous (4 KiB bf16).
// Lane l = 16*r + c holds dims 8c..8c+7 of positions 4j+r, j = 0..3: each of
// the four 16-byte loads per tile is a fully coalesced 1 KiB wave access.
// Dot products finish with a 16-lane DPP reduction inside each row of the
// wave; each row r keeps its own online-softmax state (max, sum, 8 weighted-V
// accumulators per head) over positions = r mod 4, and the four rows are
// merged once at the end.  The next page's K and V are loaded into a second
// register set while the current one is consumed.  No LDS is used.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "dah.h"
#include "dah_host.h"

namespace {

using dah::kHeadDim;
using dah::kHeads;
using dah::kKvHeads;
using dah::kPage;

constexpr int kWave = 64;
constexpr int kDecodeWavesPerBlock = 8;  // the 8 KV heads of one (sequence, split)
constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------ lane utilities

// Sum over the 16 lanes of a row; every lane of the row gets the same bits.
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum16(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ------------------------------------------------------------ cache tiles

// One (page, KV head) tile held in registers: this lane's 8 dims of the 4
// positions 4j + r.
template <int kDtype>
struct Tile;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <>
struct Tile<DAH_BF16> {
  static constexpr int64_t kTileBytes = kPage * kHeadDim * 2;
  u32x4 w[4];
  __device__ __forceinline__ void load(const char* tile, int lane) {
    const u32x4* p = reinterpret_cast<const u32x4*>(tile) + lane;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = __builtin_nontemporal_load(p + j * kWave);
  }
  __device__ __forceinline__ float get(int j, int e) const {
    const uint32_t x = w[j][e >> 1];
    return (e & 1) ? bf16_hi(x) : bf16_lo(x);
  }
  __device__ __forceinline__ void clear(int j) { w[j] = u32x4{0u, 0u, 0u, 0u}; }
};

template <>
struct Tile<DAH_F32> {
  static constexpr int64_t kTileBytes = kPage * kHeadDim * 4;
  u32x4 w[8];
  __device__ __forceinline__ void load(const char* tile, int lane) {
    const u32x4* p = reinterpret_cast<const u32x4*>(tile) + 2 * lane;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[2 * j] = __builtin_nontemporal_load(p + j * 2 * kWave);
      w[2 * j + 1] = __builtin_nontemporal_load(p + j * 2 * kWave + 1);
    }
  }
  __device__ __forceinline__ float get(int j, int e) const {
    return __uint_as_float(w[2 * j + (e >> 2)][e & 3]);
  }
  __device__ __forceinline__ void clear(int j) {
    w[2 * j] = u32x4{0u, 0u, 0u, 0u};
    w[2 * j + 1] = u32x4{0u, 0u, 0u, 0u};
  }
};

// Online-softmax state of one query head in one row of the wave: running
// max (log2 units), running sum of weights, and this lane's 8 accumulators.
struct HeadState {
  float m, l;
  float acc[8];
  __device__ __forceinline__ void init() {
    m = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  }
};

// Softmax bookkeeping for one head over this row's 4 scores of a page.
// Returns the rescale factor of the old state; p[] receives the weights.
template <bool kMasked>
__device__ __forceinline__ float softmax_update(HeadState& st, const float (&s)[4], float (&p)[4]) {
  const float pm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  const float mn = fmaxf(st.m, pm);
  // In a masked page a row may have seen no valid position yet: keep the
  // reference finite so that exp2 gives 0 instead of NaN.
  const float mu = (kMasked && mn == -INFINITY) ? 0.0f : mn;
  const float alpha = fast_exp2(st.m - mu);
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = fast_exp2(s[j] - mu);
  st.l = fmaf(st.l, alpha, (p[0] + p[1]) + (p[2] + p[3]));
  st.m = mn;
  return alpha;
}

// Consume one (page, KV head) tile for the two query heads.
template <int kDtype, bool kMasked>
__device__ __forceinline__ void attend_tile(const Tile<kDtype>& K, Tile<kDtype>& V,
                                            const float (&qa)[8], const float (&qb)[8],
                                            HeadState& A, HeadState& Bs, int row, int nvalid) {
  float sa[4], sb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float pa = 0.0f, pb = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float k = K.get(j, e);
      pa = fmaf(qa[e], k, pa);
      pb = fmaf(qb[e], k, pb);
    }
    sa[j] = row_sum16(pa);
    sb[j] = row_sum16(pb);
    if (kMasked) {
      // Positions at or past seq_len may hold anything (NaN included): the
      // select keeps them out of both the scores and the V sum.
      const bool ok = (4 * j + row) < nvalid;
      sa[j] = ok ? sa[j] : -INFINITY;
      sb[j] = ok ? sb[j] : -INFINITY;
      if (!ok) V.clear(j);
    }
  }
  float wa[4], wb[4];
  const float ala = softmax_update<kMasked>(A, sa, wa);
  const float alb = softmax_update<kMasked>(Bs, sb, wb);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    A.acc[e] *= ala;
    Bs.acc[e] *= alb;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = V.get(j, e);
      A.acc[e] = fmaf(wa[j], v, A.acc[e]);
      Bs.acc[e] = fmaf(wb[j], v, Bs.acc[e]);
    }
  }
}

// Merge the four rows' states of a head; afterwards every row holds the total.
__device__ __forceinline__ void merge_rows(HeadState& st) {
  float M = fmaxf(st.m, __shfl_xor(st.m, 16));
  M = fmaxf(M, __shfl_xor(M, 32));
  const float mu = (M == -INFINITY) ? 0.0f : M;
  const float f = fast_exp2(st.m - mu);
  float l = st.l * f;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float a = st.acc[e] * f;
    a += __shfl_xor(a, 16);
    a += __shfl_xor(a, 32);
    st.acc[e] = a;
  }
  st.m = M;
  st.l = l;
}

struct DecodeArgs {
  const float* q;
  const char* k_cache;
  const char* v_cache;
  int num_pages;
  const int32_t* block_table;
  int max_pages_per_seq;
  const int32_t* seq_lens;
  int B;
  int max_seq_len;
  int splits;
  int pages_per_split;
  float* o;         // written when splits == 1
  float* part_acc;  // [B][16][splits][128] when splits > 1
  float* part_ml;   // [B][16][splits][2]   when splits > 1
};

__device__ __forceinline__ void store8(float* dst, const float (&v)[8], float scale) {
  float4* d = reinterpret_cast<float4*>(dst);
  d[0] = make_float4(v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale);
  d[1] = make_float4(v[4] * scale, v[5] * scale, v[6] * scale, v[7] * scale);
}

template <int kDtype>
__global__ __launch_bounds__(kWave * kDecodeWavesPerBlock) void decode_split_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  // The wave index is uniform across the wave; saying so keeps everything
  // derived from it (sequence, page range, page addresses) in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x * kDecodeWavesPerBlock + wave;
  const int g = unit & (kKvHeads - 1);
  const int bs = unit >> 3;  // b + B * split
  if (bs >= a.B * a.splits) return;
  const int b = bs % a.B;
  const int split = bs / a.B;
  const int row = lane >> 4;
  const int col = lane & 15;

  const int seq_len = a.seq_lens[b];
  const bool len_ok = seq_len >= 1 && seq_len <= a.max_seq_len;
  const int npages = len_ok ? (seq_len + kPage - 1) / kPage : 0;
  const int p0 = split * a.pages_per_split;
  const int p1 = min(p0 + a.pages_per_split, npages);

  if (p0 >= p1) {
    // Empty range.  With one split this is the whole sequence: o = 0 for
    // seq_len <= 0, NaN for a length past max_seq_len.  With several splits
    // the combine kernel reads only non-empty ranges.
    if (a.splits == 1 && row < 2) {
      const float fill = seq_len <= 0 ? 0.0f : NAN;
      const float z[8] = {fill, fill, fill, fill, fill, fill, fill, fill};
      store8(a.o + ((size_t)b * kHeads + 2 * g + row) * kHeadDim + 8 * col, z, 1.0f);
    }
    return;
  }

  // Query rows 2g and 2g+1, this lane's 8 dims, pre-scaled by log2(e)/sqrt(128)
  // so that scores come out in log2 units for exp2.
  const float qscale = kLog2e * 0.08838834764831845f;  // 1/sqrt(128)
  float qa[8], qb[8];
  {
    const float4* qp = reinterpret_cast<const float4*>(a.q + ((size_t)b * kHeads + 2 * g) * kHeadDim + 8 * col);
    const float4 a0 = qp[0], a1 = qp[1];
    const float4 b0 = qp[kHeadDim / 4], b1 = qp[kHeadDim / 4 + 1];
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qa[e] = av[e] * qscale;
      qb[e] = bv[e] * qscale;
    }
  }

  HeadState A, Bs;
  A.init();
  Bs.init();

  // The block table is read-only for the whole launch: reading it through the
  // constant address space makes every (uniform) read a scalar load, counted
  // apart from the vector loads of the cache tiles.
  typedef const __attribute__((address_space(4))) int32_t* ConstI32;
  const ConstI32 bt = (ConstI32)(a.block_table + (size_t)b * a.max_pages_per_seq);
  const char* kbase = a.k_cache + (int64_t)g * Tile<kDtype>::kTileBytes;
  const char* vbase = a.v_cache + (int64_t)g * Tile<kDtype>::kTileBytes;
  const int64_t page_bytes = (int64_t)kKvHeads * Tile<kDtype>::kTileBytes;
  const int tail = seq_len - (npages - 1) * kPage;  // valid slots in the sequence's last page
  const int last = p1 - 1;                           // last page of this wave's range
  const bool last_masked = (last == npages - 1) && tail < kPage;
  bool bad_page = false;

  // Physical page ids come from scalar loads issued two pages before the
  // tile they address; an id is range-checked only when its tile is loaded.
  // An id outside the pool is replaced by page 0 and flags the sequence (its
  // output becomes NaN).
  auto offset_of = [&](int id) -> int64_t {
    const bool ok = id >= 0 && id < a.num_pages;
    bad_page |= !ok;
    return (int64_t)(ok ? id : 0) * page_bytes;
  };

  // Software pipeline over the pages: the tile of page p+1 is in flight while
  // page p is consumed.  In the steady-state loop both following pages exist,
  // so every load is unconditional; the scheduling barriers keep each tile's
  // eight loads together and ahead of the math on the other tile, so the wait
  // before a tile covers only its own loads.  The last one or two pages (the
  // only place a partial page can be) are finished after the loop.
  Tile<kDtype> K0, V0, K1, V1;
  int id1 = bt[min(p0 + 1, last)];
  int id2 = bt[min(p0 + 2, last)];
  {
    const int64_t off0 = offset_of(bt[p0]);
    K0.load(kbase + off0, lane);
    V0.load(vbase + off0, lane);
  }
  int p = p0;
  for (; p + 2 <= last; p += 2) {
    const int64_t off1 = offset_of(id1);
    K1.load(kbase + off1, lane);
    V1.load(vbase + off1, lane);
    const int id3 = bt[min(p + 3, last)];
    __builtin_amdgcn_sched_barrier(0);
    attend_tile<kDtype, false>(K0, V0, qa, qb, A, Bs, row, kPage);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t off2 = offset_of(id2);
    K0.load(kbase + off2, lane);
    V0.load(vbase + off2, lane);
    const int id4 = bt[min(p + 4, last)];
    __builtin_amdgcn_sched_barrier(0);
    attend_tile<kDtype, false>(K1, V1, qa, qb, A, Bs, row, kPage);
    __builtin_amdgcn_sched_barrier(0);
    id1 = id3;
    id2 = id4;
  }
  if (p + 1 <= last) {
    const int64_t off1 = offset_of(id1);
    K1.load(kbase + off1, lane);
    V1.load(vbase + off1, lane);
    attend_tile<kDtype, false>(K0, V0, qa, qb, A, Bs, row, kPage);
    if (last_masked)
      attend_tile<kDtype, true>(K1, V1, qa, qb, A, Bs, row, tail);
    else
      attend_tile<kDtype, false>(K1, V1, qa, qb, A, Bs, row, kPage);
  } else {
    if (last_masked)
      attend_tile<kDtype, true>(K0, V0, qa, qb, A, Bs, row, tail);
    else
      attend_tile<kDtype, false>(K0, V0, qa, qb, A, Bs, row, kPage);
  }

  merge_rows(A);
  merge_rows(Bs);
  if (bad_page) {
    A.l = NAN;
    Bs.l = NAN;
  }

  if (row < 2) {
    const HeadState& st = row == 0 ? A : Bs;
    const int h = 2 * g + row;
    if (a.splits == 1) {
      store8(a.o + ((size_t)b * kHeads + h) * kHeadDim + 8 * col, st.acc, 1.0f / st.l);
    } else {
      const size_t part = ((size_t)b * kHeads + h) * a.splits + split;
      store8(a.part_acc + part * kHeadDim + 8 * col, st.acc, bad_page ? NAN : 1.0f);
      if (col == 0) reinterpret_cast<float2*>(a.part_ml)[part] = make_float2(st.m, st.l);
    }
  }
}

// One wave per (sequence, query head): merge the non-empty split ranges.
//   M = max_s m_s,  w_s = 2^(m_s - M),  o = sum_s w_s acc_s / sum_s w_s l_s
__global__ __launch_bounds__(256) void combine_splits_kernel(const float* __restrict__ part_acc,
                                                             const float* __restrict__ part_ml,
                                                             const int32_t* __restrict__ seq_lens,
                                                             int B, int max_seq_len, int splits,
                                                             int pages_per_split,
                                                             float* __restrict__ o) {
  const int lane = threadIdx.x & (kWave - 1);
  const int unit = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (unit >= B * kHeads) return;
  const int b = unit / kHeads;
  const int seq_len = seq_lens[b];
  float2* out = reinterpret_cast<float2*>(o + (size_t)unit * kHeadDim) + lane;
  if (seq_len < 1 || seq_len > max_seq_len) {
    const float fill = seq_len < 1 ? 0.0f : NAN;
    *out = make_float2(fill, fill);
    return;
  }
  const int npages = (seq_len + kPage - 1) / kPage;
  const int nsplit = (npages + pages_per_split - 1) / pages_per_split;
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + (size_t)unit * splits;
  const float2* acc = reinterpret_cast<const float2*>(part_acc + (size_t)unit * splits * kHeadDim) + lane;

  float M = -INFINITY;
  for (int s = lane; s < nsplit; s += kWave) M = fmaxf(M, ml[s].x);
  M = fmaxf(M, __shfl_xor(M, 1));
  M = fmaxf(M, __shfl_xor(M, 2));
  M = fmaxf(M, __shfl_xor(M, 4));
  M = fmaxf(M, __shfl_xor(M, 8));
  M = fmaxf(M, __shfl_xor(M, 16));
  M = fmaxf(M, __shfl_xor(M, 32));

  float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int s = 0; s < nsplit; ++s) {
    const float2 m_l = ml[s];
    const float w = fast_exp2(m_l.x - M);
    const float2 v = acc[(size_t)s * (kHeadDim / 2)];
    L = fmaf(w, m_l.y, L);
    o0 = fmaf(w, v.x, o0);
    o1 = fmaf(w, v.y, o1);
  }
  const float inv = 1.0f / L;
  *out = make_float2(o0 * inv, o1 * inv);
}

// ------------------------------------------------------------ norm + RoPE + append

struct AppendArgs {
  const float* q;
  const float* k_new;
  const float* v_new;
  const float* q_gain;
  const float* k_gain;
  float eps;
  double log2_theta;
  char* k_cache;
  char* v_cache;
  int num_pages;
  const int32_t* block_table;
  int max_pages_per_seq;
  const int32_t* seq_lens;
  int max_len;  // longest sequence the caller allows (append skipped past it)
  float* q_out;
};

// RMSNorm of one 128-vector held as (x0 = dim lane, x1 = dim lane + 64):
// x / sqrt(sum x^2 / 128 + eps) * w.  The sum is a wave-wide tree reduction,
// which equals the spec's sum up to rounding order (theorem rmsNormTiled_eq,
// "Supported models" page).
__device__ __forceinline__ void rms_norm(float& x0, float& x1, const float* w, float eps, int lane) {
  const float ss = wave_sum(fmaf(x0, x0, x1 * x1));
  const float inv = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);
  x0 = x0 * inv * w[lane];
  x1 = x1 * inv * w[lane + 64];
}

__device__ __forceinline__ void rotate(float& x0, float& x1, float c, float s) {
  const float y0 = x0 * c - x1 * s;
  const float y1 = x0 * s + x1 * c;
  x0 = y0;
  x1 = y1;
}

// One block of 8 waves per sequence.  Wave w handles query heads w and w+8,
// key head w and value head w; lane i holds dims i and i+64 (a RoPE pair).
template <int kDtype>
__global__ __launch_bounds__(512) void norm_rope_append_kernel(AppendArgs a) {
  __shared__ float2 cs[64];
  const int b = blockIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & (kWave - 1);
  const int seq_len = a.seq_lens[b];
  const int pos = seq_len >= 1 ? seq_len - 1 : 0;
  if (w == 0) {
    // Angle pos * theta^(-2i/128) and its cos/sin in float64 (at pos near
    // 40,960 a float32 angle would be off by ~4e-3 rad).
    const double inv_freq = exp2(-(double)lane / 64.0 * a.log2_theta);
    double sn, cn;
    sincos((double)pos * inv_freq, &sn, &cn);
    cs[lane] = make_float2((float)cn, (float)sn);
  }
  // Load while wave 0 computes the angles.
  const size_t qbase0 = ((size_t)b * kHeads + w) * kHeadDim;
  const size_t qbase1 = ((size_t)b * kHeads + w + 8) * kHeadDim;
  const size_t kvbase = ((size_t)b * kKvHeads + w) * kHeadDim;
  float q0a = a.q[qbase0 + lane], q0b = a.q[qbase0 + lane + 64];
  float q1a = a.q[qbase1 + lane], q1b = a.q[qbase1 + lane + 64];
  float ka = a.k_new[kvbase + lane], kb = a.k_new[kvbase + lane + 64];
  const float va = a.v_new[kvbase + lane], vb = a.v_new[kvbase + lane + 64];
  __syncthreads();
  const float2 r = cs[lane];

  rms_norm(q0a, q0b, a.q_gain, a.eps, lane);
  rms_norm(q1a, q1b, a.q_gain, a.eps, lane);
  rms_norm(ka, kb, a.k_gain, a.eps, lane);
  rotate(q0a, q0b, r.x, r.y);
  rotate(q1a, q1b, r.x, r.y);
  rotate(ka, kb, r.x, r.y);
  a.q_out[qbase0 + lane] = q0a;
  a.q_out[qbase0 + lane + 64] = q0b;
  a.q_out[qbase1 + lane] = q1a;
  a.q_out[qbase1 + lane + 64] = q1b;

  if (seq_len < 1 || seq_len > a.max_len) return;
  const int page = a.block_table[(size_t)b * a.max_pages_per_seq + pos / kPage];
  if (page < 0 || page >= a.num_pages) return;
  const size_t elem = (((size_t)page * kKvHeads + w) * kPage + (pos % kPage)) * kHeadDim;
  if (kDtype == DAH_BF16) {
    uint16_t* kc = reinterpret_cast<uint16_t*>(a.k_cache) + elem;
    uint16_t* vc = reinterpret_cast<uint16_t*>(a.v_cache) + elem;
    kc[lane] = to_bf16(ka);
    kc[lane + 64] = to_bf16(kb);
    vc[lane] = to_bf16(va);
    vc[lane + 64] = to_bf16(vb);
  } else {
    float* kc = reinterpret_cast<float*>(a.k_cache) + elem;
    float* vc = reinterpret_cast<float*>(a.v_cache) + elem;
    kc[lane] = ka;
    kc[lane + 64] = kb;
    vc[lane] = va;
    vc[lane + 64] = vb;
  }
}

// ------------------------------------------------------------ host side

std::atomic<int> g_cu_count[64];

int device_cu_count(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return dah::set_error(DAH_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  int cached = (dev >= 0 && dev < 64) ? g_cu_count[dev].load(std::memory_order_relaxed) : 0;
  if (cached > 0) {
    *out = cached;
    return DAH_OK;
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || n < 1)
    return dah::set_error(DAH_ERR_HIP, "compute-unit count of device %d: %s", dev,
                          hipGetErrorString(e));
  if (dev >= 0 && dev < 64) g_cu_count[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return DAH_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dah::set_error(DAH_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return DAH_OK;
}

int launch_append(const float* q, const float* k_new, const float* v_new, const float* q_gain,
                  const float* k_gain, float eps, float rope_theta, void* k_cache, void* v_cache,
                  int cache_dtype, int64_t num_pages, const int32_t* block_table,
                  int max_pages_per_seq, const int32_t* seq_lens, int B, int max_len,
                  float* q_out, hipStream_t stream) {
  AppendArgs a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.q_gain = q_gain;
  a.k_gain = k_gain;
  a.eps = eps;
  a.log2_theta = log2((double)rope_theta);
  a.k_cache = static_cast<char*>(k_cache);
  a.v_cache = static_cast<char*>(v_cache);
  a.num_pages = static_cast<int>(num_pages);
  a.block_table = block_table;
  a.max_pages_per_seq = max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.max_len = max_len;
  a.q_out = q_out;
  if (cache_dtype == DAH_BF16)
    norm_rope_append_kernel<DAH_BF16><<<B, 512, 0, stream>>>(a);
  else
    norm_rope_append_kernel<DAH_F32><<<B, 512, 0, stream>>>(a);
  return check_launch("norm_rope_append_kernel");
}

int launch_decode(const float* q, const void* k_cache, const void* v_cache, int cache_dtype,
                  int64_t num_pages, const int32_t* block_table, int max_pages_per_seq,
                  const int32_t* seq_lens, int B, int max_seq_len, int num_splits, float* o,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int cus = 0;
  int st = device_cu_count(&cus);
  if (st != DAH_OK) return st;
  dah::Plan plan;
  st = dah::plan_splits(B, max_seq_len, num_splits, cus, &plan);
  if (st != DAH_OK) return st;
  if (plan.workspace > 0) {
    if (workspace == nullptr || workspace_bytes < plan.workspace)
      return dah::set_error(DAH_ERR_WORKSPACE,
                            "workspace of %zu bytes, need %zu (B=%d, max_seq_len=%d, %d splits)",
                            workspace == nullptr ? (size_t)0 : workspace_bytes, plan.workspace, B,
                            max_seq_len, plan.splits);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return dah::set_error(DAH_ERR_ALIGN, "workspace needs 256-byte alignment");
  }
  DecodeArgs a;
  a.q = q;
  a.k_cache = static_cast<const char*>(k_cache);
  a.v_cache = static_cast<const char*>(v_cache);
  a.num_pages = static_cast<int>(num_pages);
  a.block_table = block_table;
  a.max_pages_per_seq = max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.B = B;
  a.max_seq_len = max_seq_len;
  a.splits = plan.splits;
  a.pages_per_split = plan.pages_per_split;
  a.o = o;
  float* ws = static_cast<float*>(workspace);
  const size_t parts = (size_t)B * kHeads * plan.splits;
  a.part_acc = plan.splits > 1 ? ws : nullptr;
  a.part_ml = plan.splits > 1 ? ws + parts * kHeadDim : nullptr;

  const long long waves = (long long)B * kKvHeads * plan.splits;
  const long long blocks = (waves + kDecodeWavesPerBlock - 1) / kDecodeWavesPerBlock;
  if (blocks > INT32_MAX) return dah::set_error(DAH_ERR_SHAPE, "grid too large");
  if (cache_dtype == DAH_BF16)
    decode_split_kernel<DAH_BF16><<<(unsigned)blocks, kWave * kDecodeWavesPerBlock, 0, stream>>>(a);
  else
    decode_split_kernel<DAH_F32><<<(unsigned)blocks, kWave * kDecodeWavesPerBlock, 0, stream>>>(a);
  st = check_launch("decode_split_kernel");
  if (st != DAH_OK || plan.splits == 1) return st;
  const int cblocks = (B * kHeads + 3) / 4;
  combine_splits_kernel<<<cblocks, 256, 0, stream>>>(a.part_acc, a.part_ml, seq_lens, B,
                                                     max_seq_len, plan.splits,
                                                     plan.pages_per_split, o);
  return check_launch("combine_splits_kernel");
}

}  // namespace

extern "C" {

int qk_norm_rope_append(const float* q, const float* k_new, const float* v_new,
                        const float* q_gain, const float* k_gain, float eps, float rope_theta,
                        void* k_cache, void* v_cache, int cache_dtype, int64_t num_pages,
                        const int32_t* block_table, int max_pages_per_seq,
                        const int32_t* seq_lens, int B, float* q_out, void* stream) {
  int st = dah::validate_append(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache,
                                v_cache, cache_dtype, num_pages, block_table, max_pages_per_seq,
                                seq_lens, B, q_out);
  if (st != DAH_OK) return st;
  const long long max_len = (long long)max_pages_per_seq * kPage;
  return launch_append(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache, v_cache,
                       cache_dtype, num_pages, block_table, max_pages_per_seq, seq_lens, B,
                       max_len > INT32_MAX ? INT32_MAX : (int)max_len, q_out,
                       static_cast<hipStream_t>(stream));
}

int paged_decode_gqa(const float* q, const void* k_cache, const void* v_cache, int cache_dtype,
                     int64_t num_pages, const int32_t* block_table, int max_pages_per_seq,
                     const int32_t* seq_lens, int B, int max_seq_len, int num_splits, float* o,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int st = dah::validate_decode(q, k_cache, v_cache, cache_dtype, num_pages, block_table,
                                max_pages_per_seq, seq_lens, B, max_seq_len, num_splits, o);
  if (st != DAH_OK) return st;
  return launch_decode(q, k_cache, v_cache, cache_dtype, num_pages, block_table,
                       max_pages_per_seq, seq_lens, B, max_seq_len, num_splits, o, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream));
}

int decode_attn_step(const float* q, const float* k_new, const float* v_new,
                     const float* q_gain, const float* k_gain, float eps, float rope_theta,
                     void* k_cache, void* v_cache, int cache_dtype, int64_t num_pages,
                     const int32_t* block_table, int max_pages_per_seq,
                     const int32_t* seq_lens, int B, int max_seq_len, int num_splits,
                     float* q_out, float* o, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int st = dah::validate_append(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache,
                                v_cache, cache_dtype, num_pages, block_table, max_pages_per_seq,
                                seq_lens, B, q_out);
  if (st != DAH_OK) return st;
  st = dah::validate_decode(q_out, k_cache, v_cache, cache_dtype, num_pages, block_table,
                            max_pages_per_seq, seq_lens, B, max_seq_len, num_splits, o);
  if (st != DAH_OK) return st;
  // Check the workspace before anything is launched, so that a failing call
  // leaves the cache untouched.
  int cus = 0;
  st = device_cu_count(&cus);
  if (st != DAH_OK) return st;
  dah::Plan plan;
  st = dah::plan_splits(B, max_seq_len, num_splits, cus, &plan);
  if (st != DAH_OK) return st;
  if (plan.workspace > 0 && (workspace == nullptr || workspace_bytes < plan.workspace))
    return dah::set_error(DAH_ERR_WORKSPACE, "workspace of %zu bytes, need %zu",
                          workspace == nullptr ? (size_t)0 : workspace_bytes, plan.workspace);
  if (plan.workspace > 0 && reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return dah::set_error(DAH_ERR_ALIGN, "workspace needs 256-byte alignment");
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_append(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache, v_cache,
                     cache_dtype, num_pages, block_table, max_pages_per_seq, seq_lens, B,
                     max_seq_len, q_out, s);
  if (st != DAH_OK) return st;
  return launch_decode(q_out, k_cache, v_cache, cache_dtype, num_pages, block_table,
                       max_pages_per_seq, seq_lens, B, max_seq_len, num_splits, o, workspace,
                       workspace_bytes, s);
}

size_t dah_workspace_bytes(int B, int max_seq_len, int num_splits) {
  int cus = 0;
  if (device_cu_count(&cus) != DAH_OK) return 0;
  return dah_workspace_bytes_for(B, max_seq_len, num_splits, cus);
}

}  // extern "C"
