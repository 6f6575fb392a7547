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
#include "dah_rope.h"

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

// Words of one cached position for one lane (8 dims) in the cache's dtype.
template <int kDtype>
struct SlotWords {
  static constexpr int kWords = kDtype == DAH_BF16 ? 1 : 2;
  u32x4 w[kWords];
};

template <int kDtype>
__device__ __forceinline__ void unpack_slot(const SlotWords<kDtype>& s, float (&x)[8]) {
  if constexpr (kDtype == DAH_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(s.w[0][i]);
      x[2 * i + 1] = bf16_hi(s.w[0][i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __uint_as_float(s.w[0][i]);
      x[4 + i] = __uint_as_float(s.w[1][i]);
    }
  }
}

template <int kDtype>
__device__ __forceinline__ SlotWords<kDtype> pack_slot(const float (&x)[8]) {
  SlotWords<kDtype> s;
  if constexpr (kDtype == DAH_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s.w[0][i] = (uint32_t)to_bf16(x[2 * i]) | ((uint32_t)to_bf16(x[2 * i + 1]) << 16);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s.w[0][i] = __float_as_uint(x[i]);
      s.w[1][i] = __float_as_uint(x[4 + i]);
    }
  }
  return s;
}

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

// Online-softmax update with one position (score s in log2 units, this
// lane's 8 dims of v); rows that do not own the position pass s = -inf.
__device__ __forceinline__ void attend_one(HeadState& st, float s, const float (&v)[8]) {
  const float mn = fmaxf(st.m, s);
  const float mu = mn == -INFINITY ? 0.0f : mn;
  const float alpha = fast_exp2(st.m - mu);
  const float p = fast_exp2(s - mu);
  st.l = fmaf(st.l, alpha, p);
#pragma unroll
  for (int e = 0; e < 8; ++e) st.acc[e] = fmaf(p, v[e], st.acc[e] * alpha);
  st.m = mn;
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

// ---------------------------------------------------------- norm + RoPE, row layout
//
// In the decode layout lane (row r, column c) holds dims 8c..8c+7 of a head,
// the same in all four rows.  The RoPE partner of dim i < 64 is dim i + 64,
// held by column c + 8 of the same row, so pairs meet with one DPP rotation
// of the row by 8 lanes.

// cos/sin of pos * theta^(-2i/128) for this lane's eight pair indices
// i = 8 (c mod 8) + e.  Each lane forms one of the 64 angles (dah_rope.h:
// float64 angle, Cody-Waite reduction; a float32 angle at pos ~ 40,959 would
// be off by ~4e-3 rad); shuffles hand every lane the eight it needs.
__device__ __forceinline__ void rope_table(int pos, const dah::RopePowers& rp, int lane, int col,
                                           float (&c)[8], float (&s)[8]) {
  float cf, sf;
  dah::rope_cos_sin((double)pos * dah::rope_inv_freq(lane, rp), &cf, &sf);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int src = 8 * (col & 7) + e;
    c[e] = __shfl(cf, src);
    s[e] = __shfl(sf, src);
  }
}

// RMSNorm of one head held in the row layout (x / sqrt(sum x^2 / 128 + eps) * w,
// the sum as a 16-lane DPP tree, which theorem rmsNormTiled_eq of the
// "Supported models" page equates with the spec's sum), then the rotation of
// the pairs (i, i + 64).
__device__ __forceinline__ void norm_rope_row(float (&x)[8], const float (&w)[8], float eps,
                                              const float (&c)[8], const float (&s)[8], int col) {
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
  ss = row_sum16(ss);
  const float inv = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);
  float y[8], partner[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = x[e] * inv * w[e];
#pragma unroll
  for (int e = 0; e < 8; ++e)  // row_ror:8 -- column c reads column c +- 8
    partner[e] = __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(y[e]), 0x128, 0xF, 0xF, false));
  const bool upper = col >= 8;  // this lane holds dims i + 64
#pragma unroll
  for (int e = 0; e < 8; ++e)
    x[e] = upper ? partner[e] * s[e] + y[e] * c[e] : y[e] * c[e] - partner[e] * s[e];
}

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a0 = reinterpret_cast<const float4*>(p)[0];
  const float4 a1 = reinterpret_cast<const float4*>(p)[1];
  v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
  v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
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
  // The fused step only: q above is the raw (pre-norm) query.
  const float* k_new;
  const float* v_new;
  const float* q_gain;
  const float* k_gain;
  float eps;
  dah::RopePowers rope;
  float* q_out;
  char* k_cache_w;  // the pools again, writable (same addresses as k_cache / v_cache)
  char* v_cache_w;
};

__device__ __forceinline__ void store8(float* dst, const float (&v)[8], float scale) {
  float4* d = reinterpret_cast<float4*>(dst);
  d[0] = make_float4(v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale);
  d[1] = make_float4(v[4] * scale, v[5] * scale, v[6] * scale, v[7] * scale);
}

// decodeGQA over one split of one sequence, for the 8 KV heads (one wave each).
// kStep: the fused decode step -- q arrives raw and is normed and rotated here
// (split 0 also writes q_out), and the workgroup holding the sequence's last
// page norms and rotates the new key, stores the new key and value in the
// cache and uses them for that slot directly from registers.
template <int kDtype, bool kStep>
__global__ __launch_bounds__(kWave * kDecodeWavesPerBlock) void decode_split_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  // The wave index is uniform across the wave; saying so keeps everything
  // derived from it (sequence, page range, page addresses) in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x * kDecodeWavesPerBlock + wave;
  const int g = unit & (kKvHeads - 1);
  const int bs = unit >> 3;  // b + B * split, the same for the whole workgroup
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
  const bool empty = p0 >= p1;

  // Empty range.  With one split this is the whole sequence: o = 0 for
  // seq_len <= 0, NaN for a length past max_seq_len.  With several splits the
  // combine kernel reads only non-empty ranges.  (In the fused step, split 0
  // still has to write q_out first.)
  auto fill_empty_output = [&]() {
    if (a.splits == 1 && row < 2) {
      const float fill = seq_len <= 0 ? 0.0f : NAN;
      const float z[8] = {fill, fill, fill, fill, fill, fill, fill, fill};
      store8(a.o + ((size_t)b * kHeads + 2 * g + row) * kHeadDim + 8 * col, z, 1.0f);
    }
  };
  if (empty && !(kStep && split == 0)) {
    fill_empty_output();
    return;
  }

  // The block table is read-only for the whole launch: reading it through the
  // constant address space makes every (uniform) read a scalar load, counted
  // apart from the vector loads of the cache tiles.
  typedef const __attribute__((address_space(4))) int32_t* ConstI32;
  const ConstI32 bt = (ConstI32)(a.block_table + (size_t)b * a.max_pages_per_seq);
  const int64_t page_bytes = (int64_t)kKvHeads * Tile<kDtype>::kTileBytes;
  const int64_t head_bytes = (int64_t)g * Tile<kDtype>::kTileBytes;
  const char* kbase = a.k_cache + head_bytes;
  const char* vbase = a.v_cache + head_bytes;
  const int tail = seq_len - (npages - 1) * kPage;  // valid slots in the sequence's last page
  const int last = p1 - 1;                           // last page of this wave's range
  // In the fused step the last page's final slot is the new token, which is
  // taken from registers, so only tail - 1 of its slots are read from the cache.
  const bool step_last = kStep && p1 == npages && !empty;
  const int last_valid = step_last ? tail - 1 : tail;
  const bool last_masked = (last == npages - 1) && last_valid < kPage;
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

  // The small per-wave loads go first: vector loads complete in order, so the
  // prologue's wait for them must not also wait for the first tile.
  // Query rows 2g and 2g+1, this lane's 8 dims (raw in the fused step).
  float qa[8], qb[8];
  load8(a.q + ((size_t)b * kHeads + 2 * g) * kHeadDim + 8 * col, qa);
  load8(a.q + ((size_t)b * kHeads + 2 * g + 1) * kHeadDim + 8 * col, qb);
  const bool holds_last = step_last;
  float qw[8], kx[8], vx[8], kw8[8];
  if constexpr (kStep) {
    load8(a.q_gain + 8 * col, qw);
    if (holds_last) {
      load8(a.k_new + ((size_t)b * kKvHeads + g) * kHeadDim + 8 * col, kx);
      load8(a.v_new + ((size_t)b * kKvHeads + g) * kHeadDim + 8 * col, vx);
      load8(a.k_gain + 8 * col, kw8);
    }
  }

  // First tile in flight before the prologue's arithmetic.
  Tile<kDtype> K0, V0, K1, V1;
  int id1 = 0, id2 = 0;
  if (!empty) {
    id1 = bt[min(p0 + 1, last)];
    id2 = bt[min(p0 + 2, last)];
    const int64_t off0 = offset_of(bt[p0]);
    K0.load(kbase + off0, lane);
    V0.load(vbase + off0, lane);
  }

  // The fused step's outputs besides o -- q_out rows and the new token's key
  // and value in the cache dtype -- wait in LDS (per wave, written and read
  // by that wave only) and go to memory after the page loop: one counter
  // tracks vector loads and stores in issue order, so a store issued early
  // would hold up the waits for the first tiles.
  __shared__ u32x4 stash[kDecodeWavesPerBlock][2][2][16];   // [wave][k|v][word][column]
  __shared__ float4 qstash[kDecodeWavesPerBlock][2][2][16];  // [wave][head][half][column]
  if constexpr (kStep) {
    const int pos = seq_len >= 1 ? seq_len - 1 : 0;
    float cr[8], sr[8];
    rope_table(pos, a.rope, lane, col, cr, sr);
    norm_rope_row(qa, qw, a.eps, cr, sr, col);
    norm_rope_row(qb, qw, a.eps, cr, sr, col);
    if (split == 0 && row < 2) {
      const float (&q)[8] = row == 0 ? qa : qb;
      qstash[wave][row][0][col] = make_float4(q[0], q[1], q[2], q[3]);
      qstash[wave][row][1][col] = make_float4(q[4], q[5], q[6], q[7]);
    }
    if (empty) {
      if (split == 0 && row < 2) {
        float* qo = a.q_out + ((size_t)b * kHeads + 2 * g + row) * kHeadDim + 8 * col;
        reinterpret_cast<float4*>(qo)[0] = qstash[wave][row][0][col];
        reinterpret_cast<float4*>(qo)[1] = qstash[wave][row][1][col];
      }
      fill_empty_output();
      return;
    }
    if (holds_last) {
      norm_rope_row(kx, kw8, a.eps, cr, sr, col);
      const SlotWords<kDtype> kw = pack_slot<kDtype>(kx);
      const SlotWords<kDtype> vw = pack_slot<kDtype>(vx);
      if (row == 0) {
#pragma unroll
        for (int i = 0; i < SlotWords<kDtype>::kWords; ++i) {
          stash[wave][0][i][col] = kw.w[i];
          stash[wave][1][i][col] = vw.w[i];
        }
      }
    }
  }
  // Pre-scale by log2(e)/sqrt(128) so that scores come out in log2 units for exp2.
  const float qscale = kLog2e * 0.08838834764831845f;  // 1/sqrt(128)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    qa[e] *= qscale;
    qb[e] *= qscale;
  }

  HeadState A, Bs;
  A.init();
  Bs.init();

  // Software pipeline over the pages: the tile of page p+1 is in flight while
  // page p is consumed.  In the steady-state loop both following pages exist,
  // so every load is unconditional; the scheduling barriers keep each tile's
  // eight loads together and ahead of the math on the other tile, so the wait
  // before a tile covers only its own loads.  The last one or two pages (the
  // only place a partial page, or the new token, can be) are finished after
  // the loop.
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
    __builtin_amdgcn_sched_barrier(0);
    attend_tile<kDtype, false>(K0, V0, qa, qb, A, Bs, row, kPage);
    __builtin_amdgcn_sched_barrier(0);
    if (last_masked)
      attend_tile<kDtype, true>(K1, V1, qa, qb, A, Bs, row, last_valid);
    else
      attend_tile<kDtype, false>(K1, V1, qa, qb, A, Bs, row, kPage);
  } else {
    if (last_masked)
      attend_tile<kDtype, true>(K0, V0, qa, qb, A, Bs, row, last_valid);
    else
      attend_tile<kDtype, false>(K0, V0, qa, qb, A, Bs, row, kPage);
  }
  if constexpr (kStep) {
    // The new token (slot tail - 1 of the last page, read from the cache
    // above as masked) enters from the stash: the values just stored, in the
    // cache's dtype, owned by the row of that slot.
    if (holds_last) {
      SlotWords<kDtype> kw, vw;
#pragma unroll
      for (int i = 0; i < SlotWords<kDtype>::kWords; ++i) {
        kw.w[i] = stash[wave][0][i][col];
        vw.w[i] = stash[wave][1][i][col];
      }
      float kf[8], vf[8];
      unpack_slot<kDtype>(kw, kf);
      unpack_slot<kDtype>(vw, vf);
      float sa = 0.0f, sb = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sa = fmaf(qa[e], kf[e], sa);
        sb = fmaf(qb[e], kf[e], sb);
      }
      sa = row_sum16(sa);
      sb = row_sum16(sb);
      const bool mine = row == ((tail - 1) & 3);
      attend_one(A, mine ? sa : -INFINITY, vf);
      attend_one(Bs, mine ? sb : -INFINITY, vf);
    }
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
  if constexpr (kStep) {
    if (split == 0 && row < 2) {
      float* qo = a.q_out + ((size_t)b * kHeads + 2 * g + row) * kHeadDim + 8 * col;
      reinterpret_cast<float4*>(qo)[0] = qstash[wave][row][0][col];
      reinterpret_cast<float4*>(qo)[1] = qstash[wave][row][1][col];
    }
    if (holds_last && row == 0) {
      // The new token's slot: page block_table[b][npages-1], slot tail - 1.
      const int id = bt[npages - 1];
      if (id >= 0 && id < a.num_pages) {
        const int64_t slot_off = (int64_t)id * page_bytes + head_bytes +
                                 (int64_t)(tail - 1) * (Tile<kDtype>::kTileBytes / kPage);
        u32x4* kd = reinterpret_cast<u32x4*>(a.k_cache_w + slot_off) + SlotWords<kDtype>::kWords * col;
        u32x4* vd = reinterpret_cast<u32x4*>(a.v_cache_w + slot_off) + SlotWords<kDtype>::kWords * col;
#pragma unroll
        for (int i = 0; i < SlotWords<kDtype>::kWords; ++i) {
          kd[i] = stash[wave][0][i][col];
          vd[i] = stash[wave][1][i][col];
        }
      }
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
  dah::RopePowers rope;
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
    // cos/sin of pos * theta^(-2i/128), angle formed in float64 (at pos near
    // 40,960 a float32 angle would be off by ~4e-3 rad); see dah_rope.h.
    float cn, sn;
    dah::rope_cos_sin((double)pos * dah::rope_inv_freq(lane, a.rope), &cn, &sn);
    cs[lane] = make_float2(cn, sn);
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
  a.rope = dah::rope_powers((double)rope_theta);
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

// The extra inputs of the fused decode step.
struct StepInputs {
  const float* k_new;
  const float* v_new;
  const float* q_gain;
  const float* k_gain;
  float eps;
  float rope_theta;
  float* q_out;
  void* k_cache;
  void* v_cache;
};

int plan_for(int B, int max_seq_len, int num_splits, void* workspace, size_t workspace_bytes,
             dah::Plan* plan) {
  int cus = 0;
  int st = device_cu_count(&cus);
  if (st != DAH_OK) return st;
  st = dah::plan_splits(B, max_seq_len, num_splits, cus, plan);
  if (st != DAH_OK) return st;
  if (plan->workspace > 0) {
    if (workspace == nullptr || workspace_bytes < plan->workspace)
      return dah::set_error(DAH_ERR_WORKSPACE,
                            "workspace of %zu bytes, need %zu (B=%d, max_seq_len=%d, %d splits)",
                            workspace == nullptr ? (size_t)0 : workspace_bytes, plan->workspace, B,
                            max_seq_len, plan->splits);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return dah::set_error(DAH_ERR_ALIGN, "workspace needs 256-byte alignment");
  }
  return DAH_OK;
}

// Decode (step == nullptr: q is already normed and roped) or the fused
// decode step (q is raw; the kernel norms, rotates and appends).
int launch_decode(const dah::Plan& plan, const float* q, const void* k_cache,
                  const void* v_cache, int cache_dtype, int64_t num_pages,
                  const int32_t* block_table, int max_pages_per_seq, const int32_t* seq_lens,
                  int B, int max_seq_len, float* o, void* workspace, const StepInputs* step,
                  hipStream_t stream) {
  DecodeArgs a = {};
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
  if (step != nullptr) {
    a.k_new = step->k_new;
    a.v_new = step->v_new;
    a.q_gain = step->q_gain;
    a.k_gain = step->k_gain;
    a.eps = step->eps;
    a.rope = dah::rope_powers((double)step->rope_theta);
    a.q_out = step->q_out;
    a.k_cache_w = static_cast<char*>(step->k_cache);
    a.v_cache_w = static_cast<char*>(step->v_cache);
  }

  const long long blocks = (long long)B * plan.splits;  // one workgroup per (sequence, split)
  if (blocks > INT32_MAX) return dah::set_error(DAH_ERR_SHAPE, "grid too large");
  const dim3 grid((unsigned)blocks), block(kWave * kDecodeWavesPerBlock);
  const bool bf16 = cache_dtype == DAH_BF16;
  if (step == nullptr) {
    if (bf16)
      decode_split_kernel<DAH_BF16, false><<<grid, block, 0, stream>>>(a);
    else
      decode_split_kernel<DAH_F32, false><<<grid, block, 0, stream>>>(a);
  } else {
    if (bf16)
      decode_split_kernel<DAH_BF16, true><<<grid, block, 0, stream>>>(a);
    else
      decode_split_kernel<DAH_F32, true><<<grid, block, 0, stream>>>(a);
  }
  int st = check_launch("decode_split_kernel");
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
  dah::Plan plan;
  st = plan_for(B, max_seq_len, num_splits, workspace, workspace_bytes, &plan);
  if (st != DAH_OK) return st;
  return launch_decode(plan, q, k_cache, v_cache, cache_dtype, num_pages, block_table,
                       max_pages_per_seq, seq_lens, B, max_seq_len, o, workspace, nullptr,
                       static_cast<hipStream_t>(stream));
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
  // Plan and check the workspace before anything is launched, so that a
  // failing call leaves the cache untouched.
  dah::Plan plan;
  st = plan_for(B, max_seq_len, num_splits, workspace, workspace_bytes, &plan);
  if (st != DAH_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q_out == q && plan.splits > 1) {
    // In place with several splits: the workgroups of one sequence would read
    // q while another overwrites it, so norm and rotate first, then decode.
    st = launch_append(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache, v_cache,
                       cache_dtype, num_pages, block_table, max_pages_per_seq, seq_lens, B,
                       max_seq_len, q_out, s);
    if (st != DAH_OK) return st;
    return launch_decode(plan, q_out, k_cache, v_cache, cache_dtype, num_pages, block_table,
                         max_pages_per_seq, seq_lens, B, max_seq_len, o, workspace, nullptr, s);
  }
  // One launch: the decode kernel norms and rotates q, writes q_out, and
  // appends the new key and value (see decode_split_kernel).
  const StepInputs step = {k_new, v_new, q_gain, k_gain, eps, rope_theta, q_out, k_cache, v_cache};
  return launch_decode(plan, q, k_cache, v_cache, cache_dtype, num_pages, block_table,
                       max_pages_per_seq, seq_lens, B, max_seq_len, o, workspace, &step, s);
}

size_t dah_workspace_bytes(int B, int max_seq_len, int num_splits) {
  int cus = 0;
  if (device_cu_count(&cus) != DAH_OK) return 0;
  return dah_workspace_bytes_for(B, max_seq_len, num_splits, cus);
}

}  // extern "C"
