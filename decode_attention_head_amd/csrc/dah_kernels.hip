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
// K and V (bf16) and ~G flops per byte.  One wavefront owns one
// (sequence, KV head g, split) and all G query heads gG .. gG+G-1 of that KV
// head (G = 2 for Qwen3-0.6B; 4, 5, 8 for the family's larger members).
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
#include <mutex>
#include <type_traits>

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
static_assert(dah::kMaxBalancedBatch == 8 * kWave * kDecodeWavesPerBlock,
              "the balanced decode's scan gives each thread 8 sequences");
using dah::kMaxBalancedBatch;
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

// Consume one (page, KV head) tile for the kG query heads of that KV head
// (kG = 2 for Qwen3-0.6B).
template <int kDtype, bool kMasked, int kG>
__device__ __forceinline__ void attend_tile(const Tile<kDtype>& K, Tile<kDtype>& V,
                                            const float (&q)[kG][8], HeadState (&st)[kG],
                                            int row, int nvalid) {
  float sc[kG][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float part[kG];
#pragma unroll
    for (int h = 0; h < kG; ++h) part[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float k = K.get(j, e);
#pragma unroll
      for (int h = 0; h < kG; ++h) part[h] = fmaf(q[h][e], k, part[h]);
    }
#pragma unroll
    for (int h = 0; h < kG; ++h) sc[h][j] = row_sum16(part[h]);
    if (kMasked) {
      // Positions at or past seq_len may hold anything (NaN included): the
      // select keeps them out of both the scores and the V sum.
      const bool ok = (4 * j + row) < nvalid;
#pragma unroll
      for (int h = 0; h < kG; ++h) sc[h][j] = ok ? sc[h][j] : -INFINITY;
      if (!ok) V.clear(j);
    }
  }
  float w[kG][4], alpha[kG];
#pragma unroll
  for (int h = 0; h < kG; ++h) alpha[h] = softmax_update<kMasked>(st[h], sc[h], w[h]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int h = 0; h < kG; ++h) st[h].acc[e] *= alpha[h];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = V.get(j, e);
#pragma unroll
      for (int h = 0; h < kG; ++h) st[h].acc[e] = fmaf(w[h][j], v, st[h].acc[e]);
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
  int grid_splits;  // splits rounded up to a multiple of 8 (1 when splits == 1)
  int pages_per_split;
  float* o;
  // Partial results (H query heads): DAH_PLAN_SPLIT slot (b*H + h)*splits +
  // split, DAH_PLAN_BALANCED slot (b + workgroup)*H + h; 128 floats of
  // weighted V sum each, then one float2 (running max in log2 units, sum) each.
  float* part_acc;
  float* part_ml;
  // DAH_PLAN_BALANCED: prefix[b] = pages of sequences < b (b <= B), written
  // by workgroup 0 of the decode for the merge.
  int32_t* prefix;
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

// LDS a workgroup of the fused step uses to hold outputs until the end of a
// range (see decode_range).
template <int kG>
struct StepStash {
  u32x4 kv[kDecodeWavesPerBlock][2][2][16];   // [wave][k|v][word][column]
  float4 q[kDecodeWavesPerBlock][kG][2][16];  // [wave][head][half][column]
};

// Query head h (< kG) of KV head g is written by the wave rows r with
// r = h mod 4 (after merge_rows every row holds every head's result).
__device__ __forceinline__ bool row_writes(int row, int h) { return row == (h & 3); }

// The fused step for a sequence with nothing to attend to (seq_len out of
// range): q_out is still the normed query, rotated at pos = seq_len - 1 (or 0).
template <int kDtype, int kG>
__device__ void step_q_out_only(const DecodeArgs& a, int b, int seq_len, int g, int lane) {
  if (a.q_out == nullptr) return;  // the caller asked for o only
  constexpr int kH = kG * kKvHeads;
  const int row = lane >> 4, col = lane & 15;
  float qw[8], cr[8], sr[8];
  load8(a.q_gain + 8 * col, qw);
  rope_table(seq_len >= 1 ? seq_len - 1 : 0, a.rope, lane, col, cr, sr);
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    float q[8];
    const size_t rowoff = ((size_t)b * kH + g * kG + h) * kHeadDim + 8 * col;
    load8(a.q + rowoff, q);
    norm_rope_row(q, qw, a.eps, cr, sr, col);
    if (row_writes(row, h)) store8(a.q_out + rowoff, q, 1.0f);
  }
}

// decodeGQA of one KV head (this wave: g) and its kG query heads over pages
// [p0, p1) of sequence b (p0 < p1 <= npages).  The result goes to o when the
// range is the whole sequence (to_o), else to the partial slots
// part_base + h * part_stride (h = query head) as (weighted V sum, running
// max, sum).
// kStep, the fused decode step: q arrives raw and is normed and rotated here
// (write_q: this range also writes q_out), and the range holding the
// sequence's last page norms and rotates the new key, folds the new token in
// from registers and stores the new key and value in the cache.
// qb: the row block of q and o (the sequence b for a decode; a chunk
// token, attending over its own prefix of sequence b's pages, for chunks).
template <int kDtype, bool kStep, int kG, int kGS = kG>
__device__ __forceinline__ void decode_range(const DecodeArgs& a, int b, int qb, int seq_len,
                                             int npages, int p0, int p1, bool write_q, bool to_o,
                                             size_t part_base, int part_stride, int g, int lane,
                                             StepStash<kG>& stash, int h0 = 0) {
  constexpr int kH = kG * kKvHeads;
  const int wave = g;
  const int row = lane >> 4;
  const int col = lane & 15;
  // This call's query heads: h0 .. h0 + kGS - 1 of the kG of KV head g.
  const size_t qrow0 = (size_t)qb * kH + g * kG + h0;  // first query head row of the call

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
  const int last = p1 - 1;                           // last page of this range
  // In the fused step the last page's final slot is the new token, which is
  // taken from registers, so only tail - 1 of its slots are read from the cache.
  const bool holds_last = kStep && p1 == npages;
  const int last_valid = holds_last ? tail - 1 : tail;
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
  // Query rows of this KV head, this lane's 8 dims (raw in the fused step).
  float q[kGS][8];
#pragma unroll
  for (int h = 0; h < kGS; ++h) load8(a.q + (qrow0 + h) * kHeadDim + 8 * col, q[h]);
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
  constexpr bool kPrefetch = !(kDtype == DAH_F32 && kGS == 5);
  Tile<kDtype> K0, V0, K1, V1;
  int id1 = bt[min(p0 + 1, last)];
  int id2 = bt[min(p0 + 2, last)];
  {
    const int64_t off0 = offset_of(bt[p0]);
    K0.load(kbase + off0, lane);
    V0.load(vbase + off0, lane);
  }

  // The fused step's outputs besides o -- q_out rows and the new token's key
  // and value in the cache dtype -- wait in LDS (per wave, written and read
  // by that wave only) and go to memory after the page loop: one counter
  // tracks vector loads and stores in issue order, so a store issued early
  // would hold up the waits for the first tiles.
  if constexpr (kStep) {
    const int pos = seq_len - 1;
    float cr[8], sr[8];
    rope_table(pos, a.rope, lane, col, cr, sr);
#pragma unroll
    for (int h = 0; h < kGS; ++h) {
      norm_rope_row(q[h], qw, a.eps, cr, sr, col);
      if (write_q && row_writes(row, h0 + h)) {
        stash.q[wave][h0 + h][0][col] = make_float4(q[h][0], q[h][1], q[h][2], q[h][3]);
        stash.q[wave][h0 + h][1][col] = make_float4(q[h][4], q[h][5], q[h][6], q[h][7]);
      }
    }
    if (holds_last) {
      norm_rope_row(kx, kw8, a.eps, cr, sr, col);
      const SlotWords<kDtype> kw = pack_slot<kDtype>(kx);
      const SlotWords<kDtype> vw = pack_slot<kDtype>(vx);
      if (row == 0) {
#pragma unroll
        for (int i = 0; i < SlotWords<kDtype>::kWords; ++i) {
          stash.kv[wave][0][i][col] = kw.w[i];
          stash.kv[wave][1][i][col] = vw.w[i];
        }
      }
    }
  }
  // Pre-scale by log2(e)/sqrt(128) so that scores come out in log2 units for exp2.
  const float qscale = kLog2e * 0.08838834764831845f;  // 1/sqrt(128)
#pragma unroll
  for (int h = 0; h < kGS; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) q[h][e] *= qscale;

  HeadState st[kGS];
#pragma unroll
  for (int h = 0; h < kGS; ++h) st[h].init();

  // Software pipeline over the pages: the tile of page p+1 is in flight while
  // page p is consumed.  In the steady-state loop both following pages exist,
  // so every load is unconditional; the scheduling barriers keep each tile's
  // eight loads together and ahead of the math on the other tile, so the wait
  // before a tile covers only its own loads.  The last one or two pages (the
  // only place a partial page, or the new token, can be) are finished after
  // the loop.  A float32 cache with 5 query heads per KV head loads one tile
  // at a time instead: there the second tile spills (the one-tile loop is 7%
  // faster); at 8 heads both forms spill and the pipelined one is faster.
  if constexpr (!kPrefetch) {
    // One tile at a time: page p is loaded, then consumed.
    for (int p = p0; p <= last; ++p) {
      if (p > p0) {
        const int64_t off = offset_of(bt[p]);
        K0.load(kbase + off, lane);
        V0.load(vbase + off, lane);
      }
      if (p == last && last_masked)
        attend_tile<kDtype, true, kGS>(K0, V0, q, st, row, last_valid);
      else
        attend_tile<kDtype, false, kGS>(K0, V0, q, st, row, kPage);
    }
  } else {
    int p = p0;
    for (; p + 2 <= last; p += 2) {
      const int64_t off1 = offset_of(id1);
      K1.load(kbase + off1, lane);
      V1.load(vbase + off1, lane);
      const int id3 = bt[min(p + 3, last)];
      __builtin_amdgcn_sched_barrier(0);
      attend_tile<kDtype, false, kGS>(K0, V0, q, st, row, kPage);
      __builtin_amdgcn_sched_barrier(0);
      const int64_t off2 = offset_of(id2);
      K0.load(kbase + off2, lane);
      V0.load(vbase + off2, lane);
      const int id4 = bt[min(p + 4, last)];
      __builtin_amdgcn_sched_barrier(0);
      attend_tile<kDtype, false, kGS>(K1, V1, q, st, row, kPage);
      __builtin_amdgcn_sched_barrier(0);
      id1 = id3;
      id2 = id4;
    }
    if (p + 1 <= last) {
      const int64_t off1 = offset_of(id1);
      K1.load(kbase + off1, lane);
      V1.load(vbase + off1, lane);
      __builtin_amdgcn_sched_barrier(0);
      attend_tile<kDtype, false, kGS>(K0, V0, q, st, row, kPage);
      __builtin_amdgcn_sched_barrier(0);
      if (last_masked)
        attend_tile<kDtype, true, kGS>(K1, V1, q, st, row, last_valid);
      else
        attend_tile<kDtype, false, kGS>(K1, V1, q, st, row, kPage);
    } else {
      if (last_masked)
        attend_tile<kDtype, true, kGS>(K0, V0, q, st, row, last_valid);
      else
        attend_tile<kDtype, false, kGS>(K0, V0, q, st, row, kPage);
    }
  }
  if constexpr (kStep) {
    // The new token (slot tail - 1 of the last page, read from the cache
    // above as masked) enters from the stash: the values just computed, in
    // the cache's dtype, owned by the row of that slot.
    if (holds_last) {
      SlotWords<kDtype> kw, vw;
#pragma unroll
      for (int i = 0; i < SlotWords<kDtype>::kWords; ++i) {
        kw.w[i] = stash.kv[wave][0][i][col];
        vw.w[i] = stash.kv[wave][1][i][col];
      }
      float kf[8], vf[8];
      unpack_slot<kDtype>(kw, kf);
      unpack_slot<kDtype>(vw, vf);
      const bool mine = row == ((tail - 1) & 3);
#pragma unroll
      for (int h = 0; h < kGS; ++h) {
        float sc = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sc = fmaf(q[h][e], kf[e], sc);
        sc = row_sum16(sc);
        attend_one(st[h], mine ? sc : -INFINITY, vf);
      }
    }
  }

#pragma unroll
  for (int h = 0; h < kGS; ++h) {
    merge_rows(st[h]);
    if (bad_page) st[h].l = NAN;
  }
#pragma unroll
  for (int h = 0; h < kGS; ++h) {
    if (!row_writes(row, h0 + h)) continue;
    if (to_o) {
      store8(a.o + (qrow0 + h) * kHeadDim + 8 * col, st[h].acc, 1.0f / st[h].l);
    } else {
      const size_t part = part_base + (size_t)(g * kG + h0 + h) * part_stride;
      store8(a.part_acc + part * kHeadDim + 8 * col, st[h].acc, bad_page ? NAN : 1.0f);
      if (col == 0) reinterpret_cast<float2*>(a.part_ml)[part] = make_float2(st[h].m, st[h].l);
    }
  }
  if constexpr (kStep) {
    if (write_q && a.q_out != nullptr) {
#pragma unroll
      for (int h = 0; h < kGS; ++h) {
        if (!row_writes(row, h0 + h)) continue;
        float* qo = a.q_out + (qrow0 + h) * kHeadDim + 8 * col;
        reinterpret_cast<float4*>(qo)[0] = stash.q[wave][h0 + h][0][col];
        reinterpret_cast<float4*>(qo)[1] = stash.q[wave][h0 + h][1][col];
      }
    }
    if (holds_last && row == 0 && h0 == 0) {
      // The new token's slot: page block_table[b][npages-1], slot tail - 1.
      const int id = bt[npages - 1];
      if (id >= 0 && id < a.num_pages) {
        const int64_t slot_off = (int64_t)id * page_bytes + head_bytes +
                                 (int64_t)(tail - 1) * (Tile<kDtype>::kTileBytes / kPage);
        u32x4* kd = reinterpret_cast<u32x4*>(a.k_cache_w + slot_off) + SlotWords<kDtype>::kWords * col;
        u32x4* vd = reinterpret_cast<u32x4*>(a.v_cache_w + slot_off) + SlotWords<kDtype>::kWords * col;
#pragma unroll
        for (int i = 0; i < SlotWords<kDtype>::kWords; ++i) {
          kd[i] = stash.kv[wave][0][i][col];
          vd[i] = stash.kv[wave][1][i][col];
        }
      }
    }
  }
}

// decode_range over all kG query heads of the wave's KV head: for a float32
// cache with 8 heads per KV head in two sweeps of 4 over the range (the
// query rows, softmax states and two float32 tiles of all 8 heads do not fit
// in registers; the second sweep reads the range's pages again).
template <int kDtype, bool kStep, int kG>
__device__ __forceinline__ void decode_range_heads(const DecodeArgs& a, int b, int qb,
                                                   int seq_len, int npages, int p0, int p1,
                                                   bool write_q, bool to_o, size_t part_base,
                                                   int part_stride, int g, int lane,
                                                   StepStash<kG>& stash) {
  if constexpr (kDtype == DAH_F32 && kG == 8) {
    decode_range<kDtype, kStep, kG, 4>(a, b, qb, seq_len, npages, p0, p1, write_q, to_o,
                                       part_base, part_stride, g, lane, stash, 0);
    decode_range<kDtype, kStep, kG, 4>(a, b, qb, seq_len, npages, p0, p1, write_q, to_o,
                                       part_base, part_stride, g, lane, stash, 4);
  } else {
    decode_range<kDtype, kStep, kG>(a, b, qb, seq_len, npages, p0, p1, write_q, to_o, part_base,
                                    part_stride, g, lane, stash);
  }
}

// ------------------------------------------------------------ MFMA decode
//
// With 4 or more query heads per KV head (the family's 4B/8B, 14B and 32B
// shapes) the VALU form above runs out of issue slots and registers: the
// multiply-adds grow with G while the bytes do not.  For a bfloat16 cache
// both contractions of a page then go to the matrix cores with
// v_mfma_f32_16x16x32_bf16 (the planner also picks this form for G = 2
// unless the sequences are cut into fixed splits, where the VALU form's
// two workgroups per compute unit do better).  Lane l = 16 r + c.
//
// Scores.  A = 16 positions x 32 dims of K, B = 32 dims x 16 query-head
// columns, D = scores.  The lane loads K position sigma(c) = 4 (c mod 4) +
// c / 4, dims 32 kk + 8 r .. +7 (16 bytes; the four kk cover a position's
// 256 bytes in 64-byte pieces).  The permutation sigma makes D land as
// lane (r, c) = scores of head c at positions 4 v + r, v = 0..3 -- the
// positions of wave row r in the V tile, which is what the second product
// needs.  q (float32) enters as the sum of three bfloat16 terms along the
// contraction (12 products per page), which carries it to 2^-27 relative:
// the cache values are exact in bfloat16, so the scores are as accurate as
// a float32 dot product.
//
// Weighted V sum.  A = weights (16 head rows x 32), B = V (32 x 16 dims),
// the 32 contraction slots being (term, position): weights enter as two
// bfloat16 terms (2^-18 relative).  The V tile keeps the coalesced layout of
// the VALU path (lane (r, c): dims 8c..8c+7 of positions 4j + r); product
// nb = 0..7 takes dim 8c + nb of the lane's four positions as the lane's B
// column, so D holds rows = heads 4r + v, column c = dim 8c + nb.  No value
// crosses lanes between the two products.
//
// Online softmax.  All rows share one reference per head (the products mix
// rows); the page maximum is reduced across rows and the reference moves
// only when a score exceeds it by more than kMaxLag (log2 units), so weights
// stay below 2^kMaxLag and rescaling is rare.  Any reference gives the same
// softmax (theorem softmax_shift, "Supported models" page).

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr float kMaxLag = 8.0f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Stores of the matrix-core decode's outputs (o, q_out, the new cache slot).
// With 4+ query heads per KV head every workgroup ends by storing 8+ rows of
// o and q_out per wave (8-16 MB per launch at B = 256); streaming them past
// the L2 with non-temporal stores finished such launches 4-14 us sooner on
// MI355X.  At 2 heads per KV head (4 MB) they gained nothing, so kNt is
// kG >= 4.
template <bool kNt, class V>
__device__ __forceinline__ void store_out(V* dst, const V& v) {
  if constexpr (kNt)
    __builtin_nontemporal_store(v, dst);
  else
    *dst = v;
}

template <bool kNt>
__device__ __forceinline__ void store8_out(float* dst, const float (&v)[8], float scale) {
  f32x4* d = reinterpret_cast<f32x4*>(dst);
  store_out<kNt>(d, f32x4{v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale});
  store_out<kNt>(d + 1, f32x4{v[4] * scale, v[5] * scale, v[6] * scale, v[7] * scale});
}

// Two floats -> two bfloat16 (round to nearest even; v_cvt_pk_bf16_f32),
// `lo` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Maximum over the four wave rows (lanes c, c+16, c+32, c+48): the two row
// swaps pair rows (0,1),(2,3), then (0,2),(1,3).
__device__ __forceinline__ float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// K tile in the score product's A layout.
struct KTileMfma {
  u32x4 w[4];  // kk = 0..3
  __device__ __forceinline__ void load(const char* tile, int lane) {
    const int r = lane >> 4, c = lane & 15;
    const int pos = 4 * (c & 3) + (c >> 2);
    const u32x4* p = reinterpret_cast<const u32x4*>(tile) + pos * 16 + r;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) w[kk] = __builtin_nontemporal_load(p + 4 * kk);
  }
};

// LDS of one workgroup of the MFMA decode: normed queries (fused step) and
// the new token's stored words.
template <int kG>
struct MfmaStash {
  u32x4 kv[kDecodeWavesPerBlock][2][16];        // [wave][k|v][column] (bf16: one word each)
  float q[kDecodeWavesPerBlock][kG][kHeadDim];  // [wave][head][dim]
};

// Scores of one page: lane (r, c) gets head c at positions 4v + r.  One
// accumulator per query term (kT of them) keeps kT independent chains of
// four products in flight instead of one chain of 4 kT.
template <int kT>
__device__ __forceinline__ f32x4 page_scores(const KTileMfma& K, const u32x4 (&qb)[4][kT]) {
  f32x4 s[kT];
#pragma unroll
  for (int t = 0; t < kT; ++t) s[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, K.w[kk]);
#pragma unroll
    for (int t = 0; t < kT; ++t)
      s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, qb[kk][t]),
                                                      s[t], 0, 0, 0);
  }
  f32x4 r = s[0];
#pragma unroll
  for (int t = 1; t < kT; ++t) r += s[t];
  return r;
}

// Online-softmax state of the MFMA decode.  m and l are per lane for head c
// (m equal across rows; l the lane's share, summed over rows at the end);
// acc[nb] holds rows = heads 4r + v, dim 8c + nb.
struct MfmaState {
  float m, l;
  f32x4 acc[8];
};

// One page: scores -> weights -> weighted V sum.  kMasked: positions
// >= nvalid are excluded (their V is cleared: 0 * NaN would poison a row).
// kCausal (chunks of several new tokens): column c also sees only the page
// positions below climit, its own limit (per lane); those positions hold
// valid keys and values, so only the scores are masked.
template <bool kMasked, bool kCausal = false>
__device__ __forceinline__ void attend_page_mfma(const KTileMfma& K, Tile<DAH_BF16>& V,
                                                 const u32x4 (&qb)[4][3], MfmaState& st,
                                                 int lane, int nvalid, int climit = kPage) {
  const int r = lane >> 4;
  f32x4 s = page_scores(K, qb);
  if (kMasked) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const bool ok = 4 * v + r < nvalid;
      s[v] = ok ? s[v] : -INFINITY;
      if (!ok) V.clear(v);
    }
  }
  if (kCausal) {
#pragma unroll
    for (int v = 0; v < 4; ++v) s[v] = 4 * v + r < climit ? s[v] : -INFINITY;
  }
  const float pm = max_over_rows(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
  // Move the reference only when a score passes it by more than kMaxLag
  // (always from -inf); a wave-uniform branch, rarely taken after the
  // first page.
  const bool move = pm > st.m + kMaxLag;
  if (__builtin_amdgcn_ballot_w64(move) != 0) {
    const float mn = move ? pm : st.m;
    const float alpha = mn == st.m ? 1.0f : fast_exp2(st.m - mn);
    st.m = mn;
    st.l *= alpha;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float av = __shfl(alpha, 4 * r + v);  // head 4r + v's factor (column 4r + v)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) st.acc[nb][v] *= av;
    }
  }
  const float mu = st.m == -INFINITY ? 0.0f : st.m;
  float p[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) p[v] = fast_exp2(s[v] - mu);
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
  // Weights as hi + lo bfloat16 terms.
  u32x4 aw;
  aw[0] = pack_bf16x2(p[0], p[1]);
  aw[1] = pack_bf16x2(p[2], p[3]);
  aw[2] = pack_bf16x2(p[0] - bf16_lo(aw[0]), p[1] - bf16_hi(aw[0]));
  aw[3] = pack_bf16x2(p[2] - bf16_lo(aw[1]), p[3] - bf16_hi(aw[1]));
  const bf16x8 a = __builtin_bit_cast(bf16x8, aw);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const uint32_t sel = (nb & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t v01 = __builtin_amdgcn_perm(V.w[1][nb >> 1], V.w[0][nb >> 1], sel);
    const uint32_t v23 = __builtin_amdgcn_perm(V.w[3][nb >> 1], V.w[2][nb >> 1], sel);
    const u32x4 bw = {v01, v23, v01, v23};
    st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bw),
                                                          st.acc[nb], 0, 0, 0);
  }
}

// Splits 8 float32 values into kT bfloat16 terms of the score product's B
// operand, each the rounding of what the previous terms leave: three terms
// hold a float32 value exactly (8 + 8 + 8 significant bits), two to a
// relative 2^-18.
template <int kT>
__device__ __forceinline__ void split_terms(const float (&x)[8], u32x4 (&out)[kT]) {
  float rem[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) rem[e] = x[e];
#pragma unroll
  for (int t = 0; t < kT; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[t][i] = pack_bf16x2(rem[2 * i], rem[2 * i + 1]);
      rem[2 * i] -= bf16_lo(out[t][i]);
      rem[2 * i + 1] -= bf16_hi(out[t][i]);
    }
  }
}

// Ranges whose pages before the final one number at least this many (65
// pages or more in all) are visited in ascending page order
// (decode_range_mfma); shorter ones, where the sort costs more than the
// locality returns, in table order.
constexpr int kSortMinLeadingPages = 64;

// Sorts the 128 values a wave holds as element e = lane + 64 r (a0: r = 0,
// a1: r = 1) into ascending order: a bitonic network, compare-exchanges at
// distance 64 inside the lane and at shorter distances across lanes.
__device__ __forceinline__ void sort128(int& a0, int& a1, int lane) {
#pragma unroll
  for (int k = 2; k <= 128; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j == 64) {  // k = 128: ascending throughout
        const int lo = min(a0, a1), hi = max(a0, a1);
        a0 = lo;
        a1 = hi;
      } else {
        const bool lower = (lane & j) == 0;
        const int p0 = __shfl_xor(a0, j), p1 = __shfl_xor(a1, j);
        const bool min0 = ((lane & k) == 0) == lower;         // e = lane
        const bool min1 = (((lane + 64) & k) == 0) == lower;  // e = lane + 64
        a0 = min0 ? min(a0, p0) : max(a0, p0);
        a1 = min1 ? min(a1, p1) : max(a1, p1);
      }
    }
  }
}

// decode_range for a bfloat16 cache on the matrix cores; same contract.
template <bool kStep, int kG>
__device__ __forceinline__ void decode_range_mfma(const DecodeArgs& a, int b, int seq_len,
                                                  int npages, int p0, int p1, bool write_q,
                                                  bool to_o, size_t part_base, int part_stride,
                                                  int g, int lane, MfmaStash<kG>& stash) {
  static_assert(kG <= 16, "one score column per query head");
  constexpr int kH = kG * kKvHeads;
  constexpr bool kNt = kG >= 4;  // see store_out
  using TileV = Tile<DAH_BF16>;
  const int wave = g;
  const int row = lane >> 4;
  const int col = lane & 15;
  const int qh = col < kG ? col : kG - 1;            // this lane's score column's head
  const size_t qrow0 = (size_t)b * kH + g * kG;      // first query head row of this KV head

  typedef const __attribute__((address_space(4))) int32_t* ConstI32;
  const ConstI32 bt = (ConstI32)(a.block_table + (size_t)b * a.max_pages_per_seq);
  const int64_t page_bytes = (int64_t)kKvHeads * TileV::kTileBytes;
  const int64_t head_bytes = (int64_t)g * TileV::kTileBytes;
  const char* kbase = a.k_cache + head_bytes;
  const char* vbase = a.v_cache + head_bytes;
  const int tail = seq_len - (npages - 1) * kPage;
  const int last = p1 - 1;
  const bool holds_last = kStep && p1 == npages;
  const int last_valid = holds_last ? tail - 1 : tail;
  const bool last_masked = (last == npages - 1) && last_valid < kPage;
  bool bad_page = false;
  auto offset_of = [&](int id) -> int64_t {
    const bool ok = id >= 0 && id < a.num_pages;
    bad_page |= !ok;
    return (int64_t)(ok ? id : 0) * page_bytes;
  };
  const float qscale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)

  // Small loads first (see decode_range).  Without the step, q arrives
  // normed: the lane reads its B-operand slice (head qh, dims 32kk + 8r ..)
  // directly.  With the step, it reads raw rows in the row layout, each
  // 16-lane row its own heads: row r takes heads r, r + 4, ... (kJ of them),
  // so the norm and rotation cost kJ rows of work per lane instead of kG.
  // Entries past kG repeat head kG - 1 and are not used.
  constexpr int kJ = (kG + 3) / 4;
  float qv[kStep ? 1 : 4][8];
  float qr[kStep ? kJ : 1][8];
  float qw[8], kx[8], vx[8], kw8[8];
  if constexpr (!kStep) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) load8(a.q + (qrow0 + qh) * kHeadDim + 32 * kk + 8 * row, qv[kk]);
  } else {
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      load8(a.q + (qrow0 + min(row + 4 * j, kG - 1)) * kHeadDim + 8 * col, qr[j]);
    load8(a.q_gain + 8 * col, qw);
    if (holds_last) {
      load8(a.k_new + ((size_t)b * kKvHeads + g) * kHeadDim + 8 * col, kx);
      load8(a.v_new + ((size_t)b * kKvHeads + g) * kHeadDim + 8 * col, vx);
      load8(a.k_gain + 8 * col, kw8);
    }
  }

  // The range's pages before its final one are visited in ascending
  // physical order: every workgroup then sweeps the pool from low ids to
  // high at about the same pace, where table order scatters the concurrent
  // reads over the whole pool (on MI355X, B = 256, S = 2048: 0.5% off the
  // step, the sort included; 1.2% off the decode with rows sorted ahead of
  // it).  The final page, which may be masked, stays last; ranges of fewer
  // than 65 or more than 129 pages keep table order.  Each wave sorts its
  // own copy of the ids, so the 8 waves agree without a barrier.  Attention
  // is independent of the order of positions (up to float32 rounding).
  const int n_sorted = last - p0;
  const bool sorted = n_sorted >= kSortMinLeadingPages && n_sorted <= 128;
  int key0 = INT32_MAX, key1 = INT32_MAX;
  if (sorted) {
    const int32_t* ids = a.block_table + (size_t)b * a.max_pages_per_seq + p0;
    if (lane < n_sorted) key0 = ids[lane];
    if (lane + 64 < n_sorted) key1 = ids[lane + 64];
    sort128(key0, key1, lane);
  }
  auto page_id = [&](int x) -> int {  // the page visited x - p0 th, x <= last
    if (!sorted || x >= last) return bt[x];
    const int i = x - p0;
    return i < 64 ? __builtin_amdgcn_readlane(key0, i) : __builtin_amdgcn_readlane(key1, i - 64);
  };

  KTileMfma K0, K1;
  TileV V0, V1;
  int id1 = page_id(min(p0 + 1, last));
  int id2 = page_id(min(p0 + 2, last));
  {
    const int64_t off0 = offset_of(page_id(p0));
    K0.load(kbase + off0, lane);
    V0.load(vbase + off0, lane);
  }

  MfmaState st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) st.acc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4 qb[4][3];
  if constexpr (kStep) {
    const int pos = seq_len - 1;
    float cr[8], sr[8];
    rope_table(pos, a.rope, lane, col, cr, sr);
    float kf[8], vf[8];
    if (holds_last) {
      norm_rope_row(kx, kw8, a.eps, cr, sr, col);
      const SlotWords<DAH_BF16> kw = pack_slot<DAH_BF16>(kx);
      const SlotWords<DAH_BF16> vw = pack_slot<DAH_BF16>(vx);
      if (row == 0) {
        stash.kv[wave][0][col] = kw.w[0];
        stash.kv[wave][1][col] = vw.w[0];
      }
      unpack_slot<DAH_BF16>(kw, kf);  // the new token as the cache holds it
      unpack_slot<DAH_BF16>(vw, vf);
    }
    float sc_new[kJ];  // the new token's score for head row + 4j (whole row)
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int h = row + 4 * j;
      norm_rope_row(qr[j], qw, a.eps, cr, sr, col);
      if (h < kG) {
        float4* d = reinterpret_cast<float4*>(&stash.q[wave][h][8 * col]);
        d[0] = make_float4(qr[j][0], qr[j][1], qr[j][2], qr[j][3]);
        d[1] = make_float4(qr[j][4], qr[j][5], qr[j][6], qr[j][7]);
      }
      if (holds_last) {
        float sc = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sc = fmaf(qr[j][e], kf[e], sc);
        sc_new[j] = row_sum16(sc) * qscale;
      }
    }
    if (holds_last) {
      // Column c's head c was scored by row c mod 4, entry c / 4.
      float s_new = -INFINITY;
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const float v = __shfl(sc_new[j], 16 * (col & 3) + col);
        s_new = (col >> 2) == j ? v : s_new;
      }
      // Start the state with the new token: reference = its score, weight 1
      // (counted once, in row 0), value = v_new for every head of this KV head.
      st.m = col < kG ? s_new : 0.0f;
      st.l = row == 0 ? 1.0f : 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool live = 4 * row + v < kG;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) st.acc[nb][v] = live ? vf[nb] : 0.0f;
      }
    }
    // The normed rows are in LDS; read this lane's B-operand slice back.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      float x[8];
      const float4* sq = reinterpret_cast<const float4*>(&stash.q[wave][qh][32 * kk + 8 * row]);
      const float4 x0 = sq[0], x1 = sq[1];
      x[0] = x0.x * qscale; x[1] = x0.y * qscale; x[2] = x0.z * qscale; x[3] = x0.w * qscale;
      x[4] = x1.x * qscale; x[5] = x1.y * qscale; x[6] = x1.z * qscale; x[7] = x1.w * qscale;
      split_terms<3>(x, qb[kk]);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[kk][e] *= qscale;
      split_terms<3>(qv[kk], qb[kk]);
    }
  }
  if (col >= kG) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int t = 0; t < 3; ++t) qb[kk][t] = u32x4{0u, 0u, 0u, 0u};
  }

  int p = p0;
  for (; p + 2 <= last; p += 2) {
    const int64_t off1 = offset_of(id1);
    K1.load(kbase + off1, lane);
    V1.load(vbase + off1, lane);
    const int id3 = page_id(min(p + 3, last));
    __builtin_amdgcn_sched_barrier(0);
    attend_page_mfma<false>(K0, V0, qb, st, lane, kPage);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t off2 = offset_of(id2);
    K0.load(kbase + off2, lane);
    V0.load(vbase + off2, lane);
    const int id4 = page_id(min(p + 4, last));
    __builtin_amdgcn_sched_barrier(0);
    attend_page_mfma<false>(K1, V1, qb, st, lane, kPage);
    __builtin_amdgcn_sched_barrier(0);
    id1 = id3;
    id2 = id4;
  }
  if (p + 1 <= last) {
    const int64_t off1 = offset_of(id1);
    K1.load(kbase + off1, lane);
    V1.load(vbase + off1, lane);
    __builtin_amdgcn_sched_barrier(0);
    attend_page_mfma<false>(K0, V0, qb, st, lane, kPage);
    __builtin_amdgcn_sched_barrier(0);
    if (last_masked)
      attend_page_mfma<true>(K1, V1, qb, st, lane, last_valid);
    else
      attend_page_mfma<false>(K1, V1, qb, st, lane, kPage);
  } else {
    if (last_masked)
      attend_page_mfma<true>(K0, V0, qb, st, lane, last_valid);
    else
      attend_page_mfma<false>(K0, V0, qb, st, lane, kPage);
  }

  // Totals per head (column c): l summed over the rows.
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int h = 4 * row + v;  // this lane's accumulator row v
    const float lh = __shfl(l, h);
    const float mh = __shfl(st.m, h);
    if (h >= kG) continue;
    float o8[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) o8[nb] = st.acc[nb][v];
    if (to_o) {
      store8_out<kNt>(a.o + (qrow0 + h) * kHeadDim + 8 * col, o8, bad_page ? NAN : 1.0f / lh);
    } else {
      const size_t part = part_base + (size_t)(g * kG + h) * part_stride;
      store8(a.part_acc + part * kHeadDim + 8 * col, o8, bad_page ? NAN : 1.0f);
      if (col == 0)
        reinterpret_cast<float2*>(a.part_ml)[part] = make_float2(mh, bad_page ? NAN : lh);
    }
  }
  if constexpr (kStep) {
    if (write_q && a.q_out != nullptr) {
      // Two 128-float rows per wave store: lanes 0-31 row h, lanes 32-63 row h + 1.
      const int half = lane >> 5, q4 = lane & 31;
#pragma unroll
      for (int h0 = 0; h0 < kG; h0 += 2) {
        const int h = h0 + half;
        if (h < kG)
          store_out<kNt>(reinterpret_cast<f32x4*>(a.q_out + (qrow0 + h) * kHeadDim) + q4,
                         reinterpret_cast<const f32x4*>(&stash.q[wave][h][0])[q4]);
      }
    }
    if (holds_last && row == 0) {
      const int id = bt[npages - 1];
      if (id >= 0 && id < a.num_pages) {
        const int64_t slot_off = (int64_t)id * page_bytes + head_bytes +
                                 (int64_t)(tail - 1) * (TileV::kTileBytes / kPage);
        store_out<kNt>(reinterpret_cast<u32x4*>(a.k_cache_w + slot_off) + col, stash.kv[wave][0][col]);
        store_out<kNt>(reinterpret_cast<u32x4*>(a.v_cache_w + slot_off) + col, stash.kv[wave][1][col]);
      }
    }
  }
}

__device__ __forceinline__ int pages_of(int seq_len, int max_seq_len) {
  return (seq_len >= 1 && seq_len <= max_seq_len) ? (seq_len + kPage - 1) / kPage : 0;
}

// Empty sequence (seq_len <= 0: o = 0; past max_seq_len: o = NaN).
template <int kG>
__device__ __forceinline__ void fill_o(const DecodeArgs& a, int b, int seq_len, int g, int lane) {
  const int row = lane >> 4, col = lane & 15;
  const float fill = seq_len <= 0 ? 0.0f : NAN;
  const float z[8] = {fill, fill, fill, fill, fill, fill, fill, fill};
#pragma unroll
  for (int h = 0; h < kG; ++h)
    if (row_writes(row, h))
      store8(a.o + ((size_t)b * kG * kKvHeads + g * kG + h) * kHeadDim + 8 * col, z, 1.0f);
}

// One workgroup (8 waves = 8 KV heads) per (sequence, split), each split
// `pages_per_split` pages; splits == 1 writes o directly, otherwise
// combine_splits_kernel merges the partials.
template <int kDtype, bool kStep, int kG, bool kMfma>
__global__ __launch_bounds__(kWave * kDecodeWavesPerBlock) void decode_split_kernel(DecodeArgs a) {
  static_assert(!kMfma || kDtype == DAH_BF16, "the matrix-core decode reads a bfloat16 cache");
  const int lane = threadIdx.x & (kWave - 1);
  // The wave index is uniform across the wave; saying so keeps everything
  // derived from it (sequence, page range, page addresses) in scalar registers.
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // KV head
  // Workgroup -> (sequence, split).  Workgroups are handed to the 8 XCDs
  // (each with its own L2 and 1/8 of the chip's bandwidth) round-robin by
  // blockIdx.  With several splits the grid is padded to a multiple of 8
  // splits and split s of sequence b goes to XCD (s + b) mod 8, so every XCD
  // gets an eighth of each long sequence.
  int b, split;
  if (a.splits == 1) {
    b = blockIdx.x;
    split = 0;
  } else {
    const int xcd = blockIdx.x & 7;
    const int local = blockIdx.x >> 3;
    const int per = a.grid_splits >> 3;  // padded splits per XCD and sequence
    b = local / per;
    split = 8 * (local - b * per) + ((xcd - b) & 7);
  }
  if (b >= a.B) return;
  const int seq_len = a.seq_lens[b];
  const int npages = pages_of(seq_len, a.max_seq_len);
  const int p0 = split * a.pages_per_split;  // splits past a.splits are padding: empty
  const int p1 = min(p0 + a.pages_per_split, npages);
  if (p0 >= p1 || split >= a.splits) {
    // Nothing to attend to.  With one split this is the whole sequence; with
    // several, the combine kernel reads only non-empty ranges.
    if (kStep && split == 0) step_q_out_only<kDtype, kG>(a, b, seq_len, g, lane);
    if (a.splits == 1) fill_o<kG>(a, b, seq_len, g, lane);
    return;
  }
  const size_t part_base = ((size_t)b * kG * kKvHeads) * a.splits + split;
  if constexpr (kMfma) {
    __shared__ MfmaStash<kG> stash;
    decode_range_mfma<kStep, kG>(a, b, seq_len, npages, p0, p1, split == 0, a.splits == 1,
                                 part_base, a.splits, g, lane, stash);
  } else {
    __shared__ StepStash<kG> stash;
    decode_range_heads<kDtype, kStep, kG>(a, b, b, seq_len, npages, p0, p1, split == 0,
                                          a.splits == 1, part_base, a.splits, g, lane, stash);
  }
}

// Balanced decode: the batch's pages, in sequence order, are cut into
// gridDim.x equal ranges, one per workgroup, regardless of where sequences
// begin and end.  A workgroup walks the sequence segments inside its range;
// a segment that is a whole sequence writes o, any other writes partial slot
// b + k (k = workgroup), which combine_balanced_kernel merges.  Consecutive
// workgroups go to different XCDs, so every XCD gets an equal share of the
// pages however ragged the lengths are, and no workgroup is empty.
template <int kDtype, bool kStep, int kG, bool kMfma>
__global__ __launch_bounds__(kWave * kDecodeWavesPerBlock) void decode_balanced_kernel(DecodeArgs a) {
  static_assert(!kMfma || kDtype == DAH_BF16, "the matrix-core decode reads a bfloat16 cache");
  constexpr int kH = kG * kKvHeads;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // KV head
  __shared__ int prefix[kMaxBalancedBatch + 1];  // prefix[b] = pages of sequences < b
  __shared__ int wave_total[kDecodeWavesPerBlock];
  __shared__ std::conditional_t<kMfma, MfmaStash<kG>, StepStash<kG>> stash;

  // Block-wide exclusive scan of the page counts; thread t owns sequences
  // 8t .. 8t+7.
  const int t = threadIdx.x;
  int own[8], tot = 0;
  // Eight independent loads (clamped index, masked afterwards) so that they
  // are in flight together.
#pragma unroll
  for (int i = 0; i < 8; ++i) own[i] = a.seq_lens[min(8 * t + i, a.B - 1)];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    own[i] = 8 * t + i < a.B ? pages_of(own[i], a.max_seq_len) : 0;
    tot += own[i];
  }
  int incl = tot;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) wave_total[g] = incl;
  __syncthreads();
  int run = incl - tot;
  for (int w = 0; w < g; ++w) run += wave_total[w];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int bb = 8 * t + i;
    if (bb < a.B) prefix[bb] = run;
    run += own[i];
    if (bb == a.B - 1) prefix[a.B] = run;
  }
  __syncthreads();
  if (blockIdx.x == 0)  // for the merge launch
    for (int bb = t; bb <= a.B; bb += blockDim.x) a.prefix[bb] = prefix[bb];

  if constexpr (kStep) {
    // Sequences with nothing to attend to still get q_out (workgroup 0).
    if (blockIdx.x == 0)
      for (int bb = 0; bb < a.B; ++bb)
        if (prefix[bb + 1] == prefix[bb]) step_q_out_only<kDtype, kG>(a, bb, a.seq_lens[bb], g, lane);
  }

  const long long T = prefix[a.B];
  const long long G = gridDim.x, k = blockIdx.x;
  int s = (int)(k * T / G);
  const int e = (int)((k + 1) * T / G);
  if (s >= e) return;
  // The sequence holding page s: the largest b with prefix[b] <= s.
  int lo = 0, hi = a.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= s) lo = mid; else hi = mid;
  }
  int b = lo;
  for (;;) {
    b = __builtin_amdgcn_readfirstlane(b);
    const int base = __builtin_amdgcn_readfirstlane(prefix[b]);
    const int next = __builtin_amdgcn_readfirstlane(prefix[b + 1]);
    const int seg_end = min(e, next);
    const int npages = next - base;
    const int p0 = s - base, p1 = seg_end - base;
    const bool whole = p0 == 0 && p1 == npages;
    // An opaque copy of the lane index per segment: otherwise the compiler
    // hoists lane-dependent values of the range out of this loop and keeps
    // them live across it, which costs 30-50 registers (and spills).
    int lane_i = lane;
    asm volatile("" : "+v"(lane_i));
    if constexpr (kMfma)
      decode_range_mfma<kStep, kG>(a, b, a.seq_lens[b], npages, p0, p1, p0 == 0, whole,
                                   (size_t)(b + k) * kH, 1, g, lane_i, stash);
    else
      decode_range_heads<kDtype, kStep, kG>(a, b, b, a.seq_lens[b], npages, p0, p1, p0 == 0,
                                            whole, (size_t)(b + k) * kH, 1, g, lane_i, stash);
    s = seg_end;
    if (s >= e) break;
    do { ++b; } while (prefix[b + 1] == prefix[b]);  // next sequence with pages
  }
}

// ------------------------------------------------------------ log-sum-exp merge
//
// A row's partial results (weighted V sum acc_s, running max m_s in log2
// units, sum l_s) merge as  M = max_s m_s,  w_s = 2^(m_s - M),
// o = sum_s w_s acc_s / sum_s w_s l_s.  Fixed splits (merge_parts): one
// workgroup of 256 threads per (sequence, query head); thread t owns dims
// 4(t mod 32) .. +3 and every 8th partial starting at t / 32.  One pass: each thread folds its partials into a running (max,
// sum, weighted V sum), rescaling when the max moves (the same result by
// softmax_shift), and LDS merges the 8 groups the same way.  The loads of
// kMergeChunk partials per thread are issued before any is used.
constexpr int kCombineThreads = 256;
constexpr int kCombineGroups = kCombineThreads / 32;
constexpr int kMergeChunk = 8;

// Partial i of a row: split layout (row-major splits; the first n present).
struct SplitParts {
  size_t base;  // (b * H + h) * splits
  __device__ size_t slot(int i) const { return base + i; }
  __device__ bool present(int) const { return true; }
};

// Partial i of a row: balanced layout, slot (b + k0 + i) * H + h; a
// workgroup whose page range was empty wrote nothing.
struct BalancedParts {
  int b, h, k0, H;
  long long T, G;
  __device__ size_t slot(int i) const { return (size_t)(b + k0 + i) * H + h; }
  __device__ bool present(int i) const {
    const long long k = k0 + i;
    return T >= G || k * T / G < (k + 1) * T / G;
  }
};

// Running state of one thread (or group) of the merge.
struct MergeState {
  float m = -INFINITY, l = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  // Fold in (m2, l2, acc2 * s2) where acc2 is scaled by s2 = 1 on entry.
  __device__ void fold(float m2, float l2, const float4& v) {
    const float mn = fmaxf(m, m2);
    const float s1 = m == -INFINITY ? 0.0f : fast_exp2(m - mn);
    const float s2 = m2 == -INFINITY ? 0.0f : fast_exp2(m2 - mn);
    m = mn;
    l = l * s1 + l2 * s2;
    acc.x = acc.x * s1 + v.x * s2;
    acc.y = acc.y * s1 + v.y * s2;
    acc.z = acc.z * s1 + v.z * s2;
    acc.w = acc.w * s1 + v.w * s2;
  }
};

// Merges the present partials among i < n of a row (slots i < n_slots are
// read: they must lie inside the partial buffers) and writes the row, or
// `fill` in every element when !ok (a sequence outside the domain).
template <class Parts>
__device__ __forceinline__ void merge_parts(const float* __restrict__ part_acc,
                                            const float* __restrict__ part_ml, const Parts& parts,
                                            int n_slots, int n, bool ok, float fill,
                                            float* __restrict__ out_row) {
  __shared__ float red_m[kCombineGroups];
  __shared__ float4 red_acc[kCombineGroups][32];
  __shared__ float red_l[kCombineGroups];
  const int t = threadIdx.x;
  const int grp = t >> 5, dim4 = t & 31;
  const float2* ml = reinterpret_cast<const float2*>(part_ml);

  MergeState st;
  for (int i0 = grp; i0 < n_slots; i0 += kCombineGroups * kMergeChunk) {
    float2 m_l[kMergeChunk];
    float4 v[kMergeChunk];
#pragma unroll
    for (int c = 0; c < kMergeChunk; ++c) {
      const int i = i0 + kCombineGroups * c;
      if (i < n_slots) {
        const size_t slot = parts.slot(i);
        m_l[c] = ml[slot];
        v[c] = reinterpret_cast<const float4*>(part_acc + slot * kHeadDim)[dim4];
      }
    }
#pragma unroll
    for (int c = 0; c < kMergeChunk; ++c) {
      const int i = i0 + kCombineGroups * c;
      if (i < n && parts.present(i)) st.fold(m_l[c].x, m_l[c].y, v[c]);
    }
  }
  // Merge the 8 groups: the reference max first, then the rescaled sums.
  if (dim4 == 0) red_m[grp] = st.m;
  __syncthreads();
  float M = red_m[0];
#pragma unroll
  for (int g = 1; g < kCombineGroups; ++g) M = fmaxf(M, red_m[g]);
  const float s = st.m == -INFINITY ? 0.0f : fast_exp2(st.m - M);
  red_acc[grp][dim4] = make_float4(st.acc.x * s, st.acc.y * s, st.acc.z * s, st.acc.w * s);
  if (dim4 == 0) red_l[grp] = st.l * s;
  __syncthreads();
  if (grp == 0) {
    float4 sum = red_acc[0][dim4];
    float Ls = red_l[0];
#pragma unroll
    for (int g = 1; g < kCombineGroups; ++g) {
      const float4 v = red_acc[g][dim4];
      sum.x += v.x;
      sum.y += v.y;
      sum.z += v.z;
      sum.w += v.w;
      Ls += red_l[g];
    }
    const float inv = 1.0f / Ls;
    reinterpret_cast<float4*>(out_row)[dim4] =
        ok ? make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv)
           : make_float4(fill, fill, fill, fill);
  }
}

// DAH_PLAN_SPLIT: the non-empty splits of each (sequence, head); the row's
// length decides how many of its `splits` slots count.
__global__ __launch_bounds__(kCombineThreads) void combine_splits_kernel(
    const float* __restrict__ part_acc, const float* __restrict__ part_ml,
    const int32_t* __restrict__ seq_lens, int H, int max_seq_len, int splits,
    int pages_per_split, float* __restrict__ o) {
  const int unit = blockIdx.x;  // b * H + h
  const int b = unit / H;
  const int seq_len = seq_lens[b];
  const bool ok = seq_len >= 1 && seq_len <= max_seq_len;
  const int npages = ok ? (seq_len + kPage - 1) / kPage : 0;
  const int nsplit = (npages + pages_per_split - 1) / pages_per_split;
  merge_parts(part_acc, part_ml, SplitParts{(size_t)unit * splits}, splits, nsplit, ok,
              seq_len < 1 ? 0.0f : NAN, o + (size_t)unit * kHeadDim);
}

// DAH_PLAN_BALANCED: sequence b owns pages [P_b, P_b + n_b) of the batch and
// workgroup k of G owns [floor(kT/G), floor((k+1)T/G)), so the workgroups
// that saw b are owner(P_b) .. owner(P_b + n_b - 1) with
// owner(x) = floor(((x+1)G - 1)/T), their partials in slots b + k.  A
// sequence seen by one workgroup was written to o directly.  The decode
// left the prefix sums P in the workspace.  One wave per (sequence, 2
// heads): lane l merges dims 4(l mod 32) .. +3 of head 2 blockIdx + l / 32
// over the (few) workgroups that saw the sequence.
constexpr int kBalancedMergeThreads = 64;
constexpr int kBalancedMergeRows = kBalancedMergeThreads / 32;  // heads per workgroup

__global__ __launch_bounds__(kBalancedMergeThreads) void combine_balanced_kernel(
    const float* __restrict__ part_acc, const float* __restrict__ part_ml,
    const int32_t* __restrict__ prefix, const int32_t* __restrict__ seq_lens, int B, int H, int G,
    float* __restrict__ o) {
  const int groups = H / kBalancedMergeRows;
  const int b = blockIdx.x / groups;
  const int h = (blockIdx.x - b * groups) * kBalancedMergeRows + (threadIdx.x >> 5);
  const int dim4 = threadIdx.x & 31;
  const int seq_len = seq_lens[b];
  const long long P = prefix[b];
  const int np = prefix[b + 1] - prefix[b];
  const long long T = prefix[B];
  float4* out = reinterpret_cast<float4*>(o + ((size_t)b * H + h) * kHeadDim) + dim4;
  if (np == 0) {  // seq_len outside 1 .. max_seq_len
    const float fill = seq_len < 1 ? 0.0f : NAN;
    *out = make_float4(fill, fill, fill, fill);
    return;
  }
  const int k0 = (int)(((P + 1) * G - 1) / T);
  const int k1 = (int)(((P + np) * G - 1) / T);
  if (k0 == k1) return;
  const int n = k1 - k0 + 1;
  const BalancedParts parts{b, h, k0, H, T, (long long)G};
  const float2* ml = reinterpret_cast<const float2*>(part_ml);
  MergeState st;
  for (int i0 = 0; i0 < n; i0 += kMergeChunk) {
    float2 m_l[kMergeChunk];
    float4 v[kMergeChunk];
#pragma unroll
    for (int c = 0; c < kMergeChunk; ++c) {
      if (i0 + c < n) {
        const size_t slot = parts.slot(i0 + c);
        m_l[c] = ml[slot];
        v[c] = reinterpret_cast<const float4*>(part_acc + slot * kHeadDim)[dim4];
      }
    }
#pragma unroll
    for (int c = 0; c < kMergeChunk; ++c)
      if (i0 + c < n && parts.present(i0 + c)) st.fold(m_l[c].x, m_l[c].y, v[c]);
  }
  const float inv = 1.0f / st.l;
  *out = make_float4(st.acc.x * inv, st.acc.y * inv, st.acc.z * inv, st.acc.w * inv);
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

// One block of 8 waves per token row.  Wave w handles query heads w, w+8,
// ... (kG of them), key head w and value head w; lane i holds dims i and
// i+64 (a RoPE pair).  `row` indexes q, k_new, v_new and q_out; the cache
// slot is position pos of block-table row b, written only when `append`.
template <int kDtype, int kG>
__device__ __forceinline__ void norm_rope_append_row(const AppendArgs& a, size_t row, int b,
                                                     int pos, bool append) {
  constexpr int kH = kG * kKvHeads;
  __shared__ float2 cs[64];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & (kWave - 1);
  if (w == 0) {
    // cos/sin of pos * theta^(-2i/128), angle formed in float64 (at pos near
    // 40,960 a float32 angle would be off by ~4e-3 rad); see dah_rope.h.
    float cn, sn;
    dah::rope_cos_sin((double)pos * dah::rope_inv_freq(lane, a.rope), &cn, &sn);
    cs[lane] = make_float2(cn, sn);
  }
  // Load while wave 0 computes the angles.
  float qa[kG], qb[kG];
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    const size_t qbase = (row * kH + w + kKvHeads * i) * kHeadDim;
    qa[i] = a.q[qbase + lane];
    qb[i] = a.q[qbase + lane + 64];
  }
  const size_t kvbase = (row * kKvHeads + w) * kHeadDim;
  float ka = a.k_new[kvbase + lane], kb = a.k_new[kvbase + lane + 64];
  const float va = a.v_new[kvbase + lane], vb = a.v_new[kvbase + lane + 64];
  __syncthreads();
  const float2 r = cs[lane];

#pragma unroll
  for (int i = 0; i < kG; ++i) rms_norm(qa[i], qb[i], a.q_gain, a.eps, lane);
  rms_norm(ka, kb, a.k_gain, a.eps, lane);
#pragma unroll
  for (int i = 0; i < kG; ++i) rotate(qa[i], qb[i], r.x, r.y);
  rotate(ka, kb, r.x, r.y);
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    const size_t qbase = (row * kH + w + kKvHeads * i) * kHeadDim;
    a.q_out[qbase + lane] = qa[i];
    a.q_out[qbase + lane + 64] = qb[i];
  }

  if (!append) return;
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

// One workgroup per sequence: its new token at pos = seq_len - 1.
template <int kDtype, int kG>
__global__ __launch_bounds__(512) void norm_rope_append_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int seq_len = a.seq_lens[b];
  norm_rope_append_row<kDtype, kG>(a, b, b, seq_len >= 1 ? seq_len - 1 : 0,
                                   seq_len >= 1 && seq_len <= a.max_len);
}

// Chunks: workgroup (b, i) handles token i of sequence b's chunk (rows
// cu_tokens[b] .. cu_tokens[b+1]-1, n_b of them), at position
// seq_len - n_b + i.  Sequences whose length cannot hold their chunk, or
// exceeds max_len, get q_out at position 0 and no append.
template <int kDtype, int kG>
__global__ __launch_bounds__(512) void norm_rope_append_chunk_kernel(AppendArgs a,
                                                                     const int32_t* cu_tokens,
                                                                     int max_chunk, int total) {
  const int b = blockIdx.x / max_chunk;
  const int i = blockIdx.x - b * max_chunk;
  const int t0 = min(max(cu_tokens[b], 0), total);
  const int t1 = min(max(cu_tokens[b + 1], t0), total);
  const int n = t1 - t0;
  if (i >= n) return;
  const int seq_len = a.seq_lens[b];
  const bool ok = n <= max_chunk && seq_len >= n && seq_len <= a.max_len;
  norm_rope_append_row<kDtype, kG>(a, (size_t)t0 + i, b, ok ? seq_len - n + i : 0, ok);
}

// ------------------------------------------------------------ chunk attention
//
// Causal attention of a chunk of new tokens over the paged cache (their keys
// and values already appended), on the matrix cores: the 16 score columns of
// a wave are (token, query head) pairs -- 16 / G tokens of one KV head -- so
// each K/V page is read once for all of them.  Column c sees positions up to
// its token's own; pages wholly below the tile's first token need no mask.

struct ChunkArgs {
  const float* q;  // normed and roped, [tokens][H][128]
  const char* k_cache;
  const char* v_cache;
  int num_pages;
  const int32_t* block_table;
  int max_pages_per_seq;
  const int32_t* seq_lens;
  const int32_t* cu_tokens;
  int total;       // tokens
  int max_chunk;   // host bound on n_b
  int tiles;       // tiles per sequence: ceil(max_chunk / (16 / G))
  int max_seq_len;
  float* o;        // [tokens][H][128]
};

template <int kG>
__global__ __launch_bounds__(kWave * kDecodeWavesPerBlock) void chunk_attn_kernel(ChunkArgs a) {
  constexpr int kH = kG * kKvHeads;
  constexpr int kTpt = 16 / kG;  // tokens per tile
  using TileV = Tile<DAH_BF16>;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // KV head
  const int row = lane >> 4, col = lane & 15;
  const int b = blockIdx.x / a.tiles;
  const int tile = blockIdx.x - b * a.tiles;
  const int t0 = min(max(a.cu_tokens[b], 0), a.total);
  const int t1 = min(max(a.cu_tokens[b + 1], t0), a.total);
  const int n = t1 - t0;
  const int i0 = tile * kTpt;
  if (i0 >= n) return;
  const int ntok = min(kTpt, n - i0);
  const int seq_len = a.seq_lens[b];
  if (n > a.max_chunk || seq_len < n || seq_len > a.max_seq_len) {
    // Outside the preconditions: NaN for this tile's tokens (and, from tile
    // 0, for tokens past max_chunk tiles), nothing read from the cache.
    const int last = tile == 0 ? n : i0 + ntok;
    for (int i = i0; i < last; ++i) {
      if (tile == 0 && i >= ntok && i < a.tiles * kTpt) continue;  // owned by another tile
      for (int h = 0; h < kG; ++h)
        reinterpret_cast<float2*>(a.o + (((size_t)t0 + i) * kH + g * kG + h) * kHeadDim)[lane] =
            make_float2(NAN, NAN);
    }
    return;
  }

  const int pos0 = seq_len - n + i0;    // position of the tile's first token
  const int pmax = pos0 + ntok - 1;
  const int ti = col / kG, hh = col - ti * kG;
  const bool live = ti < ntok;
  const int climit_pos = pos0 + (live ? ti : ntok - 1);  // last position column col sees
  const size_t qrow = ((size_t)t0 + i0 + (live ? ti : 0)) * kH + g * kG + (live ? hh : 0);

  typedef const __attribute__((address_space(4))) int32_t* ConstI32;
  const ConstI32 bt = (ConstI32)(a.block_table + (size_t)b * a.max_pages_per_seq);
  const int64_t page_bytes = (int64_t)kKvHeads * TileV::kTileBytes;
  const int64_t head_bytes = (int64_t)g * TileV::kTileBytes;
  const char* kbase = a.k_cache + head_bytes;
  const char* vbase = a.v_cache + head_bytes;
  const int last = pmax / kPage;              // last page the tile reads
  const int first_masked = (pos0 + 1) / kPage;  // pages below are seen whole by every column
  bool bad_page = false;
  auto offset_of = [&](int id) -> int64_t {
    const bool ok = id >= 0 && id < a.num_pages;
    bad_page |= !ok;
    return (int64_t)(ok ? id : 0) * page_bytes;
  };

  float qv[4][8];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) load8(a.q + qrow * kHeadDim + 32 * kk + 8 * row, qv[kk]);

  KTileMfma K0, K1;
  TileV V0, V1;
  int id1 = bt[min(1, last)];
  int id2 = bt[min(2, last)];
  {
    const int64_t off0 = offset_of(bt[0]);
    K0.load(kbase + off0, lane);
    V0.load(vbase + off0, lane);
  }
  const float qscale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
  u32x4 qb[4][3];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[kk][e] *= qscale;
    split_terms<3>(qv[kk], qb[kk]);
  }
  if (!live) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int t = 0; t < 3; ++t) qb[kk][t] = u32x4{0u, 0u, 0u, 0u};
  }
  MfmaState st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) st.acc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Page p: positions 16p .. 16p+15; the tile needs none past pmax (their
  // slots may hold anything) and column col none past climit_pos.
  auto attend = [&](const KTileMfma& K, TileV& V, int p) {
    if (p < first_masked) {
      attend_page_mfma<false>(K, V, qb, st, lane, kPage);
    } else {
      attend_page_mfma<true, true>(K, V, qb, st, lane, pmax - kPage * p + 1,
                                   climit_pos - kPage * p + 1);
    }
  };
  int p = 0;
  for (; p + 2 <= last; p += 2) {
    const int64_t off1 = offset_of(id1);
    K1.load(kbase + off1, lane);
    V1.load(vbase + off1, lane);
    const int id3 = bt[min(p + 3, last)];
    __builtin_amdgcn_sched_barrier(0);
    attend(K0, V0, p);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t off2 = offset_of(id2);
    K0.load(kbase + off2, lane);
    V0.load(vbase + off2, lane);
    const int id4 = bt[min(p + 4, last)];
    __builtin_amdgcn_sched_barrier(0);
    attend(K1, V1, p + 1);
    __builtin_amdgcn_sched_barrier(0);
    id1 = id3;
    id2 = id4;
  }
  if (p + 1 <= last) {
    const int64_t off1 = offset_of(id1);
    K1.load(kbase + off1, lane);
    V1.load(vbase + off1, lane);
    __builtin_amdgcn_sched_barrier(0);
    attend(K0, V0, p);
    __builtin_amdgcn_sched_barrier(0);
    attend(K1, V1, p + 1);
  } else {
    attend(K0, V0, p);
  }

  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int j = 4 * row + v;   // accumulator row: column j = (token j / G, head j % G)
    const float lj = __shfl(l, j);
    const int tj = j / kG, hj = j - tj * kG;
    if (tj >= ntok) continue;
    float o8[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) o8[nb] = st.acc[nb][v];
    store8(a.o + (((size_t)t0 + i0 + tj) * kH + g * kG + hj) * kHeadDim + 8 * col, o8,
           bad_page ? NAN : 1.0f / lj);
  }
}

// Chunks with a float32 cache (strict-parity runs): every chunk token is a
// decode over positions 0 .. its own on the VALU decode path -- one
// workgroup (8 waves = 8 KV heads) per (sequence, chunk token), each reading
// its own prefix of the sequence's pages, so the cache is read once per
// token: meant for verification-sized chunks.
template <int kG>
__global__ __launch_bounds__(kWave * kDecodeWavesPerBlock) void chunk_valu_kernel(
    DecodeArgs a, const int32_t* __restrict__ cu_tokens, int total, int max_chunk) {
  constexpr int kH = kG * kKvHeads;
  __shared__ StepStash<kG> stash;  // decode_range's signature; unused without the step
  const int lane = threadIdx.x & (kWave - 1);
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // KV head
  const int b = blockIdx.x / max_chunk;
  const int i = blockIdx.x - b * max_chunk;
  const int t0 = min(max(cu_tokens[b], 0), total);
  const int t1 = min(max(cu_tokens[b + 1], t0), total);
  const int n = t1 - t0;
  if (i >= n) return;
  const int seq_len = a.seq_lens[b];
  if (n > max_chunk || seq_len < n || seq_len > a.max_seq_len) {
    // Outside the preconditions: NaN for this token (and, from token 0, for
    // tokens past max_chunk), nothing read from the cache.
    const int last = i == 0 ? n : i + 1;
    for (int j = i; j < last; ++j) {
      if (i == 0 && j >= 1 && j < max_chunk) continue;  // owned by another workgroup
      for (int h = 0; h < kG; ++h)
        reinterpret_cast<float2*>(a.o + (((size_t)t0 + j) * kH + g * kG + h) * kHeadDim)[lane] =
            make_float2(NAN, NAN);
    }
    return;
  }
  const int len = seq_len - n + i + 1;  // positions 0 .. the token's own
  const int npages = (len + kPage - 1) / kPage;
  decode_range_heads<DAH_F32, false, kG>(a, b, t0 + i, len, npages, 0, npages, false, true, 0,
                                         0, g, lane, stash);
}

// The weighted V sum of the shared-page kernel, transposed: D = V^T W^T with
// rows = dims and columns = the wave's 16 score columns, on
// v_mfma_f32_16x16x32_bf16 (lane (r, c): A row c / B column c, k 8r .. 8r+7;
// D rows 4r + v, column c), so that every lane keeps its own column's
// accumulators and the rescale needs no other lane.  The 32 contraction
// slots of lane row r are the page positions whose scores the lane holds
// (4e + r, e = 0..3) twice over: for the two pages of a step (one product
// per bfloat16 term of the weights), or, with one page per step, for the
// two terms.  A (16 dims x those positions of V) comes straight from the
// staged page with ds_read_b64_tr_b16, whose result in lane i of each
// 16-lane group is element i mod 4 of the 8-byte pieces at the addresses of
// lanes i/4 + {0, 4, 8, 12} of the group: lane (r, j) points at position
// 4 (j / 4) + r, dims 16 nb + 4 (j mod 4) .. +3, which makes lane (r, c)
// hold V[4e + r][16 nb + c], e = 0..3.  (The 16x16x16 form would take the
// same matrix-core cycles per instruction for half the work.)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* LdsS16x4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct PrefillState {
  float m, l;      // per column (m equal across rows; l the lane's share)
  f32x4 acc[8];    // acc[nb][v]: dim 16 nb + 4 r + v of column c
};

// The V stage's swizzle: 16-byte piece q of position P sits in slot
// q ^ (2 vswz(P)), so that the transpose reads of one instruction (8
// positions x 2 pieces per 32 lanes) fall on distinct banks.
__device__ __forceinline__ int vswz(int P) { return (P >> 2) + 4 * (P & 1); }

// The K stage's swizzle: piece q of position P sits in slot q ^ kswz(P).
// The score product's reads put positions sigma(c) = 4 (c mod 4) + c / 4 of
// lanes c = 0..7 (and 8..15) at one piece index; kswz takes distinct values
// modulo 8 on each such group of 8 positions (and is a bijection on 0..15),
// so 8 lanes of 16 bytes -- 32 banks -- never share a bank.
__device__ __forceinline__ int kswz(int P) { return (P >> 2) | ((P & 1) << 2) | ((P & 2) << 2); }

__device__ __forceinline__ u32x2 read_v_tr(const char* base, int off) {
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsS16x4)(const_cast<char*>(base) + off)));
}

// One step of kP pages (1 or 2) of the shared-page kernel, in two halves
// so that a wave can issue one step's score products and then work on the
// previous step's weights while the matrix cores run them.
//
// step_scores: K[j] holds page j's K tile; lane (r, c) gets column c's
// scores at positions 4v + r of each page.  kMasked: column c sees only the
// positions of page j below climit[j] (per lane; 0 = none of the page).
template <int kP, bool kMasked, int kT>
__device__ __forceinline__ void step_scores(const KTileMfma (&K)[kP], const u32x4 (&qb)[4][kT],
                                            int lane, const int (&climit)[kP], f32x4 (&s)[kP]) {
  const int r = lane >> 4;
#pragma unroll
  for (int j = 0; j < kP; ++j) {
    s[j] = page_scores(K[j], qb);
    if (kMasked) {
#pragma unroll
      for (int v = 0; v < 4; ++v) s[j][v] = 4 * v + r < climit[j] ? s[j][v] : -INFINITY;
    }
  }
}

// A lane's LDS offsets within a stage page: K piece kk of its score-product
// row (kb + 64 (kk ^ kq)) and V transpose-read nb (vb + 32 (nb ^ vx)).  With
// one block per wave the twelve offsets stay in registers; with two, whose
// state leaves no room for them, they are formed at each use.
template <bool kTable>
struct StageOffsets {
  int kb, kq, vb, vx;
  __device__ __forceinline__ int k(int kk) const { return kb + 64 * (kk ^ kq); }
  __device__ __forceinline__ int v(int nb) const { return vb + 32 * (nb ^ vx); }
};
template <>
struct StageOffsets<true> {
  int ko[4], vo[8];
  __device__ __forceinline__ int k(int kk) const { return ko[kk]; }
  __device__ __forceinline__ int v(int nb) const { return vo[nb]; }
};

// step_weights_pv: the online softmax over a step's scores and the weighted
// sum of its V pages, for the kCB 16-column blocks of a wave (each with its
// own state): vpage[j] the staged V of page j, off this lane's transpose-read
// offsets.  Every V operand read from the stage feeds all kCB blocks'
// products.  The stage holds zeros for positions past the sequence, so V
// needs no clearing.
template <int kCB, int kP, class Off>
__device__ __forceinline__ void step_weights_pv(const f32x4 (&s)[kCB][kP],
                                                 const char* const (&vpage)[kP],
                                                 const Off& off, PrefillState (&st)[kCB]) {
  uint32_t hw[kCB][kP][2], lw[kCB][kP][2];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    float pmax = fmaxf(fmaxf(s[cb][0][0], s[cb][0][1]), fmaxf(s[cb][0][2], s[cb][0][3]));
    if constexpr (kP == 2)
      pmax = fmaxf(pmax, fmaxf(fmaxf(s[cb][1][0], s[cb][1][1]), fmaxf(s[cb][1][2], s[cb][1][3])));
    const float pm = max_over_rows(pmax);
    const bool move = pm > st[cb].m + kMaxLag;
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      const float mn = move ? pm : st[cb].m;
      const float alpha = mn == st[cb].m ? 1.0f : fast_exp2(st[cb].m - mn);
      st[cb].m = mn;
      st[cb].l *= alpha;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) st[cb].acc[nb] *= alpha;
    }
    const float mu = st[cb].m == -INFINITY ? 0.0f : st[cb].m;
#pragma unroll
    for (int j = 0; j < kP; ++j) {
      float p[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) p[v] = fast_exp2(s[cb][j][v] - mu);
      st[cb].l += (p[0] + p[1]) + (p[2] + p[3]);
      hw[cb][j][0] = pack_bf16x2(p[0], p[1]);
      hw[cb][j][1] = pack_bf16x2(p[2], p[3]);
      lw[cb][j][0] = pack_bf16x2(p[0] - bf16_lo(hw[cb][j][0]), p[1] - bf16_hi(hw[cb][j][0]));
      lw[cb][j][1] = pack_bf16x2(p[2] - bf16_lo(hw[cb][j][1]), p[3] - bf16_hi(hw[cb][j][1]));
    }
  }
  if constexpr (kP == 2) {
    bf16x8 bh[kCB], bl[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      bh[cb] = __builtin_bit_cast(bf16x8, u32x4{hw[cb][0][0], hw[cb][0][1], hw[cb][1][0], hw[cb][1][1]});
      bl[cb] = __builtin_bit_cast(bf16x8, u32x4{lw[cb][0][0], lw[cb][0][1], lw[cb][1][0], lw[cb][1][1]});
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const u32x2 t0 = read_v_tr(vpage[0], off.v(nb));
      const u32x2 t1 = read_v_tr(vpage[1], off.v(nb));
      const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{t0[0], t0[1], t1[0], t1[1]});
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        st[cb].acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh[cb], st[cb].acc[nb], 0, 0, 0);
        st[cb].acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl[cb], st[cb].acc[nb], 0, 0, 0);
      }
    }
  } else {
    bf16x8 bw[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
      bw[cb] = __builtin_bit_cast(bf16x8, u32x4{hw[cb][0][0], hw[cb][0][1], lw[cb][0][0], lw[cb][0][1]});
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const u32x2 t0 = read_v_tr(vpage[0], off.v(nb));
      const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{t0[0], t0[1], t0[0], t0[1]});
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
        st[cb].acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bw[cb], st[cb].acc[nb], 0, 0, 0);
    }
  }
}

// Chunks of several tiles (prefill, longer verification): the tiles of one
// KV head share each K/V page through LDS.  A workgroup of 4 waves, one per
// SIMD, takes one sequence, kHG = 4 / kTG KV heads and kTG consecutive wave
// tiles, one (head, wave tile) per wave: 4 wave tiles of one head for long
// chunks, 2 of 2 heads for chunks of two tiles.  A wave tile is kCB
// 16-column blocks of 16/G tokens each: with kCB = 2 (long chunks, where the
// grid still gives two workgroups per compute unit) every K and V value the
// wave reads from LDS feeds the products of both blocks, which halves the LDS
// traffic per product.  Two workgroups share a CU, and since each waits only
// at its own barriers, one's matrix-core products overlap the other's LDS
// traffic and softmax; at 8 waves per workgroup the barrier put every wave of
// the CU in the same phase, and the CU's matrix cores ran about half the
// time.  Pages go in steps of kP (2 with one head and one block, else 1, for
// the registers): per step the 256 threads load the heads' K and V tiles of
// the step's pages (one 16-byte piece of K and one of V per thread, page and
// head, kDepth steps in flight) and write them to one of three LDS stages --
// K with its 16-byte pieces XOR-swizzled by position (kswz), so that the
// score product's reads (16 positions at one dim offset) fall on distinct
// banks, V swizzled for the transpose reads (vswz) and zero past the
// sequence or past the last page; each wave then scores the step's pages
// (step_scores, per block) and, one step later, weighs them and sums V
// (step_weights_pv).  The queries enter the score product as two bf16 terms
// (to a relative 2^-18, the weights' own precision) rather than the decode's
// three, which takes a sixth of the products.  The cache is read once per
// kTG wave tiles, and the workgroups of one KV head (kTG = 4) are consecutive
// modulo 8, which keeps them on one XCD, where they share the pages through
// L2.

constexpr int kChunkWaves = 4;                // (head, tile) pairs per workgroup
constexpr int kChunkQTerms = 2;               // bf16 terms of each query element
constexpr int kChunkPrefillMinTiles = 2;      // chunks of this many tiles share pages
constexpr int kChunkWideMinGroups = 512;      // workgroups two-block waves must still give

template <int kG, int kTG, int kCB>
__global__ __launch_bounds__(kWave * kChunkWaves, 2) void chunk_prefill_kernel(ChunkArgs a) {
  constexpr int kH = kG * kKvHeads;
  constexpr int kTpb = 16 / kG;            // tokens per block
  constexpr int kTpt = kCB * kTpb;         // tokens per wave tile
  constexpr int kHG = kChunkWaves / kTG;   // KV heads per workgroup
  constexpr int kP = kHG == 1 && kCB == 1 ? 2 : 1;  // pages per step
  constexpr int kDepth = kHG == 1 ? 4 : 2;  // steps in flight (8 to 16 pieces per thread)
  using TileV = Tile<DAH_BF16>;
  constexpr int kTileBytes = (int)TileV::kTileBytes;
  constexpr int kHeadBytes = 2 * kTileBytes;  // K and V of one head and page in a stage
  constexpr int kPageBytes = kHG * kHeadBytes;
  static_assert(kHG * kTG == kChunkWaves && kKvHeads % kHG == 0 && kHG <= 2,
                "heads x tiles = 4 waves");
  static_assert(kWave * kChunkWaves * 16 == kTileBytes, "one 16-byte piece per thread and tile");
  __shared__ __attribute__((aligned(16))) char stage[3][kP * kPageBytes];  // [stage][page][head][K|V]
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = wave / kTG, tw = wave - hw * kTG;   // the wave's local head and tile
  const int row = lane >> 4, col = lane & 15;
  const int wides = (a.tiles + kCB - 1) / kCB;
  const int groups = (wides + kTG - 1) / kTG;
  constexpr int kHeadGroups = kKvHeads / kHG;
  const int gh = blockIdx.x % kHeadGroups;
  const int bg = blockIdx.x / kHeadGroups;
  const int b = bg / groups;
  const int grp = bg - b * groups;
  const int g = gh * kHG + hw;   // the wave's KV head
  const int t0 = min(max(a.cu_tokens[b], 0), a.total);
  const int t1 = min(max(a.cu_tokens[b + 1], t0), a.total);
  const int n = t1 - t0;
  const int tile0 = grp * kTG;   // first wave tile of the workgroup
  if (tile0 * kTpt >= n) return;  // the whole workgroup
  const int tile = tile0 + tw;
  const int i0 = tile * kTpt;
  const bool live = i0 < n;       // wave-uniform
  const int seq_len = a.seq_lens[b];
  if (n > a.max_chunk || seq_len < n || seq_len > a.max_seq_len) {
    // Outside the preconditions: NaN for the wave's tokens (and, from tile
    // 0, for tokens past the tiles), nothing read from the cache.
    auto poison = [&](int from, int to) {
      for (int i = from; i < to; ++i)
        for (int h = 0; h < kG; ++h)
          reinterpret_cast<float2*>(a.o + (((size_t)t0 + i) * kH + g * kG + h) * kHeadDim)[lane] =
              make_float2(NAN, NAN);
    };
    if (live && kCB * tile < a.tiles) poison(i0, min(n, min(i0 + kTpt, a.tiles * kTpb)));
    if (tile == 0) poison(a.tiles * kTpb, n);
    return;  // the whole workgroup (the condition is uniform)
  }

  // Within the preconditions every live token is below a.tiles * kTpb.
  const int ntok = live ? min(kTpt, n - i0) : 1;
  const int pos0 = seq_len - n + i0;  // position of the wave's first token
  const int pmax = pos0 + ntok - 1;
  const int wave_last = live ? pmax / kPage : -1;  // last page this wave attends
  const int first_masked = (pos0 + 1) / kPage;
  const int group_tokens = min(n, (tile0 + kTG) * kTpt);
  const int last = (seq_len - n + group_tokens - 1) / kPage;  // last page of any wave
  const int ti = col / kG, hh = col - ti * kG;
  bool col_live[kCB];
  int climit_pos[kCB];
  size_t qrow[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const int tok = cb * kTpb + ti;
    col_live[cb] = live && ti < kTpb && tok < ntok;
    climit_pos[cb] = pos0 + (col_live[cb] ? tok : ntok - 1);
    qrow[cb] = ((size_t)t0 + (live ? i0 : 0) + (col_live[cb] ? tok : 0)) * kH + g * kG +
               (col_live[cb] ? hh : 0);
  }

  typedef const __attribute__((address_space(4))) int32_t* ConstI32;
  const ConstI32 bt = (ConstI32)(a.block_table + (size_t)b * a.max_pages_per_seq);
  const int64_t page_bytes = (int64_t)kKvHeads * kTileBytes;
  // This thread's 16-byte piece of every page and head's K and V tiles, and
  // its places in the stage (K and V swizzled).
  const char* ksrc = a.k_cache + (int64_t)gh * kHG * kTileBytes + 16 * tid;
  const char* vsrc = a.v_cache + (int64_t)gh * kHG * kTileBytes + 16 * tid;
  const int ppos = tid >> 4, pc = tid & 15;
  const int kdst = 256 * ppos + 16 * (pc ^ kswz(ppos));
  const int vdst = kTileBytes + 256 * ppos + 16 * (pc ^ (2 * vswz(ppos)));
  bool bad_page = false;
  // The pieces of step s's pages.  Every step loads -- pages past `last`
  // as page `last` again (their scores are masked, their V staged as zeros)
  // -- so that no load is conditional and the wait for a ring slot counts
  // only the loads issued before it.
  auto fetch = [&](u32x4 (&out)[kP][kHG][2], int s) {
#pragma unroll
    for (int j = 0; j < kP; ++j) {
      const int p = kP * s + j;
      const int id = bt[min(p, last)];
      const bool ok = id >= 0 && id < a.num_pages;
      bad_page |= !ok && p <= wave_last;
      const int64_t off = (int64_t)(ok ? id : 0) * page_bytes;
#pragma unroll
      for (int h = 0; h < kHG; ++h) {
        out[j][h][0] = *reinterpret_cast<const u32x4*>(ksrc + off + h * kTileBytes);
        out[j][h][1] = *reinterpret_cast<const u32x4*>(vsrc + off + h * kTileBytes);
      }
    }
  };
  // Steps in whole rings: those past the last page only stage (no wave
  // works on them).
  const int steps = (last + kP) / kP;
  const int steps_run = (steps + kDepth - 1) / kDepth * kDepth;
  u32x4 ring[kDepth][kP][kHG][2];
#pragma unroll
  for (int i = 0; i < kDepth; ++i) fetch(ring[i], i);

  const float qscale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
  u32x4 qb[kCB][4][kChunkQTerms];
  PrefillState st[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    float qv[4][8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) load8(a.q + qrow[cb] * kHeadDim + 32 * kk + 8 * row, qv[kk]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[kk][e] *= qscale;
      split_terms<kChunkQTerms>(qv[kk], qb[cb][kk]);
    }
    if (!col_live[cb]) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int t = 0; t < kChunkQTerms; ++t) qb[cb][kk][t] = u32x4{0u, 0u, 0u, 0u};
    }
    st[cb].m = -INFINITY;
    st[cb].l = 0.0f;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) st[cb].acc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // K: lane (row, col) reads row sigma(col) of the score product, pieces
  // row + 4 kk (swizzled).  V: transpose reads of position 4 (col / 4) + row,
  // dims 16 nb + 4 (col mod 4) of its head.  (row + 4 kk) ^ kswz splits into
  // the low two bits and the rest, since the two addends share no bit.
  const int kpos = 4 * (col & 3) + (col >> 2);  // sigma(col)
  const int kb = hw * kHeadBytes + 256 * kpos + 16 * (row ^ (kswz(kpos) & 3));
  const int kq = kswz(kpos) >> 2;
  const int vP = 4 * (col >> 2) + row;
  const int vb = hw * kHeadBytes + kTileBytes + 256 * vP + 16 * ((col & 3) >> 1) + 8 * (col & 1);
  const int vx = vswz(vP);
  StageOffsets<kCB == 1> off;
  if constexpr (kCB == 1) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) off.ko[kk] = kb + 64 * (kk ^ kq);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) off.vo[nb] = vb + 32 * (nb ^ vx);
  } else {
    off = StageOffsets<false>{kb, kq, vb, vx};
  }

  // Software pipeline across steps: after step s's barrier a wave issues
  // the score products of step s, then the softmax and V sum of step s - 1
  // (whose V is still in its stage), so the matrix cores work on one while
  // the VALU works on the other.  Three stages: step s writes stage s mod 3,
  // last read by step s - 3's K reads and step s - 2's V sum, both before
  // barrier s - 1.
  f32x4 sprev[kCB][kP];
  bool prev_on = false;  // step s - 1 awaits its softmax and V sum
  int cur = 0;           // stage of step s
  int prev = 0;          // stage of step s - 1
  for (int s0 = 0; s0 < steps_run; s0 += kDepth) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      const int s = s0 + i;
      char* stg = &stage[cur][0];
#pragma unroll
      for (int j = 0; j < kP; ++j) {
        // V rows past the sequence (never written) or past the last page
        // are staged as zeros.
        const bool past = kP * s + j > last || kPage * (kP * s + j) + ppos >= seq_len;
#pragma unroll
        for (int h = 0; h < kHG; ++h) {
          char* at = stg + j * kPageBytes + h * kHeadBytes;
          *reinterpret_cast<u32x4*>(at + kdst) = ring[i][j][h][0];
          *reinterpret_cast<u32x4*>(at + vdst) = past ? u32x4{0u, 0u, 0u, 0u} : ring[i][j][h][1];
        }
      }
      __syncthreads();
      fetch(ring[i], s + kDepth);
      const int p0 = kP * s;
      const bool on = p0 <= wave_last;
      f32x4 scur[kCB][kP];
      if (on) {
        KTileMfma K[kP];
#pragma unroll
        for (int j = 0; j < kP; ++j) {
          const char* sp = stg + j * kPageBytes;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) K[j].w[kk] = *reinterpret_cast<const u32x4*>(sp + off.k(kk));
        }
        if (p0 + kP - 1 < first_masked && p0 + kP - 1 <= wave_last) {
          const int cl[kP] = {};
#pragma unroll
          for (int cb = 0; cb < kCB; ++cb) step_scores<kP, false>(K, qb[cb], lane, cl, scur[cb]);
        } else {
#pragma unroll
          for (int cb = 0; cb < kCB; ++cb) {
            int cl[kP];
#pragma unroll
            for (int j = 0; j < kP; ++j) {
              const int p = p0 + j;
              cl[j] = p > wave_last ? 0 : p < first_masked ? kPage : climit_pos[cb] - kPage * p + 1;
            }
            step_scores<kP, true>(K, qb[cb], lane, cl, scur[cb]);
          }
        }
      }
      if (prev_on) {
        const char* vpage[kP];
#pragma unroll
        for (int j = 0; j < kP; ++j) vpage[j] = &stage[prev][j * kPageBytes];
        step_weights_pv<kCB, kP>(sprev, vpage, off, st);
      }
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int j = 0; j < kP; ++j) sprev[cb][j] = scur[cb][j];
      prev_on = on;
      prev = cur;
      cur = cur == 2 ? 0 : cur + 1;
    }
  }
  if (prev_on) {
    const char* vpage[kP];
#pragma unroll
    for (int j = 0; j < kP; ++j) vpage[j] = &stage[prev][j * kPageBytes];
    step_weights_pv<kCB, kP>(sprev, vpage, off, st);
  }
  if (!live) return;

#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    float l = st[cb].l;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!col_live[cb]) continue;
    const float scale = bad_page ? NAN : 1.0f / l;
    float* orow = a.o + (((size_t)t0 + i0 + cb * kTpb + ti) * kH + g * kG + hh) * kHeadDim + 4 * row;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      *reinterpret_cast<float4*>(orow + 16 * nb) =
          make_float4(st[cb].acc[nb][0] * scale, st[cb].acc[nb][1] * scale,
                      st[cb].acc[nb][2] * scale, st[cb].acc[nb][3] * scale);
  }
}

template <int kG, int kTG, int kCB>
void launch_chunk_prefill(const ChunkArgs& c, int B, hipStream_t stream) {
  const long long groups = ((c.tiles + kCB - 1) / kCB + kTG - 1) / kTG;
  const long long heads = kKvHeads / (kChunkWaves / kTG);
  chunk_prefill_kernel<kG, kTG, kCB>
      <<<dim3((unsigned)((long long)B * groups * heads)), kWave * kChunkWaves, 0, stream>>>(c);
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

// The allocation-free step's scratch (decode_attn_step_noalloc): the split
// partials and prefix sums that decode_attn_step_ex keeps in the caller's
// workspace.  Each device that loads the library holds its own copy until
// the process ends; every call on a device shares it.  Host code reaches it
// only through the device address hipGetSymbolAddress returns for that
// device (the array's name is a host-side stand-in, not a device pointer).
static __device__ __align__(256) unsigned char scratch[DAH_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[64];
std::mutex g_scratch_mutex;

// This device's address of `scratch`, looked up once per device (with the
// device current) and kept.
int device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return dah::set_error(DAH_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64)
    return dah::set_error(DAH_ERR_HIP, "device %d: the static scratch serves devices 0..63", dev);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return dah::set_error(DAH_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                              hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return DAH_OK;
}

// Calls f(std::integral_constant<int, G>{}) with the number G of query heads
// per KV head; num_heads is one of 16, 32, 40, 64 (checked by the caller).
template <class F>
void with_group(int num_heads, F&& f) {
  switch (num_heads) {
    case 32: f(std::integral_constant<int, 4>{}); break;
    case 40: f(std::integral_constant<int, 5>{}); break;
    case 64: f(std::integral_constant<int, 8>{}); break;
    default: f(std::integral_constant<int, 2>{}); break;
  }
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
                  int max_pages_per_seq, const int32_t* seq_lens, int B, int num_heads,
                  int max_len, float* q_out, hipStream_t stream) {
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
  with_group(num_heads, [&](auto grp) {
    constexpr int kG = decltype(grp)::value;
    if (cache_dtype == DAH_BF16)
      norm_rope_append_kernel<DAH_BF16, kG><<<B, 512, 0, stream>>>(a);
    else
      norm_rope_append_kernel<DAH_F32, kG><<<B, 512, 0, stream>>>(a);
  });
  return check_launch("norm_rope_append_kernel");
}

// The chunk step: every chunk token normed, rotated and appended, then the
// causal attention of the chunks (two launches).
int launch_chunk(const float* q, const float* k_new, const float* v_new, const float* q_gain,
                 const float* k_gain, float eps, float rope_theta, void* k_cache, void* v_cache,
                 int cache_dtype, int64_t num_pages, const int32_t* block_table,
                 int max_pages_per_seq,
                 const int32_t* seq_lens, const int32_t* cu_tokens, int B, int total,
                 int max_chunk, int max_seq_len, int num_heads, float* q_out, float* o,
                 hipStream_t stream) {
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
  a.max_len = max_seq_len;
  a.q_out = q_out;
  ChunkArgs c;
  c.q = q_out;
  c.k_cache = static_cast<const char*>(k_cache);
  c.v_cache = static_cast<const char*>(v_cache);
  c.num_pages = static_cast<int>(num_pages);
  c.block_table = block_table;
  c.max_pages_per_seq = max_pages_per_seq;
  c.seq_lens = seq_lens;
  c.cu_tokens = cu_tokens;
  c.total = total;
  c.max_chunk = max_chunk;
  c.max_seq_len = max_seq_len;
  c.o = o;
  int st = DAH_OK;
  if (cache_dtype == DAH_F32) {
    DecodeArgs d = {};
    d.q = q_out;
    d.k_cache = static_cast<const char*>(k_cache);
    d.v_cache = static_cast<const char*>(v_cache);
    d.num_pages = static_cast<int>(num_pages);
    d.block_table = block_table;
    d.max_pages_per_seq = max_pages_per_seq;
    d.seq_lens = seq_lens;
    d.B = B;
    d.max_seq_len = max_seq_len;
    d.splits = 1;
    d.grid_splits = 1;
    d.pages_per_split = max_pages_per_seq;
    d.o = o;
    with_group(num_heads, [&](auto grp) {
      constexpr int kG = decltype(grp)::value;
      norm_rope_append_chunk_kernel<DAH_F32, kG>
          <<<dim3((unsigned)((long long)B * max_chunk)), 512, 0, stream>>>(a, cu_tokens, max_chunk,
                                                                           total);
      st = check_launch("norm_rope_append_chunk_kernel");
      if (st != DAH_OK) return;
      chunk_valu_kernel<kG><<<dim3((unsigned)((long long)B * max_chunk)),
                              kWave * kDecodeWavesPerBlock, 0, stream>>>(d, cu_tokens, total,
                                                                         max_chunk);
      st = check_launch("chunk_valu_kernel");
    });
    return st;
  }
  with_group(num_heads, [&](auto grp) {
    constexpr int kG = decltype(grp)::value;
    constexpr int kTpt = 16 / kG;
    norm_rope_append_chunk_kernel<DAH_BF16, kG>
        <<<dim3((unsigned)((long long)B * max_chunk)), 512, 0, stream>>>(a, cu_tokens, max_chunk,
                                                                         total);
    st = check_launch("norm_rope_append_chunk_kernel");
    if (st != DAH_OK) return;
    c.tiles = (max_chunk + kTpt - 1) / kTpt;
    if (c.tiles >= kChunkPrefillMinTiles) {
      // Tiles per workgroup: 2 for chunks of two tiles (2 KV heads per
      // workgroup), else 4 of one head -- 4 waves of two 16-column blocks
      // each where that still gives two workgroups per compute unit.
      const long long wide_groups = ((c.tiles + 1) / 2 + 3) / 4;
      if (c.tiles <= 2)
        launch_chunk_prefill<kG, 2, 1>(c, B, stream);
      else if ((long long)B * kKvHeads * wide_groups >= kChunkWideMinGroups)
        launch_chunk_prefill<kG, 4, 2>(c, B, stream);
      else
        launch_chunk_prefill<kG, 4, 1>(c, B, stream);
      st = check_launch("chunk_prefill_kernel");
    } else {
      chunk_attn_kernel<kG><<<dim3((unsigned)((long long)B * c.tiles)),
                              kWave * kDecodeWavesPerBlock, 0, stream>>>(c);
      st = check_launch("chunk_attn_kernel");
    }
  });
  return st;
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

int plan_for(int B, int num_heads, int cache_dtype, int max_seq_len, int num_splits,
             void* workspace, size_t workspace_bytes, dah::Plan* plan) {
  int cus = 0;
  int st = device_cu_count(&cus);
  if (st != DAH_OK) return st;
  st = dah::plan_decode(B, num_heads, cache_dtype, max_seq_len, num_splits, cus, plan);
  if (st != DAH_OK) return st;
  if (plan->workspace > 0) {
    if (workspace == nullptr || workspace_bytes < plan->workspace)
      return dah::set_error(DAH_ERR_WORKSPACE,
                            "workspace of %zu bytes, need %zu (B=%d, %d heads, max_seq_len=%d)",
                            workspace == nullptr ? (size_t)0 : workspace_bytes, plan->workspace, B,
                            num_heads, max_seq_len);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return dah::set_error(DAH_ERR_ALIGN, "workspace needs 256-byte alignment");
  }
  return DAH_OK;
}

// The kernel the plan chose: the matrix-core form for a bfloat16 cache when
// plan.mfma (always for 4+ query heads per KV head), else the VALU form.
template <bool kStep, int kG>
void launch_decode_kernel(const dah::Plan& plan, bool bf16, const DecodeArgs& a,
                          hipStream_t stream) {
  const dim3 grid((unsigned)plan.workgroups), block(kWave * kDecodeWavesPerBlock);
  const bool balanced = plan.mode == DAH_PLAN_BALANCED;
  if (!bf16) {
    if (balanced)
      decode_balanced_kernel<DAH_F32, kStep, kG, false><<<grid, block, 0, stream>>>(a);
    else
      decode_split_kernel<DAH_F32, kStep, kG, false><<<grid, block, 0, stream>>>(a);
  } else if (plan.mfma) {
    if (balanced)
      decode_balanced_kernel<DAH_BF16, kStep, kG, true><<<grid, block, 0, stream>>>(a);
    else
      decode_split_kernel<DAH_BF16, kStep, kG, true><<<grid, block, 0, stream>>>(a);
  } else if constexpr (kG < 4) {
    if (balanced)
      decode_balanced_kernel<DAH_BF16, kStep, kG, false><<<grid, block, 0, stream>>>(a);
    else
      decode_split_kernel<DAH_BF16, kStep, kG, false><<<grid, block, 0, stream>>>(a);
  }
}

// Decode (step == nullptr: q is already normed and roped) or the fused
// decode step (q is raw; the kernel norms, rotates and appends).
int launch_decode(const dah::Plan& plan, const float* q, const void* k_cache,
                  const void* v_cache, int cache_dtype, int64_t num_pages,
                  const int32_t* block_table, int max_pages_per_seq, const int32_t* seq_lens,
                  int B, int num_heads, int max_seq_len, float* o, void* workspace,
                  const StepInputs* step, hipStream_t stream) {
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
  a.splits = plan.mode == DAH_PLAN_SPLIT ? plan.splits : 1;
  a.grid_splits = plan.mode == DAH_PLAN_SPLIT ? plan.grid_splits : 1;
  a.pages_per_split = plan.pages_per_split;
  a.o = o;
  // Workspace: partial rows (128 floats each), their (max, sum) pairs, then
  // for the balanced plan the page prefix sums.
  float* ws = static_cast<float*>(workspace);
  const size_t rows =
      plan.mode == DAH_PLAN_BALANCED ? ((size_t)B + plan.workgroups - 1) * num_heads
      : plan.mode == DAH_PLAN_SPLIT  ? (size_t)B * num_heads * plan.splits
                                     : 0;
  a.part_acc = rows > 0 ? ws : nullptr;
  a.part_ml = rows > 0 ? ws + rows * kHeadDim : nullptr;
  a.prefix = plan.mode == DAH_PLAN_BALANCED
                 ? reinterpret_cast<int32_t*>(ws + rows * (kHeadDim + 2))
                 : nullptr;
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
  const bool bf16 = cache_dtype == DAH_BF16;
  with_group(num_heads, [&](auto grp) {
    constexpr int kG = decltype(grp)::value;
    if (step == nullptr)
      launch_decode_kernel<false, kG>(plan, bf16, a, stream);
    else
      launch_decode_kernel<true, kG>(plan, bf16, a, stream);
  });
  int st = check_launch("decode kernel");
  if (st != DAH_OK || plan.mode == DAH_PLAN_PER_SEQUENCE) return st;
  const int cblocks = B * num_heads;  // one workgroup per (sequence, head)
  static_assert(kBalancedMergeRows == 2, "every head count is even");
  if (plan.mode == DAH_PLAN_BALANCED)
    combine_balanced_kernel<<<cblocks / kBalancedMergeRows, kBalancedMergeThreads, 0, stream>>>(
        a.part_acc, a.part_ml, a.prefix, seq_lens, B, num_heads, plan.workgroups, o);
  else
    combine_splits_kernel<<<cblocks, kCombineThreads, 0, stream>>>(
        a.part_acc, a.part_ml, seq_lens, num_heads, max_seq_len, plan.splits,
        plan.pages_per_split, o);
  return check_launch("combine kernel");
}

}  // namespace

extern "C" {

int qk_norm_rope_append_ex(const float* q, const float* k_new, const float* v_new,
                           const float* q_gain, const float* k_gain, float eps, float rope_theta,
                           void* k_cache, void* v_cache, int cache_dtype, int64_t num_pages,
                           const int32_t* block_table, int max_pages_per_seq,
                           const int32_t* seq_lens, int B, int num_heads, float* q_out,
                           void* stream) {
  int st = dah::validate_append(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache,
                                v_cache, cache_dtype, num_pages, block_table, max_pages_per_seq,
                                seq_lens, B, num_heads, q_out);
  if (st != DAH_OK) return st;
  const long long max_len = (long long)max_pages_per_seq * kPage;
  return launch_append(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache, v_cache,
                       cache_dtype, num_pages, block_table, max_pages_per_seq, seq_lens, B,
                       num_heads, max_len > INT32_MAX ? INT32_MAX : (int)max_len, q_out,
                       static_cast<hipStream_t>(stream));
}

int qk_norm_rope_append(const float* q, const float* k_new, const float* v_new,
                        const float* q_gain, const float* k_gain, float eps, float rope_theta,
                        void* k_cache, void* v_cache, int cache_dtype, int64_t num_pages,
                        const int32_t* block_table, int max_pages_per_seq,
                        const int32_t* seq_lens, int B, float* q_out, void* stream) {
  return qk_norm_rope_append_ex(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache,
                                v_cache, cache_dtype, num_pages, block_table, max_pages_per_seq,
                                seq_lens, B, kHeads, q_out, stream);
}

int paged_decode_gqa_ex(const float* q, const void* k_cache, const void* v_cache,
                        int cache_dtype, int64_t num_pages, const int32_t* block_table,
                        int max_pages_per_seq, const int32_t* seq_lens, int B, int num_heads,
                        int max_seq_len, int num_splits, float* o, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int st = dah::validate_decode(q, k_cache, v_cache, cache_dtype, num_pages, block_table,
                                max_pages_per_seq, seq_lens, B, num_heads, max_seq_len,
                                num_splits, o);
  if (st != DAH_OK) return st;
  dah::Plan plan;
  st = plan_for(B, num_heads, cache_dtype, max_seq_len, num_splits, workspace, workspace_bytes,
                &plan);
  if (st != DAH_OK) return st;
  return launch_decode(plan, q, k_cache, v_cache, cache_dtype, num_pages, block_table,
                       max_pages_per_seq, seq_lens, B, num_heads, max_seq_len, o, workspace,
                       nullptr, static_cast<hipStream_t>(stream));
}

int paged_decode_gqa(const float* q, const void* k_cache, const void* v_cache, int cache_dtype,
                     int64_t num_pages, const int32_t* block_table, int max_pages_per_seq,
                     const int32_t* seq_lens, int B, int max_seq_len, int num_splits, float* o,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return paged_decode_gqa_ex(q, k_cache, v_cache, cache_dtype, num_pages, block_table,
                             max_pages_per_seq, seq_lens, B, kHeads, max_seq_len, num_splits, o,
                             workspace, workspace_bytes, stream);
}

int decode_attn_step_ex(const float* q, const float* k_new, const float* v_new,
                        const float* q_gain, const float* k_gain, float eps, float rope_theta,
                        void* k_cache, void* v_cache, int cache_dtype, int64_t num_pages,
                        const int32_t* block_table, int max_pages_per_seq,
                        const int32_t* seq_lens, int B, int num_heads, int max_seq_len,
                        int num_splits, float* q_out, float* o, void* workspace,
                        size_t workspace_bytes, void* stream) {
  // q_out may be NULL (o only): the pointer checks then take q in its place.
  const float* q_out_chk = q_out != nullptr ? q_out : q;
  int st = dah::validate_append(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache,
                                v_cache, cache_dtype, num_pages, block_table, max_pages_per_seq,
                                seq_lens, B, num_heads, q_out_chk);
  if (st != DAH_OK) return st;
  st = dah::validate_decode(q_out_chk, k_cache, v_cache, cache_dtype, num_pages, block_table,
                            max_pages_per_seq, seq_lens, B, num_heads, max_seq_len, num_splits,
                            o);
  if (st != DAH_OK) return st;
  // Plan and check the workspace before anything is launched, so that a
  // failing call leaves the cache untouched.
  dah::Plan plan;
  st = plan_for(B, num_heads, cache_dtype, max_seq_len, num_splits, workspace, workspace_bytes,
                &plan);
  if (st != DAH_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q_out == q && plan.mode != DAH_PLAN_PER_SEQUENCE) {
    // In place with several splits: the workgroups of one sequence would read
    // q while another overwrites it, so norm and rotate first, then decode.
    st = launch_append(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache, v_cache,
                       cache_dtype, num_pages, block_table, max_pages_per_seq, seq_lens, B,
                       num_heads, max_seq_len, q_out, s);
    if (st != DAH_OK) return st;
    return launch_decode(plan, q_out, k_cache, v_cache, cache_dtype, num_pages, block_table,
                         max_pages_per_seq, seq_lens, B, num_heads, max_seq_len, o, workspace,
                         nullptr, s);
  }
  // One launch: the decode kernel norms and rotates q, writes q_out, and
  // appends the new key and value (see decode_split_kernel).
  const StepInputs step = {k_new, v_new, q_gain, k_gain, eps, rope_theta, q_out, k_cache, v_cache};
  return launch_decode(plan, q, k_cache, v_cache, cache_dtype, num_pages, block_table,
                       max_pages_per_seq, seq_lens, B, num_heads, max_seq_len, o, workspace,
                       &step, s);
}

int decode_attn_step(const float* q, const float* k_new, const float* v_new,
                     const float* q_gain, const float* k_gain, float eps, float rope_theta,
                     void* k_cache, void* v_cache, int cache_dtype, int64_t num_pages,
                     const int32_t* block_table, int max_pages_per_seq,
                     const int32_t* seq_lens, int B, int max_seq_len, int num_splits,
                     float* q_out, float* o, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return decode_attn_step_ex(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache, v_cache,
                             cache_dtype, num_pages, block_table, max_pages_per_seq, seq_lens, B,
                             kHeads, max_seq_len, num_splits, q_out, o, workspace,
                             workspace_bytes, stream);
}

int decode_attn_step_noalloc(const float* q, const float* k_new, const float* v_new,
                             const float* q_gain, const float* k_gain, float eps,
                             float rope_theta, void* k_cache, void* v_cache, int cache_dtype,
                             int64_t num_pages, const int32_t* block_table,
                             int max_pages_per_seq, const int32_t* seq_lens, int B,
                             int num_heads, int max_seq_len, int num_splits, float* q_out,
                             float* o, void* stream) {
  const float* q_out_chk = q_out != nullptr ? q_out : q;
  int st = dah::validate_append(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache,
                                v_cache, cache_dtype, num_pages, block_table, max_pages_per_seq,
                                seq_lens, B, num_heads, q_out_chk);
  if (st != DAH_OK) return st;
  st = dah::validate_decode(q_out_chk, k_cache, v_cache, cache_dtype, num_pages, block_table,
                            max_pages_per_seq, seq_lens, B, num_heads, max_seq_len, num_splits,
                            o);
  if (st != DAH_OK) return st;
  int cus = 0;
  st = device_cu_count(&cus);
  if (st != DAH_OK) return st;
  dah::Plan plan;
  st = dah::plan_decode(B, num_heads, cache_dtype, max_seq_len, num_splits, cus, &plan);
  if (st != DAH_OK) return st;
  if (plan.workspace > DAH_SCRATCH_BYTES)
    return dah::set_error(DAH_ERR_WORKSPACE,
                          "decode_attn_step_noalloc: the plan needs %zu bytes of scratch, the "
                          "static scratch holds %zu (B=%d, %d heads, max_seq_len=%d, "
                          "num_splits=%d); use decode_attn_step_ex with a workspace",
                          plan.workspace, (size_t)DAH_SCRATCH_BYTES, B, num_heads, max_seq_len,
                          num_splits);
  void* ws = nullptr;
  st = device_scratch(&ws);
  if (st != DAH_OK) return st;
  return decode_attn_step_ex(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache, v_cache,
                             cache_dtype, num_pages, block_table, max_pages_per_seq, seq_lens, B,
                             num_heads, max_seq_len, num_splits, q_out, o, ws,
                             DAH_SCRATCH_BYTES, stream);
}

int chunk_attn_step(const float* q, const float* k_new, const float* v_new, const float* q_gain,
                    const float* k_gain, float eps, float rope_theta, void* k_cache,
                    void* v_cache, int cache_dtype, int64_t num_pages,
                    const int32_t* block_table, int max_pages_per_seq, const int32_t* seq_lens,
                    const int32_t* cu_tokens, int B, int total_tokens, int max_chunk,
                    int max_seq_len, int num_heads, float* q_out, float* o, void* stream) {
  int st = dah::validate_chunk(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache, v_cache,
                               cache_dtype, num_pages, block_table, max_pages_per_seq, seq_lens,
                               cu_tokens, B, total_tokens, max_chunk, max_seq_len, num_heads,
                               q_out, o);
  if (st != DAH_OK) return st;
  return launch_chunk(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache, v_cache,
                      cache_dtype, num_pages, block_table, max_pages_per_seq, seq_lens, cu_tokens, B,
                      total_tokens, max_chunk, max_seq_len, num_heads, q_out, o,
                      static_cast<hipStream_t>(stream));
}

size_t dah_workspace_bytes_ex(int B, int num_heads, int cache_dtype, int max_seq_len,
                              int num_splits) {
  if (cache_dtype != DAH_F32 && cache_dtype != DAH_BF16) return 0;
  int cus = 0;
  if (device_cu_count(&cus) != DAH_OK) return 0;
  dah::Plan p;
  if (dah::plan_decode(B, num_heads, cache_dtype, max_seq_len, num_splits, cus, &p) != DAH_OK)
    return 0;
  return p.workspace;
}

size_t dah_workspace_bytes(int B, int max_seq_len, int num_splits) {
  return dah_workspace_bytes_ex(B, kHeads, DAH_BF16, max_seq_len, num_splits);
}

}  // extern "C"
