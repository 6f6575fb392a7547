// Host-side helpers: validation, split planner, status strings, last error.
// See dah_host.h.  No HIP calls in this file.
#include "dah_host.h"

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dah.h"

namespace dah {

namespace {
thread_local char g_last_error[512] = "";

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Policy, from sweeps of the decode kernel on MI355X (256 compute units):
//  * one workgroup per sequence when the batch alone gives every compute
//    unit a workgroup and no sequence is long;
//  * the balanced decomposition (kBalancedGroupsPerCu workgroups per compute
//    unit) for batches of at least kBalancedMinBatch sequences, where ragged
//    lengths would otherwise leave most of the device idle behind the longest
//    sequences (128 log-uniform lengths: 212 us against 233 us for the best
//    fixed split); from kBalancedMinBatchMfma sequences when 4+ query heads
//    per KV head put the decode on the matrix cores, whose one workgroup per
//    compute unit gains more from even work (32 sequences of 512-4096
//    positions, 40 heads: 61 us against 73 us; at 16 heads 58.7 us against
//    56.8 us for fixed splits on the VALU kernel);
//  * fixed splits, spread over the XCDs, for fewer sequences (4 long ones:
//    88 us against 97 us balanced), keeping splits between kMinPagesPerSplit
//    and kMaxPagesPerSplit pages and aiming at kTargetWavesPerCu waves.
// Kernel: with a bfloat16 cache the matrix-core decode runs for 4+ query
// heads per KV head always, and for 2 unless the plan is fixed splits
// (B=256, S=2048: 323 us against 329 us; 128 ragged sequences, balanced:
// 205 against 210; 4 long sequences, split: 95 against 88).
constexpr int kTargetWavesPerCu = 8;
constexpr int kMinPagesPerSplit = 4;
constexpr int kMaxPagesPerSplit = 128;
constexpr int kBalancedGroupsPerCu = 1;
constexpr int kBalancedMinBatch = 64;
constexpr int kBalancedMinBatchMfma = 32;
}  // namespace

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_last_error[0] = '\0'; }

namespace {
size_t partial_bytes(long long slots, int num_heads) {
  return static_cast<size_t>(slots) * num_heads * (kHeadDim + 2) * sizeof(float);
}

int check_heads(int num_heads) {
  if (!valid_heads(num_heads))
    return set_error(DAH_ERR_SHAPE, "num_heads = %d, need 16, 32, 40 or 64 (over 8 KV heads)",
                     num_heads);
  return DAH_OK;
}
}  // namespace

int plan_decode(int B, int num_heads, int cache_dtype, int max_seq_len, int num_splits,
                int num_cus, Plan* out) {
  if (out == nullptr) return set_error(DAH_ERR_NULL, "plan_decode: output pointer is NULL");
  if (B < 1) return set_error(DAH_ERR_SHAPE, "B = %d, need B >= 1", B);
  if (check_heads(num_heads) != DAH_OK) return DAH_ERR_SHAPE;
  if (max_seq_len < 1)
    return set_error(DAH_ERR_SHAPE, "max_seq_len = %d, need >= 1", max_seq_len);
  if (num_splits < 0)
    return set_error(DAH_ERR_SHAPE, "num_splits = %d, need >= 0 (0 = automatic)", num_splits);
  if (num_cus < 1) return set_error(DAH_ERR_SHAPE, "num_cus = %d, need >= 1", num_cus);

  const int max_pages = (max_seq_len + kPage - 1) / kPage;
  const bool bf16 = cache_dtype == DAH_BF16;
  const bool big_group = num_heads / kKvHeads >= 4;
  Plan p = {};
  const bool balanced_fits =
      B <= kMaxBalancedBatch && static_cast<long long>(B) * max_pages < (1LL << 31);
  int want = 0;  // splits for DAH_PLAN_SPLIT
  // DAH_DECODE_PLAN=per_sequence, balanced or split overrides the automatic
  // choice (num_splits == 0) where that plan applies (a measurement aid, read
  // once).
  static const int forced_plan = []() -> int {
    const char* e = getenv("DAH_DECODE_PLAN");
    if (e == nullptr) return -1;
    if (strcmp(e, "per_sequence") == 0) return DAH_PLAN_PER_SEQUENCE;
    if (strcmp(e, "balanced") == 0) return DAH_PLAN_BALANCED;
    if (strcmp(e, "split") == 0) return DAH_PLAN_SPLIT;
    return -1;
  }();
  const bool auto_plan = num_splits == 0 && forced_plan < 0;
  if (num_splits == 1 || (num_splits == 0 && forced_plan == DAH_PLAN_PER_SEQUENCE) ||
      (auto_plan && B >= num_cus && max_pages <= kMaxPagesPerSplit)) {
    p.mode = DAH_PLAN_PER_SEQUENCE;
  } else if (num_splits == 0 && balanced_fits &&
             (forced_plan == DAH_PLAN_BALANCED ||
              (auto_plan && B >= (bf16 && big_group ? kBalancedMinBatchMfma : kBalancedMinBatch)))) {
    p.mode = DAH_PLAN_BALANCED;
  } else {
    p.mode = DAH_PLAN_SPLIT;
    if (num_splits > 0) {
      want = num_splits;
    } else {
      const long long units = static_cast<long long>(B) * kKvHeads;
      const long long target = static_cast<long long>(num_cus) * kTargetWavesPerCu;
      long long w = (target + units - 1) / units;
      long long cap = max_pages / kMinPagesPerSplit;
      if (cap < 1) cap = 1;
      if (w > cap) w = cap;
      const long long floor_splits = (max_pages + kMaxPagesPerSplit - 1) / kMaxPagesPerSplit;
      if (w < floor_splits) w = floor_splits;
      want = static_cast<int>(w < 1 ? 1 : w);
    }
    if (want > max_pages) want = max_pages;
  }

  switch (p.mode) {
    case DAH_PLAN_PER_SEQUENCE:
      p.splits = 1;
      p.pages_per_split = max_pages;
      p.grid_splits = 1;
      p.workgroups = B;
      p.workspace = 0;
      break;
    case DAH_PLAN_BALANCED:
      p.splits = 0;
      p.pages_per_split = 0;
      p.grid_splits = 0;
      p.workgroups = num_cus * kBalancedGroupsPerCu;
      // partial slots, then the batch's page prefix sums (B + 1 int32) that
      // the decode writes for the merge
      p.workspace = partial_bytes(static_cast<long long>(B) + p.workgroups - 1, num_heads) +
                    static_cast<size_t>(B + 1) * sizeof(int32_t);
      break;
    default: {
      const int pps = (max_pages + want - 1) / want;
      p.pages_per_split = pps;
      p.splits = (max_pages + pps - 1) / pps;  // no split past the longest sequence is empty
      if (p.splits == 1) {
        p.mode = DAH_PLAN_PER_SEQUENCE;
        p.grid_splits = 1;
        p.workgroups = B;
        p.workspace = 0;
      } else {
        p.grid_splits = (p.splits + 7) / 8 * 8;
        const long long wg = static_cast<long long>(B) * p.grid_splits;
        if (wg > INT32_MAX) return set_error(DAH_ERR_SHAPE, "grid of %lld workgroups too large", wg);
        p.workgroups = static_cast<int>(wg);
        p.workspace = partial_bytes(static_cast<long long>(B) * p.splits, num_heads);
      }
    }
  }
  p.mfma = bf16 && (big_group || p.mode != DAH_PLAN_SPLIT);
  // DAH_DECODE_KERNEL=valu or =mfma overrides that choice where the other
  // form is built (a measurement aid, read once): the matrix-core form reads
  // a bfloat16 cache only, the VALU form is built for bfloat16 up to 2 query
  // heads per KV head.
  static const int forced = []() -> int {
    const char* e = getenv("DAH_DECODE_KERNEL");
    if (e == nullptr) return -1;
    if (strcmp(e, "valu") == 0) return DAH_KERNEL_VALU;
    if (strcmp(e, "mfma") == 0) return DAH_KERNEL_MFMA;
    return -1;
  }();
  if (forced == DAH_KERNEL_VALU && !big_group) p.mfma = false;
  if (forced == DAH_KERNEL_MFMA && bf16) p.mfma = true;
  *out = p;
  return DAH_OK;
}

int validate_append(const void* q, const void* k_new, const void* v_new, const void* q_gain,
                    const void* k_gain, float eps, float rope_theta, const void* k_cache,
                    const void* v_cache, int cache_dtype, int64_t num_pages,
                    const void* block_table, int max_pages_per_seq, const void* seq_lens, int B,
                    int num_heads, const void* q_out) {
  if (!q || !k_new || !v_new || !q_gain || !k_gain || !k_cache || !v_cache || !block_table ||
      !seq_lens || !q_out)
    return set_error(DAH_ERR_NULL, "qk_norm_rope_append: a required pointer is NULL");
  if (cache_dtype != DAH_F32 && cache_dtype != DAH_BF16)
    return set_error(DAH_ERR_DTYPE, "cache_dtype = %d, need DAH_F32 (0) or DAH_BF16 (1)",
                     cache_dtype);
  if (B < 1) return set_error(DAH_ERR_SHAPE, "B = %d, need B >= 1", B);
  if (check_heads(num_heads) != DAH_OK) return DAH_ERR_SHAPE;
  if (num_pages < 1 || num_pages > INT32_MAX)
    return set_error(DAH_ERR_SHAPE, "num_pages = %lld, need 1 <= num_pages <= 2^31-1",
                     static_cast<long long>(num_pages));
  if (max_pages_per_seq < 1)
    return set_error(DAH_ERR_SHAPE, "max_pages_per_seq = %d, need >= 1", max_pages_per_seq);
  if (!(eps >= 0.0f)) return set_error(DAH_ERR_SHAPE, "eps must be >= 0");
  if (!(rope_theta > 0.0f)) return set_error(DAH_ERR_SHAPE, "rope_theta must be > 0");
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(q_out, 16) ||
      !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(q_gain, 4) ||
      !aligned(k_gain, 4) || !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return set_error(DAH_ERR_ALIGN,
                     "q, k_new, v_new, q_out and the caches need 16-byte alignment; gains, "
                     "block_table and seq_lens 4-byte alignment");
  return DAH_OK;
}

int validate_chunk(const void* q, const void* k_new, const void* v_new, const void* q_gain,
                   const void* k_gain, float eps, float rope_theta, const void* k_cache,
                   const void* v_cache, int cache_dtype, int64_t num_pages,
                   const void* block_table, int max_pages_per_seq, const void* seq_lens,
                   const void* cu_tokens, int B, int total_tokens, int max_chunk, int max_seq_len,
                   int num_heads, const void* q_out, const void* o) {
  int st = validate_append(q, k_new, v_new, q_gain, k_gain, eps, rope_theta, k_cache, v_cache,
                           cache_dtype, num_pages, block_table, max_pages_per_seq, seq_lens, B,
                           num_heads, q_out);
  if (st != DAH_OK) return st;
  if (!cu_tokens || !o) return set_error(DAH_ERR_NULL, "chunk_attn_step: cu_tokens or o is NULL");
  if (total_tokens < 1) return set_error(DAH_ERR_SHAPE, "total_tokens = %d, need >= 1", total_tokens);
  if (max_chunk < 1 || max_chunk > total_tokens)
    return set_error(DAH_ERR_SHAPE, "max_chunk = %d, need 1 <= max_chunk <= total_tokens (%d)",
                     max_chunk, total_tokens);
  if (static_cast<long long>(B) * max_chunk > INT32_MAX)
    return set_error(DAH_ERR_SHAPE, "B * max_chunk too large");
  if (max_seq_len < 1 ||
      static_cast<long long>(max_seq_len) > static_cast<long long>(max_pages_per_seq) * kPage)
    return set_error(DAH_ERR_SHAPE, "max_seq_len = %d, need 1 .. max_pages_per_seq * 16",
                     max_seq_len);
  if (!aligned(cu_tokens, 4) || !aligned(o, 16))
    return set_error(DAH_ERR_ALIGN, "cu_tokens needs 4-byte, o 16-byte alignment");
  return DAH_OK;
}

int validate_linear(const void* x, const void* w, int T, int N, int K, const void* y) {
  if (!x || !w || !y) return set_error(DAH_ERR_NULL, "linear: a required pointer is NULL");
  if (T < 1) return set_error(DAH_ERR_SHAPE, "T = %d, need T >= 1", T);
  if (N < 64 || N % 64 != 0)
    return set_error(DAH_ERR_SHAPE, "N = %d, need a positive multiple of 64", N);
  if (K < 256 || K % 256 != 0)
    return set_error(DAH_ERR_SHAPE, "K = %d, need a positive multiple of 256", K);
  if (static_cast<long long>(T) * K > (1LL << 40) || static_cast<long long>(N) * K > (1LL << 40))
    return set_error(DAH_ERR_SHAPE, "linear: T*K or N*K too large");
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16))
    return set_error(DAH_ERR_ALIGN, "linear: x, w and y need 16-byte alignment");
  return DAH_OK;
}

int validate_decode(const void* q, const void* k_cache, const void* v_cache, int cache_dtype,
                    int64_t num_pages, const void* block_table, int max_pages_per_seq,
                    const void* seq_lens, int B, int num_heads, int max_seq_len, int num_splits,
                    const void* o) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o)
    return set_error(DAH_ERR_NULL, "paged_decode_gqa: a required pointer is NULL");
  if (cache_dtype != DAH_F32 && cache_dtype != DAH_BF16)
    return set_error(DAH_ERR_DTYPE, "cache_dtype = %d, need DAH_F32 (0) or DAH_BF16 (1)",
                     cache_dtype);
  if (B < 1) return set_error(DAH_ERR_SHAPE, "B = %d, need B >= 1", B);
  if (check_heads(num_heads) != DAH_OK) return DAH_ERR_SHAPE;
  if (num_pages < 1 || num_pages > INT32_MAX)
    return set_error(DAH_ERR_SHAPE, "num_pages = %lld, need 1 <= num_pages <= 2^31-1",
                     static_cast<long long>(num_pages));
  if (max_pages_per_seq < 1)
    return set_error(DAH_ERR_SHAPE, "max_pages_per_seq = %d, need >= 1", max_pages_per_seq);
  if (max_seq_len < 1)
    return set_error(DAH_ERR_SHAPE, "max_seq_len = %d, need >= 1", max_seq_len);
  if (static_cast<long long>(max_seq_len) > static_cast<long long>(max_pages_per_seq) * kPage)
    return set_error(DAH_ERR_SHAPE,
                     "max_seq_len = %d exceeds max_pages_per_seq * 16 = %lld", max_seq_len,
                     static_cast<long long>(max_pages_per_seq) * kPage);
  if (num_splits < 0)
    return set_error(DAH_ERR_SHAPE, "num_splits = %d, need >= 0 (0 = automatic)", num_splits);
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return set_error(DAH_ERR_ALIGN,
                     "q, o and the caches need 16-byte alignment; block_table and seq_lens "
                     "4-byte alignment");
  return DAH_OK;
}

}  // namespace dah

extern "C" {

int dah_plan_decode_ex(int B, int num_heads, int cache_dtype, int max_seq_len, int num_splits,
                       int num_cus, dah_decode_plan* out) {
  if (!out) return dah::set_error(DAH_ERR_NULL, "dah_plan_decode: output pointer is NULL");
  if (cache_dtype != DAH_F32 && cache_dtype != DAH_BF16)
    return dah::set_error(DAH_ERR_DTYPE, "cache_dtype = %d, need DAH_F32 (0) or DAH_BF16 (1)",
                          cache_dtype);
  dah::Plan p;
  int st = dah::plan_decode(B, num_heads, cache_dtype, max_seq_len, num_splits, num_cus, &p);
  if (st != DAH_OK) return st;
  out->mode = p.mode;
  out->splits = p.splits;
  out->pages_per_split = p.pages_per_split;
  out->workgroups = p.workgroups;
  out->workspace_bytes = p.workspace;
  out->kernel = p.mfma ? DAH_KERNEL_MFMA : DAH_KERNEL_VALU;
  return DAH_OK;
}

int dah_plan_decode(int B, int max_seq_len, int num_splits, int num_cus, dah_decode_plan* out) {
  return dah_plan_decode_ex(B, dah::kHeads, DAH_BF16, max_seq_len, num_splits, num_cus, out);
}

size_t dah_workspace_bytes_for(int B, int max_seq_len, int num_splits, int num_cus) {
  dah::Plan p;
  if (dah::plan_decode(B, dah::kHeads, DAH_BF16, max_seq_len, num_splits, num_cus, &p) != DAH_OK)
    return 0;
  return p.workspace;
}

const char* dah_status_string(int status) {
  switch (status) {
    case DAH_OK: return "DAH_OK";
    case DAH_ERR_NULL: return "DAH_ERR_NULL";
    case DAH_ERR_SHAPE: return "DAH_ERR_SHAPE";
    case DAH_ERR_DTYPE: return "DAH_ERR_DTYPE";
    case DAH_ERR_ALIGN: return "DAH_ERR_ALIGN";
    case DAH_ERR_WORKSPACE: return "DAH_ERR_WORKSPACE";
    case DAH_ERR_HIP: return "DAH_ERR_HIP";
    default: return "unknown status";
  }
}

const char* dah_last_error(void) { return dah::g_last_error; }

}  // extern "C"
