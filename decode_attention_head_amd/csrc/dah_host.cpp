// Host-side helpers: validation, split planner, status strings, last error.
// See dah_host.h.  No HIP calls in this file.
#include "dah_host.h"

#include <stdarg.h>
#include <stdio.h>

#include "dah.h"

namespace dah {

namespace {
thread_local char g_last_error[512] = "";

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Split policy, from split-count sweeps of the decode kernel on MI355X
// (256 compute units): aim for 8 resident waves per compute unit (2 per
// SIMD: the kernel's register use allows 3), never cut a split below 4
// pages, and never leave a split longer than 128 pages, so that a batch
// whose lengths are ragged still spreads its longest sequences.
constexpr int kTargetWavesPerCu = 8;
constexpr int kMinPagesPerSplit = 4;
constexpr int kMaxPagesPerSplit = 128;
}  // namespace

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_last_error[0] = '\0'; }

size_t workspace_bytes(int B, int splits) {
  if (splits <= 1) return 0;
  const size_t parts = static_cast<size_t>(B) * kHeads * static_cast<size_t>(splits);
  return parts * (kHeadDim + 2) * sizeof(float);
}

int plan_splits(int B, int max_seq_len, int num_splits, int num_cus, Plan* out) {
  if (out == nullptr) return set_error(DAH_ERR_NULL, "plan_splits: output pointer is NULL");
  if (B < 1) return set_error(DAH_ERR_SHAPE, "B = %d, need B >= 1", B);
  if (max_seq_len < 1)
    return set_error(DAH_ERR_SHAPE, "max_seq_len = %d, need >= 1", max_seq_len);
  if (num_splits < 0)
    return set_error(DAH_ERR_SHAPE, "num_splits = %d, need >= 0 (0 = automatic)", num_splits);
  if (num_cus < 1) return set_error(DAH_ERR_SHAPE, "num_cus = %d, need >= 1", num_cus);

  const int max_pages = (max_seq_len + kPage - 1) / kPage;
  int want;
  if (num_splits > 0) {
    want = num_splits;
  } else {
    // One wave per (sequence, KV head, split).  Ask for enough splits to give
    // every compute unit kTargetWavesPerCu waves, but keep splits at least
    // kMinPagesPerSplit pages long.
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
  const int pps = (max_pages + want - 1) / want;
  out->pages_per_split = pps;
  out->splits = (max_pages + pps - 1) / pps;  // no split past the longest sequence is empty
  out->workspace = workspace_bytes(B, out->splits);
  return DAH_OK;
}

int validate_append(const void* q, const void* k_new, const void* v_new, const void* q_gain,
                    const void* k_gain, float eps, float rope_theta, const void* k_cache,
                    const void* v_cache, int cache_dtype, int64_t num_pages,
                    const void* block_table, int max_pages_per_seq, const void* seq_lens, int B,
                    const void* q_out) {
  if (!q || !k_new || !v_new || !q_gain || !k_gain || !k_cache || !v_cache || !block_table ||
      !seq_lens || !q_out)
    return set_error(DAH_ERR_NULL, "qk_norm_rope_append: a required pointer is NULL");
  if (cache_dtype != DAH_F32 && cache_dtype != DAH_BF16)
    return set_error(DAH_ERR_DTYPE, "cache_dtype = %d, need DAH_F32 (0) or DAH_BF16 (1)",
                     cache_dtype);
  if (B < 1) return set_error(DAH_ERR_SHAPE, "B = %d, need B >= 1", B);
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

int validate_decode(const void* q, const void* k_cache, const void* v_cache, int cache_dtype,
                    int64_t num_pages, const void* block_table, int max_pages_per_seq,
                    const void* seq_lens, int B, int max_seq_len, int num_splits, const void* o) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o)
    return set_error(DAH_ERR_NULL, "paged_decode_gqa: a required pointer is NULL");
  if (cache_dtype != DAH_F32 && cache_dtype != DAH_BF16)
    return set_error(DAH_ERR_DTYPE, "cache_dtype = %d, need DAH_F32 (0) or DAH_BF16 (1)",
                     cache_dtype);
  if (B < 1) return set_error(DAH_ERR_SHAPE, "B = %d, need B >= 1", B);
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

int dah_plan_splits(int B, int max_seq_len, int num_splits, int num_cus, int* splits_out,
                    int* pages_per_split_out) {
  if (!splits_out || !pages_per_split_out)
    return dah::set_error(DAH_ERR_NULL, "dah_plan_splits: output pointer is NULL");
  dah::Plan p;
  int st = dah::plan_splits(B, max_seq_len, num_splits, num_cus, &p);
  if (st != DAH_OK) return st;
  *splits_out = p.splits;
  *pages_per_split_out = p.pages_per_split;
  return DAH_OK;
}

size_t dah_workspace_bytes_for(int B, int max_seq_len, int num_splits, int num_cus) {
  dah::Plan p;
  if (dah::plan_splits(B, max_seq_len, num_splits, num_cus, &p) != DAH_OK) return 0;
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
