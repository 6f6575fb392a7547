// Host-side helpers of the decode-attention library: argument validation, the
// split planner and error reporting.  Nothing here touches the HIP runtime, so
// it builds and runs without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "dah.h"

namespace dah {

constexpr int kHeads = 16;     // query heads of Qwen3-0.6B (the default entry points)
constexpr int kKvHeads = 8;    // key/value heads; query head h reads KV head h / (H / 8)
constexpr int kHeadDim = 128;  // head dimension
constexpr int kPage = 16;      // positions per cache page

// Query-head counts the kernels are built for: the Qwen3 family's 16, 32, 40
// and 64 heads over 8 KV heads (2, 4, 5, 8 query heads per KV head).
inline bool valid_heads(int h) { return h == 16 || h == 32 || h == 40 || h == 64; }

// Records `msg` (printf-style) as this thread's last error and returns status.
int set_error(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

constexpr int kMaxBalancedBatch = 4096;  // sequences the balanced decode's LDS scan holds

struct Plan {
  int mode;             // dah_plan_mode
  int splits;           // splits per sequence (1 per sequence, 0 balanced)
  int pages_per_split;  // pages per split (0 balanced)
  int grid_splits;      // DAH_PLAN_SPLIT: splits padded to a multiple of 8 for the XCD mapping
  int workgroups;       // grid of the decode launch
  size_t workspace;     // bytes of partial results
  bool mfma;            // matrix-core decode (bfloat16 cache only)
};

// Planner: pure integer policy from the batch size, the longest sequence, the
// compute-unit count and the kernel that will run (head count and cache
// dtype); the head count also sizes the workspace.  Returns a dah_status.
int plan_decode(int B, int num_heads, int cache_dtype, int max_seq_len, int num_splits,
                int num_cus, Plan* out);

int validate_append(const void* q, const void* k_new, const void* v_new, const void* q_gain,
                    const void* k_gain, float eps, float rope_theta, const void* k_cache,
                    const void* v_cache, int cache_dtype, int64_t num_pages,
                    const void* block_table, int max_pages_per_seq, const void* seq_lens, int B,
                    int num_heads, const void* q_out);

// chunk_attn_step: the append checks, plus cu_tokens, the token count, the
// chunk bound and max_seq_len.
int validate_chunk(const void* q, const void* k_new, const void* v_new, const void* q_gain,
                   const void* k_gain, float eps, float rope_theta, const void* k_cache,
                   const void* v_cache, int cache_dtype, int64_t num_pages,
                   const void* block_table, int max_pages_per_seq, const void* seq_lens,
                   const void* cu_tokens, int B, int total_tokens, int max_chunk, int max_seq_len,
                   int num_heads, const void* q_out, const void* o);

// dah_linear: T >= 1, N a multiple of 64, K a multiple of 256, 16-byte alignment.
int validate_linear(const void* x, const void* w, int T, int N, int K, const void* y);

int validate_decode(const void* q, const void* k_cache, const void* v_cache, int cache_dtype,
                    int64_t num_pages, const void* block_table, int max_pages_per_seq,
                    const void* seq_lens, int B, int num_heads, int max_seq_len, int num_splits,
                    const void* o);

// attn_qkv_proj, with the input row RMS-normed first (gain x_gain, eps) when
// x_gain is not NULL -- the decoder layer's input_norm folded into the
// product (dah_linear.hip).
int qkv_proj(const float* x, const float* x_gain, float eps, const void* w_qkv, int T, int hidden,
             int num_heads, float* q, float* k, float* v, void* stream);

}  // namespace dah
