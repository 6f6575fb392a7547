// One decoder layer's decode step around the attention block (the
// "Qwen3-0.6B" Model Spec page, "Compute-graph nodes", per-layer rows):
//
//   h = input_norm(x); q, k, v = qkv_proj(h); o = attention step (norm, RoPE,
//   append, decodeGQA); x1 = x + o_proj(o); h2 = post_attn_norm(x1);
//   y = x1 + down(silu(gate) * up),  [gate | up] = gate_up(h2)
//
// The products run on the matrix cores (dah_linear.hip), which also take the
// hidden-size RMSNorms on their input rows, the SwiGLU activation in gate_up's
// store, and the residual adds in their stores (or in the reduce of their k
// slices: o_proj and down); the
// attention step runs in dah_kernels.hip.  This file holds the
// composition, the SwiGLU activation's kernel and the RMSNorm as a
// standalone call (dah_rmsnorm).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "dah.h"
#include "dah_host.h"

namespace {

constexpr int kNormThreads = 256;

// One workgroup per row: y = x / sqrt(sum x^2 / H + eps) * w, H = width.
// The sum is a tree over the workgroup (equal to the spec's sum up to
// rounding order: rmsNormTiled_eq, "Supported models" page).
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ w,
                                                               float eps, int width,
                                                               float* __restrict__ y) {
  __shared__ float part[kNormThreads / 64];
  const size_t row = blockIdx.x;
  const float4* xr = reinterpret_cast<const float4*>(x + row * width);
  const int n4 = width / 4;
  float ss = 0.0f;
  for (int i = threadIdx.x; i < n4; i += kNormThreads) {
    const float4 v = xr[i];
    ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  ss = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.0f / sqrtf(ss / (float)width + eps);
  const float4* wr = reinterpret_cast<const float4*>(w);
  float4* yr = reinterpret_cast<float4*>(y + row * width);
  for (int i = threadIdx.x; i < n4; i += kNormThreads) {
    const float4 v = xr[i], g = wr[i];
    yr[i] = make_float4(v.x * inv * g.x, v.y * inv * g.y, v.z * inv * g.z, v.w * inv * g.w);
  }
}

// act[t, i] = silu(gu[t, i]) * gu[t, inter + i], silu(z) = z / (1 + e^-z).
__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ gu, int T,
                                                       int inter, float* __restrict__ act) {
  const int n4 = inter / 4;
  const long long total = (long long)T * n4;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long t = e / n4;
    const int i = (int)(e - t * n4);
    const float4 g = reinterpret_cast<const float4*>(gu + t * 2 * inter)[i];
    const float4 u = reinterpret_cast<const float4*>(gu + t * 2 * inter + inter)[i];
    float4 r;
    r.x = g.x / (1.0f + expf(-g.x)) * u.x;
    r.y = g.y / (1.0f + expf(-g.y)) * u.y;
    r.z = g.z / (1.0f + expf(-g.z)) * u.z;
    r.w = g.w / (1.0f + expf(-g.w)) * u.w;
    reinterpret_cast<float4*>(act + t * inter)[i] = r;
  }
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dah::set_error(DAH_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return DAH_OK;
}

size_t round_up(size_t n) { return (n + 255) / 256 * 256; }

// Workspace of the layer: intermediates, then one region for the
// attention's own workspace and, once the attention is done with it (the
// launches are stream-ordered), the k-slice partials of o_proj and down.
struct LayerBuffers {
  size_t q, k, v, q_out, o, x1, act, attn, total;
};

size_t shared_region(int B, int hidden, int inter, int num_heads, size_t attn_ws) {
  const size_t o_split = dah_linear_workspace_bytes(B, hidden, num_heads * dah::kHeadDim);
  const size_t down_split = dah_linear_workspace_bytes(B, hidden, inter);
  return std::max(attn_ws, std::max(o_split, down_split));
}

LayerBuffers layer_buffers(int B, int hidden, int inter, int num_heads, size_t attn_ws) {
  LayerBuffers L = {};
  const size_t f = sizeof(float);
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at += round_up(bytes);
    return here;
  };
  L.q = take((size_t)B * num_heads * dah::kHeadDim * f);
  L.k = take((size_t)B * dah::kKvHeads * dah::kHeadDim * f);
  L.v = take((size_t)B * dah::kKvHeads * dah::kHeadDim * f);
  L.q_out = take((size_t)B * num_heads * dah::kHeadDim * f);
  L.o = take((size_t)B * num_heads * dah::kHeadDim * f);
  L.x1 = take((size_t)B * hidden * f);
  L.act = take((size_t)B * inter * f);
  L.attn = take(shared_region(B, hidden, inter, num_heads, attn_ws));
  L.total = at;
  return L;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

extern "C" {

int dah_rmsnorm(const float* x, const float* w, float eps, int T, int width, float* y,
                void* stream) {
  if (!x || !w || !y) return dah::set_error(DAH_ERR_NULL, "dah_rmsnorm: a pointer is NULL");
  if (T < 1 || width < 4 || width % 4 != 0)
    return dah::set_error(DAH_ERR_SHAPE, "dah_rmsnorm: T = %d, width = %d (need T >= 1 and a "
                          "positive multiple of 4)", T, width);
  if (!(eps >= 0.0f)) return dah::set_error(DAH_ERR_SHAPE, "dah_rmsnorm: eps must be >= 0");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y))
    return dah::set_error(DAH_ERR_ALIGN, "dah_rmsnorm: x, w and y need 16-byte alignment");
  rmsnorm_kernel<<<T, kNormThreads, 0, static_cast<hipStream_t>(stream)>>>(x, w, eps, width, y);
  return check_launch("rmsnorm_kernel");
}

int dah_silu_mul(const float* gate_up, int T, int inter, float* act, void* stream) {
  if (!gate_up || !act) return dah::set_error(DAH_ERR_NULL, "dah_silu_mul: a pointer is NULL");
  if (T < 1 || inter < 4 || inter % 4 != 0)
    return dah::set_error(DAH_ERR_SHAPE, "dah_silu_mul: T = %d, inter = %d (need T >= 1 and a "
                          "positive multiple of 4)", T, inter);
  if (!aligned16(gate_up) || !aligned16(act))
    return dah::set_error(DAH_ERR_ALIGN, "dah_silu_mul: 16-byte alignment needed");
  const long long n4 = (long long)T * (inter / 4);
  const int blocks = (int)std::min<long long>((n4 + 255) / 256, 4096);
  silu_mul_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(gate_up, T, inter, act);
  return check_launch("silu_mul_kernel");
}

size_t dah_layer_workspace_bytes(int B, int hidden, int inter, int num_heads, int cache_dtype,
                                 int max_seq_len, int num_splits) {
  if (B < 1 || hidden < 1 || inter < 1 || !dah::valid_heads(num_heads)) return 0;
  const size_t attn = dah_workspace_bytes_ex(B, num_heads, cache_dtype, max_seq_len, num_splits);
  return layer_buffers(B, hidden, inter, num_heads, attn).total;
}

int decoder_layer_step(const float* x, const dah_layer_weights* w, int hidden, int inter,
                       int num_heads, float eps, float rope_theta, void* k_cache, void* v_cache,
                       int cache_dtype, int64_t num_pages, const int32_t* block_table,
                       int max_pages_per_seq, const int32_t* seq_lens, int B, int max_seq_len,
                       int num_splits, float* y, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!x || !w || !y || !workspace)
    return dah::set_error(DAH_ERR_NULL, "decoder_layer_step: x, w, y or workspace is NULL");
  if (!w->w_in || !w->w_qkv || !w->q_gain || !w->k_gain || !w->w_o || !w->w_post ||
      !w->w_gate_up || !w->w_down)
    return dah::set_error(DAH_ERR_NULL, "decoder_layer_step: a weight pointer is NULL");
  if (hidden < 256 || hidden % 256 != 0 || inter < 256 || inter % 256 != 0)
    return dah::set_error(DAH_ERR_SHAPE, "decoder_layer_step: hidden = %d, inter = %d (need "
                          "positive multiples of 256)", hidden, inter);
  if (!dah::valid_heads(num_heads))
    return dah::set_error(DAH_ERR_SHAPE, "num_heads = %d, need 16, 32, 40 or 64", num_heads);
  if (B < 1) return dah::set_error(DAH_ERR_SHAPE, "B = %d, need B >= 1", B);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return dah::set_error(DAH_ERR_ALIGN, "decoder_layer_step: workspace needs 256-byte alignment");
  if (!aligned16(x) || !aligned16(y))
    return dah::set_error(DAH_ERR_ALIGN, "decoder_layer_step: x and y need 16-byte alignment");
  // The attention's checks before anything is launched (its q, k, v, q_out
  // and o live in the workspace, so any aligned non-null stand-in will do).
  int st = dah::validate_append(workspace, workspace, workspace, w->q_gain, w->k_gain, eps,
                                rope_theta, k_cache, v_cache, cache_dtype, num_pages, block_table,
                                max_pages_per_seq, seq_lens, B, num_heads, workspace);
  if (st == DAH_OK)
    st = dah::validate_decode(workspace, k_cache, v_cache, cache_dtype, num_pages, block_table,
                              max_pages_per_seq, seq_lens, B, num_heads, max_seq_len, num_splits,
                              workspace);
  if (st != DAH_OK) return st;
  const size_t attn = dah_workspace_bytes_ex(B, num_heads, cache_dtype, max_seq_len, num_splits);
  const LayerBuffers L = layer_buffers(B, hidden, inter, num_heads, attn);
  if (workspace_bytes < L.total)
    return dah::set_error(DAH_ERR_WORKSPACE, "decoder_layer_step: workspace of %zu bytes, need %zu",
                          workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  float* q = reinterpret_cast<float*>(ws + L.q);
  float* k = reinterpret_cast<float*>(ws + L.k);
  float* v = reinterpret_cast<float*>(ws + L.v);
  float* q_out = reinterpret_cast<float*>(ws + L.q_out);
  float* o = reinterpret_cast<float*>(ws + L.o);
  float* x1 = reinterpret_cast<float*>(ws + L.x1);
  float* act = reinterpret_cast<float*>(ws + L.act);
  void* attn_ws = attn > 0 ? ws + L.attn : nullptr;
  const size_t split = shared_region(B, hidden, inter, num_heads, 0);
  void* split_ws = split > 0 ? ws + L.attn : nullptr;
  const int qdim = num_heads * dah::kHeadDim;

  // Five launches, up to eight with the attention's merge and the slice
  // reduces of o_proj and down: input_norm folded into qkv_proj and
  // post_attn_norm into gate_up (the products norm their input rows as they
  // stream them), mlp.act into gate_up's store (each tile holds the gate and
  // up columns of the same outputs), the residual adds into the stores of
  // o_proj and down (or into their slice sums).
  st = dah::qkv_proj(x, w->w_in, eps, w->w_qkv, B, hidden, num_heads, q, k, v, stream);
  if (st == DAH_OK)
    st = decode_attn_step_ex(q, k, v, w->q_gain, w->k_gain, eps, rope_theta, k_cache, v_cache,
                             cache_dtype, num_pages, block_table, max_pages_per_seq, seq_lens, B,
                             num_heads, max_seq_len, num_splits, q_out, o, attn_ws, attn, stream);
  if (st == DAH_OK) st = dah_linear_ws(o, w->w_o, x, B, hidden, qdim, x1, split_ws, split, stream);
  if (st == DAH_OK)
    st = dah_rmsnorm_swiglu(x1, w->w_post, eps, w->w_gate_up, B, inter, hidden, act, stream);
  if (st == DAH_OK)
    st = dah_linear_ws(act, w->w_down, x1, B, hidden, inter, y, split_ws, split, stream);
  return st;
}

}  // extern "C"
