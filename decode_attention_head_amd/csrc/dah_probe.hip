// Memory-system probes for the benchmark (include/dah_probe.h): a plain
// vector copy of known traffic and a non-temporal streaming read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dah.h"
#include "dah_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// Each workgroup reads a contiguous share, four 16-byte loads per thread in
// flight, and folds everything into one word so the loads stay live.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, size_t n,
                                                         uint32_t* __restrict__ sink) {
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t begin = (size_t)blockIdx.x * per;
  const size_t end = begin + per < n ? begin + per : n;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = begin + threadIdx.x;
  for (; i + 3 * 256 < end; i += 4 * 256) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + 256);
    const u32x4 c = __builtin_nontemporal_load(src + i + 512);
    const u32x4 d = __builtin_nontemporal_load(src + i + 768);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < end; i += 256) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// The decode kernel's access pattern without its arithmetic: one workgroup
// of 8 waves per sequence, wave g reading KV head g's K and V tiles (16
// positions x 128 dims, kLoads 16-byte loads per lane each) of every page of
// the sequence, two pages in flight.
template <int kLoads>
__global__ __launch_bounds__(512) void probe_paged_read_kernel(
    const char* __restrict__ k, const char* __restrict__ v, int64_t num_pages,
    const int32_t* __restrict__ block_table, int max_pages_per_seq,
    const int32_t* __restrict__ seq_lens, int max_seq_len, uint32_t* __restrict__ sink) {
  constexpr int kTileBytes = kLoads * 64 * 16;
  constexpr int64_t kPageBytes = 8LL * kTileBytes;
  const int b = blockIdx.x, g = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = seq_lens[b];
  const int npages = (n >= 1 && n <= max_seq_len) ? (n + 15) / 16 : 0;
  const int32_t* row = block_table + (size_t)b * max_pages_per_seq;
  auto load = [&](u32x4 (&t)[2 * kLoads], int p) {
    int64_t id = row[p];
    id = (id >= 0 && id < num_pages) ? id : 0;
    const u32x4* kp = reinterpret_cast<const u32x4*>(k + id * kPageBytes + g * kTileBytes) + lane;
    const u32x4* vp = reinterpret_cast<const u32x4*>(v + id * kPageBytes + g * kTileBytes) + lane;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      t[j] = __builtin_nontemporal_load(kp + 64 * j);
      t[kLoads + j] = __builtin_nontemporal_load(vp + 64 * j);
    }
  };
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 t0[2 * kLoads], t1[2 * kLoads];
  if (npages > 0) load(t0, 0);
  if (npages > 1) load(t1, 1);
  for (int p = 0; p < npages; p += 2) {
#pragma unroll
    for (int j = 0; j < 2 * kLoads; ++j) acc ^= t0[j];
    if (p + 2 < npages) load(t0, p + 2);
    if (p + 1 < npages) {
#pragma unroll
      for (int j = 0; j < 2 * kLoads; ++j) acc ^= t1[j];
      if (p + 3 < npages) load(t1, p + 3);
    }
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
  if (lane == 0) sink[(size_t)b * 8 + g] = x;
}

int check(const void* a, const void* b, size_t bytes) {
  if (!a || !b) return DAH_ERR_NULL;
  if (bytes == 0 || bytes % 16) return DAH_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(a) % 16 || reinterpret_cast<uintptr_t>(b) % 4) return DAH_ERR_ALIGN;
  return DAH_OK;
}

}  // namespace

extern "C" int dah_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  int st = check(src, dst, bytes);
  if (st != DAH_OK) return st;
  if (reinterpret_cast<uintptr_t>(dst) % 16) return DAH_ERR_ALIGN;
  const size_t n = bytes / 16;
  probe_copy_kernel<<<4096, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
  return hipGetLastError() == hipSuccess ? DAH_OK : DAH_ERR_HIP;
}

extern "C" int dah_probe_read(const void* src, size_t bytes, uint32_t* sink, int sink_words,
                              void* stream) {
  int st = check(src, sink, bytes);
  if (st != DAH_OK) return st;
  if (sink_words < 1) return DAH_ERR_SHAPE;
  const int blocks = sink_words < 65536 ? sink_words : 65536;
  probe_read_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? DAH_OK : DAH_ERR_HIP;
}

extern "C" int dah_probe_paged_read(const void* k_cache, const void* v_cache, int cache_dtype,
                                    int64_t num_pages, const int32_t* block_table,
                                    int max_pages_per_seq, const int32_t* seq_lens, int B,
                                    int max_seq_len, uint32_t* sink, void* stream) {
  if (!k_cache || !v_cache || !block_table || !seq_lens || !sink) return DAH_ERR_NULL;
  if (cache_dtype != DAH_F32 && cache_dtype != DAH_BF16) return DAH_ERR_DTYPE;
  if (B < 1 || num_pages < 1 || max_pages_per_seq < 1 || max_seq_len < 1 ||
      (int64_t)max_seq_len > (int64_t)max_pages_per_seq * 16)
    return DAH_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(k_cache) % 16 || reinterpret_cast<uintptr_t>(v_cache) % 16 ||
      reinterpret_cast<uintptr_t>(block_table) % 4 || reinterpret_cast<uintptr_t>(seq_lens) % 4 ||
      reinterpret_cast<uintptr_t>(sink) % 4)
    return DAH_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* k = static_cast<const char*>(k_cache);
  const char* v = static_cast<const char*>(v_cache);
  if (cache_dtype == DAH_BF16)
    probe_paged_read_kernel<4><<<B, 512, 0, s>>>(k, v, num_pages, block_table, max_pages_per_seq,
                                                 seq_lens, max_seq_len, sink);
  else
    probe_paged_read_kernel<8><<<B, 512, 0, s>>>(k, v, num_pages, block_table, max_pages_per_seq,
                                                 seq_lens, max_seq_len, sink);
  return hipGetLastError() == hipSuccess ? DAH_OK : DAH_ERR_HIP;
}
