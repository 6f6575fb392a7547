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
