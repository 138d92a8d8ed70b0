// stream.hip -- the read-only streaming yardstick: how fast this GPU reads
// a buffer with the access the weight streams use (128-bit nontemporal
// loads, each wave instruction one contiguous 1 KB), and nothing else.
// It is the measured ceiling the block's kernels are compared with, next to
// the 8 TB/s HBM peak ([WRITEUP] "vLLM 如何用智能体辅助优化 Kimi K3 解码性能",
// part 1 §4: small-batch decode is bound by reading weights from memory).
//
// Workgroup w of G reads the w-th of G contiguous slices of the buffer in
// steps of kStreamDepth x 4 KB (each of its 256 threads requests
// kStreamDepth 16-byte loads, 4 KB apart, before using any), XORs every
// 32-bit word it read, and stores the XOR of its slice to sink[w], so the
// loads cannot be dropped and the host can check that every byte was read.

#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kStreamThreads = 256;
constexpr int kStreamDepth = 16;                       // 16-byte loads in flight per thread
constexpr size_t kStreamStep = (size_t)kStreamThreads * 16;   // bytes per load instruction of the workgroup

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* src, size_t n16, uint32_t* sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;   // 16-byte words of this slice
  const size_t b = (size_t)blockIdx.x * per;
  const size_t e = b + per < n16 ? b + per : n16;
  uint32_t acc = 0u;
  size_t i = b + threadIdx.x;
  // whole steps: every load unconditional
  for (; i + (size_t)(kStreamDepth - 1) * kStreamThreads < e; i += (size_t)kStreamDepth * kStreamThreads) {
    u32x4 v[kStreamDepth];
#pragma unroll
    for (int u = 0; u < kStreamDepth; ++u) v[u] = __builtin_nontemporal_load(src + i + (size_t)u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < kStreamDepth; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < e; i += kStreamThreads) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  acc = wave_xor_u32(acc);
  __shared__ uint32_t s_x[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0u;
    for (int w = 0; w < kStreamThreads / 64; ++w) x ^= s_x[w];
    sink[blockIdx.x] = x;
  }
}

// Weight prefetch ([WRITEUP] part 1 §4: weights about to be used are read
// into the cache during phases that use little memory bandwidth, on a side
// stream): the same slicing as the yardstick over up to kMaxPrefetch
// ranges, with plain 128-bit loads -- cached loads, which leave the lines in
// L2 and the Infinity Cache, unlike the nontemporal loads of the weight
// streams -- and the XOR of every word per workgroup to sink[w].
__global__ __launch_bounds__(kStreamThreads) void prefetch_kernel(PrefetchRanges r, uint32_t* sink) {
  uint32_t acc = 0u;
  for (int q = 0; q < r.n; ++q) {
    const u32x4* src = reinterpret_cast<const u32x4*>(r.ptr[q]);
    const size_t n16 = r.bytes[q] / 16;
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b = (size_t)blockIdx.x * per;
    const size_t e = b + per < n16 ? b + per : n16;
    size_t i = b + threadIdx.x;
    for (; i + (size_t)(kStreamDepth - 1) * kStreamThreads < e; i += (size_t)kStreamDepth * kStreamThreads) {
      u32x4 v[kStreamDepth];
#pragma unroll
      for (int u = 0; u < kStreamDepth; ++u) v[u] = src[i + (size_t)u * kStreamThreads];
#pragma unroll
      for (int u = 0; u < kStreamDepth; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < e; i += kStreamThreads) {
      const u32x4 v = src[i];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  acc = wave_xor_u32(acc);
  __shared__ uint32_t s_x[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0u;
    for (int w = 0; w < kStreamThreads / 64; ++w) x ^= s_x[w];
    sink[blockIdx.x] = x;
  }
}

hipError_t launch_prefetch(const PrefetchRanges& r, uint32_t* sink, int workgroups, hipStream_t st) {
  launch(K_NONE, prefetch_kernel, dim3((unsigned)workgroups), dim3(kStreamThreads), 0, st, r, sink);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t st) {
  launch(K_STREAM, stream_read_kernel, dim3((unsigned)workgroups), dim3(kStreamThreads), 0, st,
         reinterpret_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
