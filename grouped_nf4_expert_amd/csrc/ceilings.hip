// Machine-ceiling probes for the roofline fractions of the GEMM kernels:
// a pure-read kernel (HBM read bandwidth against buffer size), an empty
// kernel (the fixed cost of a launch) and a matrix-core loop that reads the
// shader clock while the matrix cores are saturated.  Each probe is the
// simplest program that reaches its limit; none shares code with the GEMM
// path.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gnf4_ceilings.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;
constexpr int kMfmaThreads = 256;
constexpr int kMaxBlocks = 65536;

__global__ __launch_bounds__(kReadThreads) void read_kernel(const u32x4* __restrict__ p,
                                                            uint64_t words,
                                                            uint32_t* __restrict__ block_xor) {
  const uint64_t stride = (uint64_t)gridDim.x * kReadThreads;
  uint64_t i = (uint64_t)blockIdx.x * kReadThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kReadUnroll - 1) * stride < words; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (; i < words; i += stride) acc ^= p[i];
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  __shared__ uint32_t part[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) block_xor[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__global__ void empty_kernel() {}

__global__ __launch_bounds__(kMfmaThreads) void mfma_kernel(int iters,
                                                            uint64_t* __restrict__ stamps,
                                                            float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  half8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(float)((lane + j) & 7) * (_Float16)0.125f;
    b[j] = (_Float16)(float)((lane * 3 + j) & 7) * (_Float16)0.0625f;
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  const uint64_t gt = (uint64_t)blockIdx.x * kMfmaThreads + threadIdx.x;
  if (lane == 0) {
    uint64_t* s = stamps + 4 * (gt >> 6);
    s[0] = t0;
    s[1] = t1;
    s[2] = r0;
    s[3] = r1;
  }
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[c][e];
  sink[gt] = sum;
}

gnf4_status launched() {
  return hipGetLastError() == hipSuccess ? GNF4_OK : GNF4_ERR_HIP;
}

}  // namespace

extern "C" gnf4_status gnf4_ceil_read(const void* buf, size_t bytes, int blocks,
                                      uint32_t* block_xor, void* stream) {
  if (!buf || !block_xor || bytes == 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0 || blocks < 1 || blocks > kMaxBlocks)
    return GNF4_ERR_INVALID_ARG;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf),
                     (uint64_t)(bytes / 16), block_xor);
  return launched();
}

extern "C" gnf4_status gnf4_ceil_empty(int blocks, void* stream) {
  if (blocks < 1 || blocks > kMaxBlocks) return GNF4_ERR_INVALID_ARG;
  hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(64), 0, static_cast<hipStream_t>(stream));
  return launched();
}

extern "C" gnf4_status gnf4_ceil_mfma(int iters, int blocks, uint64_t* stamps, float* sink,
                                      void* stream) {
  if (!stamps || !sink || iters < 1 || iters > (1 << 24) || blocks < 1 || blocks > kMaxBlocks)
    return GNF4_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(kMfmaThreads), 0,
                     static_cast<hipStream_t>(stream), iters, stamps, sink);
  return launched();
}
