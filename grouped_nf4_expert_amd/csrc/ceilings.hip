// Machine-ceiling probes for the roofline fractions of the GEMM kernels:
// a pure-read kernel (HBM read bandwidth against buffer size), an empty
// kernel (the fixed cost of a launch), a matrix-core loop that reads the
// shader clock while the matrix cores are saturated, and the same loop with
// VALU and LDS work interleaved in each wavefront (what a GEMM that decodes
// its own operands can keep of the matrix-core rate).  Each probe is the
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

// The matrix-core loop with other work beside it in the same wavefront:
// five independent accumulator chains, each MFMA followed by V dependent
// v_perm_b32 (a decode-like VALU chain) and, with D = 1, one 16-byte LDS read
// that becomes the A operand of the same chain's next MFMA (five MFMAs
// later), as a GEMM reads its fragments a step ahead.  The reads use fixed
// per-lane addresses with immediate offsets (no address arithmetic);
// consecutive lanes read consecutive 16-byte words (conflict-free).
constexpr int kMixChains = 5;
constexpr int kMixLdsSlots = 2048;  // 16-byte words of LDS

template <int V, int D>
__global__ __launch_bounds__(kMfmaThreads) void mfma_mix_kernel(int iters,
                                                                uint64_t* __restrict__ stamps,
                                                                float* __restrict__ sink) {
  __shared__ u32x4 lds[kMixLdsSlots];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kMixLdsSlots; i += kMfmaThreads) {
    // small finite fp16 values: ((i + j) & 7) / 8 in each half
    const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)((float)(i & 7) * 0.125f));
    const uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)((float)((i + 1) & 7) * 0.125f));
    lds[i] = u32x4{h0 | (h1 << 16), h1 | (h0 << 16), h0 | (h0 << 16), h1 | (h1 << 16)};
  }
  __syncthreads();
  half8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(float)((lane + j) & 7) * (_Float16)0.125f;
    b[j] = (_Float16)(float)((lane * 3 + j) & 7) * (_Float16)0.0625f;
  }
  uint32_t r[4] = {(uint32_t)lane, (uint32_t)lane * 7u, (uint32_t)lane * 13u, 5u};
  const u32x4* src = lds + wave * (kMixChains * 64) + lane;  // chain c at src[64 c]
  half8 held[kMixChains];
#pragma unroll
  for (int c = 0; c < kMixChains; ++c) held[c] = a;
  f32x16 acc[kMixChains];
#pragma unroll
  for (int c = 0; c < kMixChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMixChains; ++c) {
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(D ? held[c] : a, b, acc[c], 0, 0, 0);
      if constexpr (D > 0) held[c] = __builtin_bit_cast(half8, src[64 * c]);
#pragma unroll
      for (int i = 0; i < V; ++i)
        r[i & 3] = __builtin_amdgcn_perm(r[(i + 1) & 3], r[i & 3], 0x03020100u + (uint32_t)i);
      __builtin_amdgcn_sched_barrier(0);
    }
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
  float sum = (float)((r[0] ^ r[1] ^ r[2] ^ r[3]) & 0xffu);
#pragma unroll
  for (int c = 0; c < kMixChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[c][e];
  sink[gt] = sum;
}

template <int V, int D>
void launch_mix(int iters, int blocks, uint64_t* stamps, float* sink, void* stream) {
  hipLaunchKernelGGL((mfma_mix_kernel<V, D>), dim3(blocks), dim3(kMfmaThreads), 0,
                     static_cast<hipStream_t>(stream), iters, stamps, sink);
}

// Two roles in one 512-thread workgroup (two wavefronts per SIMD): waves
// 0..3 issue only MFMAs (five chains), waves 4..7 only V dependent v_perm_b32
// per MFMA slot, for the same number of slots.  Each wave stamps its clocks,
// so the MFMA wavefronts' rate beside VALU-only neighbours can be read.
constexpr int kSplitThreads = 512;

template <int V>
__global__ __launch_bounds__(kSplitThreads) void mfma_split_kernel(int iters,
                                                                   uint64_t* __restrict__ stamps,
                                                                   float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  half8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(float)((lane + j) & 7) * (_Float16)0.125f;
    b[j] = (_Float16)(float)((lane * 3 + j) & 7) * (_Float16)0.0625f;
  }
  float sum = 0.0f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  if (wave < 4) {
    f32x16 acc[kMixChains];
#pragma unroll
    for (int c = 0; c < kMixChains; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kMixChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kMixChains; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += acc[c][e];
  } else {
    uint32_t r[4] = {(uint32_t)lane, (uint32_t)lane * 7u, (uint32_t)lane * 13u, 5u};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kMixChains; ++c)
#pragma unroll
        for (int i = 0; i < V; ++i)
          r[i & 3] = __builtin_amdgcn_perm(r[(i + 1) & 3], r[i & 3], 0x03020100u + (uint32_t)i);
    }
    sum = (float)((r[0] ^ r[1] ^ r[2] ^ r[3]) & 0xffu);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  const uint64_t gt = (uint64_t)blockIdx.x * kSplitThreads + threadIdx.x;
  if (lane == 0) {
    uint64_t* s = stamps + 4 * (gt >> 6);
    s[0] = t0;
    s[1] = t1;
    s[2] = r0;
    s[3] = r1;
  }
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

extern "C" gnf4_status gnf4_ceil_mfma_mix(int iters, int blocks, int valu, int lds_reads,
                                          uint64_t* stamps, float* sink, void* stream) {
  if (!stamps || !sink || iters < 1 || iters > (1 << 24) || blocks < 1 || blocks > kMaxBlocks ||
      (lds_reads != 0 && lds_reads != 1) || (valu != 0 && valu != 4 && valu != 8 && valu != 12))
    return GNF4_ERR_INVALID_ARG;
#define GNF4_MIX(v)                                                    \
  if (valu == v) {                                                     \
    if (lds_reads)                                                     \
      launch_mix<v, 1>(iters, blocks, stamps, sink, stream);           \
    else                                                               \
      launch_mix<v, 0>(iters, blocks, stamps, sink, stream);           \
  }
  GNF4_MIX(0)
  GNF4_MIX(4)
  GNF4_MIX(8)
  GNF4_MIX(12)
#undef GNF4_MIX
  return launched();
}

extern "C" gnf4_status gnf4_ceil_mfma_split(int iters, int blocks, int valu, uint64_t* stamps,
                                            float* sink, void* stream) {
  if (!stamps || !sink || iters < 1 || iters > (1 << 24) || blocks < 1 || blocks > kMaxBlocks ||
      (valu != 4 && valu != 8 && valu != 12))
    return GNF4_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (valu == 4)
    hipLaunchKernelGGL(mfma_split_kernel<4>, dim3(blocks), dim3(kSplitThreads), 0, st, iters,
                       stamps, sink);
  else if (valu == 8)
    hipLaunchKernelGGL(mfma_split_kernel<8>, dim3(blocks), dim3(kSplitThreads), 0, st, iters,
                       stamps, sink);
  else
    hipLaunchKernelGGL(mfma_split_kernel<12>, dim3(blocks), dim3(kSplitThreads), 0, st, iters,
                       stamps, sink);
  return launched();
}
