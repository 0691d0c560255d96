// NF4 blockwise quantisation and packing.
//
// Page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE
// expert stacks", opening section: [E, N, K/2] uint8 codes (two per byte) and
// one fp32 absmax per block, in the bitsandbytes gemm_4bit conventions;
// "Cross-vendor projections": 3.56x smaller than bf16, i.e. 64-element blocks
// with fp32 absmax.  Code values: QLoRA NormalFloat4.  Page "How do I run a
// MoE whose experts do not fit in VRAM ...", "Supported scope": the bake
// also stores the absmax as bf16 (4.25 bits per weight); then the block
// maximum is rounded to bf16 (nearest, ties to even, saturating at the
// largest finite bf16) and the codes are chosen against that stored value.
//
// A 64-element block never straddles a row (K % 64 == 0), so the stack is a
// flat run of blocks: block b covers elements [64b, 64b + 64), bytes
// [32b, 32b + 32) of `packed` and absmax[b].  Eight lanes share a block, each
// converting 8 consecutive elements (one 16-byte load for bf16, two for
// fp32); the absmax is an 8-lane max, and the code of x is the number of level
// midpoints m_i with x > m_i * absmax, compared in fp64 where both sides are
// exact -- the nearest level, ties to the lower code.  HBM-bound: 2 B in and
// 0.5625 B out per bf16 weight.

#include "gnf4_internal.h"

namespace gnf4 {
namespace {

constexpr int kPackThreads = 256;

__device__ __forceinline__ double level_mid(int i) {
  return ((double)nf4_level(i) + (double)nf4_level(i + 1)) * 0.5;
}

__device__ __forceinline__ uint32_t code_of(float x, const double* thr, bool zero_block) {
  if (zero_block) return (uint32_t)kZeroCode;
  const double xd = (double)x;
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) c += (xd > thr[i]) ? 1u : 0u;
  return c;
}

// fp32 -> bf16 bits, nearest even, saturating at the largest finite bf16
// (inputs are finite and non-negative here)
__device__ __forceinline__ uint32_t bf16_rne_sat(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return (r & 0x7fffu) == 0x7f80u ? (r & 0x8000u) | 0x7f7fu : r;
}

template <int DTYPE, bool ABS_BF16>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const void* __restrict__ w,
                                                            int64_t n_blocks,
                                                            uint8_t* __restrict__ packed,
                                                            void* __restrict__ absmax) {
  const int sub = threadIdx.x & 7;  // lane within the block's 8-lane group
  int64_t blk = ((int64_t)blockIdx.x * kPackThreads + threadIdx.x) >> 3;
  const int64_t stride = ((int64_t)gridDim.x * kPackThreads) >> 3;
  for (; blk < n_blocks; blk += stride) {
    float v[8];
    const int64_t e0 = blk * kBlock + sub * 8;
    if (DTYPE == GNF4_DTYPE_BF16) {
      const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + e0);
      const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16_to_f32(d[j] & 0xffffu);
        v[2 * j + 1] = bf16_to_f32(d[j] >> 16);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(w) + e0);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    // the 8 lanes of a block are aligned groups of 8: xor stays inside them
    m = fmaxf(m, __shfl_xor(m, 1, kWave));
    m = fmaxf(m, __shfl_xor(m, 2, kWave));
    m = fmaxf(m, __shfl_xor(m, 4, kWave));
    uint32_t m_bits = 0;
    if constexpr (ABS_BF16) {  // the stored (rounded) absmax sets the codes
      m_bits = bf16_rne_sat(m);
      m = __uint_as_float(m_bits << 16);
    }
    double thr[15];
    const double md = (double)m;
#pragma unroll
    for (int i = 0; i < 15; ++i) thr[i] = level_mid(i) * md;  // exact in fp64
    const bool zero_block = (m == 0.0f);
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t hi = code_of(v[2 * j], thr, zero_block);
      const uint32_t lo = code_of(v[2 * j + 1], thr, zero_block);
      word |= ((hi << 4) | lo) << (8 * j);
    }
    *reinterpret_cast<uint32_t*>(packed + blk * 32 + sub * 4) = word;
    if (sub == 0) {
      if constexpr (ABS_BF16)
        static_cast<uint16_t*>(absmax)[blk] = (uint16_t)m_bits;
      else
        static_cast<float*>(absmax)[blk] = m;
    }
  }
}

}  // namespace

hipError_t launch_pack(const void* w, int dtype, int64_t n_blocks, uint8_t* packed,
                       void* absmax, int abs_dtype, hipStream_t stream) {
  const int64_t blocks_needed = (n_blocks * 8 + kPackThreads - 1) / kPackThreads;
  const int64_t cap = (int64_t)device_cu_count() * 64;
  const unsigned grid = (unsigned)(blocks_needed < cap ? blocks_needed : cap);
  if (grid == 0) return hipSuccess;
  const bool ab = abs_dtype == GNF4_DTYPE_BF16;
  if (dtype == GNF4_DTYPE_BF16) {
    if (ab)
      hipLaunchKernelGGL((pack_kernel<GNF4_DTYPE_BF16, true>), dim3(grid), dim3(kPackThreads), 0,
                         stream, w, n_blocks, packed, absmax);
    else
      hipLaunchKernelGGL((pack_kernel<GNF4_DTYPE_BF16, false>), dim3(grid), dim3(kPackThreads), 0,
                         stream, w, n_blocks, packed, absmax);
  } else {
    if (ab)
      hipLaunchKernelGGL((pack_kernel<GNF4_DTYPE_F32, true>), dim3(grid), dim3(kPackThreads), 0,
                         stream, w, n_blocks, packed, absmax);
    else
      hipLaunchKernelGGL((pack_kernel<GNF4_DTYPE_F32, false>), dim3(grid), dim3(kPackThreads), 0,
                         stream, w, n_blocks, packed, absmax);
  }
  return hipGetLastError();
}

}  // namespace gnf4
