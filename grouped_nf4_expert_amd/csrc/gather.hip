// Row gather that builds the grouped activations: x_sorted[r] = x[slot_r / top_k].
//
// Page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE
// expert stacks", opening section: the GEMM consumes activations already
// sorted by expert.  Pure data movement (2 K bytes read and written per row),
// 16-byte vector copies, one workgroup per row stride.

#include "gnf4_internal.h"

namespace gnf4 {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void gather_rows_kernel(const uint16_t* __restrict__ x,
                                                               const int32_t* __restrict__ slots,
                                                               int top_k, int T, int M, int K,
                                                               uint16_t* __restrict__ out) {
  const int chunks = K / 8;  // 16-byte chunks per row (K % 64 == 0)
  for (int r = blockIdx.x; r < M; r += gridDim.x) {
    const int s = slots[r];
    if (s < 0 || s >= T * top_k) continue;  // out-of-range slot: row left as is
    const int t = s / top_k;
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * K);
    uint4* dst = reinterpret_cast<uint4*>(out + (size_t)r * K);
    for (int c = threadIdx.x; c < chunks; c += kThreads) dst[c] = src[c];
  }
}

}  // namespace

hipError_t launch_gather(const uint16_t* x, const int32_t* slots, int top_k, int T, int M, int K,
                         uint16_t* out, hipStream_t stream) {
  const int cap = device_cu_count() * 16;
  const int grid = M < cap ? M : cap;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(grid), dim3(kThreads), 0, stream, x, slots, top_k,
                     T, M, K, out);
  return hipGetLastError();
}

}  // namespace gnf4
