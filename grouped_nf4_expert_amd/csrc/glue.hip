// The MoE feed-forward steps on either side of the grouped GEMM: the SwiGLU
// activation between the two expert projections and the weighted top-k
// combine after the down projection.
//
// Landing page "grouped-nf4-gemm": "Owns" lists swiglu and combine among the
// decode glue kernels, and "Use this when" asks for each of the decode step's
// small glue operations (activation, top-k combine) to be one launch.  Both
// are pure bandwidth: every byte is read or written once, with 16-byte
// accesses along the row when the width and alignment allow (a per-element
// path otherwise), so their roofline is HBM.
//
//  * swiglu: gate_up [M, 2I] bf16 (gate half first) -> h [M, I] bf16,
//    h = silu(gate) * up computed in fp32, silu(g) = g / (1 + exp(-g)).
//  * combine: out[t] = sum_j topk_w[t, j] * y[slot_rows[t*k + j]] over the
//    token's k slots in ascending j, fp32 accumulation, bf16 store.  The
//    row of each slot comes from the sort (slot_rows), so a token reads its
//    k rows directly and the sum order is fixed: deterministic, no atomics.
//    A slot whose row lies outside [0, M) contributes nothing.

#include <math.h>

#include "gnf4_internal.h"

namespace gnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxGridY = 65535;
constexpr int kJBatch = 8;  // slots of a token whose rows are loaded together

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

__device__ __forceinline__ void bf16x8_to_f32(const uint4 v, float (&f)[8]) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(d[i] << 16);
    f[2 * i + 1] = __uint_as_float(d[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint4 f32x8_to_bf16(const float (&f)[8]) {
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// VEC: 8 outputs per thread (I % 8 == 0, 16-byte aligned rows); else one.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void swiglu_kernel(const uint16_t* __restrict__ gu,
                                                          int64_t M, int64_t I,
                                                          uint16_t* __restrict__ h) {
  const int64_t units = VEC ? I / 8 : I;
  const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (u >= units) return;
  for (int64_t r = blockIdx.y; r < M; r += gridDim.y) {
    const uint16_t* grow = gu + (size_t)r * 2 * I;
    if constexpr (VEC) {
      const uint4 gv = *reinterpret_cast<const uint4*>(grow + 8 * u);
      const uint4 uv = *reinterpret_cast<const uint4*>(grow + I + 8 * u);
      float g[8], up[8], o[8];
      bf16x8_to_f32(gv, g);
      bf16x8_to_f32(uv, up);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = silu(g[i]) * up[i];
      *reinterpret_cast<uint4*>(h + (size_t)r * I + 8 * u) = f32x8_to_bf16(o);
    } else {
      const float g = bf16_to_f32(grow[u]);
      const float up = bf16_to_f32(grow[I + u]);
      h[(size_t)r * I + u] = f32_to_bf16(silu(g) * up);
    }
  }
}

// One token per workgroup row of the grid; threads cover the H columns.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void combine_kernel(const uint16_t* __restrict__ y,
                                                           const int32_t* __restrict__ rows,
                                                           const float* __restrict__ topk_w,
                                                           int64_t T, int k, int64_t M,
                                                           int64_t H, uint16_t* __restrict__ out) {
  const int64_t units = VEC ? H / 8 : H;
  const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (u >= units) return;
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
    float acc[VEC ? 8 : 1];
#pragma unroll
    for (int i = 0; i < (VEC ? 8 : 1); ++i) acc[i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += kJBatch) {
      // rows and weights of up to kJBatch slots, then all their loads, then
      // the multiply-adds in ascending j
      int r[kJBatch];
      float w[kJBatch];
#pragma unroll
      for (int jj = 0; jj < kJBatch; ++jj) {
        const int j = j0 + jj;
        const bool ok = j < k;
        r[jj] = ok ? rows[t * k + j] : -1;
        w[jj] = ok ? topk_w[t * k + j] : 0.0f;
        if (r[jj] < 0 || r[jj] >= M) r[jj] = -1;
      }
      if constexpr (VEC) {
        uint4 v[kJBatch];
#pragma unroll
        for (int jj = 0; jj < kJBatch; ++jj) {
          v[jj] = make_uint4(0, 0, 0, 0);
          if (r[jj] >= 0) v[jj] = *reinterpret_cast<const uint4*>(y + (size_t)r[jj] * H + 8 * u);
        }
#pragma unroll
        for (int jj = 0; jj < kJBatch; ++jj) {
          if (r[jj] < 0) continue;
          float f[8];
          bf16x8_to_f32(v[jj], f);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[jj], f[i], acc[i]);
        }
      } else {
        uint32_t v[kJBatch];
#pragma unroll
        for (int jj = 0; jj < kJBatch; ++jj) v[jj] = r[jj] >= 0 ? y[(size_t)r[jj] * H + u] : 0u;
#pragma unroll
        for (int jj = 0; jj < kJBatch; ++jj)
          if (r[jj] >= 0) acc[0] = fmaf(w[jj], bf16_to_f32(v[jj]), acc[0]);
      }
    }
    if constexpr (VEC)
      *reinterpret_cast<uint4*>(out + (size_t)t * H + 8 * u) = f32x8_to_bf16(acc);
    else
      out[(size_t)t * H + u] = f32_to_bf16(acc[0]);
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

hipError_t launch_swiglu(const uint16_t* gate_up, int64_t M, int64_t I, uint16_t* h,
                         hipStream_t stream) {
  const bool vec = I % 8 == 0 && aligned16(gate_up) && aligned16(h);
  const int64_t units = vec ? I / 8 : I;
  const dim3 grid((unsigned)((units + kThreads - 1) / kThreads),
                  (unsigned)(M < kMaxGridY ? M : kMaxGridY));
  if (vec)
    hipLaunchKernelGGL(swiglu_kernel<true>, grid, dim3(kThreads), 0, stream, gate_up, M, I, h);
  else
    hipLaunchKernelGGL(swiglu_kernel<false>, grid, dim3(kThreads), 0, stream, gate_up, M, I, h);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* y, const int32_t* slot_rows, const float* topk_w,
                          int64_t T, int top_k, int64_t M, int64_t H, uint16_t* out,
                          hipStream_t stream) {
  const bool vec = H % 8 == 0 && (M == 0 || aligned16(y)) && aligned16(out);
  const int64_t units = vec ? H / 8 : H;
  const dim3 grid((unsigned)((units + kThreads - 1) / kThreads),
                  (unsigned)(T < kMaxGridY ? T : kMaxGridY));
  if (vec)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(kThreads), 0, stream, y, slot_rows,
                       topk_w, T, top_k, M, H, out);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(kThreads), 0, stream, y, slot_rows,
                       topk_w, T, top_k, M, H, out);
  return hipGetLastError();
}

}  // namespace gnf4
