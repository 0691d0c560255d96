// Opt-in device-side check of the grouping inputs (GNF4_VALIDATE=1 in the
// environment).  The grouped kernels take group sizes, expert ids and slots
// from device memory, where the host cannot see them, and skip what lies
// outside their contract rather than fault.  Landing page "grouped-nf4-gemm",
// "Do not use this when": nothing falls back silently -- so a caller who
// wants misuse reported sets GNF4_VALIDATE=1, and every grouped call then
// runs this check, synchronises its stream and returns GNF4_ERR_INVALID_ARG
// instead of launching when the inputs hold anything a kernel would skip.

#include <stdlib.h>

#include "gnf4_internal.h"

namespace gnf4 {
namespace {

// Bits of the result word.
constexpr int32_t kBadSize = 1;   // a negative group size
constexpr int32_t kBadId = 2;     // a non-empty group whose expert id lies outside [0, E)
constexpr int32_t kOverM = 4;     // the sizes (negative ones as 0) sum past M
constexpr int32_t kBadSlot = 8;   // a covered row whose slot lies outside [0, T * top_k)

__device__ int32_t g_validate_result;

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void validate_kernel(const int32_t* sizes,
                                                            const int32_t* ids, int G, int E,
                                                            int64_t M, const int32_t* slots,
                                                            int64_t slot_lim) {
  __shared__ long long s_sum[kThreads / kWave];
  __shared__ int s_bits[kThreads / kWave];
  int bits = 0;
  long long sum = 0;
  for (int g = threadIdx.x; g < G; g += kThreads) {
    const int s = sizes[g];
    if (s < 0) bits |= kBadSize;
    if (s > 0 && (ids[g] < 0 || ids[g] >= E)) bits |= kBadId;
    sum += s > 0 ? s : 0;
  }
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sum += __shfl_xor(sum, off, kWave);
    bits |= __shfl_xor(bits, off, kWave);
  }
  if (threadIdx.x % kWave == 0) {
    s_sum[wave] = sum;
    s_bits[wave] = bits;
  }
  __syncthreads();
  long long total = 0;
  bits = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) {
    total += s_sum[w];
    bits |= s_bits[w];
  }
  if (total > M) bits |= kOverM;
  if (slots) {
    const long long covered = total < M ? total : M;
    int slot_bits = 0;
    for (long long r = threadIdx.x; r < covered; r += kThreads) {
      const int v = slots[r];
      if (v < 0 || v >= slot_lim) slot_bits = kBadSlot;
    }
    bits |= __syncthreads_or(slot_bits) ? kBadSlot : 0;
  }
  if (threadIdx.x == 0) g_validate_result = bits;
}

}  // namespace

bool validate_requested() {
  const char* v = getenv("GNF4_VALIDATE");
  return v != nullptr && v[0] == '1' && v[1] == '\0';
}

hipError_t validate_groups(const int32_t* sizes, const int32_t* ids, int64_t G, int64_t E,
                           int64_t M, const int32_t* slots, int64_t slot_lim,
                           hipStream_t stream, int32_t* result) {
  *result = 0;
  // the kernel always writes the result word, so it needs no clearing
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(kThreads), 0, stream, sizes, ids, (int)G,
                     (int)E, M, slots, slot_lim);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbolAsync(result, HIP_SYMBOL(g_validate_result), sizeof(int32_t), 0,
                               hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(stream);
}

}  // namespace gnf4
