// Router top-k with softmax weights and the token->expert sort.
//
// Page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE
// expert stacks", opening section: the GEMM takes (sizes, expert_ids) "after
// the usual token->expert sort"; landing page "grouped-nf4-gemm", "Use this
// when": router softmax and top-k folded into one decode-step launch.
//
// Design (all integer work bit-exact and free of atomics that decide an
// order):
//  * top-k: one wavefront per token.  Each lane holds up to 16 logits
//    (experts lane, lane+64, ...); k rounds of a wave-wide arg-max over
//    (logit desc, id asc) pick the experts.  Weights are the softmax of the k
//    selected logits in fp32.
//  * sort: a counting sort by expert over chunks of tokens.  Per chunk an LDS
//    histogram (counts commute, so LDS atomics are safe); an exclusive scan
//    over (expert, chunk) gives every chunk's first row per expert; one
//    wavefront per chunk then walks its slots in ascending order, ranking
//    equal experts inside each 64-slot batch with ballots, so the output is
//    the stable order.
//  * small batches (every decode step) fit one chunk and run as ONE launch;
//    larger ones use three (top-k + histogram, scan, scatter).

#include <limits.h>
#include <math.h>

#include "gnf4_internal.h"

namespace gnf4 {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kChunkTokens = 64;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kEPL = kMaxE / kWave;  // logits held per lane

struct RouteArgs {
  const float* logits;
  int T, E, K;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* offsets;
  int32_t* sorted;
  int32_t* gsizes;
  int32_t* gids;
  int32_t* ngroups;
  int32_t* ws;       // [n_chunks, E] per-chunk counts, then per-chunk bases
  int n_chunks;
};

// Order-preserving unsigned key of a float; -0.0 is folded onto +0.0 so the
// two compare equal (and the lower id wins), as float comparison does.
__device__ __forceinline__ uint32_t float_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Top-k of one token by one wavefront.  Lane i ends up holding the i-th
// pick.  Each round is two DPP reductions: the largest key, then the lowest
// expert id among the lanes holding it.
__device__ void topk_token(const float* __restrict__ row, int E, int k, int lane,
                           int32_t* __restrict__ ids_out, float* __restrict__ w_out,
                           int32_t* lds_ids) {
  uint32_t key[kEPL];
  uint32_t avail = 0;
#pragma unroll
  for (int j = 0; j < kEPL; ++j) {
    const int e = lane + kWave * j;
    key[j] = 0u;  // below every finite value's key
    if (e < E) {
      key[j] = float_key(row[e]);
      avail |= 1u << j;
    }
  }
  float my_v = 0.0f;
  int my_id = 0;
  for (int i = 0; i < k; ++i) {
    uint32_t bk = 0u, bid = 0xffffffffu;
#pragma unroll
    for (int j = 0; j < kEPL; ++j) {
      if ((avail & (1u << j)) && (bid == 0xffffffffu || key[j] > bk)) {
        bk = key[j];
        bid = (uint32_t)(lane + kWave * j);
      }
    }
    const uint32_t wk = wave_max_u32(bk);
    const uint32_t wid = wave_min_u32(bk == wk ? bid : 0xffffffffu);
    if (lane == (int)(wid & (kWave - 1))) avail &= ~(1u << (wid >> 6));
    if (lane == i) {
      my_v = key_float(wk);
      my_id = (int)wid;
    }
  }
  const float vmax = __shfl(my_v, 0, kWave);
  const float ex = (lane < k) ? expf(my_v - vmax) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids_out[lane] = my_id;
    w_out[lane] = ex / sum;
    if (lds_ids) lds_ids[lane] = my_id;
  }
}

// Wave 0: exclusive scan of cnt[0..E) into base[] (LDS) and offsets[] (global),
// compaction of the non-empty experts into the group arrays.
__device__ void scan_and_groups(const int32_t* cnt, int32_t* base, const RouteArgs& a, int lane) {
  int carry = 0, gcarry = 0;
  for (int b0 = 0; b0 < a.E; b0 += kWave) {
    const int e = b0 + lane;
    const int c = (e < a.E) ? cnt[e] : 0;
    const int inc = wave_incl_scan(c);
    const int excl = carry + inc - c;
    const int f = (c > 0) ? 1 : 0;
    const int finc = wave_incl_scan(f);
    const int pos = gcarry + finc - f;
    if (e < a.E) {
      if (base) base[e] = excl;
      a.offsets[e] = excl;
      if (f) {
        a.gsizes[pos] = c;
        a.gids[pos] = e;
      }
    }
    carry += __shfl(inc, kWave - 1, kWave);
    gcarry += __shfl(finc, kWave - 1, kWave);
  }
  if (lane == 0) {
    a.offsets[a.E] = carry;
    a.ngroups[0] = gcarry;
  }
  for (int i = gcarry + lane; i < a.E; i += kWave) {
    a.gsizes[i] = 0;
    a.gids[i] = 0;
  }
}

// One wave: stable scatter of slots [s0, s1) whose experts are ids[s - s0],
// starting from per-expert bases in LDS (updated in place).
__device__ void scatter_slots(const int32_t* ids, int s0, int s1, int32_t* base, int E,
                              int32_t* __restrict__ sorted, int lane) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int b0 = s0; b0 < s1; b0 += kWave) {
    const int s = b0 + lane;
    const bool active = s < s1;
    const int e = active ? ids[s - s0] : 0;
    uint64_t peers = __ballot(active);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool b = (e >> bit) & 1;
      const uint64_t bal = __ballot(active && b);
      peers &= b ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt);
    int start = 0;
    if (active) start = base[e];
    __builtin_amdgcn_wave_barrier();  // every lane reads base[e] before any update
    if (active) {
      sorted[start + rank] = s;
      const bool leader = (peers & lt) == 0;
      if (leader) base[e] = start + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();  // LDS ops of one wave complete in order
  }
}

// Whole sort in one workgroup: T * K fits one chunk.
__global__ __launch_bounds__(kRouteThreads) void route_fused_kernel(RouteArgs a) {
  __shared__ int32_t s_ids[kChunkTokens * kMaxK];
  __shared__ int32_t s_cnt[kMaxE];
  __shared__ int32_t s_base[kMaxE];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int M = a.T * a.K;
  for (int t = wave; t < a.T; t += kRouteThreads / kWave)
    topk_token(a.logits + (size_t)t * a.E, a.E, a.K, lane, a.topk_ids + (size_t)t * a.K,
               a.topk_w + (size_t)t * a.K, s_ids + t * a.K);
  for (int e = threadIdx.x; e < a.E; e += kRouteThreads) s_cnt[e] = 0;
  __syncthreads();
  for (int s = threadIdx.x; s < M; s += kRouteThreads) atomicAdd(&s_cnt[s_ids[s]], 1);
  __syncthreads();
  if (wave == 0) {
    scan_and_groups(s_cnt, s_base, a, lane);
    __builtin_amdgcn_wave_barrier();
    scatter_slots(s_ids, 0, M, s_base, a.E, a.sorted, lane);
  }
}

// Large batches, step 1: top-k of the chunk's tokens and its expert histogram.
__global__ __launch_bounds__(kRouteThreads) void route_topk_hist_kernel(RouteArgs a) {
  __shared__ int32_t s_ids[kChunkTokens * kMaxK];
  __shared__ int32_t s_cnt[kMaxE];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int c = blockIdx.x;
  const int t0 = c * kChunkTokens;
  const int t1 = min(t0 + kChunkTokens, a.T);
  for (int t = t0 + wave; t < t1; t += kRouteThreads / kWave)
    topk_token(a.logits + (size_t)t * a.E, a.E, a.K, lane, a.topk_ids + (size_t)t * a.K,
               a.topk_w + (size_t)t * a.K, s_ids + (t - t0) * a.K);
  for (int e = threadIdx.x; e < a.E; e += kRouteThreads) s_cnt[e] = 0;
  __syncthreads();
  const int n = (t1 - t0) * a.K;
  for (int s = threadIdx.x; s < n; s += kRouteThreads) atomicAdd(&s_cnt[s_ids[s]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += kRouteThreads) a.ws[(size_t)c * a.E + e] = s_cnt[e];
}

// Large batches, step 2 (one workgroup of 1024): per-expert totals, the scan,
// the groups, and every chunk's base row per expert (in place of its count).
__global__ __launch_bounds__(1024) void route_scan_kernel(RouteArgs a) {
  __shared__ int32_t s_tot[kMaxE];
  const int e = threadIdx.x;
  if (e < a.E) {
    int run = 0;
    for (int c = 0; c < a.n_chunks; ++c) {
      int32_t* p = a.ws + (size_t)c * a.E + e;
      const int cnt = *p;
      *p = run;
      run += cnt;
    }
    s_tot[e] = run;
  }
  __syncthreads();
  __shared__ int32_t s_base[kMaxE];
  if (threadIdx.x < kWave) scan_and_groups(s_tot, s_base, a, threadIdx.x);
  __syncthreads();
  if (e < a.E) {
    const int b = s_base[e];
    for (int c = 0; c < a.n_chunks; ++c) a.ws[(size_t)c * a.E + e] += b;
  }
}

// Large batches, step 3: one wavefront per chunk scatters its slots.
__global__ __launch_bounds__(kWave) void route_scatter_kernel(RouteArgs a) {
  __shared__ int32_t s_base[kMaxE];
  __shared__ int32_t s_ids[kChunkTokens * kMaxK];
  const int c = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < a.E; e += kWave) s_base[e] = a.ws[(size_t)c * a.E + e];
  const int s0 = c * kChunkTokens * a.K;
  const int s1 = min(s0 + kChunkTokens * a.K, a.T * a.K);
  for (int s = s0 + lane; s < s1; s += kWave) s_ids[s - s0] = a.topk_ids[s];
  __builtin_amdgcn_wave_barrier();
  scatter_slots(s_ids, s0, s1, s_base, a.E, a.sorted, lane);
}

// T == 0: zero offsets and groups.
__global__ void route_empty_kernel(RouteArgs a) {
  for (int i = threadIdx.x; i <= a.E; i += blockDim.x) a.offsets[i] = 0;
  for (int i = threadIdx.x; i < a.E; i += blockDim.x) {
    a.gsizes[i] = 0;
    a.gids[i] = 0;
  }
  if (threadIdx.x == 0) a.ngroups[0] = 0;
}

}  // namespace

RoutePlan plan_route(int64_t T, int64_t E, int top_k) {
  RoutePlan p;
  p.chunk_tokens = kChunkTokens;
  p.n_chunks = (int)((T + kChunkTokens - 1) / kChunkTokens);
  p.ws_bytes = p.n_chunks > 1 ? (size_t)p.n_chunks * (size_t)E * sizeof(int32_t) : 0;
  (void)top_k;
  return p;
}

hipError_t launch_route_sort(const float* logits, int T, int E, int top_k, int32_t* topk_ids,
                             float* topk_w, int32_t* expert_offsets, int32_t* sorted_slots,
                             int32_t* group_sizes, int32_t* group_expert_ids,
                             int32_t* num_groups, int32_t* ws, const RoutePlan& plan,
                             hipStream_t stream) {
  RouteArgs a;
  a.logits = logits;
  a.T = T;
  a.E = E;
  a.K = top_k;
  a.topk_ids = topk_ids;
  a.topk_w = topk_w;
  a.offsets = expert_offsets;
  a.sorted = sorted_slots;
  a.gsizes = group_sizes;
  a.gids = group_expert_ids;
  a.ngroups = num_groups;
  a.ws = ws;
  a.n_chunks = plan.n_chunks;
  if (T == 0) {
    hipLaunchKernelGGL(route_empty_kernel, dim3(1), dim3(256), 0, stream, a);
  } else if (plan.n_chunks == 1) {
    hipLaunchKernelGGL(route_fused_kernel, dim3(1), dim3(kRouteThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(route_topk_hist_kernel, dim3(plan.n_chunks), dim3(kRouteThreads), 0,
                       stream, a);
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
    hipLaunchKernelGGL(route_scatter_kernel, dim3(plan.n_chunks), dim3(kWave), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace gnf4
