// Router top-k with softmax weights and the token->expert sort.
//
// Page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE
// expert stacks", opening section: the GEMM takes (sizes, expert_ids) "after
// the usual token->expert sort"; landing page "grouped-nf4-gemm", "Use this
// when": router softmax and top-k folded into one decode-step launch.
//
// Design (all integer work bit-exact and free of atomics that decide an
// order):
//  * top-k by rank: each logit becomes a unique 64-bit key (order-preserving
//    float key in the high half, the complement of the expert id in the low
//    half: larger = better, equal logits go to the lower id).  One
//    wavefront per token.  Up to 64 experts a lane ranks its key against
//    every key of the token (broadcast with readlane) -- independent
//    compare-adds instead of k dependent arg-max rounds; above 64, the k-th
//    largest key is found bit by bit from ballot counts and only the k picks
//    are ranked against each other.  The keys ranked below k are the picks,
//    in order.  Weights are the softmax of the k picks in fp32.
//  * a single token (every batch-1 decode step) needs no sort at all: its
//    picks are distinct experts, so each pick's place in expert order is a
//    ballot prefix count; one wavefront writes every output.
//  * more tokens: a counting sort by expert over chunks of tokens.  Per
//    chunk an LDS histogram (counts commute, so LDS atomics are safe); an
//    exclusive scan over (expert, chunk) gives every chunk's first row per
//    expert; one wavefront per chunk then walks its slots in ascending order,
//    ranking equal experts inside each 64-slot batch with ballots, so the
//    output is the stable order.  Up to 32 tokens run as ONE launch (16
//    wavefronts); larger batches use three (top-k + histogram, scan,
//    scatter) over chunks of 16 tokens, one per wavefront of a 16-wavefront
//    workgroup, so a batch of T tokens spreads over T / 16 workgroups.

#include <math.h>

#include "gnf4_internal.h"
#include "route_core.h"

namespace gnf4 {
namespace {

constexpr int kRouteThreads = 1024;  // 16 wavefronts: one token each at a time
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kFusedTokens = 32;  // the single-launch sort takes up to this many tokens
constexpr int kChunkTokens = 16;  // tokens per chunk of the three-launch sort
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;

struct RouteArgs {
  const float* logits;
  int T, E, K;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* offsets;
  int32_t* sorted;
  int32_t* rows;     // optional: grouped row of each flat slot
  int32_t* gsizes;
  int32_t* gids;
  int32_t* ngroups;
  int32_t* ws;       // [n_chunks, E] per-chunk counts, then per-chunk bases
  int n_chunks;
};

// Ranks of one token's k picks for E > 64, by threshold: the k-th largest
// key T is built bit by bit from the top, a bit kept when at least k keys
// are >= the candidate (ballot counts); the keys >= T are the k picks, and a
// pick's rank is the number of picks above it (non-picks get rank k).  The
// keys are rank_token's (float key, then the complement of the expert id;
// absent entries 0, below every real key), so the picks, their order and the
// ties are the same.  A real key's low word is 0xffffffff - e with e < 1024,
// so once the high word of T is known its bits 31..10 are all ones.
template <int EPL>
__device__ __forceinline__ void rank_picks(const float* __restrict__ row, int E, int k, int lane,
                                           float (&val)[EPL], int (&rank)[EPL]) {
  uint32_t hi[EPL];
  uint64_t key[EPL];
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    const int e = lane + kWave * s;
    val[s] = (e < E) ? row[e] : 0.0f;
    hi[s] = (e < E) ? float_key(val[s]) : 0u;
    key[s] = (e < E) ? (((uint64_t)hi[s] << 32) | (uint32_t)(0xffffffffu - (uint32_t)e)) : 0ull;
  }
  // the high word of T: the k-th largest float key, counting equal ones
  uint32_t th = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = th | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < EPL; ++s) cnt += __popcll(__ballot(hi[s] >= cand));
    if (cnt >= k) th = cand;
  }
  // the low word: bits 31..10 are ones; bits 9..0 pick among equal logits
  uint64_t t = ((uint64_t)th << 32) | 0xfffffc00u;
  for (int b = 9; b >= 0; --b) {
    const uint64_t cand = t | (1ull << b);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < EPL; ++s) cnt += __popcll(__ballot(key[s] >= cand));
    if (cnt >= k) t = cand;
  }
  // every pick against every other (k broadcasts)
#pragma unroll
  for (int s = 0; s < EPL; ++s) rank[s] = 0;
#pragma unroll
  for (int s2 = 0; s2 < EPL; ++s2) {
    uint64_t m = __ballot(key[s2] >= t);
    while (m) {
      const int src = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const uint64_t kj = readlane64(key[s2], src);
#pragma unroll
      for (int s = 0; s < EPL; ++s) rank[s] += (kj > key[s]) ? 1 : 0;
    }
  }
#pragma unroll
  for (int s = 0; s < EPL; ++s)
    if (key[s] < t) rank[s] = k;
}

// Top-k of one token: ids/weights to global memory (and ids to LDS).
template <int EPL>
__device__ void topk_token(const float* __restrict__ row, int E, int k, int lane,
                           int32_t* __restrict__ ids_out, float* __restrict__ w_out,
                           int32_t* lds_ids) {
  float val[EPL];
  int rank[EPL];
  if constexpr (EPL == 1)
    rank_token<EPL>(row, E, lane, val, rank);
  else
    rank_picks<EPL>(row, E, k, lane, val, rank);
  // the best logit (rank 0) for a stable softmax
  float vbest = 0.0f;
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    // exactly one entry of the token has rank 0
    const uint64_t has = __ballot(rank[s] == 0);
    if (has) {
      const int src = __ffsll((unsigned long long)has) - 1;
      vbest = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(val[s]), src));
    }
  }
  float ex[EPL];
  float part = 0.0f;
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    ex[s] = (rank[s] < k) ? expf(val[s] - vbest) : 0.0f;
    part += ex[s];
  }
  const float sum = wave_sum_f32(part);
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    if (rank[s] < k) {
      const int e = lane + kWave * s;
      ids_out[rank[s]] = e;
      w_out[rank[s]] = ex[s] / sum;
      if (lds_ids) lds_ids[rank[s]] = e;
    }
  }
}

// A single token: top-k and the whole sort in one wavefront.
template <int EPL>
__global__ __launch_bounds__(kWave) void route_one_token_kernel(RouteArgs a) {
  const int lane = threadIdx.x;
  float val[EPL];
  int rank[EPL];
  rank_token<EPL>(a.logits, a.E, lane, val, rank);
  RouteOneOut o;
  o.E = a.E;
  o.K = a.K;
  o.topk_ids = a.topk_ids;
  o.topk_w = a.topk_w;
  o.offsets = a.offsets;
  o.sorted = a.sorted;
  o.rows = a.rows;
  o.gsizes = a.gsizes;
  o.gids = a.gids;
  o.ngroups = a.ngroups;
  route_one_token_write<EPL>(o, lane, val, rank);
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
    carry += __builtin_amdgcn_readlane(inc, kWave - 1);
    gcarry += __builtin_amdgcn_readlane(finc, kWave - 1);
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
                              int32_t* __restrict__ sorted, int32_t* __restrict__ rows,
                              int lane) {
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
      if (rows) rows[s] = start + rank;
      const bool leader = (peers & lt) == 0;
      if (leader) base[e] = start + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();  // LDS ops of one wave complete in order
  }
}

// Whole sort in one workgroup: T * K fits one chunk.
template <int EPL>
__global__ __launch_bounds__(kRouteThreads) void route_fused_kernel(RouteArgs a) {
  __shared__ int32_t s_ids[kFusedTokens * kMaxK];
  __shared__ int32_t s_cnt[kMaxE];
  __shared__ int32_t s_base[kMaxE];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int M = a.T * a.K;
  for (int e = threadIdx.x; e < a.E; e += kRouteThreads) s_cnt[e] = 0;
  for (int t = wave; t < a.T; t += kRouteWaves)
    topk_token<EPL>(a.logits + (size_t)t * a.E, a.E, a.K, lane, a.topk_ids + (size_t)t * a.K,
                    a.topk_w + (size_t)t * a.K, s_ids + t * a.K);
  __syncthreads();
  for (int s = threadIdx.x; s < M; s += kRouteThreads) atomicAdd(&s_cnt[s_ids[s]], 1);
  __syncthreads();
  if (wave == 0) {
    scan_and_groups(s_cnt, s_base, a, lane);
    __builtin_amdgcn_wave_barrier();
    scatter_slots(s_ids, 0, M, s_base, a.E, a.sorted, a.rows, lane);
  }
}

// Large batches, step 1: top-k of the chunk's tokens and its expert histogram.
template <int EPL>
__global__ __launch_bounds__(kRouteThreads) void route_topk_hist_kernel(RouteArgs a) {
  __shared__ int32_t s_ids[kChunkTokens * kMaxK];
  __shared__ int32_t s_cnt[kMaxE];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int c = blockIdx.x;
  const int t0 = c * kChunkTokens;
  const int t1 = min(t0 + kChunkTokens, a.T);
  for (int e = threadIdx.x; e < a.E; e += kRouteThreads) s_cnt[e] = 0;
  for (int t = t0 + wave; t < t1; t += kRouteWaves)
    topk_token<EPL>(a.logits + (size_t)t * a.E, a.E, a.K, lane, a.topk_ids + (size_t)t * a.K,
                    a.topk_w + (size_t)t * a.K, s_ids + (t - t0) * a.K);
  __syncthreads();
  const int n = (t1 - t0) * a.K;
  for (int s = threadIdx.x; s < n; s += kRouteThreads) atomicAdd(&s_cnt[s_ids[s]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += kRouteThreads) a.ws[(size_t)c * a.E + e] = s_cnt[e];
}

// Large batches, step 2 (one workgroup of 1024): per-expert totals, the scan,
// the groups, and every chunk's base row per expert (in place of its count).
// Q = 1024 / E' threads per expert (E' is E rounded up to a power of two,
// at least 64, so Q is 16, 8, 4, 2 or 1) each take a contiguous range of the
// chunks with up to 16 count loads in flight: pass 1 sums the range, pass 2
// writes the bases after the expert scan.
__global__ __launch_bounds__(1024) void route_scan_kernel(RouteArgs a) {
  __shared__ int32_t s_tot[kMaxE];
  __shared__ int32_t s_base[kMaxE];
  __shared__ int32_t s_part[1024];
  constexpr int kB = 16;
  int ep = kWave;
  while (ep < a.E) ep *= 2;
  const int Q = 1024 / ep;
  const int e = threadIdx.x % ep, q = threadIdx.x / ep;
  const int per = (a.n_chunks + Q - 1) / Q;
  const int c_begin = min(q * per, a.n_chunks);
  const int c_end = min(c_begin + per, a.n_chunks);
  const bool mine = e < a.E;
  int32_t* col = a.ws + (mine ? e : 0);  // column e of the [n_chunks, E] counts
  // pass 1: this thread's share of expert e's count
  int part = 0;
  if (mine) {
    for (int c0 = c_begin; c0 < c_end; c0 += kB) {
      int v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int t = col[(size_t)min(c0 + u, c_end - 1) * a.E];
        v[u] = c0 + u < c_end ? t : 0;
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) part += v[u];
    }
  }
  s_part[threadIdx.x] = part;
  __syncthreads();
  if (threadIdx.x < ep && mine) {
    int run = 0;
    for (int qq = 0; qq < Q; ++qq) run += s_part[qq * ep + e];
    s_tot[e] = run;
  }
  __syncthreads();
  if (threadIdx.x < kWave) scan_and_groups(s_tot, s_base, a, threadIdx.x);
  __syncthreads();
  if (!mine) return;
  // pass 2: the base row of every chunk in the range
  int run = s_base[e];
  for (int qq = 0; qq < q; ++qq) run += s_part[qq * ep + e];
  for (int c0 = c_begin; c0 < c_end; c0 += kB) {
    int v[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) v[u] = col[(size_t)min(c0 + u, c_end - 1) * a.E];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      if (c0 + u < c_end) {
        col[(size_t)(c0 + u) * a.E] = run;
        run += v[u];
      }
    }
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
  scatter_slots(s_ids, s0, s1, s_base, a.E, a.sorted, a.rows, lane);
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

template <int EPL>
void launch_epl(const RouteArgs& a, const RoutePlan& plan, hipStream_t stream) {
  if (a.T == 1) {
    hipLaunchKernelGGL(route_one_token_kernel<EPL>, dim3(1), dim3(kWave), 0, stream, a);
  } else if (plan.n_chunks == 0) {
    hipLaunchKernelGGL(route_fused_kernel<EPL>, dim3(1), dim3(kRouteThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(route_topk_hist_kernel<EPL>, dim3(plan.n_chunks), dim3(kRouteThreads), 0,
                       stream, a);
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
    hipLaunchKernelGGL(route_scatter_kernel, dim3(plan.n_chunks), dim3(kWave), 0, stream, a);
  }
}

}  // namespace

RoutePlan plan_route(int64_t T, int64_t E, int top_k) {
  RoutePlan p;
  p.chunk_tokens = kChunkTokens;
  p.n_chunks = T <= kFusedTokens ? 0 : (int)((T + kChunkTokens - 1) / kChunkTokens);
  p.ws_bytes = (size_t)p.n_chunks * (size_t)E * sizeof(int32_t);
  (void)top_k;
  return p;
}

hipError_t launch_route_sort(const float* logits, int T, int E, int top_k, int32_t* topk_ids,
                             float* topk_w, int32_t* expert_offsets, int32_t* sorted_slots,
                             int32_t* slot_rows, int32_t* group_sizes, int32_t* group_expert_ids,
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
  a.rows = slot_rows;
  a.gsizes = group_sizes;
  a.gids = group_expert_ids;
  a.ngroups = num_groups;
  a.ws = ws;
  a.n_chunks = plan.n_chunks;
  if (T == 0) {
    hipLaunchKernelGGL(route_empty_kernel, dim3(1), dim3(256), 0, stream, a);
  } else if (E <= 64) {
    launch_epl<1>(a, plan, stream);
  } else if (E <= 128) {
    launch_epl<2>(a, plan, stream);
  } else if (E <= 256) {
    launch_epl<4>(a, plan, stream);
  } else if (E <= 512) {
    launch_epl<8>(a, plan, stream);
  } else {
    launch_epl<16>(a, plan, stream);
  }
  return hipGetLastError();
}

}  // namespace gnf4
