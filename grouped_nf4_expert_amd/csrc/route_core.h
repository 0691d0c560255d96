// Router top-k of a single token, shared by the route/sort kernels and the
// decode GEMM that folds a batch-1 decode step's routing into its launch
// (landing page "grouped-nf4-gemm", "Use this when": router softmax and
// top-k folded into one decode-step launch).  Both run this code, so their
// picks and weights are the same bits.
#pragma once

#include <math.h>

#include "gnf4_internal.h"

namespace gnf4 {

// Order-preserving unsigned key of a float; -0.0 is folded onto +0.0 so the
// two compare equal (and the lower id wins), as float comparison does.
__device__ __forceinline__ uint32_t float_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __int_as_float((int)dpp_u32<0xB1, 0xF>(0u, __float_as_uint(v)));
  v += __int_as_float((int)dpp_u32<0x4E, 0xF>(0u, __float_as_uint(v)));
  v += __int_as_float((int)dpp_u32<0x141, 0xF>(0u, __float_as_uint(v)));
  v += __int_as_float((int)dpp_u32<0x140, 0xF>(0u, __float_as_uint(v)));
  v += __int_as_float((int)dpp_u32<0x142, 0xA>(0u, __float_as_uint(v)));
  v += __int_as_float((int)dpp_u32<0x143, 0xC>(0u, __float_as_uint(v)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Ranks of one token's E logits.  Entry s of a lane is expert lane + 64 s;
// rank = number of better entries.  Returns the logits in `val`.
template <int EPL>
__device__ __forceinline__ void rank_token(const float* __restrict__ row, int E, int lane,
                                           float (&val)[EPL], int (&rank)[EPL]) {
  uint64_t key[EPL];
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    const int e = lane + kWave * s;
    val[s] = (e < E) ? row[e] : 0.0f;
    key[s] = (e < E) ? (((uint64_t)float_key(val[s]) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e))
                     : 0ull;
    rank[s] = 0;
  }
#pragma unroll
  for (int s2 = 0; s2 < EPL; ++s2) {
    if (kWave * s2 >= E) break;
    for (int j = 0; j < kWave; ++j) {
      const uint64_t kj = readlane64(key[s2], j);
#pragma unroll
      for (int s = 0; s < EPL; ++s) rank[s] += (kj > key[s]) ? 1 : 0;
    }
  }
}

// The route/sort outputs of a single token, as gnf4_route_sort writes them.
struct RouteOneOut {
  int E, K;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* offsets;
  int32_t* sorted;
  int32_t* rows;  // optional
  int32_t* gsizes;
  int32_t* gids;
  int32_t* ngroups;
};

// One wavefront, one token, from rank_token's logits and ranks: the picks
// (rank < K) and their softmax in fp32.  A single token needs no sort: its
// picks are distinct experts, so each pick's place in expert order is a
// ballot prefix count.
template <int EPL>
__device__ void route_one_token_write(const RouteOneOut& o, int lane, const float (&val)[EPL],
                                      const int (&rank)[EPL]) {
  float vbest = 0.0f;
  uint64_t sel[EPL];
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    const uint64_t has = __ballot(rank[s] == 0);
    if (has) vbest = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(val[s]),
                                                              __ffsll((unsigned long long)has) - 1));
    sel[s] = __ballot(rank[s] < o.K);
  }
  float ex[EPL];
  float part = 0.0f;
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    ex[s] = (rank[s] < o.K) ? expf(val[s] - vbest) : 0.0f;
    part += ex[s];
  }
  const float sum = wave_sum_f32(part);
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  int before = 0;  // picks with a lower expert id than entry (s, lane)
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    const int e = lane + kWave * s;
    const int pos = before + __popcll(sel[s] & lt);
    if (e < o.E) o.offsets[e] = pos;
    if (rank[s] < o.K) {
      o.topk_ids[rank[s]] = e;
      o.topk_w[rank[s]] = ex[s] / sum;
      o.sorted[pos] = rank[s];  // slot t * k + j with t = 0
      if (o.rows) o.rows[rank[s]] = pos;
      o.gsizes[pos] = 1;
      o.gids[pos] = e;
    }
    before += __popcll(sel[s]);
  }
  if (lane == 0) {
    o.offsets[o.E] = o.K;
    o.ngroups[0] = o.K;
  }
  for (int i = o.K + lane; i < o.E; i += kWave) {
    o.gsizes[i] = 0;
    o.gids[i] = 0;
  }
}

// The decode GEMM with a single token's routing folded into its launch
// (decode.hip): every group on the decode path, groups and slots from the
// token's picks, route/sort outputs written as ro describes.  E <= 64,
// g.slots / g.sizes / g.ids name ro's sorted / gsizes / gids arrays (read
// only by a split-K reduce, after the launch).
hipError_t launch_decode_routed(const GemmArgs& g, const DecodePlan& p, const float* logits,
                                const RouteOneOut& ro, hipStream_t stream);

// One token's expert feed-forward in one launch (decode.hip): routing,
// gate_up [E, 2I, H] (gate half first), SwiGLU, down [E, H, I].  The two
// projections use the plans their one-token decode launches would, unsplit.
struct FfnPlan {
  DecodePlan gu, dn;
  int gu_tiles, dn_tiles;  // workgroups per pick
};
bool ffn_supported(const FfnPlan& p);
int ffn_resident_per_cu(const FfnPlan& p, bool two_entries);
// bytes of the launch's synchronisation words for top_k picks
size_t ffn_sync_bytes(int top_k);
// false when the shapes have no fused kernel (the caller then runs the steps
// as separate launches)
bool plan_ffn(int64_t E, int top_k, int64_t H, int64_t I, int num_cus, FfnPlan& out);
hipError_t launch_ffn_one_token(const FfnPlan& p, const float* logits, const uint16_t* x,
                                const uint8_t* gu_packed, const void* gu_absmax,
                                const uint8_t* dn_packed, const void* dn_absmax, bool abs_bf16,
                                int E, int top_k, int H, int I, uint16_t* h, uint16_t* y,
                                int32_t* sync, const RouteOneOut& ro, hipStream_t stream);

}  // namespace gnf4
