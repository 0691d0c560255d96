// Decode path of the grouped NF4 GEMM: groups with few rows (batch-1 decode).
//
// Page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE
// expert stacks": opening section (one launch for all active experts, LUT
// decode to fp32 in registers, blockwise fp32 absmax, fp32 accumulation, bf16
// epilogue); "Layout" (a decode GEMV path beside the M-tile path); "Status /
// roadmap" (split-K for starved grids with a per-split work floor; one
// universal launch rule rather than a per-shape table).
//
// The work is bandwidth-bound: at one row per expert every weight byte is
// used once.  Layout of the work:
//  * a workgroup (4 wavefronts) owns one group (expert) and a tile of weight
//    rows n; every lane of a "team" of L lanes (L = 8..64, chosen from K so
//    a row is covered with little raggedness) reads consecutive 16-byte
//    chunks (32 codes) of the same weight row, so each wavefront load is
//    64 x 16 contiguous-per-row bytes;
//  * a lane holds NU weight rows in flight and the matching 32 activations of
//    up to R group rows converted to fp32 once, so one code decode feeds R
//    multiply-adds;
//  * codes are decoded through a 16-entry fp32 table in LDS (16 distinct
//    banks: any mix of codes reads it without bank conflicts), multiplied
//    and accumulated in fp32; the block absmax is applied once per 32-code
//    chunk;
//  * team partial sums are combined with a fixed butterfly, then either
//    rounded to bf16 or, when K is split across workgroups to fill the
//    machine, written as fp32 partials that a second kernel sums in split
//    order (deterministic).

#include <limits.h>

#include "gnf4_internal.h"

namespace gnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

struct DecodeKArgs {
  GemmArgs g;
  int S, cps, cpr, n_tiles, rows_per_block;
};

// Row offset of group g: sum of max(size, 0) over the groups before it.
__device__ __forceinline__ int group_row_offset(const int32_t* sizes, int g, int lane) {
  int sum = 0;
  for (int i = lane; i < g; i += kWave) sum += max(sizes[i], 0);
  return wave_sum(sum);
}

__device__ __forceinline__ void unpack_bf16x8(const uint4 v, float* out) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(d[j] << 16);
    out[2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
  }
}

template <int L, int NU, int R>
__device__ __forceinline__ void decode_rows(const DecodeKArgs& a, int e, int r0, int r_end,
                                            int s, int tile, const float* lut) {
  constexpr int RPW = kWave / L;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int team = lane / L, tl = lane % L;
  const int N = a.g.N, K = a.g.K;
  const int n_base = tile * a.rows_per_block + wave * (RPW * NU) + team * NU;
  const size_t row_bytes = (size_t)K / 2;
  const int blocks_per_row = K / kBlock;
  const uint8_t* wexp = a.g.packed + (size_t)e * N * row_bytes;
  const float* aexp = a.g.absmax + (size_t)e * N * blocks_per_row;
  const int c_begin = s * a.cps;
  const int c_end = min(c_begin + a.cps, a.cpr);

  float acc[NU][R];
#pragma unroll
  for (int j = 0; j < NU; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[j][r] = 0.0f;

  for (int c = c_begin + tl; c < c_end; c += L) {
    uint4 wq[NU];
    float av[NU];
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const int n = n_base + j;
      if (n < N) {
        wq[j] = *reinterpret_cast<const uint4*>(wexp + (size_t)n * row_bytes + 16 * (size_t)c);
        av[j] = aexp[(size_t)n * blocks_per_row + (c >> 1)];
      } else {
        wq[j] = make_uint4(0, 0, 0, 0);
        av[j] = 0.0f;
      }
    }
    float xs[R][32];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r0 + r < r_end) {
        const uint4* xp = reinterpret_cast<const uint4*>(a.g.x + (size_t)(r0 + r) * K + 32 * (size_t)c);
#pragma unroll
        for (int q = 0; q < 4; ++q) unpack_bf16x8(xp[q], &xs[r][8 * q]);
      } else {
#pragma unroll
        for (int q = 0; q < 32; ++q) xs[r][q] = 0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      float part[R];
#pragma unroll
      for (int r = 0; r < R; ++r) part[r] = 0.0f;
      const uint32_t d[4] = {wq[j].x, wq[j].y, wq[j].z, wq[j].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t byte = (d[w] >> (8 * b)) & 0xffu;
          const float vh = lut[byte >> 4];
          const float vl = lut[byte & 0xfu];
          const int k = 8 * w + 2 * b;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            part[r] = fmaf(xs[r][k], vh, part[r]);
            part[r] = fmaf(xs[r][k + 1], vl, part[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) acc[j][r] = fmaf(av[j], part[r], acc[j][r]);
    }
  }

#pragma unroll
  for (int j = 0; j < NU; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float v = acc[j][r];
#pragma unroll
      for (int off = L / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
      acc[j][r] = v;
    }

  if (tl == 0) {
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const int n = n_base + j;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = r0 + r;
        if (row >= r_end) continue;
        if (a.S == 1)
          a.g.y[(size_t)row * N + n] = f32_to_bf16(acc[j][r]);
        else
          a.g.partial[((size_t)s * a.g.M + row) * N + n] = acc[j][r];
      }
    }
  }
}

template <int L, int NU>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeKArgs a) {
  __shared__ float s_lut[16];
  __shared__ int s_off;
  const int g = blockIdx.y;
  const int tile = blockIdx.x % a.n_tiles;
  const int s = blockIdx.x / a.n_tiles;
  const int sz = a.g.sizes[g];
  const int e = a.g.ids[g];
  if (sz <= 0 || sz > a.g.rows_max_decode || e < 0 || e >= a.g.E) return;
  if (threadIdx.x < 16) s_lut[threadIdx.x] = nf4_level(threadIdx.x);
  if (threadIdx.x < kWave) {
    const int off = group_row_offset(a.g.sizes, g, threadIdx.x);
    if (threadIdx.x == 0) s_off = off;
  }
  __syncthreads();
  const int r_begin = s_off;
  const int r_end = min(r_begin + sz, a.g.M);
  for (int r0 = r_begin; r0 < r_end;) {
    const int rem = r_end - r0;
    if (rem >= 3) {
      decode_rows<L, NU, 4>(a, e, r0, r_end, s, tile, s_lut);
      r0 += 4;
    } else if (rem == 2) {
      decode_rows<L, NU, 2>(a, e, r0, r_end, s, tile, s_lut);
      r0 += 2;
    } else {
      decode_rows<L, NU, 1>(a, e, r0, r_end, s, tile, s_lut);
      r0 += 1;
    }
  }
}

// Sum the S split partials of every decode-path row in split order -> bf16.
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(DecodeKArgs a) {
  __shared__ int s_off;
  const int g = blockIdx.y;
  const int sz = a.g.sizes[g];
  const int e = a.g.ids[g];
  if (sz <= 0 || sz > a.g.rows_max_decode || e < 0 || e >= a.g.E) return;
  if (threadIdx.x < kWave) {
    const int off = group_row_offset(a.g.sizes, g, threadIdx.x);
    if (threadIdx.x == 0) s_off = off;
  }
  __syncthreads();
  const int r_begin = s_off;
  const int r_end = min(r_begin + sz, a.g.M);
  const int n = blockIdx.x * kThreads + threadIdx.x;
  if (n >= a.g.N) return;
  const size_t plane = (size_t)a.g.M * a.g.N;
  for (int r = r_begin; r < r_end; ++r) {
    const float* p = a.g.partial + (size_t)r * a.g.N + n;
    float sum = 0.0f;
    for (int si = 0; si < a.S; ++si) sum += p[si * plane];
    a.g.y[(size_t)r * a.g.N + n] = f32_to_bf16(sum);
  }
}

int pick_lanes(int cps) {
  // largest team that covers the split's chunks with <= 1/8 idle slots
  const int cands[4] = {64, 32, 16, 8};
  int best = 8;
  double best_waste = 2.0;
  for (int L : cands) {
    const int steps = (cps + L - 1) / L;
    const double waste = (double)(steps * L - cps) / (double)(steps * L);
    if (waste <= 0.125) return L;
    if (waste < best_waste) {
      best_waste = waste;
      best = L;
    }
  }
  return best;
}

template <int L>
hipError_t launch_L(const DecodeKArgs& a, const DecodePlan& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.n_tiles * p.S), (unsigned)a.g.G);
  switch (p.NU) {
    case 4: hipLaunchKernelGGL((decode_kernel<L, 4>), grid, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<L, 2>), grid, dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((decode_kernel<L, 1>), grid, dim3(kThreads), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int64_t M, int64_t N, int64_t K, int64_t G, int split_k, int num_cus) {
  const int cpr = (int)(K / 32);
  const int64_t g_eff = G < M ? G : M;
  const int64_t target = 2LL * num_cus;  // workgroups that keep every CU busy
  DecodePlan best{};
  int64_t best_blocks = -1;
  const int s_cands[4] = {1, 2, 4, 8};
  for (int si = 0; si < 4; ++si) {
    const int S = split_k > 0 ? split_k : s_cands[si];
    if (split_k <= 0 && si > 0) {
      // split only when it keeps at least two full team steps per split
      const int cps_try = (cpr + S - 1) / S;
      if (cps_try < 2 * pick_lanes(cps_try)) break;
    }
    const int cps = (cpr + S - 1) / S;
    const int L = pick_lanes(cps);
    const int nus[3] = {4, 2, 1};
    for (int ni = 0; ni < 3; ++ni) {
      DecodePlan p;
      p.L = L;
      p.NU = nus[ni];
      p.S = S;
      p.cps = cps;
      p.rows_per_block = kWaves * (kWave / L) * p.NU;
      p.n_tiles = (int)((N + p.rows_per_block - 1) / p.rows_per_block);
      const int64_t blocks = g_eff * p.n_tiles * S;
      if (blocks >= target) return p;
      if (blocks > best_blocks) {
        best_blocks = blocks;
        best = p;
      }
    }
    if (split_k > 0) break;
  }
  return best;
}

size_t decode_workspace_bytes(const DecodePlan& p, int64_t M, int64_t N) {
  return p.S > 1 ? (size_t)p.S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_decode(const GemmArgs& g, const DecodePlan& p, hipStream_t stream) {
  DecodeKArgs a;
  a.g = g;
  a.S = p.S;
  a.cps = p.cps;
  a.cpr = g.K / 32;
  a.n_tiles = p.n_tiles;
  a.rows_per_block = p.rows_per_block;
  hipError_t err;
  switch (p.L) {
    case 64: err = launch_L<64>(a, p, stream); break;
    case 32: err = launch_L<32>(a, p, stream); break;
    case 16: err = launch_L<16>(a, p, stream); break;
    default: err = launch_L<8>(a, p, stream); break;
  }
  if (err != hipSuccess || p.S == 1) return err;
  const dim3 grid((unsigned)((g.N + kThreads - 1) / kThreads), (unsigned)g.G);
  hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gnf4
