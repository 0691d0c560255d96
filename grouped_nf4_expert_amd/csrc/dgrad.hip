// Activation gradient of the grouped NF4 GEMM: dx[r, :] = dy[r, :] . W[e]
// for the rows r of each group (expert e), over the same packed stack.
//
// Landing page "grouped-nf4-gemm", "Owns": the grouped packed GEMM and its
// dgrad.  The contraction runs over N, across the rows of the K-contiguous
// [N, K/2] codes, so the access is the transpose of the forward GEMM's:
//  * a lane owns one 16-byte chunk (32 consecutive k) of the weight rows and
//    accumulates those 32 outputs in fp32 for up to R rows of dy; a team of
//    L lanes (64, 32, 16 or 8, from K, so few lanes sit past the row's end)
//    covers L consecutive chunks, and the 64 / L teams of a wavefront walk
//    different rows of a slice of N, 8 rows per team in flight at a time
//    (16-byte code loads coalesced across the team, the block absmax, and
//    dy[r, n], the same for the whole team);
//  * each code is decoded through a 16-entry fp32 table in LDS at an 8-byte
//    stride (conflict-free for any mix of codes) and multiplied-added with
//    dy[r, n] * absmax, computed once per row and block;
//  * the 8 wavefronts of a workgroup cover disjoint row slices; their
//    partial sums meet in LDS and are added in wavefront order;
//  * at one row of dy per pass (groups of about one row) every row has its
//    own workgroup slot, so the rows of a larger group run side by side
//    instead of as passes one after another;
//  * when N is split across workgroups to fill the machine, each split
//    writes fp32 partials that a second kernel sums in split order, so the
//    result is deterministic run to run.
// Every weight byte is read once per pass of R rows of dy: the kernel is
// bound by HBM when groups hold few rows (the decode regime).

#include <limits.h>

#include "gnf4_internal.h"

namespace gnf4 {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunkPitch = 33;  // floats per lane in the reduction buffer (conflict-free)

struct DgradKArgs {
  const uint16_t* dy;   // [M, N] bf16
  const uint8_t* packed;
  const void* absmax;   // fp32, or bf16 bits
  const int32_t* sizes;
  const int32_t* ids;
  uint16_t* dx;         // [M, K] bf16
  float* partial;       // [S, M, K] fp32 when S > 1
  int E, N, K, G, M, S, rows_per_split;
};

// (byte B of v) & mask in one VALU instruction (SDWA source byte select).
template <int B>
__device__ __forceinline__ uint32_t byte_and(uint32_t v, uint32_t mask) {
  uint32_t r;
  asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_%3 src1_sel:DWORD"
      : "=v"(r)
      : "v"(v), "s"(mask), "n"(B));
  return r;
}

__device__ __forceinline__ float lut_at(const float* lut16, uint32_t byte_off) {
  return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lut16) + byte_off);
}

// The group holding row j (0 <= j < M) when its expert id lies in [0, E):
// the group g with row(g) <= j < row(g) + size(g), sizes clamped to [0, M]
// and summed in group order as find_group does.  False when row j belongs to
// no group (past the sum of the sizes) or to one with an invalid expert id.
// Call with the whole wavefront active; every lane gets the same result.
// A wavefront's partial sums fit an int (M < 2^25); the running row count is
// 64-bit, so sizes summing far past M cannot wrap it.
__device__ __forceinline__ bool find_row_group(const int32_t* sizes, const int32_t* ids, int G,
                                               int E, int M, int j, GroupRef& out) {
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  long long rows = 0;
  for (int c0 = 0; c0 < G; c0 += 4 * kWave) {
    int sv[4], ev[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = c0 + q * kWave + lane;
      sv[q] = i < G ? min(max(sizes[i], 0), M) : 0;
      ev[q] = i < G ? ids[i] : -1;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int incl = wave_incl_scan(sv[q]);
      // the lane whose rows [end - size, end) hold j; the non-empty groups'
      // ranges tile the rows, so exactly one lane hits when j is in this batch
      const long long end = rows + incl;
      const uint64_t m = __builtin_amdgcn_ballot_w64(sv[q] > 0 && end - sv[q] <= j && j < end);
      if (m) {
        const int src = __builtin_ctzll(m);
        const int ex = __builtin_amdgcn_readlane(ev[q], src);
        if (ex < 0 || ex >= E) return false;
        const int sz = __builtin_amdgcn_readlane(sv[q], src);
        out.g = c0 + q * kWave + src;
        out.size = sz;
        out.expert = ex;
        out.row = (int)(rows + __builtin_amdgcn_readlane(incl, src) - sz);
        return true;
      }
      rows += __builtin_amdgcn_readlane(incl, 63);
    }
    if (rows > j) return false;
  }
  return false;
}

// L lanes (a team) cover L consecutive chunks of a weight row; the 64 / L
// teams of a wavefront take different weight rows.
// kNB weight rows in flight per team and batch.
template <int L, int R, int kNB, typename AbsT>
__global__ __launch_bounds__(kThreads) void dgrad_kernel(DgradKArgs a) {
  constexpr int RPW = kWave / L;  // teams per wavefront
  __shared__ float s_lut[32];  // level q at index 2q (8-byte stride)
  __shared__ float s_red[kWaves * kWave * kChunkPitch];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int team = lane / L, tl = lane % L;
  // R == 1: one workgroup slot per row, so the rows of a group run side by
  // side instead of one pass after another; otherwise one slot per group.
  GroupRef gr;
  int r_begin, r_end;
  if constexpr (R == 1) {
    if (!find_row_group(a.sizes, a.ids, a.G, a.E, a.M, blockIdx.y, gr)) return;
    r_begin = blockIdx.y;
    r_end = r_begin + 1;
  } else {
    if (!find_group(a.sizes, a.ids, a.G, a.E, a.M, 1, INT_MAX, blockIdx.y, gr)) return;
    r_begin = gr.row;
    r_end = min(r_begin + gr.size, a.M);
  }
  if (lane < 16) s_lut[2 * lane] = nf4_level(lane);
  const int N = a.N, K = a.K;
  const int cpr = K / 32;                     // 16-byte chunks per weight row
  const int c = blockIdx.x * L + tl;          // this lane's chunk
  const bool c_ok = c < cpr;
  const int cc = c_ok ? c : 0;
  const int bpr = K / kBlock;
  const size_t row_bytes = (size_t)K / 2;
  const uint8_t* wexp = a.packed + (size_t)gr.expert * N * row_bytes;
  const AbsT* aexp = static_cast<const AbsT*>(a.absmax) + (size_t)gr.expert * N * bpr;
  const int s = blockIdx.z;
  const int n_begin = s * a.rows_per_split;
  const int n_end = min(n_begin + a.rows_per_split, N);

  for (int r0 = r_begin; r0 < r_end; r0 += R) {
    float acc[R][32];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < 32; ++j) acc[r][j] = 0.0f;
    // this lane's rows: n_begin + (wave * RPW + team) + kWaves * RPW * i
    for (int n0 = n_begin + wave * RPW; n0 < n_end; n0 += kWaves * RPW * kNB) {
      // Every load is issued, from a clamped (existing) row, chunk and dy row,
      // and what does not exist is zeroed where it is used: loads in
      // branches would make the compiler wait for all of them before the
      // first row's terms.
      uint4 wq[kNB];
      float av[kNB];
      float dv[kNB][R];
      bool live[kNB];
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        const int n = n0 + team + kWaves * RPW * b;
        const bool ok = n < n_end;
        const int nn = ok ? n : n_begin;
        live[b] = ok && c_ok;
        wq[b] = *reinterpret_cast<const uint4*>(wexp + (size_t)nn * row_bytes + 16 * (size_t)cc);
        av[b] = absmax_at(aexp, (size_t)nn * bpr + (cc >> 1));
#pragma unroll
        for (int r = 0; r < R; ++r)
          dv[b][r] = bf16_to_f32(a.dy[(size_t)min(r0 + r, r_end - 1) * N + nn]);
      }
      // The empty asms pin each loaded value's first use to its row's terms,
      // so row b waits only for its own loads.
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        float ab = av[b];
        asm volatile("" : "+v"(ab));
        float sc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float db = dv[b][r];
          asm volatile("" : "+v"(db));
          sc[r] = (live[b] && r0 + r < r_end) ? db * ab : 0.0f;
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t d = w == 0 ? wq[b].x : w == 1 ? wq[b].y : w == 2 ? wq[b].z : wq[b].w;
          asm volatile("" : "+v"(d));
          // LUT byte offsets 8 * code: after a right shift by 1, bits 3..6 of
          // byte q hold its high code; after a left shift by 3, its low code
          const uint32_t dh = d >> 1, dl = d << 3;
          const uint32_t oh[4] = {byte_and<0>(dh, 0x78u), byte_and<1>(dh, 0x78u),
                                  byte_and<2>(dh, 0x78u), byte_and<3>(dh, 0x78u)};
          const uint32_t ol[4] = {byte_and<0>(dl, 0x78u), byte_and<1>(dl, 0x78u),
                                  byte_and<2>(dl, 0x78u), byte_and<3>(dl, 0x78u)};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float vh = lut_at(s_lut, oh[q]);
            const float vl = lut_at(s_lut, ol[q]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
              acc[r][8 * w + 2 * q] = fmaf(sc[r], vh, acc[r][8 * w + 2 * q]);
              acc[r][8 * w + 2 * q + 1] = fmaf(sc[r], vl, acc[r][8 * w + 2 * q + 1]);
            }
          }
        }
      }
    }
    // team partials meet in LDS; thread t sums outputs t, t + 512, ... of
    // the tile's L * 32 over the wavefronts in order, and over the teams in
    // order within each
#pragma unroll
    for (int r = 0; r < R; ++r) {
      __syncthreads();  // the previous row's readers are done
      float* mine = s_red + (wave * kWave + lane) * kChunkPitch;
#pragma unroll
      for (int j = 0; j < 32; ++j) mine[j] = acc[r][j];
      __syncthreads();
      const int row = r0 + r;
      if (row >= r_end) continue;
#pragma unroll
      for (int q = 0; q < (L * 32 + kThreads - 1) / kThreads; ++q) {
        const int p = threadIdx.x + kThreads * q;  // position in the tile: chunk p / 32, k p % 32
        if (p >= L * 32) continue;
        const int pl = p >> 5, pj = p & 31;
        const int k = 32 * (blockIdx.x * L + pl) + pj;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
#pragma unroll
          for (int t = 0; t < RPW; ++t) sum += s_red[(w * kWave + t * L + pl) * kChunkPitch + pj];
        if (k >= K) continue;
        if (a.S == 1)
          a.dx[(size_t)row * K + k] = f32_to_bf16(sum);
        else
          a.partial[((size_t)s * a.M + row) * K + k] = sum;
      }
    }
  }
}

// Sum the S split partials of every row a group covers, in split order -> bf16.
__global__ __launch_bounds__(256) void dgrad_reduce_kernel(DgradKArgs a) {
  GroupRef gr;
  if (!find_group(a.sizes, a.ids, a.G, a.E, a.M, 1, INT_MAX, blockIdx.y, gr)) return;
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= a.K) return;
  const int r_end = min(gr.row + gr.size, a.M);
  const size_t plane = (size_t)a.M * a.K;
  for (int r = gr.row; r < r_end; ++r) {
    const float sum = sum_splits(a.partial + (size_t)r * a.K + k, plane, a.S);
    a.dx[(size_t)r * a.K + k] = f32_to_bf16(sum);
  }
}

}  // namespace

// Team width for rows of cpr chunks: the widest of 64/32/16/8 lanes whose
// tiles leave less than half of the chunk slots idle, else the one with the
// least idle share.  (Narrower teams mean more tiles and more rows per
// workgroup pass: GPT-OSS's 90 chunks ran faster on two 64-lane tiles, 30%
// idle, than on three 32-lane ones; OLMoE's 32 chunks faster on 32 lanes.)
static int dgrad_lanes(int64_t cpr) {
  const int cands[4] = {64, 32, 16, 8};
  int best = 64;
  double best_waste = 2.0;
  for (int L : cands) {
    const int64_t tiles = (cpr + L - 1) / L;
    const double waste = (double)(tiles * L - cpr) / (double)(tiles * L);
    if (waste < 0.5) return L;
    if (waste < best_waste) {
      best_waste = waste;
      best = L;
    }
  }
  return best;
}

// Launch rule (host-known sizes only): R from the rows per group; the team
// width L from K; N split so the grid holds about two wavefronts per SIMD,
// each split at least one batch of rows per team.  Batches are 8 rows per
// team, or 4 at one row of dy when 8 would allow at most half the splits
// wanted (OLMoE and Qwen3 down: 16 splits, 128 workgroups, half the device;
// with 4, 32 and 6-7% faster; Qwen3 gate_up, 24 of 32, ran 4% slower on 4).
DgradPlan plan_dgrad(int64_t M, int64_t N, int64_t K, int64_t G, int num_cus) {
  DgradPlan p;
  const int64_t g_eff = G < M ? G : M;
  const double rows_per_group = (double)M / (double)(g_eff > 0 ? g_eff : 1);
  p.R = rows_per_group <= 1.5 ? 1 : (rows_per_group <= 3.0 ? 2 : 4);
  const int64_t cpr = K / 32;
  p.L = dgrad_lanes(cpr);
  p.k_tiles = (int)((cpr + p.L - 1) / p.L);
  const int64_t target_waves = 8LL * num_cus;
  const int64_t per_split = (g_eff > 0 ? g_eff : 1) * p.k_tiles * kWaves;
  int64_t S = (target_waves + per_split - 1) / per_split;
  auto max_splits = [&](int nb) {
    const int64_t rows_per_batch = (int64_t)kWaves * (kWave / p.L) * nb;
    return (N + rows_per_batch - 1) / rows_per_batch;
  };
  p.NB = (p.R == 1 && 2 * max_splits(8) <= S) ? 4 : 8;
  const int64_t max_s = max_splits(p.NB);
  if (S > max_s) S = max_s;
  if (S < 1) S = 1;
  p.rows_per_split = (int)((N + S - 1) / S);
  p.S = (int)((N + p.rows_per_split - 1) / p.rows_per_split);
  return p;
}

template <int L, typename AbsT>
static void launch_dgrad_LA(const DgradKArgs& a, int R, int NB, dim3 grid, hipStream_t stream) {
  if (R == 1 && NB == 4)
    hipLaunchKernelGGL((dgrad_kernel<L, 1, 4, AbsT>), grid, dim3(kThreads), 0, stream, a);
  else if (R == 1)
    hipLaunchKernelGGL((dgrad_kernel<L, 1, 8, AbsT>), grid, dim3(kThreads), 0, stream, a);
  else if (R == 2)
    hipLaunchKernelGGL((dgrad_kernel<L, 2, 8, AbsT>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((dgrad_kernel<L, 4, 8, AbsT>), grid, dim3(kThreads), 0, stream, a);
}

template <int L>
static void launch_dgrad_L(const DgradKArgs& a, bool abs_bf16, int R, int NB, dim3 grid,
                           hipStream_t stream) {
  if (abs_bf16)
    launch_dgrad_LA<L, uint16_t>(a, R, NB, grid, stream);
  else
    launch_dgrad_LA<L, float>(a, R, NB, grid, stream);
}

size_t dgrad_workspace_bytes(const DgradPlan& p, int64_t M, int64_t K) {
  return p.S > 1 ? (size_t)p.S * (size_t)M * (size_t)K * sizeof(float) : 0;
}

hipError_t launch_dgrad(const DgradArgs& g, const DgradPlan& p, hipStream_t stream) {
  DgradKArgs a;
  a.dy = g.dy;
  a.packed = g.packed;
  a.absmax = g.absmax;
  a.sizes = g.sizes;
  a.ids = g.ids;
  a.dx = g.dx;
  a.partial = g.partial;
  a.E = g.E;
  a.N = g.N;
  a.K = g.K;
  a.G = g.G;
  a.M = g.M;
  a.S = p.S;
  a.rows_per_split = p.rows_per_split;
  const unsigned slots = (unsigned)(p.R == 1 ? g.M : group_slots(g.G, g.M, 1));
  if (slots == 0) return hipSuccess;
  const dim3 grid((unsigned)p.k_tiles, slots, (unsigned)p.S);
  switch (p.L) {
    case 64: launch_dgrad_L<64>(a, g.abs_bf16, p.R, p.NB, grid, stream); break;
    case 32: launch_dgrad_L<32>(a, g.abs_bf16, p.R, p.NB, grid, stream); break;
    case 16: launch_dgrad_L<16>(a, g.abs_bf16, p.R, p.NB, grid, stream); break;
    case 8: launch_dgrad_L<8>(a, g.abs_bf16, p.R, p.NB, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  const dim3 rgrid((unsigned)((g.K + 255) / 256), slots);
  hipLaunchKernelGGL(dgrad_reduce_kernel, rgrid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gnf4
