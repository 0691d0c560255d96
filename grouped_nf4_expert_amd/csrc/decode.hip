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
// used once, so the kernel is built to have all weight bytes in flight as
// early as possible and to spend few VALU instructions per code:
//  * a workgroup (4 wavefronts) owns one group (expert) and a tile of weight
//    rows; within a wavefront, a "team" of L lanes (L = 8..64, chosen from K
//    so rows are covered with little raggedness) reads consecutive 16-byte
//    chunks (32 codes) of one weight row, NU rows per lane;
//  * loads are issued in the order they are consumed (group metadata, then
//    activations, then weight rows), since vector loads complete in order;
//    when a lane walks several chunks, the next one is prefetched while the
//    current one is decoded;
//  * R activation rows (a compile-time choice from the host-known rows per
//    group) are converted to fp32 once per chunk so one decoded code feeds R
//    multiply-adds; larger groups loop over chunks of R rows;
//  * a code's level is read from a 16-entry fp32 table in LDS at an 8-byte
//    stride (level q at bank 2q: conflict-free for any mix of codes whether
//    the LDS has 32 or 64 banks, and the byte offset is one masked byte of a
//    shifted packed dword), multiplied and accumulated in fp32; the block
//    absmax is applied once per 32 codes;
//  * team partial sums are combined with a fixed butterfly and either
//    rounded to bf16 or, when K is split across workgroups to fill the
//    machine, written as fp32 partials that a second kernel sums in split
//    order (deterministic).

#include <limits.h>
#include <stdlib.h>

#include "gnf4_internal.h"

namespace gnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

struct DecodeKArgs {
  GemmArgs g;
  int S, cps, cpr, n_tiles, rows_per_block;
};

__device__ __forceinline__ void unpack_bf16x8(const uint4 v, float* out) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(d[j] << 16);
    out[2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
  }
}

// (byte B of v) & mask in one VALU instruction (SDWA source byte select).
template <int B>
__device__ __forceinline__ uint32_t byte_and(uint32_t v, uint32_t mask) {
  uint32_t r;
  asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_%3 src1_sel:DWORD"
      : "=v"(r)
      : "v"(v), "s"(mask), "n"(B));
  return r;
}

// Sum over each team of L consecutive lanes on the DPP network, in a fixed
// order; the result is valid in the team's last lane.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}

template <int L>
__device__ __forceinline__ float team_sum(float v) {
  v += dpp_f32<0xB1, 0xF>(v);                   // pairs
  v += dpp_f32<0x4E, 0xF>(v);                   // quads
  v += dpp_f32<0x141, 0xF>(v);                  // half rows (8)
  if (L >= 16) v += dpp_f32<0x140, 0xF>(v);     // rows (16)
  if (L >= 32) v += dpp_f32<0x142, 0xA>(v);     // rows 0+1 and 2+3
  if (L >= 64) v += dpp_f32<0x143, 0xC>(v);     // all four rows
  return v;
}

__device__ __forceinline__ float lut_at(const float* lut16, uint32_t byte_off) {
  return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lut16) + byte_off);
}

template <int NU>
__device__ __forceinline__ void load_weights(const uint8_t* wexp, const float* aexp,
                                             size_t row_bytes, int bpr, int N, int n_base, int c,
                                             bool valid, uint4 (&wq)[NU], float (&av)[NU]) {
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    const int n = n_base + j;
    if (valid && n < N) {
      wq[j] = *reinterpret_cast<const uint4*>(wexp + (size_t)n * row_bytes + 16 * (size_t)c);
      av[j] = aexp[(size_t)n * bpr + (c >> 1)];
    } else {
      wq[j] = make_uint4(0, 0, 0, 0);
      av[j] = 0.0f;
    }
  }
}

template <int R>
__device__ __forceinline__ void load_x(const uint16_t* x, int K, const int (&xrow)[R], int c,
                                       bool valid, uint4 (&xv)[R][4]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (valid && xrow[r] >= 0) {
      const uint4* xp = reinterpret_cast<const uint4*>(x + (size_t)xrow[r] * K + 32 * (size_t)c);
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[r][q] = xp[q];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[r][q] = make_uint4(0, 0, 0, 0);
    }
  }
}

// One group, a tile of weight rows, activation rows in chunks of R.
//
// Vector-memory loads complete in issue order, so the order of issue is the
// schedule: (1) the group metadata (sizes of the preceding groups, and the
// slot table when the gather is fused) from L2, (2) the activations of the
// first chunk, (3) its NU weight rows, then per chunk the next chunk's
// activations and weights before the current chunk is decoded -- each row's
// arithmetic waits only for its own weight bytes.
template <int L, int NU, int R, bool MULTI>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeKArgs a) {
  // 16 levels at an 8-byte stride, at a fixed LDS address so a code's byte
  // offset is the whole address (no per-read base add)
  __shared__ float s_lut[32];
  constexpr int RPW = kWave / L;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const bool gather = a.g.slots != nullptr;
  const bool slots_in_lanes = gather && a.g.M <= kWave;
  // (1) metadata: the slot table (issued first, independent of the group)
  // and the group this workgroup serves
  int my_slot = 0;
  if (slots_in_lanes && lane < a.g.M) my_slot = a.g.slots[lane];
  GroupRef gr;
  if (!find_group(a.g.sizes, a.g.ids, a.g.G, a.g.E, a.g.M, 1, a.g.rows_max_decode, blockIdx.y, gr))
    return;
  const int tile = blockIdx.x % a.n_tiles;
  const int s = blockIdx.x / a.n_tiles;
  const int team = lane / L, tl = lane % L;
  const int N = a.g.N, K = a.g.K;
  const int n_base = tile * a.rows_per_block + wave * (RPW * NU) + team * NU;
  const size_t row_bytes = (size_t)K / 2;
  const int bpr = K / kBlock;
  const uint8_t* wexp = a.g.packed + (size_t)gr.expert * N * row_bytes;
  const float* aexp = a.g.absmax + (size_t)gr.expert * N * bpr;
  const int c_begin = s * a.cps;
  const int c_end = min(c_begin + a.cps, a.cpr);
  const int c_first = c_begin + tl;
  // every wavefront writes the same values before its own reads; LDS
  // operations of one wavefront complete in order, so no barrier is needed
  const float* lut = s_lut;
  if (lane < 16) s_lut[2 * lane] = nf4_level(lane);
  const int r_begin = gr.row;
  const int r_end = min(r_begin + gr.size, a.g.M);
  __builtin_amdgcn_wave_barrier();

  for (int r0 = r_begin; r0 < r_end; r0 += R) {
    // source activation row of each of the R output rows (-1: skip the row)
    int xrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = r0 + r;
      xrow[r] = row < r_end ? row : -1;
      if (gather && row < r_end) {
        const int slot = slots_in_lanes ? __builtin_amdgcn_readlane(my_slot, row) : a.g.slots[row];
        xrow[r] = (slot >= 0 && slot < a.g.T * a.g.slot_div) ? slot / a.g.slot_div : -1;
      }
    }
    // (2) + (3): first chunk's activations, then its weights
    uint4 xv[R][4];
    load_x<R>(a.g.x, K, xrow, c_first, c_first < c_end, xv);
    uint4 wq[NU];
    float av[NU];
    load_weights<NU>(wexp, aexp, row_bytes, bpr, N, n_base, c_first, c_first < c_end, wq, av);

    float acc[NU][R];
#pragma unroll
    for (int j = 0; j < NU; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[j][r] = 0.0f;

    // MULTI: a lane sees more than one chunk per row, so the next chunk is
    // prefetched; otherwise the loop body runs at most once and carries no
    // prefetch registers.
    for (int c = c_first; c < c_end; c += L) {
      const bool more = MULTI && c + L < c_end;
      uint4 xn[R][4];
      uint4 wn[NU];
      float an[NU];
      if (MULTI) {
        load_x<R>(a.g.x, K, xrow, c + L, more, xn);
        load_weights<NU>(wexp, aexp, row_bytes, bpr, N, n_base, c + L, more, wn, an);
      }
      float xs[R][32];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) unpack_bf16x8(xv[r][q], &xs[r][8 * q]);
#pragma unroll
      for (int j = 0; j < NU; ++j) {
        float pr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) pr[r] = 0.0f;
        const uint32_t d[4] = {wq[j].x, wq[j].y, wq[j].z, wq[j].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // LUT byte offsets 8 * code: after a right shift by 1, bits 3..6 of
          // byte b hold its high code; after a left shift by 3, its low code.
          const uint32_t dh = d[w] >> 1;
          const uint32_t dl = d[w] << 3;
          uint32_t oh[4], ol[4];
          oh[0] = byte_and<0>(dh, 0x78u);
          oh[1] = byte_and<1>(dh, 0x78u);
          oh[2] = byte_and<2>(dh, 0x78u);
          oh[3] = byte_and<3>(dh, 0x78u);
          ol[0] = byte_and<0>(dl, 0x78u);
          ol[1] = byte_and<1>(dl, 0x78u);
          ol[2] = byte_and<2>(dl, 0x78u);
          ol[3] = byte_and<3>(dl, 0x78u);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const float vh = lut_at(lut, oh[b]);
            const float vl = lut_at(lut, ol[b]);
            const int k = 8 * w + 2 * b;
#pragma unroll
            for (int r = 0; r < R; ++r) {
              pr[r] = fmaf(xs[r][k], vh, pr[r]);
              pr[r] = fmaf(xs[r][k + 1], vl, pr[r]);
            }
          }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[j][r] = fmaf(av[j], pr[r], acc[j][r]);
      }
      if (!MULTI) break;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[r][q] = xn[r][q];
#pragma unroll
      for (int j = 0; j < NU; ++j) {
        wq[j] = wn[j];
        av[j] = an[j];
      }
    }

#pragma unroll
    for (int j = 0; j < NU; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[j][r] = team_sum<L>(acc[j][r]);

    // the team's last lane holds the sums
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const int n = n_base + j;
      if (tl != L - 1 || n >= N) continue;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = r0 + r;
        if (xrow[r] < 0) continue;
        if (a.S == 1)
          a.g.y[(size_t)row * N + n] = f32_to_bf16(acc[j][r]);
        else
          a.g.partial[((size_t)s * a.g.M + row) * N + n] = acc[j][r];
      }
    }
  }
}

// Sum the S split partials of every decode-path row in split order -> bf16.
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(DecodeKArgs a) {
  GroupRef gr;
  if (!find_group(a.g.sizes, a.g.ids, a.g.G, a.g.E, a.g.M, 1, a.g.rows_max_decode, blockIdx.y, gr))
    return;
  const int r_begin = gr.row;
  const int r_end = min(r_begin + gr.size, a.g.M);
  const int n = blockIdx.x * kThreads + threadIdx.x;
  if (n >= a.g.N) return;
  const size_t plane = (size_t)a.g.M * a.g.N;
  for (int r = r_begin; r < r_end; ++r) {
    if (a.g.slots) {  // rows the fused gather skipped have no partials
      const int slot = a.g.slots[r];
      if (slot < 0 || slot >= a.g.T * a.g.slot_div) continue;
    }
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

template <int L, int NU, bool MULTI>
hipError_t launch_LNM(const DecodeKArgs& a, const DecodePlan& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.n_tiles * p.S), (unsigned)group_slots(a.g.G, a.g.M, 1));
  switch (p.R) {
    case 4: hipLaunchKernelGGL((decode_kernel<L, NU, 4, MULTI>), grid, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<L, NU, 2, MULTI>), grid, dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((decode_kernel<L, NU, 1, MULTI>), grid, dim3(kThreads), 0, stream, a); break;
  }
  return hipGetLastError();
}

template <int L, int NU>
hipError_t launch_LN(const DecodeKArgs& a, const DecodePlan& p, hipStream_t stream) {
  return p.cps > L ? launch_LNM<L, NU, true>(a, p, stream) : launch_LNM<L, NU, false>(a, p, stream);
}

template <int L>
hipError_t launch_L(const DecodeKArgs& a, const DecodePlan& p, hipStream_t stream) {
  switch (p.NU) {
#ifdef GNF4_TUNING
    case 8: return launch_LN<L, 8>(a, p, stream);
#endif
    case 4: return launch_LN<L, 4>(a, p, stream);
    case 2: return launch_LN<L, 2>(a, p, stream);
    default: return launch_LN<L, 1>(a, p, stream);
  }
}

}  // namespace

static DecodePlan plan_decode_rule(int64_t M, int64_t N, int64_t K, int64_t G, int split_k,
                                   int num_cus) {
  const int cpr = (int)(K / 32);
  const int64_t g_eff = G < M ? G : M;
  const int64_t target = 2LL * num_cus;  // workgroups that keep every CU busy
  // rows per group the host can infer: M rows over at most min(G, M) groups
  const double rows_per_group = (double)M / (double)(g_eff > 0 ? g_eff : 1);
  const int R = rows_per_group <= 1.5 ? 1 : (rows_per_group <= 3.0 ? 2 : 4);
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
    // Two weight rows per lane; four when two would launch more wavefronts
    // than the dispatcher places in about a microsecond (8192); one only to
    // fill a starved machine.
    const int64_t waves_nu2 = g_eff * S * ((N + (kWave / L) * 2 - 1) / ((kWave / L) * 2));
    const int nus[3] = {waves_nu2 > 8192 ? 4 : 2, waves_nu2 > 8192 ? 2 : 1, 1};
    for (int ni = 0; ni < 3; ++ni) {
      DecodePlan p;
      p.L = L;
      p.NU = nus[ni];
      p.R = R;
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

DecodePlan plan_decode(int64_t M, int64_t N, int64_t K, int64_t G, int split_k, int num_cus) {
  DecodePlan p = plan_decode_rule(M, N, K, G, split_k, num_cus);
#ifdef GNF4_TUNING  // experiment builds only: override the launch rule
  if (const char* v = getenv("GNF4_TUNE_NU")) {
    p.NU = atoi(v);
    p.rows_per_block = kWaves * (kWave / p.L) * p.NU;
    p.n_tiles = (int)((N + p.rows_per_block - 1) / p.rows_per_block);
  }
#endif
  return p;
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
  const dim3 grid((unsigned)((g.N + kThreads - 1) / kThreads), (unsigned)group_slots(g.G, g.M, 1));
  hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gnf4
