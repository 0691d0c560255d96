// Decode path of the grouped NF4 GEMM: groups with few rows (batch-1 decode).
//
// Page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE
// expert stacks": opening section (one launch for all active experts, LUT
// decode to fp32 in registers, blockwise fp32 absmax (or bf16: page "How do
// I run a MoE whose experts do not fit in VRAM ...", "Supported scope", the
// bake's --absmax-dtype), fp32 accumulation, bf16
// epilogue); "Layout" (a decode GEMV path beside the M-tile path); "Status /
// roadmap" (split-K for starved grids with a per-split work floor; one
// universal launch rule rather than a per-shape table).
//
// At one row per expert every weight byte is used once, so the kernel must
// stream the weights at HBM speed while spending as few VALU instructions as
// possible on everything else (a wave64 VALU instruction occupies its SIMD
// for 4 cycles, so per-wavefront overhead quickly becomes the bound):
//  * a workgroup (4 wavefronts) owns one group (expert), one K split and a
//    tile of weight rows; within a wavefront a "team" of L lanes (L = 8..64,
//    chosen from K so rows are covered with little raggedness) reads
//    consecutive 16-byte chunks (32 codes) of a weight row;
//  * each lane owns NU weight rows and `steps` chunks of each; all of its
//    weight loads are issued at once, before anything waits, and consumed in
//    issue order (vector loads complete in order), so a wavefront decodes
//    its first rows while the rest are still arriving.  Few, fat wavefronts
//    keep the per-wavefront costs (group lookup, staging, reductions) small
//    next to the decode itself;
//  * the activation rows of the workgroup's K range are staged once into
//    LDS as fp32 (loads issued before the weight loads), so no wavefront
//    loads or converts them again;
//  * a code's level is read from a 16-entry fp32 table in LDS at an 8-byte
//    stride (level q at bank 2q: conflict-free for any mix of codes, and the
//    byte offset is one masked byte of a shifted packed dword) and
//    multiplied-added in fp32; the block absmax is applied once per 32 codes;
//  * team partial sums are combined with a fixed butterfly and either
//    rounded to bf16 or, when K is split across workgroups to fill the
//    machine, written as fp32 partials that a second kernel sums in split
//    order (deterministic).

#include <limits.h>
#include <stddef.h>

#include <type_traits>

#include "gnf4_internal.h"
#include "route_core.h"

namespace gnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// Staged activations per workgroup: R rows x (chunks + 1) slots of 128 bytes
// (32 fp32) at most, i.e. 40 KB.
constexpr int kXSlots = 320;
// 16-byte bf16 pieces per thread per staging round for a kernel whose lanes
// cover at most L * steps chunks of R rows (4 pieces per chunk and row, and
// R * (chunks + 1) <= kXSlots): one round stages them all, so no load loop
// sits between the weight loads and the decode.
constexpr int x_batch(int R, int L, int steps) {
  const int pieces = 4 * R * L * steps < 4 * kXSlots ? 4 * R * L * steps : 4 * kXSlots;
  return (pieces + kThreads - 1) / kThreads;
}
constexpr int kMaxLoads = 4;    // weight chunks in flight per lane (NU * steps)
constexpr int kMaxSteps = 4;

struct DecodeKArgs {
  // What every wavefront reads before its weight loads, first and packed
  // (80 bytes: with the 44 bytes of preloaded leading arguments, two 64-byte
  // lines of the argument segment); copies of fields of g.
  const uint16_t* x;
  const uint8_t* packed;
  const void* absmax;
  void* out;  // y (bf16 bits) when S == 1, else the fp32 split partials
  double inv_slot_div;  // 1 / slot_div, for the fused gather's row index
  int N, K, T, slot_div, rows_max_decode;
  int S, cps, cpr, rows_per_block;
  int16_t route_k;  // picks per token of the routed launch (ro.K)
  int16_t vec_out;  // S == 1, R == 1, N % NU == 0, y aligned: one NU-wide store per lane
  // the rest: the split-K reduce's arguments and the route/sort outputs,
  // which only workgroup (0, 0, 0) of the routed launch writes
  GemmArgs g;
  // Routing folded into the launch (one token, E <= 64): the router logits
  // [E] and the route/sort outputs that workgroup (0, 0, 0) writes.
  const float* route_logits;
  RouteOneOut ro;
};
static_assert(offsetof(DecodeKArgs, g) == 80, "the hot arguments fill 80 bytes at the front");

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

// The stack's scale type also names its format: fp32 or bf16 block absmax
// (NF4 codes, 64 per block), or uint8 E8M0 scales (MXFP4: E2M1 codes, one
// scale per 32 codes, i.e. per 16-byte chunk).
template <typename AbsT>
constexpr bool kMxfp4 = std::is_same_v<AbsT, uint8_t>;

// E8M0 scale byte -> 2^(s - 127) in fp32 (2^-127 is a subnormal); 0xFF is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s == 255u ? 0x7fc00000u : s == 0u ? 0x00400000u : s << 23);
}

// Both E2M1 codes of byte B of d as fp32: .x from the low nibble (the first
// element), .y from the high nibble.
template <int B>
__device__ __forceinline__ void e2m1_pair(uint32_t d, float& first, float& second) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, B);
  first = v.x;
  second = v.y;
}

// Every lane issues every load, from row 0 / chunk 0 of the expert where its
// own row or chunk does not exist; what it loads there is never used (a lane
// past the K range skips the decode, and rows past N are never stored).
// Loads in branches, or a zeroing of their registers, would make the
// compiler wait for all of them (it cannot count loads that may not have
// been issued) before the activations staged ahead of them and before the
// first row's decode.
template <int NU, typename AbsT>
__device__ __forceinline__ void load_weights(const uint8_t* wexp, const AbsT* aexp, int row_bytes,
                                             int bpr, int N, int n_base, int c, bool valid,
                                             uint4 (&wq)[NU], float (&av)[NU]) {
  // offsets inside one expert fit 31 bits (N * K/2 < 2^31 is a call limit)
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    const int n = n_base + j;
    const bool ok = valid && n < N;
    const uint32_t nn = ok ? (uint32_t)n : 0u;
    const uint32_t cc = ok ? (uint32_t)c : 0u;
    const uint4 q = *reinterpret_cast<const uint4*>(wexp + (nn * (uint32_t)row_bytes + 16u * cc));
    float v;
    if constexpr (kMxfp4<AbsT>)
      v = e8m0_to_f32(aexp[nn * (uint32_t)(2 * bpr) + cc]);  // one scale per chunk
    else
      v = absmax_at(aexp, nn * (uint32_t)bpr + (cc >> 1));
    wq[j] = q;
    av[j] = v;
  }
}

// Activations of R rows over the workgroup's chunks [c_begin, c_begin + ncs),
// staged in LDS as fp32.  Chunk c of row r is 32 values = eight 16-byte
// pieces; piece p sits at 16-byte slot (r * 8 + p) * P + c with P = ncs + 1
// (one pad slot per plane).  The lanes of a team read piece p of
// consecutive chunks, i.e. consecutive slots: conflict-free.  A thread moves
// up to XB 16-byte bf16 pieces (= 2 fp32 pieces each) per round; the first
// round's loads are issued before the weight loads and stored after.
template <int R, int XB>
struct XStage {
  int ncs, plane, c_begin, per_row;
  uint4 v[XB];

  __device__ __forceinline__ void init(int c_begin_, int ncs_) {
    c_begin = c_begin_;
    ncs = ncs_;
    plane = ncs_ + 1;
    per_row = ncs_ * 4;
  }
  __device__ __forceinline__ int row_of(int idx) const {
    int r = 0;
#pragma unroll
    for (int q = 1; q < R; ++q) r += idx >= q * per_row;
    return r;
  }
  __device__ __forceinline__ void load(const uint16_t* x, int K, const int (&xrow)[R], int base) {
#pragma unroll
    for (int u = 0; u < XB; ++u) {
      const int idx = base + (int)threadIdx.x + u * kThreads;
      v[u] = make_uint4(0, 0, 0, 0);
      if (idx < R * per_row) {
        const int r = row_of(idx);
        const int rem = idx - r * per_row;
        int src = -1;
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
          if (rr == r) src = xrow[rr];
        if (src >= 0)
          v[u] = *reinterpret_cast<const uint4*>(x + (size_t)src * K + 32 * (size_t)c_begin +
                                                 8 * rem);
      }
    }
  }
  __device__ __forceinline__ void store(float4* s_x, int base) const {
#pragma unroll
    for (int u = 0; u < XB; ++u) {
      const int idx = base + (int)threadIdx.x + u * kThreads;
      if (idx < R * per_row) {
        const int r = row_of(idx);
        const int rem = idx - r * per_row;
        const int c = rem >> 2, q = rem & 3;
        float f[8];
        unpack_bf16x8(v[u], f);
        float4* dst = s_x + (r * 8 + 2 * q) * plane + c;
        dst[0] = make_float4(f[0], f[1], f[2], f[3]);
        dst[plane] = make_float4(f[4], f[5], f[6], f[7]);
      }
    }
  }
  __device__ __forceinline__ void all(const uint16_t* x, int K, const int (&xrow)[R], float4* s_x) {
    for (int base = 0; base < R * per_row; base += XB * kThreads) {
      load(x, K, xrow, base);
      store(s_x, base);
    }
  }
};

// Workgroup barrier for LDS data only: the wavefront's LDS operations are
// complete, global loads may still be in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// q = n / d for 0 <= n < 2^31, 1 <= d < 2^31, from a double estimate.
__device__ __forceinline__ int div_slot(int n, int d, double inv_d) {
  int q = (int)((double)n * inv_d);
  if ((long long)(q + 1) * d <= n) ++q;
  if ((long long)q * d > n) --q;
  return q;
}

// Every kernel argument the decode kernel reads before its weight loads, in
// SGPRs at this point: the compiler would otherwise read each from the
// argument segment where first used, one dependent round trip at a time.
// Only what the kernel uses: each further line of the segment costs a read.
__device__ __forceinline__ void pin_args(const DecodeKArgs& a) {
  asm volatile("" ::"s"(a.x), "s"(a.packed), "s"(a.absmax), "s"(a.out), "s"(a.inv_slot_div),
               "s"(a.N), "s"(a.K), "s"(a.T), "s"(a.slot_div), "s"(a.rows_max_decode), "s"(a.S),
               "s"(a.cps), "s"(a.cpr), "s"(a.rows_per_block), "s"(a.route_k), "s"(a.vec_out)
               : "memory");
}

// The terms of one weight dword (8 codes, 4 bytes; a byte's high nibble is
// its first element) against its 8 activations of R rows, added to pr.
template <int R, typename AbsT>
__device__ __forceinline__ void dword_terms(uint32_t d, const float (&xw)[R][8], const float* lut,
                                            float (&pr)[R]) {
  float vh[4], vl[4];  // the two elements of each byte: vh the first, vl the second
  if constexpr (kMxfp4<AbsT>) {
    // E2M1 through the hardware convert (first element = low nibble)
    e2m1_pair<0>(d, vh[0], vl[0]);
    e2m1_pair<1>(d, vh[1], vl[1]);
    e2m1_pair<2>(d, vh[2], vl[2]);
    e2m1_pair<3>(d, vh[3], vl[3]);
  } else {
    // NF4 LUT byte offsets 8 * code: after a right shift by 1, bits 3..6 of
    // byte b hold its high code (the first element); after a left shift by
    // 3, its low code.
    const uint32_t dh = d >> 1;
    const uint32_t dl = d << 3;
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
      vh[b] = lut_at(lut, oh[b]);
      vl[b] = lut_at(lut, ol[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      pr[r] = fmaf(xw[r][2 * b], vh[b], pr[r]);
      pr[r] = fmaf(xw[r][2 * b + 1], vl[b], pr[r]);
    }
  }
}

// One token routed in the launch, in every wavefront: returns the expert of
// the j-th pick in expert order.  Entry s of lane l holds expert l + 64 s's
// key, as the route/sort kernels build it (rank_token): the logit's
// order-preserving key above the complemented expert id, so keys are
// distinct, larger is better and the lower id wins a tie.  The wavefront
// finds the K-th largest key bit by bit from the top (a radix select over
// ballot counts: the largest t with at least K keys >= t); the picks are the
// keys >= t, the same set rank_token's ranks < K give.  Only the bits that
// differ between keys are searched: the 32 of the logit's key, then the low
// 7 of the id part (ids below 128 share bits 7..31 of ~id).  `issued` runs
// once the logit loads are issued and returns K and j (kernel arguments it
// reads arrive while the loads are in flight).  With `write`, the wavefront
// also writes the route/sort outputs.
struct PickQuery {
  int k, j;
};
template <int EPL, typename Issued>
__device__ __forceinline__ int route_pick(const float* __restrict__ logits, int E, int lane,
                                          bool write, const RouteOneOut& ro, Issued&& issued) {
  float val[EPL];
  uint64_t key[EPL];
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    const int e = lane + kWave * s;
    val[s] = e < E ? logits[e] : 0.0f;
  }
  const PickQuery q = issued();
  const int kpick = q.k, j = q.j;
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    const int e = lane + kWave * s;
    key[s] = e < E ? (((uint64_t)float_key(val[s]) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e))
                   : 0ull;
  }
  uint64_t t = 0;
  auto try_bit = [&](int b) {
    const uint64_t cand = t | (1ull << b);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < EPL; ++s) cnt += __popcll(__builtin_amdgcn_ballot_w64(key[s] >= cand));
    if (cnt >= kpick) t = cand;
  };
#pragma unroll
  for (int b = 63; b >= 32; --b) try_bit(b);
  t |= 0xffffff80ull;
#pragma unroll
  for (int b = 6; b >= 0; --b) try_bit(b);
  uint64_t sel[EPL];
#pragma unroll
  for (int s = 0; s < EPL; ++s) sel[s] = __builtin_amdgcn_ballot_w64(key[s] >= t);
  // the j-th pick in expert order (entry 0 of every lane, then entry 1)
  int jj = j;
  int expert = 0;
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    uint64_t m = sel[s];
    const int c = __popcll(m);
    if (jj >= 0 && jj < c) {  // uniform
      for (int q = 0; q < jj; ++q) m &= m - 1;
      expert = kWave * s + __ffsll((unsigned long long)m) - 1;
    }
    jj -= c;
  }
  if (write) {
    // the route/sort outputs need each pick's rank: the picks above it
    int rank[EPL];
#pragma unroll
    for (int s = 0; s < EPL; ++s) rank[s] = 0;
#pragma unroll
    for (int s2 = 0; s2 < EPL; ++s2)
      for (uint64_t m = sel[s2]; m; m &= m - 1) {
        const uint64_t kj = readlane64(key[s2], __ffsll((unsigned long long)m) - 1);
#pragma unroll
        for (int s = 0; s < EPL; ++s) rank[s] += kj > key[s] ? 1 : 0;
      }
#pragma unroll
    for (int s = 0; s < EPL; ++s)
      if (!((sel[s] >> lane) & 1)) rank[s] = kpick;
    route_one_token_write<EPL>(ro, lane, val, rank);
  }
  return expert;
}

// One group, one K split, a tile of weight rows; activation rows in chunks
// of R (the weights stay in registers across chunks).
//
// Vector-memory loads complete in issue order, so the order of issue is the
// schedule: (1) the group metadata (group sizes and expert ids, and the slot
// table when the gather is fused), (2) the first row chunk's activations,
// (3) every weight chunk of the lane, step by step; the decode then consumes
// the weights in the same order.
// ROUTED = 0: groups from sizes/ids; 1 or 2: a single token routed in the
// launch, over up to 64 * ROUTED experts (ROUTED router entries per lane).
//
// The first loads (router logits, or group sizes / ids and the slot table)
// need only the leading scalar arguments, which the library builds with
// kernel-argument preloading: they arrive in SGPRs at wavefront launch, so
// those loads are issued before any read of the argument segment, and every
// other argument is read in one batch while they are in flight (pin_args)
// rather than a round trip at a time where first used.
template <int L, int NU, int R, int STEPS, typename AbsT, int ROUTED = 0>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const int32_t* __restrict__ k_sizes, const int32_t* __restrict__ k_ids,
    const int32_t* __restrict__ k_slots, const float* __restrict__ k_logits, int k_G, int k_M,
    int k_E, DecodeKArgs a) {
  // 16 levels at an 8-byte stride, at a fixed LDS address so a code's byte
  // offset is the whole address (no per-read base add)
  __shared__ float s_lut[32];
  extern __shared__ float4 s_x[];
  constexpr int RPW = kWave / L;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const bool gather = k_slots != nullptr;
  const bool slots_in_lanes = gather && k_M <= kWave;
  // (1) metadata: the slot table (issued first, independent of the group)
  // and the group this workgroup serves
  int my_slot = 0;
  GroupRef gr;
  if constexpr (ROUTED > 0) {
    // Up to 64 experts every wavefront routes for itself (no wait for a
    // neighbour); with two router entries per lane the ranking is twice the
    // work and wavefront 0 does it for the workgroup, the others reading its
    // answer from LDS (measured: faster for 128 experts, slower for 64).
    const int j = blockIdx.y;
    const bool write = blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && wave == 0;
    auto issued = [&]() {
      pin_args(a);
      return PickQuery{a.route_k, j};
    };
    if constexpr (ROUTED == 1) {
      gr.expert = route_pick<ROUTED>(k_logits, k_E, lane, write, a.ro, issued);
    } else {
      __shared__ int s_expert;
      if (wave == 0) {
        const int e = route_pick<ROUTED>(k_logits, k_E, lane, write, a.ro, issued);
        if (lane == 0) s_expert = e;
      } else {
        pin_args(a);
      }
      __syncthreads();
      gr.expert = s_expert;
    }
    gr.g = j;
    gr.size = 1;
    gr.row = j;
  } else {
    if (slots_in_lanes && lane < k_M) my_slot = k_slots[lane];
    GroupChunk first;
    load_group_chunk(k_sizes, k_ids, k_G, 0, first);
    pin_args(a);
    if (!find_group_from(k_sizes, k_ids, k_G, k_E, k_M, 1, a.rows_max_decode, blockIdx.y, first,
                         gr))
      return;
  }
  const int s = blockIdx.z;
  const int team = lane / L, tl = lane % L;
  const int N = a.N, K = a.K;
  const int n_base = blockIdx.x * a.rows_per_block + wave * (RPW * NU) + team * NU;
  const size_t row_bytes = (size_t)K / 2;
  const int bpr = K / kBlock;
  const uint8_t* wexp = a.packed + (size_t)gr.expert * N * row_bytes;
  const AbsT* aexp = static_cast<const AbsT*>(a.absmax) +
                    (size_t)gr.expert * N * (kMxfp4<AbsT> ? 2 * bpr : bpr);
  const int c_begin = s * a.cps;
  const int c_end = min(c_begin + a.cps, a.cpr);
  const int ncs = max(c_end - c_begin, 0);
  const int plane = ncs + 1;
  // every wavefront writes the same values before its own reads; LDS
  // operations of one wavefront complete in order, so no barrier is needed
  const float* lut = s_lut;
  if (lane < 16) s_lut[2 * lane] = nf4_level(lane);
  const int r_begin = gr.row;
  const int r_end = min(r_begin + gr.size, k_M);
  const int slot_lim = a.T * a.slot_div;

  // source activation row of each of the R rows of a chunk (-1: skip)
  int xrow[R];
  auto rows_of = [&](int r0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = r0 + r;
      xrow[r] = row < r_end ? row : -1;
      if constexpr (ROUTED > 0) {
        xrow[r] = row < r_end ? 0 : -1;  // every pick reads the one token
        continue;
      }
      if (gather && row < r_end) {
        const int slot = slots_in_lanes ? __builtin_amdgcn_readlane(my_slot, row) : k_slots[row];
        xrow[r] = (slot >= 0 && slot < slot_lim) ? div_slot(slot, a.slot_div, a.inv_slot_div) : -1;
      }
    }
  };

  // (2) + (3): the first chunk's activations, then every weight chunk
  rows_of(r_begin);
  XStage<R, x_batch(R, L, STEPS)> stage;
  stage.init(c_begin, ncs);
  stage.load(a.x, K, xrow, 0);
  uint4 wq[STEPS][NU];
  float av[STEPS][NU];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int c = c_begin + tl + st * L;
    load_weights<NU, AbsT>(wexp, aexp, (int)row_bytes, bpr, N, n_base, c, c < c_end, wq[st],
                           av[st]);
  }
  stage.store(s_x, 0);

  // One chunk of R activation rows against the lane's weights, after the
  // barrier that publishes the chunk's staged activations.
  auto chunk = [&](int r0) {
    float acc[NU][R];
#pragma unroll
    for (int j = 0; j < NU; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[j][r] = 0.0f;

#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int c = c_begin + tl + st * L;
      if (c >= c_end) continue;
      float pr[NU][R];
#pragma unroll
      for (int j = 0; j < NU; ++j)
#pragma unroll
        for (int r = 0; r < R; ++r) pr[j][r] = 0.0f;
      // the 8 activations of weight dword w of this chunk, R rows
      auto x_of = [&](int w, float (&xw)[R][8]) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float4* src = s_x + (r * 8 + 2 * w) * plane + (c - c_begin);
          const float4 lo = src[0], hi = src[plane];
          xw[r][0] = lo.x; xw[r][1] = lo.y; xw[r][2] = lo.z; xw[r][3] = lo.w;
          xw[r][4] = hi.x; xw[r][5] = hi.y; xw[r][6] = hi.z; xw[r][7] = hi.w;
        }
      };
      // The empty asm pins each dword's first use here: hoisted out of the
      // row-chunk loop, the decode of every row would wait for every load.
      auto dword_of = [&](int j, int w) -> uint32_t {
        uint32_t d = w == 0 ? wq[st][j].x : w == 1 ? wq[st][j].y : w == 2 ? wq[st][j].z : wq[st][j].w;
        asm volatile("" : "+v"(d));
        return d;
      };
      if constexpr (R == 1 && NU > 1) {
        // Row by row: row j's terms need only row j's load, so the decode
        // of the first rows runs while the later rows are still arriving.
        float xw[4][R][8];
#pragma unroll
        for (int w = 0; w < 4; ++w) x_of(w, xw[w]);
#pragma unroll
        for (int j = 0; j < NU; ++j)
#pragma unroll
          for (int w = 0; w < 4; ++w) dword_terms<R, AbsT>(dword_of(j, w), xw[w], lut, pr[j]);
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float xw[R][8];  // shared by the NU rows
          x_of(w, xw);
#pragma unroll
          for (int j = 0; j < NU; ++j) dword_terms<R, AbsT>(dword_of(j, w), xw, lut, pr[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NU; ++j)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[j][r] = fmaf(av[st][j], pr[j][r], acc[j][r]);
    }

#pragma unroll
    for (int j = 0; j < NU; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[j][r] = team_sum<L>(acc[j][r]);

    // the team's last lane holds the sums
    if constexpr (R == 1 && (NU == 2 || NU == 4)) {
      if (a.vec_out && tl == L - 1 && xrow[0] >= 0 && n_base < N) {
        // the lane's NU outputs are consecutive in row r0: one store
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        auto pk = [](float lo, float hi) {
          return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
        };
        uint16_t* dst = static_cast<uint16_t*>(a.out) + (size_t)r0 * N + n_base;
        if constexpr (NU == 4)
          *reinterpret_cast<uint2*>(dst) =
              make_uint2(pk(acc[0][0], acc[1][0]), pk(acc[2][0], acc[3][0]));
        else
          *reinterpret_cast<uint32_t*>(dst) = pk(acc[0][0], acc[1][0]);
        return;
      }
    }
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const int n = n_base + j;
      if (tl != L - 1 || n >= N) continue;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = r0 + r;
        if (xrow[r] < 0) continue;
        if (a.S == 1)
          static_cast<uint16_t*>(a.out)[(size_t)row * N + n] = f32_to_bf16(acc[j][r]);
        else
          static_cast<float*>(a.out)[((size_t)s * k_M + row) * N + n] = acc[j][r];
      }
    }
  };

  // The first chunk outside the loop: a loop around it, with the staging
  // loads of later chunks, would make the compiler wait for every weight
  // load before the first row's decode.
  lds_barrier();
  chunk(r_begin);
  for (int r0 = r_begin + R; r0 < r_end; r0 += R) {
    lds_barrier();  // every wavefront is done with the previous chunk
    rows_of(r0);
    stage.all(a.x, K, xrow, s_x);
    lds_barrier();
    chunk(r0);
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
    const float sum = sum_splits(a.g.partial + (size_t)r * a.g.N + n, plane, a.S);
    a.g.y[(size_t)r * a.g.N + n] = f32_to_bf16(sum);
  }
}

template <int L, int NU, int R, int STEPS, typename AbsT, int ROUTED = 0>
hipError_t launch_one(const DecodeKArgs& a, const DecodePlan& p, hipStream_t stream) {
  // one staging round must cover the split's activation rows
  if (p.L != L || p.steps != STEPS || p.R != R || p.cps > L * STEPS ||
      R * (p.cps + 1) > kXSlots)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)p.n_tiles, (unsigned)group_slots(a.g.G, a.g.M, 1), (unsigned)p.S);
  const size_t lds = (size_t)R * (size_t)(p.cps + 1) * 128;
  hipLaunchKernelGGL((decode_kernel<L, NU, R, STEPS, AbsT, ROUTED>), grid, dim3(kThreads), lds,
                     stream, a.g.sizes, a.g.ids, a.g.slots, a.route_logits, a.g.G, a.g.M,
                     ROUTED > 0 ? a.ro.E : a.g.E, a);
  return hipGetLastError();
}

// The routed launch: one activation row per group (R = 1); EPL router
// entries per lane (E <= 64 * EPL).
template <int L, typename AbsT, int EPL>
hipError_t launch_L_routed(const DecodeKArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (p.R != 1) return hipErrorInvalidValue;
  switch (p.steps * 16 + p.NU) {
    case 16 + 4: return launch_one<L, 4, 1, 1, AbsT, EPL>(a, p, stream);
    case 16 + 2: return launch_one<L, 2, 1, 1, AbsT, EPL>(a, p, stream);
    case 16 + 1: return launch_one<L, 1, 1, 1, AbsT, EPL>(a, p, stream);
    case 32 + 2: return launch_one<L, 2, 1, 2, AbsT, EPL>(a, p, stream);
    case 32 + 1: return launch_one<L, 1, 1, 2, AbsT, EPL>(a, p, stream);
    case 48 + 1: return launch_one<L, 1, 1, 3, AbsT, EPL>(a, p, stream);
    case 64 + 1: return launch_one<L, 1, 1, 4, AbsT, EPL>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename AbsT, int EPL>
hipError_t launch_routed_L(const DecodeKArgs& a, const DecodePlan& p, hipStream_t stream) {
  switch (p.L) {
    case 64: return launch_L_routed<64, AbsT, EPL>(a, p, stream);
    case 32: return launch_L_routed<32, AbsT, EPL>(a, p, stream);
    case 16: return launch_L_routed<16, AbsT, EPL>(a, p, stream);
    case 8: return launch_L_routed<8, AbsT, EPL>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

// rows per lane times activation rows at most kMaxLoads (accumulators)
template <int L, int NU, int STEPS, typename AbsT>
hipError_t launch_R(const DecodeKArgs& a, const DecodePlan& p, hipStream_t stream) {
  if constexpr (NU * 4 <= kMaxLoads)
    if (p.R == 4) return launch_one<L, NU, 4, STEPS, AbsT>(a, p, stream);
  if constexpr (NU * 2 <= kMaxLoads)
    if (p.R == 2) return launch_one<L, NU, 2, STEPS, AbsT>(a, p, stream);
  if (p.R == 1) return launch_one<L, NU, 1, STEPS, AbsT>(a, p, stream);
  return hipErrorInvalidValue;
}

// (NU, steps) pairs with NU * steps <= kMaxLoads
template <int L, typename AbsT>
hipError_t launch_L(const DecodeKArgs& a, const DecodePlan& p, hipStream_t stream) {
  switch (p.steps * 16 + p.NU) {
    case 16 + 4: return launch_R<L, 4, 1, AbsT>(a, p, stream);
    case 16 + 2: return launch_R<L, 2, 1, AbsT>(a, p, stream);
    case 16 + 1: return launch_R<L, 1, 1, AbsT>(a, p, stream);
    case 32 + 2: return launch_R<L, 2, 2, AbsT>(a, p, stream);
    case 32 + 1: return launch_R<L, 1, 2, AbsT>(a, p, stream);
    case 48 + 1: return launch_R<L, 1, 3, AbsT>(a, p, stream);
    case 64 + 1: return launch_R<L, 1, 4, AbsT>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

// Team width for a split of cps chunks: the widest of 64/32/16/8 lanes whose
// steps (at most kMaxSteps) leave at most 1/8 of the chunk slots idle, else
// the one with the least idle share; 0 if no width needs <= kMaxSteps steps.
int pick_lanes(int cps) {
  const int cands[4] = {64, 32, 16, 8};
  int best = 0;
  double best_waste = 2.0;
  for (int L : cands) {
    const int steps = (cps + L - 1) / L;
    if (steps > kMaxSteps) continue;
    const double waste = (double)(steps * L - cps) / (double)(steps * L);
    if (waste <= 0.125) return L;
    if (waste < best_waste) {
      best_waste = waste;
      best = L;
    }
  }
  return best;
}

// ---------------------------------------------------------------------------
// One token's MoE expert feed-forward in one launch (batch-1 decode):
// routing, gate_up = x . W1[e]^T for each pick, h = silu(gate) * up, and
// y = h . W2[e]^T, with no launch between the two projections.
//
// The grid holds K * gu_tiles gate_up workgroups, then K * dn_tiles down
// workgroups (pick-major in both).  A gate_up workgroup computes P rows of the
// gate half and the same P rows of the up half of its pick's W1 (2P weight
// rows), finishes h for those P columns and counts itself done for the pick
// (done(j)); the pick's last one raises its ready flags.  A down workgroup
// issues its weight loads as soon as it knows its expert, then waits for its
// pick's ready flag, reads h[j] and finishes.  Workgroups are dispatched in
// grid order, so every gate_up workgroup is running or done before any down
// workgroup starts waiting, and the gate_up workgroups wait on nothing: the
// waits end.  A wait is bounded all the same (kFfnSpinLimit polls); one that
// runs out sets the error word and goes on.  The last down workgroup of a
// pick to pass the wait clears the pick's words for the next call.
//
// h and the words are written and read with device-scope atomic accesses,
// which are performed where every XCD sees them, and a tile is counted only
// after its h stores are complete: the ordering needs no cache write-back or
// invalidation (those, one per workgroup, cost more than the launch saved).

struct FfnKArgs {
  // every wavefront reads these before its weight loads: 84 bytes
  const uint8_t* gu_packed;
  const void* gu_absmax;
  const uint8_t* dn_packed;
  const void* dn_absmax;
  uint16_t* h;      // [K, I] bf16 bits
  uint16_t* y;      // [K, H] bf16 bits
  int32_t* sync;    // the counters and flags below, one per 128-byte line
  int H, I, route_k;
  int gu_tiles, dn_tiles;
  int gu_rows, dn_rows;  // weight rows per workgroup
  RouteOneOut ro;   // written by wavefront 0 of workgroup 0
};

constexpr int kFfnSpinLimit = 1 << 22;
// Synchronisation words of the fused launch, each on a 128-byte line of its
// own (index in int32 units; K picks):
//   done(j)      gate_up workgroups of pick j finished
//   passed(j)    down workgroups of pick j past their wait
//   ready(j, x)  pick j's h complete, one flag per XCD x (its workgroups poll
//                only their own XCD's line)
//   error        set when a wait ran out
constexpr int kSyncLine = 32;
constexpr int kXcds = 8;
__host__ __device__ constexpr int sync_done(int j) { return j * kSyncLine; }
__host__ __device__ constexpr int sync_passed(int K, int j) { return (K + j) * kSyncLine; }
__host__ __device__ constexpr int sync_ready(int K, int j, int x) {
  return (2 * K + j * kXcds + x) * kSyncLine;
}
__host__ __device__ constexpr int sync_error(int K) { return (2 * K + K * kXcds) * kSyncLine; }

__device__ __forceinline__ int xcd_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return (int)(v & (kXcds - 1));
}

__device__ __forceinline__ void pin_ffn_args(const FfnKArgs& a) {
  asm volatile("" ::"s"(a.gu_packed), "s"(a.gu_absmax), "s"(a.dn_packed), "s"(a.dn_absmax),
               "s"(a.h), "s"(a.y), "s"(a.sync), "s"(a.H), "s"(a.I), "s"(a.route_k),
               "s"(a.gu_tiles), "s"(a.dn_tiles), "s"(a.gu_rows), "s"(a.dn_rows)
               : "memory");
}

__device__ __forceinline__ float ffn_silu(float g) { return g / (1.0f + expf(-g)); }

// The lane's NU weight rows (consecutive from n_base) against one activation
// row staged in LDS (XStage layout, plane = chunks + 1): team-summed results,
// valid in the team's last lane.
template <int L, int NU, int STEPS, typename AbsT>
__device__ __forceinline__ void ffn_rows(const float4* s_x, int plane, const float* lut, int tl,
                                         int cpr, const uint4 (&wq)[STEPS][NU],
                                         const float (&av)[STEPS][NU], float (&acc)[NU]) {
#pragma unroll
  for (int j = 0; j < NU; ++j) acc[j] = 0.0f;
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int c = tl + st * L;
    if (c >= cpr) continue;
    float pr[NU][1];
#pragma unroll
    for (int j = 0; j < NU; ++j) pr[j][0] = 0.0f;
    float xw[4][1][8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4* src = s_x + (2 * w) * plane + c;
      const float4 lo = src[0], hi = src[plane];
      xw[w][0][0] = lo.x; xw[w][0][1] = lo.y; xw[w][0][2] = lo.z; xw[w][0][3] = lo.w;
      xw[w][0][4] = hi.x; xw[w][0][5] = hi.y; xw[w][0][6] = hi.z; xw[w][0][7] = hi.w;
    }
#pragma unroll
    for (int j = 0; j < NU; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t d = w == 0 ? wq[st][j].x : w == 1 ? wq[st][j].y : w == 2 ? wq[st][j].z : wq[st][j].w;
        asm volatile("" : "+v"(d));  // decode row j as soon as its load is in
        dword_terms<1, AbsT>(d, xw[w], lut, pr[j]);
      }
#pragma unroll
    for (int j = 0; j < NU; ++j) acc[j] = fmaf(av[st][j], pr[j][0], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < NU; ++j) acc[j] = team_sum<L>(acc[j]);
}

// At most 80 VGPRs (six wavefronts per SIMD): six workgroups per CU, so the
// OLMoE-shaped launch (1,536 workgroups) and the Qwen3-shaped one (1,280)
// fit on the device at once.
template <int LG, int NUG, int STG, int LD, int NUD, int STD, typename AbsT, int EPL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6))) void ffn_kernel(const float* __restrict__ k_logits,
                                                       const uint16_t* __restrict__ k_x, int k_E,
                                                       FfnKArgs a) {
  __shared__ float s_lut[32];
  __shared__ float s_sum[kThreads];
  extern __shared__ float4 s_x[];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int wg = blockIdx.x;
  // (1) route (every wavefront; the arguments arrive while the logits load)
  bool gate_up = false;
  int j = 0, t = 0;
  auto place = [&]() {
    pin_ffn_args(a);
    const int n_gu = a.route_k * a.gu_tiles;
    gate_up = wg < n_gu;
    const int local = gate_up ? wg : wg - n_gu;
    const int tiles = gate_up ? a.gu_tiles : a.dn_tiles;
    j = local / tiles;
    t = local - j * tiles;
    return PickQuery{a.route_k, j};
  };
  // wavefront 0 routes for the workgroup; the others place themselves and
  // read its expert from LDS
  __shared__ int s_expert;
  if (wave == 0) {
    const int e = route_pick<EPL>(k_logits, k_E, lane, wg == 0, a.ro, place);
    if (lane == 0) s_expert = e;
  } else {
    place();
  }
  __syncthreads();
  const int expert = s_expert;
  if (lane < 16) s_lut[2 * lane] = nf4_level(lane);
  const float* lut = s_lut;
  const int H = a.H, I = a.I, K = a.route_k;

  if (gate_up) {
    // (2) gate_up: weight rows {t P + r} of the gate half and {I + t P + r} of
    // the up half, r < P; K = H
    constexpr int RPW = kWave / LG;
    const int team = lane / LG, tl = lane % LG;
    const int P = a.gu_rows / 2;
    const int r0 = wave * (RPW * NUG) + team * NUG;  // a lane's rows stay in one half
    const int n_base = r0 < P ? t * P + r0 : I + t * P + (r0 - P);
    const int cpr = H / 32, bpr = H / kBlock;
    const uint8_t* wexp = a.gu_packed + (size_t)expert * (2 * I) * (H / 2);
    const AbsT* aexp = static_cast<const AbsT*>(a.gu_absmax) + (size_t)expert * (2 * I) * bpr;
    XStage<1, x_batch(1, LG, STG)> stage;
    stage.init(0, cpr);
    const int xrow[1] = {0};
    stage.load(k_x, H, xrow, 0);
    uint4 wq[STG][NUG];
    float av[STG][NUG];
#pragma unroll
    for (int st = 0; st < STG; ++st) {
      const int c = tl + st * LG;
      load_weights<NUG, AbsT>(wexp, aexp, H / 2, bpr, 2 * I, n_base, c, c < cpr, wq[st],
                              av[st]);
    }
    stage.store(s_x, 0);
    lds_barrier();
    float acc[NUG];
    ffn_rows<LG, NUG, STG, AbsT>(s_x, stage.plane, lut, tl, cpr, wq, av, acc);
    if (tl == LG - 1) {
#pragma unroll
      for (int jj = 0; jj < NUG; ++jj) s_sum[r0 + jj] = acc[jj];
    }
    __syncthreads();
    // h for the P columns, two per 32-bit word, stored at device scope (the
    // down workgroups read them from other XCDs)
    if ((int)threadIdx.x < P / 2) {
      const int i0 = 2 * threadIdx.x;
      const uint32_t lo = f32_to_bf16(ffn_silu(s_sum[i0]) * s_sum[P + i0]);
      const uint32_t hi = f32_to_bf16(ffn_silu(s_sum[i0 + 1]) * s_sum[P + i0 + 1]);
      __hip_atomic_store(reinterpret_cast<uint32_t*>(a.h + (size_t)j * I + t * P) + threadIdx.x,
                         lo | (hi << 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Count this tile done once its stores are complete (P <= 128: the
    // storing threads are wavefront 0's, which waits for them here, before
    // thread 0's count); the pick's last tile raises the ready flags, after
    // the count that shows every other tile's stores complete.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = __hip_atomic_fetch_add(a.sync + sync_done(j), 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      if (prev == a.gu_tiles - 1)
        for (int x = 0; x < kXcds; ++x)
          __hip_atomic_store(a.sync + sync_ready(K, j, x), 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }

  // (3) down: weight rows t * dn_rows + ..; K = I.  The weight loads go out
  // first, then the wait for the pick's h.
  constexpr int RPW = kWave / LD;
  const int team = lane / LD, tl = lane % LD;
  const int n_base = t * a.dn_rows + wave * (RPW * NUD) + team * NUD;
  const int cpr = I / 32, bpr = I / kBlock;
  const uint8_t* wexp = a.dn_packed + (size_t)expert * H * (I / 2);
  const AbsT* aexp = static_cast<const AbsT*>(a.dn_absmax) + (size_t)expert * H * bpr;
  uint4 wq[STD][NUD];
  float av[STD][NUD];
#pragma unroll
  for (int st = 0; st < STD; ++st) {
    const int c = tl + st * LD;
    load_weights<NUD, AbsT>(wexp, aexp, I / 2, bpr, H, n_base, c, c < cpr, wq[st], av[st]);
  }
  // One poller per workgroup, on its XCD's ready line, about every 0.25 us
  // (the first poll returns after the weight loads: loads complete in order).
  if (threadIdx.x == 0) {
    const int* flag = a.sync + sync_ready(K, j, xcd_id());
    int spins = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
      if (++spins > kFfnSpinLimit) {
        __hip_atomic_store(a.sync + sync_error(K), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    // the pick's last down workgroup past the wait re-arms its words
    const int passed = __hip_atomic_fetch_add(a.sync + sync_passed(K, j), 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (passed == a.dn_tiles - 1) {
      __hip_atomic_store(a.sync + sync_done(j), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.sync + sync_passed(K, j), 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      for (int x = 0; x < kXcds; ++x)
        __hip_atomic_store(a.sync + sync_ready(K, j, x), 0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  // h row j at device scope, 32-bit words -> fp32 in the staging layout
  // (32 values per chunk c: piece p = 4 values at slot p * plane + c)
  XStage<1, x_batch(1, LD, STD)> stage;
  stage.init(0, cpr);
  {
    const uint32_t* hw = reinterpret_cast<const uint32_t*>(a.h + (size_t)j * I);
    for (int q = threadIdx.x; q < I / 2; q += kThreads) {
      const uint32_t v = __hip_atomic_load(hw + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int e0 = 2 * q;
      const int c = e0 / 32, within = e0 % 32;
      float* dst = reinterpret_cast<float*>(s_x + (within / 4) * stage.plane + c) + within % 4;
      dst[0] = __uint_as_float(v << 16);
      dst[1] = __uint_as_float(v & 0xffff0000u);
    }
  }
  lds_barrier();
  float acc[NUD];
  ffn_rows<LD, NUD, STD, AbsT>(s_x, stage.plane, lut, tl, cpr, wq, av, acc);
  if (tl == LD - 1) {
#pragma unroll
    for (int jj = 0; jj < NUD; ++jj) {
      const int n = n_base + jj;
      if (n < H) a.y[(size_t)j * H + n] = f32_to_bf16(acc[jj]);
    }
  }
}

}  // namespace

// Launch rule (host-known sizes only).  Rows per pass R from the rows per
// group; for each K split S (1 first, more only while a split keeps two team
// steps per lane) the team width L and steps follow from the split's chunks,
// and the rows per lane NU is the largest with NU * steps <= 4 and
// NU * R <= 4 that gives four wavefronts per SIMD, else the largest that
// gives two (a split is taken only when no NU of the smaller one gives
// two); a split must fit its activations in LDS.
static DecodePlan plan_decode_rule(int64_t M, int64_t N, int64_t K, int64_t G, int split_k,
                                   int num_cus) {
  const int cpr = (int)(K / 32);
  const int64_t g_eff = G < M ? G : M;
  const int64_t min_waves = 8LL * num_cus;    // two per SIMD
  const int64_t good_waves = 16LL * num_cus;  // four per SIMD
  const double rows_per_group = (double)M / (double)(g_eff > 0 ? g_eff : 1);
  const int R0 = rows_per_group <= 1.5 ? 1 : (rows_per_group <= 3.0 ? 2 : 4);
  for (int R = R0; R >= 1; R /= 2) {
    DecodePlan best{};
    int64_t best_waves = -1;
    bool split_more = false;
    for (int S = 1; S <= 16; S = split_k > 0 ? 17 : 2 * S) {
      if (split_k > 0) S = split_k;
      const int cps = (cpr + S - 1) / S;
      if (R * (cps + 1) > kXSlots) continue;
      const int L = pick_lanes(cps);
      if (L == 0) continue;
      if (split_more && cps < 2 * L) break;
      split_more = true;
      const int steps = (cps + L - 1) / L;
      DecodePlan enough{};  // the largest NU reaching min_waves
      bool have_enough = false;
      for (int NU = kMaxLoads; NU >= 1; NU /= 2) {
        if (NU * steps > kMaxLoads || NU * R > kMaxLoads) continue;
        DecodePlan p{};
        p.L = L;
        p.NU = NU;
        p.R = R;
        p.S = S;
        p.cps = cps;
        p.steps = steps;
        p.rows_per_block = kWaves * (kWave / L) * NU;
        p.n_tiles = (int)((N + p.rows_per_block - 1) / p.rows_per_block);
        const int64_t waves = g_eff * p.n_tiles * S * kWaves;
        if (waves >= good_waves) return p;
        if (waves >= min_waves && !have_enough) {
          enough = p;
          have_enough = true;
        }
        if (waves > best_waves) {
          best_waves = waves;
          best = p;
        }
      }
      if (have_enough) return enough;
    }
    if (best_waves >= 0) return best;
  }
  return DecodePlan{};  // L == 0: no split of K fits
}

DecodePlan plan_decode(int64_t M, int64_t N, int64_t K, int64_t G, int split_k, int num_cus) {
  return plan_decode_rule(M, N, K, G, split_k, num_cus);
}

size_t decode_workspace_bytes(const DecodePlan& p, int64_t M, int64_t N) {
  return p.S > 1 ? (size_t)p.S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

static DecodeKArgs decode_args(const GemmArgs& g, const DecodePlan& p) {
  DecodeKArgs a;
  a.g = g;
  a.x = g.x;
  a.packed = g.packed;
  a.absmax = g.absmax;
  a.out = p.S == 1 ? static_cast<void*>(g.y) : static_cast<void*>(g.partial);
  a.N = g.N;
  a.K = g.K;
  a.T = g.T;
  a.slot_div = g.slot_div;
  a.rows_max_decode = g.rows_max_decode;
  a.route_k = 0;
  a.vec_out = p.S == 1 && p.R == 1 && (p.NU == 2 || p.NU == 4) && g.N % p.NU == 0 &&
              reinterpret_cast<uintptr_t>(g.y) % (2 * p.NU) == 0;
  a.S = p.S;
  a.cps = p.cps;
  a.cpr = g.K / 32;
  a.rows_per_block = p.rows_per_block;
  a.inv_slot_div = 1.0 / (double)(g.slot_div > 0 ? g.slot_div : 1);
  a.route_logits = nullptr;
  a.ro = RouteOneOut{};
  return a;
}

static hipError_t launch_reduce(const DecodeKArgs& a, hipStream_t stream) {
  const GemmArgs& g = a.g;
  const dim3 grid((unsigned)((g.N + kThreads - 1) / kThreads), (unsigned)group_slots(g.G, g.M, 1));
  hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_routed(const GemmArgs& g, const DecodePlan& p, const float* logits,
                                const RouteOneOut& ro, hipStream_t stream) {
  DecodeKArgs a = decode_args(g, p);
  a.route_logits = logits;
  a.ro = ro;
  a.route_k = (int16_t)ro.K;
  if (ro.E > 2 * kWave) return hipErrorInvalidValue;
  const bool two = ro.E > kWave;
  hipError_t err;
  if (g.abs_bf16)
    err = two ? launch_routed_L<uint16_t, 2>(a, p, stream) : launch_routed_L<uint16_t, 1>(a, p, stream);
  else
    err = two ? launch_routed_L<float, 2>(a, p, stream) : launch_routed_L<float, 1>(a, p, stream);
  // the split-K reduce runs after the launch: the groups and slots it reads
  // are the route/sort outputs the launch wrote
  if (err != hipSuccess || p.S == 1) return err;
  return launch_reduce(a, stream);
}

hipError_t launch_decode(const GemmArgs& g, const DecodePlan& p, hipStream_t stream) {
  DecodeKArgs a = decode_args(g, p);
  hipError_t err;
  if (g.mxfp4) {
    switch (p.L) {
      case 64: err = launch_L<64, uint8_t>(a, p, stream); break;
      case 32: err = launch_L<32, uint8_t>(a, p, stream); break;
      case 16: err = launch_L<16, uint8_t>(a, p, stream); break;
      case 8: err = launch_L<8, uint8_t>(a, p, stream); break;
      default: return hipErrorInvalidValue;
    }
  } else if (g.abs_bf16) {
    switch (p.L) {
      case 64: err = launch_L<64, uint16_t>(a, p, stream); break;
      case 32: err = launch_L<32, uint16_t>(a, p, stream); break;
      case 16: err = launch_L<16, uint16_t>(a, p, stream); break;
      case 8: err = launch_L<8, uint16_t>(a, p, stream); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (p.L) {
      case 64: err = launch_L<64, float>(a, p, stream); break;
      case 32: err = launch_L<32, float>(a, p, stream); break;
      case 16: err = launch_L<16, float>(a, p, stream); break;
      case 8: err = launch_L<8, float>(a, p, stream); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (err != hipSuccess || p.S == 1) return err;
  return launch_reduce(a, stream);
}

// ------------------------------------------------------------ fused FFN
// The FFN launch's two roles take the plans the one-token decode launches
// would (no K split); the kernel is instantiated for the role pairs below.
// The one-token decode plans of the two projections, with the most rows per
// lane their steps allow (NU * steps <= 4): fewer, fatter workgroups, so the
// launch fits on the device at once and fewer down workgroups wait.
static DecodePlan ffn_role_plan(int top_k, int64_t N, int64_t K, int num_cus) {
  DecodePlan p = plan_decode(top_k, N, K, top_k, 1, num_cus);
  if (p.L == 0) return p;
  p.NU = kMaxLoads / p.steps;
  p.rows_per_block = kWaves * (kWave / p.L) * p.NU;
  p.n_tiles = (int)((N + p.rows_per_block - 1) / p.rows_per_block);
  return p;
}

bool plan_ffn(int64_t E, int top_k, int64_t H, int64_t I, int num_cus, FfnPlan& out) {
  out.gu = ffn_role_plan(top_k, 2 * I, H, num_cus);
  out.dn = ffn_role_plan(top_k, H, I, num_cus);
  const DecodePlan& g = out.gu;
  const DecodePlan& d = out.dn;
  if (g.L == 0 || d.L == 0 || g.S != 1 || d.S != 1 || g.R != 1 || d.R != 1) return false;
  if (g.rows_per_block % 2 != 0 || I % (g.rows_per_block / 2) != 0) return false;
  if (g.rows_per_block > kThreads) return false;
  if (g.cps + 1 > kXSlots || d.cps + 1 > kXSlots) return false;
  out.gu_tiles = (int)(I / (g.rows_per_block / 2));
  out.dn_tiles = d.n_tiles;
  if (!ffn_supported(out)) return false;
  // Every workgroup resident at once: the down workgroups then load their
  // weights while gate_up runs (the point of the fused launch), and no
  // waiting workgroup can hold a slot a gate_up workgroup needs.
  const int64_t grid = (int64_t)top_k * (out.gu_tiles + out.dn_tiles);
  return grid <= (int64_t)ffn_resident_per_cu(out, E > kWave) * num_cus;
}

namespace {

// role plans (L, NU, steps) the kernel is built for, as pairs
#define GNF4_FFN_PAIRS(X)                  \
  X(64, 4, 1, 32, 4, 1) /* OLMoE   */     \
  X(64, 4, 1, 8, 1, 3)  /* Qwen3   */

template <int LG, int NUG, int STG, int LD, int NUD, int STD, typename AbsT, int EPL>
hipError_t launch_ffn_one(const float* logits, const uint16_t* x, int E, const FfnKArgs& a,
                          int grid, size_t lds, hipStream_t stream) {
  hipLaunchKernelGGL((ffn_kernel<LG, NUG, STG, LD, NUD, STD, AbsT, EPL>), dim3(grid),
                     dim3(kThreads), lds, stream, logits, x, E, a);
  return hipGetLastError();
}

bool pair_is(const FfnPlan& p, int lg, int nug, int stg, int ld, int nud, int std_) {
  return p.gu.L == lg && p.gu.NU == nug && p.gu.steps == stg && p.dn.L == ld &&
         p.dn.NU == nud && p.dn.steps == std_;
}

}  // namespace

// Workgroups of the fused kernel one CU holds at once (the occupancy query
// on the current device; without one, 8: 256-thread workgroups of at most
// 64 VGPRs and the kernel's LDS).
int ffn_resident_per_cu(const FfnPlan& p, bool two_entries) {
  const size_t lds = (size_t)(p.gu.cps > p.dn.cps ? p.gu.cps + 1 : p.dn.cps + 1) * 128;
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
#define GNF4_FFN_OCC(lg, nug, stg, ld, nud, std_)                                                  \
  if (pair_is(p, lg, nug, stg, ld, nud, std_))                                                     \
    e = two_entries ? hipOccupancyMaxActiveBlocksPerMultiprocessor(                                \
                          &n, ffn_kernel<lg, nug, stg, ld, nud, std_, float, 2>, kThreads, lds)    \
                    : hipOccupancyMaxActiveBlocksPerMultiprocessor(                                \
                          &n, ffn_kernel<lg, nug, stg, ld, nud, std_, float, 1>, kThreads, lds);
  GNF4_FFN_PAIRS(GNF4_FFN_OCC)
#undef GNF4_FFN_OCC
  if (e != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 8;
  }
  return n;
}

size_t ffn_sync_bytes(int top_k) {
  return (size_t)(sync_error(top_k) + kSyncLine) * sizeof(int32_t);
}

bool ffn_supported(const FfnPlan& p) {
#define GNF4_FFN_MATCH(lg, nug, stg, ld, nud, std_) \
  if (pair_is(p, lg, nug, stg, ld, nud, std_)) return true;
  GNF4_FFN_PAIRS(GNF4_FFN_MATCH)
#undef GNF4_FFN_MATCH
  return false;
}

hipError_t launch_ffn_one_token(const FfnPlan& p, const float* logits, const uint16_t* x,
                                const uint8_t* gu_packed, const void* gu_absmax,
                                const uint8_t* dn_packed, const void* dn_absmax, bool abs_bf16,
                                int E, int top_k, int H, int I, uint16_t* h, uint16_t* y,
                                int32_t* sync, const RouteOneOut& ro, hipStream_t stream) {
  FfnKArgs a;
  a.gu_packed = gu_packed;
  a.gu_absmax = gu_absmax;
  a.dn_packed = dn_packed;
  a.dn_absmax = dn_absmax;
  a.h = h;
  a.y = y;
  a.sync = sync;
  a.H = H;
  a.I = I;
  a.route_k = top_k;
  a.gu_tiles = p.gu_tiles;
  a.dn_tiles = p.dn_tiles;
  a.gu_rows = p.gu.rows_per_block;
  a.dn_rows = p.dn.rows_per_block;
  a.ro = ro;
  const int grid = top_k * (p.gu_tiles + p.dn_tiles);
  const size_t lds = (size_t)(p.gu.cps > p.dn.cps ? p.gu.cps + 1 : p.dn.cps + 1) * 128;
  const bool two = E > kWave;
#define GNF4_FFN_LAUNCH(lg, nug, stg, ld, nud, std_)                                              \
  if (pair_is(p, lg, nug, stg, ld, nud, std_)) {                                                  \
    if (abs_bf16)                                                                                 \
      return two ? launch_ffn_one<lg, nug, stg, ld, nud, std_, uint16_t, 2>(logits, x, E, a, grid, \
                                                                            lds, stream)          \
                 : launch_ffn_one<lg, nug, stg, ld, nud, std_, uint16_t, 1>(logits, x, E, a, grid, \
                                                                            lds, stream);         \
    return two ? launch_ffn_one<lg, nug, stg, ld, nud, std_, float, 2>(logits, x, E, a, grid, lds, \
                                                                       stream)                    \
               : launch_ffn_one<lg, nug, stg, ld, nud, std_, float, 1>(logits, x, E, a, grid, lds, \
                                                                       stream);                   \
  }
  GNF4_FFN_PAIRS(GNF4_FFN_LAUNCH)
#undef GNF4_FFN_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace gnf4
