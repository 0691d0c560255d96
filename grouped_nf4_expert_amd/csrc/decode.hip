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
  int route_k;  // picks per token of the routed launch (ro.K)
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
__device__ __forceinline__ void load_weights(const uint8_t* wexp, const AbsT* aexp,
                                             size_t row_bytes, int bpr, int N, int n_base, int c,
                                             bool valid, uint4 (&wq)[NU], float (&av)[NU]) {
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    const int n = n_base + j;
    const bool ok = valid && n < N;
    const size_t nn = ok ? (size_t)n : 0;
    const size_t cc = ok ? (size_t)c : 0;
    const uint4 q = *reinterpret_cast<const uint4*>(wexp + nn * row_bytes + 16 * cc);
    float v;
    if constexpr (kMxfp4<AbsT>)
      v = e8m0_to_f32(aexp[nn * (2 * bpr) + cc]);  // one scale per chunk
    else
      v = absmax_at(aexp, nn * bpr + (cc >> 1));
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
               "s"(a.cps), "s"(a.cpr), "s"(a.rows_per_block), "s"(a.route_k)
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
    // One token routed in the launch.  Entry s of lane l holds expert
    // l + 64 s's key, as the route/sort kernels build it (rank_token): the
    // logit's order-preserving key above the complemented expert id, so keys
    // are distinct, larger is better and the lower id wins a tie.  Every
    // wavefront finds the K-th largest key on its own, bit by bit from the
    // top (a radix select over ballot counts: the largest t with at least K
    // keys >= t); the picks are the keys >= t, the same set rank_token's
    // ranks < K give.  Only the bits that differ between keys are searched:
    // the 32 of the logit's key, then the low 7 of the id part (ids below
    // 128 share bits 7..31 of ~id).  Group j is the j-th pick in expert order,
    // one row (row j, token 0).
    constexpr int EPL = ROUTED;
    const int E = k_E;
    float val[EPL];
    uint64_t key[EPL];
#pragma unroll
    for (int s = 0; s < EPL; ++s) {
      const int e = lane + kWave * s;
      val[s] = e < E ? k_logits[e] : 0.0f;
    }
    pin_args(a);
    const int kpick = a.route_k;
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
    const int j = blockIdx.y;
    int jj = j;
    gr.expert = 0;
#pragma unroll
    for (int s = 0; s < EPL; ++s) {
      uint64_t m = sel[s];
      const int c = __popcll(m);
      if (jj >= 0 && jj < c) {  // uniform
        for (int q = 0; q < jj; ++q) m &= m - 1;
        gr.expert = kWave * s + __ffsll((unsigned long long)m) - 1;
      }
      jj -= c;
    }
    gr.g = j;
    gr.size = 1;
    gr.row = j;
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && wave == 0) {
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
      route_one_token_write<EPL>(a.ro, lane, val, rank);
    }
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
    load_weights<NU, AbsT>(wexp, aexp, row_bytes, bpr, N, n_base, c, c < c_end, wq[st], av[st]);
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
  a.route_k = ro.K;
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

}  // namespace gnf4
