// Internal declarations shared by the libgnf4 translation units.
// Target: gfx950 (CDNA4) only: 64-lane wavefronts, MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gnf4.h"

namespace gnf4 {

// NormalFloat4 levels (QLoRA, Dettmers et al. 2023, section 3), index = code.
// The library's own copy of the spec constants.
__host__ __device__ constexpr float nf4_level(int i) {
  return i == 0 ? -1.0f
       : i == 1 ? -0.6961928009986877f
       : i == 2 ? -0.5250730514526367f
       : i == 3 ? -0.39491748809814453f
       : i == 4 ? -0.28444138169288635f
       : i == 5 ? -0.18477343022823334f
       : i == 6 ? -0.09105003625154495f
       : i == 7 ? 0.0f
       : i == 8 ? 0.07958029955625534f
       : i == 9 ? 0.16093020141124725f
       : i == 10 ? 0.2461123913526535f
       : i == 11 ? 0.33791524171829224f
       : i == 12 ? 0.44070982933044434f
       : i == 13 ? 0.5626170039176941f
       : i == 14 ? 0.7229568362236023f
       : 1.0f;
}

constexpr int kBlock = 64;       // elements per absmax block along K
constexpr int kZeroCode = 7;     // code of the exact zero level
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32, one instruction.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// One block absmax as fp32, from either stored form (fp32, or bf16 bits).
__device__ __forceinline__ float absmax_at(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float absmax_at(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

// p[0] + p[plane] + ... + p[(S - 1) * plane] added in split order, starting
// from +0, with up to 16 loads in flight (one per split, each a memory round
// trip).  Every load is issued, clamped to the last split; the padding adds
// +0, which leaves the sum unchanged (a sum started at +0 is never -0).
__device__ __forceinline__ float sum_splits(const float* p, size_t plane, int S) {
  constexpr int kBatch = 16;
  float sum = 0.0f;
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int si = min(s0 + u, S - 1);
      const float t = p[(size_t)si * plane];
      v[u] = s0 + u < S ? t : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) sum += v[u];
  }
  return sum;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// ---- wavefront reductions on the DPP network (no LDS round trips).
// Every lane of the wave must be active.  DPP controls (gfx9): quad_perm
// [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_mirror = 0x140, row_half_mirror =
// 0x141, row_bcast:15 = 0x142, row_bcast:31 = 0x143, row_shr:n = 0x110 + n.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<0xB1, 0xF>(0u, x));
  x = max(x, dpp_u32<0x4E, 0xF>(0u, x));
  x = max(x, dpp_u32<0x141, 0xF>(0u, x));
  x = max(x, dpp_u32<0x140, 0xF>(0u, x));
  x = max(x, dpp_u32<0x142, 0xA>(0u, x));
  x = max(x, dpp_u32<0x143, 0xC>(0u, x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_u32<0xB1, 0xF>(~0u, x));
  x = min(x, dpp_u32<0x4E, 0xF>(~0u, x));
  x = min(x, dpp_u32<0x141, 0xF>(~0u, x));
  x = min(x, dpp_u32<0x140, 0xF>(~0u, x));
  x = min(x, dpp_u32<0x142, 0xA>(~0u, x));
  x = min(x, dpp_u32<0x143, 0xC>(~0u, x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Inclusive prefix sum across the wave (lane i gets sum of lanes 0..i).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += (int)dpp_u32<0x111, 0xF>(0u, (uint32_t)x);
  x += (int)dpp_u32<0x112, 0xF>(0u, (uint32_t)x);
  x += (int)dpp_u32<0x114, 0xF>(0u, (uint32_t)x);
  x += (int)dpp_u32<0x118, 0xF>(0u, (uint32_t)x);
  x += (int)dpp_u32<0x142, 0xA>(0u, (uint32_t)x);
  x += (int)dpp_u32<0x143, 0xC>(0u, (uint32_t)x);
  return x;
}

// One group of a grouped GEMM, as located by find_group.
struct GroupRef {
  int g;       // index into sizes / ids
  int size;    // rows
  int expert;  // expert id
  int row;     // first row: sum of max(size, 0) over the groups before g, capped at M
};

// The j-th group (in group order) whose size lies in [lo, hi] (lo >= 1) and
// whose expert id lies in [0, E): kernels launch one slot per group they can
// handle instead of one per entry of `sizes`, so empty groups cost no
// workgroups.  Call with the whole wavefront active; every lane gets the same
// result.  Sizes are clamped to [0, M] before summing (M < 2^25, so the
// wavefront's partial sums fit an int) and the running row count saturates at
// M, where nothing is written.  All loads of a 256-group chunk are issued
// before any is used.
// The loads of one 256-group chunk of find_group, starting at group c0.
struct GroupChunk {
  int sv[4], ev[4];
};
__device__ __forceinline__ void load_group_chunk(const int32_t* sizes, const int32_t* ids, int G,
                                                 int c0, GroupChunk& ch) {
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = c0 + q * kWave + lane;
    ch.sv[q] = i < G ? sizes[i] : 0;
    ch.ev[q] = i < G ? ids[i] : -1;
  }
}

// find_group with the first chunk's loads already issued (load_group_chunk
// at c0 = 0), so a kernel can put other work between issue and use.
__device__ __forceinline__ bool find_group_from(const int32_t* sizes, const int32_t* ids, int G,
                                                int E, int M, int lo, int hi, int j,
                                                const GroupChunk& first, GroupRef& out) {
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  int seen = 0, rows = 0;
  for (int c0 = 0; c0 < G; c0 += 4 * kWave) {
    GroupChunk ch;
    if (c0 == 0)
      ch = first;
    else
      load_group_chunk(sizes, ids, G, c0, ch);
    const int* sv = ch.sv;
    const int* ev = ch.ev;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = sv[q] >= lo && sv[q] <= hi && ev[q] >= 0 && ev[q] < E;
      const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
      const int cnt = __builtin_popcountll(m);
      const int incl = wave_incl_scan(min(max(sv[q], 0), M));
      if (j < seen + cnt) {
        const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const uint64_t pick = __builtin_amdgcn_ballot_w64(ok && below == j - seen);
        const int src = __builtin_ctzll(pick);
        const int sz = __builtin_amdgcn_readlane(sv[q], src);
        out.g = c0 + q * kWave + src;
        out.size = sz;
        out.expert = __builtin_amdgcn_readlane(ev[q], src);
        out.row = min(rows + __builtin_amdgcn_readlane(incl, src) - min(sz, M), M);
        return true;
      }
      seen += cnt;
      rows = min(rows + __builtin_amdgcn_readlane(incl, 63), M);
    }
  }
  return false;
}

__device__ __forceinline__ bool find_group(const int32_t* sizes, const int32_t* ids, int G,
                                           int E, int M, int lo, int hi, int j, GroupRef& out) {
  GroupChunk first;
  load_group_chunk(sizes, ids, G, 0, first);
  return find_group_from(sizes, ids, G, E, M, lo, hi, j, first, out);
}

// Upper bound on the groups with at least `lo` rows that start inside M
// rows, among G groups: the first c - 1 of c such groups end before the
// last one starts, so (c - 1) lo <= M - 1, i.e. c <= ceil(M / lo).  (The
// last group may be clipped at M: sizes [9, 9] with M = 17 are two groups.)
inline int64_t group_slots(int64_t G, int64_t M, int64_t lo) {
  const int64_t l = lo > 0 ? lo : 1;
  const int64_t cap = (M + l - 1) / l;
  return G < cap ? G : cap;
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are validated by
// the C-ABI layer before these are called.

// absmax is fp32 (abs_dtype GNF4_DTYPE_F32) or bf16 bits (GNF4_DTYPE_BF16).
hipError_t launch_pack(const void* w, int dtype, int64_t n_blocks, uint8_t* packed,
                       void* absmax, int abs_dtype, hipStream_t stream);

struct RoutePlan {
  int chunk_tokens;   // tokens per chunk of the sort
  int n_chunks;       // 0 => single fused launch (T <= 32)
  size_t ws_bytes;    // per-chunk counts
};
RoutePlan plan_route(int64_t T, int64_t E, int top_k);

hipError_t launch_route_sort(const float* logits, int T, int E, int top_k, int32_t* topk_ids,
                             float* topk_w, int32_t* expert_offsets, int32_t* sorted_slots,
                             int32_t* slot_rows, int32_t* group_sizes, int32_t* group_expert_ids,
                             int32_t* num_groups, int32_t* ws, const RoutePlan& plan,
                             hipStream_t stream);

struct GemmArgs {
  const uint16_t* x;
  const uint8_t* packed;
  const void* absmax;  // fp32, or bf16 bits when abs_bf16; E8M0 bytes when mxfp4
  bool abs_bf16;
  bool mxfp4;          // MXFP4 stack: E2M1 codes (first element low), E8M0 per 32
  const int32_t* sizes;
  const int32_t* ids;
  uint16_t* y;
  float* partial;     // split-K partials [S, M, N] (decode path)
  // Tile path: the activation rows staged once by stage_x as fp16 times a
  // power of two per row (xh [rows + 1, xh_ld], row `rows` all zeros) and
  // the exponents (row_exp [rows + 1]); see launch_stage_x.
  int32_t* row_exp;
  uint16_t* xh;
  int xh_ld;
  // Optional fused gather: when `slots` is set, output row r uses activation
  // row slots[r] / slot_div of x (x is then [T, K]); a slot outside
  // [0, T * slot_div) leaves row r unwritten.
  const int32_t* slots;
  int slot_div, T;
  int E, N, K, G, M;
  int rows_max_decode;  // groups with size <= this take the decode path
  int rows_min_tile;    // groups with size >= this take the tile path
};

struct DecodePlan {
  int L;        // lanes per weight row (8, 16, 32, 64)
  int NU;       // weight rows per lane
  int R;        // activation rows per pass over a weight tile
  int S;        // K splits
  int cps;      // 32-code chunks per split
  int steps;    // chunks per lane and weight row: ceil(cps / L)
  int n_tiles;  // weight-row tiles per group
  int rows_per_block;
};
DecodePlan plan_decode(int64_t M, int64_t N, int64_t K, int64_t G, int split_k, int num_cus);
size_t decode_workspace_bytes(const DecodePlan& p, int64_t M, int64_t N);

hipError_t launch_decode(const GemmArgs& a, const DecodePlan& p, hipStream_t stream);
hipError_t launch_tile(const GemmArgs& a, hipStream_t stream);

// Activation staging for the matrix-core kernels.  Rows are those of x
// itself (one per token row when the gather is fused and T <= M, else one
// per output row r < M, read through its slot), each written once as fp16
// times 2^t (t chosen per row so its largest |x| lands in [2^14, 2^15);
// every bf16 value within 2^28 of the row's largest converts exactly) into
// xh [rows + 1, ld] with ld = kStageAlign-padded K, zero-filled past K and
// in the MFMA operand order of the weight format (NF4: each 8 elements as
// {0, 2, 4, 6, 1, 3, 5, 7}; MXFP4 and the dgrad: natural order); row
// `rows` is all zeros (the source of absent rows) and row_exp[rows] = 0.
constexpr int kStageAlign = 128;
struct StagePlan {
  int rows;        // staged rows (T or M), plus one zero row
  bool by_token;   // rows are token rows of x (fused gather)
  int ld;          // fp16 elements per staged row
};
StagePlan plan_stage(const GemmArgs& g);
size_t stage_bytes(int64_t rows, int64_t width);  // row_exp + xh for `rows` rows, 256-aligned
hipError_t launch_stage_x(const GemmArgs& g, const StagePlan& p, bool natural_order,
                          hipStream_t stream);

hipError_t launch_gather(const uint16_t* x, const int32_t* slots, int top_k, int T, int M, int K,
                         uint16_t* out, hipStream_t stream);

struct DgradArgs {
  const uint16_t* dy;
  const uint8_t* packed;
  const void* absmax;  // fp32, or bf16 bits when abs_bf16
  bool abs_bf16;
  const int32_t* sizes;
  const int32_t* ids;
  uint16_t* dx;
  float* partial;     // split-N partials [S, M, K]
  int E, N, K, G, M;
};

struct DgradPlan {
  int R;               // rows of dy per pass over the weights
  int L;               // lanes per weight row (a team); 64 / L teams per wavefront
  int k_tiles;         // slices of K of L chunks of 32 (one chunk per lane)
  int S;               // N splits
  int rows_per_split;  // weight rows per split
  int NB;              // weight rows in flight per team (8, or 4 to reach more splits)
};
DgradPlan plan_dgrad(int64_t M, int64_t N, int64_t K, int64_t G, int num_cus);
size_t dgrad_workspace_bytes(const DgradPlan& p, int64_t M, int64_t K);
hipError_t launch_dgrad(const DgradArgs& a, const DgradPlan& p, hipStream_t stream);

hipError_t launch_swiglu(const uint16_t* gate_up, int64_t M, int64_t I, uint16_t* h,
                         hipStream_t stream);
hipError_t launch_combine(const uint16_t* y, const int32_t* slot_rows, const float* topk_w,
                          int64_t T, int top_k, int64_t M, int64_t H, uint16_t* out,
                          hipStream_t stream);

int device_cu_count();

// Opt-in check of device-resident grouping inputs (validate.hip).
// validate_requested(): GNF4_VALIDATE=1 in the environment (read per call).
// validate_groups() runs the check on `stream`, waits for it and stores in
// `result` a nonzero bit set when a size is negative, a non-empty group's id
// lies outside [0, E), the sizes sum past M, or (slots given) a covered row's
// slot lies outside [0, slot_lim).
bool validate_requested();
hipError_t validate_groups(const int32_t* sizes, const int32_t* ids, int64_t G, int64_t E,
                           int64_t M, const int32_t* slots, int64_t slot_lim,
                           hipStream_t stream, int32_t* result);

}  // namespace gnf4
