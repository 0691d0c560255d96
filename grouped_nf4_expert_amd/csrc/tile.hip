// Tile path of the grouped NF4 GEMM: groups with many rows (prefill), on the
// CDNA4 matrix cores.
//
// Page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE
// expert stacks": "Layout" (the M-tile path) and "The claim" (prefill is the
// compute-bound regime; the register-LUT mainloop decodes codes inside the
// GEMM loop).  The pages' kernel was written for other hardware; this one is
// built around gfx950's v_mfma_f32_32x32x16_f16.
//
// Precision: a single bf16 rounding of the decoded weights is too coarse for
// an element-wise tolerance of 8e-3 |y| + 1e-3 rms(y) at K in the thousands,
// while fp16 weights rounded ONCE from the fp32 product absmax * level are
// well inside it.  So each weight row n gets a power-of-two scale 2^-s_n that
// brings its largest block absmax into [2^14, 2^15); codes are decoded
// straight to fp16(level * absmax * 2^-s_n) (fp32 product, one rounding).
// Every block whose absmax lies within 2^25 of its row's largest then
// decodes to normal fp16 numbers (the smallest nonzero level is 0.0796), so
// its values carry fp16's full 11 bits however far below the row's largest
// it sits; only blocks further down lose bits in fp16's subnormals.  Each
// activation row m is staged once (stage_x_kernel) as fp16 times its own
// power of two 2^t_m that puts its largest |x| in [2^14, 2^15): every bf16
// value within 2^28 of the row's largest converts exactly.  Products (at
// most 2^30) accumulate in fp32 on the matrix core and the epilogue
// multiplies by 2^(s_n - t_m) exactly before rounding to bf16.
//
// Work layout (XCD-aware): a workgroup of 8 wavefronts owns one (group, 256
// output columns) tile and walks K in steps of 128 (two absmax blocks).  All
// workgroups of one group's column tiles are dispatched to the same XCD so
// the group's activation rows stay in that XCD's L2.  Each wavefront owns 32
// columns (one MFMA column tile) for every row of the group (up to 5 row
// tiles of 32 per pass), so every code is decoded exactly once per pass; one
// column tile per wavefront keeps the registers within two wavefronts per
// SIMD, so one wavefront's decode overlaps the other's matrix-core work:
//  * weights: a lane owns one weight row and one 64-code absmax block per K
//    step (lane half h = block h); it loads its 32 bytes
//    straight from HBM into registers, builds the 16-entry fp16 table of that
//    block (16 products, 8 packs, 8 byte-plane permutes) and decodes 8 codes
//    per dword with v_perm_b32 byte lookups -- no LDS traffic for weights;
//  * activations: the group's rows x 128 K of the staged fp16 rows, already
//    in the K order the weight decode produces (so A and B fragments agree
//    slot by slot), are copied through LDS (double-buffered, rows padded to
//    272 bytes so the 16-byte fragment reads are bank-conflict-free); the
//    copy has no conversion and no bounds tests: staged rows are padded to a
//    multiple of 128 and absent rows read the staged zero row.

#include <limits.h>

#include <type_traits>

#include "dgrad_tile.h"
#include "gnf4_internal.h"

namespace gnf4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
// 16 bytes as a native vector: copies of it stay in registers (a HIP uint4
// struct copied into LDS can become a memcpy that keeps its source in
// scratch memory)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;      // 8 wavefronts, two per SIMD
constexpr int kTileN = 256;        // output columns per workgroup (32 per wavefront)
constexpr int kStepK = 128;        // K per main-loop step
constexpr int kRowTiles = 5;       // 32-row MFMA tiles per pass
constexpr int kPassRows = 32 * kRowTiles;
static_assert(kPassRows <= 512, "one exponent per thread and pass");
constexpr int kLdsRow = kStepK + 8;  // fp16 elements per staged row (padded)

struct TileKArgs {
  GemmArgs g;
  StagePlan st;  // the staged activation rows (xh, row_exp) and their indexing
  int n_tiles;
  int n_work;   // group slots * n_tiles
};

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// fp16 decode table of one 64-code block: byte planes of fp16(level * a).
struct Table {
  uint32_t l0, l1, l2, l3, h0, h1, h2, h3;
};

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ Table make_table(float a) {
  uint32_t p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = pack_f16x2(nf4_level(2 * i) * a, nf4_level(2 * i + 1) * a);
  Table t;
  // low bytes of levels 4j..4j+3 and high bytes, from the packed pairs
  t.l0 = perm(p[1], p[0], 0x06040200u);
  t.h0 = perm(p[1], p[0], 0x07050301u);
  t.l1 = perm(p[3], p[2], 0x06040200u);
  t.h1 = perm(p[3], p[2], 0x07050301u);
  t.l2 = perm(p[5], p[4], 0x06040200u);
  t.h2 = perm(p[5], p[4], 0x07050301u);
  t.l3 = perm(p[7], p[6], 0x06040200u);
  t.h3 = perm(p[7], p[6], 0x07050301u);
  return t;
}

// Four codes (one per byte of c, values 0..15) -> two dwords of fp16 pairs.
// v_perm_b32 returns 0xff for a selector byte >= 13: codes 8..15 get selector
// code+8 (16..23) in the low-half lookup and codes 0..7 get code+16 in the
// high-half lookup, so AND-ing the two lookups keeps the valid byte.
__device__ __forceinline__ void lookup4(uint32_t c, const Table& t, uint32_t& o0, uint32_t& o1) {
  const uint32_t s_lo = c + (c & 0x08080808u);
  const uint32_t s_hi = s_lo ^ 0x10101010u;
  const uint32_t rl = perm(t.l1, t.l0, s_lo) & perm(t.l3, t.l2, s_hi);
  const uint32_t rh = perm(t.h1, t.h0, s_lo) & perm(t.h3, t.h2, s_hi);
  o0 = perm(rh, rl, 0x05010400u);
  o1 = perm(rh, rl, 0x07030602u);
}

// Eight codes of one packed dword -> MFMA operand in the slot order
// k = {0, 2, 4, 6, 1, 3, 5, 7} (high nibbles first).
__device__ __forceinline__ half8 decode8(uint32_t d, const Table& t) {
  uint32_t o[4];
  lookup4((d >> 4) & 0x0f0f0f0fu, t, o[0], o[1]);
  lookup4(d & 0x0f0f0f0fu, t, o[2], o[3]);
  half8 r;
  __builtin_memcpy(&r, o, sizeof(o));
  return r;
}

// decode8 as 25 single-instruction micro-steps over explicit state, so a
// caller can interleave them with other work at instruction grain: step k
// of the sequence; after step 24, o holds what decode8 returns.
struct Decode8State {
  uint32_t ch, cl, t, sl, sh, p1, p2, rl, rh;
  uint32_t o[4];
};
template <int K>
__device__ __forceinline__ void decode8_step(uint32_t d, const Table& tb, Decode8State& s) {
  if constexpr (K == 0) s.ch = d >> 4;
  else if constexpr (K == 1) s.ch &= 0x0f0f0f0fu;
  else if constexpr (K == 2) s.cl = d & 0x0f0f0f0fu;
  // high nibbles (the first elements): the four codes of s.ch
  else if constexpr (K == 3) s.t = s.ch & 0x08080808u;
  else if constexpr (K == 4) s.sl = s.ch + s.t;
  else if constexpr (K == 5) s.sh = s.sl ^ 0x10101010u;
  else if constexpr (K == 6) s.p1 = perm(tb.l1, tb.l0, s.sl);
  else if constexpr (K == 7) s.p2 = perm(tb.l3, tb.l2, s.sh);
  else if constexpr (K == 8) s.rl = s.p1 & s.p2;
  else if constexpr (K == 9) s.p1 = perm(tb.h1, tb.h0, s.sl);
  else if constexpr (K == 10) s.p2 = perm(tb.h3, tb.h2, s.sh);
  else if constexpr (K == 11) s.rh = s.p1 & s.p2;
  else if constexpr (K == 12) s.o[0] = perm(s.rh, s.rl, 0x05010400u);
  else if constexpr (K == 13) s.o[1] = perm(s.rh, s.rl, 0x07030602u);
  // low nibbles (the second elements)
  else if constexpr (K == 14) s.t = s.cl & 0x08080808u;
  else if constexpr (K == 15) s.sl = s.cl + s.t;
  else if constexpr (K == 16) s.sh = s.sl ^ 0x10101010u;
  else if constexpr (K == 17) s.p1 = perm(tb.l1, tb.l0, s.sl);
  else if constexpr (K == 18) s.p2 = perm(tb.l3, tb.l2, s.sh);
  else if constexpr (K == 19) s.rl = s.p1 & s.p2;
  else if constexpr (K == 20) s.p1 = perm(tb.h1, tb.h0, s.sl);
  else if constexpr (K == 21) s.p2 = perm(tb.h3, tb.h2, s.sh);
  else if constexpr (K == 22) s.rh = s.p1 & s.p2;
  else if constexpr (K == 23) s.o[2] = perm(s.rh, s.rl, 0x05010400u);
  else if constexpr (K == 24) s.o[3] = perm(s.rh, s.rl, 0x07030602u);
}
template <int K0, int K1>
__device__ __forceinline__ void decode8_steps(uint32_t d, const Table& tb, Decode8State& s) {
  if constexpr (K0 < K1) {
    decode8_step<K0>(d, tb, s);
    decode8_steps<K0 + 1, K1>(d, tb, s);
  }
}
constexpr int kDecodeSteps = 25;

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// The stack's scale type names its format: fp32 or bf16 block absmax (NF4),
// or uint8 E8M0 scales (MXFP4: E2M1 codes, one scale per 32, low nibble
// first).
template <typename AbsT>
constexpr bool kTileMx = std::is_same_v<AbsT, uint8_t>;

// MXFP4: the 8 codes of dword d -> MFMA operand in K order.  gfx950's
// convert applies the exponent of `scale` exactly (E8M0 scales are powers of
// two): `scale` carries the block scale times the weight row's 2^-s_n.
__device__ __forceinline__ half8 mx_decode8(uint32_t d, float scale) {
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  const h2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 0);
  const h2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 1);
  const h2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 2);
  const h2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 3);
  half8 r;
  r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
  r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
  return r;
}

// Everything one pass over K needs, shared by the row-tile specialisations.
struct PassCtx {
  const TileKArgs* a;
  _Float16* s_x;           // [2][kPassRows * kLdsRow]
  const int* s_src;        // [kPassRows] staged row of each of the pass's rows
  const int* s_exp;        // [kPassRows] their activation exponents
  const uint8_t* wrow;     // this lane's weight row (or row 0 when out of range)
  const void* arow;        // its absmax row (fp32, or bf16 bits)
  bool n_ok;               // the lane's column exists
  int sexp;                // its power-of-two scale exponent
  bool col_nan;            // MXFP4: the weight row holds a NaN scale
  int tid, i, h, N, K, bpr, n, p0, rows, r_end, n_steps, rem_k;
};

// q = n / d for 0 <= n < 2^31, 1 <= d < 2^31, from a double estimate.
__device__ __forceinline__ int div_slot(int n, int d) {
  int q = (int)((double)n / (double)d);
  if ((long long)(q + 1) * d <= n) ++q;
  if ((long long)q * d > n) --q;
  return q;
}

// One pass of up to RT row tiles (RT * 32 rows) over the whole K range.  RT
// is a compile-time constant so the row-tile loops carry no branches: every
// MFMA of a sub-step and its A-fragment reads are issued back to back, and
// the next sub-step's decode can overlap them.  Loads are unconditional (an
// absent row reads the staged zero row, an absent column an always-valid
// weight address) and an absent weight block decodes through a zero table.
template <int RT, typename AbsT>
__device__ __forceinline__ void tile_pass(const PassCtx& c) {
  const GemmArgs& g = c.a->g;
  constexpr int kChunks = RT;  // 16-byte x chunks per thread: RT*32 rows x 16 chunks / 512 threads
  float16v acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[rt][v] = 0.0f;

  const int total_steps = c.n_steps + (c.rem_k ? 1 : 0);
  // staged source of each chunk this thread copies (row-major staged rows,
  // 16 chunks of 8 fp16 per row and step)
  const uint16_t* xsrc[kChunks];
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const int q = c.tid + kThreads * j;
    xsrc[j] = g.xh + (size_t)c.s_src[q >> 4] * g.xh_ld + 8 * (q & 15);
  }

  // Two register sets (activations and weights) alternate between steps so
  // every load is issued two steps before it is used: step s computes from
  // LDS buffer s % 2, then stages step s + 1's activations (loaded during
  // step s - 1) into the other buffer; one barrier per step.  The step loop
  // is unrolled by two so the register sets are static.
  u32x4 xr[2][kChunks];
  uint4 wc[2][2];
  float wa[2];
  auto load_x = [&](auto slot_c, int step) {
    constexpr int sl = decltype(slot_c)::value;
#pragma unroll
    for (int j = 0; j < kChunks; ++j)
      xr[sl][j] = *reinterpret_cast<const u32x4*>(xsrc[j] + step * kStepK);
  };
  auto store_x = [&](auto slot_c, int buf) {
    constexpr int sl = decltype(slot_c)::value;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int q = c.tid + kThreads * j;
      *reinterpret_cast<u32x4*>(
          &c.s_x[buf * (kPassRows * kLdsRow) + (q >> 4) * kLdsRow + 8 * (q & 15)]) = xr[sl][j];
    }
  };
  // weight codes: the lane's 32 bytes of block h of the step, and its absmax
  auto load_w = [&](auto slot_c, int step) {
    constexpr int sl = decltype(slot_c)::value;
    const int blk = 2 * step + c.h;
    const bool ok = c.n_ok && blk < c.bpr;
    const uint4* p = reinterpret_cast<const uint4*>(c.wrow + (ok ? 32 * (size_t)blk : 0));
    wc[sl][0] = p[0];
    wc[sl][1] = p[1];
    if constexpr (kTileMx<AbsT>) {
      // the two E8M0 scales of the 64-code block, packed in a register
      const uint8_t* ar = static_cast<const uint8_t*>(c.arow);
      const uint32_t s0 = ar[ok ? 2 * blk : 0], s1 = ar[ok ? 2 * blk + 1 : 1];
      wa[sl] = __uint_as_float(s0 | (s1 << 8));
    } else {
      wa[sl] = absmax_at(static_cast<const AbsT*>(c.arow), ok ? blk : 0);
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  const int last = total_steps - 1;

  auto do_step = [&](auto slot_c, int step) {
    constexpr int sl = decltype(slot_c)::value;
    using SO = std::integral_constant<int, 1 - sl>;
    const uint4 cw[2] = {wc[sl][0], wc[sl][1]};
    const float ca = wa[sl];
    const bool cok = c.n_ok && 2 * step + c.h < c.bpr;
    load_x(slot_c, min(step + 2, last));
    load_w(slot_c, min(step + 2, last));
    Table tab;
    float sc0 = 0.0f, sc1 = 0.0f;
    if constexpr (kTileMx<AbsT>) {
      // an absent block converts with scale 0, which the convert treats as
      // 2^-127: its values vanish in fp16
      const uint32_t sb = __float_as_uint(ca);
      sc0 = cok ? ldexpf(1.0f, (int)(sb & 0xffu) - 127 - c.sexp) : 0.0f;
      sc1 = cok ? ldexpf(1.0f, (int)((sb >> 8) & 0xffu) - 127 - c.sexp) : 0.0f;
    } else {
      tab = make_table(cok ? ldexpf(ca, -c.sexp) : 0.0f);
    }
    const _Float16* xs = c.s_x + sl * (kPassRows * kLdsRow);
    // A wavefront's VALU work overlaps only its own matrix-core
    // instructions (another wavefront's VALU on the same SIMD waits for the
    // MFMA), so the NF4 decode of sub-step s + 1 is spread over sub-step s's
    // MFMAs at instruction grain: after each MFMA (32 cycles) come one
    // fragment read of the next sub-step and about 25 / RT decode
    // instructions, each group fenced off so the scheduler keeps it there.
    half8 ax[2][RT];
    half8 bw[2];
    auto read_a = [&](int buf, int sub, int rt) {
      ax[buf][rt] =
          *reinterpret_cast<const half8*>(xs + (rt * 32 + c.i) * kLdsRow + 64 * c.h + 8 * sub);
    };
    if constexpr (kTileMx<AbsT>) {
#pragma unroll
      for (int sub = 0; sub < 8; ++sub) {
        bw[0] = mx_decode8((&cw[0].x)[sub], sub < 4 ? sc0 : sc1);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) read_a(0, sub, rt);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ax[0][rt], bw[0], acc[rt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) read_a(0, 0, rt);
      bw[0] = decode8(cw[0].x, tab);
      auto sub_step = [&](auto sub_c) {
        constexpr int sub = decltype(sub_c)::value;
        constexpr int cur = sub & 1, nxt = cur ^ 1;
        Decode8State ds;
        const uint32_t dn = sub < 7 ? (&cw[0].x)[sub < 7 ? sub + 1 : 0] : 0u;
        auto group = [&](auto rt_c) {
          constexpr int rt = decltype(rt_c)::value;
          acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ax[cur][rt], bw[cur], acc[rt], 0, 0, 0);
          if constexpr (sub < 7) {
            read_a(nxt, sub + 1, rt);
            decode8_steps<rt * kDecodeSteps / RT, (rt + 1) * kDecodeSteps / RT>(dn, tab, ds);
          }
          __builtin_amdgcn_sched_barrier(0);
        };
        static_for<RT>(group);
        if constexpr (sub < 7) {
          half8 b;
          __builtin_memcpy(&b, ds.o, sizeof(ds.o));
          bw[nxt] = b;
        }
      };
      static_for<8>(sub_step);
    }
    if (step < last) {
      store_x(SO{}, 1 - sl);
      __syncthreads();
    }
  };

  load_x(S0{}, 0);
  load_w(S0{}, 0);
  load_x(S1{}, min(1, last));
  load_w(S1{}, min(1, last));
  store_x(S0{}, 0);
  __syncthreads();
  for (int step = 0; step < total_steps; step += 2) {
    do_step(S0{}, step);
    if (step + 1 < total_steps) do_step(S1{}, step + 1);
  }

  // epilogue: D[row][col], col = lane % 32, row = 8 (v / 4) + 4 h + v % 4
  if (!c.n_ok) return;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    // rows the fused gather skips are not written: their slots, loaded all
    // at once before any store
    uint32_t skip = 0;
    if (g.slots) {
      int sl[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = c.p0 + rt * 32 + 8 * (v >> 2) + 4 * c.h + (v & 3);
        sl[v] = g.slots[row < c.r_end ? row : c.p0];
      }
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (sl[v] < 0 || sl[v] >= g.T * g.slot_div) skip |= 1u << v;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = c.p0 + rt * 32 + 8 * (v >> 2) + 4 * c.h + (v & 3);
      if (row >= c.r_end || ((skip >> v) & 1u)) continue;
      uint16_t out = f32_to_bf16(ldexpf(acc[rt][v], c.sexp - c.s_exp[row - c.p0]));
      if constexpr (kTileMx<AbsT>)
        if (c.col_nan) out = 0x7fc0u;  // a NaN scale reaches every output of the row
      g.y[(size_t)row * c.N + c.n] = out;
    }
  }
}

template <typename AbsT>
__global__ __launch_bounds__(kThreads, 1) void tile_kernel(TileKArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 s_x[2][kPassRows * kLdsRow];
  __shared__ int s_src[kPassRows];
  __shared__ int s_exp[kPassRows];

  // XCD-aware order: consecutive work items land on one XCD.
  const int nb = gridDim.x;
  const int b = blockIdx.x;
  const int work = (b & 7) * (nb >> 3) + (b >> 3);
  if (work >= a.n_work) return;
  const int nt = work % a.n_tiles;
  GroupRef gr;
  if (!find_group(a.g.sizes, a.g.ids, a.g.G, a.g.E, a.g.M, a.g.rows_min_tile, INT_MAX,
                  work / a.n_tiles, gr))
    return;
  const int e = gr.expert;
  const int r_begin = gr.row;
  const int r_end = min(r_begin + gr.size, a.g.M);
  if (r_begin >= r_end) return;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;

  const int N = a.g.N, K = a.g.K;
  const int i = lane & 31, h = lane >> 5;
  const int n_wave = nt * kTileN + wave * 32;
  const size_t row_bytes = (size_t)K / 2;
  const int bpr = K / kBlock;
  const uint8_t* wexp = a.g.packed + (size_t)e * N * row_bytes;
  const int spr = kTileMx<AbsT> ? 2 * bpr : bpr;  // scales per weight row
  const AbsT* aexp = static_cast<const AbsT*>(a.g.absmax) + (size_t)e * N * spr;

  // staged row of output row `row`: its token's row when the rows were
  // staged per token (fused gather; an invalid slot reads the zero row),
  // else the row itself
  auto staged_row = [&](int row) -> int {
    if (!a.st.by_token) return row;
    const int slot = a.g.slots[row];
    return (slot >= 0 && slot < a.g.T * a.g.slot_div) ? div_slot(slot, a.g.slot_div) : a.st.rows;
  };
  // the first pass's staged rows are looked up now, so their latency
  // overlaps the absmax loads below
  const int src_first = tid < min(kPassRows, r_end - r_begin) ? staged_row(r_begin + tid) : a.st.rows;

  // per-row power-of-two scale from the row's largest block absmax
  const int n = n_wave + i;
  const bool n_ok = n < N;
  // (16 independent loads per round: an index past the row re-reads a block
  // of the same row, which leaves the maximum unchanged)
  int sexp = 0;
  bool col_nan = false;
  if constexpr (kTileMx<AbsT>) {
    // MXFP4: the row's largest E8M0 scale s_max; 2^-s_n = 2^-(s_max - 127)
    // puts every decoded value at or below 6 (fp16-safe)
    const uint8_t* ar = aexp + (n_ok ? (size_t)n * spr : 0);
    uint32_t mu[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) mu[u] = 0u;
    for (int b0 = h; b0 < spr; b0 += 32) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int b = b0 + 2 * u;
        mu[u] = max(mu[u], (uint32_t)ar[b < spr ? b : h]);
      }
    }
    uint32_t mx = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) mx = max(mx, mu[u]);
    if (!n_ok) mx = 0;
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, kWave));
    sexp = (int)mx - 127;
    col_nan = mx == 255u;
  } else {
    float m = 0.0f;
    {
      const AbsT* ar = aexp + (n_ok ? (size_t)n * bpr : 0);
      float mu[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) mu[u] = 0.0f;
      for (int bk0 = h; bk0 < bpr; bk0 += 32) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int bk = bk0 + 2 * u;
          mu[u] = fmaxf(mu[u], absmax_at(ar, bk < bpr ? bk : h));
        }
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) m = fmaxf(m, mu[u]);
      if (!n_ok) m = 0.0f;
    }
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    // m = f * 2^sexp with f in [0.5, 1): m * 2^-(sexp - 15) lies in [2^14, 2^15)
    (void)frexpf(m, &sexp);
    sexp -= 15;
  }

  PassCtx c;
  c.a = &a;
  c.s_x = &s_x[0][0];
  c.s_src = s_src;
  c.s_exp = s_exp;
  c.wrow = wexp + (n_ok ? (size_t)n * row_bytes : 0);
  c.arow = aexp + (n_ok ? (size_t)n * spr : 0);
  c.n_ok = n_ok;
  c.sexp = sexp;
  c.col_nan = col_nan;
  c.tid = tid;
  c.i = i;
  c.h = h;
  c.N = N;
  c.K = K;
  c.bpr = bpr;
  c.n = n;
  c.r_end = r_end;
  c.n_steps = K / kStepK;
  c.rem_k = K - c.n_steps * kStepK;  // a final 64-wide step when K % 128 == 64
  for (int p0 = r_begin; p0 < r_end; p0 += kPassRows) {
    c.p0 = p0;
    c.rows = min(kPassRows, r_end - p0);
    // the pass's staged rows (looked up ahead for the first pass) and their
    // exponents; rows past the group read the zero row
    if (tid < kPassRows) {
      int src = a.st.rows;
      if (tid < c.rows) src = p0 == r_begin ? src_first : staged_row(p0 + tid);
      s_src[tid] = src;
      s_exp[tid] = a.g.row_exp[src];
    }
    __syncthreads();
    switch ((c.rows + 31) / 32) {
      case 1: tile_pass<1, AbsT>(c); break;
      case 2: tile_pass<2, AbsT>(c); break;
      case 3: tile_pass<3, AbsT>(c); break;
      case 4: tile_pass<4, AbsT>(c); break;
      default: tile_pass<5, AbsT>(c); break;
    }
    __syncthreads();  // the next pass reuses the LDS buffers
  }
}

// ------------------------------------------------------------------ dgrad
// Matrix-core dgrad, dx[r, k] = sum_n dy[r, n] W[n, k] per group (page
// "grouped-nf4-gemm", "Owns": the grouped packed GEMM and its dgrad).  The
// contraction runs over N, across the rows of each expert's K-contiguous
// codes, so the decoded weights are written to LDS transposed, [k][n], and
// read back as MFMA operands of 8 consecutive n.  A workgroup of 8
// wavefronts owns (group, 256 columns of K) and walks N in steps of 64; each
// wavefront owns 32 of the columns for every row of the group (up to 5 row
// tiles of 32 per pass), so each code is decoded once per pass.
//  * weights: lane l of wavefront w loads the 16 bytes (32 codes, one
//    64-code absmax block) at row n0 + l, columns k0 + 32 w, and decodes them
//    through the fp16 table of fp16(level * absmax * 2^-S), one rounding,
//    where 2^-S puts the largest block absmax of that 64-column block over
//    all N rows into [2^14, 2^15) (the contraction mixes rows, so the scale
//    is per output column, applied exactly in the epilogue);
//  * dy: the rows as stage_x_kernel staged them (fp16 times each row's 2^t_r,
//    natural order, rows padded to a multiple of 128 with zeros; absent rows
//    read the zero row);
//  * fp32 accumulation on v_mfma_f32_32x32x16_f16, dx = acc * 2^(S - t_r)
//    rounded once to bf16.
// Every block whose absmax lies within 2^25 of its column block's largest
// decodes to normal fp16 numbers, the forward tile path's range with the
// roles of rows and columns exchanged.
constexpr int kDgThreads = 512;    // 8 wavefronts (two per SIMD), 32 output columns each
constexpr int kDgTileK = 256;      // output columns (of K) per workgroup
constexpr int kDgBlocks = kDgTileK / kBlock;  // absmax blocks a tile's columns span
constexpr int kDgStepN = 64;       // rows of W (contraction) per step
constexpr int kDgRowTiles = 5;     // 32-row MFMA tiles per pass
constexpr int kDgPassRows = 32 * kDgRowTiles;
constexpr int kDgLds = kDgStepN + 8;  // fp16 per LDS row: 144 bytes, conflict-free reads
static_assert(kStageAlign % kDgStepN == 0, "staged dy rows cover every step of N");

struct DgradTileKArgs {
  DgradArgs d;
  const int32_t* row_exp;  // [M + 1] exponents of the staged dy rows
  const uint16_t* dyh;     // [M + 1, ld] staged dy rows, row M all zeros
  int ld;
  int rows_min;
  int k_tiles;
  int n_work;  // group slots * k_tiles
};

struct DgPassCtx {
  const DgradTileKArgs* a;
  _Float16* s_w;   // [2][kDgTileK * kDgLds], [k][n]
  _Float16* s_dy;  // [2][kDgPassRows * kDgLds], [row][n]
  const int* s_exp;
  const uint8_t* wexp;
  const void* aexp;
  int sexp;        // this wavefront's column-block exponent S
  int tid, wave, lane, i, h, N, K, bpr, k0, p0, rows;
};

template <int RT, typename AbsT>
__device__ __forceinline__ void dgrad_pass(const DgPassCtx& c) {
  const DgradTileKArgs& a = *c.a;
  float16v acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[rt][v] = 0.0f;

  const int steps = (c.N + kDgStepN - 1) / kDgStepN;
  const size_t row_bytes = (size_t)c.K / 2;
  const int kk = c.k0 + 32 * c.wave;  // this wavefront's first code column
  const bool k_ok = kk < c.K;
  // 16-byte dy chunks per thread: RT * 32 rows x 8 chunks over the threads
  constexpr int kChunks = (RT * 256 + kDgThreads - 1) / kDgThreads;
  const uint16_t* ysrc[kChunks];
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const int q = c.tid + kDgThreads * j;
    const int row = q >> 3;
    const int src = (q < RT * 256 && row < c.rows) ? c.p0 + row : a.d.M;
    ysrc[j] = a.dyh + (size_t)src * a.ld + 8 * (q & 7);
  }
  uint4 wr;
  float war;
  u32x4 yr[kChunks];
  // Loads of step s are issued at the top of step s - 1 and consumed (staged
  // into LDS) at its end, so no loaded register lives across the loop's
  // back edge.
  auto load = [&](int step) {
    const int n = step * kDgStepN + c.lane;
    const bool ok = k_ok && n < c.N;
    wr = *reinterpret_cast<const uint4*>(c.wexp + (ok ? (size_t)n * row_bytes + kk / 2 : 0));
    war = absmax_at(static_cast<const AbsT*>(c.aexp) + (ok ? (size_t)n * c.bpr : 0),
                    ok ? kk / kBlock : 0);
#pragma unroll
    for (int j = 0; j < kChunks; ++j)
      yr[j] = *reinterpret_cast<const u32x4*>(ysrc[j] + step * kDgStepN);
  };
  auto stage = [&](int buf, int step) {
    const int n = step * kDgStepN + c.lane;
    const bool ok = k_ok && n < c.N;
    const Table tab = make_table(ok ? ldexpf(war, -c.sexp) : 0.0f);
    _Float16* sw = c.s_w + buf * (kDgTileK * kDgLds) + c.lane;
    const uint32_t dw[4] = {wr.x, wr.y, wr.z, wr.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // slot order of decode8: codes {0, 2, 4, 6, 1, 3, 5, 7} of the dword
      const half8 v = decode8(dw[q], tab);
      const int kc = 32 * c.wave + 8 * q;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kcode = e < 4 ? 2 * e : 2 * (e - 4) + 1;
        sw[(kc + kcode) * kDgLds] = v[e];
      }
    }
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int q = c.tid + kDgThreads * j;
      if (kChunks * kDgThreads > RT * 256 && q >= RT * 256) break;
      *reinterpret_cast<u32x4*>(
          &c.s_dy[buf * (kDgPassRows * kDgLds) + (q >> 3) * kDgLds + 8 * (q & 7)]) = yr[j];
    }
  };

  load(0);
  stage(0, 0);
  __syncthreads();
  for (int step = 0; step < steps; ++step) {
    const int buf = step & 1;
    const bool more = step + 1 < steps;
    if (more) load(step + 1);
    const _Float16* sw = c.s_w + buf * (kDgTileK * kDgLds) + (32 * c.wave + c.i) * kDgLds + 8 * c.h;
    const _Float16* sy = c.s_dy + buf * (kDgPassRows * kDgLds) + c.i * kDgLds + 8 * c.h;
#pragma unroll
    for (int sub = 0; sub < kDgStepN / 16; ++sub) {
      const half8 bw = *reinterpret_cast<const half8*>(sw + 16 * sub);
      half8 ax[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        ax[rt] = *reinterpret_cast<const half8*>(sy + rt * 32 * kDgLds + 16 * sub);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ax[rt], bw, acc[rt], 0, 0, 0);
    }
    if (more) stage(1 - buf, step + 1);
    __syncthreads();
  }

  // epilogue: D[row][col], col = lane % 32, row = 8 (v / 4) + 4 h + v % 4
  const int k = kk + c.i;
  if (!k_ok || k >= c.K) return;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = rt * 32 + 8 * (v >> 2) + 4 * c.h + (v & 3);
      if (row >= c.rows) continue;
      a.d.dx[(size_t)(c.p0 + row) * c.K + k] =
          f32_to_bf16(ldexpf(acc[rt][v], c.sexp - c.s_exp[row]));
    }
}

template <typename AbsT>
__global__ __launch_bounds__(kDgThreads, 1) void dgrad_tile_kernel(DgradTileKArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 s_w[2 * kDgTileK * kDgLds];
  __shared__ __attribute__((aligned(16))) _Float16 s_dy[2 * kDgPassRows * kDgLds];
  __shared__ int s_exp[kDgPassRows];
  __shared__ float s_max[kDgBlocks][kDgThreads / kWave];

  // XCD-aware order: consecutive work items land on one XCD.
  const int nb = gridDim.x;
  const int b = blockIdx.x;
  const int work = (b & 7) * (nb >> 3) + (b >> 3);
  if (work >= a.n_work) return;
  const int kt = work % a.k_tiles;
  GroupRef gr;
  if (!find_group(a.d.sizes, a.d.ids, a.d.G, a.d.E, a.d.M, a.rows_min, INT_MAX, work / a.k_tiles,
                  gr))
    return;
  const int e = gr.expert;
  const int r_begin = gr.row;
  const int r_end = min(r_begin + gr.size, a.d.M);
  if (r_begin >= r_end) return;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int N = a.d.N, K = a.d.K, bpr = K / kBlock;
  const int k0 = kt * kDgTileK;
  const int kb0 = k0 / kBlock;  // the tile's absmax blocks: kb0 .. kb0 + 3
  const AbsT* aexp = static_cast<const AbsT*>(a.d.absmax) + (size_t)e * N * bpr;

  // column-block scales: the largest absmax of each of the tile's blocks
  // over all N rows (8 rows per round per thread, all loads issued before
  // any is used; a row past N re-reads row n0, a block past K block kb0)
  float mb[kDgBlocks];
#pragma unroll
  for (int q = 0; q < kDgBlocks; ++q) mb[q] = 0.0f;
  for (int n0 = tid; n0 < N; n0 += 8 * kDgThreads) {
    float v[8][kDgBlocks];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int n = n0 + u * kDgThreads;
      const AbsT* ar = aexp + (size_t)(n < N ? n : n0) * bpr;
#pragma unroll
      for (int q = 0; q < kDgBlocks; ++q) v[u][q] = absmax_at(ar, kb0 + q < bpr ? kb0 + q : kb0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int q = 0; q < kDgBlocks; ++q) mb[q] = fmaxf(mb[q], v[u][q]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
    for (int q = 0; q < kDgBlocks; ++q) mb[q] = fmaxf(mb[q], __shfl_xor(mb[q], o, kWave));
  if (lane == 0)
#pragma unroll
    for (int q = 0; q < kDgBlocks; ++q) s_max[q][wave] = mb[q];
  __syncthreads();
  // wavefront w owns columns k0 + 32 w .. + 31, inside block kb0 + w / 2
  float m = 0.0f;
#pragma unroll
  for (int w = 0; w < kDgThreads / kWave; ++w) m = fmaxf(m, s_max[wave >> 1][w]);
  // m = f * 2^sexp with f in [0.5, 1): m * 2^-(sexp - 15) lies in [2^14, 2^15)
  int sexp = 0;
  (void)frexpf(m, &sexp);
  sexp -= 15;

  DgPassCtx c;
  c.a = &a;
  c.s_w = s_w;
  c.s_dy = s_dy;
  c.s_exp = s_exp;
  c.wexp = a.d.packed + (size_t)e * N * ((size_t)K / 2);
  c.aexp = aexp;
  c.sexp = sexp;
  c.tid = tid;
  c.wave = wave;
  c.lane = lane;
  c.i = lane & 31;
  c.h = lane >> 5;
  c.N = N;
  c.K = K;
  c.bpr = bpr;
  c.k0 = k0;
  for (int p0 = r_begin; p0 < r_end; p0 += kDgPassRows) {
    c.p0 = p0;
    c.rows = min(kDgPassRows, r_end - p0);
    if (tid < kDgPassRows) s_exp[tid] = tid < c.rows ? a.row_exp[p0 + tid] : 0;
    __syncthreads();
    switch ((c.rows + 31) / 32) {
      case 1: dgrad_pass<1, AbsT>(c); break;
      case 2: dgrad_pass<2, AbsT>(c); break;
      case 3: dgrad_pass<3, AbsT>(c); break;
      case 4: dgrad_pass<4, AbsT>(c); break;
      default: dgrad_pass<5, AbsT>(c); break;
    }
    __syncthreads();  // the next pass reuses the LDS buffers
  }
}

// Activation staging for the matrix-core kernels, one wavefront per staged
// row.  The row's source is x's own row (token rows, or rows without a
// gather), or for an output row read through the fused gather its token's
// row (an invalid slot, like the extra last row, stages zeros).  From the
// largest |x| -- taken on the bf16 bit patterns, whose magnitude order is
// integer order -- and e, its biased exponent, t = 141 - e puts that
// largest value times 2^t in [2^14, 2^15) (a row of zeros gets t = 0).
// Every value is then written as fp16(x * 2^t): x * 2^t is exact in fp32,
// and exact in fp16 down to 2^-14, i.e. for every value within 2^28 of the
// row's largest; smaller ones round to fp16's subnormals (nearest, ties to
// even).  Elements past the row's end up to the padded width are zeros.
// Rows are read 16 bytes at a time when every row starts 16-byte aligned
// (K % 8 == 0 and an aligned x), else element by element (a dgrad's dy of
// any width N).  Beside a decode launch (groups of up to 8 rows there, the
// larger ones here) the staging first looks at the group sizes and, when no
// group has enough rows for the tile kernel to take it, stages nothing: the
// tile kernel then finds no group and reads no staged row.
constexpr int kStageThreads = 256;
constexpr int kStageGateMaxGroups = 4096;  // sizes scanned per wavefront at most

struct StageKArgs {
  const uint16_t* x;
  const int32_t* slots;  // read per output row when the rows are not token rows
  int slot_div, T;
  int rows;              // staged rows; row `rows` is the zero row
  bool gather_rows;      // rows are output rows read through `slots`
  int K, ld;
  bool natural;          // natural K order (else the NF4 decode's slot order)
  bool vec;              // 16-byte row loads (K % 8 == 0, x 16-byte aligned)
  const int32_t* gate_sizes;  // non-null: stage only if some gate_sizes[g] >= gate_min
  int gate_G, gate_min;
  uint16_t* xh;
  int32_t* row_exp;
};

__device__ __forceinline__ uint32_t f16x2_rne(float lo, float hi) {
  const _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Elements 8c .. 8c + 7 of a row as four bf16 pairs, zeros past element K.
__device__ __forceinline__ uint4 load8(const uint16_t* row, int c, int K, bool vec) {
  if (vec) return reinterpret_cast<const uint4*>(row)[c];
  uint32_t d[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 8 * c + 2 * j;
    const uint32_t lo = e < K ? row[e] : 0u;
    const uint32_t hi = e + 1 < K ? row[e + 1] : 0u;
    d[j] = lo | (hi << 16);
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

__global__ __launch_bounds__(kStageThreads) void stage_x_kernel(StageKArgs s) {
  const int lane = threadIdx.x % kWave;
  const int waves = gridDim.x * (kStageThreads / kWave);
  const int chunks = (s.K + 7) / 8;
  if (s.gate_sizes) {
    bool hit = false;
    for (int g = lane; g < s.gate_G; g += kWave) hit = hit || s.gate_sizes[g] >= s.gate_min;
    if (__builtin_amdgcn_ballot_w64(hit) == 0) return;  // the same answer in every wavefront
  }
  for (int r = blockIdx.x * (kStageThreads / kWave) + threadIdx.x / kWave; r <= s.rows;
       r += waves) {
    int src = r < s.rows ? r : -1;
    if (s.gather_rows && src >= 0) {
      const int slot = s.slots[r];
      src = (slot >= 0 && slot < s.T * s.slot_div) ? slot / s.slot_div : -1;
    }
    const uint16_t* row = s.x + (size_t)(src >= 0 ? src : 0) * s.K;
    uint32_t mb = 0;
    if (src >= 0) {
      for (int c0 = lane; c0 < chunks; c0 += 4 * kWave) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int cc = c0 + u * kWave;
          v[u] = load8(row, cc < chunks ? cc : lane % chunks, s.K, s.vec);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t d[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            mb = max(mb, max(d[q] & 0x7fffu, (d[q] >> 16) & 0x7fffu));
        }
      }
    }
    mb = wave_max_u32(mb);
    const int t = mb == 0 ? 0 : 141 - (int)(mb >> 7);
    uint4* out = reinterpret_cast<uint4*>(s.xh + (size_t)r * s.ld);
    for (int c = lane; c < s.ld / 8; c += kWave) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (src >= 0 && c < chunks) v = load8(row, c, s.K, s.vec);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
      float f[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[2 * j] = ldexpf(__uint_as_float(d[j] << 16), t);
        f[2 * j + 1] = ldexpf(__uint_as_float(d[j] & 0xffff0000u), t);
      }
      uint4 o;
      if (s.natural) {
        o = make_uint4(f16x2_rne(f[0], f[1]), f16x2_rne(f[2], f[3]), f16x2_rne(f[4], f[5]),
                       f16x2_rne(f[6], f[7]));
      } else {
        // the NF4 decode's slot order: elements {0, 2, 4, 6, 1, 3, 5, 7}
        o = make_uint4(f16x2_rne(f[0], f[2]), f16x2_rne(f[4], f[6]), f16x2_rne(f[1], f[3]),
                       f16x2_rne(f[5], f[7]));
      }
      out[c] = o;
    }
    if (lane == 0) s.row_exp[r] = t;
  }
}

}  // namespace

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t stage_bytes(int64_t rows, int64_t width) {
  const int64_t ld = (width + kStageAlign - 1) / kStageAlign * kStageAlign;
  return align256((size_t)(rows + 1) * sizeof(int32_t)) +
         align256((size_t)(rows + 1) * (size_t)ld * sizeof(uint16_t));
}

// With the gather fused, token rows repeat top_k times among the M rows: they
// are staged once per token (T <= M entries fit the workspace sized for M).
StagePlan plan_stage(const GemmArgs& g) {
  StagePlan p;
  p.by_token = g.slots != nullptr && g.T <= g.M;
  p.rows = p.by_token ? g.T : g.M;
  p.ld = (g.K + kStageAlign - 1) / kStageAlign * kStageAlign;
  return p;
}

hipError_t launch_stage_x(const GemmArgs& g, const StagePlan& p, bool natural_order,
                          hipStream_t stream) {
  StageKArgs s;
  s.x = g.x;
  s.slots = g.slots;
  s.slot_div = g.slot_div;
  s.T = g.T;
  s.rows = p.rows;
  s.gather_rows = g.slots != nullptr && !p.by_token;
  s.K = g.K;
  s.ld = p.ld;
  s.natural = natural_order;
  s.vec = g.K % 8 == 0 && reinterpret_cast<uintptr_t>(g.x) % 16 == 0;
  // the tile kernel takes groups of rows_min_tile rows or more; with
  // rows_min_tile <= 1 it takes every group and the staging always runs
  const bool gate = g.rows_min_tile > 1 && g.G <= kStageGateMaxGroups;
  s.gate_sizes = gate ? g.sizes : nullptr;
  s.gate_G = g.G;
  s.gate_min = g.rows_min_tile;
  s.xh = g.xh;
  s.row_exp = g.row_exp;
  const int per_block = kStageThreads / kWave;
  const int cap = device_cu_count() * 8;
  int blocks = (p.rows + 1 + per_block - 1) / per_block;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(stage_x_kernel, dim3(blocks), dim3(kStageThreads), 0, stream, s);
  return hipGetLastError();
}

hipError_t launch_tile(const GemmArgs& g, hipStream_t stream) {
  TileKArgs a;
  a.g = g;
  a.st = plan_stage(g);
  a.n_tiles = (g.N + kTileN - 1) / kTileN;
  a.n_work = (int)group_slots(g.G, g.M, g.rows_min_tile) * a.n_tiles;
  const int grid = ((a.n_work + 7) / 8) * 8;
  if (grid == 0) return hipSuccess;
  if (g.mxfp4)
    hipLaunchKernelGGL(tile_kernel<uint8_t>, dim3(grid), dim3(kThreads), 0, stream, a);
  else if (g.abs_bf16)
    hipLaunchKernelGGL(tile_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(tile_kernel<float>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dgrad_tile(const DgradArgs& d, const int32_t* row_exp, const uint16_t* dyh,
                             int ld, int rows_min, hipStream_t stream) {
  DgradTileKArgs a;
  a.d = d;
  a.row_exp = row_exp;
  a.dyh = dyh;
  a.ld = ld;
  a.rows_min = rows_min;
  a.k_tiles = (d.K + kDgTileK - 1) / kDgTileK;
  a.n_work = (int)group_slots(d.G, d.M, rows_min) * a.k_tiles;
  const int grid = ((a.n_work + 7) / 8) * 8;
  if (grid == 0) return hipSuccess;
  if (d.abs_bf16)
    hipLaunchKernelGGL(dgrad_tile_kernel<uint16_t>, dim3(grid), dim3(kDgThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(dgrad_tile_kernel<float>, dim3(grid), dim3(kDgThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gnf4
