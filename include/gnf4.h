/*
 * gnf4.h -- C ABI of libgnf4: the grouped Mixture-of-Experts expert GEMM
 * (W4A16) computed directly on NF4-packed expert weights, for AMD Instinct
 * MI355X (gfx950).
 *
 * What is computed (page "grouped-nf4-gemm -- single-launch W4A16 GEMM over
 * fused NF4 MoE expert stacks", opening section): a stack of E expert weight
 * matrices, each [N, K], stored as NF4 -- an [E, N, K/2] uint8 array holding
 * two 4-bit codes per byte plus one fp32 absmax per 64-element block along K
 * -- is multiplied by bf16 activations that a token->expert sort has grouped
 * by expert and described with (sizes, expert_ids).  Every code is decoded
 * through the 16-entry NormalFloat4 table, scaled by its block absmax,
 * accumulated in fp32 and stored as bf16, in one launch for all active
 * experts; no dequantised copy of the weights is ever written.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers (memory from hipMalloc or a caching
 *    allocator built on it) unless stated otherwise.  A host pointer is
 *    refused with GNF4_ERR_NOT_DEVICE_PTR: there is no CPU path and nothing
 *    falls back silently (landing page "grouped-nf4-gemm", "Do not use this
 *    when": the grouped GEMM refuses CPU tensors).  The reference computation
 *    on the CPU is the oracle that ships with the tests, not this library.
 *  - bf16 values travel as their raw 16-bit patterns (uint16_t).
 *  - Arrays are dense and row-major.  Vector-loaded inputs (weights,
 *    activations, packed codes) must be 16-byte aligned; others 4-byte.
 *  - The caller owns every buffer, including workspace.  The library keeps
 *    no per-call state and never synchronises the host: each call enqueues
 *    kernels on `stream` (a hipStream_t; NULL = the default stream) and
 *    returns.  Results are valid once the stream has completed them.
 *  - Outputs must not alias inputs.  Calls on different streams may run
 *    concurrently; calls sharing a workspace must be ordered by the caller.
 *  - Status codes report host-checkable misuse synchronously.  Values that
 *    live on the device (group sizes, expert ids) are not read by the host:
 *    kernels skip a group whose size is <= 0 or whose expert id is outside
 *    [0, E), and never touch rows at or beyond M.
 *  - Opt-in validation: with GNF4_VALIDATE=1 in the environment (read at
 *    every call), each grouped GEMM and dgrad call first runs a check kernel
 *    on `stream`, waits for it (the call then synchronises the host with the
 *    stream, so this mode is for debugging, not for graph capture) and
 *    returns GNF4_ERR_INVALID_ARG without launching anything when a group
 *    size is negative, a non-empty group's expert id lies outside [0, E),
 *    the sizes sum past M, or (fused gather) a covered row's slot lies
 *    outside [0, T * top_k): everything a kernel would otherwise skip.
 */
#ifndef GNF4_H_
#define GNF4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gnf4_status {
  GNF4_OK = 0,
  GNF4_ERR_INVALID_ARG = 1,     /* null pointer, bad dimension, misalignment */
  GNF4_ERR_NOT_DEVICE_PTR = 2,  /* a pointer is not device memory */
  GNF4_ERR_UNSUPPORTED = 3,     /* a size beyond what the kernels support */
  GNF4_ERR_WORKSPACE = 4,       /* workspace missing or too small */
  GNF4_ERR_HIP = 5              /* a HIP runtime call failed; see gnf4_last_hip_error */
} gnf4_status;

typedef enum gnf4_dtype {
  GNF4_DTYPE_BF16 = 0,
  GNF4_DTYPE_F32 = 1
} gnf4_dtype;

/* Human-readable text for a status code (static storage). */
const char* gnf4_status_string(gnf4_status s);

/* hipError_t of the most recent GNF4_ERR_HIP returned on this host thread. */
int gnf4_last_hip_error(void);

/* Library version as "major.minor.patch" (static storage). */
const char* gnf4_version(void);

/*
 * gnf4_pack -- blockwise NF4 quantisation of an expert weight stack.
 *
 * Page "grouped-nf4-gemm -- single-launch W4A16 GEMM ...", opening section
 * (the [E, N, K/2] uint8 + fp32 blockwise absmax layout of the bitsandbytes
 * gemm_4bit family); "Cross-vendor projections" (3.56x smaller than bf16,
 * i.e. one fp32 absmax per 64 codes).  Code values: QLoRA (Dettmers et al.,
 * 2023), section 3, NormalFloat4.
 *
 *   w       [E, N, K] of `w_dtype` (bf16 bits or fp32), 16-byte aligned
 *   packed  [E, N, K/2] uint8 out: byte j of a row = (code[2j] << 4) | code[2j+1]
 *           (first element in the high nibble), 4-byte aligned
 *   absmax  [E, N, K/64] fp32 out: max |w| over each 64-element block
 *
 * For each block with absmax a > 0, the code of x is the index of the table
 * level nearest to x / a in exact arithmetic, ties to the lower index (the
 * comparison x > m_i * a against level midpoints m_i is done in fp64, where
 * it is exact).  A block with a == 0 stores code 7 (the exact zero level)
 * everywhere.  Inputs must be finite.  K must be a positive multiple of 64.
 * Errors: GNF4_ERR_INVALID_ARG (null pointer, E/N/K <= 0, K % 64 != 0, bad
 * dtype, misalignment), GNF4_ERR_NOT_DEVICE_PTR, GNF4_ERR_HIP.
 */
gnf4_status gnf4_pack(const void* w, int32_t w_dtype, int64_t E, int64_t N, int64_t K,
                      uint8_t* packed, float* absmax, void* stream);

/*
 * gnf4_pack_ex -- gnf4_pack with the absmax stored as fp32 (absmax_dtype =
 * GNF4_DTYPE_F32, the same as gnf4_pack) or as bf16 (GNF4_DTYPE_BF16: 4.25
 * bits per weight; page "How do I run a MoE whose experts do not fit in VRAM
 * ...", "Supported scope": the NF4 bake's --absmax-dtype f32|bf16).
 *
 *   absmax  [E, N, K/64] out: fp32, or bf16 bits (2-byte aligned)
 *
 * With bf16, each block's maximum |w| is rounded to bf16 (nearest, ties to
 * even, saturating at the largest finite bf16) and the codes are chosen
 * against that stored value: the nearest level to x / a_stored, ties to the
 * lower index, so decoding with the stored absmax follows the same rule.
 * The GEMM entry points below take the absmax dtype with the stack.
 */
gnf4_status gnf4_pack_ex(const void* w, int32_t w_dtype, int64_t E, int64_t N, int64_t K,
                         uint8_t* packed, void* absmax, int32_t absmax_dtype, void* stream);

/*
 * gnf4_route_sort -- router top-k with softmax weights, then the
 * token->expert sort that yields (sizes, expert_ids).
 *
 * Page "grouped-nf4-gemm -- single-launch W4A16 GEMM ...", opening section
 * ("(sizes, expert_ids) supplied after the usual token->expert sort");
 * landing page "grouped-nf4-gemm", "Use this when" (router softmax and
 * top-k as one decode-step glue launch).
 *
 *   logits            [T, E] fp32 router logits (finite; NaN is outside the contract)
 *   topk_ids          [T, top_k] int32 out: the top_k experts of each token,
 *                     by descending logit, equal logits to the lower id
 *   topk_w            [T, top_k] fp32 out: softmax over the top_k selected logits
 *   expert_offsets    [E + 1] int32 out: exclusive prefix sum of rows per expert
 *   sorted_slots      [T * top_k] int32 out: flat slots s = t * top_k + j grouped
 *                     by ascending expert id, ascending s inside an expert
 *                     (stable; row r of the grouped activations is token
 *                     sorted_slots[r] / top_k)
 *   slot_rows         [T * top_k] int32 out, optional (NULL: not written): the
 *                     grouped row of each flat slot, slot_rows[sorted_slots[r]]
 *                     == r; gnf4_combine reads it
 *   group_sizes       [E] int32 out: rows of each non-empty expert, in
 *                     ascending expert id; the tail after num_groups is zero
 *   group_expert_ids  [E] int32 out: the matching expert ids; tail zero
 *   num_groups        [1] int32 out: number of non-empty experts
 *   workspace         device scratch of gnf4_route_sort_workspace_size() bytes
 *                     (may be NULL when that size is 0)
 *
 * Limits: 0 <= T, 1 <= E <= 1024, 1 <= top_k <= min(E, 32).  T == 0 writes
 * zero offsets and zero groups.  Bit-exact, deterministic (no atomics decide
 * an order).  Errors: GNF4_ERR_INVALID_ARG, GNF4_ERR_UNSUPPORTED (E or top_k
 * above the limits), GNF4_ERR_NOT_DEVICE_PTR, GNF4_ERR_WORKSPACE, GNF4_ERR_HIP.
 */
size_t gnf4_route_sort_workspace_size(int64_t T, int64_t E, int32_t top_k);

gnf4_status gnf4_route_sort(const float* logits, int64_t T, int64_t E, int32_t top_k,
                            int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                            int32_t* sorted_slots, int32_t* slot_rows, int32_t* group_sizes,
                            int32_t* group_expert_ids, int32_t* num_groups,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * gnf4_route_gemm_one_token -- a batch-1 decode step's routing folded into
 * the grouped GEMM's launch: the route/sort of one token (every output as
 * gnf4_route_sort writes them for T = 1, bit for bit) and
 * y[j, :] = x[0, :] . dequant(W[e_j])^T for its picks e_j in ascending
 * expert id, in one launch.
 *
 * Landing page "grouped-nf4-gemm", "Use this when" (router softmax and top-k
 * folded into one decode-step launch); the GEMM as gnf4_grouped_gemm_gather
 * with T = 1.  Every workgroup ranks the logits itself (the same code as
 * gnf4_route_sort) and takes its expert from the picks; one writes the
 * route/sort outputs, which the down projection and gnf4_combine then read.
 *
 *   logits            [E] fp32 router logits of the token (finite)
 *   x                 [1, K] bf16 bits: the token's activations (16-byte aligned)
 *   packed, absmax    [E, N, K/2] uint8 and [E, N, K/64] fp32 or bf16 bits
 *                     (`absmax_dtype`)
 *   y                 [top_k, N] bf16 bits out: row j for the j-th pick in
 *                     ascending expert id (the grouped order)
 *   topk_ids ... num_groups: as gnf4_route_sort for T = 1 (slot_rows optional)
 *   workspace         device scratch of gnf4_route_gemm_one_token_workspace_size()
 *                     bytes for split-K partials (16-byte aligned); with
 *                     less the call runs unsplit
 *
 * Limits: 1 <= E <= 128 (GNF4_ERR_UNSUPPORTED above: at most two experts per
 * lane of the ranking wavefronts), 1 <= top_k <= min(E, 32) as
 * gnf4_route_sort,
 * K % 64 == 0, N * K/2 < 2^31.
 * Tolerance and determinism as gnf4_grouped_gemm.  Errors:
 * GNF4_ERR_INVALID_ARG, GNF4_ERR_NOT_DEVICE_PTR, GNF4_ERR_UNSUPPORTED,
 * GNF4_ERR_WORKSPACE, GNF4_ERR_HIP.
 */
size_t gnf4_route_gemm_one_token_workspace_size(int64_t E, int32_t top_k, int64_t N, int64_t K);

gnf4_status gnf4_route_gemm_one_token(const float* logits, int64_t E, int32_t top_k,
                                      const uint16_t* x, const uint8_t* packed,
                                      const void* absmax, int32_t absmax_dtype, int64_t N,
                                      int64_t K, uint16_t* y, int32_t* topk_ids, float* topk_w,
                                      int32_t* expert_offsets, int32_t* sorted_slots,
                                      int32_t* slot_rows, int32_t* group_sizes,
                                      int32_t* group_expert_ids, int32_t* num_groups,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * gnf4_moe_ffn_one_token -- one token's MoE expert feed-forward in one
 * launch: the route/sort of gnf4_route_gemm_one_token, then for each pick
 * e_j (ascending expert id, j < top_k)
 *   g = x . W1[e_j]^T          (W1: [E, 2I, H], gate rows 0..I-1, up rows I..2I-1)
 *   h[j, i] = bf16(silu(g[i]) * g[I + i]),  silu(v) = v / (1 + exp(-v))
 *   y[j, :] = bf16(h[j, :] . W2[e_j]^T)  (W2: [E, H, I])
 * with fp32 accumulation and the SwiGLU taken on the fp32 sums.
 *
 * Landing page "grouped-nf4-gemm": "Owns" (the grouped GEMM and the decode
 * glue kernels, SwiGLU among them) and "Use this when" (a decode step's small
 * operations in as few launches as possible); the projections as
 * gnf4_route_gemm_one_token and gnf4_grouped_gemm, the activation as
 * gnf4_swiglu.  The weighted combine stays a separate call (gnf4_combine
 * with y and slot_rows).  The down workgroups load their weights while the
 * gate_up workgroups run and wait, per pick, for that pick's h: no launch
 * separates the two projections.
 *
 *   logits            [E] fp32 router logits of the token (finite)
 *   x                 [H] bf16 bits, 16-byte aligned
 *   gate_up_packed, gate_up_absmax   [E, 2I, H/2] uint8, [E, 2I, H/64] absmax
 *   down_packed, down_absmax         [E, H, I/2] uint8, [E, H, I/64] absmax
 *                     (`absmax_dtype` for both; packed 16-byte aligned)
 *   h                 [top_k, I] bf16 bits out (16-byte aligned): row j the
 *                     SwiGLU of pick j
 *   y                 [top_k, H] bf16 bits out: row j the down projection of
 *                     pick j (the grouped order gnf4_combine reads)
 *   topk_ids ... num_groups: as gnf4_route_sort for T = 1 (slot_rows optional)
 *   workspace         device memory of gnf4_moe_ffn_one_token_workspace_size()
 *                     bytes (4-byte aligned): per-pick counters and flags that
 *                     MUST be zero before the first call (hipMemset once);
 *                     every call that completes normally leaves all of it zero
 *                     again, so one workspace serves any number of calls on
 *                     one stream.  Calls sharing a workspace must not overlap.
 *                     A nonzero word after a call means a wait ran out (an
 *                     error word is set and never cleared): that call's
 *                     outputs are not to be trusted.
 *
 * Limits: as gnf4_route_gemm_one_token (E <= 128, top_k <= min(E, 32)),
 * H % 64 == 0, I % 64 == 0; the fused kernel exists for the role shapes of
 * the OLMoE and Qwen3-30B expert layers, and only where all of its
 * workgroups fit on the device at once (GPT-OSS-120B's do not).
 * gnf4_moe_ffn_one_token_supported() says whether a shape is served;
 * otherwise GNF4_ERR_UNSUPPORTED, and the three steps run as separate calls.
 * Tolerance and determinism as gnf4_grouped_gemm for each projection.
 * Errors: GNF4_ERR_INVALID_ARG, GNF4_ERR_NOT_DEVICE_PTR, GNF4_ERR_UNSUPPORTED,
 * GNF4_ERR_WORKSPACE, GNF4_ERR_HIP.
 */
size_t gnf4_moe_ffn_one_token_workspace_size(int32_t top_k);

int gnf4_moe_ffn_one_token_supported(int64_t E, int32_t top_k, int64_t H, int64_t I);

gnf4_status gnf4_moe_ffn_one_token(const float* logits, int64_t E, int32_t top_k,
                                   const uint16_t* x, const uint8_t* gate_up_packed,
                                   const void* gate_up_absmax, const uint8_t* down_packed,
                                   const void* down_absmax, int32_t absmax_dtype, int64_t H,
                                   int64_t I, uint16_t* h, uint16_t* y, int32_t* topk_ids,
                                   float* topk_w, int32_t* expert_offsets, int32_t* sorted_slots,
                                   int32_t* slot_rows, int32_t* group_sizes,
                                   int32_t* group_expert_ids, int32_t* num_groups,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * gnf4_gather_rows -- build the grouped activations from token rows:
 * x_sorted[r, :] = x[sorted_slots[r] / top_k, :] for r < M.
 *
 * Page "grouped-nf4-gemm -- single-launch W4A16 GEMM ...", opening section:
 * the GEMM consumes activations already grouped by the token->expert sort.
 *
 *   x             [T, K] bf16 bits (token activations), 16-byte aligned
 *   sorted_slots  [M] int32 flat slots as gnf4_route_sort writes them
 *   x_sorted      [M, K] bf16 bits out, 16-byte aligned
 *
 * A slot outside [0, T * top_k) leaves its row untouched.  K must be a
 * positive multiple of 64.  Errors: GNF4_ERR_INVALID_ARG,
 * GNF4_ERR_UNSUPPORTED, GNF4_ERR_NOT_DEVICE_PTR, GNF4_ERR_HIP.
 */
gnf4_status gnf4_gather_rows(const uint16_t* x, int64_t T, int64_t K, const int32_t* sorted_slots,
                             int32_t top_k, int64_t M, uint16_t* x_sorted, void* stream);

/*
 * gnf4_grouped_gemm_mxfp4 -- the grouped GEMM over an MXFP4 expert stack
 * (E2M1 codes with one E8M0 scale per 32 elements along K), served from the
 * checkpoint's own bytes: y = x . W[expert_ids[g]]^T per group.
 *
 * Landing page "grouped-nf4-gemm", "Owns" (the grouped packed GEMM over NF4
 * and native MXFP4) and "Use this when" (MoEs released as MXFP4 -- e2m1 +
 * e8m0 -- served without re-quantising).  Formats: OCP Microscaling.
 *
 *   x             [M, K] bf16 bits grouped by expert (sorted_slots NULL), or
 *                 [T, K] token rows read through sorted_slots (fused gather)
 *   packed        [E, N, K/2] uint8: E2M1 codes, element 2j in the LOW nibble
 *                 of byte j (16-byte aligned)
 *   scales        [E, N, K/32] uint8 E8M0: scale 2^(s - 127); 0xFF is NaN
 *   other arguments as in gnf4_grouped_gemm_gather / gnf4_grouped_gemm_ex,
 *   `path` included (0 auto: groups of up to 8 rows on the decode path, the
 *   rest on the matrix-core tile path);
 *   workspace     gnf4_grouped_gemm_workspace_size_ex(M, N, K, G, E, path,
 *                 split_k)
 *
 * Codes are decoded by gfx950's E2M1 convert.  Decode path: each 32-code
 * partial sum, accumulated in fp32, is multiplied by its block scale.  Tile
 * path: codes convert to fp16 scaled by 2^(s - s_max), s_max the largest
 * scale of the weight row (exact: powers of two), activations as in the NF4
 * tile path, fp32 MFMA accumulation, 2^(s_max - 127) applied at the end; a
 * weight row with a NaN scale gives NaN in every output of that column.
 * bf16 output within the GEMM's tolerance.
 * Limits and errors: as gnf4_grouped_gemm_gather (K % 64 == 0).
 */
gnf4_status gnf4_grouped_gemm_mxfp4(const uint16_t* x, int64_t T, const int32_t* sorted_slots,
                                    int32_t top_k, const uint8_t* packed, const uint8_t* scales,
                                    int64_t E, int64_t N, int64_t K, const int32_t* group_sizes,
                                    const int32_t* group_expert_ids, int64_t G, int64_t M,
                                    uint16_t* y, void* workspace, size_t workspace_bytes,
                                    int32_t path, int32_t split_k, void* stream);

/*
 * gnf4_grouped_dgrad -- the activation gradient of the grouped GEMM over the
 * same packed stack: dx[r, :] = dy[r, :] . dequant(W[expert_ids[g]]) for the
 * rows r of each group g.
 *
 * Landing page "grouped-nf4-gemm", "Owns" (the grouped packed GEMM and its
 * dgrad).  The contraction runs over N, across the rows of each expert's
 * K-contiguous [N, K/2] codes.
 *
 *   dy                [M, N] bf16 bits: output gradient, rows grouped as for
 *                     gnf4_grouped_gemm (2-byte aligned)
 *   packed, absmax    [E, N, K/2] uint8 and [E, N, K/64] fp32 or bf16 bits
 *                     (`absmax_dtype`, as gnf4_pack_ex writes them)
 *   group_sizes, group_expert_ids, G, M: as gnf4_grouped_gemm
 *   dx                [M, K] bf16 bits out; only rows covered by a valid
 *                     group are written
 *   workspace         device scratch of gnf4_grouped_dgrad_workspace_size()
 *                     bytes (16-byte aligned): the GEMV path's split-N fp32
 *                     partials (with less, that path runs unsplit: correct,
 *                     slower), or the tile path's staged dy rows (required:
 *                     4 (M + 1) bytes of exponents and an fp16 copy of
 *                     2 (M + 1) ceil128(N) bytes, each rounded up to 256)
 *
 * Two kernels meet one contract, |dx - exact| <= 8e-3 |exact| + 1e-3
 * rms(exact) per element, deterministic run to run:
 *  - GEMV path: fp32 decode and accumulation, splits of N summed in fixed
 *    order.  Every weight byte is read once per pass of up to 4 rows of dy,
 *    so it suits groups of few rows (decode-sized batches).
 *  - tile path (matrix cores): codes decoded once per 160 rows of a group
 *    into fp16 scaled by a power of two per 64-column block of K (putting
 *    its largest absmax over the N rows in [2^14, 2^15)), dy rows staged
 *    once in fp16 with a power of two per row (putting the row's largest in
 *    [2^14, 2^15)), fp16 x fp16 -> fp32 MFMA, the scales applied exactly at
 *    the end; any N, dy 2-byte aligned.  Range: a block
 *    whose absmax lies within 2^25 of its column block's largest, and a dy
 *    value within 2^28 of its row's largest, enter the product with fp16's
 *    full precision; values further down round to fp16 subnormals (and
 *    below 2^-24 of the staged scale, to zero).
 * gnf4_grouped_dgrad chooses automatically: the tile path for a batch
 * averaging at least 32 rows per group (M >= 32 min(G, M)), else the GEMV
 * path.
 * Limits: as gnf4_grouped_gemm, plus M * N < 2^31.
 * Errors: GNF4_ERR_INVALID_ARG, GNF4_ERR_NOT_DEVICE_PTR, GNF4_ERR_WORKSPACE
 * (tile path without room for its exponents), GNF4_ERR_UNSUPPORTED,
 * GNF4_ERR_HIP.
 */
size_t gnf4_grouped_dgrad_workspace_size(int64_t M, int64_t N, int64_t K, int64_t G, int64_t E);

gnf4_status gnf4_grouped_dgrad(const uint16_t* dy, const uint8_t* packed, const void* absmax,
                               int64_t E, int64_t N, int64_t K, const int32_t* group_sizes,
                               const int32_t* group_expert_ids, int64_t G, int64_t M,
                               uint16_t* dx, void* workspace, size_t workspace_bytes,
                               int32_t absmax_dtype, void* stream);

/*
 * gnf4_grouped_dgrad_ex -- gnf4_grouped_dgrad with the path choice exposed,
 * for tests and tuning.  `path`: 0 = automatic (as gnf4_grouped_dgrad),
 * 1 = GEMV path, 2 = tile path.  The workspace query takes the same
 * `path`.
 */
size_t gnf4_grouped_dgrad_workspace_size_ex(int64_t M, int64_t N, int64_t K, int64_t G,
                                            int64_t E, int32_t path);

gnf4_status gnf4_grouped_dgrad_ex(const uint16_t* dy, const uint8_t* packed, const void* absmax,
                                  int64_t E, int64_t N, int64_t K, const int32_t* group_sizes,
                                  const int32_t* group_expert_ids, int64_t G, int64_t M,
                                  uint16_t* dx, void* workspace, size_t workspace_bytes,
                                  int32_t absmax_dtype, int32_t path, void* stream);

/*
 * gnf4_swiglu -- the activation between the two expert projections:
 * h[r, i] = silu(gate_up[r, i]) * gate_up[r, I + i] for r < M, i < I, with
 * silu(g) = g / (1 + exp(-g)).
 *
 * Landing page "grouped-nf4-gemm", "Owns" (swiglu among the decode glue
 * kernels) and "Use this when" (the activation as one launch of the decode
 * step).  The pages do not fix the layout: the gate half comes first.
 *
 *   gate_up  [M, 2I] bf16 bits (the gate_up GEMM's output: gate, then up)
 *   h        [M, I] bf16 bits out
 *
 * Computed in fp32 from the bf16 inputs and rounded once to bf16 (round to
 * nearest even); |h - exact| <= 2^-8 |exact| per element for finite inputs.
 * 16-byte aligned rows with I % 8 == 0 take a vectorised path; any other
 * shape or alignment is also accepted.  Errors: GNF4_ERR_INVALID_ARG (null
 * pointer, M < 0, I <= 0, odd address), GNF4_ERR_UNSUPPORTED (M * I >= 2^40),
 * GNF4_ERR_NOT_DEVICE_PTR, GNF4_ERR_HIP.
 */
gnf4_status gnf4_swiglu(const uint16_t* gate_up, int64_t M, int64_t I, uint16_t* h,
                        void* stream);

/*
 * gnf4_combine -- the weighted top-k combine after the down projection:
 * out[t, :] = sum_{j < top_k} topk_w[t, j] * y[slot_rows[t * top_k + j], :].
 *
 * Landing page "grouped-nf4-gemm", "Owns" (combine among the decode glue
 * kernels) and "Use this when" (the top-k combine as one launch); page
 * "grouped-nf4-gemm -- single-launch W4A16 GEMM ...": routing weights are not
 * applied inside the expert GEMM, so they are applied here.
 *
 *   y          [M, H] bf16 bits: expert outputs in grouped (sorted) row order
 *              (may be NULL when M == 0)
 *   slot_rows  [T * top_k] int32: grouped row of each flat slot, as
 *              gnf4_route_sort writes it
 *   topk_w     [T, top_k] fp32 routing weights
 *   out        [T, H] bf16 bits out; every row is written
 *
 * The k terms of a token are accumulated in fp32 in ascending j (fixed
 * order, deterministic) and rounded once to bf16.  A slot whose row lies
 * outside [0, M) contributes nothing (a token with no rows gets zeros).
 * Errors: GNF4_ERR_INVALID_ARG (null pointer, T < 0, M < 0, H <= 0,
 * top_k < 1, misalignment), GNF4_ERR_UNSUPPORTED (T * top_k >= 2^31),
 * GNF4_ERR_NOT_DEVICE_PTR, GNF4_ERR_HIP.
 */
gnf4_status gnf4_combine(const uint16_t* y, const int32_t* slot_rows, const float* topk_w,
                         int64_t T, int32_t top_k, int64_t M, int64_t H, uint16_t* out,
                         void* stream);

/*
 * gnf4_grouped_gemm -- y = x_sorted . dequant(W[expert_ids[g]])^T per group,
 * every active expert in one pass.
 *
 * Page "grouped-nf4-gemm -- single-launch W4A16 GEMM ...", opening section
 * and "The claim" (LUT decode, blockwise fp32 absmax, fp32 accumulation,
 * bf16 epilogue, one launch for all active experts); "Layout" (a decode GEMV
 * path and an M-tile path); "Status / roadmap" (split-K for starved grids,
 * one universal launch rule instead of per-shape tables).
 *
 *   x_sorted          [M, K] bf16 bits, rows grouped by expert, 16-byte aligned
 *   packed, absmax    [E, N, K/2] uint8 and [E, N, K/64] fp32 (as gnf4_pack writes)
 *   group_sizes       [G] int32: rows of group g (contiguous, in group order)
 *   group_expert_ids  [G] int32: expert of group g (duplicates allowed)
 *   y                 [M, N] bf16 bits out; only rows covered by a valid group
 *                     are written, the rest keep their contents
 *   workspace         device scratch of gnf4_grouped_gemm_workspace_size() bytes,
 *                     16-byte aligned: the tile path's staged activation rows
 *                     (4 (M + 1) bytes of per-row exponents and an fp16 copy
 *                     of 2 (M + 1) ceil128(K) bytes, each rounded up to 256;
 *                     with the fused gather only T + 1 rows are used) and,
 *                     when the decode path splits K, its fp32 partials
 *
 * Group g covers rows [sum_{g'<g} max(size_g', 0), + size_g) clipped to M.
 * Routing weights are not applied here (the top-k combine is separate glue).
 * Two kernels implement the same arithmetic contract: a bandwidth-bound
 * decode path for groups with few rows (fp32 decode and multiply-add, optional
 * split-K with a fixed-order fp32 reduce) and a matrix-core tile path for
 * groups with many rows (a power-of-two scale per weight row putting its
 * largest block absmax in [2^14, 2^15), codes decoded with their block
 * absmax into fp16; each activation row staged once as fp16 times a power of
 * two putting its largest |x| in [2^14, 2^15); fp16 x fp16 -> fp32 MFMA).
 * Which one runs is a performance choice made from host-known sizes only;
 * both meet |y - exact| <= 8e-3 |exact| + 1e-3 rms(exact) per element.  The
 * decode path does so for any finite inputs.  The tile path's range: every
 * block whose absmax lies within 2^25 of its weight row's largest, and every
 * activation within 2^28 of its row's largest, enters the product with
 * fp16's full precision whatever the row's magnitude; smaller ones round to
 * fp16 subnormals (below 2^-24 of the staged scale, to zero), which matters
 * only when such values carry an output.  Results are deterministic run to
 * run.  The automatic choice: groups of up to 8 rows
 * take the decode path and larger ones the tile path, except that a batch
 * averaging at least 32 rows per group (M >= 32 min(G, M), prefill) runs
 * every group on the tile path and launches no decode kernel, and that with
 * the gather fused and T <= 8 tokens (a top-k routing then puts at most T
 * rows in a group) the decode path serves every group, of any size, and no
 * tile launch runs.
 *
 * Limits: M >= 0, G >= 0 (either 0: nothing to do), E, N >= 1, K >= 64 with
 * K % 64 == 0, N * K/2 and M * K below 2^31 elements per expert and call,
 * G < 65536.  The decode path keeps one K split of an activation row in LDS,
 * at most 319 chunks of 32 (K <= 10208 unsplit); a larger K is split across
 * workgroups, which needs the workspace.  Whenever the tile path may run
 * (M > 8 unless the gather is fused with T <= 8, or path 2 of the _ex form)
 * the workspace is required.
 * Errors: GNF4_ERR_INVALID_ARG, GNF4_ERR_NOT_DEVICE_PTR, GNF4_ERR_WORKSPACE
 * (workspace missing or smaller than the size query returns; also: K too
 * large to run unsplit and no workspace given),
 * GNF4_ERR_UNSUPPORTED (a limit above exceeded), GNF4_ERR_HIP.
 */
size_t gnf4_grouped_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t G, int64_t E);

gnf4_status gnf4_grouped_gemm(const uint16_t* x_sorted, const uint8_t* packed,
                              const float* absmax, int64_t E, int64_t N, int64_t K,
                              const int32_t* group_sizes, const int32_t* group_expert_ids,
                              int64_t G, int64_t M, uint16_t* y,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * gnf4_grouped_gemm_ex -- gnf4_grouped_gemm with the path choice exposed, for
 * tests and tuning, and the absmax stored as fp32 or bf16 (`absmax_dtype`,
 * as gnf4_pack_ex writes it; `absmax` then points to fp32 or bf16 bits).
 * `path`: 0 = automatic (same as gnf4_grouped_gemm),
 * 1 = every group on the decode path, 2 = every group on the tile path.
 * `split_k`: 0 = automatic, else the number of K splits of the decode path
 * (1..16; needs workspace of gnf4_grouped_gemm_workspace_size_ex();
 * GNF4_ERR_UNSUPPORTED if a split would hold more than 319 chunks of 32).
 * Results of all paths satisfy the same tolerance contract.
 */
size_t gnf4_grouped_gemm_workspace_size_ex(int64_t M, int64_t N, int64_t K, int64_t G,
                                           int64_t E, int32_t path, int32_t split_k);

gnf4_status gnf4_grouped_gemm_ex(const uint16_t* x_sorted, const uint8_t* packed,
                                 const void* absmax, int64_t E, int64_t N, int64_t K,
                                 const int32_t* group_sizes, const int32_t* group_expert_ids,
                                 int64_t G, int64_t M, uint16_t* y,
                                 void* workspace, size_t workspace_bytes,
                                 int32_t path, int32_t split_k, int32_t absmax_dtype,
                                 void* stream);

/*
 * gnf4_grouped_gemm_gather -- gnf4_gather_rows fused into the grouped GEMM:
 * output row r is x[sorted_slots[r] / top_k, :] . dequant(W[expert])^T, so
 * the grouped activations are never written out.
 *
 * Page "grouped-nf4-gemm -- single-launch W4A16 GEMM ...", opening section
 * (grouped rows "after the usual token->expert sort"); landing page
 * "grouped-nf4-gemm", "Use this when" (fold the decode step's small launches).
 *
 *   x             [T, K] bf16 bits: token activations (not grouped), 16-byte aligned
 *   sorted_slots  [M] int32 as gnf4_route_sort writes them; top_k >= 1
 *   other arguments (absmax_dtype included) as in gnf4_grouped_gemm_ex.
 *
 * Same arithmetic and tolerance as gnf4_grouped_gemm applied to the gathered
 * rows; a row whose slot lies outside [0, T * top_k) is not written.
 * Errors: as gnf4_grouped_gemm_ex, plus GNF4_ERR_INVALID_ARG for a null
 * sorted_slots or top_k < 1.
 */
gnf4_status gnf4_grouped_gemm_gather(const uint16_t* x, int64_t T, const int32_t* sorted_slots,
                                     int32_t top_k, const uint8_t* packed, const void* absmax,
                                     int64_t E, int64_t N, int64_t K, const int32_t* group_sizes,
                                     const int32_t* group_expert_ids, int64_t G, int64_t M,
                                     uint16_t* y, void* workspace, size_t workspace_bytes,
                                     int32_t path, int32_t split_k, int32_t absmax_dtype,
                                     void* stream);

/*
 * gnf4_grouped_gemm_gather_noalloc -- gnf4_grouped_gemm_gather for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The same kernels and
 * results (bit for bit) as gnf4_grouped_gemm_gather with a workspace of
 * gnf4_grouped_gemm_workspace_size_ex(M, N, K, G, E, path, split_k) bytes,
 * but the workspace (split-K partials, staged activation rows) is a
 * library-owned static array of GNF4_NOALLOC_SCRATCH_BYTES per GPU, which
 * each GPU the library runs on holds until the process ends.  The call
 * allocates nothing: no hipMalloc, no hipFree, no allocating library routine.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap on one GPU (different streams, or host
 * threads) race and must be ordered by the caller.  Nothing in the array
 * needs to start cleared.
 *
 * Arguments as gnf4_grouped_gemm_gather, without workspace.
 * Errors: as gnf4_grouped_gemm_gather, plus GNF4_ERR_UNSUPPORTED when the
 * call needs more workspace than GNF4_NOALLOC_SCRATCH_BYTES (for example a
 * prefill batch whose staged activation rows exceed it); GNF4_ERR_HIP if the
 * array's device address cannot be looked up.
 */
#define GNF4_NOALLOC_SCRATCH_BYTES (32u << 20)

size_t gnf4_noalloc_scratch_bytes(void);

gnf4_status gnf4_grouped_gemm_gather_noalloc(const uint16_t* x, int64_t T,
                                             const int32_t* sorted_slots, int32_t top_k,
                                             const uint8_t* packed, const void* absmax, int64_t E,
                                             int64_t N, int64_t K, const int32_t* group_sizes,
                                             const int32_t* group_expert_ids, int64_t G,
                                             int64_t M, uint16_t* y, int32_t path,
                                             int32_t split_k, int32_t absmax_dtype,
                                             void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* GNF4_H_ */
