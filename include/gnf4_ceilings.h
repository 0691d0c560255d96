/*
 * gnf4_ceilings.h -- C ABI of libgnf4_ceilings: the machine ceilings the
 * roofline fractions of libgnf4's kernels are read against, measured on the
 * GPU they run on (MI355X, gfx950).
 *
 * The pages ship a ceilings tool beside their kernel and a shape census
 * (page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE
 * expert stacks", sections "Layout" and "Regenerate the machine-generated
 * artifacts").  This library is that tool's device half: probe kernels,
 * each the simplest program that reaches (or, for the mixed matrix-core
 * loop, measures the share of) one limit.  It is not part
 * of the GEMM path and libgnf4 does not link it.
 *
 * Conventions: the same as gnf4.h.  Device pointers, caller-owned buffers,
 * one enqueue on `stream` (a hipStream_t; NULL = the default stream) per
 * call, no host synchronisation; status codes are gnf4_status values.
 */
#ifndef GNF4_CEILINGS_H_
#define GNF4_CEILINGS_H_

#include <stddef.h>
#include <stdint.h>

#include "gnf4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Pure read: every 16-byte word of buf[0, bytes) is loaded exactly once
 * (grid-stride, four independent loads in flight per thread) and XOR-folded;
 * block b writes the XOR of the words it read to block_xor[b], so the XOR of
 * all `blocks` outputs equals the XOR of the whole buffer (a check that every
 * word was read).  bytes: a positive multiple of 16, buf 16-byte aligned;
 * blocks in [1, 65536], 256 threads each; block_xor holds `blocks` uint32.
 * GNF4_ERR_INVALID_ARG otherwise, GNF4_ERR_HIP if the launch fails. */
gnf4_status gnf4_ceil_read(const void* buf, size_t bytes, int blocks, uint32_t* block_xor,
                           void* stream);

/* An empty kernel of `blocks` blocks of 64 threads (blocks in [1, 65536]):
 * the fixed cost of one launch. */
gnf4_status gnf4_ceil_empty(int blocks, void* stream);

/* Matrix-core loop: each wave of `blocks` blocks of 256 threads issues
 * `iters` x 4 v_mfma_f32_32x32x16_f16 instructions (four independent
 * accumulator chains; 32768 flops each) and records, around its loop, the
 * shader-clock counter (s_memtime) and the constant 100 MHz real-time
 * counter (s_memrealtime): stamps[4 * w + {0, 1, 2, 3}] = memtime start, end,
 * realtime start, end for global wave w (blocks * 4 waves, so stamps holds
 * 16 * blocks uint64).  The clock a wave ran at is
 *   (end - start of memtime) / ((end - start of realtime) / 100 MHz).
 * sink[t] receives thread t's accumulator sum (blocks * 256 floats), which
 * keeps the products live and is checkable: lane l of a wave supplies
 * A[l % 32][8 (l / 32) + j] = ((l + j) & 7) / 8 and
 * B[8 (l / 32) + j][l % 32] = ((3 l + j) & 7) / 16 for j < 8, so the 64
 * sums of one wave add up to 4 * iters * sum_k colsum_k(A) rowsum_k(B),
 * exactly while iters <= 256.  iters in [1, 2^24], blocks in [1, 65536]. */
gnf4_status gnf4_ceil_mfma(int iters, int blocks, uint64_t* stamps, float* sink, void* stream);

/* Matrix cores with work beside them: as gnf4_ceil_mfma, with five
 * independent accumulator chains per wave (iters x 5 MFMAs), and after each
 * MFMA `valu` dependent v_perm_b32 instructions (0, 4, 8 or 12: a decode-like
 * chain) and, with lds_reads = 1, one 16-byte LDS read per lane that is the
 * A operand of the same chain's next MFMA, five MFMAs later (a fragment read
 * a step ahead; fixed conflict-free addresses).  The ratio of
 * its TFLOP/s to gnf4_ceil_mfma's at the same clock is the share of the
 * matrix-core rate a wave keeps with that much other work per MFMA.  stamps
 * and sink as gnf4_ceil_mfma (sink values are not checkable here).
 * GNF4_ERR_INVALID_ARG for other valu / lds_reads values or the limits of
 * gnf4_ceil_mfma. */
gnf4_status gnf4_ceil_mfma_mix(int iters, int blocks, int valu, int lds_reads, uint64_t* stamps,
                               float* sink, void* stream);

/* Matrix cores beside VALU-only wavefronts: `blocks` blocks of 512 threads
 * (two waves per SIMD); waves 0..3 of a block issue iters x 5
 * v_mfma_f32_32x32x16_f16 (five chains), waves 4..7 issue iters x 5 x `valu`
 * dependent v_perm_b32 (valu 4, 8 or 12) and nothing else.  stamps as
 * gnf4_ceil_mfma for the blocks * 8 waves (32 * blocks uint64): the MFMA
 * waves' cycles per MFMA against 32 give their share of the matrix-core
 * rate with a VALU-only neighbour.  sink: blocks * 512 floats.
 * GNF4_ERR_INVALID_ARG for other valu values or the limits of
 * gnf4_ceil_mfma. */
gnf4_status gnf4_ceil_mfma_split(int iters, int blocks, int valu, uint64_t* stamps, float* sink,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif  /* GNF4_CEILINGS_H_ */
