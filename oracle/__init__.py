"""CPU oracle for the grouped NF4 expert GEMM path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use it.  It shares no code, tables or helpers with the HIP
library; both sides embed the NormalFloat4 literals independently.

Everything here is plain numpy, computed in fp64 where the method is floating
point, written to be checked against the pages by eye rather than to be fast.

What the oracle computes, and the passage each step follows:

* ``nf4``   -- the 16-entry NormalFloat4 code table, blockwise absmax
  quantisation to 4-bit codes, byte packing and the fp32 LUT decode.
  Page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE expert
  stacks" (the 0.1.0 README), opening section: the `[E, N, K/2]` uint8 stack
  with fp32 blockwise absmax, LUT decode to fp32 in registers, in the
  conventions of the bitsandbytes gemm_4bit family.  The code values
  themselves come from the QLoRA paper (Dettmers et al., 2023), section 3,
  "4-bit NormalFloat Quantization".
* ``route`` -- per-token top-k with softmax weights and the token->expert
  sort that yields ``(sizes, expert_ids)``.  Same page, opening section
  ("supplied after the usual token->expert sort"); the router softmax/top-k
  is one of the glue kernels listed under "Owns" on the "grouped-nf4-gemm"
  landing page.
* ``gemm``  -- the grouped expert GEMM in fp64 over the decoded weights.
  Same README, opening section and "The claim" (fp32 accumulation, bf16
  epilogue, one launch for all active experts); and its dgrad (the
  activation gradient over the same packed stack, landing page "Owns").
* ``mxfp4`` -- the grouped GEMM over MXFP4 stacks (E2M1 codes with E8M0
  scales per 32 elements), the second packed format the landing page's
  grouped GEMM serves ("Owns", "Use this when"); the formats' definitions
  come from the OCP Microscaling specification.
* ``moe``   -- the steps on either side of the GEMM: the SwiGLU activation
  between the two expert projections and the weighted top-k combine after
  the down projection (landing page "grouped-nf4-gemm", "Owns" and "Use this
  when": decode glue kernels), and one MoE feed-forward layer composed from
  all the steps.

Readings where the pages are silent (block size 64 along K, first element in
the high nibble, ties to the lower code, top-k order and tie-break, stable
sort order) are stated in each function's docstring.

Parity pins: every function is pinned by tests under ``tests/test_oracle_*``
to something other than itself (the QLoRA quantile construction, exhaustive
byte round trips, exact-rational brute force, closed forms, invariants).
"""

from .nf4 import (NF4_TABLE, ref_pack, ref_unpack, ref_codes, ref_quantize_block,
                  ref_byte_ratio_vs_bf16, ref_round_bf16)
from .route import ref_topk, ref_sort, ref_route_sort
from .gemm import ref_group_rows, ref_grouped_gemm, ref_grouped_gemm_entries, ref_grouped_dgrad
from .moe import ref_silu, ref_swiglu, ref_combine, ref_expert_projection, ref_moe_ffn
from .mxfp4 import (E2M1_TABLE, ref_e2m1_value, ref_e8m0_value, ref_mx_codes, ref_mx_unpack,
                    ref_grouped_gemm_mxfp4)

__all__ = [
    "NF4_TABLE", "ref_pack", "ref_unpack", "ref_codes", "ref_quantize_block",
    "ref_byte_ratio_vs_bf16", "ref_round_bf16",
    "ref_topk", "ref_sort", "ref_route_sort",
    "ref_group_rows", "ref_grouped_gemm", "ref_grouped_gemm_entries", "ref_grouped_dgrad",
    "ref_silu", "ref_swiglu", "ref_combine", "ref_expert_projection", "ref_moe_ffn",
    "E2M1_TABLE", "ref_e2m1_value", "ref_e8m0_value", "ref_mx_codes", "ref_mx_unpack",
    "ref_grouped_gemm_mxfp4",
]
