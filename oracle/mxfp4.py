"""Grouped GEMM on MXFP4 expert stacks (e2m1 codes + e8m0 block scales), fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  * Landing page "grouped-nf4-gemm", "Owns" (the grouped packed GEMM over NF4
    and native MXFP4) and "Use this when" (serve MoEs whose experts are
    released as MXFP4, e2m1 + e8m0, from the checkpoint's own bytes, without
    re-quantising them).
  * The formats themselves come from the OCP Microscaling (MX) specification
    [outside the pages]: an MXFP4 block is 32 FP4 (E2M1) elements sharing one
    E8M0 scale.  E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit;
    exponent 0 is subnormal (0 or 0.5).  E8M0: an 8-bit exponent, value
    2^(s - 127); the all-ones byte is NaN.

Readings (the pages leave these open):
  * stack layout as the NF4 one: codes ``[E, N, K/2]`` uint8, two per byte,
    element 2j in the LOW nibble of byte j and 2j+1 in the high nibble (the
    order of the MXFP4 checkpoints the pages serve); scales ``[E, N, K/32]``
    uint8, one per 32 consecutive elements along K.
  * the GEMM: ``y[r, :] = x[r, :] @ W[e].T`` per group, as the NF4 GEMM.
"""

import numpy as np

from .gemm import ref_group_rows

MX_BLOCK = 32


def ref_e2m1_value(code):
    """Value of a 4-bit E2M1 code from its fields."""
    c = int(code) & 0xF
    sign = -1.0 if c & 0x8 else 1.0
    e = (c >> 1) & 0x3
    m = c & 0x1
    if e == 0:
        return sign * 0.5 * m            # subnormal: 0 or 0.5
    return sign * 2.0 ** (e - 1) * (1.0 + 0.5 * m)


E2M1_TABLE = np.array([ref_e2m1_value(c) for c in range(16)], dtype=np.float64)


def ref_e8m0_value(s):
    """Value of an E8M0 scale byte: 2^(s - 127), NaN for 0xFF."""
    s = np.asarray(s, dtype=np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def ref_mx_codes(packed):
    """Bytes -> codes ``[..., K]``, element 2j from the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    codes[..., 0::2] = p & 0x0F
    codes[..., 1::2] = p >> 4
    return codes


def ref_mx_unpack(packed, scales):
    """Decoded weights ``[..., N, K]`` in fp64: E2M1 value times the block's
    E8M0 scale (exact: products of small binary fractions and powers of two)."""
    codes = ref_mx_codes(packed)
    K = codes.shape[-1]
    s = np.asarray(scales)
    assert s.shape[-1] * MX_BLOCK == K
    return E2M1_TABLE[codes] * np.repeat(ref_e8m0_value(s), MX_BLOCK, axis=-1)


def ref_grouped_gemm_mxfp4(x_sorted, packed, scales, group_sizes, group_expert_ids):
    """The grouped GEMM over an MXFP4 stack; same group reading as the NF4
    oracle.  Returns ``(y fp64[M, N], written bool[M])``, unwritten rows NaN."""
    x = np.asarray(x_sorted, dtype=np.float32)
    M, K = x.shape
    E, N, half_k = packed.shape
    assert 2 * half_k == K
    y = np.full((M, N), np.nan, dtype=np.float64)
    written = np.zeros(M, dtype=bool)
    cache = {}
    for _g, e, r0, r1 in ref_group_rows(group_sizes, group_expert_ids, E, M):
        if e not in cache:
            cache[e] = ref_mx_unpack(packed[e], scales[e])
        y[r0:r1] = x[r0:r1].astype(np.float64) @ cache[e].T
        written[r0:r1] = True
    return y, written
