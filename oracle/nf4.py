"""NormalFloat4 table, blockwise quantisation, byte packing and LUT decode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  * Page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE
    expert stacks", opening section: weights are an ``[E, N, K/2]`` uint8
    stack (two 4-bit codes per byte) with fp32 blockwise absmax, decoded
    through a lookup table to fp32 in registers, in the bitsandbytes
    gemm_4bit conventions.  The "Cross-vendor projections" section fixes the
    footprint: NF4 with its absmax is 3.56x smaller than bf16.
  * QLoRA (Dettmers et al., 2023), section 3: the NormalFloat4 data type --
    normal quantiles for 8 positive and 7 negative levels plus an exact zero,
    normalised to [-1, 1].

Readings (the pages leave these open):
  * block = 64 consecutive elements along K, one fp32 absmax each, blocks never
    straddle rows (so K must be a multiple of 64); 64 with fp32 absmax is
    what makes the 3.56x figure come out (16 / (4 + 32/64)).
  * byte j of a row holds element 2j in its HIGH nibble and 2j+1 in its low
    nibble.
  * a code is the index of the table value nearest to w/absmax in exact
    arithmetic, ties going to the lower index; an all-zero block stores
    absmax 0 and code 7 (the table's exact zero) everywhere.
  * decode is one fp32 round-to-nearest-even multiply: fl32(NF4[q] * absmax).
"""

import numpy as np

# QLoRA NormalFloat4 levels as fp32 literals, index = 4-bit code.
NF4_TABLE = np.array([
    -1.0,
    -0.6961928009986877,
    -0.5250730514526367,
    -0.39491748809814453,
    -0.28444138169288635,
    -0.18477343022823334,
    -0.09105003625154495,
    0.0,
    0.07958029955625534,
    0.16093020141124725,
    0.2461123913526535,
    0.33791524171829224,
    0.44070982933044434,
    0.5626170039176941,
    0.7229568362236023,
    1.0,
], dtype=np.float32)

BLOCK = 64
ZERO_CODE = 7


def _midpoints_f64():
    """Decision boundaries between neighbouring levels, exact in fp64.

    Each level is an fp32 number; the sum of two of them and the halving are
    exact in fp64, so m_i = (NF4[i] + NF4[i+1]) / 2 carries no rounding.
    """
    t = NF4_TABLE.astype(np.float64)
    return (t[:-1] + t[1:]) / 2.0


def ref_quantize_block(block):
    """Quantise one 64-element block: returns (codes uint8[64], absmax fp32).

    absmax is max |w| in fp32 (exact: inputs are fp32 or wider-exact bf16).
    code(x) = #{ i in 0..14 : x > m_i * absmax }.  Both m_i and the product
    m_i * absmax are exact in fp64 (m_i needs at most 26 significant bits,
    absmax 24), so the comparison is exact and equals the nearest level to
    x / absmax with ties going to the lower index.
    """
    b = np.asarray(block, dtype=np.float32).reshape(-1)
    assert b.size == BLOCK, "one block is 64 elements"
    assert np.all(np.isfinite(b)), "non-finite weights are outside the contract"
    a = np.float32(np.max(np.abs(b)))
    if a == 0:
        return np.full(BLOCK, ZERO_CODE, dtype=np.uint8), a
    thr = _midpoints_f64() * np.float64(a)
    x = b.astype(np.float64)
    codes = np.zeros(BLOCK, dtype=np.uint8)
    for t in thr:
        codes += (x > t).astype(np.uint8)
    return codes, a


def ref_round_bf16(a):
    """fp32 -> the nearest bf16 value (ties to even), saturating at the
    largest finite bf16 instead of overflowing; returned as fp32 values.

    bf16 keeps the top 16 bits of an fp32: adding 0x7FFF plus the lowest kept
    bit to the bit pattern and truncating rounds to nearest, ties to even.
    """
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    r = np.where((r & 0x7FFF) == 0x7F80, (r & 0x8000) | 0x7F7F, r)  # saturate
    return (r.astype(np.uint32) << 16).view(np.float32)


def ref_pack(w, absmax_dtype="f32"):
    """Quantise and pack ``w[..., N, K]`` (fp32 values) blockwise along K.

    Returns ``(packed uint8[..., N, K//2], absmax float32[..., N, K//64])``.
    Vectorised form of :func:`ref_quantize_block` applied to every block.

    ``absmax_dtype="bf16"``: the 4.25-bit form (page "How do I run a MoE
    whose experts do not fit in VRAM ...", "Supported scope": the NF4 bake
    takes ``--absmax-dtype f32|bf16|auto``).  Reading: each
    block's absmax is stored rounded to bf16 (nearest, ties to even,
    saturating) and the codes are chosen against the stored value -- the
    nearest level to x / a_stored, ties to the lower code, so decoding with
    the stored absmax is the same rule as the fp32 form.  The absmax comes
    back as fp32 values that bf16 holds exactly.  m_i * a_stored is still
    exact in fp64 (26 + 8 significant bits).
    """
    assert absmax_dtype in ("f32", "bf16")
    w = np.asarray(w, dtype=np.float32)
    K = w.shape[-1]
    assert K % BLOCK == 0, "K must be a multiple of the 64-element block"
    assert np.all(np.isfinite(w)), "non-finite weights are outside the contract"
    blocks = w.reshape(w.shape[:-1] + (K // BLOCK, BLOCK))
    absmax = np.max(np.abs(blocks), axis=-1).astype(np.float32)
    if absmax_dtype == "bf16":
        absmax = ref_round_bf16(absmax)
    thr_a = absmax.astype(np.float64)[..., None]
    x = blocks.astype(np.float64)
    codes = np.zeros(blocks.shape, dtype=np.uint8)
    for m in _midpoints_f64():
        codes += (x > m * thr_a).astype(np.uint8)
    codes[absmax == 0] = ZERO_CODE
    codes = codes.reshape(w.shape)
    hi = codes[..., 0::2]
    lo = codes[..., 1::2]
    packed = ((hi << 4) | lo).astype(np.uint8)
    return packed, absmax


def ref_codes(packed):
    """Unpack bytes to codes ``uint8[..., K]``: high nibble first."""
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    codes[..., 0::2] = p >> 4
    codes[..., 1::2] = p & 0x0F
    return codes


def ref_unpack(packed, absmax):
    """Decode to fp32 weights ``[..., N, K]``: fl32(NF4[code] * absmax).

    numpy's float32 * float32 is one IEEE round-to-nearest-even multiply.
    """
    codes = ref_codes(packed)
    K = codes.shape[-1]
    a = np.asarray(absmax, dtype=np.float32)
    assert a.shape[-1] * BLOCK == K
    a_per_elem = np.repeat(a, BLOCK, axis=-1)
    return (NF4_TABLE[codes] * a_per_elem).astype(np.float32)


def ref_byte_ratio_vs_bf16(K):
    """Bytes of a bf16 row over bytes of its NF4 form (codes + fp32 absmax)."""
    assert K % BLOCK == 0
    return (2.0 * K) / (K / 2.0 + 4.0 * K / BLOCK)
