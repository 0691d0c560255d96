"""Pins for the oracle's NF4 table, quantiser, packing and decode.

Each test ties the oracle to something other than itself: the QLoRA quantile
construction, exhaustive byte enumeration, exact-rational brute force, closed
forms printed on the pages, and constructed exact inputs.  Several tests also
run a deliberately broken copy of an oracle step (the mistake planted on the
CPU) to show the pin would catch it.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.stats

import oracle
from oracle import nf4 as onf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def qlora_levels():
    """NormalFloat4 by the QLoRA recipe: normal quantiles at evenly spaced
    probabilities, 8 positive and 7 negative levels plus 0, scaled to [-1, 1]."""
    offset = 0.5 * ((1 - 1 / 32) + (1 - 1 / 30))
    pos = scipy.stats.norm.ppf(np.linspace(offset, 0.5, 9)[:-1])
    neg = -scipy.stats.norm.ppf(np.linspace(offset, 0.5, 8)[:-1])
    v = np.concatenate([pos, [0.0], neg])
    return np.sort(v / np.abs(v).max())


def test_table_matches_qlora_construction():
    ref = qlora_levels()
    t = oracle.NF4_TABLE.astype(np.float64)
    assert t.shape == (16,)
    assert np.max(np.abs(t - ref)) <= 2.5e-7


def test_table_invariants():
    t = oracle.NF4_TABLE
    assert t.dtype == np.float32
    assert np.all(np.diff(t.astype(np.float64)) > 0)
    assert t[0] == -1.0 and t[7] == 0.0 and t[15] == 1.0
    assert np.sum(t < 0) == 7 and np.sum(t > 0) == 8


def test_byte_roundtrip_exhaustive():
    b = np.arange(256, dtype=np.uint8)[None, :]
    codes = oracle.ref_codes(b)[0]
    for v in range(256):
        assert codes[2 * v] == v // 16 and codes[2 * v + 1] == v % 16
    # repacking the codes of every byte gives the byte back
    hi, lo = codes[0::2].astype(np.int64), codes[1::2].astype(np.int64)
    assert np.array_equal(hi * 16 + lo, np.arange(256))


def test_first_element_in_high_nibble():
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 0] = 1.0     # code 15
    w[0, 1] = -1.0    # code 0
    w[0, 2] = 0.5     # nearest level 0.4407 (midpoint to 0.5626 is 0.5017) -> code 12
    packed, absmax = oracle.ref_pack(w)
    assert packed[0, 0] == 0xF0
    assert packed[0, 1] == 0xC7   # (12 << 4) | 7: element 3 is zero
    assert absmax[0, 0] == 1.0


def _brute_code(x, a):
    """Nearest level to x/a in exact rationals, ties to the lower index."""
    if a == 0:
        return 7
    r = Fraction(float(x)) / Fraction(float(a))
    best, best_d = None, None
    for i, v in enumerate(oracle.NF4_TABLE):
        d = abs(r - Fraction(float(v)))
        if best_d is None or d < best_d:
            best, best_d = i, d
    return best


def _tie_block():
    # midpoints m6 = NF4[6]/2 and m7 = NF4[8]/2 are fp32 numbers: exact ties
    t = oracle.NF4_TABLE
    blk = np.zeros(64, dtype=np.float32)
    blk[0] = 1.0
    blk[1] = np.float32(t[6]) / np.float32(2)
    blk[2] = np.float32(t[8]) / np.float32(2)
    blk[3] = -np.float32(t[6]) / np.float32(2)
    blk[4] = np.float32(2.0 ** -20)   # tiny positive: rounds to the zero level
    blk[5] = -0.0
    return blk


def test_quantiser_matches_exact_rational_bruteforce():
    rng = np.random.default_rng(1234)
    blocks = [rng.standard_normal(64).astype(np.float32) * 0.02 for _ in range(40)]
    blocks.append(_tie_block())
    blocks.append(_tie_block() * np.float32(2.0 ** 40))
    blocks.append(_tie_block() * np.float32(2.0 ** -40))
    # adversarial: one outlier per block
    b = rng.standard_normal(64).astype(np.float32) * 1e-3
    b[17] = 50.0
    blocks.append(b)
    for blk in blocks:
        codes, a = oracle.ref_quantize_block(blk)
        assert a == np.max(np.abs(blk))
        for x, c in zip(blk, codes):
            assert c == _brute_code(x, a), (x, a, c)
        # the vectorised packer agrees with the per-block quantiser
        p, aa = oracle.ref_pack(blk[None, :])
        assert aa[0, 0] == a
        assert np.array_equal(oracle.ref_codes(p)[0], codes)


def test_ties_go_to_lower_code():
    codes, _ = oracle.ref_quantize_block(_tie_block())
    assert codes[1] == 6      # exactly between levels 6 and 7
    assert codes[2] == 7      # exactly between levels 7 and 8
    assert codes[3] == 8      # +0.0455 is past the 7|8 midpoint 0.0398
    assert codes[4] == 7 and codes[5] == 7


def test_ties_mutant_is_caught():
    """Planted mistake: ties to the UPPER code (>= instead of >)."""
    def mutant(block):
        b = np.asarray(block, dtype=np.float32)
        a = np.float32(np.max(np.abs(b)))
        thr = onf4._midpoints_f64() * np.float64(a)
        return np.array([(b.astype(np.float64)[i] >= thr).sum() for i in range(64)])
    blk = _tie_block()
    a = np.max(np.abs(blk))
    got = mutant(blk)
    assert any(got[i] != _brute_code(blk[i], a) for i in range(64))


def _scales():
    rng = np.random.default_rng(7)
    s = list(rng.uniform(1e-3, 1.0, 20).astype(np.float32))
    s += [np.float32(2.0 ** p) for p in (-120, -60, -1, 0, 1, 60, 120)]
    s += [np.float32(3.0e38), np.float32(1.1754944e-38), np.float32(0.0213)]
    return s


def test_sixteen_levels_reproduced_exactly_at_every_absmax():
    t = oracle.NF4_TABLE
    for a in _scales():
        vals = (t * a).astype(np.float32)          # fl32(NF4[i] * a)
        blk = np.tile(vals, 4)
        p, aa = oracle.ref_pack(blk[None, :])
        assert aa[0, 0].view(np.uint32) == np.float32(a).view(np.uint32)
        assert np.array_equal(oracle.ref_codes(p)[0], np.tile(np.arange(16), 4))
        back = oracle.ref_unpack(p, aa)[0]
        assert np.array_equal(back.view(np.uint32), blk.view(np.uint32))


def test_zero_block_and_negative_zero():
    w = np.zeros((2, 128), dtype=np.float32)
    w[1, :64] = -0.0
    w[1, 64] = 3.0
    p, a = oracle.ref_pack(w)
    assert a[0, 0] == 0 and a[0, 1] == 0 and a[1, 0] == 0
    assert np.all(oracle.ref_codes(p)[0] == 7)
    assert np.all(oracle.ref_codes(p)[1, :64] == 7)
    assert np.all(oracle.ref_unpack(p, a)[0] == 0)


def test_pack_idempotent():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((3, 16, 256)) * 0.02).astype(np.float32)
    p1, a1 = oracle.ref_pack(w)
    p2, a2 = oracle.ref_pack(oracle.ref_unpack(p1, a1))
    assert np.array_equal(p1, p2)
    assert np.array_equal(a1.view(np.uint32), a2.view(np.uint32))


def test_decode_error_closed_form_bound():
    """|w~ - w| <= a * (largest half-gap between levels) + 1 fp32 ulp of a."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((4, 8, 512)) * 0.02).astype(np.float32)
    p, a = oracle.ref_pack(w)
    wt = oracle.ref_unpack(p, a)
    t = oracle.NF4_TABLE.astype(np.float64)
    half_gap = np.max(np.diff(t)) / 2
    a_e = np.repeat(a.astype(np.float64), 64, axis=-1)
    err = np.abs(wt.astype(np.float64) - w.astype(np.float64))
    assert np.all(err <= a_e * half_gap * (1 + 1e-6) + a_e * 2.0 ** -23)


def test_absmax_index_mutant_is_caught():
    """Planted mistake: decode with the neighbouring block's absmax."""
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((2, 256)) * 0.02).astype(np.float32)
    w[:, 64:128] *= 10
    p, a = oracle.ref_pack(w)
    good = oracle.ref_unpack(p, a)
    bad = oracle.ref_unpack(p, np.roll(a, 1, axis=-1))
    t = oracle.NF4_TABLE.astype(np.float64)
    half_gap = np.max(np.diff(t)) / 2
    a_e = np.repeat(a.astype(np.float64), 64, axis=-1)
    ok_good = np.all(np.abs(good - w) <= a_e * half_gap * 1.001 + a_e * 2.0 ** -23)
    ok_bad = np.all(np.abs(bad - w) <= a_e * half_gap * 1.001 + a_e * 2.0 ** -23)
    assert ok_good and not ok_bad


def test_byte_ratio_matches_page():
    with open(os.path.join(GOLDEN, "byte_ratio.txt")) as f:
        kv = dict(line.split() for line in f if line.strip() and not line.startswith("#"))
    printed, digits = float(kv["ratio"]), int(kv["digits"])
    for K in (256, 768, 1024, 2048, 2880, 7168):
        r = oracle.ref_byte_ratio_vs_bf16(K)
        assert round(r, digits) == printed
        # bytes actually produced by the packer for one row agree with it
        p, a = oracle.ref_pack(np.ones((1, K), dtype=np.float32))
        assert math.isclose((2 * K) / (p.nbytes + a.nbytes), r)


def test_census_shape_is_whole_blocks():
    with open(os.path.join(GOLDEN, "census_shapes.txt")) as f:
        parts = [line.split() for line in f if line.strip() and not line.startswith("#")]
    for name, _, K, _, N in parts:
        assert int(K) % 64 == 0
        p, a = oracle.ref_pack(np.ones((1, int(K)), dtype=np.float32))
        assert p.shape == (1, int(K) // 2) and a.shape == (1, int(K) // 64)


def test_rejects_ragged_k():
    with pytest.raises(AssertionError):
        oracle.ref_pack(np.ones((1, 96), dtype=np.float32))


# ----------------------------------------------------------- bf16 absmax

def test_round_bf16_matches_torch_and_saturates():
    import torch
    rng = np.random.default_rng(71)
    a = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 4000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3e-39, 1e-45],
                                 np.float32)]).astype(np.float32)
    got = oracle.ref_round_bf16(a)
    want = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(got, want)
    big = np.array([3.39e38, np.finfo(np.float32).max, -np.finfo(np.float32).max], np.float32)
    sat = oracle.ref_round_bf16(big)
    assert np.all(np.isfinite(sat))
    assert sat[1] == np.float32(3.3895313892515355e38) and sat[2] == -sat[1]


def test_bf16_absmax_codes_are_nearest_to_the_stored_scale():
    """Brute force: with the bf16-rounded absmax a_s stored, every code is the
    exact-rational nearest level to x / a_s, ties to the lower code."""
    from fractions import Fraction
    rng = np.random.default_rng(73)
    w = (rng.standard_normal((3, 128)) * 0.3).astype(np.float32)
    w[1, :64] = np.float32(1.0039) * np.sign(rng.standard_normal(64)).astype(np.float32)
    packed, absmax = oracle.ref_pack(w, absmax_dtype="bf16")
    codes = oracle.ref_codes(packed)
    levels = [Fraction(float(v)) for v in oracle.NF4_TABLE]
    for n in range(3):
        for b in range(2):
            a_s = absmax[n, b]
            assert a_s == oracle.ref_round_bf16(np.abs(w[n, 64 * b:64 * b + 64]).max())
            for j in range(64):
                x = Fraction(float(w[n, 64 * b + j])) / Fraction(float(a_s))
                d = [abs(x - lv) for lv in levels]
                best = min(d)
                assert codes[n, 64 * b + j] == d.index(best)


def test_bf16_absmax_saves_a_sixteenth_of_a_byte_per_weight():
    w = np.random.default_rng(74).standard_normal((4, 256)).astype(np.float32)
    _, a32 = oracle.ref_pack(w)
    p16, a16 = oracle.ref_pack(w, absmax_dtype="bf16")
    assert a16.shape == a32.shape
    assert np.all(oracle.ref_round_bf16(a32) == a16)
    # bits per weight: 4 + 16/64 with bf16 absmax, 4 + 32/64 with fp32
    assert (p16.nbytes * 8 + a16.size * 16) / w.size == 4.25
