"""Pins for the MXFP4 oracle: the E2M1 table against the specification's
listed values (tests/golden/e2m1_values.txt), E8M0 special cases, the nibble
order, and the grouped GEMM against one-hot activations (which read single
decoded weight columns) and an explicit loop over bits on a tiny case."""

import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.txt")


def test_e2m1_table_matches_the_specification():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    want = {int(c): float(v) for c, v in rows}
    assert sorted(want) == list(range(16))
    for c in range(16):
        assert oracle.E2M1_TABLE[c] == want[c]
        assert np.signbit(oracle.E2M1_TABLE[c]) == np.signbit(want[c]) or want[c] != 0.0


def test_e8m0_values():
    assert oracle.ref_e8m0_value(127) == 1.0
    assert oracle.ref_e8m0_value(128) == 2.0
    assert oracle.ref_e8m0_value(0) == 2.0 ** -127
    assert oracle.ref_e8m0_value(254) == 2.0 ** 127
    assert np.isnan(oracle.ref_e8m0_value(255))
    v = oracle.ref_e8m0_value(np.arange(255))
    assert np.all(v[1:] == 2 * v[:-1])


def test_nibble_order_low_first():
    packed = np.array([[[0x71, 0x0F]]], np.uint8)       # bytes: (lo 1, hi 7), (lo 15, hi 0)
    codes = oracle.ref_mx_codes(packed)
    assert list(codes[0, 0]) == [1, 7, 15, 0]
    w = oracle.ref_mx_unpack(np.tile(packed, (1, 1, 8)), np.array([[[128]]], np.uint8))
    assert list(w[0, 0, :4]) == [1.0, 12.0, -12.0, 0.0]   # (0.5, 6, -6, 0) * 2


def test_gemm_one_hot_rows_read_decoded_columns():
    rng = np.random.default_rng(81)
    E, N, K = 3, 16, 96
    packed = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    scales = rng.integers(110, 140, (E, N, K // 32), dtype=np.uint8)
    sizes, ids = [2, 3], [2, 0]
    M = 5
    x = np.zeros((M, K), np.float32)
    ks = [0, 95, 31, 32, 63]
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    y, wr = oracle.ref_grouped_gemm_mxfp4(x, packed, scales, sizes, ids)
    assert wr.all()
    for r, k in enumerate(ks):
        e = 2 if r < 2 else 0
        np.testing.assert_array_equal(y[r], oracle.ref_mx_unpack(packed[e], scales[e])[:, k])


def test_gemm_matches_loops_over_bits():
    rng = np.random.default_rng(83)
    E, N, K = 2, 4, 64
    packed = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    scales = rng.integers(120, 135, (E, N, K // 32), dtype=np.uint8)
    x = rng.standard_normal((3, K)).astype(np.float32)
    y, _ = oracle.ref_grouped_gemm_mxfp4(x, packed, scales, [1, 2], [1, 0])
    for r, e in ((0, 1), (1, 0), (2, 0)):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                byte = int(packed[e, n, k // 2])
                code = (byte & 0xF) if k % 2 == 0 else (byte >> 4)
                sgn = -1.0 if code & 8 else 1.0
                ex, m = (code >> 1) & 3, code & 1
                mag = 0.5 * m if ex == 0 else (1 + m / 2) * 2.0 ** (ex - 1)
                acc += float(x[r, k]) * sgn * mag * 2.0 ** (int(scales[e, n, k // 32]) - 127)
            assert abs(y[r, n] - acc) <= 1e-12 * max(1.0, abs(acc))
