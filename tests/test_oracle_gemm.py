"""Pins for the oracle's grouped GEMM.

Exact rational dot products (``fractions.Fraction``) on the tiny workload,
one-hot activations that must return single decoded weights, an all-ones
code pattern that reduces to row sums, group semantics checked row by row
against a plain walk over the sizes, and planted mistakes (transposed
weight, wrong expert, nibble order swapped) that must fail.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from grouped_nf4_expert_amd import workloads as wls


def _tiny_case():
    wl = wls.WORKLOADS["tiny"]
    K, N = wl.gemm("w")
    w = wls.weight_stack(wl, "w")
    packed, absmax = oracle.ref_pack(w)
    r = oracle.ref_route_sort(wls.router_logits(wl), wl.top_k)
    x_tok = wls.token_activations(wl, K)
    x = x_tok[r["sorted_slots"] // wl.top_k]
    return wl, packed, absmax, r, x


def test_exact_rational_dots_on_tiny():
    wl, packed, absmax, r, x = _tiny_case()
    y, written = oracle.ref_grouped_gemm(x, packed, absmax, r["group_sizes"],
                                         r["group_expert_ids"])
    assert written.all()
    codes = oracle.ref_codes(packed)
    rng = np.random.default_rng(0)
    groups = oracle.ref_group_rows(r["group_sizes"], r["group_expert_ids"], wl.E, wl.M)
    for g, e, r0, r1 in groups:
        for rr in range(r0, r1):
            for n in rng.choice(packed.shape[1], 6, replace=False):
                exact = Fraction(0)
                for k in range(x.shape[1]):
                    wv = np.float32(oracle.NF4_TABLE[codes[e, n, k]] * absmax[e, n, k // 64])
                    exact += Fraction(float(x[rr, k])) * Fraction(float(wv))
                ref = float(exact)
                assert abs(y[rr, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_one_hot_rows_return_single_weights():
    wl, packed, absmax, r, _ = _tiny_case()
    K = packed.shape[2] * 2
    M = wl.M
    ks = np.arange(M) * 37 % K
    x = np.zeros((M, K), dtype=np.float32)
    x[np.arange(M), ks] = 1.0
    y, _ = oracle.ref_grouped_gemm(x, packed, absmax, r["group_sizes"], r["group_expert_ids"])
    wt = oracle.ref_unpack(packed, absmax)
    for g, e, r0, r1 in oracle.ref_group_rows(r["group_sizes"], r["group_expert_ids"], wl.E, M):
        for rr in range(r0, r1):
            assert np.array_equal(y[rr], wt[e, :, ks[rr]].astype(np.float64))


def test_all_top_codes_give_row_sums():
    E, N, K, M = 2, 8, 192, 5
    packed = np.full((E, N, K // 2), 0xFF, dtype=np.uint8)
    absmax = np.ones((E, N, K // 64), dtype=np.float32)
    rng = np.random.default_rng(1)
    x = wls.bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    y, _ = oracle.ref_grouped_gemm(x, packed, absmax, [3, 2], [1, 0])
    expect = np.array([sum(float(v) for v in row) for row in x])
    assert np.allclose(y, expect[:, None], rtol=0, atol=1e-12)


def _walk_groups(sizes, ids, E, M):
    owner = [-1] * M
    r = 0
    for s, e in zip(sizes, ids):
        for _ in range(max(int(s), 0)):
            if r < M and 0 <= e < E:
                owner[r] = e
            r += 1
    return owner


@pytest.mark.parametrize("sizes,ids", [
    ([0, 3, 0, 2], [5, 1, 2, 3]),
    ([2, 2, 2], [1, 1, 0]),            # duplicate expert ids
    ([1, 9, 4], [0, 3, 2]),            # runs past M
    ([2, -1, 3], [0, 1, 2]),           # negative size holds no rows
    ([2, 2, 2], [0, 7, 1]),            # expert id out of range
])
def test_group_semantics_row_by_row(sizes, ids):
    E, N, K, M = 4, 6, 128, 8
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    packed, absmax = oracle.ref_pack(w)
    wt = oracle.ref_unpack(packed, absmax).astype(np.float64)
    x = wls.bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    y, written = oracle.ref_grouped_gemm(x, packed, absmax, sizes, ids)
    owner = _walk_groups(sizes, ids, E, M)
    for r in range(M):
        if owner[r] < 0:
            assert not written[r] and np.all(np.isnan(y[r]))
        else:
            assert written[r]
            for n in range(N):
                ref = sum(float(a) * float(b) for a, b in zip(x[r], wt[owner[r], n]))
                assert abs(y[r, n] - ref) <= 1e-12


def test_entries_agree_with_full():
    wl, packed, absmax, r, x = _tiny_case()
    y, _ = oracle.ref_grouped_gemm(x, packed, absmax, r["group_sizes"], r["group_expert_ids"])
    rng = np.random.default_rng(4)
    rows = rng.integers(0, wl.M, 30)
    cols = rng.integers(0, packed.shape[1], 30)
    got = oracle.ref_grouped_gemm_entries(
        x, lambda e: (packed[e], absmax[e]), wl.E, packed.shape[1],
        r["group_sizes"], r["group_expert_ids"], rows, cols)
    assert np.allclose(got, y[rows, cols], rtol=1e-13, atol=0)


def test_planted_mistakes_are_caught():
    """Swapped nibbles, a transposed weight and a wrong expert all break the
    exact one-hot identity y[r] = W~[e, :, k]."""
    wl, packed, absmax, r, _ = _tiny_case()
    K = packed.shape[2] * 2
    x = np.zeros((wl.M, K), dtype=np.float32)
    ks = (np.arange(wl.M) * 37 + 1) % K
    x[np.arange(wl.M), ks] = 1.0
    wt = oracle.ref_unpack(packed, absmax)
    swapped = ((packed & 0x0F) << 4) | (packed >> 4)
    y_sw, _ = oracle.ref_grouped_gemm(x, swapped.astype(np.uint8), absmax,
                                      r["group_sizes"], r["group_expert_ids"])
    y_wrong_e, _ = oracle.ref_grouped_gemm(x, np.roll(packed, 1, axis=0), np.roll(absmax, 1, axis=0),
                                           r["group_sizes"], r["group_expert_ids"])
    bad_sw = bad_e = 0
    for g, e, r0, r1 in oracle.ref_group_rows(r["group_sizes"], r["group_expert_ids"], wl.E, wl.M):
        for rr in range(r0, r1):
            ref = wt[e, :, ks[rr]].astype(np.float64)
            bad_sw += not np.array_equal(y_sw[rr], ref)
            bad_e += not np.array_equal(y_wrong_e[rr], ref)
            # transposed operand: treating W[e] as [K, N] reads the wrong entries
            flat = wt[e].reshape(-1)
            trans = flat.reshape(K, -1)[ks[rr], :packed.shape[1]]
            bad_trans = not np.array_equal(trans.astype(np.float64), ref)
            assert bad_trans
    assert bad_sw > 0 and bad_e > 0


# ------------------------------------------------------------------ dgrad

def _dgrad_case(seed, E=4, N=96, K=192, sizes=(3, 0, 5, 2), ids=(1, 3, 1, 0), M=11):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((E, N, K)) * 0.05).astype(np.float32)
    packed, absmax = oracle.ref_pack(w)
    dy = rng.standard_normal((M, N)).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    return packed, absmax, list(sizes), list(ids), dy, x


def test_dgrad_is_the_adjoint_of_the_gemm():
    """<dy, x W^T> == <dy W, x> over the written rows (exact math; fp64)."""
    packed, absmax, sizes, ids, dy, x = _dgrad_case(41)
    y, wr = oracle.ref_grouped_gemm(x, packed, absmax, sizes, ids)
    dx, wr2 = oracle.ref_grouped_dgrad(dy, packed, absmax, sizes, ids)
    assert np.array_equal(wr, wr2)
    lhs = np.sum(dy[wr].astype(np.float64) * y[wr])
    rhs = np.sum(dx[wr] * x[wr].astype(np.float64))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_dgrad_one_hot_rows_select_weight_rows():
    packed, absmax, sizes, ids, _, _ = _dgrad_case(43)
    M, N = 11, 96
    dy = np.zeros((M, N), np.float32)
    picks = [(0, 5), (1, 0), (2, 95), (3, 40), (5, 7), (10, 33)]
    for r, n in picks:
        dy[r, n] = 1.0
    dx, wr = oracle.ref_grouped_dgrad(dy, packed, absmax, sizes, ids)
    owner = {r: e for _g, e, r0, r1 in oracle.ref_group_rows(sizes, ids, 4, M)
             for r in range(r0, r1)}
    for r, n in picks:
        if r in owner:
            want = oracle.ref_unpack(packed[owner[r]], absmax[owner[r]])[n]
            np.testing.assert_array_equal(dx[r], want.astype(np.float64))
        else:
            assert not wr[r] and np.all(np.isnan(dx[r]))


def test_dgrad_matches_explicit_loops():
    packed, absmax, sizes, ids, dy, _ = _dgrad_case(47, E=3, N=8, K=64, sizes=(2, 1),
                                                     ids=(2, 0), M=4)
    dx, wr = oracle.ref_grouped_dgrad(dy, packed, absmax, sizes, ids)
    table = oracle.NF4_TABLE
    codes = oracle.ref_codes(packed)
    rows_of = {0: 2, 1: 2, 2: 0}
    for r in range(4):
        if r not in rows_of:
            assert not wr[r]
            continue
        e = rows_of[r]
        for k in range(64):
            acc = 0.0
            for n in range(8):
                acc += float(dy[r, n]) * float(np.float32(table[codes[e, n, k]]) *
                                               absmax[e, n, k // 64])
            assert abs(dx[r, k] - acc) <= 1e-12 * max(1.0, abs(acc))
