"""Pins for the oracle's SwiGLU, slot-row map, top-k combine and the composed
MoE feed-forward layer.

Each is checked against something other than its own formula: scipy's
logistic function and the tanh form of silu, the odd-part identity of silu,
brute-force enumeration of the grouped order, a dense routing-matrix product
for the combine, the gather/combine round trip, and a per-token loop over
the routed experts for the whole layer (no sorting at all).
"""

import numpy as np
import pytest
import scipy.special

import oracle


def test_silu_matches_logistic_and_tanh_forms():
    g = np.concatenate([np.linspace(-30, 30, 1201), [0.0, -0.0, 1e-8, -1e-8, 700.0, -700.0]])
    s = oracle.ref_silu(g)
    np.testing.assert_allclose(s, g * scipy.special.expit(g), rtol=1e-14, atol=1e-300)
    # 1 + tanh cancels for very negative g: compare absolutely there
    np.testing.assert_allclose(s, 0.5 * g * (1.0 + np.tanh(0.5 * g)), rtol=1e-12, atol=1e-13)


def test_silu_identities_and_limits():
    x = np.random.default_rng(5).standard_normal(1000) * 8
    # sigma(x) + sigma(-x) = 1  =>  silu(x) - silu(-x) = x
    np.testing.assert_allclose(oracle.ref_silu(x) - oracle.ref_silu(-x), x, rtol=1e-12, atol=1e-12)
    assert oracle.ref_silu(0.0) == 0.0
    assert oracle.ref_silu(60.0) == 60.0
    assert 0.0 >= oracle.ref_silu(-60.0) > -1e-23
    h = 1e-6  # silu'(0) = 1/2
    assert abs((oracle.ref_silu(h) - oracle.ref_silu(-h)) / (2 * h) - 0.5) < 1e-9


def test_swiglu_takes_gate_from_the_first_half():
    M, I = 3, 5
    gu = np.concatenate([np.full((M, I), 30.0), np.ones((M, I))], axis=1)
    h = oracle.ref_swiglu(gu)
    assert h.shape == (M, I)
    np.testing.assert_allclose(h, 30.0, rtol=1e-11)      # silu(30) * 1
    # a planted half swap gives silu(1) * 30 instead
    swapped = oracle.ref_silu(gu[:, I:]) * gu[:, :I]
    assert np.all(np.abs(swapped - h) > 5.0)
    rng = np.random.default_rng(3)
    gu = rng.standard_normal((4, 2 * 7))
    np.testing.assert_allclose(oracle.ref_swiglu(gu),
                               gu[:, :7] * scipy.special.expit(gu[:, :7]) * gu[:, 7:], rtol=1e-14)
    with pytest.raises(AssertionError):
        oracle.ref_swiglu(np.zeros((2, 5)))


def _brute_rows(ids):
    """Grouped order by enumeration: slots sorted by (expert, slot)."""
    flat = [int(e) for e in np.asarray(ids).reshape(-1)]
    order = sorted(range(len(flat)), key=lambda s: (flat[s], s))
    rows = [0] * len(flat)
    for pos, s in enumerate(order):
        rows[s] = pos
    return rows


def test_slot_rows_is_the_grouped_position():
    rng = np.random.default_rng(17)
    for T, E, k in ((1, 8, 2), (4, 8, 2), (9, 64, 8), (33, 16, 4), (5, 3, 3)):
        lg = rng.standard_normal((T, E)).astype(np.float32)
        r = oracle.ref_route_sort(lg, k)
        rows = r["slot_rows"]
        assert list(rows) == _brute_rows(r["topk_ids"])
        np.testing.assert_array_equal(rows[r["sorted_slots"]], np.arange(T * k))


def _dense_combine(y, sorted_slots, topk_w, M):
    """Routing matrix P [T, M] with P[t, r] = w[t, j] for sorted_slots[r] = t*k + j."""
    T, k = topk_w.shape
    P = np.zeros((T, y.shape[0]))
    for r in range(M):
        s = int(sorted_slots[r])
        P[s // k, r] = topk_w[s // k, s % k]
    return P @ y


def test_combine_matches_dense_routing_matrix():
    rng = np.random.default_rng(23)
    for T, E, k, H in ((1, 64, 8, 16), (6, 8, 2, 5), (20, 16, 4, 9)):
        r = oracle.ref_route_sort(rng.standard_normal((T, E)).astype(np.float32), k)
        M = T * k
        y = rng.standard_normal((M, H))
        out, mag = oracle.ref_combine(y, r["slot_rows"], r["topk_w"])
        np.testing.assert_allclose(out, _dense_combine(y, r["sorted_slots"], r["topk_w"], M),
                                   rtol=1e-12, atol=1e-12)
        assert np.all(mag >= np.abs(out) - 1e-12)
        # rows past a cut-off M contribute nothing
        Mc = M // 2
        out_c, _ = oracle.ref_combine(y[:Mc], r["slot_rows"], r["topk_w"], Mc)
        np.testing.assert_allclose(out_c, _dense_combine(y, r["sorted_slots"], r["topk_w"], Mc),
                                   rtol=1e-12, atol=1e-12)


def test_combine_undoes_the_gather():
    """Gathered rows y[r] = x[token of r] combined with softmax weights (which
    sum to one) give back x."""
    rng = np.random.default_rng(29)
    T, E, k, H = 12, 32, 4, 7
    r = oracle.ref_route_sort(rng.standard_normal((T, E)).astype(np.float32), k)
    x = rng.standard_normal((T, H))
    y = x[r["sorted_slots"].astype(np.int64) // k]
    out, _ = oracle.ref_combine(y, r["slot_rows"], r["topk_w"])
    np.testing.assert_allclose(out, x, rtol=1e-6, atol=1e-6)  # fp32 weights sum to 1 +- 1e-7


def test_moe_ffn_matches_per_token_loop():
    """The composed layer (sort, gather, grouped projections, SwiGLU,
    combine) against a direct loop over each token's routed experts."""
    rng = np.random.default_rng(31)
    T, E, k, D, I = 5, 8, 3, 64, 64
    w1 = (rng.standard_normal((E, 2 * I, D)) * 0.1).astype(np.float32)
    w2 = (rng.standard_normal((E, D, I)) * 0.1).astype(np.float32)
    gu = oracle.ref_pack(w1)
    dn = oracle.ref_pack(w2)
    x = rng.standard_normal((T, D)).astype(np.float32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    got = oracle.ref_moe_ffn(x, lg, k, gu, dn)
    ids, w = oracle.ref_topk(lg, k)
    want = np.zeros((T, D))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            a = oracle.ref_unpack(gu[0][e], gu[1][e]).astype(np.float64) @ x[t].astype(np.float64)
            h = a[:I] * scipy.special.expit(a[:I]) * a[I:]
            want[t] += float(w[t, j]) * (oracle.ref_unpack(dn[0][e], dn[1][e]).astype(np.float64) @ h)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
