"""Pins for the oracle's top-k routing and token->expert sort.

Brute force with Python's own ``sorted`` / ``heapq`` on small inputs, the
invariants a counting sort must satisfy, softmax identities, and planted
mistakes (unstable order, ties to the higher id) that the pins must catch.
"""

import heapq

import numpy as np
import scipy.special

import oracle
from grouped_nf4_expert_amd import workloads as wls


def _brute_topk(row, k):
    return [e for _, e in heapq.nsmallest(k, ((-float(v), e) for e, v in enumerate(row)))]


def test_topk_matches_bruteforce():
    rng = np.random.default_rng(11)
    for T, E, k in ((4, 8, 2), (7, 64, 8), (5, 128, 4), (3, 256, 8), (2, 5, 5)):
        lg = rng.standard_normal((T, E)).astype(np.float32)
        # force some exact ties
        lg[0, 1] = lg[0, 3] = lg[0].max()
        ids, w = oracle.ref_topk(lg, k)
        for t in range(T):
            assert list(ids[t]) == _brute_topk(lg[t], k)


def test_topk_ties_and_signed_zero():
    lg = np.array([[0.0, -0.0, 0.0, -1.0, -0.0, 5.0]], dtype=np.float32)
    ids, _ = oracle.ref_topk(lg, 4)
    assert list(ids[0]) == [5, 0, 1, 2]


def test_topk_higher_id_mutant_is_caught():
    lg = np.array([[1.0, 2.0, 2.0, 0.0]], dtype=np.float32)
    good = list(oracle.ref_topk(lg, 2)[0][0])
    # planted mistake: stable sort of the reversed row -> ties to the higher id
    E = lg.shape[1]
    mutant = list(E - 1 - np.argsort(-lg[0, ::-1], kind="stable"))[:2]
    assert good == _brute_topk(lg[0], 2) == [1, 2]
    assert mutant == [2, 1] and mutant != _brute_topk(lg[0], 2)


def test_softmax_weights():
    rng = np.random.default_rng(12)
    lg = rng.standard_normal((50, 64)).astype(np.float32) * 3
    ids, w = oracle.ref_topk(lg, 8)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= 1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    ren = sel / sel.sum(1, keepdims=True)
    assert np.max(np.abs(ren - w)) <= 1e-6


def _brute_sort(ids_flat):
    return sorted(range(len(ids_flat)), key=lambda s: (int(ids_flat[s]), s))


def test_sort_matches_bruteforce_and_invariants():
    rng = np.random.default_rng(13)
    for T, E, k in ((4, 8, 2), (1, 64, 8), (8, 128, 8), (33, 16, 4), (256, 128, 4)):
        lg = rng.standard_normal((T, E)).astype(np.float32)
        r = oracle.ref_route_sort(lg, k)
        flat = r["topk_ids"].reshape(-1)
        M = T * k
        assert list(r["sorted_slots"]) == _brute_sort(flat)
        off = r["expert_offsets"]
        assert off[0] == 0 and off[-1] == M and np.all(np.diff(off) >= 0)
        assert sorted(r["sorted_slots"]) == list(range(M))
        for e in range(E):
            seg = r["sorted_slots"][off[e]:off[e + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
        G = r["num_groups"]
        assert G == np.count_nonzero(np.bincount(flat, minlength=E))
        assert r["group_sizes"][:G].sum() == M and np.all(r["group_sizes"][:G] > 0)
        assert np.all(np.diff(r["group_expert_ids"][:G]) > 0)
        assert np.all(r["group_sizes"][G:] == 0) and np.all(r["group_expert_ids"][G:] == 0)
        # ids distinct per token
        for t in range(T):
            assert len(set(r["topk_ids"][t])) == k


def test_unstable_sort_mutant_is_caught():
    flat = np.array([3, 1, 3, 1, 3, 0, 1, 3], dtype=np.int64)
    unstable = list(np.argsort(flat, kind="stable")[::-1][::-1])
    # reverse order inside each expert: a plausible atomics-ordered scatter
    by_e = {}
    for s in range(flat.size):
        by_e.setdefault(int(flat[s]), []).append(s)
    mutant = [s for e in sorted(by_e) for s in reversed(by_e[e])]
    assert unstable == _brute_sort(flat)
    assert mutant != _brute_sort(flat)


def test_skewed_router_uses_hot_set():
    wl = wls.WORKLOADS["gptoss_t256"]
    lg = wls.router_logits(wl)
    r = oracle.ref_route_sort(lg, wl.top_k)
    sizes = r["group_sizes"][: r["num_groups"]]
    # the hot experts carry most of the rows: sizes are uneven
    assert sizes.max() >= 4 * np.median(sizes)
