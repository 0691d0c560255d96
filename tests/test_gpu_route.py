"""GPU parity: gnf4_route_sort must match the oracle bit for bit (ids,
offsets, permutation, groups); weights within 1e-6."""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

from gpu_util import DEV, note

pytestmark = pytest.mark.gpu


def _run_and_compare(logits, k, what):
    T, E = logits.shape
    note(f"route {what} T={T} E={E} k={k}")
    r = gnf4.route_sort(torch.from_numpy(logits).to(DEV), k)
    torch.cuda.synchronize()
    ref = oracle.ref_route_sort(logits, k)
    ids = r.topk_ids.cpu().numpy()
    assert np.array_equal(ids, ref["topk_ids"]), f"{what}: topk ids differ"
    w = r.topk_w.cpu().numpy()
    assert np.max(np.abs(w - ref["topk_w"]), initial=0.0) <= 1e-6, f"{what}: weights"
    for key in ("expert_offsets", "sorted_slots", "slot_rows", "group_sizes", "group_expert_ids"):
        got = getattr(r, key).cpu().numpy()
        assert np.array_equal(got, ref[key]), f"{what}: {key} differs"
    assert int(r.num_groups.cpu()[0]) == ref["num_groups"], f"{what}: num_groups"
    return r


@pytest.mark.parametrize("name", ["tiny", "olmoe", "qwen3_t1", "qwen3_t8", "gptoss",
                                  "gptoss_t256", "dsv3"])
def test_route_workloads(name):
    wl = wls.WORKLOADS[name]
    _run_and_compare(wls.router_logits(wl), wl.top_k, name)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (3, 2, 2), (32, 64, 8), (33, 64, 8), (64, 64, 8), (65, 64, 8),
                                   (129, 128, 4), (7, 1024, 32), (300, 1024, 32),
                                   (1000, 256, 8), (2000, 96, 6), (1500, 512, 16)])
def test_route_shapes(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    _run_and_compare(rng.standard_normal((T, E)).astype(np.float32), k, "shape")


def test_route_ties_and_signed_zero():
    rng = np.random.default_rng(3)
    lg = np.round(rng.standard_normal((130, 64)) * 2).astype(np.float32) / 4  # many exact ties
    lg[0, :] = 0.0
    lg[1, ::2] = -0.0
    lg[2, :] = 1.0
    lg[3, 5] = np.float32(3.0e38)      # large but finite
    lg[4, :] = -np.float32(3.0e38)
    _run_and_compare(lg, 8, "ties")


def test_route_empty_batch():
    note("route T=0")
    E = 16
    r = gnf4.route_sort(torch.zeros((0, E), dtype=torch.float32, device=DEV), 4)
    torch.cuda.synchronize()
    assert np.all(r.expert_offsets.cpu().numpy() == 0)
    assert np.all(r.group_sizes.cpu().numpy() == 0)
    assert int(r.num_groups.cpu()[0]) == 0


def test_route_deterministic_and_gather():
    wl = wls.WORKLOADS["dsv3"]
    lg = wls.router_logits(wl)
    r1 = _run_and_compare(lg, wl.top_k, "dsv3 run 1")
    s1 = r1.sorted_slots.clone()
    r2 = gnf4.route_sort(torch.from_numpy(lg).to(DEV), wl.top_k)
    assert torch.equal(s1, r2.sorted_slots)
    # the gather builds exactly the oracle's grouped rows
    K = 256
    x = wls.token_activations(wl, K)
    note("gather dsv3 K=256")
    xs = gnf4.gather_rows(torch.from_numpy(x).to(DEV).to(torch.bfloat16), r2.sorted_slots,
                          wl.top_k)
    ref = oracle.ref_route_sort(lg, wl.top_k)
    expect = x[ref["sorted_slots"] // wl.top_k]
    assert np.array_equal(xs.float().cpu().numpy(), expect)
