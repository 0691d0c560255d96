"""GPU parity for gnf4_route_gemm_one_token (a batch-1 decode step's
route/sort folded into the grouped GEMM's launch): every route/sort output
equals the oracle's, and gnf4_route_sort's, bit for bit (weights: the same
bits as gnf4_route_sort, within 1e-6 of the oracle); y meets the GEMM bound
against the oracle on the routed rows.  Cases: OLMoE's shape, few experts,
ragged K, tied logits, bf16 absmax, a K that forces split-K (whose reduce
reads the groups the launch wrote), and 65 to 128 experts (two router entries
per lane: Qwen3's and GPT-OSS's expert counts, ties across the two entries).  Experts that are not picked hold 0xFF
codes and NaN absmax, so reading a wrong expert shows up as NaN.
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

from gpu_util import DEV, bf16_dev, check_gemm, note

pytestmark = pytest.mark.gpu

ROUTE_KEYS = ("expert_offsets", "sorted_slots", "slot_rows", "group_sizes", "group_expert_ids")


def _case(E, k, N, K, seed, absmax_dtype="f32", logits=None):
    rng = np.random.default_rng(seed)
    if logits is None:
        logits = rng.standard_normal((1, E)).astype(np.float32)
    ref = oracle.ref_route_sort(logits, k)
    picked = sorted(int(e) for e in ref["topk_ids"][0])
    adt = torch.bfloat16 if absmax_dtype == "bf16" else torch.float32
    packed = torch.full((E, N, K // 2), 0xFF, dtype=torch.uint8, device=DEV)
    absmax = torch.full((E, N, K // 64), float("nan"), dtype=adt, device=DEV)
    p_ref = np.zeros((E, N, K // 2), np.uint8)
    a_ref = np.zeros((E, N, K // 64), np.float32)
    for e in picked:
        w = wls.bf16_round((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        gnf4.pack(bf16_dev(w), out=(packed[e], absmax[e]))
        p_ref[e], a_ref[e] = oracle.ref_pack(w, absmax_dtype=absmax_dtype)
    x = wls.bf16_round(rng.standard_normal((1, K)).astype(np.float32))
    y_ref, written = oracle.ref_grouped_gemm(np.repeat(x, k, axis=0), p_ref, a_ref,
                                             ref["group_sizes"], ref["group_expert_ids"])
    return dict(logits=logits, ref=ref, packed=packed, absmax=absmax, x=x, y_ref=y_ref,
                written=written, k=k)


def _check(c, what, runs=2):
    lg = torch.from_numpy(c["logits"]).to(DEV)
    note(f"route+gemm one token {what}")
    ys = []
    for _ in range(runs):
        y, r = gnf4.route_gemm_one_token(lg, bf16_dev(c["x"]), c["packed"], c["absmax"], c["k"])
        torch.cuda.synchronize()
        ys.append(y.clone())
    ref = c["ref"]
    assert np.array_equal(r.topk_ids.cpu().numpy(), ref["topk_ids"]), f"{what}: topk ids"
    assert np.max(np.abs(r.topk_w.cpu().numpy() - ref["topk_w"])) <= 1e-6, f"{what}: weights"
    for key in ROUTE_KEYS:
        assert np.array_equal(getattr(r, key).cpu().numpy(), ref[key]), f"{what}: {key}"
    assert int(r.num_groups.cpu()[0]) == ref["num_groups"]
    # the same bits as the separate route/sort
    rs = gnf4.route_sort(lg, c["k"])
    torch.cuda.synchronize()
    assert torch.equal(rs.topk_w, r.topk_w), f"{what}: weights differ from gnf4_route_sort"
    for key in ROUTE_KEYS + ("topk_ids",):
        assert torch.equal(getattr(rs, key), getattr(r, key)), f"{what}: {key} vs route_sort"
    assert torch.equal(ys[0], ys[1]), f"{what}: not deterministic"
    check_gemm(ys[0], c["y_ref"], c["written"], what)


@pytest.mark.parametrize("E,k,N,K", [(64, 8, 2048, 2048), (8, 2, 384, 512), (60, 4, 256, 2880),
                                     (1, 1, 64, 64), (64, 32, 128, 256), (65, 8, 256, 512),
                                     (128, 8, 1536, 2048), (128, 4, 384, 2880),
                                     (100, 32, 128, 256)])
def test_route_gemm_shapes(E, k, N, K):
    _check(_case(E, k, N, K, seed=E * 131 + k), f"E={E} k={k} N={N} K={K}")


def test_route_gemm_olmoe_workload():
    wl = wls.WORKLOADS["olmoe"]
    K, N = wl.gemm("gate_up")
    lg = wls.router_logits(wl)
    _check(_case(wl.E, wl.top_k, N, K, seed=5, logits=lg), "olmoe gate_up")


def test_route_gemm_tied_logits():
    lg = np.zeros((1, 64), np.float32)
    lg[0, [3, 9, 17, 40]] = 1.5          # four-way tie at the top
    lg[0, [5, 6, 60]] = -0.0
    lg[0, 33] = 1.5
    _check(_case(64, 6, 192, 512, seed=7, logits=lg), "tied logits")


@pytest.mark.parametrize("name", ["qwen3_t1", "gptoss"])
def test_route_gemm_128_expert_workloads(name):
    wl = wls.WORKLOADS[name]
    K, N = wl.gemm("gate_up")
    _check(_case(wl.E, wl.top_k, N, K, seed=6, logits=wls.router_logits(wl)), f"{name} gate_up")


def test_route_gemm_tied_logits_two_entries():
    lg = np.zeros((1, 128), np.float32)
    lg[0, [3, 67, 100, 36]] = 2.0        # ties between a lane's two entries
    lg[0, [64, 0]] = -0.0
    lg[0, 127] = 2.0
    _check(_case(128, 6, 192, 512, seed=8, logits=lg), "tied logits, 128 experts")


def test_route_gemm_bf16_absmax():
    _check(_case(32, 4, 512, 1024, seed=9, absmax_dtype="bf16"), "bf16 absmax")


def test_route_gemm_split_k():
    """K = 12288 (384 chunks of 32) is above one split's 319: the launch
    writes split partials and the reduce groups its rows by the route/sort
    outputs the launch wrote."""
    _check(_case(16, 4, 96, 12288, seed=11), "split-K")
