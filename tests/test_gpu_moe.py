"""GPU parity for the steps around the grouped GEMM: gnf4_swiglu,
gnf4_combine, the route's slot_rows, and a whole MoE feed-forward layer
checked stage by stage against the oracle.

Bars (both from one rounding to bf16 after fp32 arithmetic):
  * swiglu:  |h - o| <= 2^-8 |o| + 1e-30, o = silu(g) * u in fp64;
  * combine: |out - o| <= 2^-8 |o| + k 2^-23 sum_j |w_j y_j|, o the fp64 sum
    (fp32 accumulation of k terms, then bf16 rounding).
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

from gpu_util import DEV, bf16_dev, check_gemm, host_f64, note, routed_stack

pytestmark = pytest.mark.gpu

BF16_REL = 2.0 ** -8


def _check_swiglu(h_gpu, gu_host, what):
    o = oracle.ref_swiglu(gu_host)
    g = host_f64(h_gpu)
    err = np.abs(g - o)
    bad = err > BF16_REL * np.abs(o) + 1e-30
    assert not bad.any(), f"{what}: {int(bad.sum())}/{bad.size} outside 2^-8 |o|"


def _check_combine(out_gpu, y_host, slot_rows, topk_w, M, what):
    o, mag = oracle.ref_combine(y_host, slot_rows, topk_w, M)
    k = topk_w.shape[1]
    g = host_f64(out_gpu)
    err = np.abs(g - o)
    bad = err > BF16_REL * np.abs(o) + k * 2.0 ** -23 * mag
    assert not bad.any(), f"{what}: {int(bad.sum())}/{bad.size} outside tolerance"


# ------------------------------------------------------------------ swiglu

@pytest.mark.parametrize("M,I", [(1, 8), (8, 1024), (8, 768), (4, 2880), (64, 13), (3, 4),
                                 (70000, 8), (257, 2048)])
def test_swiglu_shapes(M, I):
    note(f"swiglu M={M} I={I}")
    rng = np.random.default_rng(M * 131 + I)
    gu = (rng.standard_normal((M, 2 * I)) * 3).astype(np.float32)
    gu_dev = bf16_dev(gu)
    h = gnf4.swiglu(gu_dev)
    torch.cuda.synchronize()
    _check_swiglu(h, host_f64(gu_dev), f"swiglu {M}x{I}")


def test_swiglu_special_values_and_unaligned_rows():
    note("swiglu special values")
    I = 16
    g = np.array([0.0, -0.0, 1.0, -1.0, 10.0, -10.0, 80.0, -80.0, 100.0, -100.0, 3e4, -3e4,
                  1e-20, -1e-20, 0.5, -0.5], dtype=np.float32)
    u = np.array([1.0, 2.0, -3.0, 0.0, 1e-3, 1e3, -1.0, 1.0, 2.0, 5.0, 1.0, 1.0, 1.0, 1.0, 1e30,
                  -1e-30], dtype=np.float32)
    gu = np.concatenate([g, u])[None, :].repeat(3, axis=0)
    gu_dev = bf16_dev(gu)
    h = gnf4.swiglu(gu_dev)
    torch.cuda.synchronize()
    _check_swiglu(h, host_f64(gu_dev), "special")
    # rows starting at an odd element offset take the per-element path
    flat = torch.empty(1 + 3 * 2 * I, dtype=torch.bfloat16, device=DEV)
    flat[1:] = gu_dev.reshape(-1)
    h2 = torch.empty(1 + 3 * I, dtype=torch.bfloat16, device=DEV)
    gnf4.swiglu(flat[1:].view(3, 2 * I), out=h2[1:].view(3, I))
    torch.cuda.synchronize()
    assert torch.equal(h2[1:].view(3, I), h)


def test_swiglu_full_size_dsv3_sampled_rows():
    """DSV3 prefill gate_up output width (I = 2048) over all 32768 rows;
    the oracle checks a sample of rows."""
    M, I = 32768, 2048
    note(f"swiglu full size M={M} I={I}")
    gen = torch.Generator(device=DEV).manual_seed(7)
    gu = (torch.randn((M, 2 * I), device=DEV, generator=gen) * 2).to(torch.bfloat16)
    h = gnf4.swiglu(gu)
    torch.cuda.synchronize()
    rows = np.random.default_rng(7).choice(M, 256, replace=False)
    idx = torch.from_numpy(rows).to(DEV)
    _check_swiglu(h[idx], host_f64(gu[idx]), "dsv3 sampled")


# ------------------------------------------------------------------ combine

def _route(name, T=None):
    wl = wls.WORKLOADS[name]
    lg = wls.router_logits(wl, 0, T)
    r = gnf4.route_sort(torch.from_numpy(lg).to(DEV), wl.top_k)
    ref = oracle.ref_route_sort(lg, wl.top_k)
    assert np.array_equal(r.slot_rows.cpu().numpy(), ref["slot_rows"])
    return wl, r, ref


@pytest.mark.parametrize("name,H", [("tiny", 512), ("olmoe", 2048), ("qwen3_t8", 2048),
                                    ("gptoss", 2880), ("gptoss_t256", 2880), ("tiny", 13)])
def test_combine_workloads(name, H):
    wl, r, ref = _route(name)
    M = wl.M
    note(f"combine {name} T={wl.T} k={wl.top_k} H={H}")
    y_dev = bf16_dev(np.random.default_rng(H).standard_normal((M, H)))
    out = gnf4.combine(y_dev, r.slot_rows, r.topk_w)
    torch.cuda.synchronize()
    _check_combine(out, host_f64(y_dev), ref["slot_rows"], r.topk_w.cpu().numpy(), M, name)


def test_combine_cut_rows_and_edge_cases():
    wl, r, ref = _route("gptoss_t256")
    H = 64
    M = wl.M
    y_dev = bf16_dev(np.random.default_rng(1).standard_normal((M, H)))
    w = r.topk_w.cpu().numpy()
    for Mc in (M // 3, 1):
        note(f"combine cut M={Mc}")
        out = gnf4.combine(y_dev[:Mc].contiguous(), r.slot_rows, r.topk_w)
        torch.cuda.synchronize()
        _check_combine(out, host_f64(y_dev[:Mc]), ref["slot_rows"], w, Mc, f"cut {Mc}")
    note("combine M=0")
    out = torch.full((wl.T, H), 7.0, dtype=torch.bfloat16, device=DEV)
    gnf4.combine(torch.empty((0, H), dtype=torch.bfloat16, device=DEV), r.slot_rows, r.topk_w,
                 out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    note("combine k=1 is the inverse permutation")
    lg = np.random.default_rng(2).standard_normal((37, 16)).astype(np.float32)
    r1 = gnf4.route_sort(torch.from_numpy(lg).to(DEV), 1)
    x = bf16_dev(np.random.default_rng(3).standard_normal((37, 64)))
    xs = gnf4.gather_rows(x, r1.sorted_slots, 1)
    back = gnf4.combine(xs, r1.slot_rows, torch.ones((37, 1), device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(back, x)


def test_combine_full_size_dsv3_sampled_tokens():
    """DSV3 prefill down output (T=4096, k=8, H=7168); sampled tokens."""
    wl, r, ref = _route("dsv3")
    H, M = 7168, wl.M
    note(f"combine full size T={wl.T} H={H}")
    gen = torch.Generator(device=DEV).manual_seed(11)
    y = torch.randn((M, H), device=DEV, generator=gen).to(torch.bfloat16)
    out = gnf4.combine(y, r.slot_rows, r.topk_w)
    torch.cuda.synchronize()
    toks = np.sort(np.random.default_rng(11).choice(wl.T, 128, replace=False))
    k = wl.top_k
    rows = ref["slot_rows"].reshape(wl.T, k)[toks]            # [128, k] grouped rows
    y_sub = host_f64(y[torch.from_numpy(rows.reshape(-1).astype(np.int64)).to(DEV)])
    local = np.arange(rows.size, dtype=np.int32)              # rows renumbered 0..
    w = r.topk_w.cpu().numpy()[toks]
    _check_combine(out[torch.from_numpy(toks).to(DEV)], y_sub, local, w, rows.size, "dsv3")


# --------------------------------------------------------- whole MoE layer

@pytest.mark.parametrize("name", ["tiny_ffn", "olmoe", "qwen3_t8"])
def test_moe_layer_stage_by_stage(name):
    """route -> gate_up (fused gather) -> swiglu -> down -> combine on the GPU;
    each stage checked against the oracle applied to the GPU's own input to
    that stage, and the route checked bit for bit."""
    if name == "tiny_ffn":
        wl = wls.Workload("tiny_ffn", E=8, top_k=2, T=6,
                          gemms=(("gate_up", 256, 512), ("down", 256, 256)), seed=0)
    else:
        wl = wls.WORKLOADS[name]
    D, N1 = wl.gemm("gate_up")
    I, N2 = wl.gemm("down")
    assert N1 == 2 * I and N2 == D
    note(f"moe layer {name}")
    lg = wls.router_logits(wl)
    ref = oracle.ref_route_sort(lg, wl.top_k)
    r = gnf4.route_sort(torch.from_numpy(lg).to(DEV), wl.top_k)
    for key in ("sorted_slots", "slot_rows", "group_sizes", "group_expert_ids"):
        assert np.array_equal(getattr(r, key).cpu().numpy(), ref[key]), key
    used = ref["group_expert_ids"][: ref["num_groups"]]
    gu_p, gu_a, gu_host = routed_stack(wl, "gate_up", used)
    dn_p, dn_a, dn_host = routed_stack(wl, "down", used)
    x = bf16_dev(wls.token_activations(wl, D))

    def oracle_stack(host, N, K):
        p = np.zeros((wl.E, N, K // 2), np.uint8)
        a = np.zeros((wl.E, N, K // 64), np.float32)
        for e, w in host.items():
            p[e], a[e] = oracle.ref_pack(w)
        return p, a

    y1 = gnf4.grouped_gemm(x, gu_p, gu_a, r.group_sizes, r.group_expert_ids,
                           sorted_slots=r.sorted_slots, top_k=wl.top_k)
    h = gnf4.swiglu(y1)
    y2 = gnf4.grouped_gemm(h, dn_p, dn_a, r.group_sizes, r.group_expert_ids)
    out = gnf4.combine(y2, r.slot_rows, r.topk_w)
    torch.cuda.synchronize()

    x_sorted = host_f64(x)[ref["sorted_slots"] // wl.top_k]
    p1, a1 = oracle_stack(gu_host, N1, D)
    o1, written = oracle.ref_grouped_gemm(x_sorted, p1, a1, ref["group_sizes"],
                                          ref["group_expert_ids"])
    check_gemm(y1, o1, written, f"{name} gate_up")
    _check_swiglu(h, host_f64(y1), f"{name} swiglu")
    p2, a2 = oracle_stack(dn_host, N2, I)
    o2, written2 = oracle.ref_grouped_gemm(host_f64(h), p2, a2, ref["group_sizes"],
                                           ref["group_expert_ids"])
    check_gemm(y2, o2, written2, f"{name} down")
    _check_combine(out, host_f64(y2), ref["slot_rows"], r.topk_w.cpu().numpy(), wl.M,
                   f"{name} combine")
