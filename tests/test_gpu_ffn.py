"""GPU parity for gnf4_moe_ffn_one_token: one token's route/sort, gate_up,
SwiGLU and down projection in one launch.

Checked against the oracle on every output:
  * route/sort outputs: bit for bit as the oracle and gnf4_route_sort;
  * h [k, I]: from the oracle's fp64 gate_up of the routed rows, within the
    bound the two projections' contract implies: each gate and up sum may
    differ from fp64 by the GEMM bound (8e-3 |g| + 1e-3 rms), carried through
    silu(g) * u to first order, plus the bf16 rounding of h (2^-8 |h|);
  * y [k, H]: the GEMM bound against the oracle's down projection of the h
    the kernel wrote (bf16 values, exact inputs).
Cases: the OLMoE and Qwen3-30B expert-layer shapes (64 and 128 experts: one
and two router entries per lane; GPT-OSS-120B's layer is refused, as it does
not fit on the device at once), bf16 absmax, several calls on
one workspace (every counter and flag returns to zero, no wait runs out)
and determinism.  Experts that are not picked hold 0xFF codes and NaN absmax.
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

from gpu_util import DEV, bf16_dev, check_gemm, host_f64, note

pytestmark = pytest.mark.gpu

ROUTE_KEYS = ("expert_offsets", "sorted_slots", "slot_rows", "group_sizes", "group_expert_ids")
REL, ABS = 8e-3, 1e-3


def _stacks(wl, picked, layer, absmax_dtype="f32"):
    """Device stacks with only the picked experts filled, and the oracle's
    decoded fp64 weights of those experts."""
    (H, I2) = wl.gemm("gate_up")
    (I, H2) = wl.gemm("down")
    assert H2 == H and I2 == 2 * I
    adt = torch.bfloat16 if absmax_dtype == "bf16" else torch.float32
    out, dec = {}, {}
    for gemm, (K, N) in (("gate_up", (H, 2 * I)), ("down", (I, H))):
        p = torch.full((wl.E, N, K // 2), 0xFF, dtype=torch.uint8, device=DEV)
        a = torch.full((wl.E, N, K // 64), float("nan"), dtype=adt, device=DEV)
        d = {}
        for e in picked:
            w = wls.expert_weights_device(wl, gemm, e, DEV, layer)
            gnf4.pack(w, out=(p[e], a[e]))
            pr, ar = oracle.ref_pack(w.float().cpu().numpy(), absmax_dtype=absmax_dtype)
            d[e] = oracle.ref_unpack(pr, ar).astype(np.float64)
        out[gemm] = (p, a)
        dec[gemm] = d
    return out, dec, H, I


def _h_bound(g, u, h_ref):
    """First-order bound on |h - h_ref| from the GEMM bound on g and u and
    the bf16 rounding of h."""
    dg = REL * np.abs(g) + ABS * np.sqrt(np.mean(g * g, axis=1, keepdims=True))
    du = REL * np.abs(u) + ABS * np.sqrt(np.mean(u * u, axis=1, keepdims=True))
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    return np.abs(dsilu * u) * dg + np.abs(g * sig) * du + 2.0 ** -8 * np.abs(h_ref) + 1e-30


def _run_case(name, layer=0, absmax_dtype="f32", calls=2, workspace=None):
    wl = wls.WORKLOADS[name]
    logits = wls.router_logits(wl, layer)[:1]
    ref = oracle.ref_route_sort(logits, wl.top_k)
    picked = sorted(int(e) for e in ref["topk_ids"][0])
    stacks, dec, H, I = _stacks(wl, picked, layer, absmax_dtype)
    if not gnf4.moe_ffn_one_token_supported(wl.E, wl.top_k, H, I):
        pytest.skip(f"no fused kernel for {name}")
    x = wls.activations_device(1, H, DEV, wl.seed, 77, layer)
    lg = torch.from_numpy(logits).to(DEV)
    ws = workspace if workspace is not None else gnf4.moe_ffn_one_token_workspace(wl.top_k, DEV)
    note(f"fused ffn {name} layer {layer} absmax {absmax_dtype}: {calls} calls")
    outs = []
    for _ in range(calls):
        y, h, r = gnf4.moe_ffn_one_token(lg, x, stacks["gate_up"], stacks["down"], wl.top_k,
                                         workspace=ws)
        torch.cuda.synchronize()
        outs.append((y.clone(), h.clone()))
    what = f"{name} layer {layer}"
    words = ws.view(torch.int32).cpu().numpy()
    assert not words.any(), f"{what}: workspace words left set at {np.nonzero(words)[0][:8]}"
    # route/sort outputs
    assert np.array_equal(r.topk_ids.cpu().numpy(), ref["topk_ids"]), f"{what}: topk ids"
    assert np.max(np.abs(r.topk_w.cpu().numpy() - ref["topk_w"])) <= 1e-6, f"{what}: weights"
    for key in ROUTE_KEYS:
        assert np.array_equal(getattr(r, key).cpu().numpy(), ref[key]), f"{what}: {key}"
    for yy, hh in outs[1:]:
        assert torch.equal(yy, outs[0][0]) and torch.equal(hh, outs[0][1]), f"{what}: not deterministic"
    # h against the oracle's fp64 gate_up of the routed rows (grouped order)
    xh = host_f64(x)[0]
    ids = ref["group_expert_ids"][: ref["num_groups"]]
    gu = np.stack([dec["gate_up"][int(e)] @ xh for e in ids])  # [k, 2I]
    g, u = gu[:, :I], gu[:, I:]
    h_ref = oracle.ref_swiglu(gu)
    h_gpu = host_f64(outs[0][1])
    bad = np.abs(h_gpu - h_ref) > _h_bound(g, u, h_ref)
    assert not bad.any(), f"{what}: {int(bad.sum())}/{bad.size} h values outside the bound"
    # y against the oracle's down projection of the kernel's own h
    y_ref = np.stack([dec["down"][int(e)] @ h_gpu[j] for j, e in enumerate(ids)])
    check_gemm(outs[0][0], y_ref, np.ones(len(ids), bool), f"{what}: y")
    return ws


@pytest.mark.parametrize("name", ["olmoe", "qwen3_t1"])
def test_ffn_one_token_workloads(name):
    _run_case(name)


def test_ffn_one_token_refuses_what_does_not_fit_at_once():
    # GPT-OSS-120B's layer needs more workgroups than the device holds at
    # once, so the fused launch is not offered for it
    wl = wls.WORKLOADS["gptoss"]
    H, N = wl.gemm("gate_up")
    assert not gnf4.moe_ffn_one_token_supported(wl.E, wl.top_k, H, N // 2)


def test_ffn_one_token_bf16_absmax():
    _run_case("olmoe", layer=1, absmax_dtype="bf16")


def test_ffn_one_token_workspace_reused_across_layers():
    ws = None
    for layer in range(4):
        ws = _run_case("qwen3_t1", layer=layer, calls=1, workspace=ws)


def test_ffn_one_token_unsupported_shape_is_refused():
    E, k, H, I = 8, 2, 256, 128
    assert not gnf4.moe_ffn_one_token_supported(E, k, H, I)
    lg = torch.zeros((1, E), dtype=torch.float32, device=DEV)
    x = torch.zeros((1, H), dtype=torch.bfloat16, device=DEV)
    gp = torch.zeros((E, 2 * I, H // 2), dtype=torch.uint8, device=DEV)
    ga = torch.ones((E, 2 * I, H // 64), dtype=torch.float32, device=DEV)
    dp = torch.zeros((E, H, I // 2), dtype=torch.uint8, device=DEV)
    da = torch.ones((E, H, I // 64), dtype=torch.float32, device=DEV)
    with pytest.raises(gnf4.Gnf4Error) as ei:
        gnf4.moe_ffn_one_token(lg, x, (gp, ga), (dp, da), k)
    assert ei.value.status == 3
