"""Full-size parity in the launch configuration the benchmark times.

Every expert of every stack is drawn on the device (torch Philox, per-expert
seeds), packed by gnf4_pack and multiplied on the automatic path.  The
oracle gets the same bf16 weights copied back from the generator, packs
them itself, routes the same logits itself, and computes
  * every output of the decode-sized workloads (M <= 64 rows), and
  * for the DeepSeek-V3-sized prefill, every output of four complete groups
    (the first, last, largest and smallest) and a sample of outputs, one by
    one, across 48 more.
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

from gpu_util import DEV, bf16_dev, check_entries, check_gemm, note

pytestmark = pytest.mark.gpu


def device_stack(wl, gemm, layer=0):
    K, N = wl.gemm(gemm)
    packed = torch.empty((wl.E, N, K // 2), dtype=torch.uint8, device=DEV)
    absmax = torch.empty((wl.E, N, K // 64), dtype=torch.float32, device=DEV)
    for e in range(wl.E):
        w = wls.expert_weights_device(wl, gemm, e, DEV, layer)
        gnf4.pack(w, out=(packed[e], absmax[e]))
    return packed, absmax


def host_expert(wl, gemm, e, layer=0):
    return wls.expert_weights_device(wl, gemm, e, DEV, layer).float().cpu().numpy()


def complete_groups(groups):
    """The first, last, largest and smallest of the groups that write rows."""
    sizes = [r1 - r0 for (_g, _e, r0, r1) in groups]
    pick = {0, len(groups) - 1, int(np.argmax(sizes)), int(np.argmin(sizes))}
    return [groups[i] for i in sorted(pick)]


@pytest.mark.parametrize("name", ["olmoe", "qwen3_t1", "qwen3_t8", "gptoss"])
@pytest.mark.parametrize("gemm", ["gate_up", "down"])
def test_decode_workload_full_stack(name, gemm):
    wl = wls.WORKLOADS[name]
    K, N = wl.gemm(gemm)
    note(f"full-size {name}/{gemm}: generate + pack {wl.E} experts")
    packed, absmax = device_stack(wl, gemm)
    logits = wls.router_logits(wl)
    r = gnf4.route_sort(torch.from_numpy(logits).to(DEV), wl.top_k)
    ref = oracle.ref_route_sort(logits, wl.top_k)
    if gemm == "down":
        x_host = wls.down_input(wl, wl.M, K)
        xs = bf16_dev(x_host)
    else:
        x_tok = wls.token_activations(wl, K)
        x_host = x_tok[ref["sorted_slots"] // wl.top_k]
        xs = gnf4.gather_rows(bf16_dev(x_tok), r.sorted_slots, wl.top_k)
    note(f"full-size {name}/{gemm}: grouped GEMM (automatic path)")
    y = gnf4.grouped_gemm(xs, packed, absmax, r.group_sizes, r.group_expert_ids)
    torch.cuda.synchronize()
    used = ref["group_expert_ids"][: ref["num_groups"]]
    p_ref = np.zeros((wl.E, N, K // 2), np.uint8)
    a_ref = np.zeros((wl.E, N, K // 64), np.float32)
    for e in used:
        p_ref[e], a_ref[e] = oracle.ref_pack(host_expert(wl, gemm, int(e)))
    y_ref, written = oracle.ref_grouped_gemm(x_host, p_ref, a_ref, ref["group_sizes"],
                                             ref["group_expert_ids"])
    assert written.all()
    check_gemm(y, y_ref, written, f"{name}/{gemm} full size")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("gemm", ["gate_up", "down"])
def test_dsv3_prefill_sampled(gemm):
    wl = wls.WORKLOADS["dsv3"]
    K, N = wl.gemm(gemm)
    note(f"full-size dsv3/{gemm}: generate + pack {wl.E} experts")
    packed, absmax = device_stack(wl, gemm)
    logits = wls.router_logits(wl)
    r = gnf4.route_sort(torch.from_numpy(logits).to(DEV), wl.top_k)
    ref = oracle.ref_route_sort(logits, wl.top_k)
    if gemm == "down":
        x_host = wls.down_input(wl, wl.M, K)
        xs = bf16_dev(x_host)
    else:
        x_tok = wls.token_activations(wl, K)
        x_host = x_tok[ref["sorted_slots"] // wl.top_k]
        xs = gnf4.gather_rows(bf16_dev(x_tok), r.sorted_slots, wl.top_k)
    note(f"full-size dsv3/{gemm}: grouped GEMM (automatic path)")
    y = gnf4.grouped_gemm(xs, packed, absmax, r.group_sizes, r.group_expert_ids)
    y2 = gnf4.grouped_gemm(xs, packed, absmax, r.group_sizes, r.group_expert_ids)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "not deterministic"
    yh = y.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(yh))

    rng = np.random.default_rng(99)
    groups = oracle.ref_group_rows(ref["group_sizes"], ref["group_expert_ids"], wl.E, wl.M)
    picks = rng.choice(len(groups), 48, replace=False)
    rows, cols, owners = [], [], []
    for gi in picks:
        g, e, r0, r1 = groups[gi]
        for _ in range(8):
            rows.append(int(rng.integers(r0, r1)))
            cols.append(int(rng.integers(0, N)))
            owners.append(e)
    # every column of the last row of the last group, and the first row of group 0
    for (g, e, r0, r1), rr in ((groups[-1], groups[-1][3] - 1), (groups[0], groups[0][2])):
        for n in range(0, N, max(1, N // 64)):
            rows.append(rr)
            cols.append(n)
            owners.append(e)
    rows, cols, owners = map(np.array, (rows, cols, owners))
    expect = np.zeros(rows.size)
    for e in np.unique(owners):
        sel = np.nonzero(owners == e)[0]
        w = host_expert(wl, gemm, int(e))
        ns = np.unique(cols[sel])
        p, a = oracle.ref_pack(w[ns])
        wt = oracle.ref_unpack(p, a).astype(np.float64)
        row_of = {int(n): i for i, n in enumerate(ns)}
        for i in sel:
            expect[i] = float(np.dot(x_host[rows[i]].astype(np.float64), wt[row_of[int(cols[i])]]))
    rms = float(np.sqrt(np.mean(expect ** 2)))
    check_entries(yh[rows, cols], expect, rms, f"dsv3/{gemm} sampled")

    # every output of four complete groups: first, last, largest, smallest
    for g, e, r0, r1 in complete_groups(groups):
        note(f"full-size dsv3/{gemm}: group {g} (expert {e}, {r1 - r0} rows) in full")
        p, a = oracle.ref_pack(host_expert(wl, gemm, int(e)))
        wt = oracle.ref_unpack(p, a).astype(np.float64)
        o = x_host[r0:r1].astype(np.float64) @ wt.T
        check_gemm(y[r0:r1], o, np.ones(r1 - r0, bool),
                   f"dsv3/{gemm} group {g} (expert {e}, {r1 - r0} rows)")
