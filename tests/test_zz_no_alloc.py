"""The allocation-free entry point (gnf4_grouped_gemm_gather_noalloc, its
workspace in the library's static per-GPU scratch array) against the entry
point it mirrors, gnf4_grouped_gemm_gather with a caller workspace: the same
kernels run, so the outputs must be identical bit for bit.  Two calls in a
row, the second with a smaller input (the scratch keeps the first call's
contents), the first on the matrix-core tile path (staged activation rows in
the scratch), the second on the decode path; the smaller one is also held to
the oracle's element-wise bound.
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

from gpu_util import DEV, bf16_dev, check_gemm, note, routed_stack

pytestmark = pytest.mark.gpu


def _tile_case():
    """A prefill-like batch: 200 tokens, top-2 of 8 experts, 50 rows per group
    on average, so the automatic path runs every group on the tile path."""
    E, N, K, T, top_k = 8, 256, 512, 200, 2
    rng = np.random.default_rng(101)
    w = wls.bf16_round((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    packed, absmax = gnf4.pack(bf16_dev(w))
    logits = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).to(DEV)
    r = gnf4.route_sort(logits, top_k)
    x = bf16_dev(rng.standard_normal((T, K)))
    return dict(x=x, r=r, top_k=top_k, packed=packed, absmax=absmax, M=T * top_k, N=N)


def _decode_case():
    """OLMoE-shaped batch-1 decode: one token, top-8 of 64 experts."""
    wl = wls.WORKLOADS["olmoe"]
    K, N = wl.gemm("gate_up")
    logits = wls.router_logits(wl)
    ref = oracle.ref_route_sort(logits, wl.top_k)
    r = gnf4.route_sort(torch.from_numpy(logits).to(DEV), wl.top_k)
    used = ref["group_expert_ids"][: ref["num_groups"]]
    packed, absmax, host = routed_stack(wl, "gate_up", used)
    x_tok = wls.token_activations(wl, K)
    p_ref = np.zeros((wl.E, N, K // 2), np.uint8)
    a_ref = np.zeros((wl.E, N, K // 64), np.float32)
    for e, w in host.items():
        p_ref[e], a_ref[e] = oracle.ref_pack(w)
    y_ref, written = oracle.ref_grouped_gemm(x_tok[ref["sorted_slots"] // wl.top_k], p_ref,
                                             a_ref, ref["group_sizes"], ref["group_expert_ids"])
    return dict(x=bf16_dev(x_tok), r=r, top_k=wl.top_k, packed=packed, absmax=absmax, M=wl.M,
                N=N, y_ref=y_ref, written=written)


def _both(c):
    r = c["r"]
    y_ws = gnf4.grouped_gemm(c["x"], c["packed"], c["absmax"], r.group_sizes,
                             r.group_expert_ids, sorted_slots=r.sorted_slots, top_k=c["top_k"])
    y_na = torch.full((c["M"], c["N"]), -512.0, dtype=torch.bfloat16, device=DEV)
    gnf4.grouped_gemm_gather_noalloc(c["x"], r.sorted_slots, c["top_k"], c["packed"],
                                     c["absmax"], r.group_sizes, r.group_expert_ids, y_na)
    torch.cuda.synchronize()
    return y_ws, y_na


def test_noalloc_matches_workspace_entry_point_twice():
    note("noalloc call 1: tile path, M=400")
    big = _tile_case()
    y_ws, y_na = _both(big)
    assert torch.equal(y_na, y_ws), "tile-path call differs from the workspace entry point"

    note("noalloc call 2: decode path, olmoe M=8 (smaller)")
    small = _decode_case()
    y_ws, y_na = _both(small)
    assert torch.equal(y_na, y_ws), "decode-path call differs from the workspace entry point"
    check_gemm(y_na, small["y_ref"], small["written"], "noalloc olmoe gate_up")


def test_noalloc_refuses_oversized_call():
    """A call needing more workspace than the scratch holds is refused with
    GNF4_ERR_UNSUPPORTED before anything is launched."""
    c = _tile_case()
    r = c["r"]
    big_x = torch.zeros((40000, 4096), dtype=torch.bfloat16, device=DEV)
    slots = torch.zeros(40000, dtype=torch.int32, device=DEV)
    packed = torch.zeros((8, 64, 2048), dtype=torch.uint8, device=DEV)
    absmax = torch.ones((8, 64, 64), dtype=torch.float32, device=DEV)
    y = torch.empty((40000, 64), dtype=torch.bfloat16, device=DEV)
    note("noalloc oversized request")
    with pytest.raises(gnf4.Gnf4Error, match="supported"):
        gnf4.grouped_gemm_gather_noalloc(big_x, slots, 1, packed, absmax, r.group_sizes,
                                         r.group_expert_ids, y, path=gnf4.PATH_TILE)
