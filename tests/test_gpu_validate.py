"""GNF4_VALIDATE=1: the opt-in device-side check of the grouping inputs.

Landing page "grouped-nf4-gemm", "Do not use this when": nothing falls back
silently.  Without the variable the kernels skip groups and rows outside
their contract (tested in test_gpu_gemm's boundary cases); with it, the
call reports GNF4_ERR_INVALID_ARG and launches nothing, so the output's
canary values stay untouched.
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

from gpu_util import DEV, bf16_dev, check_gemm, note

pytestmark = pytest.mark.gpu

E, N, K = 4, 64, 128


def _stack(seed=3):
    rng = np.random.default_rng(seed)
    w = wls.bf16_round((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    packed, absmax = gnf4.pack(bf16_dev(w))
    return w, packed, absmax


def _i32(v):
    return torch.tensor(v, dtype=torch.int32, device=DEV)


BAD = {
    "negative_size": ([3, -1, 2], [0, 1, 2], 5),
    "id_out_of_range": ([2, 3], [0, 9], 5),
    "negative_id": ([2, 3], [-1, 2], 5),
    "sizes_past_M": ([4, 8], [0, 1], 10),
}


@pytest.mark.parametrize("case", sorted(BAD))
@pytest.mark.parametrize("path", [gnf4.PATH_DECODE, gnf4.PATH_TILE])
def test_validate_rejects_bad_groups(monkeypatch, case, path):
    monkeypatch.setenv("GNF4_VALIDATE", "1")
    sizes, ids, M = BAD[case]
    _, packed, absmax = _stack()
    x = bf16_dev(np.random.default_rng(4).standard_normal((M, K)))
    y = torch.full((M, N), -512.0, dtype=torch.bfloat16, device=DEV)
    note(f"validate {case} path={path}")
    with pytest.raises(gnf4.Gnf4Error, match="invalid argument"):
        gnf4.grouped_gemm(x, packed, absmax, _i32(sizes), _i32(ids), G=len(sizes), y=y,
                          path=path)
    torch.cuda.synchronize()
    assert torch.all(y.float() == -512.0), "a rejected call wrote its output"


def test_validate_rejects_bad_slots_and_dgrad_groups(monkeypatch):
    monkeypatch.setenv("GNF4_VALIDATE", "1")
    _, packed, absmax = _stack()
    T, top_k = 3, 2
    x = bf16_dev(np.random.default_rng(5).standard_normal((T, K)))
    slots = _i32([0, 1, 2, 3, 4, 6])  # 6 >= T * top_k
    y = torch.full((6, N), -512.0, dtype=torch.bfloat16, device=DEV)
    note("validate bad slot")
    with pytest.raises(gnf4.Gnf4Error, match="invalid argument"):
        gnf4.grouped_gemm(x, packed, absmax, _i32([3, 3]), _i32([0, 1]), G=2, y=y,
                          sorted_slots=slots, top_k=top_k)
    dy = bf16_dev(np.random.default_rng(6).standard_normal((5, N)))
    note("validate dgrad bad id")
    with pytest.raises(gnf4.Gnf4Error, match="invalid argument"):
        gnf4.grouped_dgrad(dy, packed, absmax, _i32([2, 3]), _i32([0, 4]), G=2)
    torch.cuda.synchronize()
    assert torch.all(y.float() == -512.0)


def test_validate_passes_good_groups(monkeypatch):
    """Valid inputs (empty groups and a zero tail included) run as usual."""
    monkeypatch.setenv("GNF4_VALIDATE", "1")
    w, packed, absmax = _stack()
    sizes, ids, M = [3, 0, 5, 0], [2, 7, 0, 0], 8   # the empty group's id is not checked
    x_host = wls.bf16_round(np.random.default_rng(7).standard_normal((M, K)).astype(np.float32))
    p, a = oracle.ref_pack(w)
    o, written = oracle.ref_grouped_gemm(x_host, p, a, sizes, ids)
    for path in (gnf4.PATH_DECODE, gnf4.PATH_TILE):
        note(f"validate good groups path={path}")
        y = gnf4.grouped_gemm(bf16_dev(x_host), packed, absmax, _i32(sizes), _i32(ids), G=4,
                              path=path)
        torch.cuda.synchronize()
        check_gemm(y, o, written, f"validated call path {path}")
