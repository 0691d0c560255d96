"""Helpers shared by the GPU parity tests (no arithmetic of the method here).

The GPU side always goes through the C ABI (grouped_nf4_expert_amd.gnf4);
the expected values always come from the oracle run on the same seeded
inputs.
"""

import sys

import numpy as np
import torch

import oracle
from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

DEV = torch.device("cuda:0")
REL_TOL = 8e-3
RMS_TOL = 1e-3


def note(msg):
    """Name the case on stdout before a GPU step (survives a lost box)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def host_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_gemm(y_gpu, y_ref, written, what=""):
    """Element-wise |y - o| <= 8e-3 |o| + 1e-3 rms(o) over the written rows."""
    yv = host_f64(y_gpu)
    o = y_ref[written]
    g = yv[written]
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
    err = np.abs(g - o)
    bound = REL_TOL * np.abs(o) + RMS_TOL * rms
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; "
                           f"worst excess {float((err - bound).max()):.3e}, rms {rms:.3e}")
    return float(np.sqrt(np.mean((g - o) ** 2))) / max(rms, 1e-300)


def check_entries(got, ref, rms, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    bound = REL_TOL * np.abs(ref) + RMS_TOL * rms
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())}/{bad.size} sampled outputs outside tolerance"


def routed_stack(wl, gemm, experts, layer=0, fill_unused=True):
    """Device packed stack where only `experts` hold generated weights.

    Experts that no group uses get 0xFF codes and NaN absmax, so a kernel
    that reads the wrong expert produces NaN.  Returns the GPU-packed stack
    and the host bf16 weights of the used experts (for the oracle)."""
    K, N = wl.gemm(gemm)
    packed = torch.full((wl.E, N, K // 2), 0xFF, dtype=torch.uint8, device=DEV)
    absmax = torch.full((wl.E, N, K // 64), float("nan"), dtype=torch.float32, device=DEV)
    host = {}
    for e in sorted(set(int(v) for v in experts)):
        w = wls.expert_weights(wl, gemm, e, layer)
        host[e] = w
        gnf4.pack(bf16_dev(w), out=(packed[e], absmax[e]))
    return packed, absmax, host


def oracle_expert_fn(host):
    cache = {}

    def fn(e):
        if e not in cache:
            cache[e] = oracle.ref_pack(host[e])
        return cache[e]
    return fn
