"""GPU parity: gnf4_pack must match the oracle's packer bit for bit."""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

from gpu_util import DEV, bf16_dev, note

pytestmark = pytest.mark.gpu


def _compare(w_host, w_dev, what, absmax_dtype="f32"):
    note(f"pack {what} shape={tuple(w_dev.shape)} dtype={w_dev.dtype} absmax={absmax_dtype}")
    tdt = torch.bfloat16 if absmax_dtype == "bf16" else torch.float32
    packed, absmax = gnf4.pack(w_dev, absmax_dtype=tdt)
    torch.cuda.synchronize()
    assert absmax.dtype == tdt
    p_ref, a_ref = oracle.ref_pack(w_host, absmax_dtype=absmax_dtype)
    p = packed.cpu().numpy()
    a = absmax.float().cpu().numpy()
    assert p.shape == p_ref.shape and a.shape == a_ref.shape
    bad = np.nonzero(p != p_ref)
    assert bad[0].size == 0, f"{what}: {bad[0].size} bytes differ, first at {tuple(b[0] for b in bad)}"
    assert np.array_equal(a.view(np.uint32), a_ref.view(np.uint32)), f"{what}: absmax bits differ"


@pytest.mark.parametrize("name,gemm", [("tiny", "w"), ("olmoe", "gate_up"), ("olmoe", "down"),
                                       ("qwen3_t1", "down"), ("gptoss", "down"),
                                       ("dsv3", "down")])
def test_pack_workload_experts(name, gemm):
    wl = wls.WORKLOADS[name]
    experts = range(min(wl.E, 3))
    w = np.stack([wls.expert_weights(wl, gemm, e) for e in experts])
    _compare(w, bf16_dev(w), f"{name}/{gemm}")


def test_pack_fp32_input():
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((2, 40, 320)) * 0.02).astype(np.float32)  # not bf16-exact
    _compare(w, torch.from_numpy(w).to(DEV), "fp32")


def _adversarial_rows():
    t = oracle.NF4_TABLE
    rows = []
    rows.append(np.zeros(128, np.float32))
    r = np.zeros(128, np.float32)
    r[:64] = -0.0
    r[64:] = np.float32(1e-3)
    rows.append(r)
    # exact midpoint ties at several scales (m6 = NF4[6]/2, m7 = NF4[8]/2 are fp32)
    for p in (-100, -20, 0, 20, 100):
        s = np.float32(2.0 ** p)
        r = np.zeros(128, np.float32)
        r[0] = s
        r[1] = np.float32(t[6]) / 2 * s
        r[2] = np.float32(t[8]) / 2 * s
        r[3] = -np.float32(t[6]) / 2 * s
        r[64] = -s
        r[65:81] = (t * s).astype(np.float32)
        rows.append(r)
    # the 16 levels reproduced at awkward absmax values
    for a in (np.float32(3.0e38), np.float32(1.1754944e-38), np.float32(1e-40),
              np.float32(0.0213), np.float32(7.0)):
        rows.append(np.tile((t * a).astype(np.float32), 8))
    # single outlier per block, and wildly different absmax across blocks
    rng = np.random.default_rng(5)
    r = (rng.standard_normal(128) * 1e-3).astype(np.float32)
    r[7], r[100] = 50.0, -3.0e5
    rows.append(r)
    r = (rng.standard_normal(128)).astype(np.float32)
    r[:64] *= np.float32(1e-30)
    r[64:] *= np.float32(1e30)
    rows.append(r)
    return np.stack(rows)[None]


@pytest.mark.parametrize("absmax_dtype", ["f32", "bf16"])
def test_pack_adversarial_fp32(absmax_dtype):
    w = _adversarial_rows()
    _compare(w, torch.from_numpy(w).to(DEV), "adversarial fp32", absmax_dtype)


@pytest.mark.parametrize("absmax_dtype", ["f32", "bf16"])
def test_pack_adversarial_bf16(absmax_dtype):
    from grouped_nf4_expert_amd.workloads import bf16_round
    w = bf16_round(_adversarial_rows())
    _compare(w, bf16_dev(w), "adversarial bf16", absmax_dtype)


@pytest.mark.parametrize("name,gemm", [("olmoe", "gate_up"), ("gptoss", "down")])
def test_pack_bf16_absmax_workload_experts(name, gemm):
    """The 4.25-bit form: absmax rounded to bf16, codes against the stored value."""
    wl = wls.WORKLOADS[name]
    w = np.stack([wls.expert_weights(wl, gemm, e) for e in range(2)])
    _compare(w, bf16_dev(w), f"{name}/{gemm}", "bf16")


def test_pack_bf16_absmax_rounding_edges():
    """Block maxima just below / at / above bf16 rounding midpoints, and
    the saturation at the largest finite bf16."""
    rng = np.random.default_rng(77)
    rows = []
    for m in (1.00390625, 1.0039, 1.0040, 1.01171875, 3.3895e38, 3.4e38, 1e-39, 7.5e-41):
        r = (rng.uniform(-1, 1, 128) * np.float32(m)).astype(np.float32)
        r[3] = np.float32(m)
        r[70] = -np.float32(m)
        rows.append(r)
    w = np.stack(rows)[None]
    _compare(w, torch.from_numpy(w).to(DEV), "bf16 absmax rounding edges", "bf16")


def test_pack_full_size_expert_device_generated():
    """One DeepSeek-V3 gate_up expert (4096 x 7168) drawn on the device."""
    wl = wls.WORKLOADS["dsv3"]
    w_dev = wls.expert_weights_device(wl, "gate_up", 17, DEV)
    w_host = w_dev.float().cpu().numpy()
    _compare(w_host, w_dev, "dsv3 gate_up expert 17")


def test_pack_rejects_host_tensor():
    w = torch.zeros((1, 4, 64), dtype=torch.bfloat16)
    packed = torch.zeros((1, 4, 32), dtype=torch.uint8, device=DEV)
    absmax = torch.zeros((1, 4, 1), dtype=torch.float32, device=DEV)
    with pytest.raises(gnf4.Gnf4Error, match="oracle"):
        gnf4.pack(w, out=(packed, absmax))
