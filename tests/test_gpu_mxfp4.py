"""GPU parity for gnf4_grouped_gemm_mxfp4 against the fp64 MXFP4 oracle:
random E2M1 code bytes and E8M0 scales (any byte is a valid code pair), the
workloads' shapes with and without the fused gather on both the decode and
the matrix-core tile path, K splits, the grouping boundary cases, scale edge
values (2^-127, 2^127, NaN), the tile path's exact range of scales within a
weight row, activation magnitudes far outside fp16, GPT-OSS's whole stack (the
model family released in MXFP4) and DeepSeek-V3's prefill shapes at full size
(sampled outputs).

Bar: |y - o| <= 8e-3 |o| + 1e-3 rms(o), as the NF4 GEMM.
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

from test_gpu_full_size import complete_groups
from gpu_util import DEV, bf16_dev, check_gemm, host_f64, note
from test_gpu_gemm import BOUNDARY_CASES

pytestmark = pytest.mark.gpu

DEC, TILE, AUTO = gnf4.PATH_DECODE, gnf4.PATH_TILE, gnf4.PATH_AUTO


def _stack(E, N, K, seed, lo=118, hi=131):
    g = torch.Generator(device=DEV).manual_seed(seed)
    packed = torch.randint(0, 256, (E, N, K // 2), dtype=torch.uint8, device=DEV, generator=g)
    scales = torch.randint(lo, hi, (E, N, K // 32), dtype=torch.uint8, device=DEV, generator=g)
    return packed, scales


def _oracle(x_host, packed, scales, sizes, ids):
    return oracle.ref_grouped_gemm_mxfp4(x_host, packed.cpu().numpy(), scales.cpu().numpy(),
                                         sizes, ids)


@pytest.mark.parametrize("name,gemm", [("tiny", "w"), ("olmoe", "gate_up"), ("olmoe", "down"),
                                       ("qwen3_t8", "gate_up"), ("gptoss", "gate_up"),
                                       ("gptoss", "down"), ("gptoss_t256", "down")])
@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("path", [DEC, TILE])
def test_mxfp4_workload_shapes(name, gemm, gather, path):
    wl = wls.WORKLOADS[name]
    K, N = wl.gemm(gemm)
    logits = wls.router_logits(wl)
    ref = oracle.ref_route_sort(logits, wl.top_k)
    r = gnf4.route_sort(torch.from_numpy(logits).to(DEV), wl.top_k)
    packed, scales = _stack(wl.E, N, K, seed=K + N)
    x_tok = wls.token_activations(wl, K)
    x_host = x_tok[ref["sorted_slots"] // wl.top_k]
    note(f"mxfp4 {name}/{gemm} gather={gather} path={path}")
    if gather:
        y = gnf4.grouped_gemm_mxfp4(bf16_dev(x_tok), packed, scales, r.group_sizes,
                                    r.group_expert_ids, path=path, sorted_slots=r.sorted_slots,
                                    top_k=wl.top_k)
    else:
        xs = gnf4.gather_rows(bf16_dev(x_tok), r.sorted_slots, wl.top_k)
        y = gnf4.grouped_gemm_mxfp4(xs, packed, scales, r.group_sizes, r.group_expert_ids,
                                    path=path)
    torch.cuda.synchronize()
    o, written = _oracle(x_host, packed, scales, ref["group_sizes"], ref["group_expert_ids"])
    check_gemm(y, o, written, f"mxfp4 {name}/{gemm} path {path}")


@pytest.mark.parametrize("split_k", [1, 2, 3, 5])
def test_mxfp4_split_k(split_k):
    wl = wls.WORKLOADS["gptoss"]
    K, N = wl.gemm("down")
    logits = wls.router_logits(wl)
    ref = oracle.ref_route_sort(logits, wl.top_k)
    r = gnf4.route_sort(torch.from_numpy(logits).to(DEV), wl.top_k)
    packed, scales = _stack(wl.E, N, K, seed=7)
    x = bf16_dev(np.random.default_rng(7).standard_normal((wl.M, K)))
    note(f"mxfp4 split_k={split_k}")
    y = gnf4.grouped_gemm_mxfp4(x, packed, scales, r.group_sizes, r.group_expert_ids,
                                path=DEC, split_k=split_k)
    torch.cuda.synchronize()
    o, written = _oracle(host_f64(x), packed, scales, ref["group_sizes"], ref["group_expert_ids"])
    check_gemm(y, o, written, f"mxfp4 split {split_k}")


@pytest.mark.parametrize("case", sorted(BOUNDARY_CASES))
@pytest.mark.parametrize("path", [DEC, TILE])
def test_mxfp4_boundaries(case, path):
    E, N, K, sizes, ids, M = BOUNDARY_CASES[case]
    note(f"mxfp4 boundary {case} path={path}")
    packed, scales = _stack(E, N, K, seed=31)
    x = bf16_dev(np.random.default_rng(31).standard_normal((M, K)))
    full = torch.full((M + 2, N), -512.0, dtype=torch.bfloat16, device=DEV)
    y = full[1:M + 1]
    st = torch.tensor(sizes, dtype=torch.int32, device=DEV)
    it = torch.tensor(ids, dtype=torch.int32, device=DEV)
    gnf4.grouped_gemm_mxfp4(x, packed, scales, st, it, G=len(sizes), y=y, path=path)
    torch.cuda.synchronize()
    o, written = _oracle(host_f64(x), packed, scales, sizes, ids)
    f = full.float().cpu().numpy()
    assert np.all(f[0] == -512.0) and np.all(f[M + 1] == -512.0), "guard rows written"
    assert np.all(f[1:M + 1][~written] == -512.0), "uncovered rows written"
    if written.any():
        check_gemm(y, o, written, f"mxfp4 {case} path {path}")


@pytest.mark.parametrize("path", [DEC, TILE])
def test_mxfp4_scale_edges_and_nan(path):
    """Expert 0 reads only blocks scaled 2^-127 (E8M0 0x00, a subnormal fp32)
    and 2^-126 (0x01), against activations near 1e30; expert 1 has a block
    scaled 2^127 (0xFE) against activations near 1e-30, and one NaN scale
    (0xFF) that must poison exactly the outputs of its weight row.

    The tile path stages activations and codes in fp16 with one power of two
    per activation row and per weight row, so it keeps a block exact only
    within 23 binades of its weight row's largest scale
    (test_mxfp4_tile_scale_range) and flushes activations 2^24 below their
    row's largest: there expert 0's other blocks sit at 2^-126 too, and the
    activations against the 2^127 block are 2^-10 (an activation of 1e-30
    against 2^127 next to ordinary products is outside that path's range)."""
    E, N, K, M = 2, 64, 256, 6
    packed, _ = _stack(E, N, K, seed=41)
    scales = torch.full((E, N, K // 32), 127, dtype=torch.uint8, device=DEV)
    if path == TILE:
        scales[0] = 1
    scales[0, :, 0] = 0
    scales[0, :, 1] = 1
    scales[1, :, 3] = 254
    scales[1, 5, 2] = 255          # NaN block in weight row n = 5 of expert 1
    rng = np.random.default_rng(41)
    mag = rng.uniform(0.5, 1.5, (M, K)) * np.sign(rng.standard_normal((M, K)))
    x = np.zeros((M, K), np.float32)
    x[:3, :64] = (mag[:3, :64] * 1e30).astype(np.float32)     # expert 0: blocks 0 and 1 only
    x[3:] = mag[3:].astype(np.float32)
    x[3:, 96:128] = (mag[3:, 96:128] * (1e-30 if path == DEC else 2.0 ** -10)).astype(np.float32)
    xd = bf16_dev(x)
    sizes, ids = [3, 3], [0, 1]
    note(f"mxfp4 scale edges path={path}")
    y = gnf4.grouped_gemm_mxfp4(xd, packed, scales, torch.tensor(sizes, dtype=torch.int32,
                                device=DEV), torch.tensor(ids, dtype=torch.int32, device=DEV),
                                path=path)
    torch.cuda.synchronize()
    o, written = _oracle(host_f64(xd), packed, scales, sizes, ids)
    g = host_f64(y)
    nan_ref = np.isnan(o)
    assert np.array_equal(np.isnan(g), nan_ref), "NaN positions differ"
    assert nan_ref[3:, 5].all() and nan_ref.sum() == 3
    for rows, what in ((slice(0, 3), "2^-127 / 2^-126 scales"), (slice(3, 6), "2^127 scale")):
        ok = ~nan_ref[rows]
        oo, gg = o[rows][ok], g[rows][ok]
        rms = float(np.sqrt(np.mean(oo ** 2)))
        assert rms > 0
        bad = np.abs(gg - oo) > 8e-3 * np.abs(oo) + 1e-3 * rms
        assert not bad.any(), f"{what}: {int(bad.sum())} outside tolerance"


def test_mxfp4_gptoss_full_stack():
    """GPT-OSS-120B-shaped gate_up: all 128 experts' MXFP4 bytes resident,
    routed decode batch (T=1, k=4), every output checked."""
    wl = wls.WORKLOADS["gptoss"]
    K, N = wl.gemm("gate_up")
    note(f"mxfp4 full stack gptoss gate_up E={wl.E} N={N} K={K}")
    packed, scales = _stack(wl.E, N, K, seed=99, lo=115, hi=128)
    logits = wls.router_logits(wl)
    ref = oracle.ref_route_sort(logits, wl.top_k)
    r = gnf4.route_sort(torch.from_numpy(logits).to(DEV), wl.top_k)
    x_tok = wls.token_activations(wl, K)
    y = gnf4.grouped_gemm_mxfp4(bf16_dev(x_tok), packed, scales, r.group_sizes,
                                r.group_expert_ids, sorted_slots=r.sorted_slots, top_k=wl.top_k)
    torch.cuda.synchronize()
    used = ref["group_expert_ids"][: ref["num_groups"]]
    p = packed[torch.from_numpy(used.astype(np.int64)).to(DEV)].cpu().numpy()
    s = scales[torch.from_numpy(used.astype(np.int64)).to(DEV)].cpu().numpy()
    x_host = x_tok[ref["sorted_slots"] // wl.top_k]
    ids_local = np.arange(len(used), dtype=np.int32)
    o, written = oracle.ref_grouped_gemm_mxfp4(x_host, p, s, ref["group_sizes"][: len(used)],
                                               ids_local)
    check_gemm(y, o, written, "mxfp4 gptoss full stack")


def test_mxfp4_tile_scale_range():
    """The tile path converts each code to fp16 times 2^(s - s_max), s_max the
    largest scale of its weight row: exact for every E2M1 value while
    s >= s_max - 23.  Rows whose scales span exactly 23 binades, with the
    activations against the small blocks 2^26 times those against the large
    ones, so the small blocks carry most of each output."""
    E, N, K, M = 2, 96, 512, 40
    packed, _ = _stack(E, N, K, seed=43)
    g = torch.Generator(device=DEV).manual_seed(43)
    base = torch.randint(100, 150, (E, N, 1), dtype=torch.int32, device=DEV, generator=g)
    nb = K // 32
    off = torch.zeros((E, N, nb), dtype=torch.int32, device=DEV)
    off[:, :, 1::2] = -23                       # odd blocks: 23 binades below the row's max
    scales = (base + off).to(torch.uint8)
    rng = np.random.default_rng(43)
    x = rng.standard_normal((M, K))
    for b in range(1, nb, 2):
        x[:, 32 * b:32 * (b + 1)] *= 2.0 ** 26
    xd = bf16_dev(x)
    sizes, ids = [24, 16], [1, 0]
    note("mxfp4 tile scale range")
    y = gnf4.grouped_gemm_mxfp4(xd, packed, scales, torch.tensor(sizes, dtype=torch.int32,
                                device=DEV), torch.tensor(ids, dtype=torch.int32, device=DEV),
                                path=TILE)
    torch.cuda.synchronize()
    o, written = _oracle(host_f64(xd), packed, scales, sizes, ids)
    check_gemm(y, o, written, "mxfp4 tile scale range")


@pytest.mark.parametrize("scale", [1e-20, 5e4, 1e30])
def test_mxfp4_tile_activation_magnitudes(scale):
    """Activation rows far outside fp16's range mixed with ordinary rows and
    an all-zero row, on the tile path (its per-row power-of-two staging, in
    the K order the MXFP4 convert produces); the bar holds per class."""
    E, N, K, M = 3, 96, 512, 48
    packed, scales = _stack(E, N, K, seed=44)
    rng = np.random.default_rng(44)
    f = np.ones((M, 1))
    f[::3] = scale
    f[7] = 0.0
    xd = bf16_dev((rng.standard_normal((M, K)) * f).astype(np.float32))
    sizes, ids = [20, 12, 16], [2, 0, 1]
    note(f"mxfp4 tile activation magnitude {scale:g}")
    y = gnf4.grouped_gemm_mxfp4(xd, packed, scales, torch.tensor(sizes, dtype=torch.int32,
                                device=DEV), torch.tensor(ids, dtype=torch.int32, device=DEV),
                                path=TILE)
    torch.cuda.synchronize()
    o, written = _oracle(host_f64(xd), packed, scales, sizes, ids)
    cls = np.zeros(M, bool)
    cls[::3] = True
    for what, mask in (("scaled", cls), ("ordinary", ~cls)):
        check_gemm(y, o, written & mask, f"mxfp4 x*{scale:g} {what} rows")
    assert np.all(host_f64(y)[7] == 0.0)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("gemm", ["gate_up", "down"])
def test_mxfp4_dsv3_prefill_sampled(gemm):
    """DeepSeek-V3-shaped prefill (E=256, T=4096, k=8) over a random MXFP4
    stack on the automatic path (every group on the tile path) with the fused
    gather; run twice (deterministic); the oracle recomputes every output of
    four complete groups (first, last, largest, smallest), sampled outputs of
    48 more groups and every 64th column of the first and last rows."""
    wl = wls.WORKLOADS["dsv3"]
    K, N = wl.gemm(gemm)
    note(f"mxfp4 full-size dsv3/{gemm}: stack E={wl.E} N={N} K={K}")
    packed, scales = _stack(wl.E, N, K, seed=45, lo=112, hi=126)
    logits = wls.router_logits(wl)
    r = gnf4.route_sort(torch.from_numpy(logits).to(DEV), wl.top_k)
    ref = oracle.ref_route_sort(logits, wl.top_k)
    x_tok = wls.token_activations(wl, K)
    xd = bf16_dev(x_tok)
    note(f"mxfp4 full-size dsv3/{gemm}: grouped GEMM (automatic path)")
    y = gnf4.grouped_gemm_mxfp4(xd, packed, scales, r.group_sizes, r.group_expert_ids,
                                sorted_slots=r.sorted_slots, top_k=wl.top_k)
    y2 = gnf4.grouped_gemm_mxfp4(xd, packed, scales, r.group_sizes, r.group_expert_ids,
                                 sorted_slots=r.sorted_slots, top_k=wl.top_k)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "not deterministic"
    yh = host_f64(y)
    assert np.all(np.isfinite(yh))
    groups = oracle.ref_group_rows(ref["group_sizes"], ref["group_expert_ids"], wl.E, wl.M)
    rng = np.random.default_rng(46)
    picks = [(int(rng.integers(r0, r1)), int(rng.integers(0, N)), int(e))
             for gi in rng.choice(len(groups), 48, replace=False)
             for (_g, e, r0, r1) in [groups[gi]] for _ in range(8)]
    for (_g, e, r0, r1), rr in ((groups[-1], groups[-1][3] - 1), (groups[0], groups[0][2])):
        picks += [(int(rr), n, int(e)) for n in range(0, N, max(1, N // 64))]
    rows = np.array([p[0] for p in picks])
    cols = np.array([p[1] for p in picks])
    wcache = {}
    expect = np.zeros(len(picks))
    for i, (rr, n, e) in enumerate(picks):
        key = (e, n)
        if key not in wcache:
            wcache[key] = oracle.ref_mx_unpack(packed[e, n:n + 1].cpu().numpy(),
                                               scales[e, n:n + 1].cpu().numpy())[0]
        expect[i] = x_tok[ref["sorted_slots"][rr] // wl.top_k].astype(np.float64) @ wcache[key]
    got = yh[rows, cols]
    rms = float(np.sqrt(np.mean(expect ** 2)))
    bad = np.abs(got - expect) > 8e-3 * np.abs(expect) + 1e-3 * rms
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} sampled outputs outside tolerance"
    # every output of four complete groups: first, last, largest, smallest
    for g, e, r0, r1 in complete_groups(groups):
        note(f"mxfp4 full-size dsv3/{gemm}: group {g} (expert {e}, {r1 - r0} rows) in full")
        wt = oracle.ref_mx_unpack(packed[e].cpu().numpy(), scales[e].cpu().numpy())
        xr = x_tok[ref["sorted_slots"][r0:r1] // wl.top_k].astype(np.float64)
        check_gemm(y[r0:r1], xr @ np.asarray(wt, np.float64).T, np.ones(r1 - r0, bool),
                   f"mxfp4 dsv3/{gemm} group {g} (expert {e}, {r1 - r0} rows)")
