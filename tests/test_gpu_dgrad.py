"""GPU parity for gnf4_grouped_dgrad (dx = dy . W per group) against the
fp64 oracle, on the GEMV path and the matrix-core tile path: the workloads'
shapes, the grouping boundary cases, adversarial absmax, dy rows far outside
fp16's range, the unsplit fallback, determinism, and the DSV3 down stack at
full size (sampled rows, automatic path = tile path).

Bar: |dx - o| <= 8e-3 |o| + 1e-3 rms(o) element by element, the forward
GEMM's bound.
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

from gpu_util import DEV, bf16_dev, check_gemm, host_f64, note, routed_stack
from test_gpu_gemm import BOUNDARY_CASES
from test_gpu_full_size import device_stack, host_expert

pytestmark = pytest.mark.gpu

DEC, TILE, AUTO = gnf4.PATH_DECODE, gnf4.PATH_TILE, gnf4.PATH_AUTO


def _oracle_stack(wl, host, N, K):
    p = np.zeros((wl.E, N, K // 2), np.uint8)
    a = np.zeros((wl.E, N, K // 64), np.float32)
    for e, w in host.items():
        p[e], a[e] = oracle.ref_pack(w)
    return p, a


@pytest.mark.parametrize("name,gemm", [("tiny", "w"), ("olmoe", "gate_up"), ("olmoe", "down"),
                                       ("qwen3_t8", "gate_up"), ("gptoss", "gate_up"),
                                       ("gptoss", "down"), ("gptoss_t256", "down")])
@pytest.mark.parametrize("path", [DEC, TILE])
def test_dgrad_workload_shapes(name, gemm, path):
    wl = wls.WORKLOADS[name]
    K, N = wl.gemm(gemm)
    logits = wls.router_logits(wl)
    ref = oracle.ref_route_sort(logits, wl.top_k)
    r = gnf4.route_sort(torch.from_numpy(logits).to(DEV), wl.top_k)
    used = ref["group_expert_ids"][: ref["num_groups"]]
    packed, absmax, host = routed_stack(wl, gemm, used)
    dy = bf16_dev(np.random.default_rng(K + N).standard_normal((wl.M, N)))
    note(f"dgrad {name}/{gemm} M={wl.M} N={N} K={K} path={path}")
    dx = gnf4.grouped_dgrad(dy, packed, absmax, r.group_sizes, r.group_expert_ids, path=path)
    torch.cuda.synchronize()
    p, a = _oracle_stack(wl, host, N, K)
    o, written = oracle.ref_grouped_dgrad(host_f64(dy), p, a, ref["group_sizes"],
                                          ref["group_expert_ids"])
    check_gemm(dx, o, written, f"dgrad {name}/{gemm} path {path}")


def _custom(E, N, K, sizes, ids, M, seed, w_scale=None, dy_scale=None):
    rng = np.random.default_rng(seed)
    w = wls.bf16_round((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    if w_scale is not None:
        w = wls.bf16_round(w * w_scale)
    dy = rng.standard_normal((M, N)).astype(np.float32)
    if dy_scale is not None:
        dy = dy * dy_scale
    dy = wls.bf16_round(dy.astype(np.float32))
    packed, absmax = gnf4.pack(bf16_dev(w))
    p, a = oracle.ref_pack(w)
    o, written = oracle.ref_grouped_dgrad(dy, p, a, sizes, ids)
    return dict(dy=bf16_dev(dy), packed=packed, absmax=absmax, o=o, written=written,
                sizes=torch.tensor(sizes, dtype=torch.int32, device=DEV),
                ids=torch.tensor(ids, dtype=torch.int32, device=DEV), M=M, K=K)


def _run(c, workspace=None, path=AUTO):
    M, K = c["M"], c["K"]
    full = torch.full((M + 2, K), -512.0, dtype=torch.bfloat16, device=DEV)
    dx = full[1:M + 1]
    gnf4.grouped_dgrad(c["dy"], c["packed"], c["absmax"], c["sizes"], c["ids"],
                       G=c["sizes"].numel(), dx=dx, workspace=workspace, path=path)
    torch.cuda.synchronize()
    f = full.float().cpu().numpy()
    assert np.all(f[0] == -512.0) and np.all(f[M + 1] == -512.0), "guard rows written"
    assert np.all(f[1:M + 1][~c["written"]] == -512.0), "uncovered rows written"
    return dx


@pytest.mark.parametrize("case", sorted(BOUNDARY_CASES))
@pytest.mark.parametrize("path", [AUTO, DEC, TILE])
def test_dgrad_boundaries(case, path):
    E, N, K, sizes, ids, M = BOUNDARY_CASES[case]
    note(f"dgrad boundary {case} path={path}")
    c = _custom(E, N, K, sizes, ids, M, seed=21)
    dx = _run(c, path=path)
    if c["written"].any():
        check_gemm(dx, c["o"], c["written"], f"dgrad {case} path {path}")


# The tile path stages dy rows of any width N, from a dy that is only 2-byte
# aligned (element by element); a prefill-sized batch takes it automatically.
@pytest.mark.parametrize("N", [1, 7, 301])
@pytest.mark.parametrize("path", [AUTO, TILE])
def test_dgrad_tile_any_width_unaligned_dy(N, path):
    note(f"dgrad tile N={N} unaligned dy path={path}")
    c = _custom(3, N, 256, [30, 34], [2, 0], 64, seed=N)
    flat = torch.empty(64 * N + 1, dtype=torch.bfloat16, device=DEV)
    dy = flat[1:].view(64, N)
    dy.copy_(c["dy"])
    assert dy.data_ptr() % 16 != 0
    c["dy"] = dy
    dx = _run(c, path=path)
    check_gemm(dx, c["o"], c["written"], f"dgrad N={N} unaligned path {path}")


# Rows of 10, 16, 24 and 32 chunks of 32 codes: the decode path's teams of
# 16, 16, 32 and 32 lanes (several weight rows per wavefront), with groups of
# one row (one workgroup slot per row) and of several rows (R > 1, and groups
# whose rows take separate slots).
@pytest.mark.parametrize("K", [320, 512, 768, 1024])
@pytest.mark.parametrize("sizes,ids,M", [([1, 1, 1, 1], [3, 0, 2, 1], 4),
                                         ([1, 3, 2, 1], [2, 0, 3, 1], 7),
                                         ([5, 3], [1, 2], 8)])
def test_dgrad_team_widths(K, sizes, ids, M):
    note(f"dgrad team widths K={K} sizes={sizes}")
    c = _custom(4, 200, K, sizes, ids, M, seed=K + M)
    dx = _run(c, path=DEC)
    check_gemm(dx, c["o"], c["written"], f"dgrad K={K} sizes={sizes}")


@pytest.mark.parametrize("sizes,M,splits", [([1, 1, 1], 3, 48), ([2, 2, 2], 6, 24)])
def test_dgrad_many_splits(sizes, M, splits):
    """Three groups of K = 2048 over N = 1536 weight rows.  One row each: the
    launch rule takes batches of 4 weight rows per team and splits N 48 ways
    (three full batches of split partials in the reduce).  Two rows each:
    batches of 8 and 24 splits, so the reduce's second batch is padded."""
    note(f"dgrad {splits} N splits, sizes {sizes}")
    lib = gnf4.library()
    assert lib.gnf4_grouped_dgrad_workspace_size(M, 1536, 2048, 3, 4) == splits * M * 2048 * 4
    c = _custom(4, 1536, 2048, sizes, [0, 2, 3], M, seed=24 + M)
    dx = _run(c, workspace=None, path=DEC)
    check_gemm(dx, c["o"], c["written"], f"dgrad {splits} splits")


def test_dgrad_ragged_splits_four_row_batches():
    """Eight one-row groups of K = 1024 (32-lane teams) over N = 1000 weight
    rows: batches of 4 rows per team, 16 splits of 63 rows, so every split
    ends inside a batch and the last one holds 55 rows."""
    note("dgrad ragged N=1000, batches of 4")
    lib = gnf4.library()
    assert lib.gnf4_grouped_dgrad_workspace_size(8, 1000, 1024, 8, 64) == 16 * 8 * 1024 * 4
    c = _custom(8, 1000, 1024, [1] * 8, [5, 1, 7, 0, 3, 6, 2, 4], 8, seed=1000)
    dx = _run(c, workspace=None, path=DEC)
    check_gemm(dx, c["o"], c["written"], "dgrad ragged N=1000")


def _absmax_scenarios(E, N, K):
    """Weight magnitudes that stress the tile path's per-column-block scale:
    blocks alternating 1e-30 / 1e30 along K, one row 1e4 above the others,
    zero blocks, one large element per block, rows spread over 20 binades."""
    s = {}
    a = np.ones((E, N, K), np.float32)
    for b in range(K // 64):
        a[:, :, 64 * b:64 * (b + 1)] = 1e-30 if b % 2 else 1e30
    s["blocks_1e-30_to_1e30"] = a
    z = np.ones((E, N, K), np.float32)
    z[:, :, 64:192] = 0.0
    z[:, 3, :] = 1e4
    s["zero_blocks_outlier_row"] = z
    p = np.ones((E, N, K), np.float32)
    p[:, :, ::64] = 500.0
    s["one_outlier_per_block"] = p
    s["rows_over_20_binades"] = np.ones((E, N, K), np.float32) * (
        2.0 ** -(np.arange(N) % 20)).astype(np.float32)[None, :, None]
    return s


@pytest.mark.parametrize("scenario", sorted(_absmax_scenarios(1, 8, 128)))
@pytest.mark.parametrize("path", [DEC, TILE])
def test_dgrad_adversarial_absmax(scenario, path):
    E, N, K, M = 3, 64, 512, 96
    scale = _absmax_scenarios(E, N, K)[scenario]
    note(f"dgrad adversarial absmax {scenario} path={path}")
    c = _custom(E, N, K, [40, 24, 32], [2, 0, 1], M, seed=23, w_scale=scale)
    dx = _run(c, path=path)
    check_gemm(dx, c["o"], c["written"], f"dgrad {scenario} path {path}")


@pytest.mark.parametrize("scale", [1e-20, 5e4, 1e30])
def test_dgrad_tile_dy_magnitudes(scale):
    """dy rows far outside fp16's range mixed with ordinary rows and a zero
    row; the tile path scales each dy row by its own power of two, so each
    class meets the bar on its own."""
    E, N, K, M = 3, 96, 256, 72
    f = np.ones((M, 1), np.float32)
    f[::3] = scale
    f[7] = 0.0
    c = _custom(E, N, K, [30, 20, 22], [1, 2, 0], M, seed=24, dy_scale=f)
    note(f"dgrad tile dy magnitude {scale:g}")
    dx = _run(c, path=TILE)
    cls = np.zeros(M, bool)
    cls[::3] = True
    for what, mask in (("scaled", cls), ("ordinary", ~cls)):
        check_gemm(dx, c["o"], c["written"] & mask, f"dgrad dy*{scale:g} {what} rows")
    assert np.all(host_f64(dx)[7] == 0.0)


def test_dgrad_unsplit_fallback_and_determinism():
    c = _custom(6, 1536, 2880, [1, 3, 1, 2, 1], [5, 0, 2, 4, 1], 8, seed=22)
    note("dgrad split vs unsplit")
    a = _run(c).clone()
    b = _run(c).clone()
    assert torch.equal(a, b), "not deterministic"
    tiny_ws = torch.empty(16, dtype=torch.uint8, device=DEV)   # too small: one split
    u = _run(c, workspace=tiny_ws)
    check_gemm(a, c["o"], c["written"], "dgrad split")
    check_gemm(u, c["o"], c["written"], "dgrad unsplit")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("gemm", ["down", "gate_up"])
def test_dgrad_dsv3_full_size_sampled_rows(gemm):
    """DSV3 stacks (down: E=256, N=7168 rows reduced, K=2048; gate_up:
    N=4096 reduced, K=7168) with every routed row, on the automatic (tile)
    path; the oracle recomputes up to 24 rows of 3 experts in full."""
    wl = wls.WORKLOADS["dsv3"]
    K, N = wl.gemm(gemm)
    note(f"dgrad full size dsv3/{gemm}: generate + pack {wl.E} experts")
    packed, absmax = device_stack(wl, gemm)
    logits = wls.router_logits(wl)
    ref = oracle.ref_route_sort(logits, wl.top_k)
    r = gnf4.route_sort(torch.from_numpy(logits).to(DEV), wl.top_k)
    gen = torch.Generator(device=DEV).manual_seed(3)
    dy = torch.randn((wl.M, N), device=DEV, generator=gen).to(torch.bfloat16)
    note(f"dgrad full size dsv3/{gemm}: run")
    dx = gnf4.grouped_dgrad(dy, packed, absmax, r.group_sizes, r.group_expert_ids)
    torch.cuda.synchronize()
    groups = oracle.ref_group_rows(ref["group_sizes"], ref["group_expert_ids"], wl.E, wl.M)
    rng = np.random.default_rng(5)
    for gi in rng.choice(len(groups), 3, replace=False):
        _g, e, r0, r1 = groups[gi]
        rows = np.unique(np.concatenate([[r0, r1 - 1], rng.integers(r0, r1, 6)]))
        p, a = oracle.ref_pack(host_expert(wl, gemm, int(e)))
        w = oracle.ref_unpack(p, a).astype(np.float64)
        idx = torch.from_numpy(rows.astype(np.int64)).to(DEV)
        o = host_f64(dy[idx]) @ w
        got = dx[idx]
        check_gemm(got, o, np.ones(rows.size, bool), f"dsv3 dgrad expert {e}")


@pytest.mark.parametrize("name,gemm", [("olmoe", "down"), ("gptoss_t256", "down")])
@pytest.mark.parametrize("path", [DEC, TILE])
def test_dgrad_bf16_absmax(name, gemm, path):
    wl = wls.WORKLOADS[name]
    K, N = wl.gemm(gemm)
    logits = wls.router_logits(wl)
    ref = oracle.ref_route_sort(logits, wl.top_k)
    r = gnf4.route_sort(torch.from_numpy(logits).to(DEV), wl.top_k)
    used = sorted(set(int(e) for e in ref["group_expert_ids"][: ref["num_groups"]]))
    packed = torch.full((wl.E, N, K // 2), 0xFF, dtype=torch.uint8, device=DEV)
    absmax = torch.full((wl.E, N, K // 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    p_ref = np.zeros((wl.E, N, K // 2), np.uint8)
    a_ref = np.zeros((wl.E, N, K // 64), np.float32)
    for e in used:
        w = wls.expert_weights(wl, gemm, e)
        gnf4.pack(bf16_dev(w), out=(packed[e], absmax[e]))
        p_ref[e], a_ref[e] = oracle.ref_pack(w, absmax_dtype="bf16")
    dy = bf16_dev(np.random.default_rng(9).standard_normal((wl.M, N)))
    note(f"dgrad bf16 absmax {name}/{gemm} path={path}")
    dx = gnf4.grouped_dgrad(dy, packed, absmax, r.group_sizes, r.group_expert_ids, path=path)
    torch.cuda.synchronize()
    o, written = oracle.ref_grouped_dgrad(host_f64(dy), p_ref, a_ref, ref["group_sizes"],
                                          ref["group_expert_ids"])
    check_gemm(dx, o, written, f"dgrad bf16 absmax {name}/{gemm}")


@pytest.mark.parametrize("gap", [8, 16, 24])
@pytest.mark.parametrize("path", [DEC, TILE])
def test_dgrad_block_range(gap, path):
    """Weight rows 2^gap below the largest in every column block carry the
    whole gradient: dy is zero against the large (even) rows.  The tile path
    scales each 64-column block of K so its largest absmax over the N rows
    lands in [2^14, 2^15), so blocks within 2^25 of it decode exactly."""
    E, N, K, M = 2, 128, 512, 40
    w_scale = np.ones((E, N, K), np.float32)
    w_scale[:, 1::2, :] = 2.0 ** -gap
    dy_scale = np.ones((M, N), np.float32)
    dy_scale[:, 0::2] = 0.0
    c = _custom(E, N, K, [24, 16], [1, 0], M, seed=90 + gap, w_scale=w_scale, dy_scale=dy_scale)
    note(f"dgrad block range 2^-{gap} path={path}")
    dx = gnf4.grouped_dgrad(c["dy"], c["packed"], c["absmax"], c["sizes"], c["ids"], path=path)
    torch.cuda.synchronize()
    check_gemm(dx, c["o"], c["written"], f"dgrad block gap 2^{gap} path {path}")

