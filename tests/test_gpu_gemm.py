"""GPU parity for gnf4_grouped_gemm: both kernel paths, every decode-path
split, the workloads' shapes and the boundary cases, against the fp64 oracle.

Bar: |y - o| <= 8e-3 |o| + 1e-3 rms(o) element by element (o = exact fp64
result of the decoded weights); bit-exact where the arithmetic is exact
(one-hot activations on the fp32 decode path).
"""

import numpy as np
import pytest
import torch

import oracle
from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

from gpu_util import DEV, bf16_dev, check_gemm, host_f64, note, routed_stack

pytestmark = pytest.mark.gpu

DEC, TILE, AUTO = gnf4.PATH_DECODE, gnf4.PATH_TILE, gnf4.PATH_AUTO


def _workload_case(name, gemm, layer=0):
    """GPU routing + gather + packed stack, and the oracle's own versions."""
    wl = wls.WORKLOADS[name]
    K, N = wl.gemm(gemm)
    logits = wls.router_logits(wl, layer)
    ref = oracle.ref_route_sort(logits, wl.top_k)
    r = gnf4.route_sort(torch.from_numpy(logits).to(DEV), wl.top_k)
    used = ref["group_expert_ids"][: ref["num_groups"]]
    packed, absmax, host = routed_stack(wl, gemm, used, layer)
    if gemm == "down":
        x_host = wls.down_input(wl, wl.M, K, layer)
        xs = bf16_dev(x_host)
    else:
        x_tok = wls.token_activations(wl, K, layer)
        x_host = x_tok[ref["sorted_slots"] // wl.top_k]
        xs = gnf4.gather_rows(bf16_dev(x_tok), r.sorted_slots, wl.top_k)
    # oracle: its own packing of the same bf16 weights, its own routing
    p_ref = np.zeros((wl.E, N, K // 2), np.uint8)
    a_ref = np.zeros((wl.E, N, K // 64), np.float32)
    for e, w in host.items():
        p_ref[e], a_ref[e] = oracle.ref_pack(w)
    y_ref, written = oracle.ref_grouped_gemm(x_host, p_ref, a_ref, ref["group_sizes"],
                                             ref["group_expert_ids"])
    return dict(wl=wl, K=K, N=N, r=r, xs=xs, packed=packed, absmax=absmax, y_ref=y_ref,
                written=written, x_host=x_host, p_ref=p_ref, a_ref=a_ref, ref=ref)


def _gemm(c, path, split_k=0, G=None):
    return gnf4.grouped_gemm(c["xs"], c["packed"], c["absmax"], c["r"].group_sizes,
                             c["r"].group_expert_ids, G=G, path=path, split_k=split_k)


@pytest.mark.parametrize("name,gemm", [("tiny", "w"), ("olmoe", "gate_up"), ("olmoe", "down"),
                                       ("qwen3_t1", "gate_up"), ("qwen3_t1", "down"),
                                       ("qwen3_t8", "gate_up"), ("qwen3_t8", "down"),
                                       ("gptoss", "gate_up"), ("gptoss", "down"),
                                       ("gptoss_t256", "down")])
@pytest.mark.parametrize("path", [AUTO, DEC, TILE])
def test_workload_shapes(name, gemm, path):
    c = _workload_case(name, gemm)
    note(f"gemm {name}/{gemm} path={path}")
    y = _gemm(c, path)
    torch.cuda.synchronize()
    check_gemm(y, c["y_ref"], c["written"], f"{name}/{gemm}/path{path}")


@pytest.mark.parametrize("split_k", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("name,gemm", [("olmoe", "down"), ("gptoss", "gate_up"),
                                       ("qwen3_t8", "down")])
def test_decode_split_k(name, gemm, split_k):
    c = _workload_case(name, gemm)
    note(f"gemm {name}/{gemm} decode split_k={split_k}")
    y = _gemm(c, DEC, split_k)
    torch.cuda.synchronize()
    check_gemm(y, c["y_ref"], c["written"], f"{name}/{gemm}/S{split_k}")


def _custom(E, N, K, sizes, ids, M, seed=0, w_scale=None, x=None):
    rng = np.random.default_rng(seed)
    w = wls.bf16_round((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    if w_scale is not None:
        w = wls.bf16_round(w * w_scale)
    if x is None:
        x = wls.bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    packed, absmax = gnf4.pack(bf16_dev(w))
    p_ref, a_ref = oracle.ref_pack(w)
    y_ref, written = oracle.ref_grouped_gemm(x, p_ref, a_ref, sizes, ids)
    return dict(xs=bf16_dev(x), packed=packed, absmax=absmax, y_ref=y_ref, written=written,
                sizes=torch.tensor(sizes, dtype=torch.int32, device=DEV),
                ids=torch.tensor(ids, dtype=torch.int32, device=DEV), M=M, N=N, K=K,
                w=w, x=x, p_ref=p_ref, a_ref=a_ref)


def _run_custom(c, path, split_k=0, canary=True):
    M, N = c["M"], c["N"]
    full = torch.full((M + 2, N), -512.0, dtype=torch.bfloat16, device=DEV)
    y = full[1:M + 1]
    gnf4.grouped_gemm(c["xs"], c["packed"], c["absmax"], c["sizes"], c["ids"],
                      G=c["sizes"].numel(), y=y, path=path, split_k=split_k)
    torch.cuda.synchronize()
    f = full.float().cpu().numpy()
    if canary:
        assert np.all(f[0] == -512.0) and np.all(f[M + 1] == -512.0), "guard rows written"
        assert np.all(f[1:M + 1][~c["written"]] == -512.0), "uncovered rows written"
    return y


BOUNDARY_CASES = {
    "empty_groups_interleaved": (6, 96, 256, [0, 3, 0, 5, 0], [2, 1, 4, 0, 5], 8),
    "duplicate_ids": (4, 64, 128, [2, 3, 2], [1, 1, 1], 7),
    "rows_past_M": (4, 64, 128, [3, 9], [0, 2], 10),
    "negative_and_bad_ids": (4, 64, 128, [2, -3, 3, 2], [0, 1, 9, -1], 9),
    "uncovered_tail": (4, 80, 192, [2, 1], [3, 0], 12),
    "one_block_K64": (3, 48, 64, [4, 4], [2, 0], 8),
    "N_not_tile_multiple": (2, 300, 256, [5, 40], [1, 0], 45),
    "single_row_N1": (2, 1, 128, [1], [1], 1),
    "tile_boundaries": (8, 96, 128, [31, 32, 33, 1, 64, 65], [0, 1, 2, 3, 4, 5], 226),
    "big_group_two_passes": (2, 64, 256, [300], [1], 300),
    "ragged_K_2880": (2, 72, 2880, [37, 3], [1, 0], 40),
    # more than 256 group entries, so the group search walks several chunks
    "many_groups_sparse": (300, 64, 128,
                           [2 if g == 5 else 1 if g == 130 else 3 if g == 270 else
                            11 if g == 299 else 0 for g in range(300)],
                           list(range(300)), 17),
    # more non-empty groups than rows: the later groups start past M
    "groups_beyond_M": (12, 64, 128, [1] * 12, list(range(12)), 8),
    # a prefill-sized batch (at least 32 rows per group on average) holding
    # groups of 1, 2 and 8 rows: the automatic path runs all on the tile path
    "prefill_small_groups": (5, 96, 256, [1, 8, 150, 2, 60], [4, 0, 3, 1, 2], 221),
    # two tile-sized groups (9 rows each, just past the decode path's 8) in 17
    # rows: the second is clipped at M, and the tile launch must still give
    # it a slot (ceil(M / 9) = 2 groups, not floor = 1)
    "tile_groups_clipped_at_M": (2, 64, 128, [9, 9], [0, 1], 17),
}


@pytest.mark.parametrize("case", sorted(BOUNDARY_CASES))
@pytest.mark.parametrize("path", [AUTO, DEC, TILE])
def test_boundaries(case, path):
    E, N, K, sizes, ids, M = BOUNDARY_CASES[case]
    c = _custom(E, N, K, sizes, ids, M, seed=len(case))
    note(f"gemm boundary {case} path={path}")
    y = _run_custom(c, path)
    if c["written"].any():
        check_gemm(y, c["y_ref"], c["written"], case)


def test_one_hot_rows_exact_on_decode_path():
    """x = unit rows: y[r, :] = bf16(W~[e, :, k_r]) exactly (nibble order,
    table, absmax index and rounding all have to be right)."""
    E, N, K, M = 4, 256, 512, 12
    ks = (np.arange(M) * 97 + 5) % K
    x = np.zeros((M, K), np.float32)
    x[np.arange(M), ks] = 1.0
    c = _custom(E, N, K, [5, 3, 4], [2, 0, 3], M, seed=4, x=x)
    wt = oracle.ref_unpack(c["p_ref"], c["a_ref"])
    for split_k in (1, 2, 4):
        note(f"gemm one-hot decode split_k={split_k}")
        y = _run_custom(c, DEC, split_k).cpu()
        owner = [2] * 5 + [0] * 3 + [3] * 4
        for r in range(M):
            expect = torch.from_numpy(wt[owner[r], :, ks[r]].copy()).to(torch.bfloat16)
            assert torch.equal(y[r], expect), f"row {r} split {split_k}"


def test_all_top_codes_give_row_sums():
    E, N, K, M = 2, 64, 256, 40
    rng = np.random.default_rng(8)
    x = wls.bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    packed = torch.full((E, N, K // 2), 0xFF, dtype=torch.uint8, device=DEV)
    absmax = torch.ones((E, N, K // 64), dtype=torch.float32, device=DEV)
    sizes = torch.tensor([15, 25], dtype=torch.int32, device=DEV)
    ids = torch.tensor([1, 0], dtype=torch.int32, device=DEV)
    expect = np.array([sum(float(v) for v in row) for row in x])[:, None] * np.ones((1, N))
    for path in (DEC, TILE):
        note(f"gemm all-15 path={path}")
        y = gnf4.grouped_gemm(bf16_dev(x), packed, absmax, sizes, ids, path=path)
        torch.cuda.synchronize()
        check_gemm(y, expect, np.ones(M, bool), f"row sums path {path}")


def _absmax_scenarios(E, N, K):
    s = {}
    a = np.ones((E, N, K), np.float32)          # blocks alternate 1e-30 / 1e30 in a row
    for b in range(K // 64):
        a[:, :, 64 * b:64 * (b + 1)] = 1e-30 if b % 2 else 1e30
    s["blocks_1e-30_to_1e30"] = a
    s["all_tiny_1e-25"] = np.full((E, N, K), 1e-25, np.float32)
    s["all_huge_1e33"] = np.full((E, N, K), 1e33, np.float32)
    z = np.ones((E, N, K), np.float32)          # zero blocks and a single outlier row
    z[:, :, 64:192] = 0.0
    z[:, 3, :] = 1e4
    s["zero_blocks_outlier_row"] = z
    p = np.ones((E, N, K), np.float32)          # one large element per block
    p[:, :, ::64] = 500.0
    s["one_outlier_per_block"] = p
    return s


@pytest.mark.parametrize("scenario", sorted(_absmax_scenarios(1, 8, 256)))
@pytest.mark.parametrize("path", [DEC, TILE])
def test_adversarial_absmax(scenario, path):
    E, N, K, M = 3, 64, 512, 24
    scale = _absmax_scenarios(E, N, K)[scenario]
    c = _custom(E, N, K, [8, 8, 8], [0, 1, 2], M, seed=10, w_scale=scale)
    note(f"gemm adversarial absmax {scenario} path={path}")
    y = _run_custom(c, path)
    check_gemm(y, c["y_ref"], c["written"], f"{scenario} path {path}")


@pytest.mark.parametrize("gap", [8, 14, 16, 20, 24])
@pytest.mark.parametrize("path", [DEC, TILE])
def test_weight_block_range(gap, path):
    """Blocks whose absmax lies 2^gap below their weight row's largest carry
    the whole output: the activations are zero against the large (even)
    blocks.  The tile path scales each weight row so its largest block absmax
    lands in [2^14, 2^15), so every block within 2^25 of it decodes to normal
    fp16 numbers; every gap here is inside that range on both paths."""
    E, N, K, M = 2, 96, 1024, 40
    scale = np.ones((E, N, K), np.float32)
    for b in range(1, K // 64, 2):
        scale[:, :, 64 * b:64 * (b + 1)] = 2.0 ** -gap
    rng = np.random.default_rng(70 + gap)
    x = rng.standard_normal((M, K)).astype(np.float32)
    for b in range(0, K // 64, 2):
        x[:, 64 * b:64 * (b + 1)] = 0.0
    c = _custom(E, N, K, [24, 16], [1, 0], M, seed=70 + gap, w_scale=scale,
                x=wls.bf16_round(x))
    note(f"gemm weight block range 2^-{gap} path={path}")
    y = _run_custom(c, path)
    check_gemm(y, c["y_ref"], c["written"], f"block gap 2^{gap} path {path}")


@pytest.mark.parametrize("gap", [10, 12, 20, 27])
@pytest.mark.parametrize("row_max", [2.0 ** -5, 1.0, 2.0 ** 20])
@pytest.mark.parametrize("path", [DEC, TILE])
def test_activation_entries_below_row_max(gap, row_max, path):
    """Each activation row holds its largest value at k = 0, where every
    weight is zero, and the rest of the row 2^gap smaller: the small entries
    carry every output.  The tile path stages each row as fp16 scaled so its
    largest lands in [2^14, 2^15), so entries within 2^28 of it are exact,
    whatever the row's own magnitude."""
    E, N, K, M = 2, 96, 512, 40
    scale = np.ones((E, N, K), np.float32)
    scale[:, :, 0] = 0.0
    rng = np.random.default_rng(80 + gap)
    x = rng.standard_normal((M, K)) * (row_max * 2.0 ** -gap)
    x[:, 0] = row_max
    c = _custom(E, N, K, [24, 16], [0, 1], M, seed=80 + gap, w_scale=scale,
                x=wls.bf16_round(x.astype(np.float32)))
    note(f"gemm activation entries 2^-{gap} below a row max {row_max:g} path={path}")
    y = _run_custom(c, path)
    check_gemm(y, c["y_ref"], c["written"], f"x gap 2^{gap}, max {row_max:g}, path {path}")


@pytest.mark.parametrize("name,gemm", [("olmoe", "gate_up"), ("gptoss", "down"),
                                       ("gptoss_t256", "down"), ("qwen3_t8", "gate_up")])
@pytest.mark.parametrize("path", [AUTO, DEC, TILE])
def test_bf16_absmax(name, gemm, path):
    """The 4.25-bit stack (absmax stored as bf16), both paths and the fused
    gather, against the oracle's own bf16-absmax packing."""
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
    x_tok = wls.token_activations(wl, K)
    x_host = x_tok[ref["sorted_slots"] // wl.top_k]
    note(f"gemm bf16 absmax {name}/{gemm} path={path}")
    y = gnf4.grouped_gemm(bf16_dev(x_tok), packed, absmax, r.group_sizes, r.group_expert_ids,
                          path=path, sorted_slots=r.sorted_slots, top_k=wl.top_k)
    torch.cuda.synchronize()
    y_ref, written = oracle.ref_grouped_gemm(x_host, p_ref, a_ref, ref["group_sizes"],
                                             ref["group_expert_ids"])
    check_gemm(y, y_ref, written, f"bf16 absmax {name}/{gemm}/path{path}")


@pytest.mark.parametrize("scale", [1e-6, 1e-20, 5e4, 1e30])
@pytest.mark.parametrize("path", [DEC, TILE])
def test_activation_magnitudes(scale, path):
    """Activation rows far outside fp16's range, tiny and huge, mixed with
    ordinary rows and an all-zero row.  The tile path scales each row by its
    own power of two, so every class of rows meets the bar on its own (the
    rms of the bound is taken per class)."""
    E, N, K, M = 3, 96, 512, 48
    rng = np.random.default_rng(13)
    f = np.ones((M, 1), np.float32)
    f[::3] = scale
    f[7] = 0.0
    x = wls.bf16_round((rng.standard_normal((M, K)) * f).astype(np.float32))
    c = _custom(E, N, K, [20, 12, 16], [2, 0, 1], M, seed=13, x=x)
    note(f"gemm activation magnitude {scale:g} path={path}")
    y = _run_custom(c, path)
    scaled = np.zeros(M, bool)
    scaled[::3] = True
    for cls, mask in (("scaled", scaled), ("ordinary", ~scaled)):
        check_gemm(y, c["y_ref"], c["written"] & mask, f"x*{scale:g} {cls} rows, path {path}")
    assert np.all(host_f64(y)[7] == 0.0)


@pytest.mark.parametrize("path", [DEC, TILE])
def test_deterministic(path):
    c = _custom(8, 512, 1024, [3, 20, 1, 40, 6], [7, 2, 2, 5, 0], 70, seed=11)
    note(f"gemm determinism path={path}")
    y1 = _run_custom(c, path, 4 if path == DEC else 0).clone()
    y2 = _run_custom(c, path, 4 if path == DEC else 0)
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("path", [DEC, TILE])
def test_fidelity_better_than_bf16_materialisation(path):
    """The fused result is closer to the exact product than dequantise-to-bf16
    then matmul (the baseline the README compares against)."""
    E, N, K, M = 4, 256, 2048, 96
    c = _custom(E, N, K, [30, 2, 64], [1, 3, 0], M, seed=12)
    note(f"gemm fidelity path={path}")
    y = host_f64(_run_custom(c, path))
    w_bf16 = wls.bf16_round(oracle.ref_unpack(c["p_ref"], c["a_ref"])).astype(np.float64)
    base = np.zeros_like(c["y_ref"])
    for g, e, r0, r1 in oracle.ref_group_rows([30, 2, 64], [1, 3, 0], E, M):
        base[r0:r1] = c["x"][r0:r1].astype(np.float64) @ w_bf16[e].T
    base = wls.bf16_round(base.astype(np.float32)).astype(np.float64)
    wr = c["written"]
    err_fused = np.sqrt(np.mean((y[wr] - c["y_ref"][wr]) ** 2))
    err_base = np.sqrt(np.mean((base[wr] - c["y_ref"][wr]) ** 2))
    assert err_fused < err_base, (err_fused, err_base)


def test_rejects_host_tensors():
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    packed = torch.zeros((1, 8, 32), dtype=torch.uint8, device=DEV)
    absmax = torch.zeros((1, 8, 1), dtype=torch.float32, device=DEV)
    s = torch.tensor([4], dtype=torch.int32, device=DEV)
    with pytest.raises(gnf4.Gnf4Error, match="oracle"):
        gnf4.grouped_gemm(x, packed, absmax, s, s.clone())


@pytest.mark.parametrize("name", ["tiny", "olmoe", "qwen3_t8", "gptoss_t256"])
@pytest.mark.parametrize("path", [AUTO, DEC, TILE])
def test_fused_gather(name, path):
    """gnf4_grouped_gemm_gather on token rows == oracle on the gathered rows."""
    wl = wls.WORKLOADS[name]
    gemm = "w" if name == "tiny" else "gate_up"
    c = _workload_case(name, gemm)
    x_tok = wls.token_activations(wl, c["K"])
    note(f"gemm fused gather {name} path={path}")
    y = gnf4.grouped_gemm(bf16_dev(x_tok), c["packed"], c["absmax"], c["r"].group_sizes,
                          c["r"].group_expert_ids, path=path, sorted_slots=c["r"].sorted_slots,
                          top_k=wl.top_k)
    torch.cuda.synchronize()
    check_gemm(y, c["y_ref"], c["written"], f"fused gather {name} path {path}")


@pytest.mark.parametrize("path", [DEC, TILE])
def test_fused_gather_bad_slots_skip_rows(path):
    E, N, K, T, top_k = 3, 64, 256, 10, 2
    sizes, ids = [4, 12, 4], [2, 0, 1]
    M = sum(sizes)
    rng = np.random.default_rng(31)
    slots = rng.integers(0, T * top_k, M).astype(np.int32)
    slots[[1, 7, 18]] = [-1, T * top_k, 10 ** 6]
    x_tok = wls.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    x_rows = np.zeros((M, K), np.float32)
    ok = (slots >= 0) & (slots < T * top_k)
    x_rows[ok] = x_tok[slots[ok] // top_k]
    c = _custom(E, N, K, sizes, ids, M, seed=32, x=x_rows)
    written = c["written"] & ok
    full = torch.full((M + 2, N), -512.0, dtype=torch.bfloat16, device=DEV)
    note(f"gemm fused gather bad slots path={path}")
    gnf4.grouped_gemm(bf16_dev(x_tok), c["packed"], c["absmax"], c["sizes"], c["ids"], G=3,
                      y=full[1:M + 1], path=path,
                      sorted_slots=torch.from_numpy(slots).to(DEV), top_k=top_k)
    torch.cuda.synchronize()
    f = full.float().cpu().numpy()
    assert np.all(f[0] == -512.0) and np.all(f[M + 1] == -512.0)
    assert np.all(f[1:M + 1][~written] == -512.0), "rows with bad slots were written"
    check_gemm(full[1:M + 1], c["y_ref"], written, f"bad slots path {path}")


# The automatic path beside the fused gather.  With T <= 8 tokens a top-k
# routing puts at most T rows in a group, so the decode launch alone serves
# every group, also a group of a caller-built grouping that breaks that bound
# (12 rows of 4 tokens: duplicate picks).  With more tokens, groups of more
# than 8 rows go to the tile launch ([10, 8]); when no group has that many
# ([8, 8, 8]) the tile launch's staging stages nothing and the decode launch
# serves them all.
@pytest.mark.parametrize("T,top_k,sizes,ids", [(4, 4, [12, 4], [0, 2]),
                                               (9, 2, [10, 8], [1, 0]),
                                               (12, 2, [8, 8, 8], [2, 0, 1])])
def test_fused_gather_auto_group_sizes(T, top_k, sizes, ids):
    E, N, K = 3, 64, 256
    M = sum(sizes)
    assert M == T * top_k
    rng = np.random.default_rng(T)
    slots = rng.permutation(M).astype(np.int32)
    x_tok = wls.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    x_rows = x_tok[slots // top_k]
    c = _custom(E, N, K, sizes, ids, M, seed=35 + T, x=x_rows)
    note(f"gemm fused gather auto T={T} top_k={top_k} sizes={sizes}")
    y = gnf4.grouped_gemm(bf16_dev(x_tok), c["packed"], c["absmax"], c["sizes"], c["ids"],
                          G=len(sizes), path=AUTO, sorted_slots=torch.from_numpy(slots).to(DEV),
                          top_k=top_k)
    torch.cuda.synchronize()
    check_gemm(y, c["y_ref"], c["written"], f"fused gather auto T={T} sizes={sizes}")


@pytest.mark.parametrize("split_k", [0, 2])
def test_fused_gather_one_token(split_k):
    """A single token behind the fused gather (a batch-1 decode step): every
    valid slot reads token 0, the decode path loads it before the group
    metadata; rows with invalid slots stay unwritten, groups of one and of
    several rows (duplicate picks of a caller-built grouping) both work."""
    E, N, K, T, top_k = 6, 96, 512, 1, 8
    sizes, ids = [1, 3, 1, 2, 1], [5, 0, 2, 4, 1]
    M = sum(sizes)
    slots = np.array([3, 0, 9, 2, 7, -1, 5, 1], dtype=np.int32)   # 9, -1: invalid
    rng = np.random.default_rng(33)
    x_tok = wls.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    ok = (slots >= 0) & (slots < T * top_k)
    x_rows = np.zeros((M, K), np.float32)
    x_rows[ok] = x_tok[0]
    c = _custom(E, N, K, sizes, ids, M, seed=34, x=x_rows)
    written = c["written"] & ok
    full = torch.full((M + 2, N), -512.0, dtype=torch.bfloat16, device=DEV)
    note(f"gemm fused gather one token split_k={split_k}")
    gnf4.grouped_gemm(bf16_dev(x_tok), c["packed"], c["absmax"], c["sizes"], c["ids"],
                      G=len(sizes), y=full[1:M + 1], path=DEC, split_k=split_k,
                      sorted_slots=torch.from_numpy(slots).to(DEV), top_k=top_k)
    torch.cuda.synchronize()
    f = full.float().cpu().numpy()
    assert np.all(f[0] == -512.0) and np.all(f[M + 1] == -512.0)
    assert np.all(f[1:M + 1][~written] == -512.0), "rows with bad slots were written"
    check_gemm(full[1:M + 1], c["y_ref"], written, f"one token split {split_k}")
