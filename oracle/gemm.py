"""The grouped expert GEMM on NF4-packed weights, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE
expert stacks", opening section and "The claim": the routed expert GEMM runs
on ``[E, N, K/2]`` packed codes with fp32 blockwise absmax, rows sorted by
expert and described by ``(sizes, expert_ids)``, every code decoded to fp32
and accumulated in fp32 with a bf16 epilogue.

Readings:
  * W[e] is ``[N, K]`` (out x in), so ``y[r, :] = x[r, :] @ W[e].T``.
  * groups are contiguous row ranges of ``x_sorted`` in group order; a group
    of size <= 0 holds no rows; rows past M are cut off; a group whose expert
    id is outside [0, E) writes nothing (its rows still occupy their place);
    rows that no group covers are not written.
  * the oracle keeps the result unrounded (fp64): the GEMM's own bf16 store
    is checked against it with a tolerance, not bit for bit.
"""

import numpy as np

from .nf4 import ref_unpack


def ref_group_rows(group_sizes, group_expert_ids, num_experts, M):
    """List of ``(g, e, r0, r1)`` for every group that writes rows."""
    sizes = np.asarray(group_sizes, dtype=np.int64).reshape(-1)
    ids = np.asarray(group_expert_ids, dtype=np.int64).reshape(-1)
    out = []
    off = 0
    for g in range(sizes.size):
        sz = max(int(sizes[g]), 0)
        r0, r1 = off, min(off + sz, M)
        off += sz
        e = int(ids[g])
        if sz > 0 and 0 <= e < num_experts and r0 < r1:
            out.append((g, e, r0, r1))
    return out


def ref_grouped_gemm(x_sorted, packed, absmax, group_sizes, group_expert_ids):
    """Full grouped GEMM.

    ``x_sorted``: fp32 array ``[M, K]`` (bf16 values widened exactly);
    ``packed``/``absmax``: ``[E, N, K/2]`` / ``[E, N, K/64]``.
    Returns ``(y fp64[M, N], written bool[M])``; unwritten rows are NaN.
    """
    x = np.asarray(x_sorted, dtype=np.float32)
    M, K = x.shape
    E, N, half_k = packed.shape
    assert half_k * 2 == K
    y = np.full((M, N), np.nan, dtype=np.float64)
    written = np.zeros(M, dtype=bool)
    cache = {}
    for g, e, r0, r1 in ref_group_rows(group_sizes, group_expert_ids, E, M):
        if e not in cache:
            cache[e] = ref_unpack(packed[e], absmax[e]).astype(np.float64)
        w = cache[e]
        y[r0:r1] = x[r0:r1].astype(np.float64) @ w.T
        written[r0:r1] = True
    return y, written


def ref_grouped_gemm_entries(x_sorted, expert_weights, num_experts, N,
                             group_sizes, group_expert_ids, rows, cols):
    """Selected outputs ``y[rows[i], cols[i]]`` one by one, in fp64.

    ``expert_weights(e)`` returns ``(packed_e [N, K/2], absmax_e [N, K/64])``
    so a caller can hand over one expert at a time.  Entries whose row no
    group writes come back as NaN.
    """
    x = np.asarray(x_sorted, dtype=np.float32)
    M = x.shape[0]
    owner = np.full(M, -1, dtype=np.int64)
    for _g, e, r0, r1 in ref_group_rows(group_sizes, group_expert_ids,
                                        num_experts, M):
        owner[r0:r1] = e
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    out = np.full(rows.shape, np.nan, dtype=np.float64)
    by_expert = {}
    for i, (r, n) in enumerate(zip(rows, cols)):
        assert 0 <= n < N
        e = owner[r]
        if e >= 0:
            by_expert.setdefault(int(e), []).append(i)
    for e, idx in by_expert.items():
        p, a = expert_weights(e)
        p = np.asarray(p)
        a = np.asarray(a)
        for i in idx:
            w = ref_unpack(p[cols[i]][None, :], a[cols[i]][None, :])[0]
            out[i] = float(np.dot(x[rows[i]].astype(np.float64),
                                  w.astype(np.float64)))
    return out


def ref_grouped_dgrad(dy_sorted, packed, absmax, group_sizes, group_expert_ids):
    """Gradient of the grouped GEMM with respect to its activations.

    Landing page "grouped-nf4-gemm", "Owns": the grouped packed GEMM and its
    dgrad (the backward of ``y = x W^T`` over the same packed stack).  For
    the rows of group g with expert e: ``dx[r, :] = dy[r, :] @ W[e]`` -- a
    contraction over N, the transpose of the forward GEMM's access to the
    K-contiguous stack.  Same group reading as ``ref_grouped_gemm``.

    ``dy_sorted``: fp32 ``[M, N]`` (bf16 values widened exactly).
    Returns ``(dx fp64[M, K], written bool[M])``; unwritten rows are NaN.
    """
    dy = np.asarray(dy_sorted, dtype=np.float32)
    M, N = dy.shape
    E, N_w, half_k = packed.shape
    assert N_w == N
    K = 2 * half_k
    dx = np.full((M, K), np.nan, dtype=np.float64)
    written = np.zeros(M, dtype=bool)
    cache = {}
    for g, e, r0, r1 in ref_group_rows(group_sizes, group_expert_ids, E, M):
        if e not in cache:
            cache[e] = ref_unpack(packed[e], absmax[e]).astype(np.float64)
        dx[r0:r1] = dy[r0:r1].astype(np.float64) @ cache[e]
        written[r0:r1] = True
    return dx, written
