"""The MoE-FFN steps on either side of the grouped GEMM, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  * Landing page "grouped-nf4-gemm", "Owns": the decode glue kernels include
    the swiglu activation and the top-k combine; "Use this when": the
    activation between the two expert projections and the top-k combine
    after them are each one launch of the decode step.
  * Page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE
    expert stacks", opening section: the expert GEMM runs on rows grouped by
    the token->expert sort, and routing weights are not applied inside it.

Readings (the pages name these operations but not their layout):
  * SwiGLU: the gate_up projection's N = 2I outputs per row are the gate
    half followed by the up half, ``[gate | up]``;
    ``h = silu(gate) * up`` with ``silu(g) = g / (1 + exp(-g))``.
  * combine: ``out[t] = sum_j topk_w[t, j] * y[slot_rows[t*k + j]]``, summed
    in ascending j.  A slot whose row is outside ``[0, M)`` (a row the
    expert GEMMs did not produce) contributes nothing.
  * the oracle keeps results unrounded (fp64); the kernels' bf16 stores are
    checked against it with a tolerance.
"""

import numpy as np

from .gemm import ref_group_rows
from .nf4 import ref_unpack
from .route import ref_route_sort


def ref_silu(g):
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g)), elementwise in fp64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def ref_swiglu(gate_up):
    """``gate_up [M, 2I]`` -> ``h [M, I] = silu(gate_up[:, :I]) * gate_up[:, I:]``."""
    gu = np.asarray(gate_up, dtype=np.float64)
    M, two_i = gu.shape
    assert two_i % 2 == 0, "the gate_up width must be even"
    I = two_i // 2
    return ref_silu(gu[:, :I]) * gu[:, I:]


def ref_combine(y, slot_rows, topk_w, M=None):
    """Weighted top-k combine of the down projection's grouped rows.

    ``y``: ``[M, H]`` rows in grouped (sorted) order; ``slot_rows``: ``[T*k]``
    row of each flat slot; ``topk_w``: ``[T, k]``.  Returns
    ``(out fp64 [T, H], mag fp64 [T, H])`` where ``mag`` is the sum of the
    absolute terms (the scale of the summation's rounding error).
    """
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(topk_w, dtype=np.float64)
    T, k = w.shape
    M = y.shape[0] if M is None else M
    rows = np.asarray(slot_rows, dtype=np.int64).reshape(T, k)
    H = y.shape[1]
    out = np.zeros((T, H), dtype=np.float64)
    mag = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        r = rows[:, j]
        ok = (r >= 0) & (r < M)
        term = np.zeros((T, H), dtype=np.float64)
        term[ok] = w[ok, j:j + 1] * y[r[ok]]
        out += term
        mag += np.abs(term)
    return out, mag


def ref_expert_projection(x_sorted, packed, absmax, group_sizes, group_expert_ids):
    """``y[r] = x_sorted[r] @ W[e].T`` for the rows of each group, all in fp64
    (the grouped GEMM of ``gemm.py`` without its fp32 input contract, so that
    fp64 intermediates pass through unrounded).  Rows no group covers are 0.
    """
    x = np.asarray(x_sorted, dtype=np.float64)
    E, N, _ = packed.shape
    y = np.zeros((x.shape[0], N), dtype=np.float64)
    for _g, e, r0, r1 in ref_group_rows(group_sizes, group_expert_ids, E, x.shape[0]):
        y[r0:r1] = x[r0:r1] @ ref_unpack(packed[e], absmax[e]).astype(np.float64).T
    return y


def ref_moe_ffn(x, logits, top_k, gate_up, down):
    """One MoE feed-forward layer composed from the steps of the path.

    ``x [T, D]`` token activations; ``gate_up = (packed, absmax)`` of an
    ``[E, 2I, D]`` stack and ``down`` of an ``[E, D, I]`` stack.  Route and
    sort, gather rows, gate_up projection, SwiGLU, down projection, combine --
    every intermediate kept in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    r = ref_route_sort(logits, top_k)
    rows = r["sorted_slots"].astype(np.int64) // top_k
    y1 = ref_expert_projection(x[rows], gate_up[0], gate_up[1], r["group_sizes"],
                               r["group_expert_ids"])
    h = ref_swiglu(y1)
    y2 = ref_expert_projection(h, down[0], down[1], r["group_sizes"], r["group_expert_ids"])
    out, _ = ref_combine(y2, r["slot_rows"], r["topk_w"])
    return out
