"""Router top-k with softmax weights and the token->expert sort.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  * Page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE
    expert stacks", opening section: activations arrive sorted by expert and
    the kernel is handed ``(sizes, expert_ids)`` "after the usual
    token->expert sort".
  * Landing page "grouped-nf4-gemm", "Use this when" / "Owns": router softmax
    and top-k are glue kernels of the decode step; routing weights are applied
    by a separate top-k combine, not inside the GEMM.

Readings (the pages leave these open):
  * top-k order: descending logit, equal logits go to the lower expert id
    (float comparison, so -0.0 and +0.0 are equal); NaN logits are outside
    the contract.
  * weights: softmax over the k selected logits, computed in fp64 and stored
    as fp32 (the same as a softmax over all experts renormalised to the k).
  * sort: flat slot s = t*top_k + j; slots are grouped by expert in ascending
    expert id and, inside one expert, by ascending s (a stable sort).
  * groups: the non-empty experts in ascending id; ``group_sizes`` and
    ``group_expert_ids`` have E entries, the unused tail is zero.
"""

import numpy as np


def ref_topk(logits, top_k):
    """Per token: the top_k largest logits and their softmax weights.

    Returns ``(topk_ids int32[T, k], topk_w float32[T, k])``.
    """
    lg = np.asarray(logits, dtype=np.float32)
    assert lg.ndim == 2
    T, E = lg.shape
    assert 1 <= top_k <= E
    assert not np.any(np.isnan(lg)), "NaN logits are outside the contract"
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float32)
    expert = np.arange(E)
    for t in range(T):
        # lexsort: last key is primary -> descending logit, then ascending id
        order = np.lexsort((expert, -lg[t].astype(np.float64)))[:top_k]
        ids[t] = order
        sel = lg[t, order].astype(np.float64)
        ex = np.exp(sel - sel.max())
        w[t] = (ex / ex.sum()).astype(np.float32)
    return ids, w


def ref_sort(topk_ids, num_experts):
    """Stable counting sort of flat slots by expert.

    Returns a dict with ``expert_offsets int32[E+1]``, ``sorted_slots
    int32[M]``, ``slot_rows int32[M]``, ``group_sizes int32[E]``,
    ``group_expert_ids int32[E]`` and ``num_groups`` (int), M = T * top_k.

    ``slot_rows[s]`` is the grouped row of flat slot s, from its definition:
    the rows of expert e start at ``expert_offsets[e]`` and a slot comes after
    every earlier slot (lower s) routed to the same expert.  It is the inverse
    of ``sorted_slots``; the combine after the down projection reads it.
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    E = int(num_experts)
    assert np.all((ids >= 0) & (ids < E))
    counts = np.bincount(ids, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_slots = np.argsort(ids, kind="stable")
    slot_rows = np.empty(ids.size, dtype=np.int64)
    seen = np.zeros(E, dtype=np.int64)
    for slot in range(ids.size):
        e = ids[slot]
        slot_rows[slot] = offsets[e] + seen[e]
        seen[e] += 1
    nonempty = np.nonzero(counts)[0]
    G = nonempty.size
    group_sizes = np.zeros(E, dtype=np.int32)
    group_ids = np.zeros(E, dtype=np.int32)
    group_sizes[:G] = counts[nonempty]
    group_ids[:G] = nonempty
    return {
        "expert_offsets": offsets.astype(np.int32),
        "sorted_slots": sorted_slots.astype(np.int32),
        "slot_rows": slot_rows.astype(np.int32),
        "group_sizes": group_sizes,
        "group_expert_ids": group_ids,
        "num_groups": int(G),
    }


def ref_route_sort(logits, top_k):
    """Top-k routing followed by the token->expert sort."""
    lg = np.asarray(logits, dtype=np.float32)
    ids, w = ref_topk(lg, top_k)
    out = ref_sort(ids, lg.shape[1])
    out["topk_ids"] = ids
    out["topk_w"] = w
    return out
