"""Worker-process side of the whole-stack pack comparison: numpy and the
oracle only (no torch, no GPU), so a spawned pool starts cheaply."""

import numpy as np

import oracle


def check_expert(w_bits, packed, absmax):
    """Oracle-pack one expert's bf16 weights (given as their 16-bit patterns)
    and count the code bytes and absmax values that differ from the GPU's."""
    w = (np.asarray(w_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    p_ref, a_ref = oracle.ref_pack(w)
    bad_bytes = int(np.count_nonzero(p_ref != packed))
    bad_abs = int(np.count_nonzero(a_ref.view(np.uint32) != np.asarray(absmax).view(np.uint32)))
    return bad_bytes, bad_abs
