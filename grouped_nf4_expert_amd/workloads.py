"""Synthetic workloads: shapes and seeded input generators.

This module only draws inputs.  It holds none of the method's arithmetic (no
NF4 table, no quantisation, no routing): the HIP library and the CPU oracle
both take what it returns and each computes its own results.

Shapes follow the MoE expert census the grouped-nf4-gemm README measures on
(page "grouped-nf4-gemm -- single-launch W4A16 GEMM over fused NF4 MoE expert
stacks", section "The claim": OLMoE, Qwen3-30B, GPT-OSS-120B gate_up + down
at batch-1 decode, DeepSeek-V3 among the off-census shapes).  No dataset is
involved: weights, activations and router logits are random.

Recipe (every tensor has its own stream, every expert its own sub-stream, so
any subset can be regenerated on its own):
  * weights   fp32 N(0, 0.02) rounded to bf16 (round-to-nearest-even), [N, K]
    per expert, then packed by whichever side is under test;
  * token activations fp32 N(0, 1) rounded to bf16, [T, K]; the gate_up input
    is the token rows gathered in sorted-slot order;
  * down-projection input: independent bf16 N(0, 1) rows [M, K_down];
  * router logits fp32 N(0, 1) [T, E]; the skewed router adds +20 to a hot
    set of 16 experts (the first 16 of a seeded permutation) for a seeded 70%
    of the tokens, so their top-k falls inside the hot set.

Two backends: numpy on the host (used wherever the oracle must see the same
values) and torch's Philox generator on the device (fast fill for the largest
shapes; a test that needs those values on the host copies the generated
tensor back -- the values come from the generator, never from a kernel).
"""

from dataclasses import dataclass, field
from typing import Dict, Tuple

import numpy as np

TAG_WEIGHTS = {"gate_up": 11, "down": 12, "w": 13}
TAG_TOKENS = 21
TAG_DOWN_INPUT = 22
TAG_LOGITS = 31
TAG_SKEW = 32


@dataclass(frozen=True)
class Workload:
    name: str
    E: int
    top_k: int
    T: int
    gemms: Tuple[Tuple[str, int, int], ...]  # (name, K, N)
    seed: int
    skewed: bool = False
    layers: int = 1  # distinct weight sets the benchmark cycles through
    note: str = ""

    @property
    def M(self):
        return self.T * self.top_k

    def gemm(self, name):
        for g, K, N in self.gemms:
            if g == name:
                return K, N
        raise KeyError(name)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", E=8, top_k=2, T=4, gemms=(("w", 256, 512),), seed=0,
                     note="correctness case, oracle finishes in well under a second"),
    "olmoe": Workload("olmoe", E=64, top_k=8, T=1,
                      gemms=(("gate_up", 2048, 2048), ("down", 1024, 2048)), seed=1,
                      layers=16, note="OLMoE-shaped batch-1 decode"),
    "qwen3_t1": Workload("qwen3_t1", E=128, top_k=8, T=1,
                         gemms=(("gate_up", 2048, 1536), ("down", 768, 2048)), seed=2,
                         layers=16, note="Qwen3-30B-A3B-shaped decode, T=1"),
    "qwen3_t8": Workload("qwen3_t8", E=128, top_k=8, T=8,
                         gemms=(("gate_up", 2048, 1536), ("down", 768, 2048)), seed=5,
                         layers=8, note="Qwen3-30B-A3B-shaped decode, T=8"),
    "gptoss": Workload("gptoss", E=128, top_k=4, T=1,
                       gemms=(("gate_up", 2880, 5760), ("down", 2880, 2880)), seed=3,
                       skewed=True, layers=8, note="GPT-OSS-120B-shaped decode, skewed router"),
    "gptoss_t256": Workload("gptoss_t256", E=128, top_k=4, T=256,
                            gemms=(("gate_up", 2880, 5760), ("down", 2880, 2880)), seed=6,
                            skewed=True, note="GPT-OSS-shaped with uneven group sizes"),
    "dsv3": Workload("dsv3", E=256, top_k=8, T=4096,
                     gemms=(("gate_up", 7168, 4096), ("down", 2048, 7168)), seed=4,
                     note="DeepSeek-V3-shaped prefill, ~128 rows per expert"),
}

HOT_SET = 16
HOT_FRACTION = 0.7
HOT_BOOST = 20.0
WEIGHT_STD = 0.02


def _rng(*key):
    return np.random.default_rng([int(k) for k in key])


def bf16_round(a):
    """Round fp32 to the nearest bf16 (ties to even), returned widened to fp32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(a.shape)


def bf16_bits(a):
    """bf16-exact fp32 values -> their 16-bit patterns (uint16)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b):
    """16-bit bf16 patterns -> fp32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- host side

def expert_weights(wl: Workload, gemm: str, expert: int, layer: int = 0):
    """One expert's weights ``[N, K]`` (bf16 values as fp32)."""
    K, N = wl.gemm(gemm)
    rng = _rng(wl.seed, TAG_WEIGHTS[gemm], layer, expert)
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(WEIGHT_STD)
    return bf16_round(w)


def weight_stack(wl: Workload, gemm: str, layer: int = 0):
    """All experts' weights ``[E, N, K]`` (bf16 values as fp32)."""
    return np.stack([expert_weights(wl, gemm, e, layer) for e in range(wl.E)])


def router_logits(wl: Workload, layer: int = 0, T: int = None):
    """Router logits ``[T, E]`` fp32."""
    T = wl.T if T is None else T
    rng = _rng(wl.seed, TAG_LOGITS, layer)
    lg = rng.standard_normal((T, wl.E), dtype=np.float32)
    if wl.skewed:
        srng = _rng(wl.seed, TAG_SKEW, layer)
        hot = srng.permutation(wl.E)[:HOT_SET]
        pick = srng.random(T) < HOT_FRACTION
        for t in np.nonzero(pick)[0]:
            lg[t, hot] += np.float32(HOT_BOOST)
    return lg


def token_activations(wl: Workload, K: int, layer: int = 0, T: int = None):
    """Token activations ``[T, K]`` (bf16 values as fp32)."""
    T = wl.T if T is None else T
    rng = _rng(wl.seed, TAG_TOKENS, layer, K)
    return bf16_round(rng.standard_normal((T, K), dtype=np.float32))


def down_input(wl: Workload, M: int, K: int, layer: int = 0):
    """Independent rows for the down projection ``[M, K]`` (bf16 as fp32)."""
    rng = _rng(wl.seed, TAG_DOWN_INPUT, layer, K)
    return bf16_round(rng.standard_normal((M, K), dtype=np.float32))


# -------------------------------------------------------------- device side

def torch_seed(*key):
    """64-bit seed for a torch generator, derived from the same key."""
    ss = np.random.SeedSequence([int(k) for k in key])
    return int(ss.generate_state(1, np.uint64)[0] & ((1 << 63) - 1))


def expert_weights_device(wl: Workload, gemm: str, expert: int, device, layer: int = 0,
                          out=None):
    """One expert's bf16 weights ``[N, K]`` drawn on ``device`` (torch Philox)."""
    import torch
    K, N = wl.gemm(gemm)
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(wl.seed, TAG_WEIGHTS[gemm], layer, expert, 7))
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    w.mul_(WEIGHT_STD)
    if out is None:
        return w.to(torch.bfloat16)
    out.copy_(w)
    return out


def activations_device(rows: int, K: int, device, *key):
    """bf16 N(0,1) rows ``[rows, K]`` drawn on ``device``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(*key))
    return torch.randn((rows, K), generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def logits_device(wl: Workload, device, layer: int = 0):
    """Router logits on the device: the host stream, copied over."""
    import torch
    return torch.from_numpy(router_logits(wl, layer)).to(device)
