"""Whole expert stacks, packed on the GPU, against the oracle's packer byte
for byte: every code byte and every absmax of one layer of each workload
configuration (Tiny, OLMoE, Qwen3-30B, GPT-OSS-120B, DeepSeek-V3 shapes;
gate_up and down).  Weights are drawn on the device per expert (torch
Philox), packed by gnf4_pack, and streamed to the host one expert at a time;
a pool of worker processes (numpy and the oracle only) re-packs each expert
from the same bf16 bits and compares.
"""

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np
import pytest
import torch

from grouped_nf4_expert_amd import gnf4
from grouped_nf4_expert_amd import workloads as wls

import pack_worker
from gpu_util import DEV, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pool():
    workers = max(1, min(14, (os.cpu_count() or 4) - 2))
    with cf.ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
        yield ex, workers


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name", ["tiny", "olmoe", "qwen3_t1", "gptoss", "dsv3"])
def test_whole_stack_pack_bit_exact(pool, name):
    ex, workers = pool
    wl = wls.WORKLOADS[name]
    for gemm, K, N in wl.gemms:
        note(f"whole-stack pack {name}/{gemm}: E={wl.E} N={N} K={K}")
        pending, bad_bytes, bad_abs = [], 0, 0

        def drain(limit):
            nonlocal bad_bytes, bad_abs
            while len(pending) > limit:
                b, a = pending.pop(0).result()
                bad_bytes += b
                bad_abs += a
        for e in range(wl.E):
            w = wls.expert_weights_device(wl, gemm, e, DEV)
            packed, absmax = gnf4.pack(w)
            bits = w.view(torch.int16).cpu().numpy().view(np.uint16)
            pending.append(ex.submit(pack_worker.check_expert, bits, packed.cpu().numpy(),
                                     absmax.cpu().numpy()))
            drain(2 * workers)
        drain(0)
        assert bad_bytes == 0 and bad_abs == 0, (
            f"{name}/{gemm}: {bad_bytes} code bytes and {bad_abs} absmax values differ")
