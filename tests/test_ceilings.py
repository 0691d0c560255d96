"""The machine-ceiling probe library loads, exports every symbol
include/gnf4_ceilings.h declares, and refuses bad arguments before touching
the GPU; on a GPU, its probes compute what the header says they do."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gnf4_ceilings.h")
LIB = os.path.join(ROOT, "grouped_nf4_expert_amd", "libgnf4_ceilings.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libgnf4_ceilings.so not built")
    h = ctypes.CDLL(LIB)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    h.gnf4_ceil_read.argtypes = [vp, ctypes.c_size_t, ci, vp, vp]
    h.gnf4_ceil_empty.argtypes = [ci, vp]
    h.gnf4_ceil_mfma.argtypes = [ci, ci, vp, vp, vp]
    h.gnf4_ceil_mfma_mix.argtypes = [ci, ci, ci, ci, vp, vp, vp]
    h.gnf4_ceil_mfma_split.argtypes = [ci, ci, ci, vp, vp, vp]
    return h


def test_every_declared_symbol_is_exported(lib):
    declared = set(re.findall(r"\b(gnf4_ceil_\w+)\s*\(", open(HEADER).read()))
    assert declared == {"gnf4_ceil_read", "gnf4_ceil_empty", "gnf4_ceil_mfma",
                        "gnf4_ceil_mfma_mix", "gnf4_ceil_mfma_split"}
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\b(gnf4_ceil_\w+)\b", out))
    assert declared <= exported


def test_bad_arguments_are_refused(lib):
    fake = ctypes.c_void_p(0x1000)
    assert lib.gnf4_ceil_read(None, 16, 1, fake, None) == 1
    assert lib.gnf4_ceil_read(fake, 24, 1, fake, None) == 1        # not a multiple of 16
    assert lib.gnf4_ceil_read(ctypes.c_void_p(0x1008), 32, 1, fake, None) == 1  # misaligned
    assert lib.gnf4_ceil_read(fake, 16, 0, fake, None) == 1
    assert lib.gnf4_ceil_read(fake, 16, 65537, fake, None) == 1
    assert lib.gnf4_ceil_empty(0, None) == 1
    assert lib.gnf4_ceil_mfma(0, 1, fake, fake, None) == 1
    assert lib.gnf4_ceil_mfma(1, 1, None, fake, None) == 1
    assert lib.gnf4_ceil_mfma(1 << 25, 1, fake, fake, None) == 1
    assert lib.gnf4_ceil_mfma_mix(1, 1, 6, 0, fake, fake, None) == 1    # valu not 0/4/8/12
    assert lib.gnf4_ceil_mfma_mix(1, 1, 8, 2, fake, fake, None) == 1    # lds_reads not 0/1
    assert lib.gnf4_ceil_mfma_mix(1, 0, 8, 1, fake, fake, None) == 1
    assert lib.gnf4_ceil_mfma_mix(1, 1, 8, 1, None, fake, None) == 1
    assert lib.gnf4_ceil_mfma_mix(0, 1, 8, 1, fake, fake, None) == 1
    assert lib.gnf4_ceil_mfma_split(1, 1, 0, fake, fake, None) == 1     # valu not 4/8/12
    assert lib.gnf4_ceil_mfma_split(1, 1, 8, None, fake, None) == 1
    assert lib.gnf4_ceil_mfma_split(1, 65537, 8, fake, fake, None) == 1


@pytest.mark.gpu
def test_read_probe_reads_every_word(lib):
    import torch
    dev = torch.device("cuda:0")
    words = 65536 + 37
    buf = torch.randint(0, 256, (16 * words,), dtype=torch.uint8, device=dev)
    want = int(np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32)))
    for blocks in (1, 3, 256, 4096):
        out = torch.empty(blocks, dtype=torch.int32, device=dev)
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert lib.gnf4_ceil_read(ctypes.c_void_p(buf.data_ptr()), 16 * words, blocks,
                                  ctypes.c_void_p(out.data_ptr()), st) == 0
        torch.cuda.synchronize()
        got = int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)))
        assert got == want, f"blocks={blocks}"


@pytest.mark.gpu
def test_mfma_probe_sum_and_stamps(lib):
    import torch
    dev = torch.device("cuda:0")
    blocks, iters = 3, 64
    stamps = torch.zeros(blocks * 16, dtype=torch.int64, device=dev)
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.gnf4_ceil_mfma(iters, blocks, ctypes.c_void_p(stamps.data_ptr()),
                              ctypes.c_void_p(sink.data_ptr()), st) == 0
    assert lib.gnf4_ceil_empty(5, st) == 0
    torch.cuda.synchronize()
    # the operands the header defines, as 32x16 A and 16x32 B
    A = np.zeros((32, 16))
    B = np.zeros((16, 32))
    for lane in range(64):
        for j in range(8):
            k = 8 * (lane // 32) + j
            A[lane % 32, k] = ((lane + j) & 7) / 8
            B[k, lane % 32] = ((3 * lane + j) & 7) / 16
    per_wave = 4 * iters * float(np.sum(A.sum(axis=0) * B.sum(axis=1)))
    s = sink.cpu().numpy().astype(np.float64).reshape(blocks * 4, 64).sum(axis=1)
    assert np.all(s == per_wave), (s, per_wave)
    t = stamps.cpu().numpy().reshape(blocks * 4, 4)
    assert np.all(t[:, 1] > t[:, 0]) and np.all(t[:, 3] >= t[:, 2])
