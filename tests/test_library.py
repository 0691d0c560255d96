"""The C-ABI library loads and exports every symbol include/gnf4.h declares.

CPU only: no kernel is launched.  Host-checkable misuse (null pointers, bad
dimensions, unsupported sizes) is rejected before any HIP call, so those
status codes are checked here as well.
"""

import ctypes
import os
import re
import subprocess

import pytest

from grouped_nf4_expert_amd import gnf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gnf4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gnf4_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gnf4.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return gnf4.library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("gnf4_pack", "gnf4_route_sort", "gnf4_grouped_gemm", "gnf4_gather_rows",
                     "gnf4_grouped_gemm_gather", "gnf4_swiglu", "gnf4_combine"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", gnf4.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gnf4_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(lib, n)


def test_status_strings(lib):
    for s in range(6):
        assert lib.gnf4_status_string(s)
    assert b"oracle" in lib.gnf4_status_string(2)
    assert lib.gnf4_version() == b"0.1.0"


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "gnf4.h"\nint main(void){return (int)GNF4_OK;}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                    "-c", str(src), "-o", str(tmp_path / "t.o")], check=True)


NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: rejected before any HIP call


def test_pack_rejects_bad_arguments(lib):
    assert lib.gnf4_pack(NULL, 0, 1, 1, 64, FAKE, FAKE, NULL) == 1
    assert lib.gnf4_pack(FAKE, 0, 1, 1, 96, FAKE, FAKE, NULL) == 1     # K % 64
    assert lib.gnf4_pack(FAKE, 0, 0, 1, 64, FAKE, FAKE, NULL) == 1     # E <= 0
    assert lib.gnf4_pack(FAKE, 7, 1, 1, 64, FAKE, FAKE, NULL) == 1     # dtype
    assert lib.gnf4_pack(ctypes.c_void_p(0x1008), 0, 1, 1, 64, FAKE, FAKE, NULL) == 1  # align


def test_route_rejects_bad_arguments(lib):
    args = [FAKE] * 8 + [NULL, 0, NULL]
    assert lib.gnf4_route_sort(FAKE, 4, 8, 0, *args) == 1        # top_k < 1
    assert lib.gnf4_route_sort(FAKE, 4, 8, 9, *args) == 1        # top_k > E
    assert lib.gnf4_route_sort(FAKE, 4, 2048, 8, *args) == 3     # E > 1024
    assert lib.gnf4_route_sort(FAKE, 4, 64, 33, *args) == 3      # top_k > 32
    assert lib.gnf4_route_sort(FAKE, -1, 8, 2, *args) == 1       # T < 0
    assert lib.gnf4_route_sort(NULL, 4, 8, 2, *args) == 1        # null logits


def test_route_gemm_one_token_rejects_bad_arguments(lib):
    f = lib.gnf4_route_gemm_one_token
    args = [None, 64, 8, None, None, None, 0, 256, 512, None, None, None, None, None, None, None,
            None, None, None, 0, None]
    bad_e = list(args)
    bad_e[1] = 129                      # more than two experts per lane of the ranking wavefronts
    assert f(*bad_e) == 3               # GNF4_ERR_UNSUPPORTED
    bad_k = list(args)
    bad_k[2] = 65                       # top_k above E
    assert f(*bad_k) == 1               # GNF4_ERR_INVALID_ARG
    big_k = list(args)
    big_k[2] = 33                       # top_k above gnf4_route_sort's 32
    assert f(*big_k) == 3
    bad_kdim = list(args)
    bad_kdim[8] = 100                   # K not a multiple of 64
    assert f(*bad_kdim) == 1
    assert f(*args) == 1                # null pointers


def test_gemm_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(x=FAKE, p=FAKE, a=FAKE, E=4, N=64, K=128, s=FAKE, i=FAKE, G=2, M=8, y=FAKE,
                 path=0, split=0, adt=1)
        a.update(kw)
        return lib.gnf4_grouped_gemm_ex(a["x"], a["p"], a["a"], a["E"], a["N"], a["K"], a["s"],
                                        a["i"], a["G"], a["M"], a["y"], NULL, 0, a["path"],
                                        a["split"], a["adt"], NULL)
    assert call(K=96) == 1
    assert call(K=32) == 1
    assert call(N=0) == 1
    assert call(M=-1) == 1
    assert call(path=3) == 1
    assert call(split=17) == 1
    assert call(x=NULL) == 1
    assert call(M=0) == 0     # nothing to do
    assert call(G=0) == 0
    assert call(x=ctypes.c_void_p(0x1004)) == 1   # x must be 16-byte aligned
    assert call(adt=7) == 1                       # absmax dtype
    assert call(a=ctypes.c_void_p(0x1002)) == 1   # fp32 absmax must be 4-byte aligned
    # pack_ex(w, w_dtype, E, N, K, packed, absmax, absmax_dtype, stream)
    assert lib.gnf4_pack_ex(FAKE, 0, 1, 1, 64, FAKE, FAKE, 5, NULL) == 1
    assert lib.gnf4_pack_ex(FAKE, 0, 1, 1, 64, FAKE, ctypes.c_void_p(0x1001), 0, NULL) == 1
    # dgrad(dy, packed, absmax, E, N, K, sizes, ids, G, M, dx, ws, ws_bytes, absmax_dtype, stream)
    assert lib.gnf4_grouped_dgrad(FAKE, FAKE, FAKE, 4, 64, 96, FAKE, FAKE, 2, 8, FAKE, NULL, 0,
                                  1, NULL) == 1   # K % 64
    assert lib.gnf4_grouped_dgrad(FAKE, FAKE, FAKE, 4, 64, 128, FAKE, FAKE, 2, 0, FAKE, NULL, 0,
                                  1, NULL) == 0   # M == 0
    assert lib.gnf4_grouped_dgrad(FAKE, FAKE, FAKE, 4, 64, 128, FAKE, FAKE, 2, 8, FAKE, NULL, 0,
                                  9, NULL) == 1   # absmax dtype
    assert lib.gnf4_gather_rows(FAKE, 4, 96, FAKE, 2, 8, FAKE, NULL) == 1


def test_glue_argument_errors(lib):
    # swiglu(gate_up, M, I, h, stream)
    assert lib.gnf4_swiglu(FAKE, 0, 8, FAKE, NULL) == 0        # M == 0: nothing to do
    assert lib.gnf4_swiglu(FAKE, -1, 8, FAKE, NULL) == 1
    assert lib.gnf4_swiglu(FAKE, 4, 0, FAKE, NULL) == 1
    assert lib.gnf4_swiglu(NULL, 4, 8, FAKE, NULL) == 1
    assert lib.gnf4_swiglu(FAKE, 4, 8, NULL, NULL) == 1
    assert lib.gnf4_swiglu(ctypes.c_void_p(0x1001), 4, 8, FAKE, NULL) == 1   # odd address
    assert lib.gnf4_swiglu(FAKE, 1 << 30, 1 << 20, FAKE, NULL) == 3          # M * I >= 2^40
    # combine(y, slot_rows, topk_w, T, k, M, H, out, stream)
    assert lib.gnf4_combine(FAKE, FAKE, FAKE, 0, 8, 8, 64, FAKE, NULL) == 0  # T == 0
    assert lib.gnf4_combine(FAKE, FAKE, FAKE, -1, 8, 8, 64, FAKE, NULL) == 1
    assert lib.gnf4_combine(FAKE, FAKE, FAKE, 1, 0, 8, 64, FAKE, NULL) == 1  # top_k < 1
    assert lib.gnf4_combine(FAKE, FAKE, FAKE, 1, 8, -1, 64, FAKE, NULL) == 1
    assert lib.gnf4_combine(FAKE, FAKE, FAKE, 1, 8, 8, 0, FAKE, NULL) == 1   # H <= 0
    assert lib.gnf4_combine(FAKE, NULL, FAKE, 1, 8, 8, 64, FAKE, NULL) == 1
    assert lib.gnf4_combine(NULL, FAKE, FAKE, 1, 8, 8, 64, FAKE, NULL) == 1  # y null, M > 0
    assert lib.gnf4_combine(FAKE, ctypes.c_void_p(0x1002), FAKE, 1, 8, 8, 64, FAKE, NULL) == 1
    assert lib.gnf4_combine(FAKE, FAKE, FAKE, 1 << 29, 8, 8, 64, FAKE, NULL) == 3  # T*k >= 2^31


def test_route_workspace_follows_the_chunk_rule(lib):
    """Up to 32 tokens sort in one launch with no workspace; beyond that,
    chunks of 16 tokens keep one int32 count per (chunk, expert)."""
    q = lib.gnf4_route_sort_workspace_size
    assert q(1, 64, 8) == 0
    assert q(32, 128, 8) == 0
    assert q(33, 128, 8) == 3 * 128 * 4
    assert q(4096, 256, 8) == 256 * 256 * 4


def test_dgrad_split_rule(lib):
    """The decode-path dgrad's N split, seen through its workspace size (fp32
    partials [S, M, K]) on a 256-CU device (the size a host without a device
    plans for): about two wavefronts per SIMD, each split at least one batch
    of 8 rows per team, or of 4 at one row of dy when batches of 8 would
    allow at most half the splits wanted.  Rows of 32 chunks use 32-lane
    teams, two per wavefront: batches of 8 would cap OLMoE down at 16 of 32
    splits, so it takes batches of 4 and 32 splits, as OLMoE gate_up's
    64-lane teams do with batches of 8; Qwen3's gate_up, capped at 24 of 32,
    keeps batches of 8."""
    q = lib.gnf4_grouped_dgrad_workspace_size
    assert q(8, 2048, 2048, 8, 64) == 32 * 8 * 2048 * 4    # OLMoE gate_up: 64-lane teams
    assert q(8, 2048, 1024, 8, 64) == 32 * 8 * 1024 * 4    # OLMoE down: 32-lane teams
    assert q(3, 1536, 2048, 3, 4) == 48 * 3 * 2048 * 4     # three rows, 48 splits
    assert q(12, 1536, 2048, 4, 4) == 24 * 12 * 2048 * 4   # three rows per group: batches of 8
    assert q(8, 1536, 2048, 8, 128) == 24 * 8 * 2048 * 4   # Qwen3 gate_up: 24 of 32, batches of 8
    assert q(8, 2048, 768, 8, 128) == 32 * 8 * 768 * 4     # Qwen3 down: 16 of 32, batches of 4


def test_dgrad_tile_workspace_any_width(lib):
    """A prefill-sized dgrad batch (M >= 32 G) plans the tile path for any
    width N: its workspace is the staged dy, 4 (M + 1) bytes of exponents and
    2 (M + 1) ceil128(N) fp16 bytes, each rounded up to 256."""
    q = lib.gnf4_grouped_dgrad_workspace_size_ex
    q.restype = ctypes.c_size_t
    q.argtypes = [ctypes.c_int64] * 5 + [ctypes.c_int32]
    def staged(M, N):
        up = lambda b: (b + 255) // 256 * 256
        return up(4 * (M + 1)) + up(2 * (M + 1) * ((N + 127) // 128 * 128))
    for N in (1, 7, 301, 2048):
        assert q(64, N, 256, 2, 3, 0) == staged(64, N)
        assert q(64, N, 256, 2, 3, 2) == staged(64, N)


def test_no_cpu_fallback_in_binding():
    """The binding never routes through the oracle or a torch fallback."""
    src = open(os.path.join(ROOT, "grouped_nf4_expert_amd", "gnf4.py")).read()
    assert "oracle" not in src
    for line in src.splitlines():
        assert "import numpy" not in line


def test_noalloc_rejects_bad_arguments(lib):
    lib.gnf4_noalloc_scratch_bytes.restype = ctypes.c_size_t
    assert lib.gnf4_noalloc_scratch_bytes() == 32 << 20
    f = lib.gnf4_grouped_gemm_gather_noalloc
    # x, T, slots, top_k, packed, absmax, E, N, K, sizes, ids, G, M, y, path, split_k, dtype, stream
    ok = [FAKE, 4, FAKE, 2, FAKE, FAKE, 4, 64, 128, FAKE, FAKE, 2, 8, FAKE, 0, 0, 1, NULL]
    bad_slots = list(ok)
    bad_slots[2] = NULL
    assert f(*bad_slots) == 1                      # the fused gather needs slots
    bad_k = list(ok)
    bad_k[8] = 96
    assert f(*bad_k) == 1                          # K % 64
    bad_path = list(ok)
    bad_path[14] = 3
    assert f(*bad_path) == 1
    assert f(*(ok[:12] + [0] + ok[13:])) == 0      # M == 0: nothing to do
    # a prefill batch whose staged rows exceed the static scratch: refused
    # before any pointer is touched
    big = list(ok)
    big[7], big[8], big[11], big[12], big[14] = 4096, 7168, 256, 32768, 2
    assert f(*big) == 3



def test_moe_ffn_one_token_rejects_bad_arguments(lib):
    lib.gnf4_moe_ffn_one_token_workspace_size.restype = ctypes.c_size_t
    lib.gnf4_moe_ffn_one_token_workspace_size.argtypes = [ctypes.c_int32]
    # 10 k + 1 words, one per 128-byte line
    assert lib.gnf4_moe_ffn_one_token_workspace_size(8) == 81 * 128
    assert lib.gnf4_moe_ffn_one_token_workspace_size(0) == 0
    sup = lib.gnf4_moe_ffn_one_token_supported
    sup.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64]
    assert sup(64, 8, 2048, 1024) == 1          # OLMoE expert layer
    assert sup(128, 8, 2048, 768) == 1          # Qwen3-30B
    assert sup(128, 4, 2880, 2880) == 0         # GPT-OSS-120B: more workgroups than fit at once
    assert sup(8, 2, 256, 128) == 0             # no fused kernel for this shape
    assert sup(200, 8, 2048, 1024) == 0         # more experts than the routing handles
    f = lib.gnf4_moe_ffn_one_token
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    f.argtypes = [vp, i64, i32, vp, vp, vp, vp, vp, i32, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                  vp, vp, vp, sz, vp]
    # logits, E, k, x, gp, ga, dp, da, dtype, H, I, h, y, 8 route outputs, ws, ws_bytes, stream
    ok = [FAKE, 64, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2048, 1024, FAKE, FAKE] + [FAKE] * 8 + \
         [FAKE, 81 * 128, NULL]
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a1=0) == 1            # E
    assert call(a2=65) == 1           # top_k > E
    assert call(a9=2000) == 1         # H % 64
    assert call(a10=96) == 1          # I % 64
    assert call(a8=7) == 1            # absmax dtype
    assert call(a3=NULL) == 1         # x
    assert call(a1=200) == 3          # E > 128
    assert call(a2=33, a1=64) == 3    # top_k > 32
    assert call(a21=NULL) == 4        # no workspace
    assert call(a22=80 * 128) == 4    # workspace too small
