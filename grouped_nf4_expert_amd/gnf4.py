"""Thin Python binding over libgnf4 (include/gnf4.h).

Argument marshalling only: tensors are checked for dtype, shape and device,
their data pointers and the current HIP stream are handed to the C ABI, and
output tensors are allocated with torch (torch is used for device memory and
streams, nothing else).  Every computation happens in the library's HIP
kernels.  The library must be built (``python -m grouped_nf4_expert_amd.build``);
if it is missing, or a tensor is not on the GPU, the call raises -- there is
no CPU path and no fallback.
"""

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgnf4.so")

GNF4_OK = 0
GNF4_DTYPE_BF16 = 0
GNF4_DTYPE_F32 = 1
PATH_AUTO, PATH_DECODE, PATH_TILE = 0, 1, 2

_lib = None


class Gnf4Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        text = library().gnf4_status_string(status).decode()
        extra = ""
        if status == 5:
            extra = f" (hipError {library().gnf4_last_hip_error()})"
        super().__init__(f"{where}: {text}{extra}")


def library():
    """Load libgnf4.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m grouped_nf4_expert_amd.build` "
            "(the grouped NF4 GEMM has no CPU implementation to fall back to)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.gnf4_status_string.restype = ctypes.c_char_p
    lib.gnf4_status_string.argtypes = [ctypes.c_int]
    lib.gnf4_last_hip_error.restype = ctypes.c_int
    lib.gnf4_last_hip_error.argtypes = []
    lib.gnf4_version.restype = ctypes.c_char_p
    lib.gnf4_version.argtypes = []
    lib.gnf4_pack.restype = ctypes.c_int
    lib.gnf4_pack.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp]
    lib.gnf4_pack_ex.restype = ctypes.c_int
    lib.gnf4_pack_ex.argtypes = [vp, i32, i64, i64, i64, vp, vp, i32, vp]
    lib.gnf4_route_sort_workspace_size.restype = sz
    lib.gnf4_route_sort_workspace_size.argtypes = [i64, i64, i32]
    lib.gnf4_route_sort.restype = ctypes.c_int
    lib.gnf4_route_sort.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                    vp]
    lib.gnf4_grouped_dgrad_workspace_size.restype = sz
    lib.gnf4_grouped_dgrad_workspace_size.argtypes = [i64, i64, i64, i64, i64]
    lib.gnf4_grouped_dgrad_workspace_size_ex.restype = sz
    lib.gnf4_grouped_dgrad_workspace_size_ex.argtypes = [i64, i64, i64, i64, i64, i32]
    lib.gnf4_grouped_dgrad_ex.restype = ctypes.c_int
    lib.gnf4_grouped_dgrad_ex.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i64, vp, vp, sz,
                                          i32, i32, vp]
    lib.gnf4_route_gemm_one_token_workspace_size.restype = sz
    lib.gnf4_route_gemm_one_token_workspace_size.argtypes = [i64, i32, i64, i64]
    lib.gnf4_route_gemm_one_token.restype = ctypes.c_int
    lib.gnf4_route_gemm_one_token.argtypes = [vp, i64, i32, vp, vp, vp, i32, i64, i64, vp, vp, vp,
                                              vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gnf4_grouped_dgrad.restype = ctypes.c_int
    lib.gnf4_grouped_dgrad.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i64, vp, vp, sz,
                                       i32, vp]
    lib.gnf4_grouped_gemm_mxfp4.restype = ctypes.c_int
    lib.gnf4_grouped_gemm_mxfp4.argtypes = [vp, i64, vp, i32, vp, vp, i64, i64, i64, vp, vp, i64,
                                            i64, vp, vp, sz, i32, i32, vp]
    lib.gnf4_swiglu.restype = ctypes.c_int
    lib.gnf4_swiglu.argtypes = [vp, i64, i64, vp, vp]
    lib.gnf4_moe_ffn_one_token_workspace_size.restype = sz
    lib.gnf4_moe_ffn_one_token_workspace_size.argtypes = [i32]
    lib.gnf4_moe_ffn_one_token_supported.restype = ctypes.c_int
    lib.gnf4_moe_ffn_one_token_supported.argtypes = [i64, i32, i64, i64]
    lib.gnf4_moe_ffn_one_token.restype = ctypes.c_int
    lib.gnf4_moe_ffn_one_token.argtypes = [vp, i64, i32, vp, vp, vp, vp, vp, i32, i64, i64, vp, vp,
                                           vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gnf4_combine.restype = ctypes.c_int
    lib.gnf4_combine.argtypes = [vp, vp, vp, i64, i32, i64, i64, vp, vp]
    lib.gnf4_gather_rows.restype = ctypes.c_int
    lib.gnf4_gather_rows.argtypes = [vp, i64, i64, vp, i32, i64, vp, vp]
    lib.gnf4_grouped_gemm_workspace_size.restype = sz
    lib.gnf4_grouped_gemm_workspace_size.argtypes = [i64, i64, i64, i64, i64]
    lib.gnf4_grouped_gemm_workspace_size_ex.restype = sz
    lib.gnf4_grouped_gemm_workspace_size_ex.argtypes = [i64, i64, i64, i64, i64, i32, i32]
    lib.gnf4_grouped_gemm.restype = ctypes.c_int
    lib.gnf4_grouped_gemm.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i64, vp, vp, sz, vp]
    lib.gnf4_grouped_gemm_gather.restype = ctypes.c_int
    lib.gnf4_grouped_gemm_gather.argtypes = [vp, i64, vp, i32, vp, vp, i64, i64, i64, vp, vp, i64,
                                             i64, vp, vp, sz, i32, i32, i32, vp]
    lib.gnf4_grouped_gemm_ex.restype = ctypes.c_int
    lib.gnf4_grouped_gemm_ex.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i64, vp, vp,
                                         sz, i32, i32, i32, vp]
    lib.gnf4_noalloc_scratch_bytes.restype = sz
    lib.gnf4_noalloc_scratch_bytes.argtypes = []
    lib.gnf4_grouped_gemm_gather_noalloc.restype = ctypes.c_int
    lib.gnf4_grouped_gemm_gather_noalloc.argtypes = [vp, i64, vp, i32, vp, vp, i64, i64, i64, vp,
                                                     vp, i64, i64, vp, i32, i32, i32, vp]
    _lib = lib
    return lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check(status, where):
    if status != GNF4_OK:
        raise Gnf4Error(status, where)


def _need(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ------------------------------------------------------------------- pack

def _absmax_dtype(absmax):
    if absmax.dtype == torch.float32:
        return GNF4_DTYPE_F32
    if absmax.dtype == torch.bfloat16:
        return GNF4_DTYPE_BF16
    raise TypeError("absmax must be float32 or bfloat16")


def pack(w, out=None, absmax_dtype=torch.float32):
    """NF4-pack ``w`` [..., N, K] (bf16 or fp32 on the GPU).

    Returns ``(packed uint8 [..., N, K/2], absmax [..., N, K/64])`` with the
    absmax in ``absmax_dtype`` (float32, or bfloat16 for 4.25 bits/weight);
    with ``out`` given, its absmax tensor's dtype decides.
    """
    if w.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("w must be bfloat16 or float32")
    _need(w, "w", w.dtype)
    if w.dim() < 2:
        raise ValueError("w must be at least 2-D")
    K = w.shape[-1]
    N = w.shape[-2]
    E = w.numel() // max(N * K, 1)
    if out is None:
        packed = torch.empty(w.shape[:-1] + (K // 2,), dtype=torch.uint8, device=w.device)
        absmax = torch.empty(w.shape[:-1] + (K // 64,), dtype=absmax_dtype, device=w.device)
    else:
        packed, absmax = out
    dt = GNF4_DTYPE_BF16 if w.dtype == torch.bfloat16 else GNF4_DTYPE_F32
    _check(library().gnf4_pack_ex(_ptr(w), dt, E, N, K, _ptr(packed), _ptr(absmax),
                                  _absmax_dtype(absmax), _stream()), "gnf4_pack_ex")
    return packed, absmax


# ------------------------------------------------------------- route_sort

@dataclass
class RouteResult:
    topk_ids: torch.Tensor        # int32 [T, k]
    topk_w: torch.Tensor          # fp32 [T, k]
    expert_offsets: torch.Tensor  # int32 [E + 1]
    sorted_slots: torch.Tensor    # int32 [T * k]
    slot_rows: torch.Tensor       # int32 [T * k]: grouped row of each flat slot
    group_sizes: torch.Tensor     # int32 [E]
    group_expert_ids: torch.Tensor  # int32 [E]
    num_groups: torch.Tensor      # int32 [1]


class RouteBuffers:
    """Preallocated outputs and workspace for repeated route_sort calls."""

    def __init__(self, T, E, top_k, device):
        i32 = dict(dtype=torch.int32, device=device)
        self.T, self.E, self.top_k = T, E, top_k
        self.result = RouteResult(
            topk_ids=torch.empty((T, top_k), **i32),
            topk_w=torch.empty((T, top_k), dtype=torch.float32, device=device),
            expert_offsets=torch.empty(E + 1, **i32),
            sorted_slots=torch.empty(T * top_k, **i32),
            slot_rows=torch.empty(T * top_k, **i32),
            group_sizes=torch.empty(E, **i32),
            group_expert_ids=torch.empty(E, **i32),
            num_groups=torch.empty(1, **i32),
        )
        nbytes = library().gnf4_route_sort_workspace_size(T, E, top_k)
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        self.ws_bytes = nbytes


def route_sort(logits, top_k, buffers=None):
    """Top-k routing with softmax weights and the stable token->expert sort."""
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    if buffers is None:
        buffers = RouteBuffers(T, E, top_k, logits.device)
    r = buffers.result
    _check(library().gnf4_route_sort(
        _ptr(logits), T, E, top_k, _ptr(r.topk_ids), _ptr(r.topk_w), _ptr(r.expert_offsets),
        _ptr(r.sorted_slots), _ptr(r.slot_rows), _ptr(r.group_sizes), _ptr(r.group_expert_ids),
        _ptr(r.num_groups), _ptr(buffers.workspace), buffers.ws_bytes, _stream()),
        "gnf4_route_sort")
    return r


def route_gemm_one_token(logits, x, packed, absmax, top_k, buffers=None, y=None,
                         workspace=None):
    """A batch-1 decode step's route/sort and grouped GEMM in one launch:
    ``logits`` [1, E] fp32 (E <= 128), ``x`` [1, K] bf16, the packed stack as
    grouped_gemm takes it.  Returns (y [top_k, N] in grouped order, the
    RouteResult written into ``buffers``, as route_sort gives for T = 1)."""
    _need(logits, "logits", torch.float32, 2)
    _need(x, "x", torch.bfloat16, 2)
    _need(packed, "packed", torch.uint8, 3)
    _need(absmax, "absmax", absmax.dtype, 3)
    adt = _absmax_dtype(absmax)
    T, E = logits.shape
    if T != 1 or x.shape[0] != 1:
        raise ValueError("route_gemm_one_token routes exactly one token")
    E_w, N, half_k = packed.shape
    K = 2 * half_k
    if E_w != E or x.shape[1] != K or absmax.shape != (E, N, K // 64):
        raise ValueError("logits/x/packed/absmax shapes do not agree")
    if buffers is None:
        buffers = RouteBuffers(1, E, top_k, logits.device)
    r = buffers.result
    if y is None:
        y = torch.empty((top_k, N), dtype=torch.bfloat16, device=x.device)
    need = library().gnf4_route_gemm_one_token_workspace_size(E, top_k, N, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().gnf4_route_gemm_one_token(
        _ptr(logits), E, top_k, _ptr(x), _ptr(packed), _ptr(absmax), adt, N, K, _ptr(y),
        _ptr(r.topk_ids), _ptr(r.topk_w), _ptr(r.expert_offsets), _ptr(r.sorted_slots),
        _ptr(r.slot_rows), _ptr(r.group_sizes), _ptr(r.group_expert_ids), _ptr(r.num_groups),
        _ptr(workspace), ws_bytes, _stream()), "gnf4_route_gemm_one_token")
    return y, r


def moe_ffn_one_token_workspace(top_k, device):
    """The per-pick counters of moe_ffn_one_token, zeroed (every call leaves
    them zero again); the last int32 is the error flag."""
    n = library().gnf4_moe_ffn_one_token_workspace_size(top_k)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_ffn_one_token_supported(E, top_k, H, I):
    return bool(library().gnf4_moe_ffn_one_token_supported(E, top_k, H, I))


def moe_ffn_one_token(logits, x, gate_up, down, top_k, buffers=None, h=None, y=None,
                      workspace=None):
    """One token's MoE expert feed-forward in one launch: route/sort,
    gate_up over the picks, SwiGLU, down.  ``logits`` [1, E] fp32 (E <= 128),
    ``x`` [1, H] bf16, ``gate_up`` = (packed [E, 2I, H/2], absmax) with the
    gate rows first, ``down`` = (packed [E, H, I/2], absmax).  Returns
    (y [top_k, H], h [top_k, I], RouteResult), rows in grouped order; the
    weighted combine is combine(y, ...).  ``workspace`` (from
    moe_ffn_one_token_workspace) may be reused across calls on one stream."""
    _need(logits, "logits", torch.float32, 2)
    _need(x, "x", torch.bfloat16, 2)
    gp, ga = gate_up
    dp, da = down
    for t, n in ((gp, "gate_up packed"), (dp, "down packed")):
        _need(t, n, torch.uint8, 3)
    for t, n in ((ga, "gate_up absmax"), (da, "down absmax")):
        _need(t, n, t.dtype, 3)
    adt = _absmax_dtype(ga)
    if _absmax_dtype(da) != adt:
        raise ValueError("gate_up and down absmax dtypes differ")
    T, E = logits.shape
    if T != 1 or x.shape[0] != 1:
        raise ValueError("moe_ffn_one_token routes exactly one token")
    H = x.shape[1]
    if gp.shape[0] != E or gp.shape[2] * 2 != H or gp.shape[1] % 2 != 0:
        raise ValueError("gate_up stack must be [E, 2I, H/2]")
    I = gp.shape[1] // 2
    if dp.shape != (E, H, I // 2) or ga.shape != (E, 2 * I, H // 64) or da.shape != (E, H, I // 64):
        raise ValueError("down stack must be [E, H, I/2] with absmax [E, H, I/64]")
    if buffers is None:
        buffers = RouteBuffers(1, E, top_k, logits.device)
    r = buffers.result
    if h is None:
        h = torch.empty((top_k, I), dtype=torch.bfloat16, device=x.device)
    if y is None:
        y = torch.empty((top_k, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = moe_ffn_one_token_workspace(top_k, x.device)
    _check(library().gnf4_moe_ffn_one_token(
        _ptr(logits), E, top_k, _ptr(x), _ptr(gp), _ptr(ga), _ptr(dp), _ptr(da), adt, H, I,
        _ptr(h), _ptr(y), _ptr(r.topk_ids), _ptr(r.topk_w), _ptr(r.expert_offsets),
        _ptr(r.sorted_slots), _ptr(r.slot_rows), _ptr(r.group_sizes), _ptr(r.group_expert_ids),
        _ptr(r.num_groups), _ptr(workspace), workspace.numel(), _stream()),
        "gnf4_moe_ffn_one_token")
    return y, h, r


# ------------------------------------------------------------------ MXFP4

def grouped_gemm_mxfp4(x, packed, scales, group_sizes, group_expert_ids, G=None, y=None,
                       workspace=None, path=PATH_AUTO, split_k=0, sorted_slots=None, top_k=1):
    """y[M, N] (bf16) over an MXFP4 stack: ``packed`` [E, N, K/2] uint8 E2M1
    codes (element 2j in the low nibble), ``scales`` [E, N, K/32] uint8 E8M0.
    With ``sorted_slots`` the gather is fused, and ``path`` picks the kernels,
    as in grouped_gemm."""
    _need(x, "x", torch.bfloat16, 2)
    _need(packed, "packed", torch.uint8, 3)
    _need(scales, "scales", torch.uint8, 3)
    _need(group_sizes, "group_sizes", torch.int32, 1)
    _need(group_expert_ids, "group_expert_ids", torch.int32, 1)
    rows, K = x.shape
    M = rows if sorted_slots is None else sorted_slots.numel()
    if sorted_slots is not None:
        _need(sorted_slots, "sorted_slots", torch.int32, 1)
    E, N, half_k = packed.shape
    if half_k * 2 != K or scales.shape != (E, N, K // 32):
        raise ValueError("packed/scales shapes do not match x's K")
    if G is None:
        G = min(group_sizes.numel(), M)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    need = gemm_workspace_size(M, N, K, G, E, path, split_k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().gnf4_grouped_gemm_mxfp4(
        _ptr(x), rows, _ptr(sorted_slots), top_k, _ptr(packed), _ptr(scales), E, N, K,
        _ptr(group_sizes), _ptr(group_expert_ids), G, M, _ptr(y), _ptr(workspace), ws_bytes,
        path, split_k, _stream()), "gnf4_grouped_gemm_mxfp4")
    return y


# ------------------------------------------------------------------ dgrad

def grouped_dgrad(dy, packed, absmax, group_sizes, group_expert_ids, G=None, dx=None,
                  workspace=None, path=PATH_AUTO):
    """dx[M, K] (bf16) = per-group dy[rows] @ dequant(W[expert]) -- the
    activation gradient of grouped_gemm over the same packed stack.  ``path``:
    PATH_AUTO, PATH_DECODE (the GEMV kernel) or PATH_TILE (matrix cores)."""
    _need(dy, "dy", torch.bfloat16, 2)
    _need(packed, "packed", torch.uint8, 3)
    _need(absmax, "absmax", absmax.dtype, 3)
    adt = _absmax_dtype(absmax)
    _need(group_sizes, "group_sizes", torch.int32, 1)
    _need(group_expert_ids, "group_expert_ids", torch.int32, 1)
    M, N = dy.shape
    E, N_w, half_k = packed.shape
    K = 2 * half_k
    if N_w != N or absmax.shape != (E, N, K // 64):
        raise ValueError("packed/absmax shapes do not match dy's N")
    if G is None:
        G = min(group_sizes.numel(), M)
    if G > group_sizes.numel() or G > group_expert_ids.numel():
        raise ValueError("G exceeds the group arrays")
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dy.device)
    _need(dx, "dx", torch.bfloat16, 2)
    need = library().gnf4_grouped_dgrad_workspace_size_ex(M, N, K, G, E, path)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dy.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().gnf4_grouped_dgrad_ex(
        _ptr(dy), _ptr(packed), _ptr(absmax), E, N, K, _ptr(group_sizes), _ptr(group_expert_ids),
        G, M, _ptr(dx), _ptr(workspace), ws_bytes, adt, path, _stream()), "gnf4_grouped_dgrad_ex")
    return dx


# ------------------------------------------------------------ swiglu / combine

def swiglu(gate_up, out=None):
    """h = silu(gate) * up for ``gate_up`` [M, 2I] bf16 (gate half first) -> [M, I]."""
    _need(gate_up, "gate_up", torch.bfloat16, 2)
    M, two_i = gate_up.shape
    if two_i % 2:
        raise ValueError("gate_up width must be even ([gate | up])")
    I = two_i // 2
    if out is None:
        out = torch.empty((M, I), dtype=torch.bfloat16, device=gate_up.device)
    _need(out, "out", torch.bfloat16, 2)
    _check(library().gnf4_swiglu(_ptr(gate_up), M, I, _ptr(out), _stream()), "gnf4_swiglu")
    return out


def combine(y, slot_rows, topk_w, out=None):
    """out[t] = sum_j topk_w[t, j] * y[slot_rows[t*k + j]] (bf16 [T, H])."""
    _need(y, "y", torch.bfloat16, 2)
    _need(slot_rows, "slot_rows", torch.int32, 1)
    _need(topk_w, "topk_w", torch.float32, 2)
    T, k = topk_w.shape
    M, H = y.shape
    if slot_rows.numel() != T * k:
        raise ValueError("slot_rows must hold T * k entries")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _need(out, "out", torch.bfloat16, 2)
    _check(library().gnf4_combine(_ptr(y) if M > 0 else ctypes.c_void_p(0), _ptr(slot_rows),
                                  _ptr(topk_w), T, k, M, H, _ptr(out), _stream()), "gnf4_combine")
    return out


# ------------------------------------------------------------ gather_rows

def gather_rows(x, sorted_slots, top_k, out=None):
    """x_sorted[r] = x[sorted_slots[r] // top_k] (bf16 rows)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(sorted_slots, "sorted_slots", torch.int32, 1)
    T, K = x.shape
    M = sorted_slots.numel()
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
    _check(library().gnf4_gather_rows(_ptr(x), T, K, _ptr(sorted_slots), top_k, M, _ptr(out),
                                      _stream()), "gnf4_gather_rows")
    return out


# ----------------------------------------------------------- grouped_gemm

def gemm_workspace_size(M, N, K, G, E, path=PATH_AUTO, split_k=0):
    return library().gnf4_grouped_gemm_workspace_size_ex(M, N, K, G, E, path, split_k)


def grouped_gemm(x_sorted, packed, absmax, group_sizes, group_expert_ids, G=None, y=None,
                 workspace=None, path=PATH_AUTO, split_k=0, sorted_slots=None, top_k=1):
    """y[M, N] (bf16) = per-group x_sorted[rows] @ dequant(W[expert])^T.

    With ``sorted_slots`` given, ``x_sorted`` holds the token rows [T, K] and
    output row r uses token sorted_slots[r] // top_k (the gather is fused
    into the GEMM); M is then ``sorted_slots.numel()``.
    ``G`` defaults to ``min(len(group_sizes), M)``, which is exact for the
    compact groups route_sort emits (non-empty groups come first).
    """
    _need(x_sorted, "x_sorted", torch.bfloat16, 2)
    _need(packed, "packed", torch.uint8, 3)
    _need(absmax, "absmax", absmax.dtype, 3)
    adt = _absmax_dtype(absmax)
    _need(group_sizes, "group_sizes", torch.int32, 1)
    _need(group_expert_ids, "group_expert_ids", torch.int32, 1)
    rows, K = x_sorted.shape
    if sorted_slots is not None:
        _need(sorted_slots, "sorted_slots", torch.int32, 1)
        M = sorted_slots.numel()
    else:
        M = rows
    E, N, half_k = packed.shape
    if half_k * 2 != K or absmax.shape != (E, N, K // 64):
        raise ValueError("packed/absmax shapes do not match x_sorted's K")
    if G is None:
        G = min(group_sizes.numel(), M)
    if G > group_sizes.numel() or G > group_expert_ids.numel():
        raise ValueError("G exceeds the group arrays")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x_sorted.device)
    need = gemm_workspace_size(M, N, K, G, E, path, split_k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x_sorted.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if sorted_slots is None:
        _check(library().gnf4_grouped_gemm_ex(
            _ptr(x_sorted), _ptr(packed), _ptr(absmax), E, N, K, _ptr(group_sizes),
            _ptr(group_expert_ids), G, M, _ptr(y), _ptr(workspace), ws_bytes, path, split_k, adt,
            _stream()), "gnf4_grouped_gemm")
    else:
        _check(library().gnf4_grouped_gemm_gather(
            _ptr(x_sorted), rows, _ptr(sorted_slots), top_k, _ptr(packed), _ptr(absmax), E, N, K,
            _ptr(group_sizes), _ptr(group_expert_ids), G, M, _ptr(y), _ptr(workspace), ws_bytes,
            path, split_k, adt, _stream()), "gnf4_grouped_gemm_gather")
    return y


def grouped_gemm_gather_noalloc(x, sorted_slots, top_k, packed, absmax, group_sizes,
                                group_expert_ids, y, G=None, path=PATH_AUTO, split_k=0):
    """gnf4_grouped_gemm_gather_noalloc: the fused-gather grouped GEMM with
    its workspace in the library's static per-GPU scratch array, writing
    into the caller's ``y`` [M, N] (nothing is allocated, here or in the
    library).  Raises Gnf4Error (GNF4_ERR_UNSUPPORTED) when the call needs
    more workspace than gnf4_noalloc_scratch_bytes()."""
    _need(x, "x", torch.bfloat16, 2)
    _need(sorted_slots, "sorted_slots", torch.int32, 1)
    _need(packed, "packed", torch.uint8, 3)
    _need(absmax, "absmax", absmax.dtype, 3)
    _need(group_sizes, "group_sizes", torch.int32, 1)
    _need(group_expert_ids, "group_expert_ids", torch.int32, 1)
    _need(y, "y", torch.bfloat16, 2)
    T, K = x.shape
    M = sorted_slots.numel()
    E, N, half_k = packed.shape
    if half_k * 2 != K or absmax.shape != (E, N, K // 64) or y.shape != (M, N):
        raise ValueError("x/packed/absmax/y shapes do not agree")
    if G is None:
        G = min(group_sizes.numel(), M)
    _check(library().gnf4_grouped_gemm_gather_noalloc(
        _ptr(x), T, _ptr(sorted_slots), top_k, _ptr(packed), _ptr(absmax), E, N, K,
        _ptr(group_sizes), _ptr(group_expert_ids), G, M, _ptr(y), path, split_k,
        _absmax_dtype(absmax), _stream()), "gnf4_grouped_gemm_gather_noalloc")
    return y

