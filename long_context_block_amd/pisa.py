"""Thin ctypes binding of libpisa.so (the C ABI in include/pisa.h).

The functions keep the C names and only marshal arguments: tensors become device pointers, the
stream defaults to torch's current stream. PyTorch only provides device memory and streams; every
step of the path runs in the HIP library. Loading fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpisa.so")

PISA_OK, PISA_EINVAL, PISA_EUNSUPPORTED, PISA_EWORKSPACE, PISA_EHIP = 0, -1, -2, -3, -4
PISA_FP32, PISA_BF16 = 0, 1
PISA_OP_SELECT, PISA_OP_ATTN, PISA_OP_DECODE, PISA_OP_BSA, PISA_OP_ATTN_BWD, PISA_OP_TRACE = 1, 2, 3, 4, 5, 6

EXPORTED = ["pisa_pyramid_layout", "pisa_workspace_size", "pisa_build_pyramid", "pisa_select", "pisa_sparse_attn",
            "pisa_decode_step", "bsa_select", "pisa_status_string", "pisa_last_error", "pisa_stage_timing",
            "pisa_stage_times", "pisa_select_noalloc", "pisa_select_noalloc_max_bytes", "pisa_flat_leaf_lse",
            "pisa_selection_quality", "pisa_build_pyramid_pooled", "pisa_select_variant",
            "pisa_sparse_attn_backward", "pisa_select_trace"]


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("branch", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("q_tile", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


def make_shape(*, batch, seq_len, n_q_heads, n_kv_heads, head_dim, block, top_k, branch=2, q_tile=1, scale=0.0,
               dtype="bf16", causal=1) -> Shape:
    dt = {"bf16": PISA_BF16, "fp32": PISA_FP32}.get(dtype, dtype)
    return Shape(batch, seq_len, n_q_heads, n_kv_heads, head_dim, block, top_k, branch, causal, q_tile, scale, dt)


PISA_POOL_MEAN, PISA_POOL_SUM, PISA_POOL_MAX = 0, 1, 2
PISA_SCORE_LSE, PISA_SCORE_MEAN, PISA_SCORE_MEAN_VAR = 0, 1, 2
PISA_BUDGET_FIXED, PISA_BUDGET_HALVING = 0, 1


class Variant(ctypes.Structure):
    _fields_ = [("score", ctypes.c_int32), ("budget", ctypes.c_int32), ("max_level", ctypes.c_int32)]


class PisaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_SP = ctypes.POINTER(Shape)


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpisa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with python -m long_context_block_amd.build")
    lib = ctypes.CDLL(path)
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "pisa_pyramid_layout": [_SP, ctypes.POINTER(i32), ctypes.POINTER(i64), ctypes.POINTER(i64)],
        "pisa_workspace_size": [_SP, i32, ctypes.POINTER(sz)],
        "pisa_build_pyramid": [_SP, _P, ctypes.POINTER(i32), _P, _P, _P],
        "pisa_select": [_SP, _P, _P, _P, _P, _P, _P, sz, _P],
        "pisa_select_noalloc": [_SP, _P, _P, _P, _P, _P, _P],
        "pisa_sparse_attn": [_SP, _P, _P, _P, _P, _P, _P, _P, sz, _P],
        "pisa_decode_step": [_SP, ctypes.POINTER(i32), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P],
        "bsa_select": [_SP, _P, _P, _P, _P, sz, _P],
        "pisa_flat_leaf_lse": [_SP, _P, _P, _P, i32, _P, _P, _P],
        "pisa_selection_quality": [_SP, _P, _P, _P, i32, _P, _P, _P, _P, _P],
        "pisa_build_pyramid_pooled": [_SP, _P, i32, _P, _P, _P],
        "pisa_select_variant": [_SP, ctypes.POINTER(Variant), _P, _P, _P, _P, _P, _P],
        "pisa_sparse_attn_backward": [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P],
        "pisa_select_trace": [_SP, _P, _P, _P, _P, i64, _P, _P, sz, _P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.pisa_status_string.argtypes = [ctypes.c_int]
    lib.pisa_status_string.restype = ctypes.c_char_p
    lib.pisa_last_error.argtypes = []
    lib.pisa_last_error.restype = ctypes.c_char_p
    lib.pisa_select_noalloc_max_bytes.argtypes = []
    lib.pisa_select_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.pisa_stage_timing.argtypes = [ctypes.c_int32]
    lib.pisa_stage_timing.restype = ctypes.c_int
    lib.pisa_stage_times.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32),
                                     ctypes.c_int32]
    lib.pisa_stage_times.restype = ctypes.c_int32
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != PISA_OK:
        raise PisaError(status, where, load().pisa_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _lens(host_lens, B):
    if host_lens is None:
        return None
    arr = (ctypes.c_int32 * B)(*[int(x) for x in host_lens])
    return arr


# ------------------------------------------------------------------------------------- host-only calls
def pisa_pyramid_layout(shape: Shape):
    n = ctypes.c_int32()
    off = (ctypes.c_int64 * 32)()
    nodes = ctypes.c_int64()
    _check(load().pisa_pyramid_layout(ctypes.byref(shape), ctypes.byref(n), off, ctypes.byref(nodes)),
           "pisa_pyramid_layout")
    return n.value, [off[i] for i in range(n.value)], nodes.value


def pisa_workspace_size(shape: Shape, op: int) -> int:
    b = ctypes.c_size_t()
    _check(load().pisa_workspace_size(ctypes.byref(shape), op, ctypes.byref(b)), "pisa_workspace_size")
    return b.value


# ------------------------------------------------------------------------------------- device calls
def pisa_build_pyramid(shape, k, pyr_mean, pyr_sum=None, host_lens=None, stream=None):
    _check(load().pisa_build_pyramid(ctypes.byref(shape), _ptr(k), _lens(host_lens, shape.batch), _ptr(pyr_mean),
                                     _ptr(pyr_sum), _stream(stream)), "pisa_build_pyramid")


def pisa_select(shape, q, k, pyr_mean, sel, sel_lse=None, ws=None, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().pisa_select(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(pyr_mean), _ptr(sel), _ptr(sel_lse),
                              _ptr(ws), nbytes, _stream(stream)), "pisa_select")


def pisa_select_trace(shape, q, k, pyr_mean, units, trace, ws=None, stream=None):
    """units: int64 [n] unit indices; trace: int32 [n, n_levels, K] (level 0 = the selection)."""
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    n = units.numel() if units is not None else 0
    _check(load().pisa_select_trace(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(pyr_mean), _ptr(units), n,
                                    _ptr(trace), _ptr(ws), nbytes, _stream(stream)), "pisa_select_trace")


def pisa_select_noalloc(shape, q, k, pyr_mean, sel, sel_lse=None, stream=None):
    _check(load().pisa_select_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(pyr_mean), _ptr(sel),
                                      _ptr(sel_lse), _stream(stream)), "pisa_select_noalloc")


def pisa_select_noalloc_max_bytes() -> int:
    return int(load().pisa_select_noalloc_max_bytes())


def pisa_sparse_attn(shape, q, k, v, sel, o, o_lse=None, ws=None, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().pisa_sparse_attn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(o), _ptr(o_lse),
                                   _ptr(ws), nbytes, _stream(stream)), "pisa_sparse_attn")


def pisa_sparse_attn_backward(shape, q, k, v, sel, o, o_lse, d_o, d_q, d_k, d_v, ws=None, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().pisa_sparse_attn_backward(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(o),
                                            _ptr(o_lse), _ptr(d_o), _ptr(d_q), _ptr(d_k), _ptr(d_v), _ptr(ws), nbytes,
                                            _stream(stream)), "pisa_sparse_attn_backward")


def pisa_decode_step(shape, host_lens, q_new, k_new, v_new, k_cache, v_cache, pyr_sum, pyr_mean, o, sel_out=None,
                     ws=None, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().pisa_decode_step(ctypes.byref(shape), _lens(host_lens, shape.batch), _ptr(q_new), _ptr(k_new),
                                   _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(pyr_sum), _ptr(pyr_mean), _ptr(o),
                                   _ptr(sel_out), _ptr(ws), nbytes, _stream(stream)), "pisa_decode_step")


def bsa_select(shape, q, k, sel, ws=None, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().bsa_select(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(sel), _ptr(ws), nbytes, _stream(stream)),
           "bsa_select")


def pisa_flat_leaf_lse(shape, q, k, positions, leaf_lse, row_lse, stream=None):
    _check(load().pisa_flat_leaf_lse(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(positions), int(positions.numel()),
                                     _ptr(leaf_lse), _ptr(row_lse), _stream(stream)), "pisa_flat_leaf_lse")


def pisa_selection_quality(shape, leaf_lse, row_lse, positions, sel, flat_sel, recall, mass, stream=None):
    _check(load().pisa_selection_quality(ctypes.byref(shape), _ptr(leaf_lse), _ptr(row_lse), _ptr(positions),
                                         int(positions.numel()), _ptr(sel), _ptr(flat_sel), _ptr(recall), _ptr(mass),
                                         _stream(stream)), "pisa_selection_quality")


def pisa_build_pyramid_pooled(shape, k, pool, summary, variance=None, stream=None):
    _check(load().pisa_build_pyramid_pooled(ctypes.byref(shape), _ptr(k), int(pool), _ptr(summary), _ptr(variance),
                                            _stream(stream)), "pisa_build_pyramid_pooled")


def pisa_select_variant(shape, variant, q, k, summary, sel, variance=None, stream=None):
    _check(load().pisa_select_variant(ctypes.byref(shape), ctypes.byref(variant), _ptr(q), _ptr(k), _ptr(summary),
                                      _ptr(variance), _ptr(sel), _stream(stream)), "pisa_select_variant")


def pisa_stage_timing(enable: bool):
    _check(load().pisa_stage_timing(1 if enable else 0), "pisa_stage_timing")


def pisa_stage_times() -> dict:
    """{stage name: (total ms, launches)} accumulated since stage timing was enabled."""
    lib = load()
    cap = 64
    names = (ctypes.c_char * 32 * cap)()
    tot = (ctypes.c_double * cap)()
    cnt = (ctypes.c_int32 * cap)()
    n = lib.pisa_stage_times(names, tot, cnt, cap)
    if n < 0:
        _check(n, "pisa_stage_times")
    return {bytes(names[i]).split(b"\0")[0].decode(): (tot[i], cnt[i]) for i in range(min(n, cap))}


# ------------------------------------------------------------------------------------- allocation helpers
def torch_dtype(shape: Shape):
    return torch.bfloat16 if shape.dtype == PISA_BF16 else torch.float32


def alloc_workspace(shape: Shape, op: int, device="cuda"):
    """Workspace for `op`; the decode step's starts zeroed, as its counters require."""
    n = pisa_workspace_size(shape, op)
    if op == PISA_OP_DECODE:
        return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def pyramid_rows(shape: Shape) -> int:
    _, _, nodes = pisa_pyramid_layout(shape)
    return shape.batch * shape.n_kv_heads * nodes


def default_scale(shape: Shape) -> float:
    return shape.scale if shape.scale > 0 else 1.0 / math.sqrt(shape.head_dim)
