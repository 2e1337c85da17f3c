"""Host-side tests of the C ABI: the library loads and exports every symbol the header declares, the
host-only calls agree with the oracle's level arithmetic, and every invalid argument is rejected before
anything is enqueued (no GPU needed)."""
import ctypes
import os
import re

import pytest

import oracle as O
from long_context_block_amd import pisa as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "pisa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported():
    lib = P.load()
    declared = _declared_functions()
    assert set(declared) == set(P.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def _shape(**kw):
    base = dict(batch=1, seq_len=1024, n_q_heads=4, n_kv_heads=1, head_dim=128, block=64, top_k=16, q_tile=4,
                dtype="bf16")
    base.update(kw)
    return P.make_shape(**base)


@pytest.mark.parametrize("N,C", [(1024, 32), (1000, 32), (65536, 64), (262144, 64), (1, 64), (131328, 64)])
def test_pyramid_layout_matches_oracle_levels(N, C):
    n, offs, nodes = P.pisa_pyramid_layout(_shape(seq_len=N, block=C, q_tile=1))
    sizes = O.level_sizes(N, C, 2)
    assert n == len(sizes)
    assert nodes == sum(sizes)
    assert offs == [sum(sizes[:l]) for l in range(len(sizes))]


def test_workspace_sizes():
    s = _shape(seq_len=65536, n_q_heads=32, n_kv_heads=8)
    sel = P.pisa_workspace_size(s, P.PISA_OP_SELECT)
    U = 8 * 65536
    assert sel >= U * 16 * (4 + 4 + 4 + 2 * 4 * 4)  # kept, ranks, pairs, leaf LSEs
    s1 = _shape(seq_len=65536, n_q_heads=32, n_kv_heads=8, q_tile=1)
    assert 0 < P.pisa_workspace_size(s1, P.PISA_OP_SELECT) < sel  # only the hi/lo pyramid
    assert P.pisa_workspace_size(_shape(dtype="fp32", q_tile=1), P.PISA_OP_SELECT) == 0
    # attention: the 8 (sequence, KV head) slices at 64K fit one chunk (16 GiB budget)
    assert P.pisa_workspace_size(s, P.PISA_OP_ATTN) >= U * 16 * 4 * 128 * 2
    assert P.pisa_workspace_size(s, P.PISA_OP_BSA) >= 8 * 1024 * 128 * 4
    # decode: one arrival counter per unit, then each candidate leaf's (2K per unit) per-head LSE and output
    assert P.pisa_workspace_size(s, P.PISA_OP_DECODE) >= 8 * 4 + 8 * 32 * 4 * (128 + 1) * 4
    with pytest.raises(P.PisaError) as e:
        P.pisa_workspace_size(s, 99)
    assert e.value.status == P.PISA_EINVAL


BAD_SHAPES = [
    (dict(batch=0), P.PISA_EINVAL),
    (dict(seq_len=0), P.PISA_EINVAL),
    (dict(n_q_heads=6, n_kv_heads=4), P.PISA_EINVAL),
    (dict(n_q_heads=3, n_kv_heads=1), P.PISA_EUNSUPPORTED),
    (dict(n_q_heads=32, n_kv_heads=1, q_tile=1), P.PISA_EUNSUPPORTED),
    (dict(head_dim=96), P.PISA_EUNSUPPORTED),
    (dict(block=16), P.PISA_EUNSUPPORTED),
    (dict(top_k=0), P.PISA_EINVAL),
    (dict(top_k=33), P.PISA_EUNSUPPORTED),
    (dict(causal=0), P.PISA_EUNSUPPORTED),  # the method is causal
    (dict(branch=3), P.PISA_EUNSUPPORTED),
    (dict(q_tile=3), P.PISA_EINVAL),
    (dict(q_tile=8), P.PISA_EUNSUPPORTED),  # 8 * G(4) > 16
    (dict(dtype=7), P.PISA_EINVAL),
    (dict(scale=-1.0), P.PISA_EINVAL),
    (dict(scale=float("inf")), P.PISA_EINVAL),
    (dict(batch=64, n_q_heads=64, n_kv_heads=16, seq_len=1 << 17), P.PISA_EUNSUPPORTED),
]


@pytest.mark.parametrize("kw,status", BAD_SHAPES)
def test_invalid_shapes_rejected(kw, status):
    with pytest.raises(P.PisaError) as e:
        P.pisa_workspace_size(_shape(**kw), P.PISA_OP_SELECT)
    assert e.value.status == status
    # the same validation guards every enqueueing call (fake pointers are never touched)
    lib = P.load()
    fake = ctypes.c_void_p(1 << 20)
    st = lib.pisa_select(ctypes.byref(_shape(**kw)), fake, fake, fake, fake, None, fake, 1 << 40, None)
    assert st == status
    assert lib.pisa_last_error()


def test_null_and_misaligned_pointers_rejected():
    lib = P.load()
    s = _shape()
    good = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 4)
    big = 1 << 40
    assert lib.pisa_select(ctypes.byref(s), None, good, good, good, None, good, big, None) == P.PISA_EINVAL
    assert b"q" in lib.pisa_last_error()
    assert lib.pisa_select(ctypes.byref(s), odd, good, good, good, None, good, big, None) == P.PISA_EINVAL
    assert b"aligned" in lib.pisa_last_error()
    assert lib.pisa_select(ctypes.byref(s), good, good, good, good, odd, good, big, None) == P.PISA_EINVAL
    assert lib.pisa_build_pyramid(ctypes.byref(s), good, None, None, None, None) == P.PISA_EINVAL
    assert lib.pisa_sparse_attn(ctypes.byref(s), good, good, None, good, good, None, good, big, None) == P.PISA_EINVAL
    assert lib.bsa_select(ctypes.byref(s), good, good, None, good, big, None) == P.PISA_EINVAL
    assert lib.pisa_select(None, good, good, good, good, None, good, big, None) == P.PISA_EINVAL


def test_workspace_too_small_rejected():
    lib = P.load()
    s = _shape()
    g = ctypes.c_void_p(1 << 20)
    need = P.pisa_workspace_size(s, P.PISA_OP_SELECT)
    assert lib.pisa_select(ctypes.byref(s), g, g, g, g, None, g, need - 1, None) == P.PISA_EWORKSPACE
    assert lib.pisa_select(ctypes.byref(s), g, g, g, g, None, None, need, None) == P.PISA_EWORKSPACE
    need_a = P.pisa_workspace_size(s, P.PISA_OP_ATTN)
    assert lib.pisa_sparse_attn(ctypes.byref(s), g, g, g, g, g, None, g, need_a - 1, None) == P.PISA_EWORKSPACE
    need_b = P.pisa_workspace_size(s, P.PISA_OP_BSA)
    assert lib.bsa_select(ctypes.byref(s), g, g, g, g, need_b - 1, None) == P.PISA_EWORKSPACE


def test_host_lens_validated():
    lib = P.load()
    s = _shape(batch=2)
    g = ctypes.c_void_p(1 << 20)
    bad = (ctypes.c_int32 * 2)(5, 2000)  # 2000 > seq_len
    assert lib.pisa_build_pyramid(ctypes.byref(s), g, bad, g, g, None) == P.PISA_EINVAL
    neg = (ctypes.c_int32 * 2)(-1, 3)
    assert lib.pisa_build_pyramid(ctypes.byref(s), g, neg, g, g, None) == P.PISA_EINVAL
    full = (ctypes.c_int32 * 2)(1024, 3)  # decode needs len < capacity
    assert lib.pisa_decode_step(ctypes.byref(s), full, g, g, g, g, g, g, g, g, None, None, 0, None) == P.PISA_EINVAL
    assert lib.pisa_decode_step(ctypes.byref(s), None, g, g, g, g, g, g, g, g, None, None, 0, None) == P.PISA_EINVAL
    ok = (ctypes.c_int32 * 2)(1000, 3)
    assert lib.pisa_decode_step(ctypes.byref(s), ok, g, g, g, g, g, g, g, g, None, None, 0, None) == P.PISA_EWORKSPACE
    need = P.pisa_workspace_size(s, P.PISA_OP_DECODE)
    assert lib.pisa_decode_step(ctypes.byref(s), ok, g, g, g, g, g, g, g, g, None, g, need - 1, None) == P.PISA_EWORKSPACE


def test_attention_workspace_is_bounded_by_the_chunk():
    """The attention workspace holds one chunk of (sequence, KV head) slices, not the whole batch: a
    batch of 8 sequences of 256K tokens (64 slices of 4.4 GB of partials) runs in 22 chunks of 3 slices
    within the 16 GiB budget, not 280 GB at once."""
    big = _shape(batch=8, seq_len=262144, n_q_heads=32, n_kv_heads=8)
    three = _shape(batch=3, seq_len=262144, n_q_heads=4, n_kv_heads=1)
    assert P.pisa_workspace_size(big, P.PISA_OP_ATTN) == P.pisa_workspace_size(three, P.PISA_OP_ATTN)
    assert P.pisa_workspace_size(big, P.PISA_OP_ATTN) <= 16 << 30
    two = _shape(batch=2, seq_len=262144, n_q_heads=4, n_kv_heads=1)
    assert P.pisa_workspace_size(big, P.PISA_OP_ATTN_BWD) in (P.pisa_workspace_size(two, P.PISA_OP_ATTN_BWD),
                                                            P.pisa_workspace_size(three, P.PISA_OP_ATTN_BWD))
    small = _shape(batch=2, seq_len=1024, n_q_heads=8, n_kv_heads=2)
    four = _shape(batch=4, seq_len=1024, n_q_heads=4, n_kv_heads=1)
    assert P.pisa_workspace_size(small, P.PISA_OP_ATTN) == P.pisa_workspace_size(four, P.PISA_OP_ATTN)


def test_status_strings():
    lib = P.load()
    for st in (0, -1, -2, -3, -4):
        assert lib.pisa_status_string(st)


def test_noalloc_rejects_oversized_shape_before_any_hip_call():
    lib = P.load()
    assert lib.pisa_select_noalloc_max_bytes() == 64 << 20
    s = _shape(seq_len=65536, n_q_heads=32, n_kv_heads=8)
    fake = ctypes.c_void_p(1 << 20)
    st = lib.pisa_select_noalloc(ctypes.byref(s), fake, fake, fake, fake, None, None)
    assert st == P.PISA_EUNSUPPORTED
    assert b"scratch" in lib.pisa_last_error()
    assert lib.pisa_select_noalloc(ctypes.byref(_shape(head_dim=96)), fake, fake, fake, fake, None, None) == \
        P.PISA_EUNSUPPORTED


def test_backward_rejects_fp32_before_any_hip_call():
    lib = P.load()
    s = _shape(dtype="fp32")
    fake = ctypes.c_void_p(1 << 20)
    st = lib.pisa_sparse_attn_backward(ctypes.byref(s), fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                       fake, 1 << 30, None)
    assert st == P.PISA_EUNSUPPORTED
    need = P.pisa_workspace_size(_shape(), P.PISA_OP_ATTN_BWD)
    assert need > 0
    assert lib.pisa_sparse_attn_backward(ctypes.byref(_shape()), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                         fake, fake, need - 1, None) == P.PISA_EWORKSPACE


def test_trace_arguments_validated_before_any_hip_call():
    lib = P.load()
    s = _shape()
    g = ctypes.c_void_p(1 << 20)
    big = 1 << 40
    # the traced walk's workspace is the routing planes alone: pisa_select's at q_tile 1
    need = P.pisa_workspace_size(s, P.PISA_OP_TRACE)
    assert need == P.pisa_workspace_size(_shape(q_tile=1), P.PISA_OP_SELECT) > 0
    assert P.pisa_workspace_size(_shape(dtype="fp32"), P.PISA_OP_TRACE) == 0
    # q_tile is ignored, also where q_tile * G would be refused by pisa_select
    assert P.pisa_workspace_size(_shape(q_tile=8), P.PISA_OP_TRACE) == need
    assert lib.pisa_select_trace(ctypes.byref(s), g, g, g, g, -1, g, g, big, None) == P.PISA_EINVAL
    assert b"n_units" in lib.pisa_last_error()
    assert lib.pisa_select_trace(ctypes.byref(s), None, None, None, None, 0, None, None, 0, None) == P.PISA_OK
    assert lib.pisa_select_trace(ctypes.byref(s), g, g, g, None, 4, g, g, big, None) == P.PISA_EINVAL
    assert b"units" in lib.pisa_last_error()
    assert lib.pisa_select_trace(ctypes.byref(s), g, g, g, g, 4, None, g, big, None) == P.PISA_EINVAL
    assert b"trace" in lib.pisa_last_error()
    assert lib.pisa_select_trace(ctypes.byref(s), None, g, g, g, 4, g, g, big, None) == P.PISA_EINVAL
    assert lib.pisa_select_trace(ctypes.byref(s), g, g, g, g, 4, g, g, need - 1, None) == P.PISA_EWORKSPACE
    assert lib.pisa_select_trace(None, g, g, g, g, 4, g, g, big, None) == P.PISA_EINVAL
    assert lib.pisa_select_trace(ctypes.byref(_shape(head_dim=96)), g, g, g, g, 4, g, g, big, None) == \
        P.PISA_EUNSUPPORTED
