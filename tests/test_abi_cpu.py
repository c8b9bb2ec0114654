"""C ABI checks that need no GPU: the library loads, exports every function
include/vq.h declares, and rejects bad arguments on the host (nothing is
enqueued, so these calls never reach the device)."""
import ctypes
import os
import re

import pytest

from oracle import vq_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def b():
    from vq_dequant_matmul_gemv_amd import binding
    return binding


def _header_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names |= set(re.findall(r"\b(vq_[a-z_0-9]+)\s*\(", txt))
    return names


def test_exports_every_declared_function(b):
    declared = _header_functions()
    assert {"vq_gemv", "vq_gemm", "vq_moe_gemv", "vq_moe_gemm", "vq_dequant"} <= declared
    for name in declared:
        assert hasattr(b.LIB, name), name
    assert declared == set(b.EXPORTED)


def test_words_per_row_matches_oracle(b):
    for cols, d, k in [(1024, 2, 8), (5120, 4, 8), (2048, 8, 12), (512, 4, 12), (66, 2, 8), (96, 2, 12)]:
        assert b.words_per_row(cols, d, k) == O.words_per_row(cols, d, k)
    assert b.words_per_row(0, 2, 8) == -1
    assert b.words_per_row(64, 3, 8) == -1
    assert b.words_per_row(64, 2, 15) == -1
    assert b.words_per_row(64, 2, 3) == -1
    assert b.words_per_row(64, 2, 9) == O.words_per_row(64, 2, 9)


def _t(b, **kw):
    base = dict(codes=0x10000, codebook=0x20000, scales=0x30000, rows=16, cols=256, d=2,
                log2_k=8, group=64, num_experts=1, codebook_per_expert=0, codebook_elems=512)
    base.update(kw)
    # buffer lengths consistent with the (possibly changed) shape unless given
    E, rows, cols, d, lk, g = (base[k] for k in ("num_experts", "rows", "cols", "d", "log2_k", "group"))
    wr = O.words_per_row(cols, d, lk) if d in (2, 4, 8) and cols > 0 else 0
    base.setdefault("code_words", E * rows * wr)
    base.setdefault("scale_elems", E * rows * (cols // g) if g > 0 else 0)
    return b.CTensor(**base)


def _gemv(b, t, x=0x40000, T=1, y=0x50000):
    return b.LIB.vq_gemv(ctypes.byref(t), x, T, y, None)


@pytest.mark.parametrize("kw,status", [
    (dict(codes=0), "VQ_ERR_NULL"),
    (dict(scales=0), "VQ_ERR_NULL"),
    (dict(d=3), "VQ_ERR_GEOMETRY"),
    (dict(log2_k=15), "VQ_ERR_GEOMETRY"),
    (dict(log2_k=3), "VQ_ERR_GEOMETRY"),
    (dict(group=32), "VQ_ERR_GEOMETRY"),
    (dict(rows=0), "VQ_ERR_SHAPE"),
    (dict(cols=320, group=128), "VQ_ERR_SHAPE"),          # cols % group
    (dict(cols=192, d=4, codebook_elems=1024), "VQ_ERR_SHAPE"),   # (cols/d) % 32
    (dict(codebook_elems=256), "VQ_ERR_SHAPE"),          # sliced codebook fails loudly
    (dict(codebook_elems=1024), "VQ_ERR_SHAPE"),
    (dict(num_experts=1 << 25), "VQ_ERR_SHAPE"),         # a stack of more than 2^28 rows
    (dict(codebook_per_expert=2), "VQ_ERR_SHAPE"),
    (dict(code_words=16 * 48), "VQ_ERR_SHAPE"),          # codes packed with 12-bit codes
    (dict(code_words=511), "VQ_ERR_SHAPE"),              # short code buffer
    (dict(scale_elems=32), "VQ_ERR_SHAPE"),              # scales for group 128
    (dict(codes=0x10004), "VQ_ERR_ALIGN"),
    (dict(codebook=0x20008), "VQ_ERR_ALIGN"),
    (dict(scales=0x30002), "VQ_ERR_ALIGN"),
])
def test_gemv_rejects(b, kw, status):
    st = _gemv(b, _t(b, **kw))
    assert b.STATUS_NAMES[st] == status, b.LIB.vq_last_error()
    assert b.LIB.vq_last_error()
    assert b.LIB.vq_status_name(st).decode() == status


def test_stack_token_limit(b):
    # a stack multiplies the tokens by its experts: T * E at most 2^24
    st = _gemv(b, _t(b, num_experts=2), T=(1 << 23) + 1)
    assert b.STATUS_NAMES[st] == "VQ_ERR_SHAPE", b.LIB.vq_last_error()
    assert "stacked" in b.LIB.vq_last_error().decode()


def test_sliced_codebook_message(b):
    st = _gemv(b, _t(b, codebook_elems=256))
    assert "sliced" in b.LIB.vq_last_error().decode()


def test_xy_checks_and_empty(b):
    t = _t(b)
    assert b.STATUS_NAMES[_gemv(b, t, x=0)] == "VQ_ERR_NULL"
    assert b.STATUS_NAMES[_gemv(b, t, y=0)] == "VQ_ERR_NULL"
    assert b.STATUS_NAMES[_gemv(b, t, x=0x40008)] == "VQ_ERR_ALIGN"
    assert b.STATUS_NAMES[_gemv(b, t, y=0x50004)] == "VQ_ERR_ALIGN"
    assert b.STATUS_NAMES[_gemv(b, t, T=-1)] == "VQ_ERR_SHAPE"
    assert _gemv(b, t, T=0) == b.VQ_OK                    # empty batch: nothing enqueued
    assert b.LIB.vq_gemm(ctypes.byref(t), 0x40000, 0, 0x50000, None) == b.VQ_OK


def test_dequant_checks(b):
    t = _t(b)
    assert b.STATUS_NAMES[b.LIB.vq_dequant(ctypes.byref(t), 1, 0x60000, None)] == "VQ_ERR_SHAPE"
    assert b.STATUS_NAMES[b.LIB.vq_dequant(ctypes.byref(t), 0, 0, None)] == "VQ_ERR_NULL"
    assert b.STATUS_NAMES[b.LIB.vq_dequant(ctypes.byref(t), 0, 0x60008, None)] == "VQ_ERR_ALIGN"
    assert b.STATUS_NAMES[b.LIB.vq_dequant(None, 0, 0x60000, None)] == "VQ_ERR_NULL"


def test_moe_checks(b):
    t = _t(b, num_experts=4)
    L = b.LIB

    def gemv(**kw):
        a = dict(x=0x40000, xps=0, ids=0x70000, T=2, k=2, y=0x50000)
        a.update(kw)
        return b.STATUS_NAMES[L.vq_moe_gemv(ctypes.byref(t), a["x"], a["xps"], a["ids"], a["T"],
                                            a["k"], a["y"], None)]

    assert gemv(ids=0) == "VQ_ERR_NULL"
    assert gemv(ids=0x70002) == "VQ_ERR_ALIGN"
    assert gemv(k=0) == "VQ_ERR_SHAPE"
    assert gemv(xps=2) == "VQ_ERR_SHAPE"
    assert gemv(T=-3) == "VQ_ERR_SHAPE"
    assert gemv(T=0) == "VQ_OK"
    need = b.workspace_bytes(2, 2, 4)
    assert need > 0 and b.workspace_bytes(0, 2, 4) == 0

    def gemm(ws, wsb):
        return b.STATUS_NAMES[L.vq_moe_gemm(ctypes.byref(t), 0x40000, 0, 0x70000, 2, 2, 0x50000,
                                            ws, wsb, None)]

    assert gemm(0, need) == "VQ_ERR_WORKSPACE"
    assert gemm(0x80000, need - 4) == "VQ_ERR_WORKSPACE"
    assert gemm(0x80004, need) == "VQ_ERR_ALIGN"
    # per-expert codebooks need E*K*d values
    t2 = _t(b, num_experts=4, codebook_per_expert=1, codebook_elems=512)
    assert b.STATUS_NAMES[L.vq_moe_gemv(ctypes.byref(t2), 0x40000, 0, 0x70000, 1, 1, 0x50000, None)] \
        == "VQ_ERR_SHAPE"


def test_workspace_grows_with_pairs_and_experts(b):
    a = b.workspace_bytes(512, 8, 256)
    assert a < b.workspace_bytes(1024, 8, 256) and a < b.workspace_bytes(512, 8, 512)
    assert a % 4 == 0


def test_buffer_size_limits(b):
    """One expert's codes or scales above 2 GiB - 1 bytes, or an x of that
    size for a routed call, is refused: the kernels address them with 32-bit
    offsets."""
    # 2^20 rows of 4096 columns at d=2, B=8: 2048 code bytes per row = 2 GiB
    big = _t(b, rows=1 << 20, cols=4096)
    assert b.STATUS_NAMES[_gemv(b, big)] == "VQ_ERR_SHAPE"
    assert "exceed" in b.LIB.vq_last_error().decode()
    ok = _t(b, rows=(1 << 20) - 1, cols=4096)
    assert b.STATUS_NAMES[b.LIB.vq_gemv(ctypes.byref(ok), 0x40000, 0, 0x50000, None)] == "VQ_OK"
    t = _t(b, num_experts=4, cols=4096)
    st = b.LIB.vq_moe_gemv(ctypes.byref(t), 0x40000, 1, 0x70000, 1 << 16, 8, 0x50000, None)
    assert b.STATUS_NAMES[st] == "VQ_ERR_SHAPE" and "x holds" in b.LIB.vq_last_error().decode()


def test_no_alloc_refuses_sizes_beyond_its_scratch_on_the_host(b):
    """The size check runs before any device call: more routing scratch than
    the library's static 4 MiB is refused with VQ_ERR_WORKSPACE."""
    t = _t(b, num_experts=4)
    T, top_k = 1 << 17, 8
    assert b.workspace_bytes(T, top_k, 4) > 4 << 20
    st = b.LIB.vq_moe_gemm_no_alloc(ctypes.byref(t), 0x40000, 0, 0x70000, T, top_k, 0x50000, None)
    assert b.STATUS_NAMES[st] == "VQ_ERR_WORKSPACE"
    assert "static scratch" in b.LIB.vq_last_error().decode()
    assert b.LIB.vq_moe_gemm_no_alloc(ctypes.byref(t), 0x40000, 0, 0x70000, 0, top_k, 0x50000, None) == b.VQ_OK


def test_io_descriptor_checks(b):
    """vq_io is validated on the host before anything is enqueued."""
    L = b.LIB

    def dense(io, fn=L.vq_gemm_ex, **kw):
        t = _t(b, **kw)
        return b.STATUS_NAMES[fn(ctypes.byref(t), ctypes.byref(io) if io is not None else None, 0x40000, 2,
                                 0x50000, None)]

    def routed(io, fn=L.vq_moe_gemv_ex, **kw):
        t = _t(b, num_experts=4, **kw)
        if fn is L.vq_moe_gemv_ex:
            st = fn(ctypes.byref(t), ctypes.byref(io), 0x40000, 0, 0x70000, 2, 2, 0x50000, None)
        else:
            st = fn(ctypes.byref(t), ctypes.byref(io), 0x40000, 0, 0x70000, 2, 2, 0x50000, 0x80000, 1 << 20, None)
        return b.STATUS_NAMES[st]

    io = b.CIo
    assert dense(io(3, 0, 0, 0, None)) == "VQ_ERR_SHAPE"                 # x dtype
    assert dense(io(b.VQ_DTYPE_F32, 0, 0, 0, None)) == "VQ_ERR_SHAPE"    # fp32 x is not an input type
    assert dense(io(1, 5, 0, 0, None)) == "VQ_ERR_SHAPE"                 # y dtype
    assert dense(io(1, 0, 7, 0, None)) == "VQ_ERR_SHAPE"                 # epilogue
    assert dense(io(1, 0, 0, 1, None)) == "VQ_ERR_SHAPE"                 # reserved
    assert dense(io(1, 0, b.VQ_EPILOGUE_SWIGLU, 0, None), rows=15) == "VQ_ERR_SHAPE"   # odd rows
    assert "interleaved" in L.vq_last_error().decode()
    assert dense(io(1, 0, b.VQ_EPILOGUE_COMBINE, 0, 0x90000)) == "VQ_ERR_SHAPE"       # dense combine
    assert routed(io(1, 1, b.VQ_EPILOGUE_COMBINE, 0, 0x90000)) == "VQ_ERR_SHAPE"      # combine -> fp32 only
    assert routed(io(1, 0, b.VQ_EPILOGUE_COMBINE, 0, None)) == "VQ_ERR_NULL"
    assert routed(io(1, 0, b.VQ_EPILOGUE_COMBINE, 0, 0x90002)) == "VQ_ERR_ALIGN"
    # the streaming GEMV holds 20480 input features per pass: wider rows only
    # with a plain fp32 y (the GEMM takes any output type)
    wide = dict(cols=20480 + 128, codebook_elems=512)
    assert dense(io(1, b.VQ_DTYPE_BF16, 0, 0, None), fn=L.vq_gemv_ex, **wide) == "VQ_ERR_SHAPE"
    assert dense(io(1, 0, b.VQ_EPILOGUE_SWIGLU, 0, None), fn=L.vq_gemv_ex, **wide) == "VQ_ERR_SHAPE"
    # valid descriptors pass validation (T = 0 enqueues nothing)
    t = _t(b)
    for good in (io(b.VQ_DTYPE_BF16, b.VQ_DTYPE_BF16, 0, 0, None), io(1, b.VQ_DTYPE_F16, 1, 0, None), None):
        st = L.vq_gemv_ex(ctypes.byref(t), ctypes.byref(good) if good is not None else None, 0x40000, 0,
                          0x50000, None)
        assert st == b.VQ_OK, L.vq_last_error()


def test_encode_checks(b):
    L = b.LIB
    ok = dict(w=0x10000, rows=8, cols=256, d=4, k=8, g=64, idx=0x20000, ns=100, u=0x30000, it=3,
              codes=0x40000, cb=0x50000, sc=0x60000, rel=0x70000, ws=0x100000, wsb=1 << 30)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return b.STATUS_NAMES[L.vq_encode(a["w"], a["rows"], a["cols"], a["d"], a["k"], a["g"], a["idx"], a["ns"],
                                          a["u"], a["it"], a["codes"], a["cb"], a["sc"], a["rel"], a["ws"],
                                          a["wsb"], None)]

    assert call(d=3) == "VQ_ERR_GEOMETRY"
    assert call(k=15) == "VQ_ERR_GEOMETRY"
    assert call(cols=192) == "VQ_ERR_SHAPE"          # not a multiple of the group
    assert call(cols=320, g=64, d=8) == "VQ_ERR_SHAPE"   # (cols/d) % 32
    assert call(ns=0) == "VQ_ERR_SHAPE"
    assert call(it=-1) == "VQ_ERR_SHAPE"
    assert call(w=0) == "VQ_ERR_NULL"
    assert call(u=0x30004) == "VQ_ERR_ALIGN"
    assert call(codes=0x40004) == "VQ_ERR_ALIGN"
    assert call(ws=0) == "VQ_ERR_WORKSPACE"
    assert call(wsb=16) == "VQ_ERR_WORKSPACE"
    assert call(ws=0x100010) == "VQ_ERR_ALIGN"
    need = L.vq_encode_workspace_bytes(8, 256, 4, 8, 100)
    assert need >= 8 * 256 * 8 and need % 256 == 0
    assert L.vq_encode_workspace_bytes(8, 250, 4, 8, 100) == 0
