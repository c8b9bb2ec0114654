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
    assert b.words_per_row(64, 2, 10) == -1


def _t(b, **kw):
    base = dict(codes=0x10000, codebook=0x20000, scales=0x30000, rows=16, cols=256, d=2,
                log2_k=8, group=64, num_experts=1, codebook_per_expert=0, codebook_elems=512)
    base.update(kw)
    return b.CTensor(**base)


def _gemv(b, t, x=0x40000, T=1, y=0x50000):
    return b.LIB.vq_gemv(ctypes.byref(t), x, T, y, None)


@pytest.mark.parametrize("kw,status", [
    (dict(codes=0), "VQ_ERR_NULL"),
    (dict(scales=0), "VQ_ERR_NULL"),
    (dict(d=3), "VQ_ERR_GEOMETRY"),
    (dict(log2_k=10), "VQ_ERR_GEOMETRY"),
    (dict(group=32), "VQ_ERR_GEOMETRY"),
    (dict(rows=0), "VQ_ERR_SHAPE"),
    (dict(cols=320, group=128), "VQ_ERR_SHAPE"),          # cols % group
    (dict(cols=192, d=4, codebook_elems=1024), "VQ_ERR_SHAPE"),   # (cols/d) % 32
    (dict(codebook_elems=256), "VQ_ERR_SHAPE"),          # sliced codebook fails loudly
    (dict(codebook_elems=1024), "VQ_ERR_SHAPE"),
    (dict(num_experts=2), "VQ_ERR_SHAPE"),               # dense entry point, stacked tensor
    (dict(codebook_per_expert=2), "VQ_ERR_SHAPE"),
    (dict(codes=0x10004), "VQ_ERR_ALIGN"),
    (dict(codebook=0x20008), "VQ_ERR_ALIGN"),
    (dict(scales=0x30002), "VQ_ERR_ALIGN"),
])
def test_gemv_rejects(b, kw, status):
    st = _gemv(b, _t(b, **kw))
    assert b.STATUS_NAMES[st] == status, b.LIB.vq_last_error()
    assert b.LIB.vq_last_error()
    assert b.LIB.vq_status_name(st).decode() == status


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
