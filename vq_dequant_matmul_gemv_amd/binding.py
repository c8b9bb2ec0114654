"""Thin ctypes binding over libvqmi.so (include/vq.h): argument marshalling only.

Every step of the computation runs in the library's HIP kernels; PyTorch only
provides device memory and the current stream.  There is no fallback: if the
library is missing this module raises on import.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libvqmi.so")

VQ_OK, VQ_ERR_NULL, VQ_ERR_GEOMETRY, VQ_ERR_SHAPE, VQ_ERR_ALIGN, VQ_ERR_WORKSPACE, VQ_ERR_HIP = range(7)
STATUS_NAMES = ["VQ_OK", "VQ_ERR_NULL", "VQ_ERR_GEOMETRY", "VQ_ERR_SHAPE", "VQ_ERR_ALIGN",
                "VQ_ERR_WORKSPACE", "VQ_ERR_HIP"]


class VQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES[status] if 0 <= status < 7 else status}: {message}")
        self.status = status
        self.message = message


class CTensor(ctypes.Structure):
    """Mirror of `vq_tensor`."""
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("codebook", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("rows", ctypes.c_int32),
        ("cols", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("log2_k", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("codebook_per_expert", ctypes.c_int32),
        ("codebook_elems", ctypes.c_int64),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m vq_dequant_matmul_gemv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    T = ctypes.POINTER(CTensor)
    sig = {
        "vq_words_per_row": (i32, [i32, i32, i32]),
        "vq_dequant": (i32, [T, i32, P, P]),
        "vq_gemv": (i32, [T, P, i32, P, P]),
        "vq_gemm": (i32, [T, P, i32, P, P]),
        "vq_moe_gemv": (i32, [T, P, i32, P, i32, i32, P, P]),
        "vq_moe_workspace_bytes": (ctypes.c_size_t, [i32, i32, i32]),
        "vq_moe_gemm": (i32, [T, P, i32, P, i32, i32, P, P, ctypes.c_size_t, P]),
        "vq_last_error": (ctypes.c_char_p, []),
        "vq_status_name": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = _load()

EXPORTED = ("vq_words_per_row", "vq_dequant", "vq_gemv", "vq_gemm", "vq_moe_gemv",
            "vq_moe_workspace_bytes", "vq_moe_gemm", "vq_last_error", "vq_status_name")


def check(status: int) -> None:
    if status != VQ_OK:
        raise VQError(status, LIB.vq_last_error().decode())


def words_per_row(cols: int, d: int, log2_k: int) -> int:
    return LIB.vq_words_per_row(cols, d, log2_k)


def workspace_bytes(T: int, top_k: int, num_experts: int) -> int:
    return LIB.vq_moe_workspace_bytes(T, top_k, num_experts)


# --------------------------------------------------------------------------
# torch-facing wrappers
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _dev_check(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


@dataclass
class VQTensor:
    """Device-resident VQ tensor (see `vq_tensor` in include/vq.h).

    codes    int32/uint32 [E][rows][Wr] (or [rows][Wr]) packed code words
    codebook fp16 [K][d] or [E][K][d]
    scales   fp16 [E][rows][cols/group] (or [rows][cols/group])
    """
    codes: object
    codebook: object
    scales: object
    rows: int
    cols: int
    d: int
    log2_k: int
    group: int
    num_experts: int = 1
    codebook_per_expert: bool = False

    def cstruct(self) -> CTensor:
        _dev_check(self.codes, self.codebook, self.scales)
        return CTensor(self.codes.data_ptr(), self.codebook.data_ptr(), self.scales.data_ptr(),
                       self.rows, self.cols, self.d, self.log2_k, self.group, self.num_experts,
                       int(self.codebook_per_expert), self.codebook.numel())

    @classmethod
    def from_host(cls, arrays: dict, spec, device="cuda", codebook_per_expert=False):
        """Copy numpy arrays (codes/codebook/scales as produced by synth.tensor)
        to the device."""
        import numpy as np
        torch = _torch()
        codes = torch.from_numpy(np.ascontiguousarray(arrays["codes"]).view(np.int32)).to(device)
        cb = torch.from_numpy(np.ascontiguousarray(arrays["codebook"])).to(device)
        sc = torch.from_numpy(np.ascontiguousarray(arrays["scales"])).to(device)
        return cls(codes, cb, sc, spec.rows, spec.cols, spec.d, spec.log2_k, spec.group,
                   spec.experts, codebook_per_expert)


def dequant(w: VQTensor, expert: int = 0, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty((w.rows, w.cols), dtype=torch.float16, device=w.codes.device)
    _dev_check(out)
    cs = w.cstruct()
    check(LIB.vq_dequant(ctypes.byref(cs), expert, _ptr(out), _stream(stream)))
    return out


def _dense(fn, w: VQTensor, x, y, stream):
    torch = _torch()
    if x.dtype != torch.float16 or x.dim() != 2 or x.shape[1] != w.cols:
        raise ValueError("x must be fp16 [T][cols]")
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, w.rows), dtype=torch.float32, device=x.device)
    _dev_check(x, y)
    cs = w.cstruct()
    check(fn(ctypes.byref(cs), _ptr(x), T, _ptr(y), _stream(stream)))
    return y


def gemv(w: VQTensor, x, y=None, stream=None):
    """y[T][rows] = x W^T through vq_gemv."""
    return _dense(LIB.vq_gemv, w, x, y, stream)


def gemm(w: VQTensor, x, y=None, stream=None):
    """y[T][rows] = x W^T through vq_gemm (MFMA)."""
    return _dense(LIB.vq_gemm, w, x, y, stream)


def _moe_prep(w, x, ids, x_per_slot, y):
    torch = _torch()
    T, top_k = ids.shape
    if ids.dtype != torch.int32:
        raise ValueError("expert ids must be int32 [T][top_k]")
    want = (T, top_k, w.cols) if x_per_slot else (T, w.cols)
    if x.dtype != torch.float16 or tuple(x.shape) != want:
        raise ValueError(f"x must be fp16 {want}")
    if y is None:
        y = torch.empty((T, top_k, w.rows), dtype=torch.float32, device=x.device)
    _dev_check(x, ids, y)
    return T, top_k, y


def moe_gemv(w: VQTensor, x, ids, x_per_slot=False, y=None, stream=None):
    T, top_k, y = _moe_prep(w, x, ids, x_per_slot, y)
    cs = w.cstruct()
    check(LIB.vq_moe_gemv(ctypes.byref(cs), _ptr(x), int(bool(x_per_slot)), _ptr(ids), T, top_k,
                          _ptr(y), _stream(stream)))
    return y


def moe_gemm(w: VQTensor, x, ids, x_per_slot=False, y=None, workspace=None, stream=None):
    torch = _torch()
    T, top_k, y = _moe_prep(w, x, ids, x_per_slot, y)
    need = workspace_bytes(T, top_k, w.num_experts)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    cs = w.cstruct()
    check(LIB.vq_moe_gemm(ctypes.byref(cs), _ptr(x), int(bool(x_per_slot)), _ptr(ids), T, top_k,
                          _ptr(y), _ptr(workspace), workspace.numel(), _stream(stream)))
    return y
