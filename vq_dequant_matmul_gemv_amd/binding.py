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


VQ_DTYPE_F32, VQ_DTYPE_F16, VQ_DTYPE_BF16 = 0, 1, 2
VQ_EPILOGUE_NONE, VQ_EPILOGUE_SWIGLU, VQ_EPILOGUE_COMBINE = 0, 1, 2
EPILOGUES = {None: VQ_EPILOGUE_NONE, "none": VQ_EPILOGUE_NONE, "swiglu": VQ_EPILOGUE_SWIGLU,
             "combine": VQ_EPILOGUE_COMBINE}


class CIo(ctypes.Structure):
    """Mirror of `vq_io`."""
    _fields_ = [
        ("x_dtype", ctypes.c_int32),
        ("y_dtype", ctypes.c_int32),
        ("epilogue", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("route_weights", ctypes.c_void_p),
    ]


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
        ("code_words", ctypes.c_int64),
        ("scale_elems", ctypes.c_int64),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m vq_dequant_matmul_gemv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    T = ctypes.POINTER(CTensor)
    IO = ctypes.POINTER(CIo)
    sig = {
        "vq_gemv_ex": (i32, [T, IO, P, i32, P, P]),
        "vq_gemm_ex": (i32, [T, IO, P, i32, P, P]),
        "vq_moe_gemv_ex": (i32, [T, IO, P, i32, P, i32, i32, P, P]),
        "vq_moe_gemm_ex": (i32, [T, IO, P, i32, P, i32, i32, P, P, ctypes.c_size_t, P]),
        "vq_words_per_row": (i32, [i32, i32, i32]),
        "vq_dequant": (i32, [T, i32, P, P]),
        "vq_gemv": (i32, [T, P, i32, P, P]),
        "vq_gemm": (i32, [T, P, i32, P, P]),
        "vq_moe_gemv": (i32, [T, P, i32, P, i32, i32, P, P]),
        "vq_moe_workspace_bytes": (ctypes.c_size_t, [i32, i32, i32]),
        "vq_moe_gemm": (i32, [T, P, i32, P, i32, i32, P, P, ctypes.c_size_t, P]),
        "vq_moe_gemm_no_alloc": (i32, [T, P, i32, P, i32, i32, P, P]),
        "vq_encode_workspace_bytes": (ctypes.c_size_t, [i32, i32, i32, i32, i32]),
        "vq_encode": (i32, [P, i32, i32, i32, i32, i32, P, i32, P, i32, P, P, P, P, P, ctypes.c_size_t, P]),
        "vq_last_error": (ctypes.c_char_p, []),
        "vq_status_name": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = _load()

EXPORTED = ("vq_words_per_row", "vq_dequant", "vq_gemv", "vq_gemm", "vq_moe_gemv", "vq_gemv_ex",
            "vq_gemm_ex", "vq_moe_gemv_ex", "vq_moe_gemm_ex",
            "vq_moe_workspace_bytes", "vq_moe_gemm", "vq_moe_gemm_no_alloc", "vq_encode_workspace_bytes",
            "vq_encode", "vq_last_error", "vq_status_name")


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


def _dev_check(*ts, device=None):
    """Every tensor on the GPU (on `device` when given), contiguous."""
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if device is not None and t.device != device:
            raise ValueError(f"tensor on {t.device}, expected {device} (the weights' device)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _check_out(y, dtype, shape, name="y"):
    torch = _torch()
    if y.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {y.dtype}")
    if tuple(y.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(y.shape)}")
    del torch


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

    @property
    def device(self):
        return self.codes.device

    def cstruct(self) -> CTensor:
        """The C descriptor; buffer lengths travel with it so the library
        refuses codes, scales or a codebook of the wrong size."""
        torch = _torch()
        _dev_check(self.codes, self.codebook, self.scales, device=self.codes.device)
        if self.codebook.dtype != torch.float16 or self.scales.dtype != torch.float16:
            raise ValueError("codebook and scales must be fp16")
        if self.codes.element_size() * self.codes.numel() % 4:
            raise ValueError("codes must hold whole uint32 words")
        return CTensor(self.codes.data_ptr(), self.codebook.data_ptr(), self.scales.data_ptr(),
                       self.rows, self.cols, self.d, self.log2_k, self.group, self.num_experts,
                       int(self.codebook_per_expert), self.codebook.numel(),
                       self.codes.numel() * self.codes.element_size() // 4, self.scales.numel())

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
    _check_out(out, torch.float16, (w.rows, w.cols), "out")
    _dev_check(out, device=w.device)
    cs = w.cstruct()
    check(LIB.vq_dequant(ctypes.byref(cs), expert, _ptr(out), _stream(stream)))
    return out


def _dtype_code(dt):
    torch = _torch()
    codes = {torch.float32: VQ_DTYPE_F32, torch.float16: VQ_DTYPE_F16, torch.bfloat16: VQ_DTYPE_BF16}
    if dt not in codes:
        raise ValueError(f"unsupported dtype {dt}")
    return codes[dt]


def _io(x, y_dtype, epilogue, route_weights):
    """The vq_io of a call, or None for the plain call (fp16 x, fp32 y)."""
    torch = _torch()
    if epilogue not in EPILOGUES:
        raise ValueError(f"epilogue must be one of {sorted(k for k in EPILOGUES if k)}")
    epi = EPILOGUES[epilogue]
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("x must be fp16 or bf16")
    if x.dtype == torch.float16 and y_dtype == torch.float32 and epi == VQ_EPILOGUE_NONE:
        return None
    rw = 0
    if epi == VQ_EPILOGUE_COMBINE:
        if route_weights is None or route_weights.dtype != torch.float32:
            raise ValueError("the combine needs fp32 route_weights [T][top_k]")
        rw = route_weights.data_ptr()
    return CIo(_dtype_code(x.dtype), _dtype_code(y_dtype), epi, 0, rw)


def _dense(fn, fn_ex, w: VQTensor, x, y, stream, y_dtype=None, epilogue=None):
    torch = _torch()
    if x.dtype not in (torch.float16, torch.bfloat16) or x.dim() != 2 or x.shape[1] != w.cols:
        raise ValueError("x must be fp16 or bf16 [T][cols]")
    T = x.shape[0]
    y_dtype = y.dtype if (y is not None and y_dtype is None) else (y_dtype or torch.float32)
    ycols = w.rows // 2 if epilogue == "swiglu" else w.rows
    if epilogue == "combine":
        raise ValueError("the combine applies to routed calls only")
    # a stack of experts (vq_gemm only): y[t][e] = W_e x[t]
    yshape = (T, ycols) if w.num_experts == 1 else (T, w.num_experts, ycols)
    if y is None:
        y = torch.empty(yshape, dtype=y_dtype, device=x.device)
    _check_out(y, y_dtype, yshape)
    _dev_check(x, y, device=w.device)
    cs = w.cstruct()
    io = _io(x, y_dtype, epilogue, None)
    if io is None:
        check(fn(ctypes.byref(cs), _ptr(x), T, _ptr(y), _stream(stream)))
    else:
        check(fn_ex(ctypes.byref(cs), ctypes.byref(io), _ptr(x), T, _ptr(y), _stream(stream)))
    return y


def gemv(w: VQTensor, x, y=None, stream=None, y_dtype=None, epilogue=None):
    """y = x W^T through vq_gemv (vq_gemv_ex for bf16 x, a non-fp32 y or an
    epilogue: "swiglu" on interleaved gate/up rows gives silu(gate) * up).
    On a stack of E experts, y is [T][E][rows]: every expert times the same x."""
    return _dense(LIB.vq_gemv, LIB.vq_gemv_ex, w, x, y, stream, y_dtype, epilogue)


def gemm(w: VQTensor, x, y=None, stream=None, y_dtype=None, epilogue=None):
    """y = x W^T through vq_gemm (MFMA); options as for gemv.  On a stack of
    E experts, y is [T][E][rows]: every expert times the same x."""
    return _dense(LIB.vq_gemm, LIB.vq_gemm_ex, w, x, y, stream, y_dtype, epilogue)


def _moe_prep(w, x, ids, x_per_slot, y, y_dtype=None, epilogue=None):
    torch = _torch()
    T, top_k = ids.shape
    if ids.dtype != torch.int32:
        raise ValueError("expert ids must be int32 [T][top_k]")
    want = (T, top_k, w.cols) if x_per_slot else (T, w.cols)
    if x.dtype not in (torch.float16, torch.bfloat16) or tuple(x.shape) != want:
        raise ValueError(f"x must be fp16 or bf16 {want}")
    y_dtype = y.dtype if (y is not None and y_dtype is None) else (y_dtype or torch.float32)
    if epilogue == "combine":
        yshape = (T, w.rows)
    else:
        yshape = (T, top_k, w.rows // 2 if epilogue == "swiglu" else w.rows)
    if y is None:
        y = torch.empty(yshape, dtype=y_dtype, device=x.device)
    _check_out(y, y_dtype, yshape)
    _dev_check(x, ids, y, device=w.device)
    return T, top_k, y, y_dtype


def moe_gemv(w: VQTensor, x, ids, x_per_slot=False, y=None, stream=None, y_dtype=None, epilogue=None,
             route_weights=None):
    """Routed experts, decode-shaped (vq_moe_gemv / vq_moe_gemv_ex).  epilogue
    "combine" with fp32 route_weights [T][top_k] gives y [T][rows] = the
    router-weighted sum over each token's slots."""
    T, top_k, y, y_dtype = _moe_prep(w, x, ids, x_per_slot, y, y_dtype, epilogue)
    if route_weights is not None:
        _dev_check(route_weights, device=w.device)
    cs = w.cstruct()
    io = _io(x, y_dtype, epilogue, route_weights)
    if io is None:
        check(LIB.vq_moe_gemv(ctypes.byref(cs), _ptr(x), int(bool(x_per_slot)), _ptr(ids), T, top_k,
                              _ptr(y), _stream(stream)))
    else:
        check(LIB.vq_moe_gemv_ex(ctypes.byref(cs), ctypes.byref(io), _ptr(x), int(bool(x_per_slot)), _ptr(ids),
                                 T, top_k, _ptr(y), _stream(stream)))
    return y


def moe_gemm(w: VQTensor, x, ids, x_per_slot=False, y=None, workspace=None, stream=None, y_dtype=None,
             epilogue=None, route_weights=None):
    """Routed experts, prefill-shaped (vq_moe_gemm / vq_moe_gemm_ex); options
    as for moe_gemv."""
    torch = _torch()
    T, top_k, y, y_dtype = _moe_prep(w, x, ids, x_per_slot, y, y_dtype, epilogue)
    if route_weights is not None:
        _dev_check(route_weights, device=w.device)
    need = workspace_bytes(T, top_k, w.num_experts)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _dev_check(workspace, device=w.device)
    cs = w.cstruct()
    io = _io(x, y_dtype, epilogue, route_weights)
    if io is None:
        check(LIB.vq_moe_gemm(ctypes.byref(cs), _ptr(x), int(bool(x_per_slot)), _ptr(ids), T, top_k,
                              _ptr(y), _ptr(workspace), workspace.numel(), _stream(stream)))
    else:
        check(LIB.vq_moe_gemm_ex(ctypes.byref(cs), ctypes.byref(io), _ptr(x), int(bool(x_per_slot)), _ptr(ids),
                                 T, top_k, _ptr(y), _ptr(workspace), workspace.numel(), _stream(stream)))
    return y


def moe_gemm_no_alloc(w: VQTensor, x, ids, x_per_slot=False, y=None, stream=None):
    """vq_moe_gemm_no_alloc: vq_moe_gemm with the library's static scratch
    instead of a workspace (allocates nothing when y is given)."""
    T, top_k, y, _ = _moe_prep(w, x, ids, x_per_slot, y)
    cs = w.cstruct()
    check(LIB.vq_moe_gemm_no_alloc(ctypes.byref(cs), _ptr(x), int(bool(x_per_slot)), _ptr(ids), T, top_k,
                                   _ptr(y), _stream(stream)))
    return y


def encode(w, d: int, log2_k: int, group: int, sample_idx, uniforms, iters: int, workspace=None, stream=None):
    """vq_encode: fit a VQ tensor to fp32 weights w [rows][cols] on the GPU.
    sample_idx: int32 [n_sample] subvector indices for k-means++; uniforms:
    fp64 [K] draws.  Returns (VQTensor, relerr as a 0-d fp64 device tensor)."""
    torch = _torch()
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be fp32 [rows][cols]")
    if sample_idx.dtype != torch.int32 or uniforms.dtype != torch.float64:
        raise ValueError("sample_idx must be int32 and uniforms fp64")
    rows, cols = w.shape
    K = 1 << log2_k
    if uniforms.numel() != K:
        raise ValueError(f"uniforms must hold K = {K} values")
    dev = w.device
    _dev_check(w, sample_idx, uniforms, device=dev)
    wr = words_per_row(cols, d, log2_k)
    if wr < 0:
        raise ValueError("unsupported geometry")
    codes = torch.empty((rows, wr), dtype=torch.int32, device=dev)
    codebook = torch.empty((K, d), dtype=torch.float16, device=dev)
    scales = torch.empty((rows, cols // group), dtype=torch.float16, device=dev)
    relerr = torch.empty((), dtype=torch.float64, device=dev)
    need = LIB.vq_encode_workspace_bytes(rows, cols, d, log2_k, sample_idx.numel())
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _dev_check(workspace, device=dev)
    check(LIB.vq_encode(_ptr(w), rows, cols, d, log2_k, group, _ptr(sample_idx), sample_idx.numel(), _ptr(uniforms),
                        iters, _ptr(codes), _ptr(codebook), _ptr(scales), _ptr(relerr), _ptr(workspace),
                        workspace.numel(), _stream(stream)))
    return VQTensor(codes, codebook, scales, rows, cols, d, log2_k, group), relerr
