"""Fused vector-quantized (VQ) weight matmul for AMD MI355X (gfx950).

The compute lives in libvqmi.so (hand-written HIP kernels behind the C ABI in
include/vq.h); `binding` is a thin ctypes layer over it and `synth` makes
seeded synthetic inputs.  Importing the package does not load the library;
the first use of a binding name does, and fails loudly if it is not built.
"""

_BINDING_NAMES = {"VQTensor", "VQError", "dequant", "gemv", "gemm", "moe_gemv", "moe_gemm",
                  "words_per_row", "workspace_bytes"}

__all__ = sorted(_BINDING_NAMES | {"synth", "binding"})


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
