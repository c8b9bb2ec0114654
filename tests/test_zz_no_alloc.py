"""vq_moe_gemm_no_alloc (the routed GEMM on the library's static scratch)
against vq_moe_gemm (caller's workspace), through the C ABI: bit for bit on
two calls in a row, the second with a smaller input, so the second call runs
on scratch the first one left behind."""
import ctypes

import numpy as np
import pytest

from vq_dequant_matmul_gemv_amd import synth
from tests.helpers import announce, to_dev, upload

pytestmark = pytest.mark.gpu


def _call_no_alloc(binding, w, x, ids, x_per_slot, y):
    import torch
    cs = w.cstruct()
    T, top_k = ids.shape
    st = binding.LIB.vq_moe_gemm_no_alloc(ctypes.byref(cs), ctypes.c_void_p(x.data_ptr()), int(x_per_slot),
                                          ctypes.c_void_p(ids.data_ptr()), T, top_k,
                                          ctypes.c_void_p(y.data_ptr()),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    binding.check(st)
    return y


@pytest.mark.parametrize("d,b,g,x_per_slot", [(4, 8, 64, False), (8, 12, 128, True)])
def test_no_alloc_matches_workspace_call_twice(d, b, g, x_per_slot):
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, top_k = 64, 160, 512, 8
    spec = synth.Spec(rows=rows, cols=cols, d=d, log2_k=b, group=g, experts=E)
    w = upload(synth.tensor(spec, "no-alloc", d, b, g), spec)
    for T in (300, 37):                     # second call smaller than the first
        ids = synth.zipf_routing(T, E, top_k, "no-alloc", d, T)
        ids[3, 2] = -1                      # a skipped slot
        shape = (T, top_k, cols) if x_per_slot else (T, cols)
        x = to_dev(synth.activations(shape, "no-alloc", d, b, g, T))
        idd = to_dev(ids)
        announce("moe_gemm_no_alloc", d, b, g, "T", T)
        ref = binding.moe_gemm(w, x, idd, x_per_slot=x_per_slot)
        y = torch.full((T, top_k, rows), float("nan"), device="cuda")
        _call_no_alloc(binding, w, x, idd, x_per_slot, y)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32)), T
        assert torch.count_nonzero(y[3, 2]).item() == 0


def test_no_alloc_refuses_more_than_its_scratch():
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    spec = synth.Spec(rows=32, cols=64, d=2, log2_k=8, group=64, experts=4)
    w = upload(synth.tensor(spec, "no-alloc-big"), spec)
    T, top_k = 1 << 17, 8                    # ~4.5 MiB of routing scratch
    x = torch.zeros((T, 64), dtype=torch.float16, device="cuda")
    ids = torch.zeros((T, top_k), dtype=torch.int32, device="cuda")
    y = torch.zeros((T, top_k, 32), device="cuda")
    announce("moe_gemm_no_alloc refuses", T)
    with pytest.raises(binding.VQError, match="static scratch"):
        _call_no_alloc(binding, w, x, ids, False, y)
