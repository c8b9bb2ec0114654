"""Shared test helpers: device upload and the output error metric."""
import sys

import numpy as np

TOL = 1e-3   # max relative error per token row (fp32 accumulation)


def row_rel_err(y, ref):
    """max over output rows of |y - ref| divided by max |ref|, per token row;
    returns the worst token row.  y, ref: [..., rows]."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(y - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if num.size else 0.0


def announce(*parts):
    """Name the case before a GPU step (flushed, so a crash still names it)."""
    print("CASE", *parts, flush=True)
    sys.stdout.flush()


def upload(arrs, spec, codebook_per_expert=False):
    from vq_dequant_matmul_gemv_amd import binding
    return binding.VQTensor.from_host(arrs, spec, codebook_per_expert=codebook_per_expert)


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()
