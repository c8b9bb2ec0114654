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


# Expert -> pairs of the hot experts of hot_expert_ids: whole 128-pair tiles,
# remainders just above and at 64 (65 -> a 128-token tile, 64 -> two
# 32-token ones), a wide tile plus a one-pair thin tile (129), thin only (33).
HOT_EXPERTS = {0: 1000, 1: 300, 2: 128, 3: 65, 4: 64, 5: 200, 6: 129, 7: 33}


def hot_expert_ids(T, top_k, E, key):
    """ids [T][top_k] (T >= 1000, top_k >= 8, E > 8 + top_k): token t < n
    takes hot expert e of HOT_EXPERTS in slot e; every other slot a distinct
    random expert of 8 .. E - 1; slot (900, 7) skipped (-1) and slot (901, 6)
    out of range (E + 1)."""
    from vq_dequant_matmul_gemv_amd import synth
    g = synth.rng("hot-ids", *key)
    ids = np.full((T, top_k), -1, dtype=np.int32)
    for e, n in HOT_EXPERTS.items():
        ids[:n, e] = e
    for t in range(T):
        free = ids[t] < 0
        ids[t, free] = g.permutation(np.arange(8, E))[: free.sum()]
    ids[900, 7] = -1
    ids[901, 6] = E + 1
    return ids
