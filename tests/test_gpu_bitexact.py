"""Bit-exactness of the dequantized weights inside the MFMA path, and
run-to-run determinism.

With a one-hot activation row x = e_c every output is a single product,
y[t][r] = W[r][c] * 1.0, accumulated in fp32 next to zeros, so it is exact:
the GEMM's output must equal the oracle's fp16 dequant of column c bit for bit,
up to the sign of a zero weight (IEEE addition gives -0 + +0 = +0) (the
textbook gather; paper "Data-Free Vector Quantization Beats Affine
Quantization at Matched Bytes Below 5 Bits", §3.4: kernels are accepted on
bit identity with a reference path).  This checks the fp16 rounding of
codebook entry x scale that the GEMM does in its own registers (not the
separate dequant kernel), on general codebooks (N(0, 0.02), subnormals
included) and scales (U[0.5, 1.5]), through both tile shapes, K-split tiles
(whose slices add into y atomically: every slice but one adds zeros) and the
routed grouped GEMM.
"""
import numpy as np
import pytest

from oracle import vq_oracle as O
from vq_dequant_matmul_gemv_amd import synth
from tests.helpers import announce, to_dev, upload

pytestmark = pytest.mark.gpu

GEOMS = [(d, b, g) for d in (2, 4, 8) for b in (8, 12) for g in (64, 128)]


def _cols_for(d, g, blocks):
    cols = 32 * d * blocks
    while cols % g:
        cols += 32 * d
    return cols


def _one_hot(T, cols, columns):
    x = np.zeros((T, cols), dtype=np.float16)
    x[np.arange(T), columns] = 1.0
    return x


def _dense(d, b, g, rows, cols, key):
    spec = synth.Spec(rows=rows, cols=cols, d=d, log2_k=b, group=g)
    arrs = synth.tensor(spec, *key)
    wdq = O.dequant(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], cols, d, b, g)
    return spec, arrs, upload(arrs, spec), wdq


def same_bits_up_to_zero_sign(y, want):
    """Bit-for-bit equality, except that a zero weight may come out as +0:
    the fp32 sum of a -0 product and +0 products is +0, and both zeros are
    the one correct value."""
    zero = want == 0
    return (y.view(np.uint32) == want.view(np.uint32)) | (zero & (y == 0))


def _assert_columns(y, wdq, columns):
    """y[t] must be column columns[t] of the dequantized W, bit for bit (up
    to the sign of a zero)."""
    want = wdq[:, columns].T.astype(np.float32)
    assert y.dtype == np.float32
    bad = np.nonzero(~same_bits_up_to_zero_sign(y, want))
    assert bad[0].size == 0, (f"{bad[0].size} outputs differ, first at token {bad[0][0]} row {bad[1][0]}: "
                              f"{y[bad[0][0], bad[1][0]]!r} vs {want[bad[0][0], bad[1][0]]!r}")


@pytest.mark.parametrize("d,b,g", GEOMS)
def test_gemm_one_hot_rows_give_the_dequantized_columns(d, b, g, monkeypatch):
    """x = identity (T = cols) on 128-token tiles (forced: at this size the
    time model takes 32-token ones) and on the tiles the model picks, and a
    32-row one-hot slice spread over the row (32-token tiles)."""
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols = 301, _cols_for(d, g, 6)
    spec, arrs, w, wdq = _dense(d, b, g, rows, cols, ("onehot", d, b, g))
    assert np.any((np.abs(wdq.astype(np.float32)) < 2.0 ** -14) & (wdq != 0)), "no subnormal weight drawn"
    for columns, tile in ((np.arange(cols), "128"), (np.arange(cols), None),
                          ((np.arange(32) * (cols // 32) + np.arange(32) % 7) % cols, None)):
        if tile:
            monkeypatch.setenv("VQMI_GEMM_TILE", tile)
        else:
            monkeypatch.delenv("VQMI_GEMM_TILE", raising=False)
        T = len(columns)
        x = _one_hot(T, cols, columns)
        announce("gemm one-hot", d, b, g, rows, cols, T, tile)
        y = binding.gemm(w, to_dev(x)).cpu().numpy()
        _assert_columns(y, wdq, columns)


@pytest.mark.parametrize("d,b,g", [(2, 8, 64), (4, 12, 128), (8, 12, 64), (4, 8, 64)])
def test_gemm_one_hot_split_k_tiles(d, b, g, monkeypatch):
    """2048 columns and too few tiles to fill the GPU: the tiles are split
    along K and their slices added atomically into a zeroed y (32-token
    tiles, and 128-token ones forced)."""
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols = 700, 2048
    spec, arrs, w, wdq = _dense(d, b, g, rows, cols, ("onehot-split", d, b, g))
    rng = synth.rng("onehot-split-cols", d, b, g)
    for T, tile in ((8, None), (200, None), (200, "128")):
        if tile:
            monkeypatch.setenv("VQMI_GEMM_TILE", tile)
        else:
            monkeypatch.delenv("VQMI_GEMM_TILE", raising=False)
        columns = rng.integers(0, cols, size=T)
        x = _one_hot(T, cols, columns)
        announce("gemm one-hot split-K", d, b, g, rows, cols, T, tile)
        y = binding.gemm(w, to_dev(x)).cpu().numpy()
        _assert_columns(y, wdq, columns)


@pytest.mark.parametrize("d,b,g", [(4, 8, 64), (8, 12, 128), (2, 8, 64), (4, 12, 128)])
def test_moe_gemm_one_hot_rows_per_pair(d, b, g):
    """Routed grouped GEMM with a per-slot one-hot x: y[t][s] is column
    c(t, s) of expert ids[t][s]'s dequantized W; skipped slots are zero."""
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, top_k, T = 6, 96, _cols_for(d, g, 4), 3, 90
    spec = synth.Spec(rows=rows, cols=cols, d=d, log2_k=b, group=g, experts=E)
    arrs = synth.tensor(spec, "onehot-moe", d, b, g)
    w = upload(arrs, spec)
    rng = synth.rng("onehot-moe-ids", d, b, g)
    ids = rng.integers(0, E, size=(T, top_k)).astype(np.int32)
    ids[5, 1] = -1
    columns = rng.integers(0, cols, size=(T, top_k))
    x = np.zeros((T, top_k, cols), dtype=np.float16)
    tt, ss = np.meshgrid(np.arange(T), np.arange(top_k), indexing="ij")
    x[tt, ss, columns] = 1.0
    announce("moe_gemm one-hot", d, b, g)
    y = binding.moe_gemm(w, to_dev(x), to_dev(ids), x_per_slot=True).cpu().numpy()
    for e in range(E):
        wdq = O.dequant(arrs["codes"][e], arrs["codebook"], arrs["scales"][e], cols, d, b, g)
        t_e, s_e = np.nonzero(ids == e)
        want = wdq[:, columns[t_e, s_e]].T.astype(np.float32)
        assert np.all(same_bits_up_to_zero_sign(y[t_e, s_e], want)), e
    assert np.all(y[5, 1] == 0)


def test_repeat_runs_bit_identical_dense():
    """The streaming GEMV (row pieces added in pass order) and GEMM tiles that
    are not split along K (one writer per output) are deterministic: three
    runs give the same bits."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    for (rows, cols, d, b, g, fn, T) in ((17408, 5120, 2, 8, 64, "gemv", 1),
                                         (5120, 17408, 4, 8, 64, "gemv", 1),
                                         (4096, 768, 2, 8, 64, "gemm", 300),    # < 1024 columns: never split
                                         (2048, 512, 8, 12, 128, "gemm", 20)):
        spec = synth.Spec(rows=rows, cols=cols, d=d, log2_k=b, group=g)
        w = upload(synth.tensor(spec, "repeat", rows, cols), spec)
        x = to_dev(synth.activations((T, cols), "repeat", rows, cols))
        announce("repeat", fn, rows, cols, T)
        outs = []
        for _ in range(3):
            y = torch.full((T, rows), float("nan"), device="cuda")
            getattr(binding, fn)(w, x, y)
            outs.append(y.cpu().numpy().view(np.uint32))
        assert all(np.array_equal(outs[0], o) for o in outs[1:]), (fn, rows, cols)
