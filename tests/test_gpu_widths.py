"""GPU parity for the code widths besides 8 and 12 bits: B = log2 K from 4 to
14 (K = 16 ... 16384; the paper's builds range from d2/K16 to d4/K16384, §1
Notation, and the published ones include d2/K512, d4/K2048 and d8/K16384).

Odd widths put every other 16-code chunk half a word into its first word, and
a lane's run of codes in the GEMM can start anywhere in a word; the cases
below cover several chunks per row, several passes per row, K slices that
start mid-row and ragged rows and tokens.  Codebooks above 64 KiB (d4/K16384,
d8/K8192, d8/K16384) are read from device memory instead of LDS."""
import numpy as np
import pytest

from oracle import vq_oracle as O
from vq_dequant_matmul_gemv_amd import synth
from tests.helpers import TOL, announce, row_rel_err, to_dev, upload
from tests.test_gpu_bitexact import same_bits_up_to_zero_sign

pytestmark = pytest.mark.gpu

WIDTHS = [4, 5, 6, 7, 9, 10, 11, 13, 14]
GEOMS = [(d, b, g) for d in (2, 4, 8) for b in WIDTHS for g in (64, 128)]
LARGE_CB = [(4, 14, 64), (8, 13, 128), (8, 14, 64)]     # codebooks of 128, 128 and 256 KiB


def _cols_for(d, g, blocks):
    cols = 32 * d * blocks
    while cols % g:
        cols += 32 * d
    return cols


def _case(d, b, g, rows, cols, key, experts=1):
    spec = synth.Spec(rows=rows, cols=cols, d=d, log2_k=b, group=g, experts=experts)
    arrs = synth.tensor(spec, *key)
    return spec, arrs, upload(arrs, spec)


@pytest.mark.parametrize("d,b,g", GEOMS)
def test_dequant_bit_exact_other_widths(d, b, g):
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols = 37, _cols_for(d, g, 5)
    announce("dequant width", d, b, g)
    spec, arrs, w = _case(d, b, g, rows, cols, ("w-dq", d, b, g))
    got = binding.dequant(w).cpu().numpy().view(np.uint16)
    want = O.dequant(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], cols, d, b, g).view(np.uint16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("d,b,g", GEOMS)
def test_dense_other_widths(d, b, g):
    """GEMV (T = 1) and GEMM (T = 1, 3, 40: both tile shapes) against the
    oracle; then a one-hot x through the GEMM gives the dequantized columns
    bit for bit."""
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols = 301, _cols_for(d, g, 7)
    spec, arrs, w = _case(d, b, g, rows, cols, ("w-dense", d, b, g))
    for fn, Ts in (("gemv", (1, 2)), ("gemm", (1, 3, 40))):
        for T in Ts:
            x = synth.activations((T, cols), "w-dense", d, b, g, T)
            announce(fn, "width", d, b, g, T)
            y = getattr(binding, fn)(w, to_dev(x)).cpu().numpy()
            ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, cols, d, b, g)
            assert row_rel_err(y, ref) <= TOL, (fn, T)
    wdq = O.dequant(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], cols, d, b, g)
    x = np.eye(cols, dtype=np.float16)
    announce("gemm one-hot width", d, b, g)
    y = binding.gemm(w, to_dev(x)).cpu().numpy()
    assert np.all(same_bits_up_to_zero_sign(y, wdq.T.astype(np.float32)))


@pytest.mark.parametrize("d,b,g", [(2, 9, 64), (4, 11, 64), (8, 13, 128), (2, 14, 128), (4, 5, 64), (8, 14, 64)])
def test_long_rows_passes_and_k_slices(d, b, g):
    """Rows of 272 chunks or more: several GEMV passes, whose widths may be
    odd (chunk parity changes from pass to pass), and GEMM K slices that
    start mid-row (a few row tiles at T = 8 and 200)."""
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols = 203, _cols_for(d, g, 17408 // (32 * d))
    spec, arrs, w = _case(d, b, g, rows, cols, ("w-long", d, b, g))
    for fn, T in (("gemv", 1), ("gemm", 8), ("gemm", 200)):
        x = synth.activations((T, cols), "w-long", d, b, g, T)
        announce(fn, "long width", d, b, g, cols, T)
        y = getattr(binding, fn)(w, to_dev(x)).cpu().numpy()
        ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, cols, d, b, g)
        assert row_rel_err(y, ref) <= TOL, (fn, T)


@pytest.mark.parametrize("fn", ["moe_gemv", "moe_gemm"])
@pytest.mark.parametrize("d,b,g", [(4, 11, 64), (2, 9, 64)] + LARGE_CB)
def test_routed_other_widths(fn, d, b, g):
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, top_k = 10, 96, _cols_for(d, g, 4), 4
    spec, arrs, w = _case(d, b, g, rows, cols, ("w-moe", d, b, g), experts=E)
    for T in (1, 45):
        ids = synth.zipf_routing(T, E, top_k, "w-moe", T)
        ids[0, 1] = -1
        x = synth.activations((T, top_k, cols), "w-moe", d, b, g, T)
        announce(fn, "width", d, b, g, T)
        y = getattr(binding, fn)(w, to_dev(x), to_dev(ids), x_per_slot=True).cpu().numpy()
        ref = O.moe_ref(arrs["codes"], arrs["codebook"], arrs["scales"], x, ids, cols=cols, d=d, log2_k=b,
                        group=g, x_per_slot=True)
        assert np.all(y[0, 1] == 0)
        assert row_rel_err(y.reshape(-1, rows), ref.reshape(-1, rows)) <= TOL


@pytest.mark.parametrize("d,b,g", LARGE_CB)
def test_device_memory_codebooks_full_index_range(d, b, g):
    """Codebooks above 64 KiB are gathered from device memory: every entry,
    the first and the last included, must be read from the right place (a
    codebook whose entry k holds k/16384 and the scale 1, dequantized)."""
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols = 64, _cols_for(d, g, 8)
    spec = synth.Spec(rows=rows, cols=cols, d=d, log2_k=b, group=g)
    arrs = synth.tensor(spec, "w-cb", d, b, g)
    K = 1 << b
    cb = (np.arange(K * d, dtype=np.float64).reshape(K, d) % 2048 / 2048.0).astype(np.float16)
    cb[0], cb[-1] = -1.0, 0.5
    arrs["codebook"] = cb
    codes = np.arange(rows * cols // d) % K
    codes[:3], codes[-3:] = 0, K - 1
    arrs["codes"] = O.pack_codes(codes.reshape(rows, cols // d), b)[None]
    w = upload(arrs, spec)
    announce("large codebook", d, b, g)
    got = binding.dequant(w).cpu().numpy().view(np.uint16)
    want = O.dequant(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], cols, d, b, g).view(np.uint16)
    assert np.array_equal(got, want)
    x = synth.activations((3, cols), "w-cb", d, b, g)
    for fn in ("gemv", "gemm"):
        y = getattr(binding, fn)(w, to_dev(x)).cpu().numpy()
        ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, cols, d, b, g)
        assert row_rel_err(y, ref) <= TOL, fn
