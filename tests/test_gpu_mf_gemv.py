"""GPU parity of the matrix-core GEMV: dense vq_gemv calls of two or more
tokens on matrices with at least one 16-row group per CU; rows longer than
one block's passes (d = 2: 5120 columns, d = 4: 6144, d = 8: 4096) run as
column slices added into y, and five to sixteen tokens in its 16-token mode.

The codebook entries go straight into the MFMA B operand and the x of four
chunk positions into a block-diagonal A operand, so every output needs the
right entry, the right x columns and the right scale group; each case is
checked against the CPU oracle on every output.  Rows past a whole number of
16-row groups, pass widths with idle chunk slots, token counts that leave a
partial four-token slice, bf16 / fp16 inputs and outputs and the SwiGLU step
are covered."""
import numpy as np
import pytest

from oracle import vq_oracle as O
from vq_dequant_matmul_gemv_amd import synth
from tests.helpers import TOL, announce, row_rel_err, to_dev, upload

pytestmark = pytest.mark.gpu

GEOMS = [(d, b, g) for d in (2, 4, 8) for b in (8, 12) for g in (64, 128)]
ROWS = 4096 + 37          # 16 rows per CU on 256 CUs, and a ragged last group


def _case(d, b, g, rows, cols, key):
    spec = synth.Spec(rows=rows, cols=cols, d=d, log2_k=b, group=g)
    arrs = synth.tensor(spec, *key)
    return spec, arrs, upload(arrs, spec)


def _ref(arrs, spec, x):
    return O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, spec.cols, spec.d,
                      spec.log2_k, spec.group)


@pytest.mark.parametrize("d,b,g", GEOMS)
def test_mf_gemv_all_geometries(d, b, g):
    from vq_dequant_matmul_gemv_amd import binding
    spec, arrs, w = _case(d, b, g, ROWS, 2048, ("mf", d, b, g))
    for T in (2, 3, 4):
        x = synth.activations((T, spec.cols), "mf", d, b, g, T)
        announce("mf-gemv", d, b, g, T)
        y = binding.gemv(w, to_dev(x)).cpu().numpy()
        assert row_rel_err(y, _ref(arrs, spec, x)) <= TOL, T


@pytest.mark.parametrize("rows,cols,d,b,g,Ts", [
    (ROWS, 5120, 2, 8, 64, (2, 4)),        # 160 chunks: 8 passes of 20 on 4 lanes x 5
    (ROWS, 6144, 4, 8, 64, (2, 4)),        # 96 chunks: 8 passes of 12 on 4 lanes x 3
    (ROWS, 5120, 4, 12, 128, (3,)),        # 80 chunks: 8 passes of 10, two idle slots
    (4096, 4096, 8, 12, 128, (2, 5, 8)),   # 32 chunks: 8 passes of 4; 16M weights keep 8 tokens
    (4608, 1088, 2, 8, 64, (4, 7)),        # 34 chunks: 2 passes of 17 on 4 lanes x 5
])
def test_mf_gemv_widths_passes_and_slices(rows, cols, d, b, g, Ts):
    from vq_dequant_matmul_gemv_amd import binding
    spec, arrs, w = _case(d, b, g, rows, cols, ("mf-wide", rows, cols, d, b, g))
    for T in Ts:
        x = synth.activations((T, cols), "mf-wide", rows, cols, T)
        announce("mf-gemv-wide", rows, cols, d, b, g, T)
        y = binding.gemv(w, to_dev(x)).cpu().numpy()
        assert row_rel_err(y, _ref(arrs, spec, x)) <= TOL, T


@pytest.mark.parametrize("rows,cols,d,b,g,Ts", [
    (ROWS, 17408, 4, 8, 64, (2, 4)),       # 272 chunks: 3 column slices of 91, 90, 91
    (ROWS, 10240, 2, 12, 128, (3,)),       # 320 chunks: 2 slices of 160
    (ROWS, 5184, 2, 8, 64, (2,)),          # 162 chunks: 2 slices of 81, the second from inside a scale group
    (4096, 8192, 8, 8, 64, (4, 7)),        # 64 chunks: 2 slices of 32; 32M weights, 2 token slices at T = 7
])
def test_mf_gemv_long_rows_in_column_slices(rows, cols, d, b, g, Ts):
    # (4096 x 8192 d = 8 has 16 one-pass slices: up to 10 tokens in the 16-token mode)
    """Rows longer than one block's passes: column slices side by side in
    one launch, each staging its own x and scale groups (slices starting
    inside a scale group included), added into a zeroed y."""
    from vq_dequant_matmul_gemv_amd import binding
    spec, arrs, w = _case(d, b, g, rows, cols, ("mf-long", rows, cols, d, b, g))
    for T in Ts:
        x = synth.activations((T, cols), "mf-long", rows, cols, T)
        announce("mf-gemv-long", rows, cols, d, b, g, T)
        y = binding.gemv(w, to_dev(x)).cpu().numpy()
        assert row_rel_err(y, _ref(arrs, spec, x)) <= TOL, T


@pytest.mark.parametrize("rows,cols,d,b,g,Ts", [
    (ROWS, 2048, 4, 8, 64, (5, 16, 21)),    # 32 chunks: 3 slices of 11, 11, 10; T = 21 past the limit: the GEMM
    (ROWS, 2048, 2, 12, 128, (9,)),          # 64 chunks: 4 slices of 16
    (ROWS, 1024, 8, 8, 64, (16,)),           # 8 chunks: 2 slices of 4, two scale groups per chunk
    (ROWS, 10240, 2, 8, 64, (12,)),          # 320 chunks: 16 slices of 20
    (4096, 4096, 4, 12, 128, (6, 13)),       # 64 chunks: 6 slices of 11 (the last 9), 128-weight groups
])
def test_mf_gemv_sixteen_token_mode(rows, cols, d, b, g, Ts):
    """Five to sixteen tokens per grid slice: one pass per column slice, x of
    all the slice's tokens staged once per block, the entries dequantized
    (times their scale, fp16) into the B operand, every item's sums added
    into y."""
    from vq_dequant_matmul_gemv_amd import binding
    spec, arrs, w = _case(d, b, g, rows, cols, ("mf16", rows, cols, d, b, g))
    for T in Ts:
        x = synth.activations((T, cols), "mf16", rows, cols, T)
        announce("mf-gemv-16", rows, cols, d, b, g, T)
        y = binding.gemv(w, to_dev(x)).cpu().numpy()
        assert row_rel_err(y, _ref(arrs, spec, x)) <= TOL, T


def test_mf_gemv_sixteen_token_mode_bf16_in_and_other_outputs():
    """bf16 x in the 16-token mode; an fp16 output (the items cannot add into
    it) keeps such calls on the other kernels."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    d, b, g, rows, cols, T = 4, 8, 64, ROWS, 2048, 9
    spec, arrs, w = _case(d, b, g, rows, cols, ("mf16-io",))
    xb = synth.activations_bf16((T, cols), "mf16-io")
    ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], O.bf16_to_f64(xb), cols, d, b, g)
    xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    announce("mf-gemv-16-io")
    y = binding.gemv(w, xd).cpu().numpy()
    assert row_rel_err(y, ref) <= TOL
    y16 = binding.gemv(w, xd, y_dtype=torch.float16).float().cpu().numpy()
    assert row_rel_err(y16, ref) <= TOL + 2.0 ** -11


@pytest.mark.parametrize("d,b,g", [(2, 8, 64), (4, 8, 64), (8, 12, 128)])
def test_mf_gemv_io_types_and_swiglu(d, b, g):
    """bf16 x, fp16 / bf16 y and the SwiGLU step over row pairs (2i, 2i + 1)."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols, T = ROWS + 1, 2048, 3
    spec, arrs, w = _case(d, b, g, rows, cols, ("mf-io", d, b, g))
    xb = synth.activations_bf16((T, cols), "mf-io", d, b, g)
    ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], O.bf16_to_f64(xb), cols, d, b, g)
    announce("mf-gemv-io", d, b, g)
    xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    y16 = binding.gemv(w, xd, y_dtype=torch.float16).float().cpu().numpy()
    assert row_rel_err(y16, ref) <= TOL + 2.0 ** -11
    h = binding.gemv(w, xd, y_dtype=torch.bfloat16, epilogue="swiglu").float().cpu().numpy()
    assert row_rel_err(h, O.swiglu_ref(ref)) <= TOL + 2.0 ** -8


def test_mf_gemv_repeat_runs_bit_identical():
    """Rows in one slice: no atomics, two runs give the same bits."""
    from vq_dequant_matmul_gemv_amd import binding
    spec, arrs, w = _case(4, 8, 64, ROWS, 2048, ("mf-rep",))
    x = to_dev(synth.activations((4, 2048), "mf-rep"))
    announce("mf-gemv-repeat")
    a = binding.gemv(w, x).cpu().numpy()
    b = binding.gemv(w, x).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
