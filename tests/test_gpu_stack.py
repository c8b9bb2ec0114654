"""GPU parity of vq_gemm and vq_gemv on a stack of experts: every expert
times the same x, y[t][e] = W_e x[t] (an MLP's gate and up projections,
which share their input, in one launch).

Each row tile takes its own expert's codes, scales and codebook, and writes
row t * E + e of y; split tiles of a last, partial round zero and add into
their own expert's region.  Checked against the oracle per expert, with y
filled with NaN beforehand (every output must be written), over ragged row
counts, token counts spanning several tiles with a ragged tail, both tile
shapes, shared and per-expert codebooks, split last rounds, fp16 / bf16
outputs (never split: bit-identical to one call per expert) and the SwiGLU
step within each expert.  The GEMV's stack runs the experts' row blocks
side by side in one grid: its streaming path (one and two tokens per grid
slice, column slices added in turn), its matrix-core path (block-diagonal
and 16-token modes, column slices added atomically) and the hand-off to the
stacked GEMM above its token limit."""
import numpy as np
import pytest

from oracle import vq_oracle as O
from vq_dequant_matmul_gemv_amd import synth
from tests.helpers import TOL, announce, row_rel_err, to_dev, upload

pytestmark = pytest.mark.gpu


def _stack(E, rows, cols, d, b, g, cbpe, key):
    spec = synth.Spec(rows=rows, cols=cols, d=d, log2_k=b, group=g, experts=E)
    arrs = synth.tensor(spec, *key, codebook_per_expert=cbpe)
    return spec, arrs, upload(arrs, spec, codebook_per_expert=cbpe)


def _ref(arrs, spec, e, x, cbpe):
    cb = arrs["codebook"][e] if cbpe else arrs["codebook"]
    return O.gemv_ref(arrs["codes"][e], cb, arrs["scales"][e], x, spec.cols, spec.d, spec.log2_k, spec.group)


def _expert(w, e):
    from vq_dequant_matmul_gemv_amd import binding
    cb = w.codebook[e] if w.codebook_per_expert else w.codebook
    return binding.VQTensor(w.codes[e], cb, w.scales[e], w.rows, w.cols, w.d, w.log2_k, w.group)


@pytest.mark.parametrize("E,rows,cols,d,b,g,cbpe,Ts,tile", [
    (2, 1000, 2048, 2, 8, 64, True, (1, 37, 200), None),      # ragged rows and tokens; split last round
    (3, 520, 1024, 4, 12, 128, False, (130,), "128"),         # shared codebook, 128-token tiles
    (2, 2048, 4096, 8, 8, 64, True, (64, 300), "32"),         # 32-token tiles, d = 8
    (2, 4096, 2048, 4, 8, 64, True, (777,), None),            # several rounds of tiles, a partial one split
    (4, 608, 1024, 2, 10, 64, True, (96,), None),             # 10-bit codes, four experts
])
def test_stack_gemm_matches_oracle(monkeypatch, E, rows, cols, d, b, g, cbpe, Ts, tile):
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    if tile:
        monkeypatch.setenv("VQMI_GEMM_TILE", tile)
    spec, arrs, w = _stack(E, rows, cols, d, b, g, cbpe, ("stack", E, rows, cols, d, b, g))
    for T in Ts:
        x = synth.activations((T, cols), "stack", E, rows, cols, T)
        announce("stack-gemm", E, rows, cols, d, b, g, T, tile)
        y = torch.full((T, E, rows), float("nan"), device="cuda")
        binding.gemm(w, to_dev(x), y)
        got = y.cpu().numpy()
        assert not np.isnan(got).any(), T
        for e in range(E):
            assert row_rel_err(got[:, e], _ref(arrs, spec, e, x, cbpe)) <= TOL, (T, e)


def test_stack_gemm_half_outputs_bit_identical_to_per_expert_calls(monkeypatch):
    """fp16 / bf16 outputs are never split along K: with the tile shape fixed,
    each expert's rows are those of a call on that expert alone, bit for bit."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    monkeypatch.setenv("VQMI_GEMM_TILE", "128")
    E, rows, cols, T = 2, 1000, 2048, 150
    spec, arrs, w = _stack(E, rows, cols, 4, 8, 64, True, ("stack-half",))
    x = to_dev(synth.activations((T, cols), "stack-half"))
    for dt in (torch.float16, torch.bfloat16):
        announce("stack-gemm-half", dt)
        y = binding.gemm(w, x, y_dtype=dt)
        assert tuple(y.shape) == (T, E, rows)
        for e in range(E):
            ye = binding.gemm(_expert(w, e), x, y_dtype=dt)
            assert torch.equal(y[:, e].view(torch.int16), ye.view(torch.int16)), (dt, e)
        ref = _ref(arrs, spec, 1, synth.activations((T, cols), "stack-half"), True)
        assert row_rel_err(y[:, 1].float().cpu().numpy(), ref) <= TOL + 2.0 ** -8


def test_stack_gemm_swiglu_within_each_expert():
    """SwiGLU over each expert's interleaved row pairs: y is [T][E][rows / 2]."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, T = 2, 1000, 2048, 70
    spec, arrs, w = _stack(E, rows, cols, 2, 8, 64, True, ("stack-swiglu",))
    x = synth.activations((T, cols), "stack-swiglu")
    announce("stack-gemm-swiglu")
    h = binding.gemm(w, to_dev(x), y_dtype=torch.bfloat16, epilogue="swiglu").float().cpu().numpy()
    assert h.shape == (T, E, rows // 2)
    for e in range(E):
        assert row_rel_err(h[:, e], O.swiglu_ref(_ref(arrs, spec, e, x, True))) <= TOL + 2.0 ** -8, e


@pytest.mark.parametrize("E,rows,cols,d,b,g,cbpe,Ts", [
    (2, 4133, 2048, 4, 8, 64, True, (1, 2, 3, 4, 9, 16, 21)),  # matrix-core modes; T = 21: the stacked GEMM
    (2, 1000, 2048, 2, 8, 64, True, (1, 2, 5)),                # streaming path, two-token slices
    (3, 1500, 10240, 2, 12, 128, False, (1, 3)),               # shared codebook; two matrix-core column slices
    (2, 512, 24576, 4, 8, 64, True, (1, 2)),                   # streaming path in two column slices
])
def test_stack_gemv_matches_oracle(E, rows, cols, d, b, g, cbpe, Ts):
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    spec, arrs, w = _stack(E, rows, cols, d, b, g, cbpe, ("stack-gemv", E, rows, cols, d, b, g))
    for T in Ts:
        x = synth.activations((T, cols), "stack-gemv", E, rows, cols, T)
        announce("stack-gemv", E, rows, cols, d, b, g, T)
        y = torch.full((T, E, rows), float("nan"), device="cuda")
        binding.gemv(w, to_dev(x), y)
        got = y.cpu().numpy()
        assert not np.isnan(got).any(), T
        for e in range(E):
            assert row_rel_err(got[:, e], _ref(arrs, spec, e, x, cbpe)) <= TOL, (T, e)


def test_stack_gemv_one_token_bit_identical_to_per_expert_and_routed_calls():
    """One token on the streaming path: every row's arithmetic is that of a
    call on its expert alone, and of the routed call with ids {0, 1}."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols = 2, 4133, 5120
    spec, arrs, w = _stack(E, rows, cols, 2, 8, 64, True, ("stack-gemv-bits",))
    x = to_dev(synth.activations((1, cols), "stack-gemv-bits"))
    announce("stack-gemv-bits")
    y = binding.gemv(w, x)
    yr = binding.moe_gemv(w, x, torch.tensor([[0, 1]], dtype=torch.int32, device="cuda"))
    assert torch.equal(y.view(torch.int32), yr.view(torch.int32))
    for e in range(E):
        assert torch.equal(y[:, e].view(torch.int32), binding.gemv(_expert(w, e), x).view(torch.int32)), e


@pytest.mark.parametrize("T", [1, 3])
def test_stack_gemv_swiglu_bf16(T):
    """SwiGLU within each expert and a bf16 y on the stacked GEMV."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols = 2, 4134, 2048
    spec, arrs, w = _stack(E, rows, cols, 4, 8, 64, True, ("stack-gemv-swiglu",))
    x = synth.activations((T, cols), "stack-gemv-swiglu", T)
    announce("stack-gemv-swiglu", T)
    h = binding.gemv(w, to_dev(x), y_dtype=torch.bfloat16, epilogue="swiglu").float().cpu().numpy()
    assert h.shape == (T, E, rows // 2)
    for e in range(E):
        assert row_rel_err(h[:, e], O.swiglu_ref(_ref(arrs, spec, e, x, True))) <= TOL + 2.0 ** -8, e


@pytest.mark.parametrize("fn,T", [("gemv", 1), ("gemv", 4), ("gemm", 130)])
def test_stack_bf16_x(fn, T):
    """bf16 x (converted to fp16 as it is staged) on both stacked calls."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols = 2, 2080, 2048
    spec, arrs, w = _stack(E, rows, cols, 4, 8, 64, True, ("stack-bf16",))
    xb = synth.activations_bf16((T, cols), "stack-bf16", T)
    xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    announce("stack-bf16", fn, T)
    y = getattr(binding, fn)(w, xd).cpu().numpy()
    assert y.shape == (T, E, rows)
    for e in range(E):
        assert row_rel_err(y[:, e], _ref(arrs, spec, e, O.bf16_to_f64(xb), True)) <= TOL, e
