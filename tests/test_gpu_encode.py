"""GPU parity of the encoder (vq_encode) against the oracle's fit (paper
"Data-Free Vector Quantization Beats Affine Quantization at Matched Bytes
Below 5 Bits", §2.2 The fit, §2.3 Packing, §2.6 relative reconstruction
error): on seeded synthetic Gaussian weights with the same subsample and
uniforms, scales, codebook and packed codes are the same bits, and the
relative error agrees to fp64 rounding.  The fitted tensor then runs through
the decode and prefill kernels."""
import numpy as np
import pytest

from oracle import vq_encoder as E
from oracle import vq_oracle as O
from vq_dequant_matmul_gemv_amd import synth
from tests.helpers import TOL, announce, row_rel_err, to_dev

pytestmark = pytest.mark.gpu

CASES = [  # rows, cols, d, log2_k, group, n_sample, iters
    (64, 512, 4, 8, 64, 4096, 8),      # d4/K256 (the 397B card's geometry)
    (48, 512, 2, 8, 64, 4096, 6),      # d2/K256
    (32, 1024, 4, 11, 64, 4096, 5),    # d4/K2048 (paper §1 Notation's example)
    (40, 512, 2, 9, 128, 3000, 5),     # d2/K512
    (64, 2048, 8, 12, 128, 8192, 3),   # d8/K4096
    (24, 256, 2, 4, 64, 1000, 10),     # d2/K16 (the smallest build)
]


def _fit_both(rows, cols, d, b, g, n_s, iters, key):
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    w = synth.weights(rows, cols, *key)
    idx, u = synth.fit_draws(rows * cols // d, n_s, 1 << b, *key)
    ref = E.fit(w, d, b, g, idx, u, iters)
    t, rel = binding.encode(to_dev(w), d, b, g, to_dev(idx), torch.from_numpy(u).cuda(), iters)
    return w, ref, t, rel


@pytest.mark.parametrize("rows,cols,d,b,g,n_s,iters", CASES)
def test_encode_matches_the_oracle_fit_bit_for_bit(rows, cols, d, b, g, n_s, iters):
    announce("encode", rows, cols, d, b, g, n_s, iters)
    w, ref, t, rel = _fit_both(rows, cols, d, b, g, n_s, iters, ("enc", rows, cols, d, b, g))
    assert np.array_equal(t.scales.cpu().numpy().view(np.uint16), ref["scales"].view(np.uint16))
    assert np.array_equal(t.codebook.cpu().numpy().view(np.uint16), ref["codebook"].view(np.uint16))
    assert np.array_equal(t.codes.cpu().numpy().view(np.uint32), ref["words"])
    assert rel.item() == pytest.approx(ref["relerr"], rel=1e-9)
    assert 0 < ref["relerr"] < 1


def test_encoded_tensor_runs_through_the_kernels_and_repeats_exactly():
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols, d, b, g = 300, 1024, 4, 8, 64
    w, ref, t, rel = _fit_both(rows, cols, d, b, g, 8192, 6, ("enc-run",))
    x = synth.activations((5, cols), "enc-run")
    want = O.gemv_ref(ref["words"], ref["codebook"], ref["scales"], x, cols, d, b, g)
    for fn, xs in (("gemv", x[:1]), ("gemm", x)):
        announce("encode then", fn)
        y = getattr(binding, fn)(t, to_dev(xs)).cpu().numpy()
        assert row_rel_err(y, want[: len(xs)]) <= TOL
    # a second fit with the same draws gives the same bits
    idx, u = synth.fit_draws(rows * cols // d, 8192, 1 << b, "enc-run")
    t2, rel2 = binding.encode(to_dev(w), d, b, g, to_dev(idx), torch.from_numpy(u).cuda(), 6)
    for a, c in ((t.codes, t2.codes), (t.codebook, t2.codebook), (t.scales, t2.scales)):
        assert torch.equal(a, c)


@pytest.mark.slow
def test_encode_expert_matrix_full_size():
    """One expert matrix of the 256-expert MoE workload (1024 x 4096,
    d4/K256/g64): a million subvectors, 65,536 sampled, 4 Lloyd iterations."""
    announce("encode expert matrix")
    w, ref, t, rel = _fit_both(1024, 4096, 4, 8, 64, 65536, 4, ("enc-expert",))
    assert np.array_equal(t.codebook.cpu().numpy().view(np.uint16), ref["codebook"].view(np.uint16))
    assert np.array_equal(t.codes.cpu().numpy().view(np.uint32), ref["words"])
    assert rel.item() == pytest.approx(ref["relerr"], rel=1e-9)
