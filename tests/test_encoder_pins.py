"""Pins for the encoder oracle (oracle/vq_encoder.py): closed forms, brute
force on tiny inputs and textbook k-means invariants on separable data, so a
dropped term, a wrong sign or index, or a transposed operand fails a test.
(paper "Data-Free Vector Quantization Beats Affine Quantization at Matched
Bytes Below 5 Bits", §2.2 The fit, §2.6 relative reconstruction error.)"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import vq_encoder as E
from oracle import vq_oracle as O


def test_group_scales_are_fp16_max_abs():
    w = np.array([[0.5, -3.0, 1.0, 2.0, 0.0, 0.0, 0.0, -0.25]], dtype=np.float32)
    s = E.group_scales(w, 4)
    assert s.dtype == np.float16 and s.tolist() == [[3.0, 0.25]]
    # a max that fp16 cannot hold exactly is rounded to nearest
    w2 = np.array([[1.0 + 2.0 ** -12, 0.0]], dtype=np.float32)
    assert E.group_scales(w2, 2)[0, 0] == np.float16(1.0)


def test_subvectors_divide_by_scale_and_keep_zero_groups():
    w = np.array([[2.0, -1.0, 0.5, 4.0, 0.0, 0.0, 0.0, 0.0]], dtype=np.float32)
    s = E.group_scales(w, 4)                       # [4, 0]
    v = E.subvectors(w, s, 2, 4)
    assert v.tolist() == [[0.5, -0.25], [0.125, 1.0], [0.0, 0.0], [0.0, 0.0]]
    # row-major subvectors: the d weights of a subvector are consecutive in a row
    w3 = np.arange(16, dtype=np.float32).reshape(2, 8) + 1
    v3 = E.subvectors(w3, E.group_scales(w3, 8), 4, 8)
    assert np.allclose(v3 * np.array([[8], [8], [16], [16]]), w3.reshape(4, 4))


def test_dist2_exact_small_values_and_symmetry():
    pts = np.array([[1.0, 2.0, -3.0], [0.0, 0.0, 0.0]], dtype=np.float32)
    c = np.array([0.5, -1.0, 1.0], dtype=np.float32)
    assert E.dist2(pts, c).tolist() == [0.25 + 9.0 + 16.0, 0.25 + 1.0 + 1.0]
    assert E.dist2(c[None], pts[0])[0] == E.dist2(pts[:1], c)[0]


def test_assign_is_the_brute_force_nearest_with_lowest_index_ties():
    g = np.random.default_rng(3)
    pts = g.integers(-4, 5, size=(50, 2)).astype(np.float32) / 4
    cent = g.integers(-4, 5, size=(7, 2)).astype(np.float32) / 4
    cent[5] = cent[2]                                # a duplicate: ties go to 2
    got = E.assign(pts, cent)
    for i, p in enumerate(pts):
        ds = [sum((Fraction(float(p[t])) - Fraction(float(c[t]))) ** 2 for t in range(2)) for c in cent]
        assert got[i] == min(range(7), key=lambda k: (ds[k], k))
    assert 5 not in got


def test_kmeanspp_draw_rule_by_hand():
    # sample on a line: 0, 1, 3 (d = 1).  First centre: floor(0.5 * 3) = 1 -> x = 1.
    # D2 = [1, 0, 4] -> q = [2^32, 0, 4 * 2^32], S = 5 * 2^32.
    # u = 0.1: target = floor(0.5 * 2^32) -> first running sum above it is index 0.
    # u = 0.3: target = floor(1.5 * 2^32) -> index 2.
    sample = np.array([[0.0], [1.0], [3.0]], dtype=np.float32)
    assert E.kmeanspp(sample, 2, [0.5, 0.1])[:, 0].tolist() == [1.0, 0.0]
    assert E.kmeanspp(sample, 2, [0.5, 0.3])[:, 0].tolist() == [1.0, 3.0]
    # third centre after {1, 3}: D2 = [1, 0, 0] -> always index 0
    assert E.kmeanspp(sample, 3, [0.5, 0.3, 0.99])[:, 0].tolist() == [1.0, 3.0, 0.0]
    # every point already a centre (S = 0): the fallback floor(u * n)
    assert E.kmeanspp(sample, 4, [0.5, 0.3, 0.99, 0.4])[3, 0] == 1.0


def _clusters(n_per=64, centres=((0.5, 0.5), (-0.5, 0.5), (0.5, -0.5), (-0.5, -0.5)), spread=1e-3, seed=5):
    g = np.random.default_rng(seed)
    pts = np.concatenate([np.asarray(c, np.float32) + g.uniform(-spread, spread, size=(n_per, 2)).astype(np.float32)
                          for c in centres])
    return pts, np.asarray(centres, np.float32)


def test_kmeanspp_picks_one_centre_per_separated_cluster():
    pts, centres = _clusters()
    g = np.random.default_rng(9)
    for _ in range(5):
        c = E.kmeanspp(pts, 4, g.uniform(size=4))
        owner = E.assign(c, centres)
        assert sorted(owner.tolist()) == [0, 1, 2, 3]


def test_lloyd_update_is_the_exact_mean_and_keeps_empty_clusters():
    pts = np.array([[0.25, 1.0], [0.75, -1.0], [0.5, 0.5], [0.0, 0.0]], dtype=np.float32)
    codes = np.array([0, 0, 2, 2])
    prev = np.array([[9.0, 9.0], [7.0, -7.0], [1.0, 1.0]], dtype=np.float32)
    new = E.lloyd_update(pts, codes, prev)
    assert new.tolist() == [[0.5, 0.0], [7.0, -7.0], [0.25, 0.25]]


def test_lloyd_never_increases_the_objective_and_finds_separated_clusters():
    pts, centres = _clusters(n_per=40, seed=2)
    rng = np.random.default_rng(4)
    cent = pts[rng.choice(len(pts), 4, replace=False)]
    cent[1] = cent[0] + 1e-4                          # a poor start
    obj = []
    for _ in range(6):
        codes = E.assign(pts, cent)
        obj.append(float(sum(E.dist2(pts[codes == k], cent[k]).sum() for k in range(4))))
        cent = E.lloyd_update(pts, codes, cent)
    assert all(b <= a * (1 + 1e-6) for a, b in zip(obj, obj[1:]))
    # from a k-means++ start the fit lands on the four cluster means
    cent = E.kmeanspp(pts, 4, rng.uniform(size=4))
    for _ in range(5):
        cent = E.lloyd_update(pts, E.assign(pts, cent), cent)
    truth = np.stack([pts[i * 40:(i + 1) * 40].mean(axis=0) for i in range(4)])
    assert np.allclose(np.sort(cent, axis=0), np.sort(truth, axis=0), atol=1e-6)


def test_relerr_closed_forms():
    # a tensor the codebook and scales represent exactly: relerr 0
    d, b, g = 2, 4, 64
    cb = (np.arange(32).reshape(16, 2) / 16 - 1).astype(np.float16)
    codes = np.random.default_rng(1).integers(0, 16, size=(3, 64))
    scales = np.array([[2.0, 1.0], [0.5, 0.25], [1.0, 4.0]], dtype=np.float16)
    words = O.pack_codes(codes, b)
    w = O.dequant(words, cb, scales, 128, d, b, g).astype(np.float32)
    assert E.relerr(w, words, cb, scales, d, b, g) == 0.0
    # every weight off by the same relative amount: relerr is that amount
    assert E.relerr(w * 1.25, words, cb, scales, d, b, g) == pytest.approx(0.2, rel=1e-12)


def test_fit_end_to_end_on_exactly_representable_weights():
    """Weights built from a 16-entry codebook (d = 2) with distinct entries and
    max-abs-normalised groups: the fit recovers a codebook and codes that
    reconstruct them with relerr far below that of random assignment."""
    rng = np.random.default_rng(11)
    d, b, g = 2, 4, 64
    grid = np.array(list(itertools.product([-1.0, -0.5, 0.5, 1.0], repeat=2)), dtype=np.float32)
    codes = rng.integers(0, 16, size=(8, 64))
    w = grid[codes].reshape(8, 128) * np.repeat(rng.uniform(0.5, 2.0, size=(8, 2)), 64, axis=1).astype(np.float32)
    n = 8 * 64
    res = E.fit(w, d, b, g, sample_idx=rng.choice(n, 256, replace=False), uniforms=rng.uniform(size=16), iters=10)
    assert res["words"].shape == (8, 128 * b // (32 * d))
    assert np.array_equal(O.unpack_codes(res["words"], 128, d, b), res["codes"])
    assert res["relerr"] < 0.05
    base = E.relerr(w, O.pack_codes(rng.integers(0, 16, size=(8, 64)), b), res["codebook"], res["scales"], d, b, g)
    assert base > 0.5
