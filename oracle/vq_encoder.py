"""Plain CPU oracle for the VQ encoder (the fit that produces codes, codebook
and scales from a weight tensor).

TEST INFRASTRUCTURE ONLY: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it; it shares no code with the GPU
path.

What it follows (paper "Data-Free Vector Quantization Beats Affine
Quantization at Matched Bytes Below 5 Bits"):
  §2.2 The fit: for each tensor, reshape the weights into d-dimensional
    subvectors, scale each group of 64 (here: of `group`) by its maximum
    absolute value, fit a K-entry codebook by k-means with k-means++
    initialization on a random subsample of the subvectors and plain Lloyd
    iterations, store codes, scales and codebook;
  §2.3 Packing: codes packed to their true bit width (vq_oracle.pack_codes);
  §2.6: the fitter's default seed 1234; relative reconstruction error
    ||W - W_hat|| / ||W|| as the corruption check.

Readings where the pages leave a step open (the plainest the rest supports,
each chosen so that a GPU run can reproduce it bit for bit):
  * scale = fp16(max |w| of the group); subvectors are w / f32(scale) in fp32
    (a group of zeros keeps scale 0 and zero subvectors);
  * squared distance = sum over t = 0 .. d-1, in that order, of (x_t - c_t)^2,
    each step an fp32 subtract, multiply and add rounded to nearest (no fused
    multiply-add); ties go to the lowest centroid index;
  * k-means++: the first centre is sample[floor(u_0 * n)]; centre k is the
    first sample point whose running sum of weights q exceeds
    floor(u_k * S), where q_i = round(D2_i * 2^32) as an integer (D2_i the
    squared distance to the nearest centre so far) and S = sum q_i -- integer
    sums are exact in any order; floor(u_k * S) is taken in fp64 and capped at
    S - 1; if S = 0 the draw falls back to floor(u_k * n).  The subsample indices and the uniforms u_k are inputs;
  * Lloyd: assign every subvector to its nearest centroid, then move each
    centroid to the mean of its subvectors, the mean taken as
    f32(f64(sum_i round(x_i * 2^32)) / n_k * 2^-32) (again an exact integer
    sum); an empty cluster keeps its centroid.  A fixed number of
    iterations (a converged iteration changes nothing, so stopping early
    gives the same result);
  * the codebook is stored in fp16 and the codes are the final assignment
    to that stored codebook.

Parity status: pinned by tests/test_encoder_pins.py (closed forms, brute
force, textbook k-means invariants on separable data).
"""

from __future__ import annotations

import numpy as np

from .vq_oracle import dequant, pack_codes

__all__ = ["group_scales", "subvectors", "dist2", "assign", "kmeanspp", "lloyd_update", "fit",
           "relerr", "FIXED_ONE"]

FIXED_ONE = float(2 ** 32)   # fixed-point unit of the exact sums


def group_scales(w: np.ndarray, group: int) -> np.ndarray:
    """fp16 [rows][cols/group]: the max |w| of each (row, group)."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    return np.abs(w.reshape(rows, cols // group, group)).max(axis=2).astype(np.float16)


def subvectors(w: np.ndarray, scales16: np.ndarray, d: int, group: int) -> np.ndarray:
    """fp32 [rows * cols / d][d]: each weight divided by its group's scale
    (fp32 division), consecutive d weights of a row forming one subvector;
    zero where the scale is zero."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    s = np.repeat(np.asarray(scales16, dtype=np.float16).astype(np.float32), group, axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        v = np.where(s == 0, np.float32(0), w / np.where(s == 0, np.float32(1), s)).astype(np.float32)
    return v.reshape(rows * cols // d, d)


def dist2(points: np.ndarray, c: np.ndarray) -> np.ndarray:
    """fp32 squared distances of points [n][d] to one centre c [d]: the sum
    over t in order of (x_t - c_t)^2, every operation rounded in fp32."""
    points = np.asarray(points, dtype=np.float32)
    acc = np.zeros(points.shape[0], dtype=np.float32)
    for t in range(points.shape[1]):
        diff = points[:, t] - np.float32(c[t])
        acc = acc + diff * diff
    return acc


def assign(points: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """int64 index of each point's nearest centroid (lowest index on ties)."""
    best = np.full(points.shape[0], np.inf, dtype=np.float32)
    code = np.zeros(points.shape[0], dtype=np.int64)
    for k in range(centroids.shape[0]):
        dk = dist2(points, centroids[k])
        closer = dk < best
        best = np.where(closer, dk, best)
        code = np.where(closer, k, code)
    return code


def _fixed(v) -> np.ndarray:
    """round(v * 2^32) as int64 (round half to even), v fp32."""
    return np.rint(np.asarray(v, dtype=np.float32).astype(np.float64) * FIXED_ONE).astype(np.int64)


def kmeanspp(sample: np.ndarray, k: int, uniforms: np.ndarray) -> np.ndarray:
    """k-means++ seeding: k centres [k][d] (fp32) drawn from the sample
    points, each with probability proportional to its squared distance to
    the nearest centre already drawn; uniforms [k] in [0, 1) decide the
    draws."""
    sample = np.asarray(sample, dtype=np.float32)
    n = sample.shape[0]
    u = np.asarray(uniforms, dtype=np.float64)
    centres = np.empty((k, sample.shape[1]), dtype=np.float32)
    centres[0] = sample[int(np.floor(u[0] * n))]
    d2 = dist2(sample, centres[0])
    for j in range(1, k):
        q = _fixed(d2)
        total = int(q.sum())
        if total == 0:
            idx = int(np.floor(u[j] * n))
        else:
            target = min(int(np.floor(u[j] * float(total))), total - 1)
            idx = int(np.argmax(np.cumsum(q) > target))
        centres[j] = sample[idx]
        d2 = np.minimum(d2, dist2(sample, centres[j]))
    return centres


def lloyd_update(points: np.ndarray, codes: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """Each centroid moved to the mean of its points (exact integer sums of
    round(x * 2^32), one fp64 division, fp32 result); empty clusters stay."""
    k, d = centroids.shape
    q = _fixed(points)
    sums = np.zeros((k, d), dtype=np.int64)
    np.add.at(sums, codes, q)
    counts = np.bincount(codes, minlength=k).astype(np.int64)
    new = centroids.astype(np.float32).copy()
    live = counts > 0
    mean = sums[live].astype(np.float64) / counts[live][:, None].astype(np.float64) / FIXED_ONE
    new[live] = mean.astype(np.float32)
    return new


def fit(w: np.ndarray, d: int, log2_k: int, group: int, sample_idx, uniforms, iters: int) -> dict:
    """The whole fit of one tensor w [rows][cols] (fp32): scales, subvectors,
    k-means++ on the subsample, `iters` Lloyd iterations, fp16 codebook,
    final codes and their packed words, relative reconstruction error."""
    k = 1 << log2_k
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    scales = group_scales(w, group)
    pts = subvectors(w, scales, d, group)
    cent = kmeanspp(pts[np.asarray(sample_idx)], k, uniforms)
    for _ in range(iters):
        codes = assign(pts, cent)
        new = lloyd_update(pts, codes, cent)
        if np.array_equal(new, cent):        # converged: further iterations change nothing
            break
        cent = new
    codebook = cent.astype(np.float16)
    codes = assign(pts, codebook.astype(np.float32)).reshape(rows, cols // d)
    words = pack_codes(codes, log2_k)
    return {"scales": scales, "codebook": codebook, "codes": codes, "words": words,
            "relerr": relerr(w, words, codebook, scales, d, log2_k, group)}


def relerr(w, words, codebook, scales, d, log2_k, group) -> float:
    """||W - dequant|| / ||W|| (Frobenius, float64; paper §2.6)."""
    w = np.asarray(w, dtype=np.float64)
    wq = dequant(words, codebook, scales, w.shape[1], d, log2_k, group).astype(np.float64)
    return float(np.sqrt(((w - wq) ** 2).sum()) / np.sqrt((w ** 2).sum()))
