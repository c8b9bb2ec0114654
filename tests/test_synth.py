"""The seeded generators: determinism, shapes, distributions, routing."""
import numpy as np

from vq_dequant_matmul_gemv_amd import synth


def test_same_seed_same_bytes_and_streams_differ():
    s = synth.Spec(rows=64, cols=256, d=4, log2_k=8, group=64, experts=2)
    a = synth.tensor(s, "det")
    b = synth.tensor(s, "det")
    c = synth.tensor(s, "other")
    for k in a:
        assert a[k].tobytes() == b[k].tobytes()
    assert a["codes"].tobytes() != c["codes"].tobytes()
    assert a["codes"].shape == (2, 64, 256 // 4 // 32 * 8)
    assert a["codebook"].shape == (256, 4) and a["codebook"].dtype == np.float16
    assert a["scales"].shape == (2, 64, 4) and a["scales"].dtype == np.float16


def test_distributions():
    s = synth.Spec(rows=512, cols=1024, d=2, log2_k=8, group=64)
    t = synth.tensor(s, "dist")
    codes = t["codes"].view(np.uint8).ravel()       # 8-bit codes are the bytes
    hist = np.bincount(codes, minlength=256)
    assert hist.min() > 0.8 * hist.mean() and hist.max() < 1.2 * hist.mean()
    sc = t["scales"].astype(np.float32)
    assert sc.min() >= 0.5 and sc.max() <= 1.5
    x = synth.activations((4, 4096), "dist").astype(np.float64)
    assert abs(x.std() - 1.0) < 0.05
    big = synth.tensor(synth.Spec(rows=32, cols=4096, d=4, log2_k=12, group=128), "cb")["codebook"]
    assert abs(big.astype(np.float64).std() - 0.02) < 0.002
    assert (np.abs(big.astype(np.float32)) < 2.0 ** -14).any()       # fp16 subnormals kept


def test_exact_variant_values():
    s = synth.Spec(rows=16, cols=256, d=4, log2_k=8, group=64)
    t = synth.tensor(s, "ex", exact=True)
    assert set(np.unique(t["scales"]).tolist()) <= {0.5, 1.0, 2.0}
    assert set((t["codebook"].astype(np.float64) * 16).ravel().tolist()) <= set(range(-8, 9))
    x = synth.activations((3, 256), "ex", exact=True)
    assert set(np.unique(x).tolist()) <= {-1.0, 0.0, 1.0}


def test_zipf_routing_distinct_and_skewed():
    ids = synth.zipf_routing(1024, 256, 8, "moe", 0)
    assert ids.shape == (1024, 8) and ids.dtype == np.int32
    assert all(len(set(r)) == 8 for r in ids.tolist())
    counts = np.bincount(ids.ravel(), minlength=256)
    assert counts.argmax() == 0 and counts[0] > 500            # head expert gets most tokens
    assert (counts > 0).sum() > 200                             # long tail is still hit


def test_mixed_tier_assignment_counts():
    tiers = synth.mixed_tier_assignment()
    assert len(tiers) == 75
    assert tiers.count("T1") == 48 and tiers.count("T2") == 12 and tiers.count("T3") == 15
    assert tiers == synth.mixed_tier_assignment()
