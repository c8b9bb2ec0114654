"""Parity at the full workload sizes, in the launch configuration the
benchmark uses (the library picks kernels and grids from the shapes alone).

The oracle cannot afford every output of a 2048-token GEMM over a
17408 x 5120 matrix in float64, so each case checks a seeded sample of output
rows (first, last and random rows, every token), and for routed experts a
sample of (token, slot) pairs x rows.  Each sampled output depends only on
its own W row and x row, so slicing the oracle's inputs to the sample is the
same computation the full oracle would do for those outputs.
"""
import numpy as np
import pytest

from helpers import TOL, announce, row_rel_err, to_dev, upload
from oracle import vq_oracle as O
from vq_dequant_matmul_gemv_amd import synth

pytestmark = pytest.mark.gpu

N_ROWS = 48     # sampled output rows per matrix
N_PAIRS = 96    # sampled (token, slot) pairs per routed case


def _sample_rows(rows, *key):
    g = synth.rng("sample-rows", *key)
    pick = g.choice(rows, size=min(rows, N_ROWS - 2), replace=False)
    return np.unique(np.concatenate([[0, rows - 1], pick])).astype(np.int64)


def _dense_ref(arrs, spec, x, rsel):
    return O.gemv_ref(np.ascontiguousarray(arrs["codes"][0][rsel]), arrs["codebook"],
                      np.ascontiguousarray(arrs["scales"][0][rsel]), x, spec.cols, spec.d,
                      spec.log2_k, spec.group)


def _dense_case(wl, name, fn, T):
    from vq_dequant_matmul_gemv_amd import binding
    spec = synth.WORKLOADS[wl]["tensors"][name]
    arrs = synth.tensor(spec, wl, name)
    w = upload(arrs, spec)
    x = synth.activations((T, spec.cols), wl, "x", name, T)
    announce(wl, name, fn, "T", T, "rows", spec.rows, "cols", spec.cols)
    y = getattr(binding, fn)(w, to_dev(x)).cpu().numpy()
    assert np.isfinite(y).all()
    rsel = _sample_rows(spec.rows, wl, name, T)
    ref = _dense_ref(arrs, spec, x, rsel)
    err = row_rel_err(y[:, rsel], ref)
    assert err <= TOL, err


def test_gemv_1024_full():
    """The small dense case checked on every output."""
    from vq_dequant_matmul_gemv_amd import binding
    spec = synth.WORKLOADS["gemv_1024"]["tensors"]["w"]
    arrs = synth.tensor(spec, "gemv_1024", "w")
    w = upload(arrs, spec)
    x = synth.activations((1, spec.cols), "gemv_1024", "x")
    announce("gemv_1024 full")
    y = binding.gemv(w, to_dev(x)).cpu().numpy()
    ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, spec.cols, spec.d,
                     spec.log2_k, spec.group)
    assert row_rel_err(y, ref) <= TOL


@pytest.mark.parametrize("name", ["gate", "up", "down"])
@pytest.mark.parametrize("fn,T", [("gemv", 1), ("gemm", 2048)])
def test_dense_mlp_trio(name, fn, T):
    _dense_case("dense_mlp_5120x17408_d2k256", name, fn, T)


@pytest.mark.parametrize("fn,T", [("moe_gemv", 1), ("gemm", 2048)])
def test_dense_mlp_gate_up_stack(fn, T):
    """Gate and up as the benchmark runs them: one two-expert stack with
    per-expert codebooks, decoded by one routed GEMV with ids {0, 1} and
    prefilled by one vq_gemm over the stack (y [T][2][rows])."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    wl = "dense_mlp_5120x17408_d2k256"
    spec = synth.WORKLOADS[wl]["tensors"]["gate"]
    arrs = {n: synth.tensor(spec, wl, n) for n in ("gate", "up")}
    t = [upload(arrs[n], spec) for n in ("gate", "up")]
    w = binding.VQTensor(torch.stack([t[0].codes, t[1].codes]), torch.stack([t[0].codebook, t[1].codebook]),
                         torch.stack([t[0].scales, t[1].scales]), spec.rows, spec.cols, spec.d, spec.log2_k,
                         spec.group, 2, True)
    del t
    x = synth.activations((T, spec.cols), wl, "x", "gate_up", T)
    announce(wl, "gate+up stack", fn, "T", T)
    if fn == "moe_gemv":
        ids = torch.tensor([[0, 1]] * T, dtype=torch.int32, device="cuda")
        y = binding.moe_gemv(w, to_dev(x), ids).cpu().numpy()
    else:
        y = binding.gemm(w, to_dev(x)).cpu().numpy()
    assert y.shape == (T, 2, spec.rows) and np.isfinite(y).all()
    for e, n in enumerate(("gate", "up")):
        rsel = _sample_rows(spec.rows, wl, "stack", n, T)
        err = row_rel_err(y[:, e][:, rsel], _dense_ref(arrs[n], spec, x, rsel))
        assert err <= TOL, (n, err)


@pytest.mark.parametrize("name", ["A", "B"])
@pytest.mark.parametrize("fn,T", [("gemv", 1), ("gemv", 2), ("gemv", 3), ("gemv", 4), ("gemv", 16), ("gemm", 16),
                                  ("gemm", 256), ("gemm", 4096)])
def test_sweep_17408x5120_d4k256(name, fn, T):
    _dense_case("sweep_17408x5120_d4k256", name, fn, T)


def test_dense_full_size_dequant_bit_exact_sampled_rows():
    from vq_dequant_matmul_gemv_amd import binding
    wl = "dense_mlp_5120x17408_d2k256"
    spec = synth.WORKLOADS[wl]["tensors"]["down"]
    arrs = synth.tensor(spec, wl, "down")
    w = upload(arrs, spec)
    announce(wl, "down dequant")
    got = binding.dequant(w).cpu().numpy()
    rsel = _sample_rows(spec.rows, wl, "dequant")
    ref = O.dequant(np.ascontiguousarray(arrs["codes"][0][rsel]), arrs["codebook"],
                    np.ascontiguousarray(arrs["scales"][0][rsel]), spec.cols, spec.d, spec.log2_k,
                    spec.group)
    assert np.array_equal(got[rsel].view(np.uint16), ref.view(np.uint16))


def _moe_case(spec, arrs, w, key, fn, T, top_k, x_per_slot):
    """Run one routed call at full size; check sampled pairs x rows."""
    from vq_dequant_matmul_gemv_amd import binding
    E = spec.experts
    ids = synth.zipf_routing(T, E, top_k, *key, "ids", T)
    shape = (T, top_k, spec.cols) if x_per_slot else (T, spec.cols)
    x = synth.activations(shape, *key, "x", T, x_per_slot)
    announce(*key, fn, "T", T, "top_k", top_k, "x_per_slot", x_per_slot, "rows", spec.rows,
             "cols", spec.cols, "d", spec.d, "log2_k", spec.log2_k, "g", spec.group)
    y = getattr(binding, fn)(w, to_dev(x), to_dev(ids), x_per_slot=x_per_slot).cpu().numpy()
    assert y.shape == (T, top_k, spec.rows)
    assert np.isfinite(y).all()
    g = synth.rng("sample-pairs", *key, fn, T)
    npairs = T * top_k
    psel = np.unique(np.concatenate([[0, npairs - 1],
                                     g.choice(npairs, size=min(npairs, N_PAIRS), replace=False)]))
    rsel = _sample_rows(spec.rows, *key, fn, T)
    # oracle on the sampled pairs only: each sampled pair becomes a token with
    # one slot, carrying its own x row and expert id
    ids_s = ids.reshape(-1)[psel].reshape(-1, 1)
    if x_per_slot:
        xs = x.reshape(npairs, spec.cols)[psel]
    else:
        xs = x[psel // top_k]
    ref = O.moe_ref(np.ascontiguousarray(arrs["codes"][:, rsel]), arrs["codebook"],
                    np.ascontiguousarray(arrs["scales"][:, rsel]), xs, ids_s, cols=spec.cols, d=spec.d,
                    log2_k=spec.log2_k, group=spec.group, x_per_slot=False)
    got = y.reshape(npairs, spec.rows)[psel][:, rsel]
    err = row_rel_err(got, ref.reshape(len(psel), len(rsel)))
    assert err <= TOL, err


@pytest.mark.parametrize("name,x_per_slot", [("gate", False), ("down", True)])
def test_moe_e256_4096x1024_d4k256(name, x_per_slot):
    wl = "moe_e256_4096x1024_d4k256"
    spec = synth.WORKLOADS[wl]["tensors"][name]
    top_k = synth.WORKLOADS[wl]["top_k"]
    arrs = synth.tensor(spec, wl, name)
    w = upload(arrs, spec)
    for fn, T in (("moe_gemv", 1), ("moe_gemm", 1024)):
        _moe_case(spec, arrs, w, (wl, name), fn, T, top_k, x_per_slot)


@pytest.mark.parametrize("tier", ["T1", "T2", "T3"])
@pytest.mark.parametrize("index", [0, 2])   # gate-shaped and down-shaped tensors
def test_moe_mixed_tier_e256_2048x512(tier, index):
    wl = "moe_mixed_tier_e256_2048x512"
    spec = synth.mixed_tier_spec(index, tier)
    top_k = synth.WORKLOADS[wl]["top_k"]
    arrs = synth.tensor(spec, wl, tier, index)
    w = upload(arrs, spec)
    for fn, T in (("moe_gemv", 1), ("moe_gemm", 512)):
        _moe_case(spec, arrs, w, (wl, tier, index), fn, T, top_k, index == 2)
