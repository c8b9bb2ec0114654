"""GPU parity of the input/output types and fused output steps (vq_io):
bf16 activations in, fp16 / bf16 results out (the runtime profile the paper
scores takes and returns bf16: §7 Reproducibility), the SwiGLU activation of
an MLP's interleaved gate/up rows (paper §2.1: the gate, up and down
projections), and the router-weighted top-k combine of routed experts.

Tolerances (row-normalised, as for the plain calls): fp32 results 1e-3; a
result rounded to fp16 adds at most 2^-11 of its magnitude, to bf16 2^-8.
On exact-arithmetic inputs the fp32 result is exact, so its fp16 / bf16
rounding must equal the oracle value's rounding bit for bit."""
import numpy as np
import pytest

from oracle import vq_oracle as O
from vq_dequant_matmul_gemv_amd import synth
from tests.helpers import TOL, announce, hot_expert_ids, row_rel_err, to_dev, upload

pytestmark = pytest.mark.gpu

OUT_TOL = {"f32": TOL, "f16": TOL + 2.0 ** -11, "bf16": TOL + 2.0 ** -8}


def _torch_dtype(name):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def _host(y):
    """Device result as float64 (bf16 decoded from its bit patterns)."""
    import torch
    if y.dtype == torch.bfloat16:
        return O.bf16_to_f64(y.view(torch.int16).cpu().numpy().view(np.uint16))
    return y.float().cpu().numpy().astype(np.float64)


def _bf16_round(v):
    """Nearest bf16 value of each float64 (ties to the even pattern), found
    among all finite bf16 values: independent of the kernels' bit trick."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = O.bf16_to_f64(pats)
    keep = np.isfinite(vals) & ~((vals == 0) & (pats >= 0x8000))
    vals, pats = vals[keep], pats[keep]
    order = np.argsort(vals, kind="stable")
    vals, pats = vals[order], pats[order]
    v = np.asarray(v, dtype=np.float64)
    hi = np.clip(np.searchsorted(vals, v), 1, len(vals) - 1)
    lo = hi - 1
    dl, dh = v - vals[lo], vals[hi] - v
    pick_hi = (dh < dl) | ((dh == dl) & (pats[hi] % 2 == 0))
    return np.where(pick_hi, vals[hi], vals[lo])


def _dense_case(d, b, g, rows, cols, key, exact=False):
    spec = synth.Spec(rows=rows, cols=cols, d=d, log2_k=b, group=g)
    arrs = synth.tensor(spec, *key, exact=exact)
    return spec, arrs, upload(arrs, spec)


def _ref(arrs, x64, spec):
    return O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x64, spec.cols, spec.d,
                      spec.log2_k, spec.group)


@pytest.mark.parametrize("fn", ["gemv", "gemm"])
@pytest.mark.parametrize("d,b,g", [(2, 8, 64), (4, 8, 64), (4, 12, 128), (8, 12, 128)])
def test_bf16_in_every_output_type(fn, d, b, g):
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols = 301, 32 * d * 8
    spec, arrs, w = _dense_case(d, b, g, rows, cols, ("io", d, b, g))
    for T in (1, 5, 40):
        xb = synth.activations_bf16((T, cols), "io", d, b, g, T)
        x = to_dev(xb.view(np.int16)).view(torch.bfloat16)
        ref = _ref(arrs, O.bf16_to_f64(xb), spec)
        for out in ("f32", "f16", "bf16"):
            announce(fn, "bf16-in", out, d, b, g, T)
            y = getattr(binding, fn)(w, x, y_dtype=_torch_dtype(out))
            assert row_rel_err(_host(y), ref) <= OUT_TOL[out], (out, T)


@pytest.mark.parametrize("fn", ["gemv", "gemm"])
def test_fp16_and_bf16_outputs_round_to_nearest_even(fn):
    """Exact inputs: the fp32 result is exact, so the stored fp16 / bf16
    values are the oracle's rounded bit for bit; bf16 x in {-1, 0, 1}."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    d, b, g, rows, cols = 4, 8, 64, 260, 512
    spec, arrs, w = _dense_case(d, b, g, rows, cols, ("io-exact",), exact=True)
    for T in (1, 33):
        for xdt in ("f16", "bf16"):
            if xdt == "f16":
                xh = synth.activations((T, cols), "io-exact", T, exact=True)
                x, x64 = to_dev(xh), xh.astype(np.float64)
            else:
                xb = synth.activations_bf16((T, cols), "io-exact", T, exact=True)
                x, x64 = to_dev(xb.view(np.int16)).view(torch.bfloat16), O.bf16_to_f64(xb)
            ref = _ref(arrs, x64, spec)
            announce(fn, "exact rounding", xdt, T)
            y16 = getattr(binding, fn)(w, x, y_dtype=torch.float16).cpu().numpy()
            assert np.array_equal(y16.view(np.uint16), ref.astype(np.float16).view(np.uint16))
            yb = _host(getattr(binding, fn)(w, x, y_dtype=torch.bfloat16))
            assert np.array_equal(yb, _bf16_round(ref))


def _gate_up(rows_i, cols, d, b, g, key, experts=1):
    """A tensor of 2 * rows_i interleaved rows (gate i at 2i, up i at 2i + 1)."""
    spec = synth.Spec(rows=2 * rows_i, cols=cols, d=d, log2_k=b, group=g, experts=experts)
    arrs = synth.tensor(spec, *key)
    return spec, arrs, upload(arrs, spec)


@pytest.mark.parametrize("fn", ["gemv", "gemm"])
@pytest.mark.parametrize("d,b,g", [(2, 8, 64), (4, 8, 64), (8, 12, 128), (4, 12, 64)])
def test_swiglu_dense(fn, d, b, g):
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    spec, arrs, w = _gate_up(151, 32 * d * 6, d, b, g, ("swiglu", d, b, g))
    for T in (1, 3, 45):
        x = synth.activations((T, spec.cols), "swiglu", d, b, g, T)
        h_ref = O.swiglu_ref(_ref(arrs, x, spec))
        for out in ("f32", "f16", "bf16"):
            announce(fn, "swiglu", out, d, b, g, T)
            h = getattr(binding, fn)(w, to_dev(x), y_dtype=_torch_dtype(out), epilogue="swiglu")
            assert tuple(h.shape) == (T, 151)
            assert row_rel_err(_host(h), h_ref) <= OUT_TOL[out], (out, T)


def test_swiglu_gemm_on_shapes_that_would_split_k():
    """2048 columns and few tiles: plain fp32 calls split K and add slices
    atomically; the SwiGLU output needs whole sums, so those tiles run whole."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    spec, arrs, w = _gate_up(350, 2048, 2, 8, 64, ("swiglu-split",))
    for T in (4, 130):
        x = synth.activations((T, 2048), "swiglu-split", T)
        h_ref = O.swiglu_ref(_ref(arrs, x, spec))
        announce("gemm swiglu split shape", T)
        h = binding.gemm(w, to_dev(x), y_dtype=torch.float16, epilogue="swiglu")
        assert row_rel_err(_host(h), h_ref) <= OUT_TOL["f16"]


@pytest.mark.parametrize("fn", ["moe_gemv", "moe_gemm"])
@pytest.mark.parametrize("d,b,g", [(4, 8, 64), (8, 12, 128)])
def test_swiglu_routed(fn, d, b, g):
    """Routed gate/up experts with interleaved rows: h[t][s] = SwiGLU of
    expert ids[t][s]'s gate and up rows; skipped slots are zero rows."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    E, top_k, I = 12, 4, 48
    spec, arrs, w = _gate_up(I, 32 * d * 4, d, b, g, ("swiglu-moe", d, b, g), experts=E)
    for T in (1, 50):
        ids = synth.zipf_routing(T, E, top_k, "swiglu-moe", T)
        ids[0, 1] = -1
        x = synth.activations((T, spec.cols), "swiglu-moe", d, b, g, T)
        yref = O.moe_ref(arrs["codes"], arrs["codebook"], arrs["scales"], x, ids, cols=spec.cols, d=d,
                         log2_k=b, group=g, x_per_slot=False)
        h_ref = O.swiglu_ref(yref)
        announce(fn, "swiglu", d, b, g, T)
        h = getattr(binding, fn)(w, to_dev(x), to_dev(ids), y_dtype=torch.float16, epilogue="swiglu")
        assert tuple(h.shape) == (T, top_k, I)
        hh = _host(h)
        assert np.all(hh[0, 1] == 0)
        assert row_rel_err(hh.reshape(-1, I), h_ref.reshape(-1, I)) <= OUT_TOL["f16"]


@pytest.mark.parametrize("fn", ["moe_gemv", "moe_gemm"])
@pytest.mark.parametrize("d,b,g,x_per_slot", [(4, 8, 64, True), (2, 8, 64, False), (8, 12, 128, True)])
def test_combine_routed(fn, d, b, g, x_per_slot):
    """y[t] = sum of router weight x expert output over the token's valid
    slots, into a y the library zeroes first (filled with NaN here)."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    E, top_k, rows, cols = 16, 8, 96, 32 * d * 4
    spec = synth.Spec(rows=rows, cols=cols, d=d, log2_k=b, group=g, experts=E)
    arrs = synth.tensor(spec, "combine", d, b, g)
    w = upload(arrs, spec)
    for T in (1, 3, 70):
        ids = synth.zipf_routing(T, E, top_k, "combine", T)
        ids[0, 2] = -1
        if T > 1:
            ids[1, 0] = E + 3
        rw = synth.router_weights(T, top_k, "combine", T)
        shape = (T, top_k, cols) if x_per_slot else (T, cols)
        x = synth.activations(shape, "combine", d, b, g, T)
        yref = O.moe_ref(arrs["codes"], arrs["codebook"], arrs["scales"], x, ids, cols=cols, d=d, log2_k=b,
                         group=g, x_per_slot=x_per_slot)
        ref = O.moe_combine_ref(yref, rw, ids, E)
        y = torch.full((T, rows), float("nan"), device="cuda")
        announce(fn, "combine", d, b, g, "xps", x_per_slot, T)
        getattr(binding, fn)(w, to_dev(x), to_dev(ids), x_per_slot=x_per_slot, y=y, epilogue="combine",
                             route_weights=to_dev(rw))
        assert row_rel_err(y.cpu().numpy(), ref) <= TOL, T


def test_routed_gemm_output_steps_over_mixed_tile_kinds():
    """The routed GEMM's output steps where the routing lists 128-token tiles
    for hot experts, 32-token tiles and row halves (1024 tokens x top-8,
    992-row experts): SwiGLU of interleaved gate/up rows into bf16 h, then
    the combine of per-slot h through a down tensor of 992 rows."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    E, top_k, T, I, cols = 32, 8, 1024, 496, 256
    spec, arrs, w = _gate_up(I, cols, 4, 8, 64, ("mix-swiglu",), experts=E)
    ids = hot_expert_ids(T, top_k, E, ("mix-epi",))
    x = synth.activations((T, cols), "mix-swiglu")
    announce("moe_gemm mixed tiles swiglu")
    h = binding.moe_gemm(w, to_dev(x), to_dev(ids), y_dtype=torch.bfloat16, epilogue="swiglu")
    yref = O.moe_ref(arrs["codes"], arrs["codebook"], arrs["scales"], x, ids, cols=cols, d=4, log2_k=8, group=64,
                     x_per_slot=False)
    hh = _host(h)
    assert np.all(hh[900, 7] == 0) and np.all(hh[901, 6] == 0)
    assert row_rel_err(hh.reshape(-1, I), O.swiglu_ref(yref).reshape(-1, I)) <= OUT_TOL["bf16"]
    # down: 992 rows over the bf16 h of each slot, router-weighted combine
    dspec = synth.Spec(rows=992, cols=I + 16, d=4, log2_k=8, group=64, experts=E)
    darrs = synth.tensor(dspec, "mix-down")
    dw = upload(darrs, dspec)
    hx = np.zeros((T, top_k, I + 16), dtype=np.float16)
    hx[:, :, :I] = np.asarray(hh, dtype=np.float16)
    rw = synth.router_weights(T, top_k, "mix-down")
    y = torch.full((T, 992), float("nan"), device="cuda")
    announce("moe_gemm mixed tiles combine")
    binding.moe_gemm(dw, to_dev(hx), to_dev(ids), x_per_slot=True, y=y, epilogue="combine", route_weights=to_dev(rw))
    dref = O.moe_ref(darrs["codes"], darrs["codebook"], darrs["scales"], hx, ids, cols=I + 16, d=4, log2_k=8,
                     group=64, x_per_slot=True)
    assert row_rel_err(y.cpu().numpy(), O.moe_combine_ref(dref, rw, ids, E)) <= TOL


def test_bf16_profile_routed_gate_up_swiglu_then_down_combine():
    """The bf16 profile through a routed MLP: bf16 x -> gate/up SwiGLU (bf16
    h per slot) -> down with per-slot bf16 h and the router-weighted combine,
    against the oracle's chain on the same bf16 values."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    E, top_k, H, I, T = 16, 4, 512, 128, 40
    sgu = synth.Spec(rows=2 * I, cols=H, d=4, log2_k=8, group=64, experts=E)
    sdn = synth.Spec(rows=H, cols=I, d=4, log2_k=8, group=64, experts=E)
    agu, adn = synth.tensor(sgu, "bf16-mlp", "gu"), synth.tensor(sdn, "bf16-mlp", "dn")
    wgu, wdn = upload(agu, sgu), upload(adn, sdn)
    ids = synth.zipf_routing(T, E, top_k, "bf16-mlp")
    rw = synth.router_weights(T, top_k, "bf16-mlp")
    xb = synth.activations_bf16((T, H), "bf16-mlp")
    x = to_dev(xb.view(np.int16)).view(torch.bfloat16)
    for fn in ("moe_gemv", "moe_gemm"):
        announce("bf16 MLP", fn)
        h = getattr(binding, fn)(wgu, x, to_dev(ids), y_dtype=torch.bfloat16, epilogue="swiglu")
        out = getattr(binding, fn)(wdn, h, to_dev(ids), x_per_slot=True, epilogue="combine",
                                   route_weights=to_dev(rw))
        # oracle chain: h from the oracle, rounded to bf16 as the kernel stores it
        h_ref = O.swiglu_ref(O.moe_ref(agu["codes"], agu["codebook"], agu["scales"], O.bf16_to_f64(xb), ids,
                                       cols=H, d=4, log2_k=8, group=64, x_per_slot=False))
        assert row_rel_err(_host(h).reshape(-1, I), h_ref.reshape(-1, I)) <= OUT_TOL["bf16"]
        y_ref = O.moe_ref(adn["codes"], adn["codebook"], adn["scales"], _bf16_round(h_ref), ids, cols=I, d=4,
                          log2_k=8, group=64, x_per_slot=True)
        ref = O.moe_combine_ref(y_ref, rw, ids, E)
        # h's bf16 rounding can differ by one unit between the two sides near
        # rounding ties: 2^-8 of h propagates into the down projection
        assert row_rel_err(out.cpu().numpy(), ref) <= OUT_TOL["bf16"]
