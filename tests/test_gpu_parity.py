"""GPU parity against the CPU oracle at sizes the oracle finishes in seconds.

Every geometry (d in {2,4,8}, K in {256, 4096}, g in {64,128}), several tiles
and a ragged tail in rows, tokens and columns; bit-exact dequant; outputs
within 1e-3 (row-normalised); bit-identical outputs on exact-arithmetic
inputs; routed experts with skipped and duplicate ids."""
import numpy as np
import pytest

from oracle import vq_oracle as O
from vq_dequant_matmul_gemv_amd import synth
from tests.helpers import hot_expert_ids, TOL, announce, row_rel_err, to_dev, upload

pytestmark = pytest.mark.gpu

GEOMS = [(d, b, g) for d in (2, 4, 8) for b in (8, 12) for g in (64, 128)]


def _case(d, b, g, rows, cols, key, exact=False, experts=1, cbpe=False):
    spec = synth.Spec(rows=rows, cols=cols, d=d, log2_k=b, group=g, experts=experts)
    arrs = synth.tensor(spec, *key, exact=exact, codebook_per_expert=cbpe)
    return spec, arrs, upload(arrs, spec, codebook_per_expert=cbpe)


def _cols_for(d, g, blocks):
    cols = 32 * d * blocks
    while cols % g:
        cols += 32 * d
    return cols


@pytest.mark.parametrize("d,b,g", GEOMS)
def test_dequant_bit_exact(d, b, g):
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols = 37, _cols_for(d, g, 5)
    announce("dequant", d, b, g, rows, cols)
    spec, arrs, w = _case(d, b, g, rows, cols, ("dq", d, b, g))
    got = binding.dequant(w).cpu().numpy().view(np.uint16)
    want = O.dequant(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], cols, d, b, g).view(np.uint16)
    assert np.array_equal(got, want)


def test_dequant_subnormal_and_extreme_entries():
    from vq_dequant_matmul_gemv_amd import binding
    d, b, g, rows, cols = 2, 8, 64, 8, 256
    spec = synth.Spec(rows=rows, cols=cols, d=d, log2_k=b, group=g)
    arrs = synth.tensor(spec, "dq-sub")
    cb = arrs["codebook"].view(np.uint16).copy()
    cb[:64] = np.arange(1, 129, dtype=np.uint16).reshape(64, 2)          # subnormals
    cb[64:80] = 0x7BFF                                                   # max finite
    cb[80:96] = 0x8000                                                   # -0
    arrs["codebook"] = cb.view(np.float16)
    sc = arrs["scales"].view(np.uint16).copy()
    sc[0, 0, :2] = [0x0001, 0x3C00]
    sc[0, 1, :2] = [0x7BFF, 0x0400]
    arrs["scales"] = sc.view(np.float16)
    announce("dequant-subnormal")
    w = upload(arrs, spec)
    got = binding.dequant(w).cpu().numpy().view(np.uint16)
    want = O.dequant(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], cols, d, b, g).view(np.uint16)
    assert np.array_equal(got, want)


def test_dequant_expert_and_per_expert_codebook():
    from vq_dequant_matmul_gemv_amd import binding
    spec, arrs, w = _case(4, 12, 128, 20, 256, ("dq-e",), experts=3, cbpe=True)
    for e in range(3):
        announce("dequant-expert", e)
        got = binding.dequant(w, expert=e).cpu().numpy().view(np.uint16)
        want = O.dequant(arrs["codes"][e], arrs["codebook"][e], arrs["scales"][e], 256, 4, 12, 128)
        assert np.array_equal(got, want.view(np.uint16))


@pytest.mark.parametrize("fn", ["gemv", "gemm"])
@pytest.mark.parametrize("d,b,g", GEOMS)
def test_dense_all_geometries(fn, d, b, g):
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols = 301, _cols_for(d, g, 7)
    spec, arrs, w = _case(d, b, g, rows, cols, ("dense", d, b, g))
    for T in (1, 3, 18):
        x = synth.activations((T, cols), "dense", d, b, g, T)
        announce(fn, d, b, g, rows, cols, T)
        y = getattr(binding, fn)(w, to_dev(x)).cpu().numpy()
        ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, cols, d, b, g)
        err = row_rel_err(y, ref)
        assert err <= TOL, (fn, T, err)


@pytest.mark.parametrize("fn", ["gemv", "gemm"])
@pytest.mark.parametrize("d,b,g", [(2, 8, 64), (4, 8, 64), (4, 12, 128), (8, 12, 128), (8, 8, 64)])
def test_dense_exact_inputs_bit_identical(fn, d, b, g):
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols = 260, _cols_for(d, g, 6)
    spec, arrs, w = _case(d, b, g, rows, cols, ("exact", d, b, g), exact=True)
    for T in (1, 2, 5, 33):
        x = synth.activations((T, cols), "exact", d, b, g, T, exact=True)
        announce(fn, "exact", d, b, g, T)
        y = getattr(binding, fn)(w, to_dev(x)).cpu().numpy()
        ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, cols, d, b, g)
        assert np.array_equal(y.astype(np.float64), ref), (fn, T)


@pytest.mark.parametrize("d,b,g", GEOMS)
def test_gemm_128_token_tiles_all_geometries(d, b, g, monkeypatch):
    """The 128-token tiles (forced: at these sizes the time model takes
    32-token ones) in every geometry: ragged rows and tokens, an odd number of
    super-steps, and a K split whose slices hold an odd number of super-steps
    (the main loop's second half-step is skipped).  Then the tiles the model
    picks at T = 129."""
    from vq_dequant_matmul_gemv_amd import binding
    monkeypatch.setenv("VQMI_GEMM_TILE", "128")
    ss = 64 if d == 2 else 128                      # columns per super-step
    for rows, cols, Ts in ((301, _cols_for(d, g, 7), (40, 129)),
                           (1030, ss * (25 if d == 2 else 13 if d == 4 else 18), (130,))):
        if cols % g or (cols // d) % 32:
            cols = _cols_for(d, g, cols // (32 * d))
        spec, arrs, w = _case(d, b, g, rows, cols, ("t128", d, b, g, rows))
        for T in Ts:
            x = synth.activations((T, cols), "t128", d, b, g, rows, T)
            announce("gemm", "t128", d, b, g, rows, cols, T)
            y = binding.gemm(w, to_dev(x)).cpu().numpy()
            ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, cols, d, b, g)
            err = row_rel_err(y, ref)
            assert err <= TOL, (rows, cols, T, err)
            if T == 129:
                monkeypatch.delenv("VQMI_GEMM_TILE")
                y = binding.gemm(w, to_dev(x)).cpu().numpy()
                monkeypatch.setenv("VQMI_GEMM_TILE", "128")
                assert row_rel_err(y, ref) <= TOL, (rows, cols, T)


@pytest.mark.parametrize("fn", ["gemv", "gemm"])
def test_dense_shapes_and_tokens(fn):
    """Ragged tokens around the tile sizes, tiny and tall shapes, a column
    count with a half super-step (d=2, cols % 128 == 64), a row count that
    is not a multiple of 4, and K split over slices of a few tiles."""
    from vq_dequant_matmul_gemv_amd import binding
    cases = [(1, 64, 2, 8, 64, [1, 2]), (3, 192, 2, 8, 64, [1, 7, 16, 17]),
             (513, 320, 2, 8, 64, [1, 4, 129]), (257, 128, 4, 8, 64, [5, 64, 65]),
             (64, 512, 8, 12, 128, [1, 63, 64, 65]), (1030, 256, 4, 8, 128, [1, 130]),
             # several 8-group scale windows, K split into slices that start
             # inside a window; 20 groups per row (windows not 16-byte aligned)
             # and 40 (aligned)
             (700, 1280, 2, 8, 64, [300]), (300, 2560, 4, 8, 64, [200])]
    for rows, cols, d, b, g, Ts in cases:
        spec, arrs, w = _case(d, b, g, rows, cols, ("shapes", rows, cols))
        for T in Ts:
            x = synth.activations((T, cols), "shapes", rows, cols, T)
            announce(fn, "shape", rows, cols, d, b, g, T)
            y = getattr(binding, fn)(w, to_dev(x)).cpu().numpy()
            ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, cols, d, b, g)
            assert row_rel_err(y, ref) <= TOL, (rows, cols, T)


@pytest.mark.parametrize("b,g", [(8, 64), (8, 128), (12, 64), (12, 128)])
def test_gemm_d2_thin_tiles_both_super_step_lengths(b, g):
    """d = 2 thin tiles (T <= 32) take 128-column super-steps when the
    columns are a multiple of 128 and 64-column ones otherwise (possible only
    with 64-weight groups); against the oracle, several row tiles and a
    ragged token count."""
    from vq_dequant_matmul_gemv_amd import binding
    for rows, cols in ((600, 1024), (600, 1088 if g == 64 else 1280)):
        spec, arrs, w = _case(2, b, g, rows, cols, ("thin", b, g, cols))
        for T in (1, 7, 32):
            x = synth.activations((T, cols), "thin", b, g, cols, T)
            announce("gemm-thin", b, g, rows, cols, T)
            y = binding.gemm(w, to_dev(x)).cpu().numpy()
            ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, cols, 2, b, g)
            assert row_rel_err(y, ref) <= TOL, (b, g, cols, T)


def test_gemv_wide_rows_split_into_column_slices():
    """More than 1024 16-code chunks per row: the GEMV runs column slices
    and accumulates them."""
    from vq_dequant_matmul_gemv_amd import binding
    d, b, g = 2, 8, 64
    rows, cols = 40, 2 * 16 * 1030      # 1030 chunks per row
    spec, arrs, w = _case(d, b, g, rows, cols, ("wide",))
    for T in (1, 2):
        x = synth.activations((T, cols), "wide", T)
        announce("gemv-wide", T)
        y = binding.gemv(w, to_dev(x)).cpu().numpy()
        ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, cols, d, b, g)
        assert row_rel_err(y, ref) <= TOL


def test_gemv_multi_pass_rows():
    """Long rows covered in several column passes of equal width: narrower
    than the lane tile (idle lane slots), pass counts that divide the eight
    waves (each wave keeps one pass) and one that does not (x reloaded per
    item)."""
    from vq_dequant_matmul_gemv_amd import binding
    cases = [(41, 6400, 4, 8, 64),       # 100 chunks: 2 passes of 50 on 32 lanes x 2
             (37, 17408, 4, 8, 64),      # 272 chunks: 4 passes of 68 on 32 lanes x 3
             (23, 17408, 2, 8, 64),      # 544 chunks: 4 passes of 136 on 32 lanes x 5
             (29, 15360, 2, 8, 64),      # 480 chunks: 4 passes of 120 on 32 lanes x 5
             (19, 17408, 8, 12, 128)]    # 136 chunks: 5 passes of 28 on 32 lanes x 1
    for rows, cols, d, b, g in cases:
        spec, arrs, w = _case(d, b, g, rows, cols, ("passes", rows, cols))
        for T in (1, 2):
            x = synth.activations((T, cols), "passes", rows, cols, T)
            announce("gemv-passes", rows, cols, d, b, g, T)
            y = binding.gemv(w, to_dev(x)).cpu().numpy()
            ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, cols, d, b, g)
            assert row_rel_err(y, ref) <= TOL, (rows, cols, d, T)


def test_gemv_partial_last_rounds():
    """Blocks whose row groups leave a partial last round over the 8 waves
    (32 lanes x 5 chunks per row, 2-row groups): 2 and 7 groups left over
    (the latter with a 1-row last group), no whole round, an exact round."""
    from vq_dequant_matmul_gemv_amd import binding
    cases = [(5000, 5120),     # 19-20 rows per block: 10 groups, 2 left
             (7500, 5120),     # 29-30 rows: 15 groups, 7 left
             (2600, 5120),     # 10-11 rows: 5-6 groups, no whole round
             (4096, 5120)]     # 16 rows: 8 groups, none left
    for rows, cols in cases:
        spec, arrs, w = _case(2, 8, 64, rows, cols, ("rounds", rows, cols))
        for T in (1, 2):
            x = synth.activations((T, cols), "rounds", rows, cols, T)
            announce("gemv-rounds", rows, cols, T)
            y = binding.gemv(w, to_dev(x)).cpu().numpy()
            ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, cols, 2, 8, 64)
            assert row_rel_err(y, ref) <= TOL, (rows, cols, T)


@pytest.mark.parametrize("d,b,g", [(2, 8, 64), (4, 8, 64), (4, 12, 128), (8, 12, 128)])
def test_gemv_two_token_slices(d, b, g):
    """Two tokens per grid slice (rows whose x fits 16 KiB): each code and
    codebook entry read once for both tokens.  Matrices above 16M weights
    hand T = 2 to this path; odd token counts (a last slice of one token) go
    through the same kernel on smaller matrices.  fp32, fp16 and bf16
    outputs and the SwiGLU step."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    rows, cols = 3584, 5120            # 18.4M weights: T = 2 stays on the GEMV
    spec, arrs, w = _case(d, b, g, rows, cols, ("two-tok", d, b, g))
    x = synth.activations((2, cols), "two-tok", d, b, g)
    ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, cols, d, b, g)
    announce("gemv two-token", d, b, g)
    y = binding.gemv(w, to_dev(x)).cpu().numpy()
    assert row_rel_err(y, ref) <= TOL
    y16 = binding.gemv(w, to_dev(x), y_dtype=torch.float16).float().cpu().numpy()
    assert row_rel_err(y16, ref) <= TOL + 2.0 ** -11
    h = binding.gemv(w, to_dev(x), y_dtype=torch.bfloat16, epilogue="swiglu").float().cpu().numpy()
    assert row_rel_err(h, O.swiglu_ref(ref)) <= TOL + 2.0 ** -8
    # odd token counts on a matrix that keeps up to 6 tokens on the GEMV
    spec, arrs, w = _case(d, b, g, 301, 2048, ("two-tok-odd", d, b, g))
    for T in (3, 5):
        x = synth.activations((T, 2048), "two-tok-odd", d, b, g, T)
        announce("gemv two-token odd", d, b, g, T)
        y = binding.gemv(w, to_dev(x)).cpu().numpy()
        ref = O.gemv_ref(arrs["codes"][0], arrs["codebook"], arrs["scales"][0], x, 2048, d, b, g)
        assert row_rel_err(y, ref) <= TOL, T


def test_zero_tokens_is_a_no_op():
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    spec, arrs, w = _case(2, 8, 64, 8, 64, ("empty",))
    y = torch.full((0, 8), 7.0, device="cuda")
    binding.gemv(w, torch.zeros((0, 64), dtype=torch.float16, device="cuda"), y)
    binding.gemm(w, torch.zeros((0, 64), dtype=torch.float16, device="cuda"), y)


# ---------------------------------------------------------------------------
# routed experts
# ---------------------------------------------------------------------------

def _moe_ids(T, top_k, E, key):
    ids = synth.zipf_routing(T, E, top_k, *key) if E >= top_k else \
        synth.rng("ids", *key).integers(0, E, size=(T, top_k)).astype(np.int32)
    return ids


@pytest.mark.parametrize("fn", ["moe_gemv", "moe_gemm"])
@pytest.mark.parametrize("x_per_slot", [False, True])
@pytest.mark.parametrize("d,b,g", [(4, 8, 64), (8, 12, 128), (4, 12, 128), (2, 8, 64)])
def test_moe_matches_oracle(fn, x_per_slot, d, b, g):
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, top_k = 16, 96, _cols_for(d, g, 4), 4
    spec, arrs, w = _case(d, b, g, rows, cols, ("moe", d, b, g), experts=E)
    for T in (1, 3, 70):
        ids = _moe_ids(T, top_k, E, ("moe", T))
        ids[0, 1] = -1                     # skipped slot
        if T > 1:
            ids[1, 2] = E + 5              # out of range: skipped
            ids[2, 0] = ids[2, 3]          # duplicate within a token
        shape = (T, top_k, cols) if x_per_slot else (T, cols)
        x = synth.activations(shape, "moe", d, b, g, T)
        announce(fn, d, b, g, "xps", x_per_slot, "T", T)
        y = getattr(binding, fn)(w, to_dev(x), to_dev(ids), x_per_slot=x_per_slot).cpu().numpy()
        ref = O.moe_ref(arrs["codes"], arrs["codebook"], arrs["scales"], x, ids, cols=cols, d=d,
                        log2_k=b, group=g, x_per_slot=x_per_slot)
        assert np.all(y[0, 1] == 0)
        assert row_rel_err(y.reshape(-1, rows), ref.reshape(-1, rows)) <= TOL


def test_moe_per_expert_codebooks():
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, top_k, T = 5, 64, 256, 2, 9
    spec, arrs, w = _case(4, 8, 64, rows, cols, ("moe-cbpe",), experts=E, cbpe=True)
    ids = synth.rng("ids-cbpe").integers(0, E, size=(T, top_k)).astype(np.int32)
    x = synth.activations((T, cols), "moe-cbpe")
    ref = O.moe_ref(arrs["codes"], arrs["codebook"], arrs["scales"], x, ids, cols=cols, d=4,
                    log2_k=8, group=64, x_per_slot=False, codebook_per_expert=True)
    for fn in ("moe_gemv", "moe_gemm"):
        announce(fn, "cbpe")
        y = getattr(binding, fn)(w, to_dev(x), to_dev(ids)).cpu().numpy()
        assert row_rel_err(y.reshape(-1, rows), ref.reshape(-1, rows)) <= TOL


@pytest.mark.parametrize("rows,cols", [(17408, 512), (4352, 5120)])
def test_gate_up_stack_in_one_routed_call(rows, cols):
    """Two projections that share x (an MLP's gate and up), stored as a
    two-expert stack with per-expert codebooks, run as one routed GEMV with
    ids {0, 1}: at 17408 rows a block holds 136 rows (two pairs over the
    CUs); at 4352 x 5120 the blocks' row groups leave a partial last round.
    The outputs match the oracle and, bit for bit, two dense GEMV calls on
    the experts (same lane tiling per row)."""
    from vq_dequant_matmul_gemv_amd import binding
    spec, arrs, w = _case(2, 8, 64, rows, cols, ("gate-up", rows, cols), experts=2, cbpe=True)
    x = synth.activations((1, cols), "gate-up")
    ids = np.array([[0, 1]], dtype=np.int32)
    announce("gate-up stack", rows, cols)
    y = binding.moe_gemv(w, to_dev(x), to_dev(ids)).cpu().numpy()
    ref = O.moe_ref(arrs["codes"], arrs["codebook"], arrs["scales"], x, ids, cols=cols, d=2,
                    log2_k=8, group=64, x_per_slot=False, codebook_per_expert=True)
    assert row_rel_err(y.reshape(-1, rows), ref.reshape(-1, rows)) <= TOL
    for e in range(2):
        we = binding.VQTensor(w.codes[e], w.codebook[e], w.scales[e], rows, cols, 2, 8, 64)
        ye = binding.gemv(we, to_dev(x)).cpu().numpy()
        assert np.array_equal(ye[0], y[0, e]), e


def test_routed_gate_up_interleaved_in_one_call():
    """Routed gate and up projections (same x per token) stored as experts
    2e and 2e + 1 of one stack, run by one call with ids 2e, 2e + 1 (top_k
    doubled): bit for bit the two separate routed calls, GEMV and GEMM."""
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, top_k, T = 12, 96, 256, 3, 4
    specs = synth.Spec(rows=rows, cols=cols, d=4, log2_k=8, group=64, experts=E)
    g = synth.tensor(specs, "gu-routed", "gate")
    u = synth.tensor(specs, "gu-routed", "up")
    wg, wu = upload(g, specs), upload(u, specs)
    codes = torch.stack([wg.codes, wu.codes], 1).reshape(2 * E, rows, -1).contiguous()
    scales = torch.stack([wg.scales, wu.scales], 1).reshape(2 * E, rows, -1).contiguous()
    cbs = torch.stack([wg.codebook, wu.codebook]).repeat(E, 1, 1).contiguous()
    w2 = binding.VQTensor(codes, cbs, scales, rows, cols, 4, 8, 64, 2 * E, True)
    ids = synth.rng("ids-gu").integers(0, E, size=(T, top_k)).astype(np.int32)
    ids2 = np.stack([2 * ids, 2 * ids + 1], -1).reshape(T, 2 * top_k).astype(np.int32)
    x = to_dev(synth.activations((T, cols), "gu-routed"))
    announce("routed gate+up interleaved")
    yg = binding.moe_gemv(wg, x, to_dev(ids)).cpu().numpy()
    yu = binding.moe_gemv(wu, x, to_dev(ids)).cpu().numpy()
    y2 = binding.moe_gemv(w2, x, to_dev(ids2)).cpu().numpy()
    assert np.array_equal(y2[:, 0::2], yg) and np.array_equal(y2[:, 1::2], yu)
    # the grouped GEMM: a pair's row depends only on its expert and x row
    zg = binding.moe_gemm(wg, x, to_dev(ids)).cpu().numpy()
    zu = binding.moe_gemm(wu, x, to_dev(ids)).cpu().numpy()
    z2 = binding.moe_gemm(w2, x, to_dev(ids2)).cpu().numpy()
    assert np.array_equal(z2[:, 0::2], zg) and np.array_equal(z2[:, 1::2], zu)


def test_moe_gemm_more_experts_than_lds_counters():
    """8200 experts: the routing kernel keeps its per-expert counters in the
    workspace rather than in LDS (which holds 8192)."""
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, top_k, T = 8200, 32, 64, 4, 40
    spec, arrs, w = _case(2, 8, 64, rows, cols, ("moe-many",), experts=E)
    ids = synth.rng("ids-many").integers(0, E, size=(T, top_k)).astype(np.int32)
    ids[0, :] = 17                      # a hot expert with several slots
    ids[1, 2] = -1                      # skipped slot
    x = synth.activations((T, cols), "moe-many")
    announce("moe-many-experts", E)
    y = binding.moe_gemm(w, to_dev(x), to_dev(ids)).cpu().numpy()
    ref = O.moe_ref(arrs["codes"], arrs["codebook"], arrs["scales"], x, ids, cols=cols, d=2,
                    log2_k=8, group=64, x_per_slot=False)
    assert np.all(y[1, 2] == 0)
    assert row_rel_err(y.reshape(-1, rows), ref.reshape(-1, rows)) <= TOL


def test_moe_gemm_routing_beyond_one_pass():
    """The routing block keeps up to 16 pairs per thread (16 x 1024) in
    registers and places them in one pass; more pairs take the two-pass path
    with the same result.  2600 tokens x top-8 = 20800 pairs, skipped and out
    of range slots among them, and the same call at 2000 tokens (one pass):
    both match the oracle on a sample of pairs, and the pairs both calls share
    give the same rows bit for bit."""
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, top_k = 64, 64, 128, 8
    # exact-arithmetic inputs: a row's value does not depend on which tile
    # kind (32 or 128 tokens, whose k-steps group the columns differently)
    # the routing put its pair in, so shared pairs must agree bit for bit
    spec, arrs, w = _case(2, 8, 64, rows, cols, ("moe-2pass",), exact=True, experts=E)
    ys = {}
    for T in (2600, 2000):
        ids = _moe_ids(T, top_k, E, ("moe-2pass",))
        ids[5, 3] = -1
        ids[7, 1] = E + 2
        x = synth.activations((T, cols), "moe-2pass", exact=True)
        announce("moe-2pass", T, T * top_k)
        y = binding.moe_gemm(w, to_dev(x), to_dev(ids)).cpu().numpy()
        assert np.all(y[5, 3] == 0) and np.all(y[7, 1] == 0)
        pick = np.random.default_rng(T).choice(T, size=64, replace=False)
        ref = O.moe_ref(arrs["codes"], arrs["codebook"], arrs["scales"], x[pick], ids[pick], cols=cols, d=2,
                        log2_k=8, group=64, x_per_slot=False)
        assert row_rel_err(y[pick].reshape(-1, rows), ref.reshape(-1, rows)) <= TOL
        ys[T] = (y, ids)
    # the first 2000 tokens draw the same ids and x in both calls (seeded by key)
    y_big, ids_big = ys[2600]
    y_small, ids_small = ys[2000]
    same = np.all(ids_big[:2000] == ids_small, axis=1)
    assert same.sum() > 1000
    assert np.array_equal(y_big[:2000][same], y_small[same])


@pytest.mark.parametrize("d,b,g", [(2, 8, 64), (4, 8, 64), (4, 12, 128), (8, 12, 128)])
def test_moe_gemm_mixed_tile_kinds(d, b, g):
    """1024 tokens x top-8 over 992-row experts: enough 32-token units to
    fill the GPU twice, so hot experts get 128-token tiles (listed first)
    and the rest 32-token ones, and a last round at most half full runs as
    256-row halves.  Every output row against the oracle; skipped and
    out-of-range slots are zero rows."""
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, top_k, T = 32, 992, 512, 8, 1024
    spec, arrs, w = _case(d, b, g, rows, cols, ("moe-mix", d, b, g), experts=E)
    ids = hot_expert_ids(T, top_k, E, ("moe-mix", d, b, g))
    x = synth.activations((T, cols), "moe-mix", d, b, g)
    announce("moe-mix", d, b, g, rows, cols)
    y = binding.moe_gemm(w, to_dev(x), to_dev(ids)).cpu().numpy()
    ref = O.moe_ref(arrs["codes"], arrs["codebook"], arrs["scales"], x, ids, cols=cols, d=d, log2_k=b,
                    group=g, x_per_slot=False)
    assert np.all(y[900, 7] == 0) and np.all(y[901, 6] == 0)
    assert row_rel_err(y.reshape(-1, rows), ref.reshape(-1, rows)) <= TOL


def test_moe_gemm_mixed_tiles_place_rows_exactly():
    """The same routing on exact-arithmetic inputs: the grouped GEMM over
    mixed tile kinds and halves, the per-slot GEMV and the oracle agree bit
    for bit, so every pair's row lands where it belongs."""
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, top_k, T = 32, 992, 256, 8, 1024
    spec, arrs, w = _case(4, 8, 64, rows, cols, ("moe-mix-exact",), exact=True, experts=E)
    ids = hot_expert_ids(T, top_k, E, ("moe-mix-exact",))
    x = synth.activations((T, cols), "moe-mix-exact", exact=True)
    announce("moe-mix-exact")
    a = binding.moe_gemm(w, to_dev(x), to_dev(ids)).cpu().numpy()
    bgv = binding.moe_gemv(w, to_dev(x), to_dev(ids)).cpu().numpy()
    ref = O.moe_ref(arrs["codes"], arrs["codebook"], arrs["scales"], x, ids, cols=cols, d=4, log2_k=8, group=64,
                    x_per_slot=False)
    assert np.array_equal(a, bgv)
    assert np.array_equal(a.astype(np.float64), ref)


def test_moe_grouped_equals_per_slot_bit_identical_on_exact_inputs():
    """Grouping by expert does not change any row: on exact-arithmetic
    inputs grouped GEMM, per-slot GEMV and the oracle agree bit for bit."""
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, top_k, T = 32, 128, 512, 8, 100
    spec, arrs, w = _case(4, 8, 64, rows, cols, ("moe-exact",), exact=True, experts=E)
    ids = synth.zipf_routing(T, E, top_k, "moe-exact")
    x = synth.activations((T, cols), "moe-exact", exact=True)
    announce("moe-exact")
    a = binding.moe_gemm(w, to_dev(x), to_dev(ids)).cpu().numpy()
    bgv = binding.moe_gemv(w, to_dev(x), to_dev(ids)).cpu().numpy()
    ref = O.moe_ref(arrs["codes"], arrs["codebook"], arrs["scales"], x, ids, cols=cols, d=4,
                    log2_k=8, group=64, x_per_slot=False)
    assert np.array_equal(a, bgv)
    assert np.array_equal(a.astype(np.float64), ref)


def test_moe_all_slots_skipped_and_repeat_runs_identical():
    import torch
    from vq_dequant_matmul_gemv_amd import binding
    E, rows, cols, top_k, T = 8, 64, 256, 2, 33
    spec, arrs, w = _case(2, 8, 64, rows, cols, ("moe-skip",), experts=E)
    x = to_dev(synth.activations((T, cols), "moe-skip"))
    ids = torch.full((T, top_k), -1, dtype=torch.int32, device="cuda")
    for fn in ("moe_gemv", "moe_gemm"):
        announce(fn, "all-skipped")
        y = torch.full((T, top_k, rows), 3.0, device="cuda")
        getattr(binding, fn)(w, x, ids, y=y)
        assert torch.count_nonzero(y).item() == 0
    ids = to_dev(synth.zipf_routing(T, E, top_k, "moe-rep"))
    outs = [binding.moe_gemm(w, x, ids).cpu().numpy() for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
