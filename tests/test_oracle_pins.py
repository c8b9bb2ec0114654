"""Pins for the CPU oracle: each checks it against something other than itself.

* closed forms the pages print (bits per weight, byte counts),
* hand-derived packed words (tests/golden/packed_words_hand.txt),
* the pages' statement that uint8 codes already are the packed-8 layout,
* an independent IEEE binary16 round-to-nearest-even routine (integer
  arithmetic on exact fractions, not numpy's float16),
* brute force with exact rational arithmetic on tiny tensors,
* textbook invariants (one-hot columns, linearity, permutation, MoE routing).
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import vq_oracle as O
from vq_dequant_matmul_gemv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GEOMS = [(d, b, g) for d in (2, 4, 8) for b in (8, 12) for g in (64, 128)]
# the other code widths (K = 16 ... 16384), one group size each
GEOMS_WIDE = [(d, b, 64 if (b + d) % 2 else 128) for d in (2, 4, 8) for b in (4, 5, 9, 10, 11, 13, 14)]


# --------------------------------------------------------------------------
# independent helpers (no numpy float16, no shifts into words)
# --------------------------------------------------------------------------

def f16_bits_to_fraction(h: int) -> Fraction:
    """Value of a finite binary16 bit pattern, from the IEEE 754 definition."""
    sign = -1 if h >> 15 else 1
    exp = (h >> 10) & 0x1F
    man = h & 0x3FF
    assert exp != 0x1F
    if exp == 0:
        return sign * Fraction(man, 1 << 24)
    return sign * Fraction(1024 + man, 1024) * Fraction(2) ** (exp - 15)


def round_to_f16(v: Fraction) -> Fraction:
    """Round an exact rational to binary16, ties to even (inf on overflow)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -14) - 10)          # spacing of binary16 near a
    n = a / q
    m = n.numerator // n.denominator
    rem = n - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    r = m * q
    if r >= 65520:                                   # beyond max finite half
        return sign * Fraction(10 ** 9)
    return sign * r


def bitstring_codes(words_row, n_codes, bits):
    """Codes from a row of words via a '0'/'1' string, least significant bit first."""
    s = "".join(format(int(w), "032b")[::-1] for w in words_row)
    return [int(s[j * bits:(j + 1) * bits][::-1], 2) for j in range(n_codes)]


def bitstring_pack(codes, bits):
    s = "".join(format(c, f"0{bits}b")[::-1] for c in codes)
    assert len(s) % 32 == 0
    return [int(s[i:i + 32][::-1], 2) for i in range(0, len(s), 32)]


def _f16(a):
    return np.asarray(a, dtype=np.float16)


# --------------------------------------------------------------------------
# P-1: sizes
# --------------------------------------------------------------------------

def _golden_bpw():
    rows = []
    with open(os.path.join(GOLDEN, "bits_per_weight.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            d, k, g, bpw = line.split()[:4]
            rows.append((int(d), int(k), None if g == "-" else int(g), float(bpw)))
    return rows


@pytest.mark.parametrize("d,k,g,bpw", _golden_bpw())
def test_bits_per_weight_matches_pages(d, k, g, bpw):
    assert O.bits_per_weight(d, int(math.log2(k)), g) == pytest.approx(bpw, abs=1e-12)


def test_group128_scale_overhead_and_tier_mix():
    # "+0.125 bpw" for fp16 group scales (aquaman164 card, Recipe) -> g = 128
    assert O.bits_per_weight(4, 8, 128) - O.bits_per_weight(4, 8, None) == 0.125
    # 51 tensors at 1.5 bit, 13 at 2 bit, 16 at 3 bit: "2.0 bpw effective" with scales
    mix = (51 * O.bits_per_weight(8, 12, None) + 13 * O.bits_per_weight(4, 8, None)
           + 16 * O.bits_per_weight(4, 12, None)) / 80
    assert abs(mix + 0.125 - 2.0) < 0.01


@pytest.mark.parametrize("rows,cols,d,b,g", [
    (17408, 5120, 2, 8, 64), (5120, 17408, 2, 8, 64), (17408, 5120, 4, 8, 64),
    (5120, 17408, 4, 8, 64), (1024, 4096, 4, 8, 64), (512, 2048, 8, 12, 128),
    (2048, 512, 4, 12, 128), (1024, 1024, 2, 8, 64)])
def test_byte_counts_equal_closed_form(rows, cols, d, b, g):
    total_bits = O.bits_per_weight(d, b, g) * rows * cols
    assert (O.code_bytes(rows, cols, d, b) + O.scale_bytes(rows, cols, g)) * 8 == total_bits
    assert O.code_bytes(rows, cols, d, b) == rows * cols * b // d // 8


def test_dense_trio_byte_counts():
    # gate/up [17408][5120], d2/K256/g64: 47,349,760 B of codes + scales each
    per = O.code_bytes(17408, 5120, 2, 8) + O.scale_bytes(17408, 5120, 64)
    assert per == 47_349_760
    assert O.code_bytes(17408, 5120, 4, 8) == 22_282_240


def _golden_cb():
    rows = []
    with open(os.path.join(GOLDEN, "codebook_bytes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            d, k, nbytes = line.split()[:3]
            rows.append((int(d), int(k), int(nbytes)))
    return rows


@pytest.mark.parametrize("d,k,nbytes", _golden_cb())
def test_codebook_bytes_matches_pages(d, k, nbytes):
    assert O.codebook_bytes(d, int(math.log2(k))) == nbytes


def test_codebook_bytes_threadgroup_thresholds_and_staging_sizes():
    # paper §3.1: a d4 codebook above K = 2048 and a d2 codebook above K = 4096
    # outgrow the 32 KB threadgroup memory; the two thresholds are the same size
    # (d * K equal) and the next codebook of either kind reaches 32 KB.
    limit = 32 * 1024
    assert O.codebook_bytes(4, 11) == O.codebook_bytes(2, 12) < limit
    assert O.codebook_bytes(4, 12) >= limit and O.codebook_bytes(2, 13) >= limit
    # the staging sizes of the geometries the kernels hold in LDS
    assert O.codebook_bytes(2, 8) == 1024 and O.codebook_bytes(4, 8) == 2048
    assert O.codebook_bytes(4, 12) == 32 * 1024 and O.codebook_bytes(8, 12) == 64 * 1024
    # one codebook per expert: E times one tensor's
    assert O.codebook_bytes(4, 8, n_codebooks=256) == 256 * O.codebook_bytes(4, 8)
    # the codebook a synthetic tensor carries has exactly that many bytes
    for d, b in ((2, 8), (4, 12), (8, 12)):
        spec = synth.Spec(rows=4, cols=32 * d, d=d, log2_k=b, group=64 if d < 8 else 128)
        assert synth.tensor(spec, "cb-bytes", d, b)["codebook"].nbytes == O.codebook_bytes(d, b)


def test_words_per_row_pads_to_whole_blocks():
    assert O.words_per_row(64, 2, 8) == 8          # exactly one 32-code block
    assert O.words_per_row(66, 2, 8) == 16         # 33 codes -> 2 blocks
    assert O.words_per_row(2048, 8, 12) == 96


# --------------------------------------------------------------------------
# P-2 / P-3: packing layout
# --------------------------------------------------------------------------

def _golden_words():
    """name -> (bits, words) from the fixture; the code spec column is
    documentation only (the codes are rebuilt by _golden_codes)."""
    out = {}
    with open(os.path.join(GOLDEN, "packed_words_hand.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            toks = line.split()
            words = [t for t in toks[2:] if len(t) == 8 and all(ch in "0123456789abcdef" for ch in t)]
            out[toks[0]] = (int(toks[1]), [int(w, 16) for w in words])
    return out


def _golden_codes(name):
    if name == "ramp8":
        return list(range(32))
    if name == "alt12":
        return [0xABC, 0x123] * 16
    if name == "ones12":
        return [0xFFF] * 32
    if name == "ramp12":
        return list(range(32))
    raise KeyError(name)


@pytest.mark.parametrize("name", ["ramp8", "alt12", "ones12", "ramp12"])
def test_hand_packed_words(name):
    bits, words = _golden_words()[name]
    codes = _golden_codes(name)
    packed = O.pack_codes(np.array([codes]), bits)[0]
    assert [int(w) for w in packed[:len(words)]] == words
    # bit-string construction agrees on the whole block
    assert [int(w) for w in packed] == bitstring_pack(codes, bits)
    # and the oracle's unpack inverts it
    d = 4
    assert O.unpack_codes(packed[None], 32 * d, d, bits)[0].tolist() == codes


def test_uint8_codes_are_the_packed8_layout():
    g = np.random.default_rng(7)
    codes = g.integers(0, 256, size=(5, 64), dtype=np.uint8)        # [rows][cols/d]
    words = codes.view("<u4")                                         # zero-copy view
    assert np.array_equal(O.unpack_codes(words, 64 * 2, 2, 8), codes)
    assert np.array_equal(O.pack_codes(codes, 8), words)


@pytest.mark.parametrize("bits", list(range(4, 15)))
def test_unpack_matches_bitstring_on_random_words(bits):
    g = np.random.default_rng(bits)
    d = 4
    words = g.integers(0, 1 << 32, size=(3, 2 * bits), dtype=np.uint32)   # 2 blocks per row
    codes = O.unpack_codes(words, 64 * d, d, bits)
    for r in range(3):
        assert codes[r].tolist() == bitstring_codes(words[r], 64, bits)


@pytest.mark.parametrize("bits", [4, 5, 7, 9, 10, 11, 13, 14])
def test_pack_matches_bitstring_construction_other_widths(bits):
    """Codes of every width the kernels take (paper §1 Notation: builds from
    d2/K16 to d4/K16384), packed by the oracle and by the independent
    bit-string construction: ramps, all ones, and random codes."""
    g = np.random.default_rng(100 + bits)
    for codes in ([j % (1 << bits) for j in range(32)], [(1 << bits) - 1] * 32,
                  g.integers(0, 1 << bits, size=64).tolist()):
        packed = O.pack_codes(np.array([codes]), bits)[0]
        assert [int(w) for w in packed] == bitstring_pack(codes, bits)
        assert len(packed) == len(codes) // 32 * bits
        d = 2
        assert O.unpack_codes(packed[None], len(codes) * d, d, bits)[0].tolist() == codes


def test_pack_unpack_roundtrip_property():
    hyp = pytest.importorskip("hypothesis")
    st = pytest.importorskip("hypothesis.strategies")

    @hyp.settings(max_examples=60, deadline=None)
    @hyp.given(bits=st.sampled_from([8, 12]), blocks=st.integers(1, 3), rows=st.integers(1, 3),
               seed=st.integers(0, 2 ** 32 - 1))
    def prop(bits, blocks, rows, seed):
        g = np.random.default_rng(seed)
        codes = g.integers(0, 1 << bits, size=(rows, 32 * blocks))
        words = O.pack_codes(codes, bits)
        assert words.shape == (rows, blocks * bits)
        assert np.array_equal(O.unpack_codes(words, 32 * blocks * 2, 2, bits), codes)

    prop()


# --------------------------------------------------------------------------
# P-4: dequant rounding
# --------------------------------------------------------------------------

def _dequant_one(cb_bits, s_bits, d=2):
    """Dequant a single weight through the oracle: 1-row tensor, code 0."""
    cb = np.zeros((256, d), dtype=np.uint16)
    cb[0, 0] = cb_bits
    cb = cb.view(np.float16)
    scales = np.array([[s_bits]], dtype=np.uint16).view(np.float16)
    words = np.zeros((1, 8), dtype=np.uint32)
    return int(O.dequant(words, cb, scales, 64, d, 8, 64).view(np.uint16)[0, 0])


def _finite_f16_patterns():
    h = np.arange(1 << 16, dtype=np.uint32)
    return h[((h >> 10) & 0x1F) != 0x1F]


def test_dequant_rounding_against_independent_binary16():
    g = np.random.default_rng(11)
    pats = _finite_f16_patterns()
    subn = pats[((pats >> 10) & 0x1F) == 0]
    cbs = np.concatenate([g.choice(pats, 48), g.choice(subn, 16)]).astype(np.uint16)
    ss = np.concatenate([g.choice(pats, 48), g.choice(subn, 16),
                         np.array([0x3800, 0x3C00, 0x3E00, 0x0001, 0x8001, 0x7BFF])]).astype(np.uint16)
    # vectorised: one tensor with many rows, each row a (cb, scale) pair
    n = len(cbs) * len(ss)
    cb_pairs = np.repeat(cbs, len(ss))
    s_pairs = np.tile(ss, len(cbs))
    d, K = 2, 256
    codebook = np.zeros((K, d), dtype=np.uint16)
    words = np.zeros((n, 8), dtype=np.uint32)
    # put each pair's codebook value at entry (i % 256) and point code 0 of row i at it
    out = []
    for base in range(0, n, K):
        m = min(K, n - base)
        codebook[:m, 0] = cb_pairs[base:base + m]
        w = np.zeros((m, 8), dtype=np.uint32)
        w[:, 0] = np.arange(m, dtype=np.uint32)         # code 0 = i (8-bit, byte 0)
        sc = np.repeat(s_pairs[base:base + m, None], 1, axis=1).view(np.float16)
        out.append(O.dequant(w, codebook.view(np.float16), sc, 64, d, 8, 64).view(np.uint16)[:, 0])
    got = np.concatenate(out)
    for i in range(n):
        a = f16_bits_to_fraction(int(cb_pairs[i]))
        b = f16_bits_to_fraction(int(s_pairs[i]))
        want = round_to_f16(a * b)
        gv = int(got[i])
        if abs(want) >= 10 ** 9:
            assert (gv & 0x7FFF) == 0x7C00, (hex(cb_pairs[i]), hex(s_pairs[i]))
        else:
            assert f16_bits_to_fraction(gv) == want, (hex(cb_pairs[i]), hex(s_pairs[i]), hex(gv))
            if want == 0:   # sign of an exact zero follows the product's sign
                assert (gv >> 15) == ((int(cb_pairs[i]) ^ int(s_pairs[i])) >> 15)


def test_dequant_rounding_all_scale_patterns():
    # every finite scale pattern against a few codebook values incl. a subnormal
    pats = _finite_f16_patterns().astype(np.uint16)
    for cb_bits in (0x2A66, 0x0155, 0xB3FF, 0x3C01):
        a = f16_bits_to_fraction(cb_bits)
        rows = len(pats)
        codebook = np.zeros((256, 2), dtype=np.uint16)
        codebook[0, 0] = cb_bits
        words = np.zeros((rows, 8), dtype=np.uint32)
        got = O.dequant(words, codebook.view(np.float16), pats[:, None].view(np.float16),
                        64, 2, 8, 64).view(np.uint16)[:, 0]
        # exact products checked against the independent rounding on a sample,
        # all of them against float64-product rounding through numpy
        want64 = (np.float64(np.uint16(cb_bits).view(np.float16)) *
                  pats.view(np.float16).astype(np.float64)).astype(np.float16).view(np.uint16)
        assert np.array_equal(got, want64)
        for i in np.random.default_rng(cb_bits).choice(rows, 300, replace=False):
            want = round_to_f16(a * f16_bits_to_fraction(int(pats[i])))
            if abs(want) < 10 ** 9:
                assert f16_bits_to_fraction(int(got[i])) == want


def test_dequant_gather_recovers_codes():
    """Distinct codebook entries + unit scales: reading W back through the
    codebook gives the codes that the bit-string unpack gives."""
    for d, b, g in [(2, 8, 64), (4, 12, 128), (8, 12, 64), (4, 8, 128)]:
        K = 1 << b
        rng = np.random.default_rng(d * 100 + b)
        # distinct finite positive fp16 patterns per (entry, component)
        pool = np.concatenate([np.arange(0x0400, 0x7C00), np.arange(0x8400, 0xFC00)]).astype(np.uint16)
        pats = rng.choice(pool, size=K * d, replace=False)
        cb = pats.reshape(K, d).view(np.float16)
        cols = 32 * d * 2
        words = rng.integers(0, 1 << 32, size=(3, O.words_per_row(cols, d, b)), dtype=np.uint32)
        scales = np.ones((3, cols // g), dtype=np.float16)
        w = O.dequant(words, cb, scales, cols, d, b, g).view(np.uint16)
        lookup = {int(p): (i // d, i % d) for i, p in enumerate(pats)}
        for r in range(3):
            ref_codes = bitstring_codes(words[r], cols // d, b)
            for c in range(cols):
                e, t = lookup[int(w[r, c])]
                assert (e, t) == (ref_codes[c // d], c % d)


@pytest.mark.parametrize("g", [64, 128])
def test_dequant_scale_groups(g):
    """Unit codebook: row r of W is each scale repeated over its g weights."""
    rng = np.random.default_rng(g)
    d, b, cols, rows = 4, 8, 512, 3
    cb = np.ones((256, d), dtype=np.float16)
    scales = rng.uniform(0.5, 1.5, size=(rows, cols // g)).astype(np.float16)
    words = rng.integers(0, 1 << 32, size=(rows, O.words_per_row(cols, d, b)), dtype=np.uint32)
    w = O.dequant(words, cb, scales, cols, d, b, g)
    for r in range(rows):
        for c in range(cols):
            assert w[r, c] == scales[r, c // g]


# --------------------------------------------------------------------------
# P-5 .. P-10: matmul, exactness, invariants, brute force
# --------------------------------------------------------------------------

def brute_force(words, codebook, scales, x, cols, d, b, g):
    """Pure-Python reference with exact rational arithmetic throughout."""
    rows = words.shape[0]
    cbb = np.asarray(codebook, dtype=np.float16).reshape(-1, d).view(np.uint16)
    sb = np.asarray(scales, dtype=np.float16).view(np.uint16)
    xb = np.asarray(x, dtype=np.float16).view(np.uint16)
    out = []
    for t in range(x.shape[0]):
        yrow = []
        for r in range(rows):
            codes = bitstring_codes(words[r], cols // d, b)
            acc = Fraction(0)
            for c in range(cols):
                w = round_to_f16(f16_bits_to_fraction(int(cbb[codes[c // d], c % d])) *
                                 f16_bits_to_fraction(int(sb[r, c // g])))
                acc += w * f16_bits_to_fraction(int(xb[t, c]))
            yrow.append(acc)
        out.append(yrow)
    return out


@pytest.mark.parametrize("d,b,g", GEOMS + GEOMS_WIDE)
def test_brute_force_all_geometries(d, b, g):
    spec = synth.Spec(rows=3, cols=max(32 * d, g) * (1 if d == 8 else 2), d=d, log2_k=b, group=g)
    t = synth.tensor(spec, "pin-bf", d, b, g)
    x = synth.activations((2, spec.cols), "pin-bf", d, b, g)
    ref = O.gemv_ref(t["codes"][0], t["codebook"], t["scales"][0], x, spec.cols, d, b, g)
    bf = brute_force(t["codes"][0], t["codebook"], t["scales"][0], x, spec.cols, d, b, g)
    for ti in range(2):
        for r in range(3):
            exact = float(bf[ti][r])
            assert abs(ref[ti, r] - exact) <= 1e-12 * max(1.0, abs(exact))


def test_exact_inputs_give_exact_outputs():
    spec = synth.Spec(rows=4, cols=256, d=4, log2_k=8, group=64)
    t = synth.tensor(spec, "pin-exact", exact=True)
    x = synth.activations((3, spec.cols), "pin-exact", exact=True)
    ref = O.gemv_ref(t["codes"][0], t["codebook"], t["scales"][0], x, 256, 4, 8, 64)
    bf = brute_force(t["codes"][0], t["codebook"], t["scales"][0], x, 256, 4, 8, 64)
    for ti in range(3):
        for r in range(4):
            assert Fraction(ref[ti, r]) == bf[ti][r]
            assert float(np.float32(ref[ti, r])) == ref[ti, r]     # representable in fp32


def test_one_hot_x_selects_columns_and_ones_give_row_sums():
    spec = synth.Spec(rows=5, cols=128, d=2, log2_k=8, group=64)
    t = synth.tensor(spec, "pin-onehot")
    w = O.dequant(t["codes"][0], t["codebook"], t["scales"][0], 128, 2, 8, 64)
    eye = np.eye(128, dtype=np.float16)
    y = O.gemv_ref(t["codes"][0], t["codebook"], t["scales"][0], eye, 128, 2, 8, 64)
    assert np.array_equal(y, w.astype(np.float64).T)
    ones = np.ones((1, 128), dtype=np.float16)
    y1 = O.gemv_ref(t["codes"][0], t["codebook"], t["scales"][0], ones, 128, 2, 8, 64)
    for r in range(5):
        assert y1[0, r] == pytest.approx(math.fsum(float(v) for v in w[r]), rel=1e-14, abs=1e-14)


def test_matmul_matches_triple_loop():
    rng = np.random.default_rng(3)
    w = rng.normal(size=(4, 64)).astype(np.float16)
    x = rng.normal(size=(3, 64)).astype(np.float16)
    y = O.matmul_f64(w, x)
    for t in range(3):
        for r in range(4):
            exact = sum(Fraction(float(w[r, c])) * Fraction(float(x[t, c])) for c in range(64))
            assert abs(y[t, r] - float(exact)) <= 1e-13


def test_linearity_powers_of_two():
    spec = synth.Spec(rows=6, cols=256, d=2, log2_k=8, group=64)
    t = synth.tensor(spec, "pin-lin")
    x = synth.activations((2, 256), "pin-lin")
    y = O.gemv_ref(t["codes"][0], t["codebook"], t["scales"][0], x, 256, 2, 8, 64)
    y2 = O.gemv_ref(t["codes"][0], t["codebook"], t["scales"][0], (x * 2).astype(np.float16),
                    256, 2, 8, 64)
    assert np.array_equal(y2, 2 * y)
    s2 = (t["scales"][0].astype(np.float32) * 2).astype(np.float16)
    y3 = O.gemv_ref(t["codes"][0], t["codebook"], s2, x, 256, 2, 8, 64)
    assert np.array_equal(y3, 2 * y)


def _moe_case(x_per_slot, E=4, T=5, top_k=2, seed="pin-moe"):
    spec = synth.Spec(rows=8, cols=128, d=4, log2_k=8, group=64, experts=E)
    t = synth.tensor(spec, seed)
    shape = (T, top_k, 128) if x_per_slot else (T, 128)
    x = synth.activations(shape, seed)
    return spec, t, x


@pytest.mark.parametrize("x_per_slot", [False, True])
def test_moe_equals_dense_per_slot(x_per_slot):
    spec, t, x = _moe_case(x_per_slot)
    ids = np.array([[0, 3], [1, 1], [2, -1], [4, 0], [3, 2]], dtype=np.int32)   # dup, skip, out-of-range
    ref = O.moe_ref(t["codes"], t["codebook"], t["scales"], x, ids, cols=128, d=4, log2_k=8,
                    group=64, x_per_slot=x_per_slot)
    for ti in range(5):
        for s in range(2):
            e = ids[ti, s]
            xr = x[ti, s] if x_per_slot else x[ti]
            if 0 <= e < 4:
                want = O.gemv_ref(t["codes"][e], t["codebook"], t["scales"][e], xr[None], 128, 4, 8, 64)[0]
            else:
                want = np.zeros(8)
            assert np.array_equal(ref[ti, s], want)


def test_moe_all_same_expert_is_dense_and_permutes_with_tokens():
    spec, t, x = _moe_case(False, T=6, top_k=1)
    ids = np.full((6, 1), 2, dtype=np.int32)
    ref = O.moe_ref(t["codes"], t["codebook"], t["scales"], x, ids, cols=128, d=4, log2_k=8,
                    group=64, x_per_slot=False)
    dense = O.gemv_ref(t["codes"][2], t["codebook"], t["scales"][2], x, 128, 4, 8, 64)
    assert np.array_equal(ref[:, 0], dense)
    perm = np.array([3, 1, 5, 0, 2, 4])
    ref_p = O.moe_ref(t["codes"], t["codebook"], t["scales"], x[perm], ids, cols=128, d=4,
                      log2_k=8, group=64, x_per_slot=False)
    assert np.array_equal(ref_p, ref[perm])


def test_moe_per_expert_codebooks():
    spec = synth.Spec(rows=4, cols=64, d=2, log2_k=8, group=64, experts=3)
    t = synth.tensor(spec, "pin-cbpe", codebook_per_expert=True)
    x = synth.activations((2, 64), "pin-cbpe")
    ids = np.array([[2, 0], [1, 2]], dtype=np.int32)
    ref = O.moe_ref(t["codes"], t["codebook"], t["scales"], x, ids, cols=64, d=2, log2_k=8,
                    group=64, x_per_slot=False, codebook_per_expert=True)
    for ti in range(2):
        for s in range(2):
            e = ids[ti, s]
            want = O.gemv_ref(t["codes"][e], t["codebook"][e], t["scales"][e], x[ti][None], 64, 2, 8, 64)
            assert np.array_equal(ref[ti, s], want[0])


# --------------------------------------------------------------------------
# bf16 activations, SwiGLU and the router-weighted combine
# --------------------------------------------------------------------------

def _bf16_value_from_fields(h: int) -> float:
    """Value of a bf16 pattern from its fields (1 sign, 8 exponent, 7
    mantissa bits, bias 127), written from the format's definition."""
    sign = -1.0 if h >> 15 else 1.0
    exp = (h >> 7) & 0xFF
    man = h & 0x7F
    if exp == 0xFF:
        return sign * math.inf if man == 0 else math.nan
    if exp == 0:
        return sign * math.ldexp(man, -133)          # subnormal: man * 2^(1 - 127 - 7)
    return sign * math.ldexp(128 + man, exp - 134)   # (1 + man/128) * 2^(exp - 127)


def test_bf16_values_from_the_format_definition():
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_to_f64(pats)
    want = np.array([_bf16_value_from_fields(int(h)) for h in pats])
    finite = ~np.isnan(want)
    assert np.array_equal(got[finite], want[finite])
    assert np.all(np.isnan(got[~finite]))
    assert O.bf16_to_f64([0x3F80, 0xC040, 0x4049])[:].tolist() == [1.0, -3.0, 3.140625]


def test_silu_closed_forms():
    assert O.silu(0.0) == 0.0
    assert O.silu(1.0) == pytest.approx(1.0 / (1.0 + 1.0 / math.e), rel=1e-15)
    x = np.linspace(-30, 30, 601)
    # sigma(x) + sigma(-x) = 1, so silu(x) - silu(-x) = x
    assert np.allclose(O.silu(x) - O.silu(-x), x, rtol=0, atol=1e-13)
    assert O.silu(60.0) == 60.0 and 0 > O.silu(-60.0) > -1e-24
    from scipy.special import expit                  # an independent logistic routine
    assert np.allclose(O.silu(x), x * expit(x), rtol=1e-14, atol=1e-300)


def test_swiglu_pairs_interleaved_gate_and_up_rows():
    # rows: gate0, up0, gate1, up1 -> silu(gate_i) * up_i
    y = np.array([[0.0, 5.0, 2.0, -1.0], [-3.0, 0.5, 1.0, 4.0]])
    s2 = 2.0 / (1.0 + math.exp(-2.0))
    want = np.array([[0.0, -s2], [-3.0 / (1.0 + math.exp(3.0)) * 0.5, 4.0 / (1.0 + math.exp(-1.0))]])
    assert np.allclose(O.swiglu_ref(y), want, rtol=1e-15, atol=0)
    # gate and up are not interchangeable
    assert not np.allclose(O.swiglu_ref(y[:, [1, 0, 3, 2]]), want)


def test_moe_combine_brute_force_and_skips():
    rng = synth.rng("pin-combine")
    T, k, rows, E = 5, 3, 7, 4
    y = rng.normal(size=(T, k, rows))
    w = rng.uniform(0, 1, size=(T, k))
    ids = rng.integers(0, E, size=(T, k))
    ids[1, 2] = -1
    ids[3, 0] = E                                   # out of range
    want = np.zeros((T, rows))
    for t in range(T):
        for s in range(k):
            if 0 <= ids[t, s] < E:
                for r in range(rows):
                    want[t, r] += w[t, s] * y[t, s, r]
    assert np.allclose(O.moe_combine_ref(y, w, ids, E), want, rtol=1e-14, atol=1e-14)
    # the slot order does not matter
    perm = [2, 0, 1]
    assert np.allclose(O.moe_combine_ref(y[:, perm], w[:, perm], ids[:, perm], E), want, rtol=1e-14, atol=1e-14)


def test_moe_combine_of_routed_dense_rows():
    """Every slot of a token on one expert with weights summing to one: the
    combine is that expert's dense product."""
    spec = synth.Spec(rows=12, cols=64, d=2, log2_k=8, group=64, experts=3)
    a = synth.tensor(spec, "pin-combine-dense")
    x = synth.activations((4, 64), "pin-combine-dense")
    ids = np.full((4, 2), 1)
    w = np.array([[0.25, 0.75]] * 4)
    ys = O.moe_ref(a["codes"], a["codebook"], a["scales"], x, ids, cols=64, d=2, log2_k=8, group=64,
                   x_per_slot=False)
    dense = O.gemv_ref(a["codes"][1], a["codebook"], a["scales"][1], x, 64, 2, 8, 64)
    assert np.allclose(O.moe_combine_ref(ys, w, ids, 3), dense, rtol=1e-14, atol=1e-14)
