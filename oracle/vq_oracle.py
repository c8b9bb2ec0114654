"""Plain CPU oracle for the fused vector-quantized (VQ) weight matmul.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library, its C ABI
or its Python binding) imports, links or calls this module.  Only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code with the GPU path: it does not know about LDS, tiles,
chunks or launch shapes, only about what the format means.

Sources (web pages; cited by title and section):

* [paper]   "Data-Free Vector Quantization Beats Affine Quantization at Matched
            Bytes Below 5 Bits" (N. Zelezny, 2026): Abstract, §1 Notation,
            §2.2 The fit, §2.3 Packing, §3.1, §3.4.
* [397B]    model card "Qwen3.5-397B-A17B-VQ-2.4bpw": Methodology (one 8-bit
            index per 4-weight subvector into a per-tensor 256-entry fp16
            codebook, fp16 scale per (row, 64 weights), codes packed into
            uint32 words in row-local 32-code blocks); Runtime update
            (8-bit codes are already in the packed-8 layout, zero copy).
* [27B-4.5] model card "Qwen3.8-27B-VQ-4.5bpw": How it was built (d=2, K=256,
            4.25 bits per weight).
* [27B-3.9] model card "Qwen3.8-27B-VQ-3.9bpw": How it was built (d=4,
            K=4096, 12-bit indices, 3.25 bits per weight).
* [35B-aq]  model card "aquaman164/Qwen3.6-35B-A3B-MLX-VQ-2.4bpw": Recipe
            (tiers d8/K4096, d4/K256, d4/K4096 with packed 8/12-bit indices
            and fp16 group scales adding 0.125 bpw, i.e. one per 128).

What it computes, in the pages' notation (dN/KM: subvector length d, codebook
size K, B = log2 K bits per code; W is [rows = out][cols = in]):

1. unpack: code j of row r is bits [j*B, (j+1)*B) of that row's code stream,
   read as a little-endian bit string (least significant bit first).  A row's
   stream is ceil(cols/d/32) blocks of 32 codes, each block exactly B uint32
   words, so rows start on a word boundary (each row packed on its own in
   blocks of 32 codes).
2. dequant: W[r][j*d + t] = f16( f32(codebook[code][t]) * f32(scale[r][c // g]) )
   with c = j*d + t.  The fp32 product of two fp16 values is exact, so this
   is one round-to-nearest-even to fp16, the same as an IEEE fp16 multiply.
3. matmul: ref[t][r] = sum_c f64(W[r][c]) * f64(x[t][c]) in float64.
4. MoE: ref[t][s] = W_e @ xrow for e = ids[t][s] when 0 <= e < E, where xrow
   is x[t] (shared input) or x[t][s] (per-slot input); otherwise a zero row.
5. bf16 activations ([paper] §7 Reproducibility: the scored runtime profile
   takes and returns bf16): a bf16 bit pattern is the upper half of an IEEE
   binary32 value; the matmul uses that value exactly.
6. SwiGLU on the MLP trio's gate and up outputs ([paper] §2.1: the gate, up
   and down projections; the activation is not on the pages, SiLU gating is
   the reading): h_i = silu(g_i) * u_i, silu(g) = g / (1 + exp(-g)), with the
   gate and up rows interleaved (row 2i gate, row 2i + 1 up) in one tensor.
7. Router-weighted top-k combine: out[t] = sum over the valid slots s of
   weights[t][s] * ref[t][s].

Readings where the pages are silent (the plainest the rest supports):
  d consecutive weights run along the input dimension of one output row;
  scale index c // g; LSB-first bit order (pinned by the pages only for 8-bit:
  a uint8 array *is* the packed layout); codebook stored entry-major [K][d];
  one rounding to fp16 in the dequant; out-of-range expert ids give zeros.

Parity status: every public function here is pinned by tests/test_oracle_pins.py
against something other than itself (closed forms, hand-packed words, an
independent binary16 rounding routine, brute force, textbook invariants).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "words_per_row",
    "code_bytes",
    "scale_bytes",
    "codebook_bytes",
    "bits_per_weight",
    "pack_codes",
    "unpack_codes",
    "dequant",
    "matmul_f64",
    "gemv_ref",
    "moe_ref",
    "bf16_to_f64",
    "silu",
    "swiglu_ref",
    "moe_combine_ref",
    "ROW_BLOCK",
]

# Rows processed at once.  Only bounds host memory; every output element is
# computed independently, so this changes no result.
ROW_BLOCK = 256


# --------------------------------------------------------------------------
# sizes  ([paper] §1 Notation: log2(K)/d bits per weight before scales;
#         [397B] Methodology: fp16 scale per (row, 64 weights))
# --------------------------------------------------------------------------

def words_per_row(cols: int, d: int, log2_k: int) -> int:
    """uint32 words one row's code stream occupies: ceil(cols/d/32) blocks of
    32 codes, each block B words ([397B] Methodology: row-local 32-code blocks)."""
    n_codes = cols // d
    blocks = -(-n_codes // 32)
    return blocks * log2_k


def code_bytes(rows: int, cols: int, d: int, log2_k: int, experts: int = 1) -> int:
    return experts * rows * words_per_row(cols, d, log2_k) * 4


def scale_bytes(rows: int, cols: int, group: int, experts: int = 1) -> int:
    return experts * rows * (cols // group) * 2


def codebook_bytes(d: int, log2_k: int, n_codebooks: int = 1) -> int:
    """Bytes of K entries of d fp16 values, times the number of codebooks
    ([397B] Methodology: per-tensor fp16 codebook; [paper] §4.2: the d4
    codebook of 65,536 entries is sixteen times a 32 KB threadgroup memory,
    i.e. two bytes per value)."""
    return n_codebooks * (1 << log2_k) * d * 2


def bits_per_weight(d: int, log2_k: int, group: int | None) -> float:
    """Stored bits per weight: code rate log2(K)/d ([paper] §1 Notation) plus
    one fp16 scale per `group` weights (None = code rate only)."""
    rate = log2_k / d
    return rate if group is None else rate + 16.0 / group


# --------------------------------------------------------------------------
# packing  ([paper] §2.3: packed to true bit width; [397B] Methodology)
# --------------------------------------------------------------------------

def pack_codes(codes: np.ndarray, log2_k: int) -> np.ndarray:
    """Pack integer codes [rows][n] (n a multiple of 32) into uint32 words
    [rows][n*B/32]: code j occupies bits [j*B, (j+1)*B) of the row's
    little-endian bit stream."""
    codes = np.asarray(codes, dtype=np.int64)
    rows, n = codes.shape
    assert n % 32 == 0, "rows hold whole 32-code blocks"
    assert codes.min(initial=0) >= 0 and codes.max(initial=0) < (1 << log2_k)
    bit_idx = np.arange(log2_k)
    bits = ((codes[:, :, None] >> bit_idx) & 1).astype(np.uint8)  # [rows][n][B], LSB first
    stream = bits.reshape(rows, n * log2_k)
    packed = np.packbits(stream, axis=1, bitorder="little")        # bytes, LSB-first
    return np.ascontiguousarray(packed).view("<u4").reshape(rows, -1)


def unpack_codes(words: np.ndarray, cols: int, d: int, log2_k: int) -> np.ndarray:
    """Codes [rows][cols/d] from packed words [rows][Wr] (uint32).

    Straight from the definition: view each row's words as little-endian
    bytes, expand to a bit string least-significant bit first, and read code j
    as the B bits starting at bit j*B."""
    words = np.ascontiguousarray(words, dtype="<u4")
    rows = words.shape[0]
    n = cols // d
    assert words.shape[1] == words_per_row(cols, d, log2_k)
    out = np.empty((rows, n), dtype=np.int64)
    place = (np.int64(1) << np.arange(log2_k, dtype=np.int64))
    for r0 in range(0, rows, ROW_BLOCK):
        blk = words[r0:r0 + ROW_BLOCK]
        bits = np.unpackbits(blk.view(np.uint8), axis=1, bitorder="little")
        bits = bits[:, : n * log2_k].reshape(blk.shape[0], n, log2_k)
        out[r0:r0 + ROW_BLOCK] = bits.astype(np.int64) @ place
    return out


# --------------------------------------------------------------------------
# dequant  ([paper] §2.2: codebook fit on max-abs-scaled subvectors, so a
#           weight is codebook entry x its group's scale; [397B] Methodology)
# --------------------------------------------------------------------------

def dequant(words: np.ndarray, codebook: np.ndarray, scales: np.ndarray,
            cols: int, d: int, log2_k: int, group: int) -> np.ndarray:
    """fp16 weights [rows][cols].

    W[r][c] = f16(f32(codebook[code(r, c // d)][c % d]) * f32(scales[r][c // group])).
    codebook: fp16 [K][d] (or flat K*d); scales: fp16 [rows][cols/group]."""
    k = 1 << log2_k
    cb = np.asarray(codebook, dtype=np.float16).reshape(k, d)
    scales = np.asarray(scales, dtype=np.float16)
    rows = words.shape[0]
    assert scales.shape == (rows, cols // group)
    codes = unpack_codes(words, cols, d, log2_k)
    out = np.empty((rows, cols), dtype=np.float16)
    for r0 in range(0, rows, ROW_BLOCK):
        c = codes[r0:r0 + ROW_BLOCK]
        vals = cb[c].reshape(c.shape[0], cols).astype(np.float32)           # gather
        s = np.repeat(scales[r0:r0 + ROW_BLOCK].astype(np.float32), group, axis=1)
        with np.errstate(over="ignore"):       # overflow to inf is the IEEE result
            out[r0:r0 + ROW_BLOCK] = (vals * s).astype(np.float16)           # one RNE rounding
    return out


# --------------------------------------------------------------------------
# matmul
# --------------------------------------------------------------------------

def matmul_f64(w16: np.ndarray, x16: np.ndarray) -> np.ndarray:
    """ref[t][r] = sum_c W[r][c] * x[t][c] in float64.  x: [T][cols]."""
    return np.asarray(x16, dtype=np.float64) @ np.asarray(w16, dtype=np.float64).T


def gemv_ref(words, codebook, scales, x16, cols, d, log2_k, group):
    """Dequant then float64 matmul: the decode (GEMV) and prefill (GEMM)
    paths compute the same thing and differ only in speed."""
    w = dequant(words, codebook, scales, cols, d, log2_k, group)
    return matmul_f64(w, x16)


def moe_ref(words, codebook, scales, x16, ids, *, cols, d, log2_k, group,
            x_per_slot: bool, codebook_per_expert: bool = False):
    """Routed-expert matmul (top-k MoE, one output row per (token, slot)).

    words [E][rows][Wr]; codebook [K][d] shared by the stacked tensor
    ([paper] Appendix A: one target tensor per (layer, projection) holds
    all experts; [397B] Methodology: per-tensor codebooks) or [E][K][d];
    scales [E][rows][cols/g]; x [T][cols] (x_per_slot False) or
    [T][top_k][cols]; ids [T][top_k].  Returns float64 [T][top_k][rows];
    a slot whose id is outside [0, E) is a zero row."""
    n_exp, rows = words.shape[0], words.shape[1]
    ids = np.asarray(ids)
    t_count, top_k = ids.shape
    x = np.asarray(x16)
    ref = np.zeros((t_count, top_k, rows), dtype=np.float64)
    for e in np.unique(ids):
        if not (0 <= e < n_exp):
            continue
        cb = codebook[e] if codebook_per_expert else codebook
        w = dequant(words[e], cb, scales[e], cols, d, log2_k, group)
        tt, ss = np.nonzero(ids == e)
        xrows = x[tt, ss] if x_per_slot else x[tt]
        ref[tt, ss] = matmul_f64(w, xrows)
    return ref


# --------------------------------------------------------------------------
# input / output types and the MLP epilogues
# --------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Values of bf16 bit patterns (uint16): a bf16 value is the binary32
    value whose upper 16 bits are the pattern and whose lower 16 are zero."""
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def silu(g) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_ref(y) -> np.ndarray:
    """h[..., i] = silu(y[..., 2i]) * y[..., 2i + 1]: the gate and up outputs
    of a tensor whose rows interleave gate row i (2i) and up row i (2i + 1)."""
    y = np.asarray(y, dtype=np.float64)
    assert y.shape[-1] % 2 == 0
    return silu(y[..., 0::2]) * y[..., 1::2]


def moe_combine_ref(y_slots, weights, ids, num_experts: int) -> np.ndarray:
    """out[t] = sum_s weights[t][s] * y_slots[t][s] over the slots whose id
    is in [0, num_experts); y_slots [T][top_k][rows], weights and ids
    [T][top_k].  float64."""
    y = np.asarray(y_slots, dtype=np.float64)
    ids = np.asarray(ids)
    valid = (ids >= 0) & (ids < num_experts)
    w = np.where(valid, np.asarray(weights, dtype=np.float64), 0.0)
    return np.einsum("ts,tsr->tr", w, y)
