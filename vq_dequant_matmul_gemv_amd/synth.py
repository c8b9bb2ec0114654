"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it draws random bytes and
values of the right shapes and distributions and nothing else.  Packed code
streams are drawn as uniformly random uint32 words: every 32-code block of a
row is exactly B whole words, so uniform random bits are uniform random codes
in [0, K) with no packing step.

Distributions (the pages publish no layer tensors, so these stand in for the
weights of the models the pages quantize):
  codes     uniform over [0, K)
  codebook  N(0, 0.02) rounded to fp16 (about 0.24 % land in the fp16
            subnormal range and are kept)
  scales    U[0.5, 1.5] rounded to fp16
  x         N(0, 1) rounded to fp16
  routing   top-k distinct experts per token from a finite Zipf(1.1) over
            expert ranks (sequential sampling without replacement, done as
            Gumbel-top-k on log-probabilities); rank k is expert id k - 1.
An "exact" variant draws codebook entries from {k/16 : -8 <= k <= 8},
scales from {0.5, 1, 2} and x from {-1, 0, 1}: every product and partial sum
of the matmul is then exactly representable in fp32, so any summation order
gives the same bits.

The root seed is 1234, the fitter's default seed in the paper "Data-Free
Vector Quantization Beats Affine Quantization at Matched Bytes Below 5 Bits"
(§2.6).  Each tensor draws from its own stream keyed by name.
"""

from __future__ import annotations

import dataclasses
import zlib

import numpy as np

ROOT_SEED = 1234


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape of one VQ tensor: W is [experts][rows = out][cols = in]."""
    rows: int
    cols: int
    d: int
    log2_k: int
    group: int
    experts: int = 1

    @property
    def k(self) -> int:
        return 1 << self.log2_k

    @property
    def words(self) -> int:
        """uint32 words per row of packed codes (rows hold whole 32-code blocks)."""
        assert (self.cols // self.d) % 32 == 0, "cols/d must be a multiple of 32"
        return (self.cols // self.d) // 32 * self.log2_k


def _key(*parts) -> list[int]:
    out = []
    for p in parts:
        if isinstance(p, str):
            out.append(zlib.crc32(p.encode()))
        else:
            out.append(int(p))
    return out


def rng(*key) -> np.random.Generator:
    """Independent PCG64 stream for a named purpose, rooted at seed 1234."""
    return np.random.default_rng(np.random.SeedSequence(ROOT_SEED, spawn_key=_key(*key)))


def tensor(spec: Spec, *key, exact: bool = False, codebook_per_expert: bool = False) -> dict:
    """Host arrays for one VQ tensor.

    codes    uint32 [E][rows][Wr]  (dense tensors: E == 1)
    codebook fp16   [K][d], or [E][K][d] when codebook_per_expert
    scales   fp16   [E][rows][cols/group]
    """
    g = rng("tensor", *key)
    e = spec.experts
    codes = g.integers(0, 1 << 32, size=(e, spec.rows, spec.words), dtype=np.uint32)
    n_cb = e if codebook_per_expert else 1
    cb_shape = (n_cb, spec.k, spec.d)
    if exact:
        codebook = (g.integers(-8, 9, size=cb_shape) / 16.0).astype(np.float16)
        scales = g.choice(np.array([0.5, 1.0, 2.0]), size=(e, spec.rows, spec.cols // spec.group))
        scales = scales.astype(np.float16)
    else:
        codebook = g.normal(0.0, 0.02, size=cb_shape).astype(np.float16)
        scales = g.uniform(0.5, 1.5, size=(e, spec.rows, spec.cols // spec.group)).astype(np.float16)
    if not codebook_per_expert:
        codebook = codebook[0]
    return {"codes": codes, "codebook": codebook, "scales": scales}


def activations(shape, *key, exact: bool = False) -> np.ndarray:
    """fp16 activations of the given shape ([T][cols] or [T][top_k][cols])."""
    g = rng("x", *key)
    if exact:
        return g.integers(-1, 2, size=shape).astype(np.float16)
    return g.normal(0.0, 1.0, size=shape).astype(np.float16)


def activations_bf16(shape, *key, exact: bool = False) -> np.ndarray:
    """bf16 activations as uint16 bit patterns: N(0, 1) drawn in fp32 and
    rounded to the nearest bf16 (ties to even); exact: values in {-1, 0, 1}."""
    g = rng("x-bf16", *key)
    if exact:
        f = g.integers(-1, 2, size=shape).astype(np.float32)
    else:
        f = g.normal(0.0, 1.0, size=shape).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def router_weights(tokens: int, top_k: int, *key) -> np.ndarray:
    """fp32 [tokens][top_k] router weights: positive, summing to one per token
    (a softmax-like draw over the chosen slots)."""
    g = rng("router-w", *key)
    w = g.exponential(1.0, size=(tokens, top_k))
    return (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def weights(rows: int, cols: int, *key, std: float = 0.02) -> np.ndarray:
    """fp32 [rows][cols] synthetic weights, N(0, std): the tensors the
    encoder fits (the pages fit real model weights, which are not here)."""
    return rng("weights", *key).normal(0.0, std, size=(rows, cols)).astype(np.float32)


def fit_draws(n_subvectors: int, n_sample: int, k: int, *key):
    """The random numbers of one fit: k-means++ subsample indices (int32
    [n_sample], without replacement) and its k uniforms (fp64 [k])."""
    g = rng("fit", *key)
    idx = g.choice(n_subvectors, size=n_sample, replace=False).astype(np.int32)
    return idx, g.uniform(size=k)


def zipf_routing(tokens: int, num_experts: int, top_k: int, *key, alpha: float = 1.1) -> np.ndarray:
    """int32 [tokens][top_k]: distinct expert ids per token, Zipf(alpha) over ranks."""
    g = rng("route", *key)
    logp = -alpha * np.log(np.arange(1, num_experts + 1, dtype=np.float64))
    keys = logp[None, :] + g.gumbel(size=(tokens, num_experts))
    order = np.argsort(-keys, axis=1, kind="stable")[:, :top_k]
    return order.astype(np.int32)


# --------------------------------------------------------------------------
# workloads (shapes of the layer tensors the pages quantize)
# --------------------------------------------------------------------------

# Mixed-tier MoE tiers (aquaman164/Qwen3.6-35B-A3B-MLX-VQ-2.4bpw card, Recipe):
# 1.5-bit d8/K4096, 2-bit d4/K256, 3-bit d4/K4096, fp16 scale per 128 weights.
TIERS = {
    "T1": dict(d=8, log2_k=12, group=128),
    "T2": dict(d=4, log2_k=8, group=128),
    "T3": dict(d=4, log2_k=12, group=128),
}


def mixed_tier_assignment(n_layers: int = 25, counts=(48, 12, 15)) -> list[str]:
    """Tier of each of the 3*n_layers tensors (gate, up, down per layer) by a
    seeded shuffle of exact counts (64 % / 16 % / 20 % of 75)."""
    tiers = ["T1"] * counts[0] + ["T2"] * counts[1] + ["T3"] * counts[2]
    assert len(tiers) == 3 * n_layers
    perm = rng("tiers").permutation(len(tiers))
    return [tiers[i] for i in perm]


WORKLOADS = {
    # single 1024x1024 GEMV, d=2 K=256 g=64, batch 1
    "gemv_1024": dict(
        tensors={"w": Spec(1024, 1024, 2, 8, 64)}, decode_tokens=[1], prefill_tokens=[]),
    # dense MLP trio, hidden 5120, intermediate 17408, d=2 K=256 g=64 (4.25 bpw)
    "dense_mlp_5120x17408_d2k256": dict(
        tensors={"gate": Spec(17408, 5120, 2, 8, 64),
                 "up": Spec(17408, 5120, 2, 8, 64),
                 "down": Spec(5120, 17408, 2, 8, 64)},
        decode_tokens=[1], prefill_tokens=[2048]),
    # MoE experts: 256 experts, hidden 4096, expert intermediate 1024, d=4 K=256 g=64
    "moe_e256_4096x1024_d4k256": dict(
        tensors={"gate": Spec(1024, 4096, 4, 8, 64, experts=256),
                 "up": Spec(1024, 4096, 4, 8, 64, experts=256),
                 "down": Spec(4096, 1024, 4, 8, 64, experts=256)},
        top_k=8, decode_tokens=[1], prefill_tokens=[1024]),
    # mixed-tier MoE: 256 experts, hidden 2048, expert intermediate 512, g=128
    "moe_mixed_tier_e256_2048x512": dict(
        layers=25, top_k=8, decode_tokens=[1], prefill_tokens=[512]),
    # large GEMM sweep: 17408x5120 and 5120x17408, d=4 K=256 g=64
    "sweep_17408x5120_d4k256": dict(
        tensors={"A": Spec(17408, 5120, 4, 8, 64), "B": Spec(5120, 17408, 4, 8, 64)},
        tokens=[1, 4, 16, 256, 4096]),
}


def mixed_tier_spec(tensor_index: int, tier: str) -> Spec:
    """Spec of tensor `tensor_index` (gate, up, down repeating) of the mixed-tier MoE."""
    t = TIERS[tier]
    if tensor_index % 3 == 2:   # down: [256][2048][512]
        return Spec(2048, 512, t["d"], t["log2_k"], t["group"], experts=256)
    return Spec(512, 2048, t["d"], t["log2_k"], t["group"], experts=256)
