"""Seeded synthetic inputs for the MoE-layer hot path.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It only *draws* inputs: it contains none of the layer's own
arithmetic (no routing, no permutation, no expert FFN, no combine).

Shapes follow the models the source pages talk about:
  * "tiny"      : a small fp32 layer the oracle finishes in a blink;
  * "qwen3_30b" : 128 experts, top-8 softmax routing (the reranker paper's
                  MoE backbone, "Tevatron Meets Megatron", section 3);
  * "dsv_30b"   : 128 experts, top-6 sigmoid routing, hidden 2688, expert
                  ffn 1856 (the Megatron-Bridge deep-dive's "Motivation"
                  example of a DeepSeek-style 30B-A3B model);
  * "skew_shared": 256 experts, top-8, a gated shared expert (the TorchSpec
                  MTP pull request's Qwen3.5 MoE layer) with a Zipf-ranked
                  logit bias that makes the hottest expert ~10x the mean;
  * "ep_share"  : one expert-parallel rank's share (32 of 128 experts) for
                  the forward + backward of the grouped GEMM.

Random-number recipe (stated once, used by everything):
  * one ``numpy.random.SeedSequence(1000 + cfg.index)`` per workload;
  * ``spawn(11)`` children in the fixed order
    [x, w_router, w1, w2, ws1, ws2, w_gate, bias_perm, ep_logits,
     ep_multinomial, dy];
  * expert weight tensors spawn one grandchild per expert so any single
    expert can be regenerated on its own;
  * samples are fp32 normals, then rounded to bf16 with round-to-nearest-even
    (for bf16 workloads) -- the rounded values are the inputs both sides see.
  * x ~ N(0, 1); router rows and the shared-gate vector ~ N(0, variance 1/d);
    expert weights ~ N(0, std 0.02).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "round_to_bf16_bits", "bf16_bits_to_f32",
    "LayerInputs", "EpShareInputs", "make_layer_inputs", "make_ep_share_inputs",
    "make_small_layer_inputs", "ZIPF_EXPONENT", "SKEW_BIAS_SCALE",
]

# Zipf exponent of the expert-popularity ranking used by the skewed workload.
ZIPF_EXPONENT = 1.1
# Scale lambda applied to the log-Zipf rank bias.  Produced by
# tests/golden/calibrate_skew_bias.py (which calls only the oracle): it is the
# value in [0, 8] that brings max_e(count_e) / mean_e(count_e) closest to 10
# on the skewed workload's own seeded tokens and router.
SKEW_BIAS_SCALE = 0.29578399658203125


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    T: int            # tokens (for ep_share: routed token-slots N)
    d: int            # hidden size
    E: int            # experts (local experts for ep_share)
    k: int            # top-k
    F: int            # expert ffn size
    Fs: int           # shared-expert ffn size (0: none)
    dtype: str        # "f32" or "bf16"
    score: str        # "softmax" or "sigmoid"
    normalize: bool
    skew: bool        # Zipf logit bias
    backward: bool    # ep_share forward + backward

    @property
    def N(self) -> int:
        return self.T if self.backward else self.T * self.k


WORKLOADS = (
    Workload(0, "tiny", T=256, d=128, E=8, k=2, F=256, Fs=0, dtype="f32",
             score="softmax", normalize=True, skew=False, backward=False),
    Workload(1, "qwen3_30b", T=4096, d=2048, E=128, k=8, F=768, Fs=0,
             dtype="bf16", score="softmax", normalize=True, skew=False,
             backward=False),
    Workload(2, "dsv_30b", T=8192, d=2688, E=128, k=6, F=1856, Fs=0,
             dtype="bf16", score="sigmoid", normalize=True, skew=False,
             backward=False),
    Workload(3, "skew_shared", T=16384, d=2048, E=256, k=8, F=512, Fs=512,
             dtype="bf16", score="softmax", normalize=True, skew=True,
             backward=False),
    Workload(4, "ep_share", T=32768, d=2048, E=32, k=8, F=768, Fs=0,
             dtype="bf16", score="softmax", normalize=True, skew=False,
             backward=True),
)


def get(name_or_index) -> Workload:
    for w in WORKLOADS:
        if w.name == name_or_index or w.index == name_or_index:
            return w
    raise KeyError(name_or_index)


# --------------------------------------------------------------------------
# bf16 helpers (input rounding only)
# --------------------------------------------------------------------------
def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even.

    Inputs are finite normals, so no NaN/Inf special-casing is needed; an
    assertion guards that assumption.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    assert np.isfinite(a).all()
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(seed: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _finish(a: np.ndarray, dtype: str) -> np.ndarray:
    """Return the input as the GPU sees it: fp32 array or bf16 bit array."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    return round_to_bf16_bits(a)


def _per_expert(seed: np.random.SeedSequence, E: int, shape, std: float,
                dtype: str, threads: int) -> np.ndarray:
    kids = seed.spawn(E)
    out_dtype = np.float32 if dtype == "f32" else np.uint16
    out = np.empty((E,) + tuple(shape), dtype=out_dtype)

    def fill(e):
        out[e] = _finish(_normal(kids[e], shape, std), dtype)

    if threads > 1 and E > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(E)))
    else:
        for e in range(E):
            fill(e)
    return out


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _children(cfg: Workload):
    return np.random.SeedSequence(1000 + cfg.index).spawn(11)


@dataclasses.dataclass
class LayerInputs:
    cfg: Workload
    x: np.ndarray                 # [T, d]  (fp32, or bf16 bits as uint16)
    w_router: np.ndarray          # [E, d]
    w1: np.ndarray                # [E, 2F, d]  rows 0..F-1 gate, F..2F-1 up
    w2: np.ndarray                # [E, d, F]
    logit_bias: Optional[np.ndarray] = None   # [E] fp32
    w_gate: Optional[np.ndarray] = None       # [d]
    ws1: Optional[np.ndarray] = None          # [2Fs, d]
    ws2: Optional[np.ndarray] = None          # [d, Fs]

    def as_f32(self, name: str) -> Optional[np.ndarray]:
        a = getattr(self, name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a)
        return a


def skew_bias(cfg: Workload, scale: float = SKEW_BIAS_SCALE) -> np.ndarray:
    """Per-expert logit bias b_e = scale * (-s * ln r_e) with r_e a seeded
    random popularity rank (1 = hottest).  -s ln r is the log of the Zipf
    probability mass up to an additive constant."""
    ch = _children(cfg)
    g = np.random.Generator(np.random.PCG64(ch[7]))
    rank = g.permutation(cfg.E).astype(np.float64) + 1.0
    return (scale * (-ZIPF_EXPONENT * np.log(rank))).astype(np.float32)


def make_layer_inputs(cfg: Workload, with_experts: bool = True,
                      threads: Optional[int] = None) -> LayerInputs:
    """Inputs of a forward workload (index 0..3)."""
    assert not cfg.backward
    threads = threads or _threads()
    ch = _children(cfg)
    T, d, E, F = cfg.T, cfg.d, cfg.E, cfg.F
    x = _finish(_normal(ch[0], (T, d), 1.0), cfg.dtype)
    wr = _finish(_normal(ch[1], (E, d), 1.0 / math.sqrt(d)), cfg.dtype)
    if with_experts:
        w1 = _per_expert(ch[2], E, (2 * F, d), 0.02, cfg.dtype, threads)
        w2 = _per_expert(ch[3], E, (d, F), 0.02, cfg.dtype, threads)
    else:
        w1 = w2 = None
    inp = LayerInputs(cfg, x, wr, w1, w2)
    if cfg.Fs:
        inp.ws1 = _finish(_normal(ch[4], (2 * cfg.Fs, d), 0.02), cfg.dtype)
        inp.ws2 = _finish(_normal(ch[5], (d, cfg.Fs), 0.02), cfg.dtype)
        inp.w_gate = _finish(_normal(ch[6], (d,), 1.0 / math.sqrt(d)), cfg.dtype)
    if cfg.skew:
        inp.logit_bias = skew_bias(cfg)
    return inp


def expert_weights(cfg: Workload, e: int):
    """Regenerate expert e's (w1[e], w2[e]) alone (same values as the full
    tensors from make_layer_inputs / make_ep_share_inputs)."""
    # SeedSequence.spawn is stateful (n_children_spawned); _children builds
    # fresh parents, so the e-th grandchild is the one the full draw used.
    ch = _children(cfg)
    g1 = ch[2].spawn(cfg.E)[e]
    g2 = ch[3].spawn(cfg.E)[e]
    w1 = _finish(_normal(g1, (2 * cfg.F, cfg.d), 0.02), cfg.dtype)
    w2 = _finish(_normal(g2, (cfg.d, cfg.F), 0.02), cfg.dtype)
    return w1, w2


@dataclasses.dataclass
class EpShareInputs:
    cfg: Workload
    counts: np.ndarray     # [E] int32 rows per local expert
    offsets: np.ndarray    # [E+1] int32 segment starts
    x_perm: np.ndarray     # [N, d] bf16 bits
    w1: np.ndarray         # [E, 2F, d]
    w2: np.ndarray         # [E, d, F]
    dy: np.ndarray         # [N, d] bf16 bits


def ep_counts(cfg: Workload) -> np.ndarray:
    """Rows per local expert ~ Multinomial(N, softmax(l)), l ~ N(0, 1)."""
    ch = _children(cfg)
    g = np.random.Generator(np.random.PCG64(ch[8]))
    logits = g.standard_normal(cfg.E)
    p = np.exp(logits - logits.max())
    p /= p.sum()
    g2 = np.random.Generator(np.random.PCG64(ch[9]))
    return g2.multinomial(cfg.N, p).astype(np.int32)


def make_ep_share_inputs(cfg: Workload, threads: Optional[int] = None,
                         with_experts: bool = True) -> EpShareInputs:
    assert cfg.backward
    threads = threads or _threads()
    ch = _children(cfg)
    counts = ep_counts(cfg)
    offsets = np.zeros(cfg.E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    N, d, E, F = cfg.N, cfg.d, cfg.E, cfg.F
    x_perm = _finish(_normal(ch[0], (N, d), 1.0), cfg.dtype)
    if with_experts:
        w1 = _per_expert(ch[2], E, (2 * F, d), 0.02, cfg.dtype, threads)
        w2 = _per_expert(ch[3], E, (d, F), 0.02, cfg.dtype, threads)
    else:
        w1 = w2 = None
    dy = _finish(_normal(ch[10], (N, d), 1.0), cfg.dtype)
    return EpShareInputs(cfg, counts, offsets, x_perm, w1, w2, dy)


def make_small_layer_inputs(seed: int, T: int, d: int, E: int, F: int,
                            dtype: str = "f32", Fs: int = 0,
                            bias: bool = False, x_std: float = 1.0,
                            w_std: float = 0.02):
    """Free-shape inputs for parity sweeps over odd sizes (same recipe,
    one SeedSequence(seed))."""
    ch = np.random.SeedSequence(seed).spawn(8)
    x = _finish(_normal(ch[0], (T, d), x_std), dtype)
    wr = _finish(_normal(ch[1], (E, d), 1.0 / math.sqrt(d)), dtype)
    w1 = _finish(_normal(ch[2], (E, 2 * F, d), w_std), dtype)
    w2 = _finish(_normal(ch[3], (E, d, F), w_std), dtype)
    cfg = Workload(-1, f"small{seed}", T=T, d=d, E=E, k=0, F=F, Fs=Fs,
                   dtype=dtype, score="softmax", normalize=True, skew=bias,
                   backward=False)
    inp = LayerInputs(cfg, x, wr, w1, w2)
    if Fs:
        inp.ws1 = _finish(_normal(ch[4], (2 * Fs, d), w_std), dtype)
        inp.ws2 = _finish(_normal(ch[5], (d, Fs), w_std), dtype)
        inp.w_gate = _finish(_normal(ch[6], (d,), 1.0 / math.sqrt(d)), dtype)
    if bias:
        g = np.random.Generator(np.random.PCG64(ch[7]))
        inp.logit_bias = g.standard_normal(E).astype(np.float32)
    return inp
