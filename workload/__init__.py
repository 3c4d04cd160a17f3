"""Seeded synthetic workloads for the activation-sparse FFN decode path.

This module only draws inputs: layer weights, predictor weights, the neuron
table and decode tokens.  It holds none of the method's arithmetic (no
predictor evaluation, no thresholding, no FFN) and imports neither the GPU
package nor the oracle, so both can be fed from it.

Recipe (no dataset or trained checkpoint is used; these stand in for the
hidden states at the FFN input of OPT/Llama-class ReLU models during
ChatGPT/Alpaca-style decode):

* Firing law.  Every original neuron gets a hotness rank from a seeded random
  permutation, so hot neurons are scattered in original order.  Its firing
  probability is p_i = min(0.99, C * rank_i^-1.1), with C found by bisection
  so that mean(p) equals the configured activation fraction rho (a power law,
  as the pages describe for LLM neuron activity).
* Mask-defining matrix W (W_up for the plain FFN, W_gate for the gated one):
  low rank plus residual, W = alpha*U@V + beta*R with r = H/2,
  U ~ N(0,1)[f,r], V ~ N(0,1/d)[r,d], R ~ N(0,1)[f,d],
  alpha^2 r/d = phi*sigma^2 and beta^2 = (1-phi)*sigma^2, sigma = 0.02,
  so elements are ~N(0, sigma^2).
* FC1 (gate) bias b_i = ||w_i||_2 * Phi^-1(p_i) computed on the stored
  (rounded) row, so that P(w_i.x + b_i > 0) = p_i for x ~ N(0, I).
* Other matrices (W_down, and W_up of the gated FFN) are i.i.d. N(0, sigma^2);
  b2 ~ N(0, sigma^2).
* Predictor without training: P1 = [V; -V], c1 = 0, P2 = [alpha*U, -alpha*U],
  c2 = b.  Its score equals the true pre-activation minus the unseen
  residual beta*R@x.  phi is fixed at 0.99 (recall near 0.95).
* Neuron table: stored slot s holds the neuron of hotness rank s+1 (hot
  first), i.e. the order an offline activation profile would give.
* Tokens: x ~ N(0, 1)[d], float32.
* Seeds: layer weights 1000 + 10*config + layer, tokens 2000 + config.

Attention-head predictor (the pages' DejaVu appendix: a two-layer MLP with
one sigmoid output per head; about 20% of the heads are needed per token):
* Each head j gets a selection probability p_j from the same capped power
  law over a seeded random head rank (mean ``frac``, cap 0.95).
* Q1 ~ N(0, 1/d)[H][d], c1 = 0, so each hidden pre-activation is ~N(0, 1)
  for x ~ N(0, I) and ReLU of it has mean 1/sqrt(2 pi) and variance
  1/2 - 1/(2 pi).
* Q2 ~ N(0, 1/H)[heads][H]; c2_j = -m_j + s_j Phi^-1(p_j) with m_j and s_j
  the mean and standard deviation those moments give Q2[j] . h on the stored
  (rounded) row, so P(select head j) is near p_j.
* Shapes: the OPT-30B-shaped attention (d_model 7168, 56 heads) and the
  pages' example of 256 heads (d_model 4096), hidden size 1024, fp16.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
from scipy.special import ndtri

SIGMA = 0.02
PHI = 0.99
ZIPF_S = 1.1
P_CAP = 0.99


@dataclasses.dataclass(frozen=True)
class LayerShape:
    d: int            # d_model
    f: int            # d_ffn (neurons)
    H: int            # predictor hidden size
    rho: float        # mean firing probability
    wdtype: str       # "f32" or "f16"
    gated: bool = False


# The workloads.  Index = config number used in the seeds.
CONFIGS = {
    "tiny_f32": (0, LayerShape(256, 1024, 64, 0.10, "f32")),
    "opt6.7b_ffn": (1, LayerShape(4096, 16384, 1024, 0.07, "f16")),
    "llama7b_gated_relu": (2, LayerShape(4096, 11008, 1024, 0.10, "f16", gated=True)),
    "opt13b_batched": (4, LayerShape(5120, 20480, 1024, 0.05, "f16")),
}

# 48-layer OPT-30B-shaped stack: activation grows with depth and each
# predictor's hidden size follows its layer's sparsity (sparser layers get
# smaller predictors).
STACK_LAYERS = 48
STACK_D, STACK_F = 7168, 28672


def stack_layer_shape(l: int) -> LayerShape:
    rho = 0.03 + 0.12 * l / (STACK_LAYERS - 1)
    H = 512 if rho < 0.07 else (1024 if rho < 0.11 else 2048)
    return LayerShape(STACK_D, STACK_F, H, rho, "f16")


def firing_probabilities(f: int, rho: float, rng: np.random.Generator,
                         s: float = ZIPF_S, cap: float = P_CAP):
    """Return (p by original id, rank by original id, 1-based)."""
    order = rng.permutation(f)                  # order[k] = id of rank k+1
    rank = np.empty(f, np.int64)
    rank[order] = np.arange(1, f + 1)
    return law_by_rank(f, rho, s, cap)[rank - 1], rank


def law_by_rank(f: int, rho: float, s: float = ZIPF_S, cap: float = P_CAP) -> np.ndarray:
    """Firing probability of the neuron of hotness rank 1..f: min(cap, C r^-s),
    C by bisection so that the mean is rho."""
    base = np.arange(1, f + 1, dtype=np.float64) ** (-s)
    lo, hi = 0.0, 1.0
    while np.minimum(cap, hi * base).mean() < rho:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(cap, mid * base).mean() < rho:
            lo = mid
        else:
            hi = mid
    return np.minimum(cap, hi * base)


def sampled_sets(perm: np.ndarray, rho: float, n: int, seed: int):
    """n independent active sets (original ids, ascending) drawn from the
    firing law at mean activation rho, with the hotness order of a layer's
    neuron table (perm[slot] = id of hotness rank slot + 1)."""
    f = perm.shape[0]
    p = np.empty(f, np.float64)
    p[perm] = law_by_rank(f, rho)
    rng = np.random.Generator(np.random.PCG64(seed))
    return [np.flatnonzero(rng.random(f) < p).astype(np.int32) for _ in range(n)]


@dataclasses.dataclass
class Layer:
    shape: LayerShape
    w_up: np.ndarray                 # [f][d]
    w_gate: Optional[np.ndarray]     # [f][d] or None
    b1: np.ndarray                   # [f] float32 (gate bias when gated)
    w_down: np.ndarray               # [d][f]
    b2: np.ndarray                   # [d] float32
    p1: np.ndarray                   # [H][d]
    c1: Optional[np.ndarray]         # [H] float32 or None (zero)
    p2: np.ndarray                   # [f][H]
    c2: np.ndarray                   # [f] float32
    perm: np.ndarray                 # [f] int32, slot -> original id (hot first)
    p: np.ndarray                    # [f] firing probability by original id

    @property
    def wtype(self):
        return np.float16 if self.shape.wdtype == "f16" else np.float32


def make_layer(shape: LayerShape, seed: int, phi: float = PHI) -> Layer:
    rng = np.random.Generator(np.random.PCG64(seed))
    d, f, H = shape.d, shape.f, shape.H
    wt = np.float16 if shape.wdtype == "f16" else np.float32
    r = H // 2
    p, rank = firing_probabilities(f, shape.rho, rng)
    U = rng.standard_normal((f, r), dtype=np.float32)
    V = (rng.standard_normal((r, d), dtype=np.float32) * np.float32(1.0 / np.sqrt(d)))
    alpha = SIGMA * np.sqrt(phi * d / r)
    beta = SIGMA * np.sqrt(1.0 - phi)
    W = (np.float32(alpha) * U) @ V
    W += np.float32(beta) * rng.standard_normal((f, d), dtype=np.float32)
    W = W.astype(wt)
    norms = np.sqrt((W.astype(np.float64) ** 2).sum(axis=1))
    b = (norms * ndtri(p)).astype(np.float32)
    other = (rng.standard_normal((f, d), dtype=np.float32) * np.float32(SIGMA)).astype(wt) \
        if shape.gated else None
    w_down = (rng.standard_normal((d, f), dtype=np.float32) * np.float32(SIGMA)).astype(wt)
    b2 = (rng.standard_normal(d, dtype=np.float32) * np.float32(SIGMA)).astype(np.float32)
    p1 = np.concatenate([V, -V], axis=0).astype(wt)
    aU = np.float32(alpha) * U
    p2 = np.concatenate([aU, -aU], axis=1).astype(wt)
    perm = np.argsort(rank, kind="stable").astype(np.int32)
    if shape.gated:
        w_up, w_gate = other, W
    else:
        w_up, w_gate = W, None
    return Layer(shape, np.ascontiguousarray(w_up),
                 None if w_gate is None else np.ascontiguousarray(w_gate),
                 b, np.ascontiguousarray(w_down), b2, np.ascontiguousarray(p1), None,
                 np.ascontiguousarray(p2), b.copy(), perm, p)


def layer_seed(config_index: int, layer: int = 0) -> int:
    return 1000 + 10 * config_index + layer


def token_seed(config_index: int) -> int:
    return 2000 + config_index


def calib_seed(config_index: int) -> int:
    return 3000 + config_index


def make_tokens(d: int, n: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((n, d), dtype=np.float32)


def config_layer(name: str, layer: int = 0, shape: Optional[LayerShape] = None) -> Layer:
    idx, sh = CONFIGS[name]
    return make_layer(shape or sh, layer_seed(idx, layer))


def config_tokens(name: str, n: int) -> np.ndarray:
    idx, sh = CONFIGS[name]
    return make_tokens(sh.d, n, token_seed(idx))


def config_calib_tokens(name: str, n: int) -> np.ndarray:
    """Calibration tokens (activation profiling), drawn apart from the
    decode tokens."""
    idx, sh = CONFIGS[name]
    return make_tokens(sh.d, n, calib_seed(idx))


def scaled_shape(shape: LayerShape, d: int, f: int, H: int) -> LayerShape:
    """Same law and dtype at a smaller size (parity cases the oracle finishes
    in seconds)."""
    return dataclasses.replace(shape, d=d, f=f, H=H)


def random_layer(d: int, f: int, H: int, wdtype: str, gated: bool, seed: int,
                 scale: float = SIGMA) -> Layer:
    """Unstructured i.i.d. layer (no firing law), for edge-case parity."""
    rng = np.random.Generator(np.random.PCG64(seed))
    wt = np.float16 if wdtype == "f16" else np.float32

    def mat(shape):
        return (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(wt)

    sh = LayerShape(d, f, H, 0.5, wdtype, gated)
    w_up = mat((f, d))
    w_gate = mat((f, d)) if gated else None
    b1 = (rng.standard_normal(f, dtype=np.float32) * np.float32(scale)).astype(np.float32)
    w_down = mat((d, f))
    b2 = (rng.standard_normal(d, dtype=np.float32) * np.float32(scale)).astype(np.float32)
    p1 = (rng.standard_normal((H, d), dtype=np.float32) / np.float32(np.sqrt(d))).astype(wt)
    c1 = (rng.standard_normal(H, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    p2 = (rng.standard_normal((f, H), dtype=np.float32) / np.float32(np.sqrt(H))).astype(wt)
    c2 = (rng.standard_normal(f, dtype=np.float32) * np.float32(0.5) - np.float32(0.5)).astype(np.float32)
    perm = rng.permutation(f).astype(np.int32)
    return Layer(sh, w_up, w_gate, b1, w_down, b2, p1, c1, p2, c2, perm, np.full(f, 0.5))


# ---------------------------------------------------------------- attention-head predictor
@dataclasses.dataclass(frozen=True)
class HeadShape:
    d: int            # d_model
    heads: int        # outputs (attention heads)
    H: int            # hidden size
    frac: float       # mean selection probability
    wdtype: str       # "f32" or "f16"


HEAD_CONFIGS = {
    "opt30b_heads": (5, HeadShape(7168, 56, 1024, 0.20, "f16")),
    "heads256": (6, HeadShape(4096, 256, 1024, 0.20, "f16")),
}


@dataclasses.dataclass
class HeadPredictor:
    shape: HeadShape
    q1: np.ndarray                   # [H][d]
    c1: Optional[np.ndarray]         # [H] float32 or None (zero)
    q2: np.ndarray                   # [heads][H]
    c2: np.ndarray                   # [heads] float32
    p: np.ndarray                    # [heads] selection probability


def make_head_predictor(shape: HeadShape, seed: int) -> HeadPredictor:
    rng = np.random.Generator(np.random.PCG64(seed))
    d, nh, H = shape.d, shape.heads, shape.H
    wt = np.float16 if shape.wdtype == "f16" else np.float32
    p, _ = firing_probabilities(nh, shape.frac, rng, s=ZIPF_S, cap=0.95)
    q1 = (rng.standard_normal((H, d), dtype=np.float32) / np.float32(np.sqrt(d))).astype(wt)
    q2 = (rng.standard_normal((nh, H), dtype=np.float32) / np.float32(np.sqrt(H))).astype(wt)
    q2d = q2.astype(np.float64)
    mean_h = 1.0 / np.sqrt(2.0 * np.pi)
    var_h = 0.5 - 1.0 / (2.0 * np.pi)
    m = mean_h * q2d.sum(axis=1)
    sd = np.sqrt(var_h * (q2d ** 2).sum(axis=1))
    c2 = (-m + sd * ndtri(p)).astype(np.float32)
    return HeadPredictor(shape, np.ascontiguousarray(q1), None, np.ascontiguousarray(q2), c2, p)


def head_config(name: str) -> HeadPredictor:
    idx, sh = HEAD_CONFIGS[name]
    return make_head_predictor(sh, layer_seed(idx))


def head_config_tokens(name: str, n: int) -> np.ndarray:
    idx, sh = HEAD_CONFIGS[name]
    return make_tokens(sh.d, n, token_seed(idx))
