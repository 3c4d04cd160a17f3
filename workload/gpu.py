"""Seeded generation of large layers directly in device memory (torch), for the
48-layer OPT-30B-shaped stack (~40 GB of fp16 weights), which is too large to
draw on the host in reasonable time.

Same recipe as ``workload.make_layer`` (firing law, low-rank-plus-residual
mask-defining matrix, bias from the stored row norms, training-free
predictor, hot-first neuron table), drawn with torch's device generator
instead of numpy's, so the numbers differ from the host generator's for the
same seed.  Nothing here evaluates the method: parity tests read the produced
weights back and hand them to the oracle.

Stack reading.  A token passes through the layers in order and layer l+1
takes layer l's FFN output as its input (no attention, no normalisation).
To keep every layer's input near the unit-variance hidden state the firing
law is calibrated for, layer l's W_down is drawn with standard deviation
1/sqrt(sum_i E[a_i^2]), where a_i = ReLU(z_i), z_i ~ N(b_i, ||w_i||^2) is
neuron i's activation for x ~ N(0, I); then E[y_j^2] ~ 1 (slightly less, by
the predictor's missed neurons).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import ndtr, ndtri

from . import (PHI, SIGMA, STACK_LAYERS, LayerShape, firing_probabilities, layer_seed,
               stack_layer_shape)

STACK_CONFIG = 3          # seeds of the stack: 1000 + 10*3 + layer


def relu_second_moment(mu: np.ndarray, s: np.ndarray) -> np.ndarray:
    """E[ReLU(z)^2] for z ~ N(mu, s^2): (mu^2 + s^2) Phi(mu/s) + mu s phi(mu/s)."""
    t = mu / s
    phi = np.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)
    return (mu * mu + s * s) * ndtr(t) + mu * s * phi


class DeviceLayer:
    """Original-layout weights of one layer as device tensors."""

    def __init__(self, shape, w_up, w_gate, b1, w_down, b2, p1, c1, p2, c2, perm, p,
                 down_std):
        self.shape = shape
        self.w_up, self.w_gate, self.b1, self.w_down, self.b2 = w_up, w_gate, b1, w_down, b2
        self.p1, self.c1, self.p2, self.c2, self.perm, self.p = p1, c1, p2, c2, perm, p
        self.down_std = down_std

    def to_numpy(self):
        """Host copies in the layout of workload.Layer (for the oracle)."""
        from . import Layer

        def h(t):
            return None if t is None else t.detach().cpu().numpy()
        return Layer(self.shape, h(self.w_up), h(self.w_gate), h(self.b1), h(self.w_down),
                     h(self.b2), h(self.p1), h(self.c1), h(self.p2), h(self.c2), h(self.perm),
                     self.p)


def make_layer_device(shape: LayerShape, seed: int, device, unit_output: bool = True,
                      phi: float = PHI) -> DeviceLayer:
    import torch
    d, f, H = shape.d, shape.f, shape.H
    wt = torch.float16 if shape.wdtype == "f16" else torch.float32
    r = H // 2
    rng = np.random.Generator(np.random.PCG64(seed))
    p, rank = firing_probabilities(f, shape.rho, rng)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    alpha = SIGMA * math.sqrt(phi * d / r)
    beta = SIGMA * math.sqrt(1.0 - phi)
    U = torch.randn((f, r), generator=g, device=device, dtype=torch.float32)
    V = torch.randn((r, d), generator=g, device=device, dtype=torch.float32) / math.sqrt(d)
    aU = U.mul_(alpha)
    W = aU @ V
    W.add_(torch.randn((f, d), generator=g, device=device, dtype=torch.float32), alpha=beta)
    W = W.to(wt)
    norms = W.double().pow(2).sum(dim=1).sqrt().cpu().numpy()
    b_np = (norms * ndtri(p)).astype(np.float32)
    b = torch.from_numpy(b_np).to(device)
    other = None
    if shape.gated:
        other = (torch.randn((f, d), generator=g, device=device, dtype=torch.float32)
                 * SIGMA).to(wt)
    if unit_output:
        down_std = 1.0 / math.sqrt(float(relu_second_moment(b_np.astype(np.float64),
                                                            norms).sum()))
    else:
        down_std = SIGMA
    w_down = (torch.randn((d, f), generator=g, device=device, dtype=torch.float32)
              * down_std).to(wt)
    b2 = torch.randn(d, generator=g, device=device, dtype=torch.float32) * SIGMA
    p1 = torch.cat([V, -V], dim=0).to(wt).contiguous()
    p2 = torch.cat([aU, -aU], dim=1).to(wt).contiguous()
    del U, V, aU
    perm = torch.from_numpy(np.argsort(rank, kind="stable").astype(np.int32)).to(device)
    if shape.gated:
        w_up, w_gate = other, W
    else:
        w_up, w_gate = W, None
    return DeviceLayer(shape, w_up.contiguous(), None if w_gate is None else w_gate.contiguous(),
                       b, w_down.contiguous(), b2, p1, None, p2, b.clone(), perm, p, down_std)


def stack_layer_device(l: int, device, shape: LayerShape = None) -> DeviceLayer:
    """Layer l of the 48-layer stack (or the same law at `shape`)."""
    return make_layer_device(shape or stack_layer_shape(l), layer_seed(STACK_CONFIG, l), device)


def stack_tokens(n: int, d: int = None):
    from . import STACK_D, make_tokens, token_seed
    return make_tokens(d or STACK_D, n, token_seed(STACK_CONFIG))


__all__ = ["DeviceLayer", "make_layer_device", "stack_layer_device", "stack_tokens",
           "relu_second_moment", "STACK_LAYERS", "STACK_CONFIG"]
