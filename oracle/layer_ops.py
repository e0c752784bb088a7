"""CPU oracle for the two layer steps around the KDA kernel (TEST INFRASTRUCTURE ONLY).

Plain numpy in fp64 on the exact values the GPU receives.  Only ``tests/``
and the benchmark's CPU-baseline leg may import this module; it shares no
code with the HIP library.

Both steps come from the layer pipeline of the page "feat(kda): integrate
KDA attention with tokamax backend and CP support" (Implementation Details,
Layer architecture): step 1, the short convolution that q, k and v each pass
through (causal, depthwise, 1D, SiLU activation, kernel size
``linear_conv_kernel_dim`` from the configuration table, default 4), and the
output stage, a per-head RMSNorm with a sigmoid output gate applied after the
kernel.  The same page's review notes make the convolution segment-aware: it
must not reach across packed segments.

Readings where the pages are silent (stated in the library's design notes
too): no convolution bias; a tap reaches only earlier tokens of the same
contiguous run of one non-zero segment id (the segment rule of the KDA
forward), zeros elsewhere; padding tokens (id 0) output zero; the output gate
is elementwise over [B, T, H, V]; the RMSNorm weight has one entry per value
channel and is shared by the heads; eps is a parameter.

Pins: ``tests/test_oracle_layer_pins.py``.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def segment_starts(segment_ids: Optional[np.ndarray], B: int, T: int) -> np.ndarray:
    """start[b, t]: first token of t's segment (t itself for padding).
    A segment is a maximal run of equal non-zero ids."""
    start = np.zeros((B, T), dtype=np.int64)
    for b in range(B):
        s = 0
        for t in range(T):
            if segment_ids is None:
                start[b, t] = 0
                continue
            cur = segment_ids[b, t]
            if t == 0 or cur == 0 or cur != segment_ids[b, t - 1]:
                s = t
            start[b, t] = s
    return start


def short_conv(x, weight, segment_ids=None, activation: str = "silu"):
    """Causal depthwise convolution of x [B, T, D] with weight [D, W]:
        y[b, t, d] = act( sum_{j<W} weight[d, j] * x[b, t - (W-1) + j, d] ),
    where taps before the start of t's segment (or before t = 0) read zero,
    and padding tokens give y = 0.  act is SiLU (x sigmoid(x)) or identity."""
    x = _f64(x)
    w = _f64(weight)
    B, T, D = x.shape
    W = w.shape[1]
    if w.shape != (D, W) or W < 1:
        raise ValueError("weight must be [D, W] with W >= 1")
    seg = None if segment_ids is None else np.asarray(segment_ids)
    start = segment_starts(seg, B, T)
    y = np.zeros((B, T, D))
    for b in range(B):
        for t in range(T):
            if seg is not None and seg[b, t] == 0:
                continue
            acc = np.zeros(D)
            for j in range(W):
                tau = t - (W - 1) + j
                if tau >= start[b, t]:
                    acc += w[:, j] * x[b, tau]
            y[b, t] = acc * _sigmoid(acc) if activation == "silu" else acc
    return y


def gated_rmsnorm(o, gate, weight, eps: float = 1e-6):
    """Per-head RMSNorm with a sigmoid output gate, over the last axis (V):
        y = weight * o / sqrt(mean(o^2) + eps) * sigmoid(gate)."""
    o = _f64(o)
    z = _f64(gate)
    w = _f64(weight)
    if z.shape != o.shape or w.shape != (o.shape[-1],):
        raise ValueError("gate must match o and weight must be [V]")
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return w * (o / rms) * _sigmoid(z)
