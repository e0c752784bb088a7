"""Seeded synthetic inputs for the KDA chunked forward.

This module only draws random numbers and shapes them into the value
distributions of the workloads; it holds none of the recurrence's arithmetic.
Both sides of every parity check (the CPU oracle and the HIP path) consume the
exact arrays produced here: for a bf16 workload the values are rounded to bf16
once, and the oracle receives those same values widened exactly to fp32.

Distributions follow the workloads described for the KDA layer on the
"feat(kda): integrate KDA attention with tokamax backend" page (Layer
architecture: beta is a sigmoid-activated scalar per head, q/k are optionally
L2-normalised) and the representative training shapes of the tokamax packed
forward megakernel page (B=1, H=32, T=8192, K=V=128, packed N=25 balanced).

Recipe (per workload, numpy ``Generator(PCG64(seed))``):
  draw order q, k, v, beta_raw, g_raw, initial_state; each drawn in fp32 at
  its full shape in C order from N(0, 1) (initial_state from N(0, 0.1^2));
  then q, k are L2-normalised per (b, t, h) vector unless the workload asks for
  the in-kernel normalisation, beta = sigmoid(beta_raw), and
  g = logsigmoid(g_raw) or g = -5 * sigmoid(g_raw) (the safe-gate range);
  finally everything except the fp32 states is rounded to bf16 (round to
  nearest even) for bf16 workloads.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_inputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "segment_ids_from_lengths",
    "balanced_lengths",
    "to_device",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns exactly to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def balanced_lengths(total: int, n: int) -> list[int]:
    """Split ``total`` tokens into ``n`` segments whose lengths differ by at most one,
    longer ones first (8192 tokens in 25 segments gives 17 x 328 then 8 x 327)."""
    base, extra = divmod(total, n)
    return [base + 1] * extra + [base] * (n - extra)


def segment_ids_from_lengths(lengths_per_row: Sequence[Sequence[int]], T: int) -> np.ndarray:
    """1-based segment ids [B, T]; tokens past the last segment are padding (id 0)."""
    B = len(lengths_per_row)
    ids = np.zeros((B, T), dtype=np.int32)
    for b, lengths in enumerate(lengths_per_row):
        t = 0
        for s, n in enumerate(lengths):
            if n <= 0 or t + n > T:
                raise ValueError(f"segment lengths {list(lengths)} do not fit T={T}")
            ids[b, t:t + n] = s + 1
            t += n
    return ids


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                      # "f32" or "bf16": q, k, v, g, beta and o
    B: int
    T: int
    H: int
    K: int
    V: int
    # Segment lengths applied to every row, or None for one segment per row
    # (no segment_ids passed at all).
    segment_lengths: Optional[tuple] = None
    gate: str = "logsigmoid"        # "logsigmoid" or "neg5_sigmoid"
    l2norm_in_kernel: bool = False  # False: q, k are normalised here, before the call
    initial_state: bool = False
    final_state: bool = False
    safe_gate: bool = False
    lower_bound: Optional[float] = None
    seed: int = 0
    # Upper bound on segments per row passed with packed inputs.
    max_segments: int = 0
    notes: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        return self.B * self.T


WORKLOADS: dict[str, Workload] = {w.name: w for w in [
    Workload("fp32_b1_h2_t256_k64", "f32", 1, 256, 2, 64, 64,
             final_state=True, seed=0,
             notes="fp32, no segments, zero initial state, final state out"),
    Workload("bf16_b1_h8_t1024_fixed", "bf16", 1, 1024, 8, 128, 128, seed=1,
             notes="one segment per row"),
    Workload("bf16_b1_h8_t1024_packed4", "bf16", 1, 1024, 8, 128, 128,
             segment_lengths=(200, 317, 151, 356), max_segments=4, seed=2,
             notes="four non-64-aligned segments"),
    Workload("bf16_b1_h32_t8192_fixed_state", "bf16", 1, 8192, 32, 128, 128,
             gate="neg5_sigmoid", initial_state=True, final_state=True,
             safe_gate=True, lower_bound=-5.0, seed=3,
             notes="fixed length, initial and final state, safe-gate range"),
    Workload("bf16_b1_h32_t8192_packed25_l2", "bf16", 1, 8192, 32, 128, 128,
             segment_lengths=tuple(balanced_lengths(8192, 25)), max_segments=25,
             l2norm_in_kernel=True, seed=4,
             notes="packed N=25 balanced segments, q/k L2 norm in kernel"),
]}


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    # Input distribution only: unit-norm q/k vectors as the layer feeds them.
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return (np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


def make_inputs(w: Workload, segment_ids: Optional[np.ndarray] = None) -> dict:
    """Draw the seeded inputs of workload ``w``.

    Returns a dict with float32 arrays q, k, v, g [B,T,H,K|V], beta [B,T,H],
    initial_state [B,H,K,V] or [B,N_max,H,K,V] (or None), segment_ids [B,T]
    int32 (or None), plus ``scale``, ``max_segments`` and, for bf16 workloads,
    the uint16 bit arrays ``*_bits`` that hold exactly the same values.
    ``segment_ids`` overrides the workload's segment layout when given.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    q = rng.standard_normal((B, T, H, K), dtype=np.float32)
    k = rng.standard_normal((B, T, H, K), dtype=np.float32)
    v = rng.standard_normal((B, T, H, V), dtype=np.float32)
    beta_raw = rng.standard_normal((B, T, H), dtype=np.float32)
    g_raw = rng.standard_normal((B, T, H, K), dtype=np.float32)

    if segment_ids is None and w.segment_lengths is not None:
        segment_ids = segment_ids_from_lengths([w.segment_lengths] * B, T)
    max_segments = w.max_segments
    if segment_ids is not None:
        segment_ids = np.ascontiguousarray(segment_ids, dtype=np.int32)
        if max_segments <= 0:
            max_segments = int(T)

    init = None
    if w.initial_state:
        shape = (B, H, K, V) if segment_ids is None else (B, max_segments, H, K, V)
        init = (0.1 * rng.standard_normal(shape, dtype=np.float32)).astype(np.float32)

    if not w.l2norm_in_kernel:
        q = _l2_normalise(q)
        k = _l2_normalise(k)
    beta = _sigmoid(beta_raw)
    if w.gate == "logsigmoid":
        g = _logsigmoid(g_raw)
    elif w.gate == "neg5_sigmoid":
        g = (-5.0 * _sigmoid(g_raw)).astype(np.float32)
    else:
        raise ValueError(f"unknown gate distribution {w.gate!r}")

    out = dict(segment_ids=segment_ids, initial_state=init,
               scale=float(1.0 / np.sqrt(K)), max_segments=max_segments)
    for name, arr in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        if w.dtype == "bf16":
            bits = f32_to_bf16_bits(arr)
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_f32(bits)
        elif w.dtype == "f32":
            out[name] = np.ascontiguousarray(arr, dtype=np.float32)
        else:
            raise ValueError(f"unknown dtype {w.dtype!r}")
    return out


def to_device(inp: dict, dtype: str, device="cuda") -> dict:
    """Upload the arrays of ``make_inputs`` as torch tensors (bf16 from the
    exact bit patterns, fp32 as is); states fp32, segment ids int32."""
    import torch
    out = {}
    for name in ("q", "k", "v", "g", "beta"):
        if dtype == "bf16":
            bits = np.ascontiguousarray(inp[name + "_bits"]).view(np.int16)
            out[name] = torch.from_numpy(bits).to(device).view(torch.bfloat16)
        else:
            out[name] = torch.from_numpy(np.ascontiguousarray(inp[name], dtype=np.float32)).to(device)
    out["initial_state"] = None if inp["initial_state"] is None else \
        torch.from_numpy(np.ascontiguousarray(inp["initial_state"], dtype=np.float32)).to(device)
    out["segment_ids"] = None if inp["segment_ids"] is None else \
        torch.from_numpy(np.ascontiguousarray(inp["segment_ids"], dtype=np.int32)).to(device)
    return out
