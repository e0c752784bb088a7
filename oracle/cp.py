"""CPU oracle for context-parallel state chaining (TEST INFRASTRUCTURE ONLY).

Plain numpy in fp64.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this module; it shares no code with
the HIP library.

Source: the page "feat(kda): integrate KDA attention with tokamax backend and
CP support" (Context Parallelism Support: sequence metadata per rank derived
from segment_ids, the recurrent state coordinated across ranks; its tests
split T over 2 or 4 ranks, including packed segments that cross a split or
begin exactly at one), with the update of its "Delta Rule formulation"
(Implementation Details).  Written as one linear map per token, that update
is S_t = A_t S_{t-1} + beta_t k_t v_t^T with A_t = (I - beta_t k_t k_t^T)
diag(exp(g_t)), so the state after a run of tokens is affine in the state the
run starts from, and its derivative is the product of the A_t, latest on the
left.  That product is what a rank hands on besides its end state.

Readings (also in the library's design notes): ranks take equal, contiguous
slices of T; a slice "continues" a segment when its first token and the
previous slice's last token carry the same non-zero id; a segment's state
slot is its index among the row's segments in order of appearance.

Pins: ``tests/test_oracle_cp_pins.py``.
"""
from __future__ import annotations

import numpy as np


def segment_runs(ids_row) -> list:
    """Maximal runs of one non-zero id in a row, as (first, last + 1), in order."""
    runs = []
    T = len(ids_row)
    t = 0
    while t < T:
        if ids_row[t] == 0:
            t += 1
            continue
        s = t
        while t + 1 < T and ids_row[t + 1] == ids_row[s]:
            t += 1
        runs.append((s, t + 1))
        t += 1
    return runs


def transition(k, g, beta, segment_ids=None, use_qk_l2norm: bool = False) -> np.ndarray:
    """M [B, H, K, K]: d(state after token T-1) / d(state the row's first
    segment starts from), i.e. A_{T-1} ... A_1 A_0 with
    A_t = (I - beta_t k_t k_t^T) diag(exp(g_t)), for rows whose first and
    last tokens lie in one segment; zero for every other row (the end state
    then does not depend on that start state)."""
    k = np.asarray(k, dtype=np.float32).astype(np.float64)
    g = np.asarray(g, dtype=np.float32).astype(np.float64)
    beta = np.asarray(beta, dtype=np.float32).astype(np.float64)
    B, T, H, K = k.shape
    out = np.zeros((B, H, K, K))
    for b in range(B):
        if T == 0:
            continue
        if segment_ids is not None:
            runs = segment_runs(np.asarray(segment_ids)[b])
            if runs != [(0, T)]:
                continue
        for h in range(H):
            M = np.eye(K)
            for t in range(T):
                kt = k[b, t, h]
                if use_qk_l2norm:
                    kt = kt / np.sqrt(np.sum(kt * kt) + 1e-6)
                M = np.exp(g[b, t, h])[:, None] * M                     # diag(exp(g_t)) M
                M = M - beta[b, t, h] * np.outer(kt, kt @ M)            # (I - beta k k^T) M
            out[b, h] = M
    return out


def cp_plan(segment_ids, B: int, T: int, P: int, n_states: int) -> np.ndarray:
    """int32 [B, P, 4] per slice r of row b (tokens [r L, (r+1) L), L = T/P):
    (continues the previous slice's segment, index of the first segment that
    overlaps the slice -- or, if none does, of the next segment to start --,
    number of segments overlapping the slice, whether that first index plus
    the count exceeds n_states)."""
    if T % P:
        raise ValueError("T must be a multiple of P")
    L = T // P
    plan = np.zeros((B, P, 4), dtype=np.int32)
    for b in range(B):
        runs = [(0, T)] if segment_ids is None else segment_runs(np.asarray(segment_ids)[b])
        for r in range(P):
            lo, hi = r * L, (r + 1) * L
            hit = [i for i, (s, e) in enumerate(runs) if s < hi and e > lo]
            first = hit[0] if hit else sum(1 for s, _ in runs if s < lo)
            carried = bool(hit) and runs[hit[0]][0] < lo
            plan[b, r] = (int(carried), first, len(hit), int(first + len(hit) > n_states))
    return plan
