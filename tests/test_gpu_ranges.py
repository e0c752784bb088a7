"""Inputs of extreme and changing magnitude against the fp64 oracle (GPU).

With bf16 inputs the recurrence's state update multiplies Kt, stored as fp16
scaled by a power of two per 16-key block, with Delta as an fp16 pair scaled
by 2^4; a 32-token slab whose Delta that pair does not carry falls back to
Delta's bf16 pair.  These cases move magnitudes through and past that range:
values scaled by 2^+-20, magnitudes
that jump by 2^10 from chunk to chunk or fall to zero, 16-token blocks of
very different magnitude inside one chunk, and keys scaled by 2^+-20 without
the in-kernel norm (the Kt block scale).  The bar is the usual 2e-2 of rms,
taken per 64-token chunk (or 16-token block) where magnitudes differ, so
that a loss of accuracy in the small ones cannot hide behind the large
ones.  A chunk's output is judged against the larger of its own rms and the
previous chunk's: the state entering a chunk has the earlier chunk's size,
and a chunk whose output is a small remainder of terms of that size (v = 0
after a large chunk) carries the bf16 record operands' error at that size.
"""
import sys

import numpy as np
import pytest

from gated_delta_rule_33_amd.inputs import Workload, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs
from tests.gpu_helpers import TOL_BF16, check, oracle_ref, run_gpu

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _set(inp, name, x):
    inp[name + "_bits"] = f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    inp[name] = bf16_bits_to_f32(inp[name + "_bits"])


def _workload(seed, **kw):
    base = dict(dtype="bf16", B=1, T=700, H=3, K=128, V=128, seed=seed, initial_state=True, final_state=True)
    base.update(kw)
    return Workload(f"ranges_{seed}", base.pop("dtype"), base.pop("B"), base.pop("T"), base.pop("H"),
                    base.pop("K"), base.pop("V"), **base)


def _check_chunks(name, o, o_ref, tol, L=64):
    """max|err| per L-token chunk (and head) over the larger of the chunk's
    rms and the previous chunk's."""
    B, T, H, V = o.shape
    worst = 0.0
    for h in range(H):
        prev = 0.0
        for t0 in range(0, T, L):
            a, r = o[:, t0:t0 + L, h], o_ref[:, t0:t0 + L, h]
            rms = float(np.sqrt(np.mean(r * r)))
            den, prev = max(rms, prev), rms
            if den == 0.0:
                assert np.all(a == 0.0), f"{name}: chunk {t0 // L} head {h} should be zero"
                continue
            worst = max(worst, float(np.abs(a - r).max()) / den)
    assert worst <= tol, f"{name}: worst chunk max|err|/rms = {worst:.3e} > {tol:.1e}"
    return worst


@pytest.mark.parametrize("e", [20, -20])
def test_values_scaled(e):
    """v and the initial state times 2^e: o and the final state scale exactly."""
    w = _workload(300 + e)
    inp = make_inputs(w)
    _set(inp, "v", inp["v"] * 2.0 ** e)
    inp["initial_state"] = inp["initial_state"] * 2.0 ** e
    _say(f"[ranges] values x 2^{e}")
    o, fin = run_gpu(inp, w)
    o_ref, fin_ref = oracle_ref(inp, w)
    _check_chunks(f"v x 2^{e} o", o, o_ref, TOL_BF16)
    check(f"v x 2^{e} final", fin, fin_ref, TOL_BF16)


JUMPS = [1.0, 2.0 ** 10, 0.0, 2.0 ** -10, 2.0 ** -10]   # v's factor per chunk, repeated


def jump_factors(T):
    f = np.ones(T)
    for c in range((T + 63) // 64):
        f[64 * c:64 * c + 64] = JUMPS[c % len(JUMPS)]
    return f


def test_values_jump_between_chunks():
    """v's factor per chunk cycles through 1, 2^10, 0, 2^-10, 2^-10: each
    chunk's Delta scale follows its own magnitude, and the next chunk's
    output reads the state that update left."""
    w = _workload(311, T=640, initial_state=False)
    inp = make_inputs(w)
    f = jump_factors(w.T)
    _set(inp, "v", inp["v"] * f[None, :, None, None])
    _say("[ranges] values jumping between chunks")
    o, fin = run_gpu(inp, w)
    o_ref, fin_ref = oracle_ref(inp, w)
    _check_chunks("jumps o", o, o_ref, TOL_BF16)
    check("jumps final", fin, fin_ref, TOL_BF16)


def test_blocks_of_different_magnitude():
    """Inside every chunk the 16-token blocks of v are scaled by 2^20, 1, 1
    and 2^-10: one Delta scale per chunk spans 2^30.  Strong decay (g = -4)
    keeps each block's output dominated by its own tokens, and the final
    state by the last block's: it checks that the smallest block's share of
    the update keeps its accuracy."""
    w = _workload(312, T=512, initial_state=False)
    inp = make_inputs(w)
    f = np.tile(np.repeat([2.0 ** 20, 1.0, 1.0, 2.0 ** -10], 16), w.T // 64)
    _set(inp, "v", inp["v"] * f[None, :, None, None])
    _set(inp, "g", np.full_like(inp["g"], -4.0))
    _say("[ranges] blocks of different magnitude")
    o, fin = run_gpu(inp, w)
    o_ref, fin_ref = oracle_ref(inp, w)
    _check_chunks("blocks o", o, o_ref, TOL_BF16, L=16)   # each block has its own scale
    check("blocks final", fin, fin_ref, TOL_BF16)


@pytest.mark.parametrize("e", [20, -20])
def test_keys_scaled(e):
    """k and v times 2^e, beta times 2^-2e (no in-kernel norm): the delta
    rule's steps beta k k^T and beta k v^T are unchanged, so is the output,
    while inside the kernel Kt scales by 2^e and Delta by 2^-e."""
    w = _workload(320 + e, T=400)
    inp = make_inputs(w)
    _set(inp, "k", inp["k"] * 2.0 ** e)
    _set(inp, "v", inp["v"] * 2.0 ** e)
    _set(inp, "beta", inp["beta"] * 2.0 ** (-2 * e))
    _say(f"[ranges] keys x 2^{e}")
    o, fin = run_gpu(inp, w)
    o_ref, fin_ref = oracle_ref(inp, w)
    check(f"k x 2^{e} o", o, o_ref, TOL_BF16)
    check(f"k x 2^{e} final", fin, fin_ref, TOL_BF16)
