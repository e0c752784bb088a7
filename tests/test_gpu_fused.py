"""The fused forward (one persistent kernel for the intra-chunk step and the
recurrence, records handed over through L2) against the two-kernel path
(intra-chunk kernel, then recurrence kernel, records through HBM) on the
same inputs, and against the fp64 oracle.

Both schedules build every record with the same source, and the fused
recurrence lanes run the register-direct recurrence kernel's loop; but the
kernels are compiled separately (the compiler may fuse a multiply and an
add in one and not the other), so an fp32 intermediate can differ in its
last bit and a record operand rounded to bf16 can then land one bf16 step
(2^-8 relative) apart, and beyond B H V / 16 = 512 workgroups the
two-kernel path also sums in another order.  The outputs therefore agree
to max|diff| <= 5e-4 rms (a few such flips), forty times inside the 2e-2
bar against the oracle.  Each fused call must leave the workspace's flag
word clear (no bounded wait ran out).

Shapes cover: one sequence-head (seven XCDs without work), head counts that
do not divide among the XCDs, a single chunk, a single token, ragged tails,
initial and final state, q/k L2 norm, the gate activated in the kernel, a
bf16 output, and more sequence-heads than the kernel has workgroups.
"""
import dataclasses
import sys

import numpy as np
import pytest

from gated_delta_rule_33_amd.inputs import WORKLOADS, make_inputs
from tests.gpu_helpers import TOL_BF16, check, oracle_ref, run_gpu

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


BASE = WORKLOADS["bf16_b1_h8_t1024_fixed"]

CASES = {
    "h8_t1024": {},
    "b1_h1_t640_state": dict(H=1, T=640, initial_state=True, final_state=True),
    "b2_h5_t1000_l2": dict(B=2, H=5, T=1000, l2norm_in_kernel=True, final_state=True),
    "b3_h3_t64": dict(B=3, H=3, T=64, final_state=True),
    "b2_h3_t1": dict(B=2, H=3, T=1, initial_state=True, final_state=True),
    "b1_h11_t777_safe": dict(H=11, T=777, gate="neg5_sigmoid", safe_gate=True, lower_bound=-5.0,
                             initial_state=True, final_state=True),
    "b4_h32_t512": dict(B=4, H=32, T=512, final_state=True),
}


def _workload(case):
    return dataclasses.replace(BASE, name=f"fused_{case}", seed=100 + sorted(CASES).index(case), **CASES[case])


def _workspace(w):
    import torch
    from gated_delta_rule_33_amd import kda
    desc = kda.make_desc(w.B, w.T, w.H, w.K, w.V, kda.KDA_BF16, kda.KDA_F32, None, w.l2norm_in_kernel,
                         w.safe_gate, w.lower_bound if w.safe_gate else None, 0)
    return torch.empty(max(kda.workspace_size(desc, False), 1), dtype=torch.uint8, device="cuda")


def _both(inp, w, **over):
    """(fused o, fused final, two-kernel o, two-kernel final); checks the flags."""
    from gated_delta_rule_33_amd import kda
    ws = _workspace(w)
    kda.set_fused_forward(True)
    try:
        o_f, fin_f = run_gpu(inp, w, workspace=ws, **over)
        assert kda.read_flags(ws) == 0, "a bounded wait of the fused kernel ran out"
    finally:
        kda.set_fused_forward(False)
    kda.set_fused_forward(False)
    o_t, fin_t = run_gpu(inp, w, workspace=ws, **over)
    return o_f, fin_f, o_t, fin_t


SCHEDULE_TOL = 5e-4   # max|fused - two-kernel| / rms(two-kernel)


@pytest.mark.parametrize("case", list(CASES))
def test_fused_matches_two_kernel_path(case):
    w = _workload(case)
    _say(f"[fused] {case}: B={w.B} T={w.T} H={w.H}")
    inp = make_inputs(w)
    o_f, fin_f, o_t, fin_t = _both(inp, w)
    check(f"{case} o vs two-kernel", o_f, o_t, SCHEDULE_TOL)
    if w.final_state:
        check(f"{case} final vs two-kernel", fin_f, fin_t, SCHEDULE_TOL)
    if w.B * w.H * w.T <= 8 * 1024:
        o_ref, fin_ref = oracle_ref(inp, w)
        e = check(f"{case} o", o_f, o_ref, TOL_BF16)
        _say(f"[fused] {case} o rel err {e:.3e}")
        if w.final_state:
            check(f"{case} final", fin_f, fin_ref, TOL_BF16)
    _say(f"[fused] {case} ok")


def test_fused_gate_in_kernel_and_bf16_output():
    import torch
    w = _workload("b2_h5_t1000_l2")
    inp = make_inputs(w)
    rng = np.random.default_rng(7)
    a_log = torch.tensor(rng.uniform(-1.0, 1.0, w.H), dtype=torch.float32, device="cuda")
    dt_bias = torch.tensor(rng.uniform(-0.5, 0.5, (w.H, w.K)), dtype=torch.float32, device="cuda")
    _say("[fused] gate in kernel, bf16 output")
    o_f, fin_f, o_t, fin_t = _both(inp, w, use_gate_in_kernel=True, A_log=a_log, dt_bias=dt_bias,
                                   out_dtype=torch.bfloat16)
    # Both outputs are rounded to bf16: nearly equal values may round one bf16
    # step (at most 2^-7 relative) apart.
    gap = np.maximum(np.abs(o_f - o_t) - 2.0 ** -7 * np.abs(o_t), 0.0)
    rms = float(np.sqrt(np.mean(o_t * o_t)))
    assert gap.max() <= SCHEDULE_TOL * rms, f"gated o vs two-kernel: {gap.max() / rms:.3e}"
    check("gated final vs two-kernel", fin_f, fin_t, SCHEDULE_TOL)
    _say("[fused] gate in kernel ok")


def test_fused_repeat_on_one_workspace_is_bitwise():
    """Calls in a row on one workspace: the control block and ready words are
    reset by each call, so the result never depends on the one before."""
    from gated_delta_rule_33_amd import kda
    w = _workload("b1_h11_t777_safe")
    inp = make_inputs(w)
    ws = _workspace(w)
    kda.set_fused_forward(True)
    try:
        first = run_gpu(inp, w, workspace=ws)
        for _ in range(3):
            again = run_gpu(inp, w, workspace=ws)
            assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])
        assert kda.read_flags(ws) == 0
    finally:
        kda.set_fused_forward(False)
    _say("[fused] repeat ok")
