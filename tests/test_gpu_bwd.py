"""Parity of the HIP backward (kda_chunk_bwd, through the C ABI) with the
backward oracle: dq, dk, dv, dg, dbeta and the initial-state gradient for
the loss sum(o * d_o) + sum(final_state * d_final_state).  The backward is
the pass the page "feat(kda): integrate KDA attention with tokamax backend and
CP support" tests beside the forward (its CP gradient-equivalence test); the
workloads are the forward's (fixed and packed rows, the in-kernel L2 norm,
partial chunks, the safe-gate range).
Bar: max|err| / rms(ref) <= 1e-4 for fp32 inputs, <= 2e-2 for bf16 inputs,
per gradient tensor.
"""
import sys

import numpy as np
import pytest

import oracle
from gated_delta_rule_33_amd.inputs import WORKLOADS, Workload, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs
from tests.gpu_helpers import TOL_BF16, TOL_F32, check, subset_heads, to_device

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _tol(w):
    return TOL_F32 if w.dtype == "f32" else TOL_BF16


def _cotangents(inp, w, seed):
    rng = np.random.default_rng(seed)
    B, T, H, V, K = w.B, w.T, w.H, w.V, w.K
    d_o = rng.standard_normal((B, T, H, V)).astype(np.float32)
    shape = (B, H, K, V) if inp["segment_ids"] is None else (B, inp["max_segments"], H, K, V)
    d_fin = rng.standard_normal(shape).astype(np.float32) if w.final_state else None
    return d_o, d_fin


def _run_gpu(inp, w, d_o, d_fin, do_bf16=False):
    import torch
    from gated_delta_rule_33_amd import kda
    d = to_device(inp, w.dtype)
    t_do = torch.from_numpy(d_o).cuda()
    if do_bf16:
        t_do = torch.from_numpy(f32_to_bf16_bits(d_o).view(np.int16)).cuda().view(torch.bfloat16)
    t_fin = None if d_fin is None else torch.from_numpy(d_fin).cuda()
    out = kda.chunk_kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], t_do, scale=inp["scale"],
                            initial_state=d["initial_state"], d_final_state=t_fin,
                            use_qk_l2norm_in_kernel=w.l2norm_in_kernel, segment_ids=d["segment_ids"],
                            N_max=inp["max_segments"] if d["segment_ids"] is not None else None)
    torch.cuda.synchronize()
    return {n: (None if t is None else t.cpu().numpy().astype(np.float64)) for n, t in zip(NAMES, out)}


def _run_oracle(inp, w, d_o, d_fin):
    return oracle.kda_backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], d_o, scale=inp["scale"],
                               initial_state=inp["initial_state"], d_final_state=d_fin,
                               use_qk_l2norm=w.l2norm_in_kernel, segment_ids=inp["segment_ids"],
                               max_segments=inp["max_segments"])


def _compare(tag, got, ref, w, names=NAMES):
    for n in names:
        e = check(f"{tag} {n}", got[n], ref[n], _tol(w))
        _say(f"[bwd] {tag} {n} rel err {e:.3e}")


def _scaled_g(inp, w, factor):
    g = (inp["g"] * np.float32(factor)).astype(np.float32)
    if w.dtype == "bf16":
        inp["g_bits"] = f32_to_bf16_bits(g)
        g = bf16_bits_to_f32(inp["g_bits"])
    inp["g"] = g


CASES = [
    Workload("bwd_f32_fixed", "f32", 2, 200, 2, 64, 64, initial_state=True, final_state=True, seed=101),
    Workload("bwd_f32_fixed_l2_kv", "f32", 1, 77, 3, 128, 64, l2norm_in_kernel=True, final_state=True, seed=102),
    Workload("bwd_bf16_fixed", "bf16", 1, 1024, 4, 128, 128, gate="neg5_sigmoid", initial_state=True,
             final_state=True, safe_gate=True, lower_bound=-5.0, seed=103),
    Workload("bwd_bf16_packed", "bf16", 2, 640, 3, 128, 128, segment_lengths=(100, 37, 1, 200, 250),
             initial_state=True, final_state=True, max_segments=6, seed=104),
    Workload("bwd_bf16_packed_l2", "bf16", 1, 512, 2, 64, 128, segment_lengths=(16, 17, 300, 150),
             l2norm_in_kernel=True, final_state=True, max_segments=4, seed=105),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_matches_oracle(w):
    _say(f"[bwd] {w.name}")
    inp = make_inputs(w)
    d_o, d_fin = _cotangents(inp, w, w.seed + 1)
    got = _run_gpu(inp, w, d_o, d_fin)
    ref = _run_oracle(inp, w, d_o, d_fin)
    if inp["segment_ids"] is not None:
        pad = inp["segment_ids"] == 0
        for n in ("dq", "dk", "dv", "dg", "dbeta"):
            assert np.all(got[n][pad] == 0.0), f"{n}: padding tokens must get zero gradients"
    _compare(w.name, got, ref, w)


def test_backward_bf16_cotangent_and_no_state():
    """d_o in bf16, no initial state and no final-state gradient: the
    initial-state gradient is still that of a zero start state."""
    w = Workload("bwd_bf16_plain", "bf16", 1, 300, 2, 128, 128, seed=106)
    inp = make_inputs(w)
    d_o, _ = _cotangents(inp, w, 7)
    d_o = bf16_bits_to_f32(f32_to_bf16_bits(d_o))
    got = _run_gpu(inp, w, d_o, None, do_bf16=True)
    ref = _run_oracle(inp, w, d_o, None)
    _compare(w.name, got, ref, w)


def test_backward_wide_gate_span_takes_the_elementwise_path():
    """Decays of -8 per token give 16-row spans of 120 (beyond the split's
    range): those chunks evaluate exp(G_r - G_i) per element."""
    w = Workload("bwd_f32_wide", "f32", 1, 96, 2, 64, 64, initial_state=True, final_state=True, seed=107)
    inp = make_inputs(w)
    inp["g"] = np.where(np.arange(96)[None, :, None, None] % 32 < 16, -8.0, inp["g"]).astype(np.float32)
    d_o, d_fin = _cotangents(inp, w, 8)
    got = _run_gpu(inp, w, d_o, d_fin)
    ref = _run_oracle(inp, w, d_o, d_fin)
    assert all(np.all(np.isfinite(got[n])) for n in NAMES)
    _compare(w.name, got, ref, w)


def test_backward_is_deterministic():
    w = CASES[3]
    inp = make_inputs(w)
    d_o, d_fin = _cotangents(inp, w, 9)
    a = _run_gpu(inp, w, d_o, d_fin)
    b = _run_gpu(inp, w, d_o, d_fin)
    for n in NAMES:
        np.testing.assert_array_equal(a[n], b[n])


def test_autograd_wrapper_matches_the_entry_point():
    """chunk_kda_autograd: loss.backward() gives the kda_chunk_bwd gradients."""
    import torch
    from gated_delta_rule_33_amd import kda
    w = CASES[0]
    inp = make_inputs(w)
    d = to_device(inp, w.dtype)
    leaves = {n: d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta", "initial_state")}
    o, fin = kda.chunk_kda_autograd(leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                                    initial_state=leaves["initial_state"], scale=inp["scale"])
    d_o, d_fin = _cotangents(inp, w, 10)
    loss = (o * torch.from_numpy(d_o).cuda()).sum() + (fin * torch.from_numpy(d_fin).cuda()).sum()
    loss.backward()
    ref = _run_gpu(inp, w, d_o, d_fin)
    for n, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                   ("initial_state", "d_initial_state")):
        np.testing.assert_allclose(leaves[n].grad.cpu().numpy(), ref[key], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("name", ["bf16_b1_h32_t8192_fixed_state", "bf16_b1_h32_t8192_packed25_l2"])
def test_backward_full_size_sampled_heads(name):
    """Full-size launch; the oracle checks three heads end to end."""
    w = WORKLOADS[name]
    _say(f"[bwd] {name} full size")
    inp = make_inputs(w)
    d_o, d_fin = _cotangents(inp, w, 11)
    got = _run_gpu(inp, w, d_o, d_fin)
    heads = [0, 15, 31]
    sub = subset_heads(inp, heads)
    ax = 1 if inp["segment_ids"] is None else 2
    sub_fin = None if d_fin is None else np.ascontiguousarray(np.take(d_fin, heads, axis=ax))
    ref = _run_oracle(sub, w, np.ascontiguousarray(d_o[:, :, heads]), sub_fin)
    for n in NAMES:
        if got[n] is None:
            continue
        g = np.take(got[n], heads, axis=ax) if n == "d_initial_state" else got[n][:, :, heads]
        e = check(f"{name} {n}", g, ref[n], TOL_BF16)
        _say(f"[bwd] {name} {n} rel err (heads {heads}) {e:.3e}")


def test_backward_empty_and_padding_only_inputs():
    """T = 0: every initial-state gradient is zero (fixed and packed); a row of
    padding only gets zero gradients everywhere and zero state gradients."""
    import torch
    from gated_delta_rule_33_amd import kda
    for seg in (None, torch.zeros((1, 0), dtype=torch.int32, device="cuda")):
        z = torch.zeros((1, 0, 2, 64), dtype=torch.float32, device="cuda")
        zb = torch.zeros((1, 0, 2), dtype=torch.float32, device="cuda")
        out = kda.chunk_kda_bwd(z, z, z, z, zb, z, segment_ids=seg, N_max=2 if seg is not None else None)
        torch.cuda.synchronize()
        d_init = out[5]
        assert d_init.shape == ((1, 2, 64, 64) if seg is None else (1, 2, 2, 64, 64)) and torch.all(d_init == 0)
    w = Workload("bwd_pad_rows", "f32", 2, 40, 2, 64, 64, initial_state=True, final_state=True, max_segments=2,
                 seed=150)
    seg = np.zeros((2, 40), np.int32)
    seg[1, 3:20] = 1
    seg[1, 20:40] = 2
    inp = make_inputs(w, segment_ids=seg)
    d_o, d_fin = _cotangents(inp, w, 12)
    got = _run_gpu(inp, w, d_o, d_fin)
    ref = _run_oracle(inp, w, d_o, d_fin)
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.all(got[n][0] == 0.0)
    assert np.all(got["d_initial_state"][0] == 0.0)
    _compare(w.name, got, ref, w)


def test_backward_segments_past_the_bound_get_zero_gradients():
    """A row with more segments than N_max: the forward gives the excess
    segments o = 0, so their tokens' gradients are zero; the recorded
    segments are unaffected (compared with a run that stops at the bound)."""
    w = Workload("bwd_overflow", "f32", 1, 64, 2, 64, 64, final_state=True, max_segments=2, seed=151)
    seg = np.repeat(np.arange(1, 5, dtype=np.int32), 16)[None]        # four segments, bound two
    inp = make_inputs(w, segment_ids=seg)
    d_o, d_fin = _cotangents(inp, w, 13)
    got = _run_gpu(inp, w, d_o, d_fin)
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.all(got[n][:, 32:] == 0.0)
    sub = {k_: (v_[:, :32] if isinstance(v_, np.ndarray) and v_.ndim >= 2 and v_.shape[:2] == (1, 64) else v_)
           for k_, v_ in inp.items()}
    ref = oracle.kda_backward(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], d_o[:, :32], scale=inp["scale"],
                              d_final_state=d_fin, segment_ids=seg[:, :32], max_segments=2)
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        check(f"overflow {n}", got[n][:, :32], ref[n], TOL_F32)
    check("overflow d_initial_state", got["d_initial_state"], ref["d_initial_state"], TOL_F32)
