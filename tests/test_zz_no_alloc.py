"""kda_chunk_fwd_noalloc: the forward with its workspace in the library's fixed
per-GPU region, for callers that cannot allocate.  Called through the C ABI
and compared with kda_chunk_fwd on the same inputs (bit for bit: the same
kernels run on the same data) and with the oracle, on two calls in a row,
the second with a smaller input than the first (the region keeps the first
call's contents, which must not leak into the second)."""
import ctypes

import numpy as np
import pytest

from gated_delta_rule_33_amd import kda
from gated_delta_rule_33_amd.inputs import WORKLOADS, Workload, make_inputs, to_device
from tests.gpu_helpers import TOL_BF16, check, oracle_ref


def _noalloc(d, w, inp):
    """One kda_chunk_fwd_noalloc call on the device copy d of inp; (o, final)."""
    import torch
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    seg = d["segment_ids"]
    desc = kda.make_desc(B, T, H, K, V, kda.KDA_BF16, kda.KDA_F32, inp["scale"], w.l2norm_in_kernel, w.safe_gate,
                         w.lower_bound if w.safe_gate else None, inp["max_segments"] if seg is not None else 0)
    o = torch.full((B, T, H, V), float("nan"), device="cuda")
    fin = None
    if w.final_state:
        shape = (B, H, K, V) if seg is None else (B, inp["max_segments"], H, K, V)
        fin = torch.full(shape, float("nan"), device="cuda")
    st = kda.load_library().kda_chunk_fwd_noalloc(
        ctypes.byref(desc), *(ctypes.c_void_p(d[n].data_ptr()) for n in ("q", "k", "v", "g", "beta")),
        kda._ptr(d["initial_state"]), kda._ptr(seg), ctypes.c_void_p(o.data_ptr()), kda._ptr(fin),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == kda.KDA_OK, kda.load_library().kda_last_error().decode()
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), None if fin is None else fin.cpu().numpy().astype(np.float64)


def _allocating(d, w, inp):
    import torch
    o, fin = kda.chunk_kda(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=inp["scale"],
                           initial_state=d["initial_state"], output_final_state=w.final_state,
                           use_qk_l2norm_in_kernel=w.l2norm_in_kernel, safe_gate=w.safe_gate,
                           lower_bound=w.lower_bound, segment_ids=d["segment_ids"],
                           N_max=inp["max_segments"] if d["segment_ids"] is not None else None)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), None if fin is None else fin.cpu().numpy().astype(np.float64)


@pytest.mark.gpu
def test_noalloc_matches_the_allocating_forward_on_two_calls():
    first = WORKLOADS["bf16_b1_h8_t1024_packed4"]
    second = Workload("noalloc_small", "bf16", 1, 200, 2, 128, 128, seed=5, initial_state=True, final_state=True,
                      gate="neg5_sigmoid", safe_gate=True, lower_bound=-5.0)
    for w in (first, second):
        print(f"[noalloc] {w.name}", flush=True)
        inp = make_inputs(w)
        d = to_device(inp, "bf16")
        o_n, f_n = _noalloc(d, w, inp)
        o_a, f_a = _allocating(d, w, inp)
        np.testing.assert_array_equal(o_n, o_a)
        if w.final_state:
            np.testing.assert_array_equal(f_n, f_a)
        o_ref, f_ref = oracle_ref(inp, w)
        check(f"{w.name} o", o_n, o_ref, TOL_BF16)
        if w.final_state:
            check(f"{w.name} final", f_n, f_ref, TOL_BF16)


def test_noalloc_rejects_requests_beyond_the_region():
    """The H=32, T=8192 forward needs more workspace than the fixed region:
    rejected before any GPU work, with the sizes in the message."""
    desc = kda.make_desc(1, 8192, 32, 128, 128, kda.KDA_BF16, kda.KDA_F32)
    lib = kda.load_library()
    assert kda.workspace_size(desc, False) > kda.KDA_STATIC_WORKSPACE_BYTES
    fake = ctypes.c_void_p(1 << 20)
    st = lib.kda_chunk_fwd_noalloc(ctypes.byref(desc), fake, fake, fake, fake, fake, None, None, fake, None, None)
    assert st == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    assert "fixed region" in lib.kda_last_error().decode()
