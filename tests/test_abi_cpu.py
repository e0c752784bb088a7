"""CPU-side checks of the C ABI: the library loads, exports every function
include/kda.h declares, and rejects invalid requests before touching the GPU
(status codes follow the chunk_kda runtime guards: NotImplementedError for
unsupported shapes, ValueError for invalid configurations)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_33_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "kda.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\**\s+\**(kda_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_exported_set():
    assert _declared_functions() == sorted(kda.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = kda.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.kda_version().decode().startswith("kda-mi355x")
    assert "debug" not in lib.kda_version().decode()


def test_debug_library_exports_every_declared_symbol():
    """libkda_debug.so (device checks of preconditions) has the same ABI."""
    lib = kda.open_library(kda.DEBUG_LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.kda_version().decode().endswith("debug-checks")


def _desc(**kw):
    base = dict(B=1, T=128, H=2, K=128, V=128, dtype=kda.KDA_BF16, o_dtype=kda.KDA_F32)
    base.update(kw)
    return kda.make_desc(base.pop("B"), base.pop("T"), base.pop("H"), base.pop("K"), base.pop("V"),
                         base.pop("dtype"), base.pop("o_dtype"), **base)


@pytest.mark.parametrize("kw,exc", [
    (dict(K=96), NotImplementedError),
    (dict(V=256), NotImplementedError),
    (dict(chunk_size=32), NotImplementedError),
    (dict(safe_gate=True, lower_bound=0.0), ValueError),
    (dict(safe_gate=True, lower_bound=-5.5), ValueError),
    (dict(safe_gate=True, lower_bound=float("nan")), ValueError),
    (dict(scale=float("inf")), ValueError),
    (dict(B=-1), ValueError),
    (dict(dtype=7), ValueError),
])
def test_invalid_descriptors_are_rejected(kw, exc):
    with pytest.raises(exc):
        kda.workspace_size(_desc(**kw), False)


def test_packed_input_needs_a_segment_bound():
    with pytest.raises(ValueError, match="max_segments"):
        kda.workspace_size(_desc(), True)
    assert kda.workspace_size(_desc(max_segments=3), True) > kda.workspace_size(_desc(), False)


def test_safe_gate_bounds_accepted():
    for lb in (-5.0, -1.0, -1e-3):
        assert kda.workspace_size(_desc(safe_gate=True, lower_bound=lb), False) > 0


def test_workspace_size_scales_with_chunks():
    a = kda.workspace_size(_desc(T=128), False)
    b = kda.workspace_size(_desc(T=256), False)
    c = kda.workspace_size(_desc(T=129), False)
    d = kda.workspace_size(_desc(T=192), False)
    assert a < c == d < b


def test_forward_rejects_before_any_launch():
    lib = kda.load_library()
    d = _desc()
    fake = ctypes.c_void_p(0x1000)
    # too small a workspace
    st = lib.kda_chunk_fwd(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, fake, None, fake,
                           ctypes.c_size_t(16), None)
    assert st == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    assert "workspace needs" in lib.kda_last_error().decode()
    # misaligned pointer
    n = kda.workspace_size(d, False)
    st = lib.kda_chunk_fwd(ctypes.byref(d), ctypes.c_void_p(0x1004), fake, fake, fake, fake, None, None, fake,
                           None, fake, ctypes.c_size_t(n), None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT
    # NULL input
    st = lib.kda_chunk_fwd(ctypes.byref(d), None, fake, fake, fake, fake, None, None, fake, None, fake,
                           ctypes.c_size_t(n), None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT
    # packed without a bound
    st = lib.kda_chunk_fwd(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake, fake, None, fake,
                           ctypes.c_size_t(n), None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT


def test_gated_forward_rejects_before_any_launch():
    lib = kda.load_library()
    d = _desc()
    fake = ctypes.c_void_p(0x1000)
    n = kda.workspace_size(d, False)
    # misaligned gate parameter
    st = lib.kda_chunk_fwd_gated(ctypes.byref(d), fake, fake, fake, fake, fake, ctypes.c_void_p(0x1002), None,
                                 None, None, fake, None, fake, ctypes.c_size_t(n), None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT
    # the safe gate's bound is checked as for the plain entry point
    bad = _desc(safe_gate=True, lower_bound=-6.0)
    st = lib.kda_chunk_fwd_gated(ctypes.byref(bad), fake, fake, fake, fake, fake, None, None, None, None, fake,
                                 None, fake, ctypes.c_size_t(n), None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT
    # too small a workspace
    st = lib.kda_chunk_fwd_gated(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, None, None, fake,
                                 None, fake, ctypes.c_size_t(16), None)
    assert st == kda.KDA_ERR_WORKSPACE_TOO_SMALL


def test_layer_steps_reject_before_any_launch():
    lib = kda.load_library()
    fake = ctypes.c_void_p(0x1000)
    conv = lambda B, T, D, W, dt=kda.KDA_BF16, x=fake: lib.kda_short_conv_fwd(B, T, D, W, dt, x, fake, None, fake, None)
    assert conv(1, 8, 64, 0) == kda.KDA_ERR_INVALID_ARGUMENT      # W = 0: the caller skips the call
    assert conv(1, 8, 64, 9) == kda.KDA_ERR_NOT_IMPLEMENTED
    assert conv(1, 8, 68, 4) == kda.KDA_ERR_NOT_IMPLEMENTED
    assert conv(1, 8, 64, 4, x=ctypes.c_void_p(0x1008)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert conv(0, 8, 64, 4) == kda.KDA_OK                          # empty: nothing to do
    norm = lambda rows, V, eps=1e-6: lib.kda_gated_rmsnorm_fwd(rows, V, kda.KDA_F32, kda.KDA_BF16, kda.KDA_F32,
                                                               fake, fake, fake, eps, fake, None)
    assert norm(4, 96) == kda.KDA_ERR_NOT_IMPLEMENTED
    assert norm(4, 128, eps=-1.0) == kda.KDA_ERR_INVALID_ARGUMENT
    assert norm(0, 128) == kda.KDA_OK


def test_transition_and_rerun_reject_before_any_launch():
    lib = kda.load_library()
    d = _desc()
    fake = ctypes.c_void_p(0x1000)
    n = kda.workspace_size(d, False)
    # no transition buffer
    st = lib.kda_chunk_fwd_transition(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, fake, None, None,
                                      fake, ctypes.c_size_t(n), None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT
    # misaligned transition buffer
    st = lib.kda_chunk_fwd_transition(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, fake, None,
                                      ctypes.c_void_p(0x1004), fake, ctypes.c_size_t(n), None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT
    # the rerun needs o and a workspace of the forward's size
    st = lib.kda_chunk_fwd_rerun(ctypes.byref(d), None, None, None, None, fake, ctypes.c_size_t(n), None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT
    st = lib.kda_chunk_fwd_rerun(ctypes.byref(d), None, None, fake, None, fake, ctypes.c_size_t(16), None)
    assert st == kda.KDA_ERR_WORKSPACE_TOO_SMALL


def test_cp_steps_reject_before_any_launch():
    lib = kda.load_library()
    fake = ctypes.c_void_p(0x1000)

    def cp(**kw):
        base = dict(B=1, T=256, H=2, K=128, V=128, P=2, n_states=1)
        base.update(kw)
        return kda.KdaCpDesc(**base)

    plan = lambda d, seg=None, out=fake: lib.kda_cp_plan(ctypes.byref(d), seg, out, None)
    assert plan(cp(P=0)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert plan(cp(T=250, P=4)) == kda.KDA_ERR_INVALID_ARGUMENT       # T not a multiple of P
    assert plan(cp(T=0)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert plan(cp(K=96)) == kda.KDA_ERR_NOT_IMPLEMENTED
    assert plan(cp(n_states=0)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert plan(cp(), out=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert plan(cp(), seg=ctypes.c_void_p(0x1004)) == kda.KDA_ERR_INVALID_ARGUMENT
    assert plan(cp(B=0)) == kda.KDA_OK                                 # empty: nothing to do
    d = cp()
    assert lib.kda_cp_gather_states(ctypes.byref(d), fake, None, None, None, None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_cp_chain(ctypes.byref(d), fake, fake, None, fake, None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_cp_chain(ctypes.byref(d), fake, fake, fake, ctypes.c_void_p(0x1008), None) == \
        kda.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_cp_scatter_states(ctypes.byref(cp(V=32)), fake, fake, fake, None) == kda.KDA_ERR_NOT_IMPLEMENTED
    assert lib.kda_cp_scatter_states(ctypes.byref(d), fake, None, fake, None) == kda.KDA_ERR_INVALID_ARGUMENT
    # the backward's glue
    assert lib.kda_cp_gather_final_grads(ctypes.byref(d), fake, None, None, None, None) == \
        kda.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_cp_gather_final_grads(ctypes.byref(cp(P=3)), fake, None, None, fake, None) == \
        kda.KDA_ERR_INVALID_ARGUMENT                                   # T not a multiple of P
    assert lib.kda_cp_chain_bwd(ctypes.byref(d), fake, fake, None, fake, None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_cp_scatter_initial_grads(ctypes.byref(cp(K=32)), fake, fake, fake, None) == \
        kda.KDA_ERR_NOT_IMPLEMENTED
    assert lib.kda_cp_scatter_initial_grads(ctypes.byref(d), fake, fake, ctypes.c_void_p(0x1004), None) == \
        kda.KDA_ERR_INVALID_ARGUMENT


def test_backward_rejects_before_any_launch():
    lib = kda.load_library()
    d = _desc()
    fake = ctypes.c_void_p(0x1000)
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_bwd_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == kda.KDA_OK and n.value > 0
    assert lib.kda_chunk_bwd_workspace_size(ctypes.byref(_desc(K=96)), 0, ctypes.byref(n)) == \
        kda.KDA_ERR_NOT_IMPLEMENTED
    args = lambda **kw: [kw.get(x, fake) for x in ("q", "k", "v", "g", "beta")] + \
        [kw.get("init"), kw.get("seg"), kw.get("d_o", fake), kw.get("d_fin")] + \
        [kw.get(x, fake) for x in ("dq", "dk", "dv", "dg", "dbeta")] + [kw.get("d_init")]
    for fn in (lib.kda_chunk_bwd, lib.kda_chunk_bwd_rerun):
        # a missing gradient buffer
        assert fn(ctypes.byref(d), *args(dg=None), fake, ctypes.c_size_t(1 << 40), None) == kda.KDA_ERR_INVALID_ARGUMENT
        # a misaligned cotangent
        assert fn(ctypes.byref(d), *args(d_o=ctypes.c_void_p(0x1008)), fake, ctypes.c_size_t(1 << 40), None) == \
            kda.KDA_ERR_INVALID_ARGUMENT
        # too small a workspace
        assert fn(ctypes.byref(d), *args(), fake, ctypes.c_size_t(64), None) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
        # packed without a segment bound
        assert fn(ctypes.byref(d), *args(seg=fake), fake, ctypes.c_size_t(1 << 40), None) == \
            kda.KDA_ERR_INVALID_ARGUMENT


def test_python_wrapper_rejects_unsupported_options():
    torch = pytest.importorskip("torch")
    z = torch.zeros(1)
    with pytest.raises(ValueError, match="use_gate_in_kernel"):
        kda.chunk_kda(z, z, z, z, z, A_log=z)
    with pytest.raises(NotImplementedError):
        kda.chunk_kda(z, z, z, z, z, cp_context=object())
    with pytest.raises(ValueError, match="device tensor"):
        kda.chunk_kda(z, z, z, z, z)
    with pytest.raises(ValueError, match="device tensor"):
        kda.chunk_kda_cp(z, z, z, z, z, cp_size=2)
