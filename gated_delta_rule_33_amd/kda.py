"""Python binding of the KDA forward library (libkda.so, C ABI in include/kda.h).

Argument marshalling only: every step of the forward runs in the HIP kernels.
PyTorch supplies device memory and the current stream.  The argument list of
``chunk_kda`` mirrors the chunk_kda entry point of the page "feat(kda):
integrate KDA attention with tokamax backend and CP support" (Public API).
There is no CPU or PyTorch fallback: without the built library, or without a
GPU, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import warnings
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libkda_debug.so")   # same ABI, device checks of preconditions

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_NOT_IMPLEMENTED, KDA_ERR_WORKSPACE_TOO_SMALL, KDA_ERR_HIP = range(5)
KDA_F32, KDA_BF16 = 0, 1
KDA_FLAG_SEGMENT_OVERFLOW = 0x1
KDA_FLAG_FUSED_TIMEOUT = 0x2
KDA_FLAG_GATE_POSITIVE = 0x4   # raised only by libkda_debug.so
KDA_STATIC_WORKSPACE_BYTES = 64 << 20   # the fixed workspace region of kda_chunk_fwd_noalloc, per GPU

EXPORTED = ("kda_chunk_fwd_workspace_size", "kda_chunk_fwd", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_gated",
            "kda_chunk_fwd_transition",
            "kda_chunk_bwd_workspace_size", "kda_chunk_bwd", "kda_chunk_bwd_rerun", "kda_cp_gather_final_grads",
            "kda_cp_chain_bwd", "kda_cp_scatter_initial_grads",
            "kda_chunk_fwd_rerun", "kda_cp_plan", "kda_cp_gather_states", "kda_cp_chain", "kda_cp_scatter_states",
            "kda_short_conv_fwd", "kda_gated_rmsnorm_fwd", "kda_chunk_fwd_flags", "kda_set_launch_observer", "kda_set_fused_forward",
            "kda_last_error", "kda_version")

# void (*)(const char* kernel_name, void* stream, int phase, void* user)
LAUNCH_OBSERVER = ctypes.CFUNCTYPE(None, ctypes.c_char_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p)


class KdaFwdDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("K", ctypes.c_int64), ("V", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("chunk_size", ctypes.c_int32),
                ("use_qk_l2norm", ctypes.c_int32), ("safe_gate", ctypes.c_int32),
                ("lower_bound", ctypes.c_float), ("max_segments", ctypes.c_int32)]


class KdaCpDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("K", ctypes.c_int64), ("V", ctypes.c_int64),
                ("P", ctypes.c_int32), ("n_states", ctypes.c_int32)]


class KdaError(RuntimeError):
    pass


_lib = None


def load_library(path: Optional[str] = None):
    """Load the library once for this process (raises if it has not been
    built): libkda.so, or libkda_debug.so (device checks of the input
    preconditions, reported through the workspace flags) when the
    environment sets KDA_LIBRARY=debug."""
    global _lib
    if _lib is None:
        if path is None:
            path = DEBUG_LIB_PATH if os.environ.get("KDA_LIBRARY", "") == "debug" else LIB_PATH
        _lib = open_library(path)
    return _lib


def open_library(path: str):
    """Open a build of the library (libkda.so or libkda_debug.so) with its
    argument types declared; not cached.  torch is imported first, so that
    the library binds to the HIP runtime torch loaded (torch ships its own
    copy; a process holding two runtimes cannot share device memory between
    them)."""
    import torch  # noqa: F401  (loads torch's HIP runtime before the library's dependency is resolved)
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with gated_delta_rule_33_amd/build.py "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    p, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.kda_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(KdaFwdDesc), ctypes.c_int, ctypes.POINTER(sz)]
    lib.kda_chunk_fwd_workspace_size.restype = ctypes.c_int
    lib.kda_chunk_fwd.argtypes = [ctypes.POINTER(KdaFwdDesc), p, p, p, p, p, p, p, p, p, p, sz, p]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(KdaFwdDesc), p, p, p, p, p, p, p, p, p, p]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_chunk_fwd_gated.argtypes = [ctypes.POINTER(KdaFwdDesc), p, p, p, p, p, p, p, p, p, p, p, p, sz, p]
    lib.kda_chunk_fwd_gated.restype = ctypes.c_int
    lib.kda_chunk_fwd_transition.argtypes = [ctypes.POINTER(KdaFwdDesc), p, p, p, p, p, p, p, p, p, p, p, sz, p]
    lib.kda_chunk_fwd_transition.restype = ctypes.c_int
    lib.kda_chunk_fwd_rerun.argtypes = [ctypes.POINTER(KdaFwdDesc), p, p, p, p, p, sz, p]
    lib.kda_chunk_fwd_rerun.restype = ctypes.c_int
    lib.kda_chunk_bwd_workspace_size.argtypes = [ctypes.POINTER(KdaFwdDesc), ctypes.c_int, ctypes.POINTER(sz)]
    lib.kda_chunk_bwd_workspace_size.restype = ctypes.c_int
    lib.kda_chunk_bwd.argtypes = [ctypes.POINTER(KdaFwdDesc)] + [p] * 16 + [sz, p]
    lib.kda_chunk_bwd.restype = ctypes.c_int
    lib.kda_chunk_bwd_rerun.argtypes = lib.kda_chunk_bwd.argtypes
    lib.kda_chunk_bwd_rerun.restype = ctypes.c_int
    cpd = ctypes.POINTER(KdaCpDesc)
    lib.kda_cp_plan.argtypes = [cpd, p, p, p]
    lib.kda_cp_gather_states.argtypes = [cpd, p, p, p, p, p]
    lib.kda_cp_chain.argtypes = [cpd, p, p, p, p, p]
    lib.kda_cp_scatter_states.argtypes = [cpd, p, p, p, p]
    lib.kda_cp_gather_final_grads.argtypes = [cpd, p, p, p, p, p]
    lib.kda_cp_chain_bwd.argtypes = [cpd, p, p, p, p, p]
    lib.kda_cp_scatter_initial_grads.argtypes = [cpd, p, p, p, p]
    for f in (lib.kda_cp_plan, lib.kda_cp_gather_states, lib.kda_cp_chain, lib.kda_cp_scatter_states,
              lib.kda_cp_gather_final_grads, lib.kda_cp_chain_bwd, lib.kda_cp_scatter_initial_grads):
        f.restype = ctypes.c_int
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.kda_short_conv_fwd.argtypes = [i64, i64, i64, i32, i32, p, p, p, p, p]
    lib.kda_short_conv_fwd.restype = ctypes.c_int
    lib.kda_gated_rmsnorm_fwd.argtypes = [i64, i64, i32, i32, i32, p, p, p, ctypes.c_float, p, p]
    lib.kda_gated_rmsnorm_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_flags.argtypes = [p, sz, p, ctypes.POINTER(ctypes.c_uint32)]
    lib.kda_chunk_fwd_flags.restype = ctypes.c_int
    lib.kda_set_launch_observer.argtypes = [LAUNCH_OBSERVER, ctypes.c_void_p]
    lib.kda_set_launch_observer.restype = None
    lib.kda_set_fused_forward.argtypes = [ctypes.c_int]
    lib.kda_set_fused_forward.restype = None
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_version.restype = ctypes.c_char_p
    return lib


def _raise_for(status: int, what: str):
    if status == KDA_OK:
        return
    msg = f"{what}: {load_library().kda_last_error().decode()}"
    if status == KDA_ERR_NOT_IMPLEMENTED:
        raise NotImplementedError(msg)
    if status == KDA_ERR_INVALID_ARGUMENT:
        raise ValueError(msg)
    raise KdaError(msg)


def make_desc(B, T, H, K, V, dtype, o_dtype, scale=None, use_qk_l2norm=False, safe_gate=False,
              lower_bound=None, max_segments=0, chunk_size=64) -> KdaFwdDesc:
    return KdaFwdDesc(B=B, T=T, H=H, K=K, V=V, dtype=dtype, o_dtype=o_dtype,
                      scale=float("nan") if scale is None else float(scale), chunk_size=chunk_size,
                      use_qk_l2norm=int(bool(use_qk_l2norm)), safe_gate=int(bool(safe_gate)),
                      lower_bound=0.0 if lower_bound is None else float(lower_bound),
                      max_segments=int(max_segments or 0))


def workspace_size(desc: KdaFwdDesc, has_segment_ids: bool) -> int:
    n = ctypes.c_size_t(0)
    _raise_for(load_library().kda_chunk_fwd_workspace_size(ctypes.byref(desc), int(has_segment_ids),
                                                           ctypes.byref(n)), "kda_chunk_fwd_workspace_size")
    return int(n.value)


def _dtype_code(t):
    import torch
    if t == torch.float32:
        return KDA_F32
    if t == torch.bfloat16:
        return KDA_BF16
    raise NotImplementedError(f"dtype {t} is not supported (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def chunk_kda(q, k, v, g, beta, scale: Optional[float] = None, initial_state=None,
              output_final_state: bool = False, chunk_size: int = 64, A_log=None, dt_bias=None,
              use_gate_in_kernel: bool = False, use_qk_l2norm_in_kernel: bool = False,
              safe_gate: bool = False, lower_bound: Optional[float] = None, segment_ids=None,
              disable_recompute: bool = False, N_max: Optional[int] = None, cp_context=None,
              out_dtype=None, workspace=None):
    """KDA chunked forward on the GPU.

    q, k, g: [B,T,H,K]; v: [B,T,H,V]; beta: [B,T,H]; all float32 or all bfloat16,
    contiguous, on one HIP device.  initial_state: fp32 [B,H,K,V] ([B,N_max,H,K,V]
    with segment_ids).  segment_ids: int32 [B,T], 1-based, 0 = padding; needs N_max.
    out_dtype: dtype of o (default float32: see the precision notes of the
    library; bfloat16 rounds the result once more).
    use_gate_in_kernel: g holds raw gate values, activated inside the kernel
    with A_log (fp32 [H] or None) and dt_bias (fp32 [H, K] or None):
    z = exp(A_log) (g + dt_bias), log decay lower_bound * sigmoid(z) with
    safe_gate, log sigmoid(z) without.
    Returns (o, final_state or None).
    """
    import torch
    if (A_log is not None or dt_bias is not None) and not use_gate_in_kernel:
        raise ValueError("A_log and dt_bias are used only with use_gate_in_kernel=True")
    if disable_recompute:
        raise NotImplementedError("disable_recompute is not implemented: the backward (chunk_kda_bwd) always "
                                  "recomputes the chunk quantities")
    if cp_context is not None:
        raise NotImplementedError("context parallelism across devices is not implemented; chunk_kda_cp runs "
                                  "its state chaining with the ranks' slices on one device")
    if lower_bound is not None and not safe_gate:
        warnings.warn("lower_bound is ignored without safe_gate", stacklevel=2)
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype:
            raise ValueError("q, k, v, g and beta must share one dtype")
    B, T, H, K = q.shape
    V = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or tuple(v.shape[:3]) != (B, T, H) or tuple(beta.shape) != (B, T, H):
        raise ValueError("shape mismatch: q, k, g [B,T,H,K], v [B,T,H,V], beta [B,T,H]")
    gate_args = _gate_tensors(use_gate_in_kernel, A_log, dt_bias, H, K, q.device)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    n_max = 0
    if segment_ids is not None:
        if segment_ids.dtype != torch.int32 or tuple(segment_ids.shape) != (B, T) or not segment_ids.is_contiguous():
            raise ValueError("segment_ids must be a contiguous int32 [B, T] tensor")
        if N_max is None or N_max < 1:
            raise ValueError("packed input (segment_ids) needs a positive N_max (max segments per row)")
        n_max = int(N_max)
    desc = make_desc(B, T, H, K, V, _dtype_code(q.dtype), _dtype_code(out_dtype), scale,
                     use_qk_l2norm_in_kernel, safe_gate, lower_bound if safe_gate else None, n_max, chunk_size)
    state_shape = (B, H, K, V) if segment_ids is None else (B, n_max, H, K, V)
    if initial_state is not None:
        if initial_state.dtype != torch.float32 or tuple(initial_state.shape) != state_shape \
                or not initial_state.is_contiguous():
            raise ValueError(f"initial_state must be a contiguous float32 {state_shape} tensor")
    ws_bytes = workspace_size(desc, segment_ids is not None)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty((B, T, H, V), dtype=out_dtype, device=q.device)
    fin = torch.empty(state_shape, dtype=torch.float32, device=q.device) if output_final_state else None
    stream = torch.cuda.current_stream(q.device).cuda_stream
    lib = load_library()
    seg_arg = segment_ids
    if segment_ids is not None and segment_ids.numel() == 0:
        # an empty tensor has no address, and NULL would mean "no segment ids"
        seg_arg = torch.zeros(4, dtype=torch.int32, device=q.device)
    tail = (_ptr(initial_state), _ptr(seg_arg), _ptr(o), _ptr(fin), _ptr(workspace),
            ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream))
    if use_gate_in_kernel:
        st = lib.kda_chunk_fwd_gated(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(gate_args[0]), _ptr(gate_args[1]), *tail)
        _raise_for(st, "kda_chunk_fwd_gated")
    else:
        st = lib.kda_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), *tail)
        _raise_for(st, "kda_chunk_fwd")
    return o, fin


def _gate_tensors(use_gate_in_kernel, A_log, dt_bias, H, K, device):
    """Checked (A_log, dt_bias) for the gated entry point (each None or a
    contiguous fp32 device tensor of shape [H] / [H, K])."""
    import torch
    if not use_gate_in_kernel:
        return None, None
    out = []
    for name, t, shape in (("A_log", A_log, (H,)), ("dt_bias", dt_bias, (H, K))):
        if t is None:
            out.append(None)
            continue
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous() or t.device != device:
            raise ValueError(f"{name} must be a contiguous float32 {shape} tensor on the inputs' device")
        out.append(t)
    return tuple(out)


def short_convolution(x, weight, segment_ids=None, out=None):
    """Causal depthwise short convolution with SiLU (the layer step q, k and v
    pass through before the kernel): x [B, T, D] (fp32 or bf16, contiguous,
    D a multiple of 8), weight [D, W] fp32 (or PyTorch's [D, 1, W]),
    segment_ids None or int32 [B, T].  A tap never reaches before the start
    of its token's segment; padding tokens get 0.  W = 0 disables the
    convolution (x is returned as is)."""
    import torch
    if weight.dim() == 3:
        weight = weight.reshape(weight.shape[0], weight.shape[2])
    D, W = weight.shape
    if W == 0:
        return x
    if x.dim() != 3 or x.shape[2] != D:
        raise ValueError("x must be [B, T, D] with D = weight.shape[0]")
    if not x.is_contiguous() or weight.dtype != torch.float32 or not weight.is_contiguous():
        raise ValueError("x must be contiguous and weight a contiguous float32 [D, W] tensor")
    if segment_ids is not None and (segment_ids.dtype != torch.int32 or tuple(segment_ids.shape) != tuple(x.shape[:2])
                                    or not segment_ids.is_contiguous()):
        raise ValueError("segment_ids must be a contiguous int32 [B, T] tensor")
    B, T, _ = x.shape
    y = torch.empty_like(x) if out is None else out
    stream = torch.cuda.current_stream(x.device).cuda_stream
    _raise_for(load_library().kda_short_conv_fwd(B, T, D, W, _dtype_code(x.dtype), _ptr(x), _ptr(weight),
                                                 _ptr(segment_ids), _ptr(y), ctypes.c_void_p(stream)),
               "kda_short_conv_fwd")
    return y


def gated_rmsnorm(o, gate, weight, eps: float = 1e-6, out_dtype=None, out=None):
    """Output stage after the kernel: per-head RMSNorm over the last axis (V)
    with a sigmoid output gate, y = weight * o / sqrt(mean(o^2) + eps) *
    sigmoid(gate).  o, gate [..., V] (fp32 or bf16, contiguous, same shape),
    weight fp32 [V]; V in {64, 128, 256}."""
    import torch
    if gate.shape != o.shape or not o.is_contiguous() or not gate.is_contiguous():
        raise ValueError("o and gate must be contiguous tensors of one shape")
    V = o.shape[-1]
    if weight.dtype != torch.float32 or tuple(weight.shape) != (V,) or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous float32 [V] tensor")
    out_dtype = o.dtype if out_dtype is None else out_dtype
    y = torch.empty(o.shape, dtype=out_dtype, device=o.device) if out is None else out
    rows = o.numel() // V if V else 0
    stream = torch.cuda.current_stream(o.device).cuda_stream
    _raise_for(load_library().kda_gated_rmsnorm_fwd(rows, V, _dtype_code(o.dtype), _dtype_code(gate.dtype),
                                                    _dtype_code(out_dtype), _ptr(o), _ptr(gate), _ptr(weight),
                                                    float(eps), _ptr(y), ctypes.c_void_p(stream)),
               "kda_gated_rmsnorm_fwd")
    return y


def set_fused_forward(enable: bool) -> None:
    """Select the forward schedule for later calls (process-wide): the fused
    persistent kernel where it applies, or always the two-kernel path
    (intra-chunk kernel, then recurrence kernel; the default)."""
    load_library().kda_set_fused_forward(1 if enable else 0)


def set_launch_observer(fn):
    """Install fn(kernel_name: str, stream: int, phase: int) around every kernel
    launch (None removes it).  Returns the ctypes callback, which the caller
    must keep alive while it is installed."""
    lib = load_library()
    if fn is None:
        lib.kda_set_launch_observer(LAUNCH_OBSERVER(), None)
        return None
    cb = LAUNCH_OBSERVER(lambda name, stream, phase, user: fn(name.decode(), stream, phase))
    lib.kda_set_launch_observer(cb, None)
    return cb


class PreparedCall:
    """kda_chunk_fwd (or kda_chunk_fwd_gated) with every argument marshalled
    once: ``enqueue()`` only crosses the C ABI (for timing loops).  Holds
    references to its tensors."""

    def __init__(self, desc: KdaFwdDesc, tensors: dict, workspace, stream: int, gated: bool = False):
        self.desc, self.tensors, self.workspace = desc, tensors, workspace
        names = ("q", "k", "v", "g", "beta") + (("A_log", "dt_bias") if gated else ()) + \
            ("initial_state", "segment_ids", "o", "final_state")
        self.args = [ctypes.byref(desc)] + [_ptr(tensors.get(n)) for n in names] + \
            [_ptr(workspace), ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream)]
        lib = load_library()
        self.fn = lib.kda_chunk_fwd_gated if gated else lib.kda_chunk_fwd

    def enqueue(self):
        _raise_for(self.fn(*self.args), "kda_chunk_fwd")


def prepare_call(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=False,
                 use_qk_l2norm_in_kernel=False, safe_gate=False, lower_bound=None, segment_ids=None,
                 N_max=None, out_dtype=None, use_gate_in_kernel=False, A_log=None,
                 dt_bias=None) -> PreparedCall:
    """Allocate o, final state and workspace for one shape and return a
    PreparedCall that enqueues the forward on the current stream."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    B, T, H, K = q.shape
    V = v.shape[-1]
    n_max = int(N_max) if segment_ids is not None else 0
    desc = make_desc(B, T, H, K, V, _dtype_code(q.dtype), _dtype_code(out_dtype), scale, use_qk_l2norm_in_kernel,
                     safe_gate, lower_bound if safe_gate else None, n_max)
    ws = torch.empty(max(workspace_size(desc, segment_ids is not None), 1), dtype=torch.uint8, device=q.device)
    state_shape = (B, H, K, V) if segment_ids is None else (B, n_max, H, K, V)
    a_log, dt_b = _gate_tensors(use_gate_in_kernel, A_log, dt_bias, H, K, q.device)
    t = dict(q=q, k=k, v=v, g=g, beta=beta, A_log=a_log, dt_bias=dt_b, initial_state=initial_state,
             segment_ids=segment_ids, o=torch.empty((B, T, H, V), dtype=out_dtype, device=q.device),
             final_state=torch.empty(state_shape, dtype=torch.float32, device=q.device) if output_final_state
             else None)
    return PreparedCall(desc, t, ws, torch.cuda.current_stream(q.device).cuda_stream,
                        gated=bool(use_gate_in_kernel))


def read_flags(workspace) -> int:
    """Synchronise the current stream and read the KDA_FLAG_* word of a workspace."""
    import torch
    flags = ctypes.c_uint32(0)
    stream = torch.cuda.current_stream(workspace.device).cuda_stream
    _raise_for(load_library().kda_chunk_fwd_flags(_ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                                  ctypes.c_void_p(stream), ctypes.byref(flags)),
               "kda_chunk_fwd_flags")
    return int(flags.value)


def chunk_kda_bwd(q, k, v, g, beta, d_o, scale: Optional[float] = None, initial_state=None, d_final_state=None,
                  use_qk_l2norm_in_kernel: bool = False, segment_ids=None, N_max: Optional[int] = None,
                  want_d_initial_state: bool = True, workspace=None):
    """Gradients of chunk_kda (g as the log decay) for the loss
    sum(o * d_o) + sum(final_state * d_final_state): returns fp32
    (dq, dk, dv, dg, dbeta, d_initial_state or None).  Inputs as for
    chunk_kda; d_o [B,T,H,V] fp32 or bf16; d_final_state None or fp32 in the
    state shape."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a contiguous device tensor of q's dtype")
    B, T, H, K = q.shape
    V = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or tuple(v.shape[:3]) != (B, T, H) or tuple(beta.shape) != (B, T, H):
        raise ValueError("shape mismatch: q, k, g [B,T,H,K], v [B,T,H,V], beta [B,T,H]")
    if tuple(d_o.shape) != (B, T, H, V) or not d_o.is_contiguous():
        raise ValueError("d_o must be a contiguous [B,T,H,V] tensor")
    n_max = 0
    if segment_ids is not None:
        if segment_ids.dtype != torch.int32 or tuple(segment_ids.shape) != (B, T) or not segment_ids.is_contiguous():
            raise ValueError("segment_ids must be a contiguous int32 [B, T] tensor")
        if N_max is None or N_max < 1:
            raise ValueError("packed input (segment_ids) needs a positive N_max (max segments per row)")
        n_max = int(N_max)
    state_shape = (B, H, K, V) if segment_ids is None else (B, n_max, H, K, V)
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != state_shape or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 {state_shape} tensor")
    desc = make_desc(B, T, H, K, V, _dtype_code(q.dtype), _dtype_code(d_o.dtype), scale, use_qk_l2norm_in_kernel,
                     False, None, n_max)
    lib = load_library()
    n = ctypes.c_size_t(0)
    _raise_for(lib.kda_chunk_bwd_workspace_size(ctypes.byref(desc), int(segment_ids is not None), ctypes.byref(n)),
               "kda_chunk_bwd_workspace_size")
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=q.device)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq, dk, dg = (torch.empty((B, T, H, K), **f32) for _ in range(3))
    dv = torch.empty((B, T, H, V), **f32)
    dbeta = torch.empty((B, T, H), **f32)
    d_init = torch.empty(state_shape, **f32) if want_d_initial_state else None
    seg_arg = segment_ids
    if segment_ids is not None and segment_ids.numel() == 0:
        seg_arg = torch.zeros(4, dtype=torch.int32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.kda_chunk_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                           _ptr(seg_arg), _ptr(d_o), _ptr(d_final_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                           _ptr(dbeta), _ptr(d_init), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                           ctypes.c_void_p(stream))
    _raise_for(st, "kda_chunk_bwd")
    return dq, dk, dv, dg, dbeta, d_init


def _autograd_function():
    import torch

    class ChunkKDA(torch.autograd.Function):
        """chunk_kda with its backward (kda_chunk_bwd) for torch autograd.
        Gradients come back in fp32 and are cast to each input's dtype."""

        @staticmethod
        def forward(ctx, q, k, v, g, beta, initial_state, scale, use_qk_l2norm_in_kernel, segment_ids, N_max):
            o, fin = chunk_kda(q, k, v, g, beta, scale=scale, initial_state=initial_state, output_final_state=True,
                               use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel, segment_ids=segment_ids,
                               N_max=N_max)
            ctx.save_for_backward(q, k, v, g, beta, initial_state, segment_ids)
            ctx.opts = (scale, use_qk_l2norm_in_kernel, N_max)
            return o, fin

        @staticmethod
        def backward(ctx, d_o, d_fin):
            q, k, v, g, beta, init, seg = ctx.saved_tensors
            scale, l2, n_max = ctx.opts
            d_o = torch.zeros_like(q[..., :1].expand(*q.shape[:3], v.shape[-1]), dtype=torch.float32) \
                if d_o is None else d_o.contiguous()
            d_fin = None if d_fin is None else d_fin.contiguous().float()
            dq, dk, dv, dg, db, dinit = chunk_kda_bwd(q, k, v, g, beta, d_o, scale=scale, initial_state=init,
                                                      d_final_state=d_fin, use_qk_l2norm_in_kernel=l2,
                                                      segment_ids=seg, N_max=n_max,
                                                      want_d_initial_state=init is not None)
            return (dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dg.to(g.dtype), db.to(beta.dtype), dinit,
                    None, None, None, None)

    return ChunkKDA


def chunk_kda_autograd(q, k, v, g, beta, initial_state=None, scale: Optional[float] = None,
                       use_qk_l2norm_in_kernel: bool = False, segment_ids=None, N_max: Optional[int] = None):
    """chunk_kda as a differentiable torch op: returns (o, final_state), and
    backward() runs kda_chunk_bwd."""
    return _autograd_function().apply(q, k, v, g, beta, initial_state, scale, use_qk_l2norm_in_kernel,
                                      segment_ids, N_max)


class CpCall:
    """The context-parallel forward of ``chunk_kda_cp`` with every buffer
    allocated and every argument marshalled once; ``enqueue()`` makes the
    seven C-ABI calls on the current stream (for timing loops too)."""

    def __init__(self, q, k, v, g, beta, cp_size: int, scale=None, initial_state=None,
                 output_final_state=False, use_qk_l2norm_in_kernel=False, safe_gate=False, lower_bound=None,
                 segment_ids=None, N_max=None, out_dtype=None):
        import torch
        for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
            if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
                raise ValueError(f"{name} must be a contiguous device tensor of q's dtype")
        B, T, H, K = q.shape
        V = v.shape[-1]
        if k.shape != q.shape or g.shape != q.shape or tuple(v.shape[:3]) != (B, T, H) \
                or tuple(beta.shape) != (B, T, H):
            raise ValueError("shape mismatch: q, k, g [B,T,H,K], v [B,T,H,V], beta [B,T,H]")
        P = int(cp_size)
        if P < 1 or T == 0 or T % P != 0:
            raise ValueError("cp_size must be >= 1 and divide T >= 1")
        L = T // P
        out_dtype = torch.float32 if out_dtype is None else out_dtype
        packed = segment_ids is not None
        if packed:
            if segment_ids.dtype != torch.int32 or tuple(segment_ids.shape) != (B, T) \
                    or not segment_ids.is_contiguous():
                raise ValueError("segment_ids must be a contiguous int32 [B, T] tensor")
            if N_max is None or N_max < 1:
                raise ValueError("packed input (segment_ids) needs a positive N_max (max segments per row)")
        nm = int(N_max) if packed else 1
        gshape = (B, H, K, V) if not packed else (B, nm, H, K, V)
        if initial_state is not None and (initial_state.dtype != torch.float32
                                          or tuple(initial_state.shape) != gshape
                                          or not initial_state.is_contiguous()):
            raise ValueError(f"initial_state must be a contiguous float32 {gshape} tensor")
        dev = q.device
        rows = B * P
        lshape = (rows, H, K, V) if not packed else (rows, nm, H, K, V)
        f32 = dict(dtype=torch.float32, device=dev)
        self.plan = torch.empty((B, P, 4), dtype=torch.int32, device=dev)
        self.local_init = torch.empty(lshape, **f32)
        self.local_fin = torch.empty(lshape, **f32)
        self.transition = torch.empty((rows, H, K, K), **f32)
        self.carry = torch.empty((rows, H, K, V), **f32)
        self.o = torch.empty((B, T, H, V), dtype=out_dtype, device=dev)
        self.final_state = torch.empty(gshape, **f32) if output_final_state else None
        self.cp = KdaCpDesc(B=B, T=T, H=H, K=K, V=V, P=P, n_states=nm)
        self.desc = make_desc(rows, L, H, K, V, _dtype_code(q.dtype), _dtype_code(out_dtype), scale,
                              use_qk_l2norm_in_kernel, safe_gate, lower_bound if safe_gate else None,
                              nm if packed else 0)
        ws_bytes = max(workspace_size(self.desc, packed), 1)
        self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        self.views = [t.view((rows, L) + tuple(t.shape[2:])) for t in (q, k, v, g, beta)]
        self.keep = (q, k, v, g, beta, initial_state, segment_ids)
        self.packed, self.gshape, self.lshape, self.dev = packed, gshape, lshape, dev
        seg_local = segment_ids.view(rows, L) if packed else None
        self.seg_local = seg_local
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        cp, d, ws = ctypes.byref(self.cp), ctypes.byref(self.desc), (_ptr(self.workspace), ctypes.c_size_t(ws_bytes))
        lib = load_library()
        plan, init = _ptr(self.plan), _ptr(initial_state)
        self.steps = [
            (lib.kda_cp_plan, (cp, _ptr(segment_ids), plan, stream)),
            (lib.kda_cp_gather_states, (cp, plan, init, None, _ptr(self.local_init), stream)),
            (lib.kda_chunk_fwd_transition, (d, *[_ptr(t) for t in self.views], _ptr(self.local_init),
                                            _ptr(seg_local), _ptr(self.o), _ptr(self.local_fin),
                                            _ptr(self.transition), *ws, stream)),
            (lib.kda_cp_chain, (cp, plan, _ptr(self.local_fin), _ptr(self.transition), _ptr(self.carry), stream)),
            (lib.kda_cp_gather_states, (cp, plan, init, _ptr(self.carry), _ptr(self.local_init), stream)),
            (lib.kda_chunk_fwd_rerun, (d, _ptr(self.local_init), _ptr(seg_local), _ptr(self.o),
                                       _ptr(self.local_fin), *ws, stream)),
        ]
        if output_final_state:
            self.steps.append((lib.kda_cp_scatter_states, (cp, plan, _ptr(self.local_fin), _ptr(self.final_state),
                                                           stream)))

    def enqueue(self):
        for fn, args in self.steps:
            _raise_for(fn(*args), fn.__name__)

    def backward(self, d_o, d_final_state=None, want_d_initial_state=True):
        """The gradients of sum(o * d_o) + sum(final_state * d_final_state)
        under the same slicing, after enqueue(): each slice's backward, the
        reverse chain of hand-off gradients, the backward again on the same
        workspace.  Returns fp32 (dq, dk, dv, dg, dbeta, d_initial_state)."""
        import torch
        q, k, v, g, beta, init, _ = self.keep
        B, T, H, K = q.shape
        V = v.shape[-1]
        rows, L = self.desc.B, self.desc.T
        if tuple(d_o.shape) != (B, T, H, V) or not d_o.is_contiguous():
            raise ValueError("d_o must be a contiguous [B,T,H,V] tensor")
        if d_final_state is not None and (d_final_state.dtype != torch.float32 or not d_final_state.is_contiguous()
                                          or tuple(d_final_state.shape) != self.gshape):
            raise ValueError(f"d_final_state must be a contiguous float32 {self.gshape} tensor")
        lib = load_library()
        stream = ctypes.c_void_p(torch.cuda.current_stream(self.dev).cuda_stream)
        f32 = dict(dtype=torch.float32, device=self.dev)
        desc = make_desc(rows, L, H, K, V, self.desc.dtype, _dtype_code(d_o.dtype), self.desc.scale,
                         bool(self.desc.use_qk_l2norm), False, None, self.desc.max_segments)
        n = ctypes.c_size_t(0)
        _raise_for(lib.kda_chunk_bwd_workspace_size(ctypes.byref(desc), int(self.packed), ctypes.byref(n)),
                   "kda_chunk_bwd_workspace_size")
        ws = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=self.dev)
        dq, dk, dg = (torch.empty((B, T, H, K), **f32) for _ in range(3))
        dv = torch.empty((B, T, H, V), **f32)
        dbeta = torch.empty((B, T, H), **f32)
        local_dfin = torch.empty(self.lshape, **f32)
        local_dinit = torch.empty(self.lshape, **f32)
        xg = torch.empty((rows, H, K, V), **f32)
        cp, plan = ctypes.byref(self.cp), _ptr(self.plan)
        grads = [_ptr(t.view((rows, L) + tuple(t.shape[2:]))) for t in (dq, dk, dv, dg, dbeta)]
        bwd_args = (ctypes.byref(desc), *[_ptr(t) for t in self.views], _ptr(self.local_init), _ptr(self.seg_local),
                    _ptr(d_o.view(rows, L, H, V)), _ptr(local_dfin), *grads, _ptr(local_dinit), _ptr(ws),
                    ctypes.c_size_t(ws.numel()), stream)
        _raise_for(lib.kda_cp_gather_final_grads(cp, plan, _ptr(d_final_state), None, _ptr(local_dfin), stream),
                   "kda_cp_gather_final_grads")
        _raise_for(lib.kda_chunk_bwd(*bwd_args), "kda_chunk_bwd")
        _raise_for(lib.kda_cp_chain_bwd(cp, plan, _ptr(local_dinit), _ptr(self.transition), _ptr(xg), stream),
                   "kda_cp_chain_bwd")
        _raise_for(lib.kda_cp_gather_final_grads(cp, plan, _ptr(d_final_state), _ptr(xg), _ptr(local_dfin), stream),
                   "kda_cp_gather_final_grads")
        _raise_for(lib.kda_chunk_bwd_rerun(*bwd_args), "kda_chunk_bwd_rerun")
        d_init = None
        if want_d_initial_state:
            d_init = torch.empty(self.gshape, **f32)
            _raise_for(lib.kda_cp_scatter_initial_grads(cp, plan, _ptr(local_dinit), _ptr(d_init), stream),
                       "kda_cp_scatter_initial_grads")
        return dq, dk, dv, dg, dbeta, d_init


def chunk_kda_cp(q, k, v, g, beta, cp_size: int, scale: Optional[float] = None, initial_state=None,
                 output_final_state: bool = False, use_qk_l2norm_in_kernel: bool = False, safe_gate: bool = False,
                 lower_bound: Optional[float] = None, segment_ids=None, N_max: Optional[int] = None,
                 out_dtype=None, return_internals: bool = False):
    """The forward with T cut into cp_size equal slices, one per
    context-parallel rank, and the recurrent state carried across the cuts
    (the state chaining of the page "feat(kda): integrate KDA attention with
    tokamax backend and CP support", Context Parallelism Support), all
    slices on one device.  Arguments and results are those of chunk_kda
    (T must be a multiple of cp_size); the result equals the unsplit forward
    up to rounding.  The C-ABI steps, in order: plan, gather (zero carried
    states), forward with transitions, chain, gather (chained states), rerun
    of the recurrence, scatter of the final states.
    With return_internals, also returns a dict with the plan [B, P, 4], the
    transitions [B*P, H, K, K] and the chained states [B*P, H, K, V]."""
    if lower_bound is not None and not safe_gate:
        warnings.warn("lower_bound is ignored without safe_gate", stacklevel=2)
    call = CpCall(q, k, v, g, beta, cp_size, scale, initial_state, output_final_state, use_qk_l2norm_in_kernel,
                  safe_gate, lower_bound, segment_ids, N_max, out_dtype)
    call.enqueue()
    if return_internals:
        return call.o, call.final_state, dict(plan=call.plan, transition=call.transition, carry=call.carry)
    return call.o, call.final_state
