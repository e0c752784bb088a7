"""CPU oracle for the KDA chunked forward (TEST INFRASTRUCTURE ONLY).

The oracle is the token-by-token gated delta rule written out plainly in C
(``kda_oracle.c``), compiled twice from the same source: an fp64 build (the
reference every parity check uses) and an fp32 build (to measure how far a
plain fp32 evaluation sits from fp64).  It follows the "Delta Rule
formulation" of the page "feat(kda): integrate KDA attention with tokamax
backend and CP support" (Implementation Details) and the chunk_kda options of
its Public API section.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``gated_delta_rule_33_amd/`` and never imports it.

The backward (``kda_oracle_bwd.c``, ``kda_backward``) is the reverse mode of
the same token loop, written out by hand.

Parity pins: the forward is pinned by ``tests/test_oracle_pins.py`` (closed
forms, a transition-matrix product form, a chunk-size-independent block
evaluation, invariants), the backward by ``tests/test_oracle_bwd_pins.py``
(finite differences of the forward, closed forms).  No part is left
unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIBS = {"f64": os.path.join(_HERE, "libkda_oracle_f64.so"),
         "f32": os.path.join(_HERE, "libkda_oracle_f32.so")}
_BWD_SRC = os.path.join(_HERE, "kda_oracle_bwd.c")
_BWD_LIBS = {"f64": os.path.join(_HERE, "libkda_oracle_bwd_f64.so"),
             "f32": os.path.join(_HERE, "libkda_oracle_bwd_f32.so")}
_REAL = {"f64": "double", "f32": "float"}
_loaded: dict = {}
_bwd_loaded: dict = {}

ORACLE_ERRORS = {1: "bad arguments", 2: "more segments in a row than n_max", 3: "out of memory"}


def build(force: bool = True) -> None:
    """Compile both builds of the forward and backward oracles with gcc (plain
    -O2: no fast-math, no reordering)."""
    for src, libs in ((_SRC, _LIBS), (_BWD_SRC, _BWD_LIBS)):
        for prec, out in libs.items():
            if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
                continue
            tmp = out + ".tmp"
            subprocess.run(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                            f"-DREAL={_REAL[prec]}", "-o", tmp, src, "-lm", "-lpthread"],
                           check=True)
            os.replace(tmp, out)


def _lib(prec: str):
    if prec not in _loaded:
        path = _LIBS[prec]
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(force=False)
        lib = ctypes.CDLL(path)
        fn = lib.kda_oracle_fwd
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        fn.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, ctypes.c_double, ctypes.c_int,
                       p, p, i64, p, p, ctypes.c_int]
        fn.restype = ctypes.c_int
        fg = lib.kda_oracle_fwd_gate
        fg.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, ctypes.c_double, ctypes.c_int,
                       ctypes.c_int, ctypes.c_double, p, p, p, p, i64, p, p, ctypes.c_int]
        fg.restype = ctypes.c_int
        lib.kda_oracle_real_bytes.restype = ctypes.c_int
        _loaded[prec] = lib
    return _loaded[prec]


def _bwd_lib(prec: str):
    if prec not in _bwd_loaded:
        path = _BWD_LIBS[prec]
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_BWD_SRC):
            build(force=False)
        lib = ctypes.CDLL(path)
        p, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.kda_oracle_bwd.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, ctypes.c_double, ctypes.c_int,
                                       p, p, i64, p, p, p, p, p, p, p, p, ctypes.c_int]
        lib.kda_oracle_bwd.restype = ctypes.c_int
        _bwd_loaded[prec] = lib
    return _bwd_loaded[prec]


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count() or 1)


def kda_forward(q, k, v, g, beta, scale: Optional[float] = None, initial_state=None,
                output_final_state: bool = False, use_qk_l2norm: bool = False,
                segment_ids=None, max_segments: int = 0, precision: str = "f64",
                num_threads: Optional[int] = None, use_gate_in_kernel: bool = False,
                A_log=None, dt_bias=None, safe_gate: bool = False,
                lower_bound: Optional[float] = None):
    """Token-by-token KDA forward on the CPU.

    q, k, g: [B,T,H,K]; v: [B,T,H,V]; beta: [B,T,H]; all converted to fp32
    (callers pass the exact values the GPU sees).  initial_state: None, or fp32
    [B,H,K,V] (no segment_ids) / [B,max_segments,H,K,V] (with segment_ids).
    segment_ids: None or int32 [B,T], 1-based, 0 = padding.
    use_gate_in_kernel: g holds raw gate values, activated with A_log (fp32
    [H] or None) and dt_bias (fp32 [H,K] or None) as described in
    kda_oracle.c: lower_bound * sigmoid(z) with safe_gate, log sigmoid(z)
    without.
    Returns (o, final_state_or_None) as float64 arrays.
    """
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    q, k, v, g, beta = f32(q), f32(k), f32(v), f32(g), f32(beta)
    B, T, H, K = q.shape
    V = v.shape[-1]
    if k.shape != (B, T, H, K) or g.shape != (B, T, H, K) or v.shape[:3] != (B, T, H) \
            or beta.shape != (B, T, H):
        raise ValueError("shape mismatch among q, k, v, g, beta")
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    seg = None if segment_ids is None else np.ascontiguousarray(segment_ids, dtype=np.int32)
    if seg is not None and seg.shape != (B, T):
        raise ValueError("segment_ids must be [B, T]")
    if seg is not None and (initial_state is not None or output_final_state) and max_segments < 1:
        raise ValueError("max_segments must be >= 1 with segment_ids and states")
    state_shape = (B, H, K, V) if seg is None else (B, max_segments, H, K, V)
    init = None
    if initial_state is not None:
        init = f32(initial_state)
        if init.shape != state_shape:
            raise ValueError(f"initial_state must be {state_shape}")
    a_log = dtb = None
    gate_mode, lb = 0, 0.0
    if use_gate_in_kernel:
        gate_mode = 2 if safe_gate else 1
        if safe_gate:
            if lower_bound is None:
                raise ValueError("the safe gate needs a lower_bound")
            lb = float(lower_bound)
        if A_log is not None:
            a_log = f32(A_log)
            if a_log.shape != (H,):
                raise ValueError("A_log must be [H]")
        if dt_bias is not None:
            dtb = f32(dt_bias)
            if dtb.shape != (H, K):
                raise ValueError("dt_bias must be [H, K]")
    elif A_log is not None or dt_bias is not None:
        raise ValueError("A_log and dt_bias need use_gate_in_kernel")
    o = np.zeros((B, T, H, V), dtype=np.float64)
    fin = np.zeros(state_shape, dtype=np.float64) if output_final_state else None
    if num_threads is None:
        num_threads = default_threads()
    rc = _lib(precision).kda_oracle_fwd_gate(B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                              _ptr(beta), float(scale), int(bool(use_qk_l2norm)),
                                              gate_mode, lb, _ptr(a_log), _ptr(dtb),
                                              _ptr(init), _ptr(seg), int(max_segments), _ptr(o),
                                              _ptr(fin), int(num_threads))
    if rc != 0:
        raise ValueError(f"oracle: {ORACLE_ERRORS.get(rc, rc)}")
    return o, fin


def kda_backward(q, k, v, g, beta, d_o, scale: Optional[float] = None, initial_state=None, d_final_state=None,
                 use_qk_l2norm: bool = False, segment_ids=None, max_segments: int = 0,
                 want_d_initial_state: bool = True, precision: str = "f64", num_threads: Optional[int] = None):
    """Gradients of the token-by-token KDA forward (``kda_oracle_bwd.c``).

    The loss is sum(o * d_o) + sum(final_state * d_final_state); inputs as
    for ``kda_forward`` (converted to fp32), d_o [B,T,H,V] and d_final_state
    (None = zero, else the state shape) in fp64.  Returns a dict of float64
    arrays dq, dk, dv, dg, dbeta and d_initial_state (None unless wanted).
    """
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    f64 = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    q, k, v, g, beta = f32(q), f32(k), f32(v), f32(g), f32(beta)
    B, T, H, K = q.shape
    V = v.shape[-1]
    d_o = f64(d_o)
    if d_o.shape != (B, T, H, V):
        raise ValueError("d_o must be [B,T,H,V]")
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    seg = None if segment_ids is None else np.ascontiguousarray(segment_ids, dtype=np.int32)
    state_shape = (B, H, K, V) if seg is None else (B, max_segments, H, K, V)
    init = None if initial_state is None else f32(initial_state)
    dfin = None if d_final_state is None else f64(d_final_state)
    for name, a in (("initial_state", init), ("d_final_state", dfin)):
        if a is not None and a.shape != state_shape:
            raise ValueError(f"{name} must be {state_shape}")
    out = {n: np.zeros(a.shape) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    dinit = np.zeros(state_shape) if want_d_initial_state else None
    if num_threads is None:
        num_threads = default_threads()
    rc = _bwd_lib(precision).kda_oracle_bwd(B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                            float(scale), int(bool(use_qk_l2norm)), _ptr(init), _ptr(seg),
                                            int(max_segments), _ptr(d_o), _ptr(dfin), _ptr(out["dq"]),
                                            _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
                                            _ptr(dinit), int(num_threads))
    if rc != 0:
        raise ValueError(f"oracle: {ORACLE_ERRORS.get(rc, rc)}")
    out["d_initial_state"] = dinit
    return out


def forward_inputs(inp: dict, workload, precision: str = "f64", num_threads: Optional[int] = None,
                   segment_ids="workload"):
    """Run the oracle on a dict produced by ``gated_delta_rule_33_amd.inputs.make_inputs``."""
    seg = inp["segment_ids"] if isinstance(segment_ids, str) else segment_ids
    return kda_forward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], scale=inp["scale"],
                       initial_state=inp["initial_state"], output_final_state=workload.final_state,
                       use_qk_l2norm=workload.l2norm_in_kernel, segment_ids=seg,
                       max_segments=inp["max_segments"], precision=precision,
                       num_threads=num_threads)


def rel_err(x, ref, mask=None) -> float:
    """max|x - ref| / rms(ref) in fp64, optionally over a boolean mask of elements."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        x, ref = x[mask], ref[mask]
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(x - ref)))
    if rms == 0.0:
        return 0.0 if err == 0.0 else float("inf")
    return err / rms
