"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a private copy of the oracle's C source
(CPU only), builds it, swaps it in for the real oracle and runs every pin in
``test_oracle_pins``; at least one pin must fail for every planted mistake.
"""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

_OUT_LOOP = """    /* o_t = scale q_t^T S */
    for (int64_t x = 0; x < V; ++x) {
      REAL acc = 0;
      for (int64_t c = 0; c < K; ++c) acc += qq[c] * S[c * V + x];
      orow[x] = (double)((REAL)j->scale * acc);
    }
"""

MUTATIONS = {
    "residual sign": ("r[x] = (REAL)j->v[v_off + x] - acc;", "r[x] = (REAL)j->v[v_off + x] + acc;"),
    "beta dropped": ("const REAL w = bt * kk[c];", "const REAL w = kk[c];"),
    "decay on value axis": ("for (int64_t x = 0; x < V; ++x) row[x] *= d;",
                            "for (int64_t x = 0; x < V; ++x) S[x * V + c] *= d;"),
    "decay sign": ("const REAL d = rexp(gate_log_decay(j, h, c, (REAL)j->g[qk_off + c]));",
                   "const REAL d = rexp(-gate_log_decay(j, h, c, (REAL)j->g[qk_off + c]));"),
    "gate sigmoid mirrored": ("const REAL sig = (REAL)1 / ((REAL)1 + rexp(-z));",
                              "const REAL sig = (REAL)1 / ((REAL)1 + rexp(z));"),
    "gate A_log not exponentiated": ("const REAL a = j->a_log ? rexp((REAL)j->a_log[h]) : (REAL)1;",
                                     "const REAL a = j->a_log ? (REAL)j->a_log[h] : (REAL)1;"),
    "gate dt_bias dropped": ("(j->dt_bias ? (REAL)j->dt_bias[h * j->K + c] : (REAL)0)", "((REAL)0)"),
    "gate dt_bias per head only": ("(REAL)j->dt_bias[h * j->K + c]", "(REAL)j->dt_bias[h * j->K]"),
    "gate lower bound dropped": ("if (j->gate_mode == 2) return (REAL)j->lower_bound * sig;",
                                 "if (j->gate_mode == 2) return -sig;"),
    "gate log dropped": ("return (REAL)log((double)sig);", "return -sig;"),
    "decay skipped": ("row[x] *= d;", "row[x] *= (REAL)1;"),
    "residual on transposed state": ("for (int64_t c = 0; c < K; ++c) acc += kk[c] * S[c * V + x];",
                                     "for (int64_t c = 0; c < K; ++c) acc += kk[c] * S[x * V + c];"),
    "no segment restart": ("if (t == 0 || s != prev) {", "if (t == 0) {"),
    "padding keeps segment open": ("      prev = 0;\n      continue;", "      continue;"),
    "l2 norm inverted": ("qq[c] /= nq; kk[c] /= nk;", "qq[c] *= nq; kk[c] *= nk;"),
    "scale dropped": ("orow[x] = (double)((REAL)j->scale * acc);", "orow[x] = (double)(acc);"),
    "read-out before write": (None, None),
    "initial state ignored": ("for (int64_t i = 0; i < n; ++i) S[i] = (REAL)src[i];",
                              "for (int64_t i = 0; i < n; ++i) S[i] = (REAL)0 * src[i];"),
    "final state of first segment kept": ("if (live) store_state(j, b, seg, h, S);\n      seg += 1;",
                                          "seg += 1;"),
}


def _mutant_source(name):
    src = open(SRC).read()
    if name == "read-out before write":
        assert _OUT_LOOP in src
        src = src.replace(_OUT_LOOP, "")
        anchor = "    /* S = S' + beta_t k_t residual^T */\n"
        assert anchor in src
        return src.replace(anchor, _OUT_LOOP + anchor)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name!r} not unique"
    return src.replace(old, new)


def _build(src_text, real, out_dir, tag):
    c = os.path.join(out_dir, f"{tag}_{real}.c")
    so = os.path.join(out_dir, f"{tag}_{real}.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", f"-DREAL={real}", "-o", so, c,
                    "-lm", "-lpthread"], check=True)
    return so


def _pin_functions():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argname, values = params[0].args
            for val in values:
                out.append((f"{name}[{val}]", lambda fn=fn, a=argname, v=val: fn(**{a: v})))
        else:
            out.append((name, fn))
    return out


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_planted_mistake_fails_a_pin(mutation, tmp_path, monkeypatch):
    src = _mutant_source(mutation)
    tag = mutation.replace(" ", "_")
    libs = {}
    for prec, real in (("f64", "double"), ("f32", "float")):
        lib = ctypes.CDLL(_build(src, real, str(tmp_path), tag))
        ref = oracle._lib(prec)
        for fn_name in ("kda_oracle_fwd", "kda_oracle_fwd_gate"):
            getattr(lib, fn_name).argtypes = getattr(ref, fn_name).argtypes
            getattr(lib, fn_name).restype = ctypes.c_int
        lib.kda_oracle_real_bytes.restype = ctypes.c_int
        libs[prec] = lib
    monkeypatch.setattr(oracle, "_loaded", libs)
    failed = []
    for name, fn in _pin_functions():
        try:
            fn()
        except (KeyboardInterrupt, SystemExit):
            raise
        except BaseException:      # an assertion, or pytest.raises/fail outcomes
            failed.append(name)
    assert failed, f"no pin caught the planted mistake {mutation!r}"
