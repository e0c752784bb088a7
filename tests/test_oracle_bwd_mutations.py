"""The backward oracle's pins must catch plausible mistakes.

Each case plants one mistake in a private copy of kda_oracle_bwd.c (CPU
only), builds it, swaps it in for the real backward oracle and runs every pin
of ``test_oracle_bwd_pins``; at least one pin must fail for every mistake.
"""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_bwd_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle_bwd.c")

MUTATIONS = {
    "read-out gradient sign": ("dS[c * V + x] += sc * qq[c] * (REAL)dot[x];",
                               "dS[c * V + x] -= sc * qq[c] * (REAL)dot[x];"),
    "read-out from the previous state": ("acc += St[c * V + x] * (REAL)dot[x];",
                                         "acc += Sprev[c * V + x] * (REAL)dot[x];"),
    "scale dropped from dq": ("dqq[c] = sc * acc;", "dqq[c] = acc;"),
    "beta dropped from dk": ("dkk[c] = bt * acc;", "dkk[c] = acc;"),
    "beta dropped from dr": ("dr[x] = bt * acc;", "dr[x] = acc;"),
    "residual term dropped from dS": ("dS[c * V + x] -= kk[c] * dr[x];", "dS[c * V + x] -= 0 * kk[c] * dr[x];"),
    "state term dropped from dk": ("dkk[c] -= acc;", "dkk[c] -= 0 * acc;"),
    "dg from the undecayed state": ("acc += dS[c * V + x] * Sa[c * V + x];",
                                    "acc += dS[c * V + x] * Sprev[c * V + x];"),
    "decay not carried into dS": ("dS[c * V + x] *= d;", "dS[c * V + x] *= (REAL)1;"),
    "l2 norm projection dropped": ("tmp[c] = dx[c] / nn - (REAL)x[qk + c] * xd / (nn * nn * nn);",
                                   "tmp[c] = dx[c] / nn;"),
    "final-state gradient ignored": ("dS[i] = j->d_final ? (REAL)j->d_final[slot(j, b, seg, h) + i] : (REAL)0;",
                                     "dS[i] = (REAL)0;"),
    "segments run through id changes": ("while (e < j->T && ids[e] == ids[t]) ++e;",
                                        "while (e < j->T && ids[e] != 0) ++e;"),
    "dbeta without the key": ("db += kk[c] * acc;", "db += acc;"),
}


def _build(src_text, real, out_dir, tag):
    c = os.path.join(out_dir, f"{tag}_{real}.c")
    so = os.path.join(out_dir, f"{tag}_{real}.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", f"-DREAL={real}", "-o", so, c, "-lm",
                    "-lpthread"], check=True)
    return so


def _pins():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if params:
            argnames, values = params[0].args
            names = [a.strip() for a in argnames.split(",")]
            for val in values:
                val = val if isinstance(val, tuple) else (val,)
                out.append((f"{name}{val}", lambda fn=fn, v=val: fn(**dict(zip(names, v)))))
        else:
            out.append((name, fn))
    return out


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_planted_mistake_fails_a_pin(mutation, tmp_path, monkeypatch):
    src = open(SRC).read()
    old, new = MUTATIONS[mutation]
    assert src.count(old) == 1, f"mutation anchor for {mutation!r} not unique"
    lib = ctypes.CDLL(_build(src.replace(old, new), "double", str(tmp_path), mutation.replace(" ", "_")))
    lib.kda_oracle_bwd.argtypes = oracle._bwd_lib("f64").kda_oracle_bwd.argtypes
    lib.kda_oracle_bwd.restype = ctypes.c_int
    monkeypatch.setattr(oracle, "_bwd_loaded", {"f64": lib})
    failed = []
    for name, fn in _pins():
        try:
            fn()
        except (KeyboardInterrupt, SystemExit):
            raise
        except BaseException:
            failed.append(name)
    assert failed, f"no pin caught the planted mistake {mutation!r}"
