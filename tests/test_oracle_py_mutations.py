"""The pins of the numpy parts of the oracle must catch plausible mistakes.

Each case plants one mistake in a private copy of an oracle module's source
(CPU only), swaps the mutant's functions in for the real ones and runs every
pin of that module's pin file; at least one pin must fail for every planted
mistake.  (The C token loop has its own mutation test.)
"""
import inspect
import types

import pytest

from oracle import cp, layer_ops
from tests import test_oracle_cp_pins, test_oracle_layer_pins

TARGETS = {"cp": (cp, test_oracle_cp_pins), "layer_ops": (layer_ops, test_oracle_layer_pins)}

MUTATIONS = {
    # context-parallel oracle
    ("cp", "transition decays on the wrong side"): ("M = np.exp(g[b, t, h])[:, None] * M",
                                                    "M = M * np.exp(g[b, t, h])[None, :]"),
    ("cp", "transition drops beta"): ("M = M - beta[b, t, h] * np.outer(kt, kt @ M)",
                                      "M = M - np.outer(kt, kt @ M)"),
    ("cp", "transition adds the key term"): ("M = M - beta[b, t, h] * np.outer(kt, kt @ M)",
                                             "M = M + beta[b, t, h] * np.outer(kt, kt @ M)"),
    ("cp", "transition applied earliest-first"): ("M = M - beta[b, t, h] * np.outer(kt, kt @ M)",
                                                  "M = M - beta[b, t, h] * np.outer(M @ kt, kt)"),
    ("cp", "transition ignores segments"): ("if runs != [(0, T)]:", "if False:"),
    ("cp", "transition ignores the l2 norm"): ("if use_qk_l2norm:\n", "if False:\n"),
    ("cp", "plan continues at a segment's first token"): ("carried = bool(hit) and runs[hit[0]][0] < lo",
                                                          "carried = bool(hit) and runs[hit[0]][0] <= lo"),
    ("cp", "plan first index off by one"): ("first = hit[0] if hit else", "first = hit[0] + 1 if hit else"),
    ("cp", "plan counts only new segments"): ("plan[b, r] = (int(carried), first, len(hit),",
                                              "plan[b, r] = (int(carried), first, len(hit) - int(carried),"),
    ("cp", "runs merge different ids"): ("while t + 1 < T and ids_row[t + 1] == ids_row[s]:",
                                         "while t + 1 < T and ids_row[t + 1] != 0:"),
    # layer steps
    ("layer_ops", "conv taps reversed"): ("tau = t - (W - 1) + j", "tau = t - j"),
    ("layer_ops", "conv reaches across segments"): ("if tau >= start[b, t]:", "if tau >= 0:"),
    ("layer_ops", "conv keeps padding outputs"): ("if seg is not None and seg[b, t] == 0:", "if False:"),
    ("layer_ops", "conv activation is a sigmoid"): ("acc * _sigmoid(acc) if", "_sigmoid(acc) if"),
    ("layer_ops", "segment start misses an id change"): ("if t == 0 or cur == 0 or cur != segment_ids[b, t - 1]:",
                                                         "if t == 0 or cur == 0:"),
    ("layer_ops", "norm eps outside the root"): ("np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)",
                                                 "(np.sqrt(np.mean(o * o, axis=-1, keepdims=True)) + eps)"),
    ("layer_ops", "norm over the wrong axis"): ("np.mean(o * o, axis=-1, keepdims=True)",
                                                "np.mean(o * o, axis=0, keepdims=True)"),
    ("layer_ops", "output gate mirrored"): ("return w * (o / rms) * _sigmoid(z)", "return w * (o / rms) * _sigmoid(-z)"),
}


def _mutant(module, old, new):
    src = inspect.getsource(module)
    assert src.count(old) == 1, f"mutation anchor {old!r} not unique in {module.__name__}"
    mod = types.ModuleType(module.__name__ + "_mutant")
    exec(compile(src.replace(old, new), module.__file__ + " (mutant)", "exec"), mod.__dict__)
    return mod


def _pins(pin_module):
    out = []
    for name, fn in inspect.getmembers(pin_module, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if params:
            argname, values = params[0].args
            out += [(f"{name}[{v}]", lambda fn=fn, a=argname, v=v: fn(**{a: v})) for v in values]
        else:
            out.append((name, fn))
    return out


@pytest.mark.parametrize("key", list(MUTATIONS), ids=lambda k: f"{k[0]}: {k[1]}")
def test_planted_mistake_fails_a_pin(key, monkeypatch):
    module, pin_module = TARGETS[key[0]]
    mutant = _mutant(module, *MUTATIONS[key])
    for name, obj in vars(mutant).items():
        if inspect.isfunction(obj) and getattr(module, name, None) is not None:
            monkeypatch.setattr(module, name, obj)
    failed = []
    for name, fn in _pins(pin_module):
        try:
            fn()
        except (KeyboardInterrupt, SystemExit):
            raise
        except BaseException:
            failed.append(name)
    assert failed, f"no pin caught the planted mistake {key!r}"
