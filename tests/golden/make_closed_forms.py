"""Write closed_forms.json: exact selected log-probabilities of rows whose
log-sum-exp has a closed form, computed with Python's decimal module at 40
significant digits (no numpy, no oracle, no GPU).

Operator: "Batch-Invariant LogP" -- opening definition and Reference
Semantics: logp = x[t] - log(sum_j exp(x[j])), lse = log(sum_j exp(x[j])).

Row families (x has V entries, t is the target):
  constant   every x_j = c:                lse = c + ln V,  logp = -ln V
  log_ladder x_j = ln(j + 1):              sum = V (V + 1) / 2,
                                           logp = ln(t + 1) - ln(V (V + 1) / 2)
  two_level  x_j = a for j < k, else b:    sum = k e^a + (V - k) e^b
  spike      x_j = 0 except x_s = D:       sum = e^D + V - 1
Each entry also carries the gradient of logp wrt x at three columns for
g = 1 (d_j = [j == t] - exp(x_j - lse)).

Run:  python tests/golden/make_closed_forms.py  (rewrites the JSON beside it)
"""

import json
import os
from decimal import Decimal, getcontext

getcontext().prec = 40


def row_value(spec, j):
    kind = spec["kind"]
    if kind == "constant":
        return Decimal(repr(spec["value"]))
    if kind == "log_ladder":
        return Decimal(j + 1).ln()
    if kind == "two_level":
        return Decimal(repr(spec["a"])) if j < spec["k"] else Decimal(repr(spec["b"]))
    if kind == "spike":
        return Decimal(repr(spec["height"])) if j == spec["col"] else Decimal(0)
    raise ValueError(kind)


def row_lse(spec, v):
    kind = spec["kind"]
    if kind == "constant":
        return Decimal(repr(spec["value"])) + Decimal(v).ln()
    if kind == "log_ladder":
        return (Decimal(v) * Decimal(v + 1) / 2).ln()
    if kind == "two_level":
        a, b, k = Decimal(repr(spec["a"])), Decimal(repr(spec["b"])), spec["k"]
        return (k * a.exp() + (v - k) * b.exp()).ln()
    if kind == "spike":
        return (Decimal(repr(spec["height"])).exp() + (v - 1)).ln()
    raise ValueError(kind)


CASES = [
    ("uniform_v8_zero", 8, {"kind": "constant", "value": 0.0}, [0, 5, 7]),
    ("uniform_v8_1p7", 8, {"kind": "constant", "value": 1.7}, [3]),
    ("uniform_v300", 300, {"kind": "constant", "value": -2.25}, [0, 299]),
    ("uniform_v4096", 4096, {"kind": "constant", "value": 0.0}, [0, 4095]),
    ("uniform_v4096_1p7", 4096, {"kind": "constant", "value": 1.7}, [17]),
    ("uniform_v151936", 151936, {"kind": "constant", "value": 0.0}, [151935]),
    ("ladder_v8", 8, {"kind": "log_ladder"}, list(range(8))),
    ("ladder_v1000", 1000, {"kind": "log_ladder"}, [0, 1, 499, 999]),
    ("two_level_v4096", 4096, {"kind": "two_level", "a": 2.5, "b": -1.25, "k": 3},
     [0, 2, 3, 4095]),
    ("spike_v151936", 151936, {"kind": "spike", "col": 77777, "height": 40.0},
     [77777, 0, 151935]),
    ("spike_v4096_small", 4096, {"kind": "spike", "col": 5, "height": 4.0},
     [5, 6]),
    # Logits far outside exp's float64 range (|x| > 709): only a shifted
    # log-sum-exp evaluates these rows.
    ("uniform_v8_big", 8, {"kind": "constant", "value": 1000.0}, [0, 7]),
    ("two_level_v8_big", 8, {"kind": "two_level", "a": 800.0, "b": -800.0, "k": 2},
     [0, 5]),
]


def main():
    out = {
        "citation": ("Batch-Invariant LogP -- opening definition and Reference "
                     "Semantics (logp = logit at target minus the row "
                     "log-sum-exp); closed forms derived by hand, evaluated "
                     "with decimal at 40 digits"),
        "cases": [],
    }
    for name, v, spec, targets in CASES:
        lse = row_lse(spec, v)
        entries = []
        for t in targets:
            xt = row_value(spec, t)
            probe = sorted({0, t, v - 1})
            grad = {str(j): str((Decimal(1) if j == t else Decimal(0))
                                - (row_value(spec, j) - lse).exp())
                    for j in probe}
            entries.append({"target": t, "logp": str(xt - lse), "grad_g1": grad})
        out["cases"].append({"name": name, "v": v, "row": spec,
                             "lse": str(lse), "targets": entries})
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "closed_forms.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
