"""Turns the worked examples in tests/golden/worked_examples.json into arrays."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


def load_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _dense(spec, dtype):
    shape = tuple(spec["shape"])
    a = np.zeros(shape, dtype=dtype)
    if "nonzero" in spec:
        for idx, val in spec["nonzero"]:
            a[tuple(idx)] = float(val)
    elif "fill_rows" in spec:
        rows = np.array(spec["fill_rows"], dtype=np.float64)
        a[...] = rows.reshape(shape)
    elif "fill" in spec:
        a[...] = float(spec["fill"])
    elif "values" in spec:
        a[...] = np.array([float(x) for x in spec["values"]]).reshape(shape)
    return a


def build_case(case):
    q = _dense(case["q"], np.float32)
    k = _dense(case["k"], np.float32)
    v = _dense(case["v"], np.float32)
    o = _dense(case["o"], np.float64)
    lse = _dense(case["lse"], np.float64)
    return q, k, v, float(case["scale"]), bool(case["causal"]), o, lse
