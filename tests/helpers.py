"""Small test helpers (no method arithmetic here)."""
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


_ENV = {"__builtins__": {}, "ln": math.log, "sqrt": math.sqrt, "exp": math.exp,
        "cos": math.cos, "sin": math.sin}


def ev(x):
    """Evaluate a hand-written closed-form expression of a golden fixture."""
    if isinstance(x, list):
        return np.array([ev(e) for e in x], dtype=np.float64)
    if isinstance(x, (int, float)):
        return float(x)
    return float(eval(x, _ENV))


def normwise(got, ref):
    """max|got - ref| / max|ref| (0 when both are exactly zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
