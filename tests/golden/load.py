"""Loader for the hand-derived fixtures in this folder.

Numbers may be written as JSON numbers or as the strings "lnX" (natural log of
X) and "a/b" (an exact fraction); they are turned into float64 here.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _num(x):
    if isinstance(x, str):
        if x.startswith("ln"):
            return math.log(float(x[2:]))
        return float(Fraction(x))
    return float(x)


def _arr(x):
    if isinstance(x, list):
        return [_arr(e) for e in x]
    return _num(x)


def load(name):
    with open(os.path.join(HERE, name)) as f:
        raw = json.load(f)
    out = {}
    for k, v in raw.items():
        if k in ("citation", "derivation"):
            out[k] = v
        elif isinstance(v, dict):
            out[k] = {kk: np.array(_arr(vv), dtype=np.float64) for kk, vv in v.items()}
        elif isinstance(v, list):
            out[k] = np.array(_arr(v), dtype=np.float64)
        else:
            out[k] = _num(v)
    return out
