"""Parser for the hand-worked fixtures: "lnX" is ln(X), "a/b" is an exact rational."""
import json
import math
import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def value(x):
    if isinstance(x, str):
        if x.startswith("ln"):
            return math.log(float(Fraction(x[2:])))
        return float(Fraction(x))
    return float(x)


def array(nested):
    if isinstance(nested, list):
        return np.array([array(e) for e in nested], dtype=np.float64)
    return value(nested)


def load(name="hand_worked.json"):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)
