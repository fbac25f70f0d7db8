"""Reader for the hand-worked fixtures under tests/golden (key = value lines)."""
import math
import os
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (x.strip() for x in line.split("=", 1))
            out[key] = val.split()
    return out


def num(tok):
    """A fraction 'p/q', an integer, or 'lnX' (natural log of X) as float."""
    if tok.startswith("ln"):
        return math.log(float(tok[2:]))
    return float(Fraction(tok))


def nums(toks):
    return [num(t) for t in toks]


def ints(toks):
    out = []
    for t in toks:
        if ".." in t:
            lo, hi = t.split("..")
            out.extend(range(int(lo), int(hi) + 1))
        else:
            out.append(int(t))
    return out
