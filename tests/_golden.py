"""Readers for the hand-worked fixtures under tests/golden/."""
import math
import os

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            yield line.split()


def _num(s):
    s = s.lower()
    if s in ("nan",):
        return math.nan
    if s in ("inf", "+inf"):
        return math.inf
    if s == "-inf":
        return -math.inf
    if s == "-0":
        return -0.0
    return float(s)


def fp8_values():
    return [(r[0], int(r[1], 16), _num(r[2])) for r in _rows("fp8_values.txt")]


def encode_cases():
    return [(r[0], _num(r[1]), int(r[2], 16)) for r in _rows("encode_cases.txt")]


def bias_cases():
    return [(r[0], _num(r[1]), int(r[2]), int(r[3]), int(r[4])) for r in _rows("bias_cases.txt")]
