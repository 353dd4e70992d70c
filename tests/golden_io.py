"""Readers for the hand-worked fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            s = raw.split("#", 1)[0].strip()
            if s:
                key, val = s.split("=", 1)
                yield key.strip(), val.strip()


def nums(s, cast=float):
    return [cast(v, 0) if cast is int and v.startswith("0x") else cast(v) for v in s.split()]


def ints(s):
    return [int(v, 0) for v in s.split()]
