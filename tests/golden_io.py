"""Reader for the hand-expanded fixtures in tests/golden/ (key: value lines, # comments)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out[key.strip()] = val.strip()
    return out


def hexbytes(s: str) -> list:
    return [int(t, 16) for t in s.split()]


def floats(s: str) -> list:
    return [float(t) for t in s.split()]


def ints(s: str) -> list:
    return [int(t) for t in s.split()]
