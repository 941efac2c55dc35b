"""Readers for the small text fixtures under tests/golden (each cites its page)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                yield line


def worked_example():
    out = {}
    for line in _lines("worked_example.txt"):
        key, val = (x.strip() for x in line.split("=", 1))
        nums = [float(x) for x in val.split()]
        out[key] = nums if len(nums) > 1 else nums[0]
    return out


def materialised_scores():
    rows = []
    for line in _lines("materialised_scores.txt"):
        n, heads, bpe, value, unit = line.split()
        rows.append((int(n), int(heads), int(bpe), float(value), unit))
    return rows
