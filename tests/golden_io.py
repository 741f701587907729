"""Readers for the small text fixtures under tests/golden/ (values printed on
the pages, each file citing where)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows(name):
    """Non-comment lines of a fixture, split on '|' and stripped."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append([x.strip() for x in line.split("|")])
    return out


def kv(text):
    """'a=1 b=2,3' -> {'a': '1', 'b': '2,3'}"""
    return dict(item.split("=", 1) for item in text.split())


def ints(text):
    return [int(x) for x in text.split(",")] if text not in ("-", "") else []
