"""Readers for the cited text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows(name: str):
    """Rows of a 'values | citation' fixture: (list of fields, citation)."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals, _, cite = line.partition("|")
            out.append((vals.split(), cite.strip()))
    return out


def keyvals(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#") or line.startswith("|"):
                continue
            k, *v = line.split()
            out[k] = [int(x) for x in v]
    return out
