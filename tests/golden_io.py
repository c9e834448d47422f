"""Readers for the text fixtures under tests/golden/."""

import os
import re
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _scale(text):
    text = text.strip()
    m = re.fullmatch(r"2\*\*(-?\d+)", text)
    if m:
        return Fraction(2) ** int(m.group(1))
    return Fraction(text)


def _ints(text):
    out = []
    for tok in text.split():
        if "*" in tok:
            v, n = tok.split("*")
            out.extend([int(v)] * int(n))
        else:
            out.append(int(tok))
    return out


def read_blocks():
    """-> list of dicts {name, fmt, data(bytes), expect(list of Fraction)}."""
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "blocks.txt")) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest}
            elif key == "fmt":
                cur["fmt"] = rest
            elif key == "hex":
                cur["data"] = bytes.fromhex(rest.replace(" ", ""))
            elif key == "scale":
                cur["scale"] = _scale(rest)
            elif key == "ints":
                cur["ints"] = _ints(rest)
            elif key == "end":
                cur["expect"] = [cur["scale"] * v for v in cur["ints"]]
                cases.append(cur)
                cur = None
    return cases


def read_tile_choice():
    rows = []
    with open(os.path.join(GOLDEN, "tile_choice.txt")) as f:
        for raw in f:
            line = raw.strip()
            if line and not line.startswith("#"):
                n, mod, chosen = (int(v) for v in line.split())
                rows.append((n, mod, chosen))
    return rows
