"""Reader for the worked-example fixtures under tests/golden/."""
from __future__ import annotations

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _placements(tokens):
    out = []
    for t in tokens:
        if t == "R":
            out.append("R")
        elif t.startswith("S"):
            out.append(("S", int(t[1:])))
        else:
            raise ValueError(t)
    return out


def load_example(name: str) -> dict:
    """Parse an example fixture: shape, src/dst layouts and the stated holdings."""
    ex = {"hold": {"src": {}, "dst": {}}}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "shape":
                ex["shape"] = tuple(int(t) for t in tok[1:])
            elif tok[0] in ("src", "dst") and tok[1] == "mesh":
                i = tok.index("start")
                dims = [int(t) for t in tok[2:i]]
                start = int(tok[i + 1])
                pl = _placements(tok[tok.index("placements") + 1:])
                ex[tok[0]] = (dims, start, pl)
            elif tok[0] == "hold":
                side, rank = tok[1], int(tok[2])
                r0, r1 = int(tok[4]), int(tok[5])
                c0, c1 = int(tok[7]), int(tok[8])
                ex["hold"][side][rank] = ((r0, r1), (c0, c1))
            else:
                raise ValueError(line)
    return ex
