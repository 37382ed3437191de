"""Reader for the ``key = value`` text fixtures in this folder (comments start with '#')."""
from __future__ import annotations

import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(HERE, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition("=")
            val = val.strip()
            try:
                out[key.strip()] = int(val)
            except ValueError:
                out[key.strip()] = float(val)
    return out
