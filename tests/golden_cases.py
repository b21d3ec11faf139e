"""Reader for tests/golden/edge_cases.txt (see tests/golden/make_golden.py)."""
from pathlib import Path

import numpy as np

GOLDEN = Path(__file__).resolve().parent / "golden" / "edge_cases.txt"


def load():
    cases = []
    cur = {}
    for line in GOLDEN.read_text().splitlines():
        if not line.strip():
            continue
        key, _, rest = line.partition(" ")
        if key == "case":
            cur = {"name": rest}
            cases.append(cur)
        elif key == "cite":
            cur["cite"] = rest
        elif key == "dtype":
            cur["dtype"] = rest
        elif key == "shape":
            cur["shape"] = tuple(int(v) for v in rest.split())
        elif key == "x":
            store = np.uint16 if cur["dtype"] == "bf16" else np.uint32
            bits = np.array([int(v, 16) for v in rest.split()], dtype=store)
            x = bits.reshape(cur["shape"])
            cur["x"] = x if cur["dtype"] == "bf16" else x.view(np.float32)
        elif key == "out":
            cur["out"] = np.array([float("nan") if v == "nan" else float.fromhex(v)
                                   for v in rest.split()])
    return cases
