"""Reader for the hand-worked fixtures under tests/golden/ (format described in each file)."""
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _value_bits(tok):
    v = float.fromhex(tok) if "0x" in tok.lower() else float(tok)
    (u,) = struct.unpack("<I", struct.pack("<f", v))
    if u & 0xFFFF:
        raise ValueError(f"fixture value {tok} is not exactly representable in bf16")
    return u >> 16


def load(filename):
    """List of cases; each is a dict with inputs (list of uint16 arrays (1, hidden)), residual,
    weight, eps, and expect_* arrays of bits."""
    cases, cur = [], None
    with open(os.path.join(GOLDEN, filename)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, *rest = line.split()
            if key == "case":
                cur = {"name": rest[0], "inputs": []}
            elif key == "end":
                hidden = cur["hidden"]
                for k in ("residual",) + tuple(x for x in cur if x.startswith("expect_")):
                    assert cur[k].size == hidden, (cur["name"], k)
                assert len(cur["inputs"]) == cur["n"], cur["name"]
                cases.append(cur)
                cur = None
            elif key in ("n", "hidden"):
                cur[key] = int(rest[0])
            elif key == "eps":
                cur[key] = float(rest[0])
            elif key == "in":
                cur["inputs"].append(np.array([[_value_bits(t) for t in rest]], dtype=np.uint16))
            elif key == "residual":
                cur[key] = np.array([[_value_bits(t) for t in rest]], dtype=np.uint16)
            elif key == "weight":
                cur[key] = np.array([_value_bits(t) for t in rest], dtype=np.uint16)
            elif key.startswith("expect_"):
                cur[key] = np.array([[int(t, 16) for t in rest]], dtype=np.uint16)
            else:
                raise ValueError(f"unknown fixture key {key}")
    return cases
