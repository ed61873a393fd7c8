"""Reader for the hand-built block fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_blocks(name):
    """Return [(label, bytes uint8[bb], expected float64[32])] from a fixture file."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            raw = np.frombuffer(bytes.fromhex(parts[1]), dtype=np.uint8).copy()
            vals = np.array([float(v) for v in parts[2:]], dtype=np.float64)
            assert vals.size == 32
            out.append((parts[0], raw, vals))
    return out
