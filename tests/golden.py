"""Reader of the text fixtures under tests/golden/ (no arithmetic)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_rank_example(name):
    """Return (list of per-rank float32 inputs, float32 expected)."""
    inputs, expected = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "input":
                inputs[int(parts[1])] = np.array([float(v) for v in parts[2:]], np.float32)
            elif parts[0] == "expected":
                expected = np.array([float(v) for v in parts[1:]], np.float32)
    return [inputs[r] for r in sorted(inputs)], expected
