"""Reader for the worked-number fixtures under tests/golden."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split(":", 1)
            rows = [r.split() for r in val.split(";")]
            arr = np.array([[float(x) for x in r] for r in rows])
            if arr.shape[0] == 1:
                arr = arr[0]
                if arr.shape[0] == 1:
                    arr = float(arr[0])
            out[key.strip()] = arr
    return out
