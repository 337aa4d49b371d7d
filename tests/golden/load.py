"""Reader for the small ``key = value[, value...]`` golden fixtures."""

import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name):
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            vals = [float(int(v, 0)) if v.strip().lower().startswith("0x") else float(v)
                    for v in val.split(",")]
            out[key] = vals if len(vals) > 1 else vals[0]
    return out
