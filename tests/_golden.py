"""Reader for the hand-derived fixtures under tests/golden/ (``key: values``
lines, ``#`` comments)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            toks = val.split()
            vals = []
            for t in toks:
                if t.startswith("0x") or t.startswith("0X"):
                    vals.append(int(t, 16))
                else:
                    try:
                        vals.append(int(t))
                    except ValueError:
                        try:
                            vals.append(float(t))
                        except ValueError:
                            vals.append(t)
            out[key.strip()] = vals if len(vals) != 1 else vals[0]
    return out
