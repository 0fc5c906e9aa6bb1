"""Reader for the small text fixtures under tests/golden/ ("key: values" lines, # comments)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if ":" in line:
                key, val = line.split(":", 1)
                out[key.strip()] = val.split()
            else:
                parts = line.split()
                out[parts[0]] = parts[1:]
    return out


def hex_bytes(vals):
    return [int(v, 16) for v in vals]


def floats(vals):
    return [float(v) for v in vals]
