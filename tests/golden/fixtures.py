"""Reader for the small text fixtures in this folder (``key = json-value`` lines)."""
import json
import os

_HERE = os.path.dirname(os.path.abspath(__file__))


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(_HERE, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split("=", 1)
            out[key.strip()] = json.loads(val.strip())
    return out
