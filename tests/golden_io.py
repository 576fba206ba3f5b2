"""Reader for the small text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(tok: str):
    if tok.lower().startswith("0x") or tok.lower().startswith("-0x"):
        return int(tok, 16)
    try:
        return int(tok)
    except ValueError:
        return float(tok)


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            nums = []
            for v in vals:
                try:
                    nums.append(_num(v))
                except ValueError:
                    nums.append(v)
            out[key] = nums if len(nums) != 1 else nums[0]
    return out
