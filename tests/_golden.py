"""Reader for the cited text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line


def values(name):
    """A list of floats, one per non-comment line."""
    return [float(s) for s in _lines(name)]


def table(name):
    """key = value pairs; values are int, float or comma lists."""
    out = {}
    for line in _lines(name):
        k, v = (s.strip() for s in line.split("=", 1))
        if "," in v:
            out[k] = [float(x) for x in v.split(",")]
        else:
            out[k] = int(v) if v.lstrip("-").isdigit() else float(v)
    return out
