"""Reader for the small text fixtures under tests/golden (key = value lines, '#' comments)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read(name):
    """Return a list of (key, [tokens]) pairs in file order."""
    out = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition("=")
            out.append((key.strip(), val.split()))
    return out


def as_dict(name):
    """Keys that occur once map to their token list; repeated keys map to a list of token lists."""
    d = {}
    for k, v in read(name):
        if k in d:
            if not isinstance(d[k][0], list):
                d[k] = [d[k]]
            d[k].append(v)
        else:
            d[k] = v
    return d


def tolerances():
    """{dtype: (atol, rtol)} from the tolerance table fixture."""
    return {k: (float(v[0]), float(v[1])) for k, v in read("faq_q10_tolerances.txt")}
