"""Parser for the hand-written codec fixtures under tests/golden/."""
import os
import re

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_CODECS = {"q4_0": 1, "mlx4_g64": 2, "q2_0": 3, "q8_0": 4, "mlx4_g32": 5, "q4_k": 6, "ternary": 7}


def _expand(tokens, conv):
    out = []
    i = 0
    while i < len(tokens):
        t = tokens[i]
        if t.startswith("("):
            grp = []
            t = t[1:]
            while True:
                m = re.fullmatch(r"(.*)\)x(\d+)", t)
                if m:
                    if m.group(1):
                        grp.append(m.group(1))
                    out.extend([conv(v) for v in grp] * int(m.group(2)))
                    break
                if t:
                    grp.append(t)
                i += 1
                t = tokens[i]
        else:
            m = re.fullmatch(r"(.+)x(\d+)", t) if conv is _hexbyte else None
            if m:
                out.extend([conv(m.group(1))] * int(m.group(2)))
            else:
                out.append(conv(t))
        i += 1
    return out


def _hexbyte(t):
    v = int(t, 16)
    assert 0 <= v <= 255, t
    return v


def load(fname):
    cases = []
    cur = None
    with open(os.path.join(GOLDEN, fname)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, rest = line.partition(" ")
            toks = rest.split()
            if key == "case":
                cur = {"name": toks[0], "bytes": [], "expect": []}
            elif key == "codec":
                cur["codec"] = _CODECS[toks[0]]
            elif key == "shape":
                cur["n"], cur["k"] = int(toks[0]), int(toks[1])
            elif key == "bytes":
                cur["bytes"] += _expand(toks, _hexbyte)
            elif key == "expect":
                cur["expect"] += _expand(toks, float)
            elif key == "end":
                cases.append(cur)
                cur = None
            else:
                raise ValueError(f"bad fixture line: {raw!r}")
    return cases


def all_cases():
    out = []
    for f in sorted(os.listdir(GOLDEN)):
        if f.endswith(".txt"):
            out += load(f)
    return out
