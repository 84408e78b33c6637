"""Readers for the hand-written fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _expand(tokens, conv):
    out = []
    for tok in tokens:
        if "*" in tok:
            n, v = tok.split("*")
            out += [conv(v)] * int(n)
        else:
            out.append(conv(tok))
    return out


def quant_vectors():
    blocks, cur = [], {}
    for line in open(os.path.join(GOLDEN, "quant_vectors.txt")):
        line = line.strip()
        if line.startswith("#"):
            continue
        if not line:
            if cur:
                blocks.append(cur)
                cur = {}
            continue
        key, val = [s.strip() for s in line.split(":", 1)]
        cur[key] = val
    if cur:
        blocks.append(cur)
    vecs = []
    for b in blocks:
        vecs.append({
            "name": b["name"],
            "input": _expand(b["input"].split(), lambda s: int(s, 16)),
            "scale": int(b["scale"], 16),
            "zero": int(b["zero"], 16),
            "codes": _expand(b["codes"].split(), int),
        })
    return vecs


def key_values(fname):
    out = {}
    for line in open(os.path.join(GOLDEN, fname)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = [s.strip() for s in line.split(":", 1)]
        out[k] = float(v) if "." in v else int(v)
    return out


def layout_tiles():
    """Entries of layout_tiles.txt: ("onehot", kind, t, j, offset, shift) and
    ("pattern", kind, offset, byte)."""
    out = []
    for line in open(os.path.join(GOLDEN, "layout_tiles.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        f = line.split()
        if f[0] == "onehot":
            out.append(("onehot", f[1], int(f[2]), int(f[3]), int(f[4]), int(f[5])))
        elif f[0] == "pattern":
            out.append(("pattern", f[1], int(f[2]), int(f[3], 16)))
        else:
            raise ValueError(f"layout_tiles.txt: unknown entry {line!r}")
    return out
