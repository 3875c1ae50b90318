"""Readers for the hand-derived fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [c.strip() for c in line.split("|")]


def quantizer_groups():
    out = []
    for name, vals, s16, z16, codes in _rows("quantizer_groups.txt"):
        values = []
        for item in vals.split(","):
            v, n = item.split(":")
            values += [float(v)] * int(n)
        assert len(values) == 64, name
        cmap = {float(v): int(c) for v, c in (x.split(":") for x in codes.split(","))}
        out.append(dict(name=name, values=values, s16=int(s16, 16), z16=int(z16, 16), codes=cmap))
    return out


def kv_write_spikes():
    out = []
    for kind, k, clip, slot, loc, params in _rows("kv_write_spikes.txt"):
        what, rest = loc.split(" ", 1)
        idx, val = rest.split("=")
        out.append(dict(kind=kind, k=int(k), clip=float(clip), slot=int(slot),
                        unit=what, index=int(idx), value=int(val, 16),
                        params=[int(p, 16) for p in params.split()]))
    return out
