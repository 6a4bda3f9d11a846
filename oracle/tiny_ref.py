"""Second, independent oracle: pure-Python scalar loops, no numpy arithmetic.

TEST INFRASTRUCTURE ONLY (see oracle/tileq_ref.py).  It serves as a check of
the numpy oracle on tiny grids (d_in, d_out <= 64), following the same
definition from "TileQ: Efficient Low-Rank Quantization of Mixture-of-Experts
with 2D Tiling" (gist.science technical summary, section 2.1 steps 4-5): the
expert at tile (m, n) has weight  sum_r U[m*d_out+o][r] sigma[r]
V[n*d_in+i][r]  +  s[o][i//G] * (q[o][i] - z[o][i//G]).

Inputs are plain nested lists of Python floats/ints (the caller converts the
stored arrays exactly).
"""
import math


def code_at(words_row, i, bits=2):
    """Code of input i from a row of uint32 words: 2-bit codes 16 per word;
    3-bit codes as a little-endian bit string (bits 3i, 3i+1, 3i+2)."""
    if bits == 2:
        w = int(words_row[i // 16])
        return (w >> (2 * (i % 16))) & 3
    q = 0
    for j in range(3):
        n = 3 * i + j
        q |= ((int(words_row[n // 32]) >> (n % 32)) & 1) << j
    return q


def weight(p, e, o, i):
    """W_e[o][i] as a Python float sum, in the order of the definition."""
    tile = p["tile"][e]
    m, n = tile // p["N"], tile % p["N"]
    lr = 0.0
    for r in range(p["rank"]):
        lr += p["U"][m * p["d_out"] + o][r] * p["sigma"][r] * p["V"][n * p["d_in"] + i][r]
    g = i // p["G"]
    res = p["s"][e][o][g] * (code_at(p["codes"][e][o], i, p.get("bits", 2)) - p["z"][e][o][g])
    return lr + res


def apply(p, e, vec):
    return [sum(weight(p, e, o, i) * vec[i] for i in range(p["d_in"]))
            for o in range(p["d_out"])]


def forward_single(p, x, ids, gates):
    out = []
    for t in range(len(x)):
        y = [0.0] * p["d_out"]
        for j in range(len(ids[t])):
            e = ids[t][j]
            if not (0 <= e < p["K"]):
                continue
            v = apply(p, e, x[t])
            for o in range(p["d_out"]):
                y[o] += gates[t][j] * v[o]
        out.append(y)
    return out


def silu(v):
    return v / (1.0 + math.exp(-v)) if v > -700 else 0.0


def forward_swiglu(pg, pu, pd, x, ids, gates, rnd):
    """rnd: rounding of the SwiGLU intermediate to the activation format."""
    out = []
    for t in range(len(x)):
        y = [0.0] * pd["d_out"]
        for j in range(len(ids[t])):
            e = ids[t][j]
            if not (0 <= e < pg["K"]):
                continue
            a = apply(pg, e, x[t])
            b = apply(pu, e, x[t])
            h = [rnd(silu(a[o]) * b[o]) for o in range(len(a))]
            d = apply(pd, e, h)
            for o in range(pd["d_out"]):
                y[o] += gates[t][j] * d[o]
        out.append(y)
    return out
