"""Brute-force pure-Python versions of the oracle (tiny inputs only).

Written independently of the numpy oracle: exact rationals for every
rounding, explicit loops with ``math.sin``/``math.exp``/``math.erf`` for every
sum, per-cell loops for the volume stages, a push formulation for child
marking (the numpy oracle pulls), and a full stable sort for top-k. The tests
require the numpy oracle to match these on integers exactly and on floats to
1e-12. Test infrastructure only.
"""

from __future__ import annotations

import itertools
import math
from fractions import Fraction
from typing import Dict, List, Sequence, Tuple


# ---------------------------------------------------------------- rounding

def round_to_bits(x: Fraction, sig_bits: int, min_exp: int) -> Fraction:
    """Round an exact rational to the nearest binary float with ``sig_bits``
    significant bits, ties to even; ``min_exp`` is the exponent of the
    smallest normal number (subnormal spacing below it)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = 0  # find e with 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, min_exp) - (sig_bits - 1))
    lo = (a // q) * q
    hi = lo + q
    if a - lo < hi - a:
        r = lo
    elif hi - a < a - lo:
        r = hi
    else:
        r = lo if (lo / q) % 2 == 0 else hi
    return sign * r


def f32(x) -> float:
    return float(round_to_bits(Fraction(x), 24, -126))


def bf16(x) -> float:
    return float(round_to_bits(Fraction(x), 8, -126))


# ---------------------------------------------------------------- decoder

def coord(i: int, R: int) -> float:
    return float(round_to_bits(Fraction(2 * i - R, R), 24, -126))


def embed(p: Sequence[float]) -> List[float]:
    pi32 = round_to_bits(Fraction(math.pi), 24, -126)
    e = [float(c) for c in p]
    sins, coss = [], []
    for axis in range(3):
        for k in range(8):
            arg = round_to_bits(pi32 * 2 ** k * Fraction(p[axis]), 24, -126)
            sins.append(math.sin(float(arg)))
            coss.append(math.cos(float(arg)))
    return e + sins + coss


def matvec(W, x) -> List[float]:
    out = []
    for row in W:
        s = 0.0
        for a, b in zip(row, x):
            s += float(a) * float(b)
        out.append(s)
    return out


def decode_point(p, W: Dict, K: List[List[float]], V: List[List[float]], H: int,
                 prims, net_scale: float, dtype: str, tokens=None, head_tokens=None) -> float:
    """tokens: one token subset for every head; head_tokens: a subset per head."""
    q = matvec(W["Wq"], embed(p))
    if dtype == "bf16":
        q = [bf16(v) for v in q]
    o = []
    for h in range(H):
        if head_tokens is not None:
            toks = head_tokens[h]
        else:
            toks = range(len(K)) if tokens is None else tokens
        cols = range(64 * h, 64 * h + 64)
        logits = []
        for j in toks:
            s = 0.0
            for c in cols:
                s += q[c] * K[j][c]
            logits.append(s / 8.0)
        mx = max(logits)
        ex = [math.exp(s - mx) for s in logits]
        tot = sum(ex)
        for c in cols:
            acc = 0.0
            for w, j in zip(ex, toks):
                acc += w * V[j][c]
            o.append(acc / tot)
    a = matvec(W["Wo"], o)
    hdn = [0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in matvec(W["W1"], a)]
    y = [ai + bi for ai, bi in zip(a, matvec(W["W2"], hdn))]
    net = sum(float(w) * v for w, v in zip(W["w_head"], y))
    return analytic(p, prims) + f32(net_scale) * net  # the scale is a float32 parameter


def project_kv(Z, Wk, Wv, dtype: str) -> Tuple[List[List[float]], List[List[float]]]:
    K = [matvec(Wk, z) for z in Z]
    V = [matvec(Wv, z) for z in Z]
    if dtype == "bf16":
        K = [[bf16(v) for v in row] for row in K]
        V = [[bf16(v) for v in row] for row in V]
    return K, V


def analytic(p, prims) -> float:
    best = math.inf
    for pr in prims:
        c = [float(v) for v in pr.centre]
        if pr.kind == 0:
            d = math.sqrt(sum((p[i] - c[i]) ** 2 for i in range(3))) - float(pr.size[0])
        else:
            q = [abs(p[i] - c[i]) - float(pr.size[i]) for i in range(3)]
            outside = math.sqrt(sum(max(v, 0.0) ** 2 for v in q))
            d = outside + min(max(q), 0.0)
        best = min(best, d)
    return best


# ---------------------------------------------------------------- volume stages

def key(I: int, J: int, K: int, P: int) -> int:
    NB = (P + 7) // 8
    return (((I // 8) * NB + J // 8) * NB + K // 8) * 512 + ((I % 8) * 8 + J % 8) * 8 + K % 8


def cell_active(vol: Dict[Tuple[int, int, int], float], R: int, tested, tau: float):
    act = set()
    for (i, j, k) in tested:
        vals = [f32(vol[(i + a, j + b, k + c)]) for a in (0, 1) for b in (0, 1) for c in (0, 1)]
        sign_change = any(v < 0 for v in vals) and any(v >= 0 for v in vals)
        band = min(abs(v) for v in vals) < f32(tau)
        if sign_change or band:
            act.add((i, j, k))
    return act


def dilate(cells, R: int):
    out = set()
    for (i, j, k) in cells:
        for a, b, c in itertools.product((-1, 0, 1), repeat=3):
            n = (i + a, j + b, k + c)
            if all(0 <= v < R for v in n):
                out.add(n)
    return out


def hvd(decode_fn, R0: int, levels: int, tau: float, dilation: int = 1):
    """decode_fn(R, (I,J,K)) -> float. Returns (final volume dict, per-level records)."""
    P = R0 + 1
    pts = sorted(itertools.product(range(P), repeat=3), key=lambda t: key(*t, P))
    vol = {t: decode_fn(R0, t) for t in pts}
    computed = set(pts)
    tested = set(itertools.product(range(R0), repeat=3))
    R = R0
    recs = []
    for L in range(levels):
        act = cell_active(vol, R, tested, tau)
        rec = {"R": R, "list": [(t[0] * (R + 1) + t[1]) * (R + 1) + t[2] for t in pts],
               "active": act, "tested": tested}
        if L == levels - 1:
            recs.append(rec)
            break
        kept = set(act)
        for _ in range(dilation):
            kept = dilate(kept, R)
        rec["kept"] = kept
        recs.append(rec)
        R1 = 2 * R
        P1 = R1 + 1
        cand = set()
        for (i, j, k) in kept:  # push: mark every corner of every child
            for a, b, c in itertools.product((0, 1), repeat=3):
                ci, cj, ck = 2 * i + a, 2 * j + b, 2 * k + c
                for x, y, z in itertools.product((0, 1), repeat=3):
                    cand.add((ci + x, cj + y, ck + z))
        prev = {(2 * i, 2 * j, 2 * k) for (i, j, k) in computed}
        new = sorted((t for t in cand if t not in prev), key=lambda t: key(*t, P1))
        vol1 = {}
        for t in itertools.product(range(P1), repeat=3):
            vol1[t] = vol[(t[0] // 2, t[1] // 2, t[2] // 2)]
        for t in new:
            vol1[t] = decode_fn(R1, t)
        tested = set()
        for (i, j, k) in kept:
            for a, b, c in itertools.product((0, 1), repeat=3):
                tested.add((2 * i + a, 2 * j + b, 2 * k + c))
        vol, computed, pts, R = vol1, prev | set(new), new, R1
    return vol, recs


# ---------------------------------------------------------------- KV selection

def scores(qs, K, H: int) -> List[List[float]]:
    """Head-mean softmax probability of every token for every probe."""
    out = []
    M = len(K)
    for q in qs:
        acc = [0.0] * M
        for h in range(H):
            cols = range(64 * h, 64 * h + 64)
            lg = [sum(q[c] * K[j][c] for c in cols) / 8.0 for j in range(M)]
            mx = max(lg)
            ex = [math.exp(v - mx) for v in lg]
            tot = sum(ex)
            for j in range(M):
                acc[j] += ex[j] / tot / H
        out.append(acc)
    return out


def scores_per_head(qs, K, H: int) -> List[List[List[float]]]:
    """[H][probe][token]: each head's softmax probability."""
    M = len(K)
    out = [[] for _ in range(H)]
    for q in qs:
        for h in range(H):
            cols = range(64 * h, 64 * h + 64)
            lg = [sum(q[c] * K[j][c] for c in cols) / 8.0 for j in range(M)]
            mx = max(lg)
            ex = [math.exp(v - mx) for v in lg]
            tot = sum(ex)
            out[h].append([e / tot for e in ex])
    return out


def select(sc: List[List[float]], k: int, cap: int) -> List[int]:
    s32 = [[f32(v) for v in row] for row in sc]
    union = set()
    for row in s32:
        order = sorted(range(len(row)), key=lambda j: (-row[j], j))
        union.update(order[:k])
    union = sorted(union)
    if len(union) > cap:
        best = {j: max(row[j] for row in s32) for j in union}
        union = sorted(sorted(union, key=lambda j: (-best[j], j))[:cap])
    return union


# ---------------------------------------------------------------- local KNN decoder (AVS-Conv)

def local_neighbours(P, x, K: int) -> List[int]:
    """K nearest supports of point x: float32 squared distances from exact
    rational arithmetic rounded at each step (difference, square, x + y, + z),
    sorted as (distance, index) tuples."""
    def d2(p):
        dx = [f32(Fraction(float(p[a])) - Fraction(float(x[a]))) for a in range(3)]
        sq = [f32(Fraction(v) * Fraction(v)) for v in dx]
        return f32(Fraction(f32(Fraction(sq[0]) + Fraction(sq[1]))) + Fraction(sq[2]))

    keyed = sorted((d2(P[j]), j) for j in range(len(P)))
    return [j for _, j in keyed[:K]]


def local_point(P, Fe, x, W: Dict, K: int, prims, net_scale: float) -> float:
    """SDF of the local decoder at one point, with explicit loops."""
    nb = local_neighbours(P, x, K)
    A, a, B = W["A"], W["a"], W["B"]
    C = len(Fe[0])
    Hw = len(a)
    gelu = lambda u: 0.5 * u * (1.0 + math.erf(u / math.sqrt(2.0)))  # noqa: E731
    h = [0.0] * C
    for j in nb:
        delta = [f32(Fraction(float(P[j][t])) - Fraction(float(x[t]))) for t in range(3)]
        g = []
        for m in range(Hw):
            u = float(a[m])
            for t in range(3):
                u += float(A[m][t]) * delta[t]
            g.append(gelu(u))
        for c in range(C):
            wc = 0.0
            for m in range(Hw):
                wc += float(B[c][m]) * g[m]
            h[c] += (wc * float(Fe[j][c]) + float(Fe[j][c])) / K
    W1, W2, wh = W["W1"], W["W2"], W["w_head"]
    hid = [gelu(sum(float(W1[f][c]) * h[c] for c in range(C))) for f in range(len(W1))]
    y = [h[c] + sum(float(W2[c][f]) * hid[f] for f in range(len(hid))) for c in range(C)]
    net = sum(float(wh[c]) * y[c] for c in range(C))
    return analytic([float(v) for v in x], prims) + f32(net_scale) * net
