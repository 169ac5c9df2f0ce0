"""Pure-Python brute force of the MoE layer for tiny inputs.

Written independently of the oracle, with different algorithms wherever one
exists, so that a slip in either shows up as a mismatch:
  * top-k by repeated arg-max (first maximum wins), not by sorting;
  * rank-limited top-k two ways: a greedy walk down the experts that skips any
    expert whose rank would be one too many, and an exhaustive search for the
    allowed k-subset whose scores, best first, are lexicographically largest;
  * capacity as the smallest integer C with C*E >= cf*k*T in exact rationals;
  * slots from per-expert counters walked in token order, not from a sort;
  * every dot product as an explicit Python loop in double precision.
Only the standard library is used.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def f32(v: float) -> float:
    """Round a double to the nearest binary32 value (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def capacity(T: int, E: int, k: int, cf32: float) -> int:
    need = Fraction(cf32) * k * T
    c = 0
    while c * E < need:
        c += 1
    return c


def argmax_first(vals, banned):
    best = None
    for i, v in enumerate(vals):
        if i in banned:
            continue
        if best is None or v > vals[best]:
            best = i
    return best


def topk(row, k):
    chosen = []
    for _ in range(k):
        chosen.append(argmax_first(row, set(chosen)))
    return chosen


def rank_of(e, E, P):
    return e // (E // P)


def rank_limited_greedy(row, k, P, M):
    """Walk experts best first; take one unless its rank would be rank M+1."""
    E = len(row)
    chosen, ranks = [], []
    banned = set()
    while len(chosen) < k:
        e = argmax_first(row, banned)
        banned.add(e)
        r = rank_of(e, E, P)
        if r in ranks or len(ranks) < M:
            chosen.append(e)
            if r not in ranks:
                ranks.append(r)
    return chosen


def rank_limited_exhaustive(row, k, P, M):
    """Among all k-subsets touching at most M ranks, the one whose members,
    ordered best first (lower index first on equal scores), compare largest."""
    import itertools
    E = len(row)
    best_key, best = None, None
    for sub in itertools.combinations(range(E), k):
        if len({rank_of(e, E, P) for e in sub}) > M:
            continue
        ordered = sorted(sub, key=lambda e: (-row[e], e))
        key = [(-row[e], e) for e in ordered]
        if best_key is None or key < best_key:
            best_key, best = key, ordered
    return best


def gates(vals):
    m = vals[0]
    ex = [math.exp(v - m) for v in vals]
    s = sum(ex)
    return [f32(e / s) for e in ex]


def dot(a, b):
    s = 0.0
    for u, v in zip(a, b):
        s += u * v
    return s


def silu(z):
    return z / (1.0 + math.exp(-z))


def mlp(xrow, wg, wu, wd):
    h = [silu(dot(g, xrow)) * dot(u, xrow) for g, u in zip(wg, wu)]
    return [dot(r, h) for r in wd]


def layer(x, wr, bias, wg, wu, wd, k, cf32, P=1, M=0, caps=None):
    """x: T lists of d doubles; wr: E lists; wg/wu: E x d_ff x d; wd: E x d x d_ff.
    M > 0 limits every token to experts of at most M of the P ranks. caps, if
    given, is a capacity per expert (in units of C) instead of C for all.

    Returns dict with logits, idx, w, C, slot, src, routed, kept, out (doubles).
    """
    T, E = len(x), len(wr)
    logits = [[f32(dot(x[t], wr[e]) + (bias[e] if bias is not None else 0.0)) for e in range(E)]
              for t in range(T)]
    if 0 < M < P:
        idx = [rank_limited_greedy(logits[t], k, P, M) for t in range(T)]
    else:
        idx = [topk(logits[t], k) for t in range(T)]
    w = [gates([logits[t][e] for e in idx[t]]) for t in range(T)]
    C = capacity(T, E, k, cf32)
    fill = [0] * E
    slot = [[-1] * k for _ in range(T)]
    src = [-1] * (E * C)
    for t in range(T):
        for j in range(k):
            e = idx[t][j]
            s = fill[e]
            fill[e] += 1
            if s < (C if caps is None else caps[e] * C):
                slot[t][j] = s
                if caps is None:
                    src[e * C + s] = t * k + j
    kept = [min(f, C if caps is None else caps[e] * C) for e, f in enumerate(fill)]
    out = []
    for t in range(T):
        row = list(x[t])
        for j in range(k):
            if slot[t][j] < 0:
                continue
            e = idx[t][j]
            y = mlp(x[t], wg[e], wu[e], wd[e])
            row = [r + w[t][j] * v for r, v in zip(row, y)]
        out.append(row)
    return {"logits": logits, "idx": idx, "w": w, "C": C, "slot": slot, "src": src,
            "routed": fill, "kept": kept, "out": out}
