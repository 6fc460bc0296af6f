"""A second, loop-by-loop rendering of the same layer, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Pure Python: no
NumPy matmul, no sorting routine for the selection, every dot product an
exactly rounded `math.fsum`.  It exists so that the vectorised oracle in
moe_oracle.py is checked against an independent rendering rather than
trusted on its own word.  Definitions and sources are those listed in
moe_oracle.py; the selection here is written as a repeated arg-max and
the permutation as an explicit per-expert scan of the pairs, so neither
shares a construction with the vectorised code.

Inputs are Python lists of floats (bf16 values already widened) except
where noted.
"""
from __future__ import annotations

import math
import struct


def f32(v: float) -> float:
    """Round a Python float (binary64) to the nearest binary32 value."""
    if math.isnan(v):
        return v
    try:
        return struct.unpack("<f", struct.pack("<f", v))[0]
    except OverflowError:
        return math.copysign(math.inf, v)


def bf16(v: float) -> float:
    """Round to bf16 via binary32, nearest-even, working on the bit pattern."""
    v = f32(v)
    if math.isnan(v):
        return v
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def _beats(a: int, sa: float, b: int, sb: float) -> bool:
    """True when expert a ranks before expert b: larger biased score, a
    number before NaN, lower id on equal scores."""
    na, nb = math.isnan(sa), math.isnan(sb)
    if na or nb:
        if na and nb:
            return a < b
        return nb
    if sa != sb:
        return sa > sb
    return a < b


def route_token(logits_row, bias, k: int, rsf: float):
    """One token: sigmoid scores, biased scores, k repeated arg-max picks,
    ids ascending, unbiased scaled weights."""
    E = len(logits_row)
    s = []
    for l in logits_row:
        try:
            e = math.exp(-l)
        except OverflowError:
            e = math.inf
        s.append(f32(1.0 / (1.0 + e)))
    sb = [f32(s[e] + bias[e]) for e in range(E)]
    chosen = []
    for _ in range(k):
        best = None
        for e in range(E):
            if e in chosen:
                continue
            if best is None or _beats(e, sb[e], best, sb[best]):
                best = e
        chosen.append(best)
    ids = sorted(chosen)
    w = [f32(f32(rsf) * s[e]) for e in ids]
    return ids, w, s, sb


def permute_loops(ids, E: int):
    """For each expert in order, walk the pairs (t, j) in order and collect
    those routed to it."""
    T = len(ids)
    k = len(ids[0]) if T else 0
    offsets = [0]
    sorted_token = []
    inv_pos = [None] * (T * k)
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t][j] == e:
                    inv_pos[t * k + j] = len(sorted_token)
                    sorted_token.append(t)
        offsets.append(len(sorted_token))
    return offsets, sorted_token, inv_pos


def ffn_row(a, wg, wu, wd, L: float, round_h: bool = True):
    """One row through a clamped SwiGLU FFN: wg, wu [I][H], wd [H][I]."""
    I = len(wg)
    h = []
    for i in range(I):
        g = math.fsum(a[c] * wg[i][c] for c in range(len(a)))
        u = math.fsum(a[c] * wu[i][c] for c in range(len(a)))
        g = min(g, L)
        u = max(-L, min(u, L))
        try:
            sg = g / (1.0 + math.exp(-g))
        except OverflowError:
            sg = -0.0
        v = sg * u
        h.append(bf16(v) if round_h else v)
    y = [math.fsum(h[i] * wd[c][i] for i in range(I)) for c in range(len(wd))]
    return h, y


def forward_loops(x, w_router, bias, wgu, wd, wsgu, wsd, *, k, rsf, L,
                  x_shared=None, round_h=True):
    """The plain (non-ScMoE) layer, token by token.

    x [T][H], w_router [E][H], bias [E], wgu [E][2I][H], wd [E][H][I],
    wsgu [2I_s][H] or None, wsd [H][I_s].  All values already widened.
    Returns dict(ids, w, offsets, sorted_token, inv_pos, z, out).
    """
    T, H = len(x), len(x[0])
    E = len(w_router)
    x_shared = x if x_shared is None else x_shared
    ids_all, w_all = [], []
    for t in range(T):
        l = [f32(math.fsum(x[t][c] * w_router[e][c] for c in range(H))) for e in range(E)]
        ids, w, _, _ = route_token(l, bias, k, rsf)
        ids_all.append(ids)
        w_all.append(w)
    offsets, sorted_token, inv_pos = permute_loops(ids_all, E)
    I = len(wgu[0]) // 2
    y_perm = [None] * (T * k)
    for e in range(E):
        for p in range(offsets[e], offsets[e + 1]):
            t = sorted_token[p]
            _, y = ffn_row(x[t], wgu[e][:I], wgu[e][I:], wd[e], L, round_h)
            y_perm[p] = y
    z, out = [], []
    for t in range(T):
        terms = [[] for _ in range(H)]
        for j in range(k):
            y = y_perm[inv_pos[t * k + j]]
            for c in range(H):
                terms[c].append(float(w_all[t][j]) * y[c])
        if wsgu is not None:
            Is = len(wsgu) // 2
            _, ys = ffn_row(x_shared[t], wsgu[:Is], wsgu[Is:], wsd, L, round_h)
            for c in range(H):
                terms[c].append(ys[c])
        zt = [math.fsum(v) for v in terms]
        z.append(zt)
        out.append([bf16(v) for v in zt])
    return dict(ids=ids_all, w=w_all, offsets=offsets, sorted_token=sorted_token,
                inv_pos=inv_pos, z=z, out=out)
