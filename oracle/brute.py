"""Pure-Python brute force for tiny inputs (test infrastructure only).

Independent second derivation of the oracle's results, written with plain
loops and Python floats (IEEE double) and no numpy linear algebra, so that a
slip in the vectorised oracle (a transposed operand, a wrong axis, an
off-by-one in the segment bounds) shows up as a mismatch.  Only the test
suite imports it.  It follows the same passages as ``moe_oracle``.
"""
from __future__ import annotations

import math
import struct


def f32(v: float) -> float:
    """Round a Python float to the nearest float32 value."""
    return struct.unpack("f", struct.pack("f", v))[0]


def route(x, w_router, k, score_fn="softmax", normalize=True, bias=None,
          selection_bias=None):
    """Per token: all E scores, fully sorted by (-fp32 key, index); the key is
    the fp32 score, plus the fp32 selection bias when given (the weights stay
    the unbiased scores)."""
    T, d, E = len(x), len(x[0]), len(w_router)
    idx_out, w_out = [], []
    for t in range(T):
        z = []
        for e in range(E):
            acc = 0.0
            for i in range(d):
                acc += float(x[t][i]) * float(w_router[e][i])
            if bias is not None:
                acc += float(bias[e])
            z.append(acc)
        if score_fn == "softmax":
            m = max(z)
            ex = [math.exp(v - m) for v in z]
            tot = sum(ex)
            s = [v / tot for v in ex]
        else:
            s = [1.0 / (1.0 + math.exp(-v)) for v in z]
        if selection_bias is None:
            ranked = sorted(range(E), key=lambda e: (-f32(s[e]), e))
        else:
            ranked = sorted(range(E), key=lambda e: (-f32(f32(s[e]) + f32(selection_bias[e])), e))
        chosen = ranked[:k]
        sel = [s[e] for e in chosen]
        tot = sum(sel)
        idx_out.append(chosen)
        w_out.append([v / tot for v in sel] if normalize else sel)
    return idx_out, w_out


def permute(topk_idx, E):
    """Walk experts in order, then tokens in order, then slots."""
    T, k = len(topk_idx), len(topk_idx[0])
    row_token, slot_of = [], [[None] * k for _ in range(T)]
    offsets = [0]
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if topk_idx[t][j] == e:
                    slot_of[t][j] = len(row_token)
                    row_token.append(t)
        offsets.append(len(row_token))
    return offsets, slot_of, row_token


def matvec_t(w, v):
    """out[r] = sum_c w[r][c] * v[c]."""
    return [sum(float(w[r][c]) * float(v[c]) for c in range(len(v)))
            for r in range(len(w))]


def swiglu_row(xrow, w1, w2):
    F = len(w1) // 2
    h = matvec_t(w1, xrow)
    a = []
    for f in range(F):
        g, u = h[f], h[F + f]
        a.append(g / (1.0 + math.exp(-g)) * u)
    return matvec_t(w2, a)


def layer_forward(x, w_router, w1, w2, k, score_fn="softmax", normalize=True,
                  bias=None, w_gate=None, ws1=None, ws2=None):
    idx, w = route(x, w_router, k, score_fn, normalize, bias)
    T, d = len(x), len(x[0])
    y = []
    for t in range(T):
        acc = [0.0] * d
        for j in range(k):
            yr = swiglu_row(x[t], w1[idx[t][j]], w2[idx[t][j]])
            for c in range(d):
                acc[c] += w[t][j] * yr[c]
        if ws1 is not None:
            g = sum(float(x[t][i]) * float(w_gate[i]) for i in range(d))
            gate = 1.0 / (1.0 + math.exp(-g))
            ys = swiglu_row(x[t], ws1, ws2)
            for c in range(d):
                acc[c] += gate * ys[c]
        y.append(acc)
    return y, idx, w
