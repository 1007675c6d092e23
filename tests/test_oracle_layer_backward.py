"""Pins of the oracle's full-layer backward (CPU only).

* central finite differences, in float64, of L = sum(dy * y) through the
  oracle's own forward, for every parameter of a tiny layer with a logit
  bias and a gated shared expert, for softmax / sigmoid scores with and
  without renormalisation (the expert selection is held fixed, so L is
  smooth in every parameter);
* closed forms: the softmax logit gradient sums to zero per token; with
  k = 1 and renormalisation the routed output does not depend on the router,
  so the router gets exactly zero gradient;
* combine / permute backward against pure-Python loops.
"""
import itertools

import numpy as np
import pytest

import oracle.moe_oracle as mo

T, D, E, K, F, FS = 5, 6, 5, 2, 4, 3


def _params(seed):
    rng = np.random.default_rng(seed)
    return dict(
        x=rng.standard_normal((T, D)),
        w_router=rng.standard_normal((E, D)) * 0.5,
        w1=rng.standard_normal((E, 2 * F, D)) * 0.5,
        w2=rng.standard_normal((E, D, F)) * 0.5,
        ws1=rng.standard_normal((2 * FS, D)) * 0.5,
        ws2=rng.standard_normal((D, FS)) * 0.5,
        w_gate=rng.standard_normal(D) * 0.5,
    ), rng.standard_normal((T, D)), rng.standard_normal(E) * 0.3


@pytest.mark.parametrize("score,normalize", list(itertools.product(["softmax", "sigmoid"],
                                                                   [True, False])))
def test_layer_backward_matches_finite_differences(score, normalize):
    P, dy, bias = _params(11 if score == "softmax" else 12)
    sel = mo.route(P["x"], P["w_router"], K, score, normalize, bias).topk_idx

    def loss(Q):
        y, _, _ = mo.moe_layer_forward(Q["x"], Q["w_router"], Q["w1"], Q["w2"], K, score,
                                       normalize, bias, Q["w_gate"], Q["ws1"], Q["ws2"],
                                       topk_idx=sel)
        return float((dy * y).sum())

    g = mo.moe_layer_backward(P["x"], P["w_router"], P["w1"], P["w2"], K, dy, score, normalize,
                              bias, P["w_gate"], P["ws1"], P["ws2"], topk_idx=sel)
    names = dict(x="dx", w_router="dw_router", w1="dw1", w2="dw2", ws1="dws1", ws2="dws2",
                 w_gate="dw_gate")
    h = 1e-6
    for pname, gname in names.items():
        num = np.zeros_like(P[pname])
        it = np.nditer(P[pname], flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            Q = {kk: v.copy() for kk, v in P.items()}
            Q[pname][i] += h
            lp = loss(Q)
            Q[pname][i] -= 2 * h
            lm = loss(Q)
            num[i] = (lp - lm) / (2 * h)
        ana = np.asarray(g[gname])
        scale = max(np.abs(num).max(), 1e-3)
        assert np.abs(ana - num).max() <= 1e-6 * scale, (pname, np.abs(ana - num).max(), scale)


def test_softmax_logit_gradient_sums_to_zero():
    P, dy, bias = _params(3)
    rng = np.random.default_rng(4)
    idx = mo.route(P["x"], P["w_router"], K, "softmax", True, bias).topk_idx
    for normalize in (True, False):
        _, _, dz, _ = mo.route_backward(P["x"], P["w_router"], idx, rng.standard_normal((T, K)),
                                        "softmax", normalize, bias)
        assert np.abs(dz.sum(axis=1)).max() < 1e-14


def test_top1_renormalised_router_gets_no_gradient():
    P, dy, bias = _params(5)
    g = mo.moe_layer_backward(P["x"], P["w_router"], P["w1"], P["w2"], 1, dy, "softmax", True,
                              bias)
    assert np.all(g["dz"] == 0.0) and np.all(g["dw_router"] == 0.0)
    # with sigmoid scores the single weight is s / s = 1 as well
    g = mo.moe_layer_backward(P["x"], P["w_router"], P["w1"], P["w2"], 1, dy, "sigmoid", True,
                              bias)
    assert np.all(g["dz"] == 0.0)


def test_combine_and_permute_backward_against_loops():
    rng = np.random.default_rng(9)
    Tn, d, k, N = 4, 3, 3, 12
    slot = rng.permutation(N).reshape(Tn, k).astype(np.int32)
    slot[2, 1] = -1                                      # a dropped choice
    Y = rng.standard_normal((N, d))
    w = rng.random((Tn, k))
    dy = rng.standard_normal((Tn, d))
    ysh = rng.standard_normal((Tn, d))
    gate = rng.random(Tn)
    dY, dw, dg = mo.combine_backward(dy, Y, slot, w, ysh, gate)
    for t in range(Tn):
        assert dg[t] == pytest.approx(sum(dy[t, c] * ysh[t, c] for c in range(d)), abs=1e-14)
        for j in range(k):
            r = slot[t, j]
            if r < 0:
                assert dw[t, j] == 0.0
                continue
            assert dw[t, j] == pytest.approx(sum(dy[t, c] * Y[r, c] for c in range(d)), abs=1e-14)
            for c in range(d):
                assert dY[r, c] == pytest.approx(w[t, j] * dy[t, c], abs=1e-15)
    dX = rng.standard_normal((N, d))
    dx = mo.permute_backward(dX, slot)
    for t in range(Tn):
        for c in range(d):
            ref = sum(dX[slot[t, j], c] for j in range(k) if slot[t, j] >= 0)
            assert dx[t, c] == pytest.approx(ref, abs=1e-14)
