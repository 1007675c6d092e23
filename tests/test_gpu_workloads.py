"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times (``MoELayer.forward``: route -> permute -> grouped
SwiGLU with the routing weight as fc2 row scale -> [shared expert] ->
combine), plus the forward + backward of the grouped GEMM on one
expert-parallel rank's share.

  * routing: compared with the oracle on every token (bit-exact expert sets
    outside the 1e-5 near-tie margin; excluded tokens counted and checked
    to be legal near-tie choices);
  * permutation: the GPU's maps equal the oracle's for the GPU's own expert
    choice, bit for bit, and every permuted row is a bitwise copy;
  * layer output: a seeded sample of tokens recomputed one by one by the
    oracle (float64) with the GPU's expert choice and the oracle's weights;
  * backward: dW1, dW2 and dX of sampled experts recomputed by the oracle.
"""
import numpy as np
import pytest
import torch

import moe_workloads as mw
from oracle import moe_oracle as mo
import gpu_helpers as gh

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

moe = pytest.importorskip("mixture_experts_layer_05_amd")


def _layer(inp, cfg, gather=True):
    g = lambda a: None if a is None else gh.to_gpu(a)  # noqa: E731
    return moe.MoELayer(g(inp.w_router), g(inp.w1), g(inp.w2), cfg.k, cfg.T, cfg.score,
                        cfg.normalize, g(inp.logit_bias), g(inp.w_gate), g(inp.ws1), g(inp.ws2),
                        gather=gather)


@pytest.mark.parametrize("name", ["tiny", "qwen3_30b", "dsv_30b", "skew_shared"])
def test_layer_forward_full_size(name):
    cfg = mw.get(name)
    inp = mw.make_layer_inputs(cfg)
    f = inp.as_f32
    x = gh.to_gpu(inp.x)
    layer = _layer(inp, cfg)
    y = layer.forward(x)
    y2 = layer.forward(x).clone()
    torch.cuda.synchronize()
    assert gh.bits_equal(y, y2)

    # ---- routing, all tokens
    ref = mo.route(f("x"), f("w_router"), cfg.k, cfg.score, cfg.normalize,
                   inp.logit_bias, f("w_gate"))
    idx = layer.route_out[0].cpu().numpy()
    w = layer.route_out[1].cpu().numpy()
    cnt = layer.route_out[2].cpu().numpy()
    n_excl, n_diff = gh.check_routing(idx, w, ref, cfg.k)
    assert (cnt == np.bincount(idx.reshape(-1), minlength=cfg.E)).all()
    if n_diff == 0:
        assert (cnt == ref.counts).all()
    if f("w_gate") is not None:
        assert np.abs(layer.route_out[3].cpu().numpy() - ref.gate).max() <= gh.TOL_ROUTE_W
    print(f"\n[{name}] excluded near-tie tokens: {n_excl} of {cfg.T} "
          f"({100.0 * n_excl / cfg.T:.2f}%), of which choose differently: {n_diff}; "
          f"hottest/mean = {cnt.max() / (cfg.T * cfg.k / cfg.E):.2f}")

    # ---- permutation, all pairs, for the GPU's own choice
    pref = mo.permute(None, idx, w, cfg.E)
    off, slot, rtok, rw, xp = layer.perm_out
    assert xp is None   # the layer gathers rows inside fc1
    assert np.array_equal(off.cpu().numpy(), pref.offsets)
    assert np.array_equal(slot.cpu().numpy(), pref.slot_of)
    assert np.array_equal(rtok.cpu().numpy(), pref.row_token)
    assert np.array_equal(rw.cpu().numpy().view(np.uint32), pref.row_w.view(np.uint32))

    # ---- the same layer with the row copy materialised: x_perm exact, y bit-identical
    layer_c = _layer(inp, cfg, gather=False)
    y_c = layer_c.forward(x)
    torch.cuda.synchronize()
    xp = layer_c.perm_out[4]
    assert gh.bits_equal(xp, x[rtok.long()])
    assert gh.bits_equal(xp[slot[:, 0].long()], x)
    assert gh.bits_equal(y_c, y)

    # ---- layer output on a seeded token sample (forced routing)
    rng = np.random.default_rng(cfg.index)
    ns = min(cfg.T, 192)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, ns, replace=False)]))
    yref, _, _ = mo.moe_layer_forward(f("x")[toks], f("w_router"), f("w1"), f("w2"), cfg.k,
                                      cfg.score, cfg.normalize, inp.logit_bias, f("w_gate"),
                                      f("ws1"), f("ws2"), topk_idx=idx[toks])
    yg = gh.to_f64(y[torch.from_numpy(toks).to(y.device)])
    tol = gh.TOL_F32 if cfg.dtype == "f32" else gh.TOL_BF16
    err = gh.normwise(yg, yref)
    print(f"[{name}] layer output normwise error on {toks.size} sampled tokens: {err:.3e}")
    assert err <= tol


def test_ep_share_forward_backward_full_size():
    cfg = mw.get("ep_share")
    inp = mw.make_ep_share_inputs(cfg)
    x, w1, w2 = gh.to_gpu(inp.x_perm), gh.to_gpu(inp.w1), gh.to_gpu(inp.w2)
    off = gh.to_gpu(inp.offsets)
    dy = gh.to_gpu(inp.dy)
    y, gu = moe.grouped_swiglu_fwd(x, w1, w2, off, save_gu=True)
    dx, dw1, dw2 = moe.grouped_swiglu_bwd(dy, x, w1, w2, off, gu)
    dx_r, dw1_r, dw2_r = moe.grouped_swiglu_bwd(dy, x, w1, w2, off, None)   # recompute path
    torch.cuda.synchronize()
    # the recompute path gives the same bits (same kernels, same G/U rounding)
    assert gh.bits_equal(dx, dx_r) and gh.bits_equal(dw1, dw1_r) and gh.bits_equal(dw2, dw2_r)
    counts = inp.counts
    order = np.argsort(counts)
    experts = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})
    print(f"\n[ep_share] rows per expert min/median/max = {counts.min()}/"
          f"{int(np.median(counts))}/{counts.max()}; checking experts {experts}")
    xf = mw.bf16_bits_to_f32(inp.x_perm)
    dyf = mw.bf16_bits_to_f32(inp.dy)
    for e in experts:
        lo, hi = int(inp.offsets[e]), int(inp.offsets[e + 1])
        W1 = mw.bf16_bits_to_f32(inp.w1[e])[None]
        W2 = mw.bf16_bits_to_f32(inp.w2[e])[None]
        seg = np.array([0, hi - lo])
        yr = mo.grouped_swiglu_fwd(xf[lo:hi], W1, W2, seg)
        dxr, dw1r, dw2r = mo.grouped_swiglu_bwd(dyf[lo:hi], xf[lo:hi], W1, W2, seg)
        e_y = gh.normwise(gh.to_f64(y[lo:hi]), yr)
        e_dx = gh.normwise(gh.to_f64(dx[lo:hi]), dxr)
        e_w1 = gh.normwise(gh.to_f64(dw1[e]), dw1r[0])
        e_w2 = gh.normwise(gh.to_f64(dw2[e]), dw2r[0])
        print(f"[ep_share] expert {e} ({hi - lo} rows): y {e_y:.2e} dx {e_dx:.2e} "
              f"dw1 {e_w1:.2e} dw2 {e_w2:.2e}")
        assert e_y <= gh.TOL_BF16
        assert max(e_dx, e_w1, e_w2) <= gh.TOL_BF16_GRAD
