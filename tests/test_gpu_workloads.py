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
  * layer output: every token, against the oracle (float64, expert segment
    by expert segment) run with the GPU's expert choice and the oracle's
    weights for it;
  * backward: dX of every slot and dW1, dW2 of every expert, against the
    oracle over all expert segments (dW: worst expert's normwise error).
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
    # the layer's route skips the per-expert counts; the permute's offsets hold them
    cnt = np.diff(layer.perm_out[0].cpu().numpy())
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

    # ---- layer output on every token (forced routing): the oracle, float64,
    # run expert segment by expert segment with the GPU's expert choice
    yref, _, _ = mo.moe_layer_forward(f("x"), f("w_router"), gh.expert_weights_view(inp, "w1"),
                                      gh.expert_weights_view(inp, "w2"), cfg.k, cfg.score,
                                      cfg.normalize, inp.logit_bias, f("w_gate"), f("ws1"),
                                      f("ws2"), topk_idx=idx)
    yg = gh.to_f64(y)
    tol = gh.TOL_F32 if cfg.dtype == "f32" else gh.TOL_BF16
    err = gh.normwise(yg, yref)
    # the worst token (the measure is a max over all elements, so a fault
    # confined to one tile of rows or columns shows in it)
    row_err = np.abs(yg - yref).max(axis=1) / np.abs(yref).max()
    print(f"[{name}] layer output normwise error on all {cfg.T} tokens: {err:.3e} "
          f"(worst token {int(row_err.argmax())}: {row_err.max():.3e})")
    assert err <= tol
    assert np.isfinite(yg).all()


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
    print(f"\n[ep_share] rows per expert min/median/max = {counts.min()}/"
          f"{int(np.median(counts))}/{counts.max()}; checking all {cfg.E} experts")
    xf = mw.bf16_bits_to_f32(inp.x_perm)
    dyf = mw.bf16_bits_to_f32(inp.dy)
    w1v, w2v = gh.expert_weights_view(inp, "w1"), gh.expert_weights_view(inp, "w2")
    # the oracle (float64) over every expert segment
    yr = mo.grouped_swiglu_fwd(xf, w1v, w2v, inp.offsets)
    dxr, dw1r, dw2r = mo.grouped_swiglu_bwd(dyf, xf, w1v, w2v, inp.offsets)
    e_y = gh.normwise(gh.to_f64(y), yr)
    e_dx = gh.normwise(gh.to_f64(dx), dxr)
    dw1g, dw2g = dw1.cpu().numpy(), dw2.cpu().numpy()
    e_w1 = gh.normwise_per_expert(dw1g, dw1r, inp.offsets)
    e_w2 = gh.normwise_per_expert(dw2g, dw2r, inp.offsets)
    print(f"[ep_share] all experts: y {e_y:.2e} dx {e_dx:.2e} dw1 (worst expert) {e_w1:.2e} "
          f"dw2 (worst expert) {e_w2:.2e}")
    assert e_y <= gh.TOL_BF16
    assert max(e_dx, e_w1, e_w2) <= gh.TOL_BF16_GRAD
