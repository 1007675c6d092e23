"""GPU parity of the full-layer backward (combine, grouped GEMM, permute and
router backward, shared expert and gate) against the oracle's
moe_layer_backward, with the GPU's own expert selection held fixed.

* small bf16 layers: softmax / sigmoid scores, with and without
  renormalisation, logit bias and gated shared expert;
* the combine and route backward kernels alone in fp32 (tolerance 1e-5),
  and the dense router backward of softmax without renormalisation at
  sizes that span several 64 x 64 tiles of its two products with ragged
  edges and up to 1024 experts;
* the qwen3_30b workload at full size: dx of every token, the router
  gradient and dW1 / dW2 of every expert.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import moe_workloads as mw  # noqa: E402
import oracle.moe_oracle as mo  # noqa: E402
import gpu_helpers as gh  # noqa: E402

moe = pytest.importorskip("mixture_experts_layer_05_amd")


def _g(a):
    return None if a is None else gh.to_gpu(a)


CASES = [
    # seed, T, d, E, k, F, Fs, score, normalize, bias
    (21, 96, 128, 12, 3, 64, 0, "softmax", True, False),
    (22, 130, 136, 10, 4, 72, 64, "sigmoid", True, True),
    (23, 77, 64, 8, 2, 64, 0, "sigmoid", False, False),
    (24, 160, 128, 16, 2, 96, 64, "softmax", True, True),
    (25, 200, 136, 70, 4, 64, 64, "softmax", False, True),   # dense router dz
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_layer_backward_parity(case):
    seed, T, d, E, k, F, Fs, score, normalize, bias = case
    inp = mw.make_small_layer_inputs(seed, T=T, d=d, E=E, F=F, dtype="bf16", Fs=Fs,
                                     bias=bias, w_std=0.05)
    rng = np.random.default_rng(seed)
    dy = mw.round_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    layer = moe.MoELayer(_g(inp.w_router), _g(inp.w1), _g(inp.w2), k, T, score, normalize,
                         _g(inp.logit_bias), _g(inp.w_gate), _g(inp.ws1), _g(inp.ws2), train=True)
    x = gh.to_gpu(inp.x)
    y = layer.forward(x)
    g1 = {kk: v.clone() for kk, v in layer.backward(gh.to_gpu(dy)).items()}
    g2 = layer.backward(gh.to_gpu(dy))
    torch.cuda.synchronize()
    for kk in g1:
        assert gh.bits_equal(g1[kk], g2[kk]), f"{kk} not deterministic"
    idx = layer.route_out[0].cpu().numpy()
    f = inp.as_f32
    ref = mo.moe_layer_backward(f("x"), f("w_router"), f("w1"), f("w2"), k,
                                mw.bf16_bits_to_f32(dy), score, normalize, inp.logit_bias,
                                f("w_gate"), f("ws1"), f("ws2"), topk_idx=idx)
    yref, _, _ = mo.moe_layer_forward(f("x"), f("w_router"), f("w1"), f("w2"), k, score,
                                      normalize, inp.logit_bias, f("w_gate"), f("ws1"), f("ws2"),
                                      topk_idx=idx)
    assert gh.normwise(gh.to_f64(y), yref) <= gh.TOL_BF16
    errs = {}
    for kk in g1:
        errs[kk] = gh.normwise(gh.to_f64(g1[kk]), np.asarray(ref[kk]))
    print(f"\n[{case}] normwise errors: " + ", ".join(f"{a} {b:.2e}" for a, b in errs.items()))
    for kk, e in errs.items():
        assert e <= gh.TOL_BF16_GRAD, (kk, e)


def test_combine_and_route_backward_fp32():
    """The two kernels alone, fp32 storage, against the oracle's functions."""
    rng = np.random.default_rng(5)
    T, d, E, k = 70, 64, 9, 3
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((E, d)) * 0.3).astype(np.float32)
    wg = (rng.standard_normal(d) * 0.3).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.2).astype(np.float32)
    for score, normalize in (("softmax", True), ("softmax", False), ("sigmoid", True),
                             ("sigmoid", False)):
        r = mo.route(x, wr, k, score, normalize, bias, wg)
        idx = r.topk_idx
        w = r.topk_w.astype(np.float32)
        p = mo.permute(x, idx, w, E)
        N = T * k
        Y = rng.standard_normal((N, d)).astype(np.float32)
        ysh = rng.standard_normal((T, d)).astype(np.float32)
        gate = r.gate.astype(np.float32)
        dy = rng.standard_normal((T, d)).astype(np.float32)
        dXp = rng.standard_normal((N, d)).astype(np.float32)
        dxa = rng.standard_normal((T, d)).astype(np.float32)
        dYr, dwr_, dgr = mo.combine_backward(dy, Y, p.slot_of, w, ysh, gate)
        dyp, dtw, dg = moe.combine_backward(_g(dy), _g(Y), _g(p.slot_of), _g(w), _g(ysh))
        torch.cuda.synchronize()
        assert gh.normwise(gh.to_f64(dyp), dYr) <= gh.TOL_F32
        assert gh.normwise(gh.to_f64(dtw), dwr_) <= gh.TOL_F32
        assert gh.normwise(gh.to_f64(dg), dgr) <= gh.TOL_F32
        dx_ref, dwr_ref, _, dwg_ref = mo.route_backward(x, wr, idx, dwr_, score, normalize, bias,
                                                        wg, dgr)
        dx_ref = dx_ref + mo.permute_backward(dXp, p.slot_of) + dxa
        dx, dwr_g, dwg_g = moe.route_backward(
            _g(x), _g(wr), _g(idx), _g(w), dtw, _g(p.offsets), _g(p.slot_of), _g(p.row_token),
            score, normalize, _g(bias), _g(wg), dg, dx_perm=_g(dXp), dx_add=_g(dxa))
        torch.cuda.synchronize()
        assert gh.normwise(gh.to_f64(dx), dx_ref) <= gh.TOL_F32, score
        assert gh.normwise(gh.to_f64(dwr_g), dwr_ref) <= gh.TOL_F32, score
        assert gh.normwise(gh.to_f64(dwg_g), dwg_ref) <= gh.TOL_F32, score


def test_layer_backward_full_size_qwen3_30b():
    """Every token's dx, every expert's dW1 / dW2 and the whole router
    gradient at full size, against the oracle (float64) run over all
    tokens with the GPU's selection."""
    cfg = mw.get("qwen3_30b")
    inp = mw.make_layer_inputs(cfg)
    f = inp.as_f32
    rng = np.random.default_rng(77)
    dy = mw.round_to_bf16_bits(rng.standard_normal((cfg.T, cfg.d)).astype(np.float32))
    layer = moe.MoELayer(_g(inp.w_router), _g(inp.w1), _g(inp.w2), cfg.k, cfg.T, cfg.score,
                         cfg.normalize, train=True)
    layer.forward(gh.to_gpu(inp.x))
    g = layer.backward(gh.to_gpu(dy))
    torch.cuda.synchronize()
    idx = layer.route_out[0].cpu().numpy()
    ref = mo.moe_layer_backward(f("x"), f("w_router"), gh.expert_weights_view(inp, "w1"),
                                gh.expert_weights_view(inp, "w2"), cfg.k,
                                mw.bf16_bits_to_f32(dy), cfg.score, cfg.normalize,
                                topk_idx=idx)
    off = ref["offsets"]
    tol = gh.TOL_BF16_GRAD
    errs = {
        "dx": gh.normwise(gh.to_f64(g["dx"]), ref["dx"]),
        "dw_router": gh.normwise(gh.to_f64(g["dw_router"]), ref["dw_router"]),
        "dw1 (worst expert)": gh.normwise_per_expert(g["dw1"].cpu().numpy(), ref["dw1"], off),
        "dw2 (worst expert)": gh.normwise_per_expert(g["dw2"].cpu().numpy(), ref["dw2"], off),
    }
    print("\n[qwen3_30b backward, all tokens and experts] "
          + ", ".join(f"{a} {b:.2e}" for a, b in errs.items()))
    for kk, e in errs.items():
        assert e <= tol, (kk, e)


@pytest.mark.parametrize("T,d,E,k,dtype", [(1, 8, 1, 1, "f32"), (333, 200, 300, 8, "f32"),
                                           (130, 72, 1024, 32, "f32"),
                                           (517, 256, 128, 8, "bf16")])
def test_route_backward_dense_softmax(T, d, E, k, dtype):
    """Softmax scores without renormalisation: dz is dense over all E experts.
    dx and dW_r against the oracle's route_backward (float64), with
    accumulate onto a non-zero dW_r."""
    rng = np.random.default_rng(T + E)
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((E, d)) * 0.3).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.2).astype(np.float32)
    if dtype == "bf16":
        x = mw.bf16_bits_to_f32(mw.round_to_bf16_bits(x))
        wr = mw.bf16_bits_to_f32(mw.round_to_bf16_bits(wr))
    r = mo.route(x, wr, k, "softmax", False, bias)
    idx = r.topk_idx
    w = r.topk_w.astype(np.float32)
    p = mo.permute(x, idx, w, E)
    dtw = rng.standard_normal((T, k)).astype(np.float32)
    dw0 = rng.standard_normal((E, d)).astype(np.float32)
    dx_ref, dwr_ref, _, _ = mo.route_backward(x, wr, idx, dtw, "softmax", False, bias)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    dwr = _g(dw0)
    dx, dwr_g, _ = moe.route_backward(
        _g(x).to(tdt), _g(wr).to(tdt), _g(idx), _g(w), _g(dtw), _g(p.offsets), _g(p.slot_of),
        _g(p.row_token), "softmax", False, _g(bias), accumulate=True, dw_router=dwr)
    torch.cuda.synchronize()
    tol_dx = gh.TOL_F32 if dtype == "f32" else gh.TOL_BF16
    assert gh.normwise(gh.to_f64(dx), dx_ref) <= tol_dx
    assert gh.normwise(gh.to_f64(dwr_g) - dw0, dwr_ref) <= gh.TOL_F32
