"""GPU parity of each C-ABI call against the CPU oracle at small, odd shapes
(several tiles plus ragged tails, empty experts, k = 1 and k = E, E not a
multiple of 64, d and F not multiples of the tile sizes).

Every output buffer is poison-filled first (NaN / -1) so an unwritten
element fails, and every call is run twice to check bitwise determinism.
"""
import numpy as np
import pytest
import torch

import moe_workloads as mw
from oracle import moe_oracle as mo
import gpu_helpers as gh

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("mixture_experts_layer_05_amd")


def _dtype(s):
    return torch.float32 if s == "f32" else torch.bfloat16


ROUTE_CASES = [
    # T, d, E, k, score, bias, gate, dtype
    (1, 64, 8, 2, "softmax", False, False, "f32"),
    (257, 128, 8, 2, "softmax", False, False, "f32"),
    (300, 64, 33, 5, "sigmoid", True, True, "f32"),
    (33, 136, 8, 8, "softmax", False, False, "bf16"),     # k = E
    (513, 256, 130, 6, "sigmoid", False, False, "bf16"),
    (700, 512, 256, 8, "softmax", True, True, "bf16"),
    (129, 264, 1000, 32, "softmax", False, False, "bf16"),
    (100, 64, 1, 1, "softmax", False, False, "bf16"),      # E = 1
    (1000, 256, 256, 8, "softmax", True, True, "bf16"),   # 16 lanes x 16 scores per token
    (77, 128, 17, 16, "sigmoid", False, False, "f32"),    # k > 16: two choices per lane
    (200, 64, 300, 32, "softmax", False, True, "f32"),    # a wavefront per token, k = 32
    (129, 72, 600, 3, "sigmoid", True, False, "bf16"),
]


def _block_hist(idx, E, blk=64):
    """Per-64-token-block expert counts of a [T, k] choice matrix (entries
    outside [0, E) dropped)."""
    T = idx.shape[0]
    nb = -(-T // blk)
    h = np.zeros((nb, E), dtype=np.int32)
    for b in range(nb):
        v = idx[b * blk:(b + 1) * blk].reshape(-1)
        v = v[(v >= 0) & (v < E)]
        h[b] = np.bincount(v, minlength=E)
    return h


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_route_parity(case):
    T, d, E, k, score, bias, gate, dt = case
    inp = mw.make_small_layer_inputs(11 + T + E, T=T, d=d, E=E, F=8, dtype=dt,
                                     Fs=8 if gate else 0, bias=bias)
    ref = mo.route(inp.as_f32("x"), inp.as_f32("w_router"), k, score, True,
                   inp.logit_bias, inp.as_f32("w_gate"))
    x = gh.to_gpu(inp.x)
    wr = gh.to_gpu(inp.w_router)
    b = gh.to_gpu(inp.logit_bias) if bias else None
    wg = gh.to_gpu(inp.w_gate) if gate else None
    outs, bcs = [], []
    for _ in range(2):
        out = (gh.poison((T, k), torch.int32), gh.poison((T, k), torch.float32),
               gh.poison((E,), torch.int32), gh.poison((T,), torch.float32) if gate else None)
        bc = gh.poison(((T + 63) // 64, E), torch.int32)
        moe.route(x, wr, k, score, True, b, wg, out=out, block_counts=bc)
        torch.cuda.synchronize()
        outs.append(out)
        bcs.append(bc)
    for a, c in zip(outs[0], outs[1]):
        if a is not None:
            assert gh.bits_equal(a, c)
    # without the per-expert counts (NULL): the same choice, weights and gate
    out = (gh.poison((T, k), torch.int32), gh.poison((T, k), torch.float32), None,
           gh.poison((T,), torch.float32) if gate else None)
    moe.route(x, wr, k, score, True, b, wg, out=out)
    torch.cuda.synchronize()
    for a, c in zip(outs[0], out):
        if c is not None:
            assert gh.bits_equal(a, c)
    idx, w, cnt, g = (o.cpu().numpy() if o is not None else None for o in outs[0])
    gh.check_routing(idx, w, ref, k)
    assert (cnt == np.bincount(idx.reshape(-1), minlength=E)).all()
    assert np.array_equal(bcs[0].cpu().numpy(), _block_hist(idx, E))
    if gate:
        assert np.abs(g - ref.gate).max() <= gh.TOL_ROUTE_W


TIE_CASES = [
    # T, d, E, k, score, normalize, bias ("logit": added to the logits,
    # "select": selection only), dtype
    (300, 128, 64, 7, "softmax", True, None, "bf16"),
    (300, 128, 128, 6, "sigmoid", True, None, "bf16"),
    (257, 64, 256, 8, "softmax", True, "logit", "f32"),
    (129, 64, 130, 5, "sigmoid", True, "select", "bf16"),
    (200, 64, 256, 8, "sigmoid", False, None, "bf16"),
    (90, 64, 600, 9, "softmax", True, None, "bf16"),
]


@pytest.mark.parametrize("case", TIE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_route_exact_ties(case):
    """Expert 2i+1 is a copy of expert 2i (router row and bias), so every
    token's scores come in exactly equal pairs.  Equal scores rank the lower
    index first: a chosen odd expert has its even twin chosen at an earlier
    place, with a bitwise equal weight."""
    T, d, E, k, score, norm, bias, dt = case
    inp = mw.make_small_layer_inputs(29 + T + E, T=T, d=d, E=E, F=8, dtype=dt,
                                     Fs=0, bias=bias == "logit")
    inp.w_router = inp.w_router.copy()
    inp.w_router[1::2] = inp.w_router[0::2]
    lb = sb = None
    if bias == "logit":
        lb = inp.logit_bias.copy()
        lb[1::2] = lb[0::2]
    elif bias == "select":
        sb = (np.random.default_rng(E).standard_normal(E) * 0.1).astype(np.float32)
        sb[1::2] = sb[0::2]
    ref = mo.route(inp.as_f32("x"), inp.as_f32("w_router"), k, score, norm, lb, None,
                   selection_bias=sb)
    out = (gh.poison((T, k), torch.int32), gh.poison((T, k), torch.float32),
           gh.poison((E,), torch.int32), None)
    g = lambda a: None if a is None else gh.to_gpu(a)  # noqa: E731
    moe.route(g(inp.x), g(inp.w_router), k, score, norm, g(lb), None, out=out,
              selection_bias=g(sb))
    torch.cuda.synchronize()
    idx, w = out[0].cpu().numpy(), out[1].cpu().numpy()
    gh.check_routing(idx, w, ref, k)
    n_pairs = 0
    for t in range(T):
        place = {int(e): j for j, e in enumerate(idx[t])}
        for e, j in place.items():
            if e % 2:
                assert e - 1 in place and place[e - 1] < j, (t, idx[t])
                assert w[t, j] == w[t, place[e - 1]], (t, e)
                n_pairs += 1
    assert n_pairs > 0
    assert (out[2].cpu().numpy() == np.bincount(idx.reshape(-1), minlength=E)).all()


MASK_CASES = [
    # T, d, E, k, score, normalize, masked experts, dtype
    (200, 64, 16, 8, "softmax", True, 12, "bf16"),     # 4 finite: 4 masked places
    (200, 64, 16, 8, "sigmoid", True, 12, "f32"),
    (257, 64, 64, 8, "sigmoid", True, 20, "bf16"),     # masked never needed
    (200, 64, 64, 6, "softmax", False, 60, "bf16"),    # ranking on scores
    (150, 64, 300, 8, "softmax", True, 296, "bf16"),   # a wavefront per token
]


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: "-".join(map(str, c)))
def test_route_masked_experts(case):
    """A -inf logit bias masks an expert: its score and weight are 0 and it is
    chosen only after every expert with a finite logit, lower index first,
    as the oracle's descending stable sort of the scores does."""
    T, d, E, k, score, norm, nmask, dt = case
    inp = mw.make_small_layer_inputs(53 + T + E, T=T, d=d, E=E, F=8, dtype=dt, Fs=0, bias=True)
    masked = np.random.default_rng(E + nmask).permutation(E)[:nmask]
    lb = inp.logit_bias.copy()
    lb[masked] = -np.inf
    ref = mo.route(inp.as_f32("x"), inp.as_f32("w_router"), k, score, norm, lb, None)
    g = lambda a: gh.to_gpu(a)  # noqa: E731
    idx, w, cnt, _ = moe.route(g(inp.x), g(inp.w_router), k, score, norm, g(lb), None)
    torch.cuda.synchronize()
    idx, w, cnt = idx.cpu().numpy(), w.cpu().numpy(), cnt.cpu().numpy()
    is_m = np.zeros(E, bool)
    is_m[masked] = True
    nfin = min(k, E - nmask)
    # the finite experts: the oracle's choice (near ties aside)
    fin_ref = ref.topk_idx[:, :nfin]
    assert not is_m[fin_ref].any()
    assert not is_m[idx[:, :nfin]].any()
    same = (np.sort(idx[:, :nfin], 1) == np.sort(fin_ref, 1)).all(1)
    assert same.mean() > 0.95, same.mean()
    # the masked places: exactly the oracle's (lowest masked indices, ascending), weight 0
    assert np.array_equal(idx[:, nfin:], ref.topk_idx[:, nfin:])
    assert (w[:, nfin:] == 0.0).all()
    ow = ref.topk_w[same][:, :nfin]
    gw = w[same][:, :nfin]
    o_order = np.argsort(ref.topk_idx[same][:, :nfin], 1)
    g_order = np.argsort(idx[same][:, :nfin], 1)
    assert np.abs(np.take_along_axis(ow, o_order, 1) -
                  np.take_along_axis(gw, g_order, 1)).max() <= gh.TOL_ROUTE_W
    assert (cnt == np.bincount(idx.reshape(-1), minlength=E)).all()


def test_route_nan_token():
    """A token whose logits are all NaN has no selectable expert: every place
    gets index E (dropped by the permute); the other tokens are unaffected."""
    T, d, E, k = 130, 64, 64, 6
    inp = mw.make_small_layer_inputs(71, T=T, d=d, E=E, F=8, dtype="bf16", Fs=0)
    x = inp.x.copy()
    bad = np.array([0, 77, 129])
    x[bad] = 0x7FC0                       # bf16 quiet NaN
    idx, w, cnt, _ = moe.route(gh.to_gpu(x), gh.to_gpu(inp.w_router), k, "softmax", True)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    assert (idx[bad] == E).all()
    good = np.setdiff1d(np.arange(T), bad)
    ref = mo.route(inp.as_f32("x")[good], inp.as_f32("w_router"), k, "softmax", True)
    gh.check_routing(idx[good], w.cpu().numpy()[good], ref, k)
    assert (cnt == np.bincount(idx[good].reshape(-1), minlength=E)).all()


SELB_CASES = [
    # T, d, E, k, score, dtype, bias std
    (300, 64, 33, 5, "sigmoid", "f32", 0.1),
    (513, 256, 130, 6, "sigmoid", "bf16", 0.1),
    (700, 128, 128, 8, "softmax", "bf16", 0.01),
]


@pytest.mark.parametrize("case", SELB_CASES, ids=lambda c: "-".join(map(str, c)))
def test_route_selection_bias_parity(case):
    """Selection-only expert bias: the choice ranks by score + bias, the
    weights are the unbiased scores of the chosen experts."""
    T, d, E, k, score, dt, std = case
    inp = mw.make_small_layer_inputs(40 + T + E, T=T, d=d, E=E, F=8, dtype=dt)
    sb = (np.random.default_rng(T + E).standard_normal(E) * std).astype(np.float32)
    ref = mo.route(inp.as_f32("x"), inp.as_f32("w_router"), k, score, True,
                   selection_bias=sb)
    plain = mo.route(inp.as_f32("x"), inp.as_f32("w_router"), k, score, True)
    moved = (np.sort(ref.topk_idx, 1) != np.sort(plain.topk_idx, 1)).any(1).mean()
    assert moved > 0.05, f"bias changed only {moved:.1%} of the choices"
    idx, w, cnt, _ = moe.route(gh.to_gpu(inp.x), gh.to_gpu(inp.w_router), k, score, True,
                               selection_bias=gh.to_gpu(sb))
    torch.cuda.synchronize()
    idx, w, cnt = idx.cpu().numpy(), w.cpu().numpy(), cnt.cpu().numpy()
    gh.check_routing(idx, w, ref, k)
    assert (cnt == np.bincount(idx.reshape(-1), minlength=E)).all()


def test_shared_overlap_matches_serial():
    """The shared expert on a second stream (unscaled, gate applied in the
    combine) equals the serial path up to where the gate is rounded."""
    T, k = 160, 2
    inp = mw.make_small_layer_inputs(8, T=T, d=128, E=16, F=96, dtype="bf16", Fs=64, bias=True,
                                     w_std=0.05)
    g = lambda a: None if a is None else gh.to_gpu(a)  # noqa: E731
    args = (g(inp.w_router), g(inp.w1), g(inp.w2), k, T, "softmax", True, g(inp.logit_bias),
            g(inp.w_gate), g(inp.ws1), g(inp.ws2))
    x = gh.to_gpu(inp.x)
    y1 = moe.MoELayer(*args, overlap_shared=True).forward(x).clone()
    y2 = moe.MoELayer(*args, overlap_shared=False).forward(x).clone()
    torch.cuda.synchronize()
    f = inp.as_f32
    layer = moe.MoELayer(*args)
    layer.forward(x)
    idx = layer.route_out[0].cpu().numpy()
    ref, _, _ = mo.moe_layer_forward(f("x"), f("w_router"), f("w1"), f("w2"), k, "softmax", True,
                                     inp.logit_bias, f("w_gate"), f("ws1"), f("ws2"), topk_idx=idx)
    assert gh.normwise(gh.to_f64(y1), ref) <= gh.TOL_BF16
    assert gh.normwise(gh.to_f64(y2), ref) <= gh.TOL_BF16
    assert gh.normwise(gh.to_f64(y1), gh.to_f64(y2)) <= gh.TOL_BF16


def test_layer_packed_matches_unpacked():
    """The inference layer on tile-packed weights (its default) equals the layer
    on the weights as stored, bit for bit; repack() follows a weight change."""
    T, k = 300, 4
    inp = mw.make_small_layer_inputs(9, T=T, d=192, E=12, F=136, dtype="bf16", Fs=72,
                                     bias=True, w_std=0.05)
    g = lambda a: None if a is None else gh.to_gpu(a)  # noqa: E731
    args = (g(inp.w_router), g(inp.w1), g(inp.w2), k, T, "softmax", True, g(inp.logit_bias),
            g(inp.w_gate), g(inp.ws1), g(inp.ws2))
    x = gh.to_gpu(inp.x)
    lp = moe.MoELayer(*args)
    lu = moe.MoELayer(*args, packed=False)
    assert lp.packed and not lu.packed
    y1, y2 = lp.forward(x).clone(), lu.forward(x).clone()
    torch.cuda.synchronize()
    assert gh.bits_equal(y1, y2)
    lp.w2.mul_(0.5)                     # shared storage: both layers see the change
    lp.repack()
    y3, y4 = lp.forward(x).clone(), lu.forward(x).clone()
    torch.cuda.synchronize()
    assert gh.bits_equal(y3, y4) and not gh.bits_equal(y1, y3)



@pytest.mark.parametrize("gated", [True, False])
def test_layer_fold_shared(gated):
    """A shared expert whose ffn equals the routed experts' runs as group E of
    the routed grouped GEMM (the layer's default then): bit for bit the
    layer with its own shared call, and the oracle's layer to the bf16
    tolerance (gated); without a gate its rows take row scale 1."""
    T, k, F = 300, 4, 136
    inp = mw.make_small_layer_inputs(10, T=T, d=192, E=12, F=F, dtype="bf16", Fs=F, bias=True,
                                     w_std=0.05)
    g = lambda a: None if a is None else gh.to_gpu(a)  # noqa: E731
    wg = g(inp.w_gate) if gated else None
    args = (g(inp.w_router), g(inp.w1), g(inp.w2), k, T, "softmax", True, g(inp.logit_bias),
            wg, g(inp.ws1), g(inp.ws2))
    x = gh.to_gpu(inp.x)
    lf = moe.MoELayer(*args)
    lu = moe.MoELayer(*args, fold_shared=False)
    assert lf.fold_shared and not lu.fold_shared
    y1, y2 = lf.forward(x).clone(), lu.forward(x).clone()
    y3 = lf.forward(x).clone()
    torch.cuda.synchronize()
    assert gh.bits_equal(y1, y2) and gh.bits_equal(y1, y3)
    assert gh.bits_equal(lf.y_shared, lu.y_shared)
    if gated:      # the oracle's shared expert is the gated one
        f = inp.as_f32
        idx = lf.route_out[0].cpu().numpy()
        ref, _, _ = mo.moe_layer_forward(f("x"), f("w_router"), f("w1"), f("w2"), k, "softmax",
                                         True, inp.logit_bias, f("w_gate"), f("ws1"), f("ws2"),
                                         topk_idx=idx)
        assert gh.normwise(gh.to_f64(y1), ref) <= gh.TOL_BF16
    assert not moe.MoELayer(*args, save_gu=True).fold_shared   # G, U kept for the routed rows only
    with pytest.raises(moe.MoEError):   # ffn mismatch: cannot fold
        moe.MoELayer(g(inp.w_router), g(inp.w1), g(inp.w2), k, T, "softmax", True, None, wg,
                     g(inp.ws1)[: 2 * 64].contiguous(), g(inp.ws2)[:, :64].contiguous(),
                     fold_shared=True)

PERM_CASES = [
    # T, d, E, k, dtype, pattern
    (1, 64, 4, 1, "bf16", "random"),
    (300, 64, 16, 4, "bf16", "random"),
    (1000, 136, 130, 6, "bf16", "random"),
    (257, 128, 8, 2, "f32", "random"),
    (500, 64, 64, 1, "bf16", "one_expert"),          # every token on expert 0
    (300, 64, 40, 8, "bf16", "few_experts"),         # most experts empty
    (99, 64, 1024, 32, "bf16", "random"),            # E = 1024, k = 32
    (1000, 64, 256, 8, "bf16", "random"),            # 16 blocks of 64 tokens, a ragged last
    (500, 64, 64, 4, "bf16", "dup"),                 # a token may name an expert twice
    (130, 64, 8, 32, "bf16", "dup"),                 # k > E: every token repeats experts
]


def _idx(rng, T, E, k, pattern):
    if pattern == "one_expert":
        return np.zeros((T, k), dtype=np.int32)
    if pattern == "dup":
        return rng.integers(0, E, (T, k)).astype(np.int32)
    pool = np.arange(E) if pattern == "random" else np.arange(0, E, 5)[: max(k, 8)]
    return np.stack([rng.choice(pool, size=k, replace=False) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("case", PERM_CASES, ids=lambda c: "-".join(map(str, c)))
def test_permute_parity(case):
    T, d, E, k, dt, pattern = case
    rng = np.random.default_rng(T + E + k)
    idx = _idx(rng, T, E, k, pattern)
    w = rng.random((T, k)).astype(np.float32)
    inp = mw.make_small_layer_inputs(5, T=T, d=d, E=1, F=8, dtype=dt)
    ref = mo.permute(inp.x, idx, w, E)
    x = gh.to_gpu(inp.x)
    gi, gw = gh.to_gpu(idx), gh.to_gpu(w)
    N = T * k
    res = []
    for _ in range(2):
        out = (gh.poison((E + 1,), torch.int32), gh.poison((T, k), torch.int32),
               gh.poison((N,), torch.int32), gh.poison((N,), torch.float32),
               gh.poison((N, d), x.dtype))
        moe.permute(x, gi, gw, E, out=out)
        torch.cuda.synchronize()
        res.append(out)
    # with the counts pass replaced by given block histograms (moe_route's)
    bc = gh.to_gpu(_block_hist(idx, E))
    bc_before = bc.clone()
    out = (gh.poison((E + 1,), torch.int32), gh.poison((T, k), torch.int32),
           gh.poison((N,), torch.int32), gh.poison((N,), torch.float32),
           gh.poison((N, d), x.dtype))
    moe.permute(x, gi, gw, E, out=out, block_counts=bc)
    torch.cuda.synchronize()
    res.append(out)
    assert gh.bits_equal(bc, bc_before)         # an input only
    for r in res[1:]:
        for a, c in zip(res[0], r):
            assert gh.bits_equal(a, c)
    off, slot, rtok, rw, xp = res[0]
    assert off.cpu().numpy().tolist() == ref.offsets.tolist()
    assert np.array_equal(slot.cpu().numpy(), ref.slot_of)
    assert np.array_equal(rtok.cpu().numpy(), ref.row_token)
    assert np.array_equal(rw.cpu().numpy().view(np.uint32), ref.row_w.view(np.uint32))
    xp_ref = gh.to_gpu(ref.x_perm)
    assert gh.bits_equal(xp, xp_ref)
    # unpermute(permute(x)) == x for every copy
    for j in range(k):
        assert gh.bits_equal(xp[slot[:, j].long()], x)


def test_permute_drops_out_of_range_experts():
    T, d, E, k = 50, 64, 8, 2
    rng = np.random.default_rng(1)
    idx = _idx(rng, T, E, k, "random")
    idx[3, 1] = -1
    idx[7, 0] = E
    x = gh.to_gpu(mw.make_small_layer_inputs(2, T=T, d=d, E=1, F=8, dtype="bf16").x)
    off, slot, rtok, _, xp = moe.permute(x, gh.to_gpu(idx), None, E)
    slot = slot.cpu().numpy()
    assert slot[3, 1] == -1 and slot[7, 0] == -1
    assert off.cpu().numpy()[-1] == T * k - 2
    valid = slot >= 0
    assert sorted(slot[valid].tolist()) == list(range(T * k - 2))


def _segments(rng, E, pattern, scale):
    if pattern == "ragged":
        c = rng.integers(0, scale, E)
        c[::3] = 0                              # empty experts
        c[1] = 1                                # a one-row expert
        return c
    if pattern == "one_hot":
        c = np.zeros(E, dtype=np.int64)
        c[E // 2] = scale
        return c
    if pattern == "heavy":                      # one expert holds most rows
        c = rng.integers(0, max(2, scale // 30), E)
        c[0] = scale
        c[2 % E] = 0
        return c
    raise ValueError(pattern)


FFN_CASES = [
    # E, d, F, dtype, pattern, scale
    (5, 64, 64, "f32", "ragged", 150),
    (4, 128, 256, "f32", "ragged", 90),
    (6, 64, 64, "bf16", "ragged", 300),
    (7, 136, 72, "bf16", "ragged", 200),       # K and N tails
    (3, 256, 192, "bf16", "one_hot", 517),
    (9, 192, 136, "bf16", "ragged", 140),
]


@pytest.mark.parametrize("case", FFN_CASES, ids=lambda c: "-".join(map(str, c)))
def test_grouped_fwd_parity(case):
    E, d, F, dt, pattern, scale = case
    rng = np.random.default_rng(E * 1000 + d + F)
    counts = _segments(rng, E, pattern, scale)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(off[-1])
    inp = mw.make_small_layer_inputs(E + d + F, T=N, d=d, E=E, F=F, dtype=dt, w_std=0.05)
    rs = (rng.random(N) + 0.5).astype(np.float32)
    y_ref, gu_ref = mo.grouped_swiglu_fwd(inp.as_f32("x"), inp.as_f32("w1"), inp.as_f32("w2"),
                                          off, rs, return_gu=True)
    x, w1, w2 = gh.to_gpu(inp.x), gh.to_gpu(inp.w1), gh.to_gpu(inp.w2)
    go, grs = gh.to_gpu(off), gh.to_gpu(rs)
    res = []
    for _ in range(2):
        y = gh.poison((N, d), x.dtype)
        gu = gh.poison((N, 2 * F), x.dtype)
        moe.grouped_swiglu_fwd(x, w1, w2, go, grs, save_gu=True, out=y, gu_out=gu)
        torch.cuda.synchronize()
        res.append((y, gu))
    assert gh.bits_equal(res[0][0], res[1][0]) and gh.bits_equal(res[0][1], res[1][1])
    tol = gh.TOL_F32 if dt == "f32" else gh.TOL_BF16
    y, gu = (gh.to_f64(t) for t in res[0])
    assert np.isfinite(y).all()
    assert gh.normwise(y, y_ref) <= tol
    assert gh.normwise(gu, gu_ref) <= tol


GATHER_CASES = [
    # E, d, F, dtype, T (rows of x), bad tokens
    (6, 64, 64, "f32", 70, False),
    (7, 136, 72, "bf16", 45, False),
    (5, 192, 136, "bf16", 300, True),
]


@pytest.mark.parametrize("case", GATHER_CASES, ids=lambda c: "-".join(map(str, c)))
def test_grouped_fwd_gather_parity(case):
    """fc1 reading x[row_token] directly equals the forward on the copied rows,
    bit for bit, and the oracle to the usual tolerance; a row_token outside
    [0, T) reads as a zero row."""
    E, d, F, dt, T, bad = case
    rng = np.random.default_rng(E * 31 + d + T)
    counts = _segments(rng, E, "ragged", 200)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(off[-1])
    inp = mw.make_small_layer_inputs(E + d + T, T=T, d=d, E=E, F=F, dtype=dt, w_std=0.05)
    rtok = rng.integers(0, T, N).astype(np.int32)
    if bad:
        rtok[rng.choice(N, 5, replace=False)] = np.array([-1, T, T + 7, -100, 2 ** 30], np.int32)
    rs = (rng.random(N) + 0.5).astype(np.float32)
    xf = inp.as_f32("x")
    ok = (rtok >= 0) & (rtok < T)
    xp_ref = np.where(ok[:, None], xf[np.clip(rtok, 0, T - 1)], 0.0)
    y_ref, gu_ref = mo.grouped_swiglu_fwd(xp_ref, inp.as_f32("w1"), inp.as_f32("w2"), off, rs,
                                          return_gu=True)
    x, w1, w2 = gh.to_gpu(inp.x), gh.to_gpu(inp.w1), gh.to_gpu(inp.w2)
    go, grs, gtok = gh.to_gpu(off), gh.to_gpu(rs), gh.to_gpu(rtok)
    y = gh.poison((N, d), x.dtype)
    gu = gh.poison((N, 2 * F), x.dtype)
    moe.grouped_swiglu_fwd_gather(x, gtok, w1, w2, go, grs, save_gu=True, out=y, gu_out=gu)
    # the same rows materialised (zero rows where the token is out of range)
    xp = torch.zeros((N, d), dtype=x.dtype, device=x.device)
    okg = torch.from_numpy(ok).to(x.device)
    xp[okg] = x[gtok[okg].long()]
    y2, gu2 = moe.grouped_swiglu_fwd(xp, w1, w2, go, grs, save_gu=True)
    torch.cuda.synchronize()
    assert gh.bits_equal(y, y2) and gh.bits_equal(gu, gu2)
    tol = gh.TOL_F32 if dt == "f32" else gh.TOL_BF16
    assert gh.normwise(gh.to_f64(y), y_ref) <= tol
    assert gh.normwise(gh.to_f64(gu), gu_ref) <= tol


def _pack_reference(w, gated, bn=256, bk=64):
    """The tile-packed layout written out from its definition in include/moe.h
    (a data reordering only), for comparison with moe_pack_weights."""
    E, rows, K = w.shape
    if gated:
        F = rows // 2
        nt = -(-F // (bn // 2))
    else:
        nt = -(-rows // bn)
    nkt = -(-K // bk)
    out = np.zeros((E, nt, nkt, bn, bk), dtype=w.dtype)
    for t in range(nt):
        for r in range(bn):
            if gated:
                f = t * (bn // 2) + (r if r < bn // 2 else r - bn // 2)
                row = (f if r < bn // 2 else F + f) if f < F else -1
            else:
                row = t * bn + r if t * bn + r < rows else -1
            if row < 0:
                continue
            for kt in range(nkt):
                k0, k1 = kt * bk, min(K, kt * bk + bk)
                out[:, t, kt, r, :k1 - k0] = w[:, row, k0:k1]
    return out


@pytest.mark.parametrize("case", [(3, 2 * 72, 136, True), (2, 200, 72, False),
                                  (1, 2 * 256, 64, True), (2, 520, 8, False)],
                         ids=lambda c: "-".join(map(str, c)))
def test_pack_weights_layout(case):
    """moe_pack_weights places every weight where the layout says, zeros elsewhere."""
    E, rows, K, gated = case
    rng = np.random.default_rng(rows + K)
    w = mw.round_to_bf16_bits(rng.standard_normal((E, rows, K)).astype(np.float32))
    ref = _pack_reference(w, gated)
    wp = moe.pack_weights(gh.to_gpu(w), gated)
    torch.cuda.synchronize()
    got = wp.buf.view(torch.int16).cpu().numpy().view(np.uint16)
    assert got.size == ref.size
    assert (got == ref.reshape(-1)).all()


PACKED_CASES = [
    # E, d, F, T (rows of x; 0: no gather), pattern, scale
    (6, 64, 64, 0, "ragged", 300),
    (7, 136, 72, 45, "ragged", 200),          # K and N tails, gathered rows
    (3, 256, 192, 0, "one_hot", 517),
    (9, 200, 136, 300, "ragged", 140),        # d not a multiple of 64
    (4, 512, 320, 0, "ragged", 600),          # several column tiles of both GEMMs
]


@pytest.mark.parametrize("case", PACKED_CASES, ids=lambda c: "-".join(map(str, c)))
def test_grouped_fwd_packed_parity(case):
    """The forward on tile-packed weights equals the forward on the weights as
    stored, bit for bit (with and without the gathered first operand), and
    the oracle to the bf16 tolerance."""
    E, d, F, T, pattern, scale = case
    rng = np.random.default_rng(E * 7 + d + F + T)
    counts = _segments(rng, E, pattern, scale)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(off[-1])
    rows = T if T else N
    inp = mw.make_small_layer_inputs(E + d + F + 5, T=rows, d=d, E=E, F=F, dtype="bf16",
                                     w_std=0.05)
    rs = (rng.random(N) + 0.5).astype(np.float32)
    x, w1, w2 = gh.to_gpu(inp.x), gh.to_gpu(inp.w1), gh.to_gpu(inp.w2)
    go, grs = gh.to_gpu(off), gh.to_gpu(rs)
    w1p, w2p = moe.pack_weights(w1, True), moe.pack_weights(w2, False)
    if T:
        rtok = rng.integers(0, T, N).astype(np.int32)
        gtok = gh.to_gpu(rtok)
        y_u, gu_u = moe.grouped_swiglu_fwd_gather(x, gtok, w1, w2, go, grs, save_gu=True)
        xp_ref = inp.as_f32("x")[rtok]
    else:
        gtok = None
        y_u, gu_u = moe.grouped_swiglu_fwd(x, w1, w2, go, grs, save_gu=True)
        xp_ref = inp.as_f32("x")
    res = []
    for _ in range(2):
        y = gh.poison((N, d), x.dtype)
        gu = gh.poison((N, 2 * F), x.dtype)
        moe.grouped_swiglu_fwd_packed(x, gtok, w1p, w2p, go, grs, save_gu=True, out=y, gu_out=gu)
        torch.cuda.synchronize()
        res.append((y, gu))
    assert gh.bits_equal(res[0][0], res[1][0]) and gh.bits_equal(res[0][1], res[1][1])
    assert gh.bits_equal(res[0][0], y_u) and gh.bits_equal(res[0][1], gu_u)
    y_ref, gu_ref = mo.grouped_swiglu_fwd(xp_ref, inp.as_f32("w1"), inp.as_f32("w2"), off, rs,
                                          return_gu=True)
    assert gh.normwise(gh.to_f64(res[0][0]), y_ref) <= gh.TOL_BF16
    assert gh.normwise(gh.to_f64(res[0][1]), gu_ref) <= gh.TOL_BF16


BWD_CASES = [
    # E, d, F, pattern, scale, save_gu, row_scale, accumulate
    (5, 64, 64, "ragged", 200, True, False, False),
    (7, 136, 72, "ragged", 200, True, True, False),
    (4, 128, 128, "ragged", 300, False, True, True),
    (3, 256, 192, "one_hot", 517, True, False, True),
    # one dominant expert: its weight-gradient tiles are split along K
    (5, 128, 64, "heavy", 3000, True, True, False),
    (4, 256, 192, "heavy", 2500, False, False, True),
    # the most experts the calls take, a third of them empty
    (1024, 64, 64, "ragged", 8, True, True, False),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_grouped_bwd_parity(case):
    E, d, F, pattern, scale, save_gu, use_rs, acc = case
    rng = np.random.default_rng(E * 7 + d + F)
    counts = _segments(rng, E, pattern, scale)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(off[-1])
    inp = mw.make_small_layer_inputs(3 * E + d, T=N, d=d, E=E, F=F, dtype="bf16", w_std=0.05)
    dy = mw.round_to_bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    rs = (rng.random(N) + 0.5).astype(np.float32) if use_rs else None
    f = inp.as_f32
    dx_ref, dw1_ref, dw2_ref = mo.grouped_swiglu_bwd(mw.bf16_bits_to_f32(dy), f("x"), f("w1"),
                                                     f("w2"), off, rs)
    x, w1, w2 = gh.to_gpu(inp.x), gh.to_gpu(inp.w1), gh.to_gpu(inp.w2)
    go = gh.to_gpu(off)
    grs = gh.to_gpu(rs) if use_rs else None
    gdy = gh.to_gpu(dy)
    gu = None
    if save_gu:
        _, gu = moe.grouped_swiglu_fwd(x, w1, w2, go, grs, save_gu=True)
    base1 = torch.full((E, 2 * F, d), 0.25, dtype=torch.float32, device=gh.dev())
    base2 = torch.full((E, d, F), -0.5, dtype=torch.float32, device=gh.dev())
    res = []
    for _ in range(2):
        dw1 = base1.clone() if acc else gh.poison((E, 2 * F, d), torch.float32)
        dw2 = base2.clone() if acc else gh.poison((E, d, F), torch.float32)
        dx = gh.poison((N, d), x.dtype)
        moe.grouped_swiglu_bwd(gdy, x, w1, w2, go, gu, grs, acc, dw1, dw2, dx_out=dx)
        torch.cuda.synchronize()
        res.append((dx, dw1, dw2))
    for a, c in zip(res[0], res[1]):
        assert gh.bits_equal(a, c)
    dx, dw1, dw2 = (gh.to_f64(t) for t in res[0])
    if acc:
        dw1 = dw1 - 0.25
        dw2 = dw2 + 0.5
    assert gh.normwise(dx, dx_ref) <= gh.TOL_BF16_GRAD
    for e in range(E):
        if counts[e] == 0:
            assert np.abs(dw1[e]).max() <= (1e-6 if acc else 0.0)
            assert np.abs(dw2[e]).max() <= (1e-6 if acc else 0.0)
            continue
        assert gh.normwise(dw1[e], dw1_ref[e]) <= gh.TOL_BF16_GRAD, e
        assert gh.normwise(dw2[e], dw2_ref[e]) <= gh.TOL_BF16_GRAD, e


@pytest.mark.parametrize("acc", [False, True])
def test_grouped_no_rows(acc):
    """N = 0 (every expert empty, e.g. an expert-parallel rank that receives
    no tokens): the forward computes nothing, the backward writes dW = 0, or
    leaves dW as it was when accumulating."""
    E, d, F = 3, 64, 64
    inp = mw.make_small_layer_inputs(77, T=1, d=d, E=E, F=F, dtype="bf16", w_std=0.05)
    w1, w2 = gh.to_gpu(inp.w1), gh.to_gpu(inp.w2)
    off = gh.to_gpu(np.zeros(E + 1, dtype=np.int32))
    x = torch.empty((0, d), dtype=torch.bfloat16, device=gh.dev())
    y, _ = moe.grouped_swiglu_fwd(x, w1, w2, off)
    torch.cuda.synchronize()
    assert y.shape == (0, d)
    base = 0.75 if acc else float("nan")
    dw1 = torch.full((E, 2 * F, d), base, dtype=torch.float32, device=gh.dev())
    dw2 = torch.full((E, d, F), base, dtype=torch.float32, device=gh.dev())
    dx = torch.empty((0, d), dtype=torch.bfloat16, device=gh.dev())
    moe.grouped_swiglu_bwd(x, x, w1, w2, off, None, None, acc, dw1, dw2, dx_out=dx)
    torch.cuda.synchronize()
    want = 0.75 if acc else 0.0
    assert torch.all(dw1 == want).item() and torch.all(dw2 == want).item()


COMB_CASES = [(1, 64, 1, "bf16", False), (300, 136, 6, "bf16", True),
              (257, 128, 2, "f32", True), (100, 64, 8, "bf16", False)]


@pytest.mark.parametrize("case", COMB_CASES, ids=lambda c: "-".join(map(str, c)))
def test_combine_parity(case):
    T, d, k, dt, shared = case
    rng = np.random.default_rng(T + d + k)
    N = T * k
    ypf = rng.standard_normal((N, d)).astype(np.float32)
    yp = ypf if dt == "f32" else mw.round_to_bf16_bits(ypf)
    slot = rng.permutation(N).reshape(T, k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    ysh = None
    if shared:
        s = rng.standard_normal((T, d)).astype(np.float32)
        ysh = s if dt == "f32" else mw.round_to_bf16_bits(s)
    as32 = (lambda a: a) if dt == "f32" else mw.bf16_bits_to_f32
    ref = mo.unpermute_combine(as32(yp), slot, w, None if ysh is None else as32(ysh))
    g = [moe.unpermute_combine(gh.to_gpu(yp), gh.to_gpu(slot), gh.to_gpu(w),
                               None if ysh is None else gh.to_gpu(ysh)) for _ in range(2)]
    torch.cuda.synchronize()
    assert gh.bits_equal(g[0], g[1])
    tol = gh.TOL_F32 if dt == "f32" else gh.TOL_BF16
    assert gh.normwise(gh.to_f64(g[0]), ref) <= tol
