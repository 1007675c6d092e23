"""Plain CPU oracle of the MoE layer's hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the entry
module and the benchmark's ``cpu_baseline`` leg may import or run this file.
It shares no code with the HIP library and imports nothing from it.

What it computes, step by step, with the passage each step follows:

* routing -- a router turns each token into top-k expert choices with
  scores ("Megatron-Bridge 深度剖析", section "MoE 加速深度剖析 / Expert
  Parallel 基础", step-1 diagram "Router 决策": the router emits TopK scores,
  e.g. top-6 sigmoid);  the score function is softmax or sigmoid (same page,
  "Megatron-Core 架构速览": TransformerConfig's moe_router_score_function);
* permutation -- tokens regrouped so that each expert's tokens are contiguous
  (same section, step-2 "after dispatch the GPU holds tokens grouped by
  expert", and section "计算融合 / Grouped GEMM": one call over segments
  [E0: 20 tok, E1: 5 tok, ...]);
* expert FFN -- SwiGLU with gate_proj, up_proj, down_proj ("Motivation":
  3 x ffn x hidden parameters per expert); fc1 is the concatenation
  [gate; up] of shape (2*ffn, hidden) (section "权重映射策略",
  GatedMLPMapping);
* combine -- expert results return to token order (step-3 diagram) and
  are summed with the routing weights;
* shared expert -- every token passes through it ("Shared Expert Overlap";
  "核心模块架构": shared_experts is optional), scaled by a per-token gate
  (TorchSpec pull request "Add Megatron-Core MTP training for Qwen3.5 MoE",
  "What's in it": the ported layer has a gate on its shared expert);
* backward -- the grouped GEMM's dgrad and wgrad ("通信隐藏与混合精度 / TP
  通信重叠" names the backward's dgrad/wgrad GEMMs); the rest of the layer's
  backward runs through the router softmax and the dispatch permute, the
  operations the backward recomputes ("Activation Recomputation": selective
  recompute of the router softmax and the dispatch permute in MoE layers):
  combine backward, permute backward, router backward (chain rule of the
  forward's definition).

Readings where the pages are silent (each listed in the design notes):
  * routing weights are renormalised over the selected k (softmax over all
    experts, then divided by the selected sum);
  * the top-k order is score descending, equal scores -> lower expert index;
  * the ranking decision is taken on fp32 scores (the kernel's precision);
  * rows inside an expert segment keep ascending token order;
  * SwiGLU is silu(gate) * up with silu(z) = z * sigmoid(z), gate rows first;
  * the down projection W2[e] is stored (hidden, ffn), y = a @ W2[e].T;
  * shared-expert output is added after the routed sum, scaled by
    sigmoid(x . w_gate), not included in the routed normalisation;
  * no token is dropped or padded.

Floating point: every value is computed in float64 (``prec=np.float64``,
the default).  ``prec=np.float32`` runs the same steps in float32 and is
used only to bound the oracle's own rounding.  The routing decision always
uses float32 scores, matching the precision the kernel ranks in.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "logits", "scores", "route", "route_weights_for", "permute",
    "silu", "silu_grad", "swiglu_ffn", "grouped_swiglu_fwd",
    "grouped_swiglu_bwd", "unpermute_combine", "shared_expert",
    "moe_layer_forward", "RouteResult", "PermuteResult",
    "combine_backward", "permute_backward", "route_backward", "moe_layer_backward",
]


def _as(a, prec):
    return None if a is None else np.asarray(a).astype(prec, copy=False)


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------
def logits(x, w_router, logit_bias=None, prec=np.float64):
    """z[t, e] = sum_i x[t, i] * W_r[e, i]  (+ b_e)."""
    z = _as(x, prec) @ _as(w_router, prec).T
    if logit_bias is not None:
        z = z + _as(logit_bias, prec)[None, :]
    return z


def scores(z, score_fn):
    """softmax over the experts of each token (max-subtracted), or the
    element-wise logistic sigmoid."""
    if score_fn == "softmax":
        m = z.max(axis=1, keepdims=True)
        ez = np.exp(z - m)
        return ez / ez.sum(axis=1, keepdims=True)
    if score_fn == "sigmoid":
        with np.errstate(over="ignore"):
            return 1.0 / (1.0 + np.exp(-z))
    raise ValueError(score_fn)


class RouteResult:
    """Result of :func:`route`.

    topk_idx   [T, k] int32  experts by descending fp32 score (tie: lower idx)
    topk_w     [T, k]        routing weights (prec)
    counts     [E] int32     tokens per expert
    gate       [T] or None   sigmoid shared-expert gate
    s32        [T, E] fp32   the keys the decision was taken on (the fp32
                             scores, plus the selection bias when given)
    margin     [T]           s_(k) - s_(k+1) in those fp32 scores (+inf if k=E)
    logit_margin [T]         z_(k) - z_(k+1) by the same order (+inf if k=E)
    """

    def __init__(self, **kw):
        self.__dict__.update(kw)

    def excluded(self, threshold=1e-5):
        return self.margin < threshold


def route(x, w_router, k, score_fn="softmax", normalize=True,
          logit_bias=None, w_gate=None, prec=np.float64, selection_bias=None):
    """Router -> score -> top-k -> weight normalisation (+ shared gate).

    ``selection_bias`` is the DeepSeek-style expert-bias correction named by
    the pages' MoE config listings (moe_router_enable_expert_bias): it
    shifts only the choice -- experts are ranked by the fp32 sum s + b --
    while the weights come from the unbiased scores."""
    z = logits(x, w_router, logit_bias, prec)
    s = scores(z, score_fn)
    T, E = s.shape
    if not 1 <= k <= E:
        raise ValueError("k must be in [1, E]")
    s32 = s.astype(np.float32)
    if selection_bias is not None:
        # the ranking key, added in fp32 like the decision itself
        s32 = (s32 + np.asarray(selection_bias, dtype=np.float32)[None, :]).astype(np.float32)
    # descending fp32 key; a stable sort keeps the lower expert index first
    # among equal keys
    order = np.argsort(-s32, axis=1, kind="stable")
    topk_idx = order[:, :k].astype(np.int32)
    rows = np.arange(T)[:, None]
    sel = s[rows, topk_idx]
    if normalize:
        w = sel / sel.sum(axis=1, keepdims=True)
    else:
        w = sel
    if k < E:
        nxt = order[:, k]
        kth = order[:, k - 1]
        margin = (s32[np.arange(T), kth].astype(np.float64)
                  - s32[np.arange(T), nxt].astype(np.float64))
        with np.errstate(invalid="ignore"):   # two masked (-inf) logits: NaN margin
            logit_margin = (z[np.arange(T), kth] - z[np.arange(T), nxt]).astype(np.float64)
    else:
        margin = np.full(T, np.inf)
        logit_margin = np.full(T, np.inf)
    counts = np.bincount(topk_idx.reshape(-1), minlength=E).astype(np.int32)
    gate = None
    if w_gate is not None:
        g = _as(x, prec) @ _as(w_gate, prec)
        with np.errstate(over="ignore"):
            gate = 1.0 / (1.0 + np.exp(-g))
    return RouteResult(topk_idx=topk_idx, topk_w=w, counts=counts, gate=gate,
                       s32=s32, margin=margin, logit_margin=logit_margin,
                       z=z, s=s)


def route_weights_for(x, w_router, topk_idx, score_fn="softmax",
                      normalize=True, logit_bias=None, prec=np.float64):
    """The oracle's weights for a *given* choice of experts (used to compare
    layer outputs when a near-tie token picked a different, equally legal
    expert set)."""
    s = scores(logits(x, w_router, logit_bias, prec), score_fn)
    sel = s[np.arange(s.shape[0])[:, None], topk_idx]
    return sel / sel.sum(axis=1, keepdims=True) if normalize else sel


# --------------------------------------------------------------------------
# Permutation
# --------------------------------------------------------------------------
class PermuteResult:
    """offsets [E+1], slot_of [T, k], row_token [N], row_w [N], x_perm [N, d]"""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def permute(x, topk_idx, topk_w, E):
    """Counting-sort the (token, slot) pairs by expert.

    Slots are enumerated token-major (s = t*k + j); a stable sort by expert
    gives rows ordered by (expert, token, slot).  Row r of the permuted
    matrix is the token ``row_token[r]``; ``slot_of[t, j]`` is the row that
    holds token t's j-th choice.
    """
    T, k = topk_idx.shape
    expert_of_slot = np.asarray(topk_idx).reshape(-1)
    order = np.argsort(expert_of_slot, kind="stable")
    counts = np.bincount(expert_of_slot, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    slot_of = np.empty(T * k, dtype=np.int64)
    slot_of[order] = np.arange(T * k)
    row_token = order // k
    row_w = None if topk_w is None else np.asarray(topk_w).reshape(-1)[order]
    x_perm = None if x is None else np.asarray(x)[row_token]
    return PermuteResult(offsets=offsets.astype(np.int32),
                         slot_of=slot_of.reshape(T, k).astype(np.int32),
                         row_token=row_token.astype(np.int32),
                         row_w=row_w, x_perm=x_perm,
                         counts=counts.astype(np.int32))


# --------------------------------------------------------------------------
# Expert FFN (SwiGLU), grouped over expert segments
# --------------------------------------------------------------------------
def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def silu_grad(z):
    """d/dz [z * sigmoid(z)] = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def swiglu_ffn(x, w1, w2, prec=np.float64):
    """One SwiGLU expert: g = x W1[:F]^T, u = x W1[F:]^T, a = silu(g) * u,
    y = a W2^T.  Returns (y, g, u, a)."""
    x = _as(x, prec)
    w1 = _as(w1, prec)
    w2 = _as(w2, prec)
    F = w1.shape[0] // 2
    g = x @ w1[:F].T
    u = x @ w1[F:].T
    a = silu(g) * u
    return a @ w2.T, g, u, a


def grouped_swiglu_fwd(x_perm, w1, w2, offsets, row_scale=None,
                       prec=np.float64, return_gu=False):
    """Y[R_e] = SwiGLU_e(X[R_e]) (* row_scale[R_e]) for each segment R_e."""
    x_perm = _as(x_perm, prec)
    E = w1.shape[0]
    N, d = x_perm.shape
    F = w1.shape[1] // 2
    y = np.zeros((N, w2.shape[1]), dtype=prec)
    gu = np.zeros((N, 2 * F), dtype=prec) if return_gu else None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        ye, g, u, _ = swiglu_ffn(x_perm[lo:hi], w1[e], w2[e], prec)
        if row_scale is not None:
            ye = ye * _as(row_scale, prec)[lo:hi, None]
        y[lo:hi] = ye
        if return_gu:
            gu[lo:hi, :F] = g
            gu[lo:hi, F:] = u
    return (y, gu) if return_gu else y


def grouped_swiglu_bwd(dy_perm, x_perm, w1, w2, offsets, row_scale=None,
                       prec=np.float64):
    """Gradients of L = sum(dY * Y) for Y from :func:`grouped_swiglu_fwd`.

    Per expert e with rows R_e:
      dYs = dY * row_scale;  dA = dYs W2[e];  dW2[e] = dYs^T A
      dG = dA * U * silu'(G);  dU = dA * silu(G);  dH = [dG | dU]
      dX = dH W1[e];  dW1[e] = dH^T X
    An expert with no rows gets zero weight gradients.
    """
    x_perm = _as(x_perm, prec)
    dy_perm = _as(dy_perm, prec)
    E = w1.shape[0]
    N, d = x_perm.shape
    F = w1.shape[1] // 2
    dx = np.zeros((N, d), dtype=prec)
    dw1 = np.zeros((E, 2 * F, d), dtype=prec)
    dw2 = np.zeros((E, d, F), dtype=prec)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        X = x_perm[lo:hi]
        W1 = _as(w1[e], prec)
        W2 = _as(w2[e], prec)
        dY = dy_perm[lo:hi]
        if row_scale is not None:
            dY = dY * _as(row_scale, prec)[lo:hi, None]
        G = X @ W1[:F].T
        U = X @ W1[F:].T
        A = silu(G) * U
        dA = dY @ W2
        dw2[e] = dY.T @ A
        dG = dA * U * silu_grad(G)
        dU = dA * silu(G)
        dH = np.concatenate([dG, dU], axis=1)
        dx[lo:hi] = dH @ W1
        dw1[e] = dH.T @ X
    return dx, dw1, dw2


# --------------------------------------------------------------------------
# Combine and shared expert
# --------------------------------------------------------------------------
def unpermute_combine(y_perm, slot_of, topk_w=None, y_shared=None,
                      prec=np.float64):
    """y[t] = sum_j w[t, j] * Y[slot_of[t, j]]  (+ y_shared[t]).

    With ``topk_w=None`` the rows are taken as already weighted."""
    y_perm = _as(y_perm, prec)
    T, k = slot_of.shape
    y = np.zeros((T, y_perm.shape[1]), dtype=prec)
    for j in range(k):
        rows = y_perm[slot_of[:, j]]
        if topk_w is not None:
            rows = rows * _as(topk_w, prec)[:, j:j + 1]
        y += rows
    if y_shared is not None:
        y += _as(y_shared, prec)
    return y


def shared_expert(x, ws1, ws2, gate, prec=np.float64):
    """gate[t] * SwiGLU_shared(x[t])."""
    y, _, _, _ = swiglu_ffn(x, ws1, ws2, prec)
    return y * _as(gate, prec)[:, None]


def moe_layer_forward(x, w_router, w1, w2, k, score_fn="softmax",
                      normalize=True, logit_bias=None, w_gate=None,
                      ws1=None, ws2=None, prec=np.float64, topk_idx=None,
                      selection_bias=None):
    """The whole layer: route -> permute -> grouped SwiGLU -> combine
    (+ gated shared expert).  ``topk_idx`` forces a given expert choice
    (the weights are then the oracle's own for that choice)."""
    E = w_router.shape[0]
    r = route(x, w_router, k, score_fn, normalize, logit_bias, w_gate, prec, selection_bias)
    idx = r.topk_idx if topk_idx is None else np.asarray(topk_idx)
    w = r.topk_w if topk_idx is None else route_weights_for(
        x, w_router, idx, score_fn, normalize, logit_bias, prec)
    p = permute(x, idx, w, E)
    y_perm = grouped_swiglu_fwd(p.x_perm, w1, w2, p.offsets, None, prec)
    y_sh = None
    if ws1 is not None:
        y_sh = shared_expert(x, ws1, ws2, r.gate, prec)
    y = unpermute_combine(y_perm, p.slot_of, w, y_sh, prec)
    return y, r, p


# --------------------------------------------------------------------------
# Full-layer backward: the chain rule of the forward above, for a fixed
# expert selection (the selection itself is piecewise constant).
# --------------------------------------------------------------------------
def combine_backward(dy, y_perm, slot_of, topk_w, y_shared=None, gate=None,
                     prec=np.float64):
    """Gradients of L = sum(dy * y) for
         y[t] = sum_j w[t, j] Y[slot_of[t, j]] + gate[t] Ysh[t]
    (Y and Ysh unweighted):
         dY[slot_of[t, j]] = w[t, j] dy[t]
         dw[t, j]          = <dy[t], Y[slot_of[t, j]]>
         dgate[t]          = <dy[t], Ysh[t]>
    A slot of -1 (a dropped choice) contributes nothing and gets dw = 0.
    Returns (dY [N, d], dw [T, k], dgate [T] or None)."""
    dy = _as(dy, prec)
    y_perm = _as(y_perm, prec)
    w = _as(topk_w, prec)
    T, k = slot_of.shape
    dY = np.zeros_like(y_perm)
    dw = np.zeros((T, k), dtype=prec)
    for j in range(k):
        ok = slot_of[:, j] >= 0
        rows = slot_of[ok, j]
        dY[rows] = w[ok, j:j + 1] * dy[ok]
        dw[ok, j] = np.einsum("td,td->t", dy[ok], y_perm[rows])
    dgate = None
    if y_shared is not None and gate is not None:
        dgate = np.einsum("td,td->t", dy, _as(y_shared, prec))
    return dY, dw, dgate


def permute_backward(dx_perm, slot_of, prec=np.float64):
    """dx[t] = sum_j dX[slot_of[t, j]]: each row of x went to k rows."""
    dx_perm = _as(dx_perm, prec)
    T, k = slot_of.shape
    dx = np.zeros((T, dx_perm.shape[1]), dtype=prec)
    for j in range(k):
        ok = slot_of[:, j] >= 0
        dx[ok] += dx_perm[slot_of[ok, j]]
    return dx


def route_backward(x, w_router, topk_idx, d_topk_w, score_fn="softmax",
                   normalize=True, logit_bias=None, w_gate=None, d_gate=None,
                   prec=np.float64):
    """Back through the routing weights of the selection topk_idx to the
    logits, then to x and the router weights (the bias is a constant).

      s = score(z)                  softmax over E, or sigmoid
      w[t, j] = s[t, e_j] / S_t     S_t = sum_j s[t, e_j]   (normalize)
              = s[t, e_j]                                   (otherwise)
      ds[t, e_i] = (dw[t, i] - sum_j dw[t, j] w[t, j]) / S_t   (normalize)
                 = dw[t, i]                                    (otherwise)
      dz = s * (ds - <ds, s>)  (softmax)   or   ds * s * (1 - s)  (sigmoid)
      dW_r = dz^T x,   dx = dz W_r
    Shared gate g = sigmoid(x . w_gate): dgl = d_gate * g (1 - g),
      dw_gate = dgl^T x,  dx += dgl w_gate.
    Returns (dx [T, d], dw_router [E, d], dz [T, E], dw_gate [d] or None)."""
    x = _as(x, prec)
    wr = _as(w_router, prec)
    z = logits(x, w_router, logit_bias, prec)
    s = scores(z, score_fn)
    T, E = s.shape
    rows = np.arange(T)[:, None]
    idx = np.asarray(topk_idx)
    dw = _as(d_topk_w, prec)
    sel = s[rows, idx]
    ds = np.zeros((T, E), dtype=prec)
    if normalize:
        S = sel.sum(axis=1, keepdims=True)
        w = sel / S
        ds_sel = (dw - (dw * w).sum(axis=1, keepdims=True)) / S
    else:
        ds_sel = dw
    ds[rows, idx] = ds_sel
    if score_fn == "softmax":
        dz = s * (ds - (ds * s).sum(axis=1, keepdims=True))
    elif score_fn == "sigmoid":
        dz = ds * s * (1.0 - s)
    else:
        raise ValueError(score_fn)
    dx = dz @ wr
    dw_router = dz.T @ x
    dw_gate = None
    if w_gate is not None and d_gate is not None:
        g = x @ _as(w_gate, prec)
        with np.errstate(over="ignore"):
            gs = 1.0 / (1.0 + np.exp(-g))
        dgl = _as(d_gate, prec) * gs * (1.0 - gs)
        dw_gate = dgl @ x
        dx = dx + dgl[:, None] * _as(w_gate, prec)[None, :]
    return dx, dw_router, dz, dw_gate


def moe_layer_backward(x, w_router, w1, w2, k, dy, score_fn="softmax",
                       normalize=True, logit_bias=None, w_gate=None, ws1=None,
                       ws2=None, prec=np.float64, topk_idx=None):
    """Gradients of L = sum(dy * y) for y from :func:`moe_layer_forward`
    with the selection held fixed (``topk_idx``, or the oracle's own):
    combine backward -> grouped-GEMM backward (and the shared expert's, row
    scale = gate) -> permute backward -> router backward.  Returns a dict
    with dx, dw_router, dw1, dw2 (and dws1, dws2, dw_gate with a shared
    expert) plus the intermediates d_topk_w, d_gate, dz, dx_perm."""
    E = w_router.shape[0]
    T = x.shape[0]
    r = route(x, w_router, k, score_fn, normalize, logit_bias, w_gate, prec)
    idx = r.topk_idx if topk_idx is None else np.asarray(topk_idx)
    w = r.topk_w if topk_idx is None else route_weights_for(
        x, w_router, idx, score_fn, normalize, logit_bias, prec)
    p = permute(x, idx, w, E)
    y_perm = grouped_swiglu_fwd(p.x_perm, w1, w2, p.offsets, None, prec)
    ysh = swiglu_ffn(x, ws1, ws2, prec)[0] if ws1 is not None else None
    dY, dw, dgate = combine_backward(dy, y_perm, p.slot_of, w, ysh, r.gate, prec)
    dx_perm, dw1, dw2 = grouped_swiglu_bwd(dY, p.x_perm, w1, w2, p.offsets, None, prec)
    dx = permute_backward(dx_perm, p.slot_of, prec)
    dxr, dw_router, dz, dw_gate = route_backward(x, w_router, idx, dw, score_fn, normalize,
                                                 logit_bias, w_gate, dgate, prec)
    out = dict(dx_perm=dx_perm, d_topk_w=dw, d_gate=dgate, dz=dz, dw1=dw1, dw2=dw2,
               dw_router=dw_router, topk_idx=idx, topk_w=w, offsets=p.offsets,
               slot_of=p.slot_of, row_token=p.row_token)
    dx = dx + dxr
    if ws1 is not None:
        off = np.array([0, T])
        dxs, dws1, dws2 = grouped_swiglu_bwd(dy, x, _as(ws1, prec)[None], _as(ws2, prec)[None],
                                             off, r.gate, prec)
        dx = dx + dxs
        out.update(dws1=dws1[0], dws2=dws2[0], dw_gate=dw_gate)
    out["dx"] = dx
    return out
