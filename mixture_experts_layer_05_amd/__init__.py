"""MI355X (gfx950) MoE-layer hot path: Python binding of libmoe_mi355x.so.

The binding only marshals arguments: it turns torch tensors that live on
the GPU into device pointers, passes torch's current HIP stream, allocates
outputs and workspaces with torch, and raises on a non-zero status.  Every
step of the layer runs in the library's HIP kernels; there is no fallback.

Calls (same names and semantics as include/moe.h):
    route, permute, grouped_swiglu_fwd, grouped_swiglu_bwd, unpermute_combine
plus ``moe_layer_forward`` that chains them, and ``MoELayer`` that keeps its
buffers between calls (no allocation per forward).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "MoEError", "lib", "route", "permute", "permute_noalloc", "grouped_swiglu_fwd", "grouped_swiglu_fwd_gather",
    "PackedWeights", "pack_weights", "grouped_swiglu_fwd_packed",
    "MxTensor", "quantize_mx", "pack_weights_mx", "grouped_swiglu_fwd_mx",
    "grouped_swiglu_bwd", "unpermute_combine", "combine_backward", "route_backward",
    "moe_layer_forward",
    "MoELayer", "LIB_PATH", "EXPORTED",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_F32, MOE_BF16 = 0, 1
SCORE = {"softmax": 0, "sigmoid": 1}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

# name -> (restype, argtypes); the public symbols of include/moe.h
EXPORTED = {
    "moe_abi_version": (_i32, []),
    "moe_status_string": (ctypes.c_char_p, [_i32]),
    "moe_route_workspace_size": (_sz, [_i64, _i64, _i32, _i32]),
    "moe_route": (_i32, [_vp, _i32, _i64, _i64, _i32, _i32, _i32, _i32,
                         _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz]),
    "moe_permute_workspace_size": (_sz, [_i64, _i32, _i32]),
    "moe_permute_noalloc": (_i32, [_vp, _i32, _i64, _i64, _i32, _i32, _vp, _vp, _vp,
                                   _vp, _vp, _vp, _vp, _vp]),
    "moe_permute": (_i32, [_vp, _i32, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp,
                           _vp, _vp, _vp, _vp, _vp, _vp, _sz]),
    "moe_grouped_swiglu_fwd_workspace_size": (_sz, [_i64, _i64, _i32]),
    "moe_grouped_swiglu_fwd": (_i32, [_vp, _i32, _i64, _i64, _i64, _i32,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz]),
    "moe_grouped_swiglu_fwd_gather": (_i32, [_vp, _i32, _i64, _i64, _i64, _i32, _i64,
                                             _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz]),
    "moe_pack_weights_size": (_sz, [_i32, _i64, _i64, _i32]),
    "moe_pack_weights": (_i32, [_vp, _i32, _i32, _i64, _i64, _i32, _vp, _vp]),
    "moe_grouped_swiglu_fwd_packed": (_i32, [_vp, _i32, _i64, _i64, _i64, _i32, _i64,
                                             _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz]),
    "moe_quantize_mx_scales_size": (_sz, [_i64, _i64]),
    "moe_quantize_mx": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "moe_pack_weights_mx_size": (_sz, [_i32, _i64, _i64, _i32, _i32]),
    "moe_pack_weights_mx": (_i32, [_vp, _i32, _i64, _i64, _i32, _vp, _vp, _vp]),
    "moe_grouped_swiglu_fwd_mx_workspace_size": (_sz, [_i64, _i64]),
    "moe_grouped_swiglu_fwd_mx": (_i32, [_vp, _i64, _i64, _i64, _i32, _i64, _vp, _vp, _vp,
                                         _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz]),
    "moe_grouped_swiglu_bwd_workspace_size": (_sz, [_i64, _i64, _i32, _i32]),
    "moe_grouped_swiglu_bwd": (_i32, [_vp, _i32, _i64, _i64, _i64, _i32,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                      _vp, _vp, _vp, _vp, _sz]),
    "moe_unpermute_combine": (_i32, [_vp, _i32, _i64, _i64, _i32, _i64,
                                     _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_combine_backward": (_i32, [_vp, _i32, _i64, _i64, _i32, _i64,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_route_backward_workspace_size": (_sz, [_i64, _i64, _i32, _i32, _i32, _i32, _i32]),
    "moe_route_backward": (_i32, [_vp, _i32, _i64, _i64, _i32, _i32, _i32, _i32,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz]),
}


class MoEError(RuntimeError):
    pass


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise MoEError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mixture_experts_layer_05_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTED.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int, what: str):
    if status != 0:
        name = lib().moe_status_string(status).decode()
        raise MoEError(f"{what} failed: {name} ({status})")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise MoEError(f"unsupported dtype {t.dtype}")


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise MoEError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise MoEError("tensor must be contiguous")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
def route_workspace_size(T, d, E, dtype):
    return lib().moe_route_workspace_size(T, d, E, MOE_BF16 if dtype == torch.bfloat16 else MOE_F32)


ROUTE_BLOCK_TOKENS = 64   # MOE_ROUTE_BLOCK_TOKENS


def route_block_counts(T, E, device):
    """An int32 buffer for route()'s per-64-token-block expert histograms."""
    return torch.empty(((T + ROUTE_BLOCK_TOKENS - 1) // ROUTE_BLOCK_TOKENS, E), dtype=torch.int32,
                       device=device)


def route(x, w_router, k, score="softmax", normalize=True, logit_bias=None,
          w_gate=None, out=None, ws=None, selection_bias=None, block_counts=None):
    """-> (topk_idx [T,k] int32, topk_w [T,k] fp32, counts [E] int32 (None when `out`
    holds None there: not computed), gate [T] or None).
    block_counts (route_block_counts(T, E)): also filled with the block
    histograms that permute(block_counts=...) takes."""
    T, d = x.shape
    E = w_router.shape[0]
    dev = x.device
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((E,), dtype=torch.int32, device=dev),
               torch.empty((T,), dtype=torch.float32, device=dev) if w_gate is not None else None)
    idx, w, cnt, gate = out
    if ws is None:
        ws = _ws(route_workspace_size(T, d, E, x.dtype), dev)
    _check(lib().moe_route(_stream(), _dt(x), T, d, E, k, SCORE[score], int(bool(normalize)),
                           _p(x), _p(w_router), _p(logit_bias), _p(selection_bias), _p(w_gate),
                           _p(idx), _p(w), _p(cnt), _p(block_counts), _p(gate), _p(ws), ws.numel()),
           "moe_route")
    return idx, w, cnt, gate


def permute_workspace_size(T, E, k):
    return lib().moe_permute_workspace_size(T, E, k)


def permute(x, topk_idx, topk_w, E, out=None, ws=None, copy_rows=True, block_counts=None):
    """-> (expert_offsets [E+1], slot_of [T,k], row_token [N], row_w [N] or None,
    x_perm [N,d] or None).  copy_rows=False skips the row copy (for a consumer
    that gathers rows by row_token); block_counts: route()'s block histograms
    of this topk_idx (skips the counting pass)."""
    T, d = x.shape
    k = topk_idx.shape[1]
    N = T * k
    dev = x.device
    if out is None:
        out = (torch.empty((E + 1,), dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.int32, device=dev),
               torch.empty((N,), dtype=torch.int32, device=dev),
               torch.empty((N,), dtype=torch.float32, device=dev) if topk_w is not None else None,
               torch.empty((N, d), dtype=x.dtype, device=dev) if copy_rows else None)
    off, slot, rtok, rw, xp = out
    nbytes = permute_workspace_size(T, E, k)
    if ws is None:
        ws = _ws(nbytes, dev)
    if not copy_rows:
        xp = None
    _check(lib().moe_permute(_stream(), _dt(x), T, d, E, k, _p(x), _p(topk_idx), _p(topk_w),
                             _p(block_counts), _p(off), _p(slot), _p(rtok), _p(rw), _p(xp),
                             _p(ws), ws.numel()),
           "moe_permute")
    return off, slot, rtok, rw, xp


def permute_noalloc(x, topk_idx, topk_w, E, out=None, copy_rows=True):
    """moe_permute_noalloc: permute() with the library's static scratch
    instead of a workspace (for callers that cannot allocate around the call;
    calls overlapping on one GPU race)."""
    T, d = x.shape
    k = topk_idx.shape[1]
    N = T * k
    dev = x.device
    if out is None:
        out = (torch.empty((E + 1,), dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.int32, device=dev),
               torch.empty((N,), dtype=torch.int32, device=dev),
               torch.empty((N,), dtype=torch.float32, device=dev) if topk_w is not None else None,
               torch.empty((N, d), dtype=x.dtype, device=dev) if copy_rows else None)
    off, slot, rtok, rw, xp = out
    if not copy_rows:
        xp = None
    _check(lib().moe_permute_noalloc(_stream(), _dt(x), T, d, E, k, _p(x), _p(topk_idx),
                                     _p(topk_w), _p(off), _p(slot), _p(rtok), _p(rw), _p(xp)),
           "moe_permute_noalloc")
    return off, slot, rtok, rw, xp


def fwd_workspace_size(N, F, dtype):
    return lib().moe_grouped_swiglu_fwd_workspace_size(N, F, MOE_BF16 if dtype == torch.bfloat16 else MOE_F32)


def grouped_swiglu_fwd(x_perm, w1, w2, expert_offsets, row_scale=None, save_gu=False,
                       out=None, gu_out=None, ws=None):
    """-> (y_perm [N,d], gu_save [N,2F] or None)"""
    N, d = x_perm.shape
    E, twoF, _ = w1.shape
    F = twoF // 2
    dev = x_perm.device
    y = out if out is not None else torch.empty((N, d), dtype=x_perm.dtype, device=dev)
    gu = gu_out
    if save_gu and gu is None:
        gu = torch.empty((N, 2 * F), dtype=x_perm.dtype, device=dev)
    nbytes = fwd_workspace_size(N, F, x_perm.dtype)
    if ws is None:
        ws = _ws(nbytes, dev)
    _check(lib().moe_grouped_swiglu_fwd(_stream(), _dt(x_perm), N, d, F, E, _p(x_perm), _p(w1),
                                        _p(w2), _p(expert_offsets), _p(row_scale), _p(y), _p(gu),
                                        _p(ws), ws.numel()), "moe_grouped_swiglu_fwd")
    return y, gu


def grouped_swiglu_fwd_gather(x, row_token, w1, w2, expert_offsets, row_scale=None,
                              save_gu=False, out=None, gu_out=None, ws=None):
    """grouped_swiglu_fwd on x[row_token] without materialising it.
    -> (y_perm [N,d], gu_save [N,2F] or None)"""
    T, d = x.shape
    N = row_token.shape[0]
    E, twoF, _ = w1.shape
    F = twoF // 2
    dev = x.device
    y = out if out is not None else torch.empty((N, d), dtype=x.dtype, device=dev)
    gu = gu_out
    if save_gu and gu is None:
        gu = torch.empty((N, 2 * F), dtype=x.dtype, device=dev)
    nbytes = fwd_workspace_size(N, F, x.dtype)
    if ws is None:
        ws = _ws(nbytes, dev)
    _check(lib().moe_grouped_swiglu_fwd_gather(_stream(), _dt(x), N, d, F, E, T, _p(x),
                                               _p(row_token), _p(w1), _p(w2), _p(expert_offsets),
                                               _p(row_scale), _p(y), _p(gu), _p(ws), ws.numel()),
           "moe_grouped_swiglu_fwd_gather")
    return y, gu


class PackedWeights:
    """Expert weights [E, rows, K] in the tile-packed layout of moe_pack_weights
    (a flat bf16 device buffer plus the logical shape)."""

    def __init__(self, buf, E, rows, K, gated):
        self.buf, self.E, self.rows, self.K, self.gated = buf, E, rows, K, bool(gated)


def pack_weights(w, gated, out=None):
    """w [E, rows, K] bf16 -> PackedWeights (gated: the fc1 [gate; up] layout)."""
    E, rows, K = w.shape
    nbytes = lib().moe_pack_weights_size(E, rows, K, int(bool(gated)))
    if nbytes == 0:
        raise MoEError(f"cannot pack weights of shape {tuple(w.shape)} (gated={gated})")
    buf = out if out is not None else torch.empty(nbytes // 2, dtype=torch.bfloat16, device=w.device)
    if buf.numel() * buf.element_size() < nbytes:
        raise MoEError("packed-weight buffer too small")
    _check(lib().moe_pack_weights(_stream(), _dt(w), E, rows, K, int(bool(gated)), _p(w), _p(buf)),
           "moe_pack_weights")
    return PackedWeights(buf, E, rows, K, gated)


def grouped_swiglu_fwd_packed(x, row_token, w1p, w2p, expert_offsets, row_scale=None,
                              save_gu=False, out=None, gu_out=None, ws=None):
    """grouped_swiglu_fwd (row_token None: x is x_perm [N, d]) or
    grouped_swiglu_fwd_gather (x [T, d], N = len(row_token)) on packed weights
    (pack_weights(w1, True), pack_weights(w2, False)).
    -> (y_perm [N,d], gu_save [N,2F] or None)"""
    T, d = x.shape
    N = row_token.shape[0] if row_token is not None else T
    E, F = w1p.E, w1p.rows // 2
    if not (w1p.gated and not w2p.gated and w1p.K == d and w2p.rows == d and w2p.K == F
            and w2p.E == E):
        raise MoEError("packed weights do not match x and each other")
    dev = x.device
    y = out if out is not None else torch.empty((N, d), dtype=x.dtype, device=dev)
    gu = gu_out
    if save_gu and gu is None:
        gu = torch.empty((N, 2 * F), dtype=x.dtype, device=dev)
    nbytes = fwd_workspace_size(N, F, x.dtype)
    if ws is None:
        ws = _ws(nbytes, dev)
    _check(lib().moe_grouped_swiglu_fwd_packed(_stream(), _dt(x), N, d, F, E, T, _p(x),
                                               _p(row_token), _p(w1p.buf), _p(w2p.buf),
                                               _p(expert_offsets), _p(row_scale), _p(y), _p(gu),
                                               _p(ws), ws.numel()),
           "moe_grouped_swiglu_fwd_packed")
    return y, gu


class MxTensor:
    """MX (microscaled FP8 E4M3) data: uint8 codes and uint8 E8M0 scale bytes
    in the layouts of include/moe.h, plus the logical shape."""

    def __init__(self, codes, scales, shape, gated=None):
        self.codes, self.scales, self.shape, self.gated = codes, scales, tuple(shape), gated


def quantize_mx(x, out=None):
    """x [R, K] bf16 -> MxTensor (codes [R, K], scales [ceil(K/512)][R][16])."""
    R, K = x.shape
    if out is None:
        out = MxTensor(torch.empty((R, K), dtype=torch.uint8, device=x.device),
                       torch.empty(lib().moe_quantize_mx_scales_size(R, K), dtype=torch.uint8,
                                   device=x.device), (R, K))
    _check(lib().moe_quantize_mx(_stream(), R, K, _p(x), _p(out.codes), _p(out.scales)),
           "moe_quantize_mx")
    return out


def pack_weights_mx(w, gated):
    """w [E, rows, K] bf16 -> MxTensor in the packed layout (gated: fc1 panels)."""
    E, rows, K = w.shape
    L = lib()
    nc = L.moe_pack_weights_mx_size(E, rows, K, int(bool(gated)), 0)
    ns = L.moe_pack_weights_mx_size(E, rows, K, int(bool(gated)), 1)
    if nc == 0:
        raise MoEError(f"cannot pack weights of shape {tuple(w.shape)} (gated={gated})")
    codes = torch.empty(nc, dtype=torch.uint8, device=w.device)
    scales = torch.empty(ns, dtype=torch.uint8, device=w.device)
    _check(L.moe_pack_weights_mx(_stream(), E, rows, K, int(bool(gated)), _p(w), _p(codes),
                                 _p(scales)), "moe_pack_weights_mx")
    return MxTensor(codes, scales, (E, rows, K), gated)


def fwd_mx_workspace_size(N, F):
    return lib().moe_grouped_swiglu_fwd_mx_workspace_size(N, F)


def grouped_swiglu_fwd_mx(xq, row_token, w1q, w2q, expert_offsets, row_scale=None, out=None,
                          ws=None):
    """MXFP8 grouped SwiGLU forward: xq = quantize_mx(x [T, d]) with row_token
    (fc1 gathers x[row_token[r]]), or quantize_mx(x_perm [N, d]) without;
    w1q = pack_weights_mx(w1, True), w2q = pack_weights_mx(w2, False).
    -> y_perm [N, d] bf16"""
    T, d = xq.shape
    N = row_token.shape[0] if row_token is not None else T
    E, twoF, _ = w1q.shape
    F = twoF // 2
    if not (w1q.gated and not w2q.gated and w1q.shape[2] == d and w2q.shape == (E, d, F)):
        raise MoEError("MX weights do not match x and each other")
    dev = xq.codes.device
    y = out if out is not None else torch.empty((N, d), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = _ws(fwd_mx_workspace_size(N, F), dev)
    _check(lib().moe_grouped_swiglu_fwd_mx(_stream(), N, d, F, E, T, _p(xq.codes), _p(xq.scales),
                                           _p(row_token), _p(w1q.codes), _p(w1q.scales),
                                           _p(w2q.codes), _p(w2q.scales), _p(expert_offsets),
                                           _p(row_scale), _p(y), _p(ws), ws.numel()),
           "moe_grouped_swiglu_fwd_mx")
    return y


def bwd_workspace_size(N, F, dtype, recompute):
    return lib().moe_grouped_swiglu_bwd_workspace_size(
        N, F, MOE_BF16 if dtype == torch.bfloat16 else MOE_F32, int(bool(recompute)))


def grouped_swiglu_bwd(dy_perm, x_perm, w1, w2, expert_offsets, gu_save=None, row_scale=None,
                       accumulate=False, dw1=None, dw2=None, dx_out=None, ws=None):
    """-> (dx_perm [N,d], dw1 [E,2F,d] fp32, dw2 [E,d,F] fp32)"""
    N, d = x_perm.shape
    E, twoF, _ = w1.shape
    F = twoF // 2
    dev = x_perm.device
    dx = dx_out if dx_out is not None else torch.empty((N, d), dtype=x_perm.dtype, device=dev)
    if dw1 is None:
        dw1 = torch.empty((E, 2 * F, d), dtype=torch.float32, device=dev)
    if dw2 is None:
        dw2 = torch.empty((E, d, F), dtype=torch.float32, device=dev)
    nbytes = bwd_workspace_size(N, F, x_perm.dtype, gu_save is None)
    if ws is None:
        ws = _ws(nbytes, dev)
    _check(lib().moe_grouped_swiglu_bwd(_stream(), _dt(x_perm), N, d, F, E, _p(dy_perm),
                                        _p(x_perm), _p(w1), _p(w2), _p(expert_offsets),
                                        _p(gu_save), _p(row_scale), int(bool(accumulate)),
                                        _p(dx), _p(dw1), _p(dw2), _p(ws), ws.numel()),
           "moe_grouped_swiglu_bwd")
    return dx, dw1, dw2


def unpermute_combine(y_perm, slot_of, topk_w=None, y_shared=None, out=None, shared_gate=None):
    """-> y [T, d]"""
    T, k = slot_of.shape
    N, d = y_perm.shape
    y = out if out is not None else torch.empty((T, d), dtype=y_perm.dtype, device=y_perm.device)
    _check(lib().moe_unpermute_combine(_stream(), _dt(y_perm), T, d, k, N, _p(y_perm),
                                       _p(slot_of), _p(topk_w), _p(y_shared), _p(shared_gate),
                                       _p(y)),
           "moe_unpermute_combine")
    return y


def combine_backward(dy, y_perm, slot_of, topk_w, y_shared=None, dy_perm=None, d_topk_w=None,
                     d_gate=None):
    """-> (dy_perm [N,d], d_topk_w [T,k] fp32, d_gate [T] fp32 or None)"""
    T, d = dy.shape
    k = slot_of.shape[1]
    N = y_perm.shape[0]
    dev = dy.device
    if dy_perm is None:
        dy_perm = torch.empty((N, d), dtype=dy.dtype, device=dev)
    if d_topk_w is None:
        d_topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if y_shared is not None and d_gate is None:
        d_gate = torch.empty((T,), dtype=torch.float32, device=dev)
    _check(lib().moe_combine_backward(_stream(), _dt(dy), T, d, k, N, _p(dy), _p(y_perm),
                                      _p(slot_of), _p(topk_w), _p(y_shared), _p(dy_perm),
                                      _p(d_topk_w), _p(d_gate if y_shared is not None else None)),
           "moe_combine_backward")
    return dy_perm, d_topk_w, d_gate if y_shared is not None else None


def route_backward_workspace_size(T, d, E, k, dtype, score="softmax", normalize=True):
    """Workspace bytes of route_backward; dtype is the activations' torch dtype."""
    dt = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}[dtype]
    return lib().moe_route_backward_workspace_size(T, d, E, k, dt, SCORE[score],
                                                   int(bool(normalize)))


def route_backward(x, w_router, topk_idx, topk_w, d_topk_w, expert_offsets, slot_of, row_token,
                   score="softmax", normalize=True, logit_bias=None, w_gate=None, d_gate=None,
                   dx_perm=None, dx_add=None, accumulate=False, dx=None, dw_router=None,
                   dw_gate=None, ws=None):
    """-> (dx [T,d], dw_router [E,d] fp32, dw_gate [d] fp32 or None)"""
    T, d = x.shape
    E = w_router.shape[0]
    k = topk_idx.shape[1]
    dev = x.device
    if dx is None:
        dx = torch.empty((T, d), dtype=x.dtype, device=dev)
    if dw_router is None:
        dw_router = torch.zeros((E, d), dtype=torch.float32, device=dev)
    if w_gate is not None and dw_gate is None:
        dw_gate = torch.zeros((d,), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _ws(route_backward_workspace_size(T, d, E, k, x.dtype, score, normalize), dev)
    _check(lib().moe_route_backward(_stream(), _dt(x), T, d, E, k, SCORE[score], int(bool(normalize)),
                                    _p(x), _p(w_router), _p(logit_bias), _p(w_gate), _p(topk_idx),
                                    _p(topk_w), _p(d_topk_w), _p(d_gate), _p(expert_offsets),
                                    _p(slot_of), _p(row_token), _p(dx_perm), _p(dx_add), _p(dx),
                                    _p(dw_router), _p(dw_gate if w_gate is not None else None),
                                    int(bool(accumulate)), _p(ws), ws.numel()),
           "moe_route_backward")
    return dx, dw_router, dw_gate if w_gate is not None else None


# ---------------------------------------------------------------------------
class MoELayer:
    """The whole forward of one MoE layer with buffers kept between calls.

    route -> permute -> grouped SwiGLU (routing weight applied as the fc2
    row scale) -> [shared expert as a one-expert grouped call, row scale =
    gate] -> combine.  Only kernel launches happen in ``forward``.  With
    ``gather`` (default) the permute makes no row copy and fc1 reads the
    token rows from x by row_token; otherwise x_perm is materialised.

    ``train=True`` keeps what :meth:`backward` needs: x_perm, G and U (of the
    routed and the shared expert), and the expert outputs unweighted (fc2
    without a row scale; combine applies the routing weights and the gate).

    ``packed`` (default: on for a bf16 inference layer) keeps the expert
    weights also in the tile-packed layout (pack_weights) and runs the
    grouped GEMMs on it; call :meth:`repack` after changing the weights.

    ``fp8`` runs the expert GEMMs (routed and shared) in MXFP8: the expert
    weights are quantised once (pack_weights_mx; :meth:`repack` after a
    change), x is quantised at the start of each forward, fc1 quantises its
    SwiGLU output for fc2; routing stays in bf16 / fp32.  Inference only,
    with gathered rows; d, F and the shared ffn must be multiples of 32.

    ``fold_shared`` (default: on when it applies) runs a shared expert whose
    ffn equals the routed experts' as one more group of the routed grouped
    GEMM (inference without save_gu, gathered rows, packed or fp8 weights):
    its T rows (row t gathers x[t], row scale = the gate) follow the N
    routed rows, so one persistent launch covers both and the shared output
    is read by the combine from behind Y_perm.  The route writes the gate straight into
    the row-scale array.

    ``overlap_shared`` runs the shared expert, which depends only on x, on a
    second stream (default priority) concurrently with route, permute and
    the routed GEMM; its output stays unscaled and the combine applies the
    gate, so it does not wait for the router.  Off by default: measured on
    MI355X (16384 tokens, 256 experts, shared ffn 512) the shared GEMM's
    one-workgroup-per-CU tiles starve the small route and permute kernels
    (route 93 -> 176 us) and the layer was 2% slower than running it
    serially.
    """

    def __init__(self, w_router, w1, w2, k, T, score="softmax", normalize=True,
                 logit_bias=None, w_gate=None, ws1=None, ws2=None, save_gu=False,
                 gather=True, train=False, overlap_shared=False, selection_bias=None,
                 packed=None, fp8=False, fold_shared=None):
        self.train = train
        self.fp8 = fp8
        if fp8:
            Fs_ = ws1.shape[0] // 2 if ws1 is not None else 32
            if train or not gather or overlap_shared or w1.dtype != torch.bfloat16:
                raise MoEError("fp8 serves the bf16 inference forward with gathered rows, "
                               "without the shared-expert overlap")
            if w1.shape[2] % 32 or w1.shape[1] % 64 or Fs_ % 32:
                raise MoEError("fp8 needs d, F and the shared ffn to be multiples of 32")
            packed = False
        if packed is None:
            packed = not train and w1.dtype == torch.bfloat16
        if packed and (train or w1.dtype != torch.bfloat16):
            raise MoEError("packed weights serve the bf16 inference forward only")
        self.packed = packed
        self.selection_bias = selection_bias
        self.overlap_shared = overlap_shared and ws1 is not None
        if train:
            save_gu, gather = True, False
        self.gather = gather
        self.w_router, self.w1, self.w2 = w_router, w1, w2
        self.k, self.T, self.score, self.normalize = k, T, score, normalize
        self.logit_bias, self.w_gate, self.ws1, self.ws2 = logit_bias, w_gate, ws1, ws2
        dev, dt = w1.device, w1.dtype
        E, twoF, d = w1.shape
        self.E, self.F, self.d = E, twoF // 2, d
        N = T * k
        self.N = N
        i32, f32 = torch.int32, torch.float32
        # (no per-expert counts: the permute's offsets hold them)
        self.route_out = (torch.empty((T, k), dtype=i32, device=dev),
                          torch.empty((T, k), dtype=f32, device=dev),
                          None,
                          torch.empty((T,), dtype=f32, device=dev) if w_gate is not None else None)
        self.perm_out = (torch.empty((E + 1,), dtype=i32, device=dev),
                         torch.empty((T, k), dtype=i32, device=dev),
                         torch.empty((N,), dtype=i32, device=dev),
                         torch.empty((N,), dtype=f32, device=dev),
                         None if gather else torch.empty((N, d), dtype=dt, device=dev))
        self.perm_ws = _ws(permute_workspace_size(T, E, k), dev)
        self.route_ws = _ws(route_workspace_size(T, d, E, dt), dev)
        self.block_counts = route_block_counts(T, E, dev)   # route -> permute
        self.y_perm = torch.empty((N, d), dtype=dt, device=dev)
        self.gu = torch.empty((N, 2 * self.F), dtype=dt, device=dev) if save_gu else None
        ws_f = fwd_workspace_size(N, self.F, dt)
        if ws1 is not None:
            Fs = ws1.shape[0] // 2
            ws_f = max(ws_f, fwd_workspace_size(T, Fs, dt))
            self.shared_off = torch.tensor([0, T], dtype=i32, device=dev)
            self.y_shared = torch.empty((T, d), dtype=dt, device=dev)
            self.ws1_e = ws1.unsqueeze(0)
            self.ws2_e = ws2.unsqueeze(0)
            self.gu_sh = torch.empty((T, 2 * Fs), dtype=dt, device=dev) if train else None
            if self.overlap_shared:
                self.side = torch.cuda.Stream(device=dev)          # default priority
                self.ev_x = torch.cuda.Event()
                self.ev_sh = torch.cuda.Event()
                self.shared_ws = _ws(fwd_workspace_size(T, Fs, dt), dev)
        if fp8:
            ws_f = fwd_mx_workspace_size(N, self.F)
            if ws1 is not None:
                ws_f = max(ws_f, fwd_mx_workspace_size(T, ws1.shape[0] // 2))
            self.xq = MxTensor(torch.empty((T, d), dtype=torch.uint8, device=dev),
                               torch.empty(lib().moe_quantize_mx_scales_size(T, d),
                                           dtype=torch.uint8, device=dev), (T, d))
        can_fold = (ws1 is not None and not train and not save_gu and gather
                    and not self.overlap_shared and (packed or fp8)
                    and ws1.shape[0] // 2 == self.F and N % 4 == 0)
        if fold_shared is None:
            fold_shared = can_fold
        if fold_shared and not can_fold:
            raise MoEError("fold_shared needs a shared expert with the routed ffn, inference "
                           "without save_gu, gathered rows, packed or fp8 weights, and T*k a "
                           "multiple of 4")
        self.fold_shared = bool(fold_shared)
        if self.fold_shared:
            # [routed rows | shared rows]: offsets gain group E = [N, N + T), the
            # shared rows gather x[t] and take the gate (written by the route)
            # as their row scale; Y_perm's tail is the shared output
            self.off_ext = torch.empty((E + 2,), dtype=i32, device=dev)
            self.off_ext[E + 1] = N + T
            self.rtok_ext = torch.empty((N + T,), dtype=i32, device=dev)
            self.rtok_ext[N:] = torch.arange(T, dtype=i32, device=dev)
            self.rw_ext = torch.empty((N + T,), dtype=f32, device=dev)
            self.y_perm_ext = torch.empty((N + T, d), dtype=dt, device=dev)
            self.y_perm = self.y_perm_ext[:N]
            self.y_shared = self.y_perm_ext[N:]
            if w_gate is not None:
                self.route_out = self.route_out[:3] + (self.rw_ext[N:],)
            else:                                # an ungated shared expert: row scale 1
                self.rw_ext[N:] = 1.0
            self.perm_out = (self.off_ext[:E + 1], self.perm_out[1], self.rtok_ext[:N],
                             self.rw_ext[:N], None)
            ws_f = fwd_mx_workspace_size(N + T, self.F) if fp8 else \
                fwd_workspace_size(N + T, self.F, dt)
        self.ffn_ws = _ws(ws_f, dev)
        self.y = torch.empty((T, d), dtype=dt, device=dev)
        if train:
            self._alloc_backward(dev, dt)
        if packed or fp8:
            self.repack()

    def repack(self):
        """(Re)build the tile-packed (bf16) or MX-quantised (fp8) copies of
        the expert weights."""
        w1, w2 = self.w1, self.w2
        if getattr(self, "fold_shared", False):    # the shared expert as group E
            w1 = torch.cat([self.w1, self.ws1_e])
            w2 = torch.cat([self.w2, self.ws2_e])
        if self.fp8:
            self.w1q = pack_weights_mx(w1, True)
            self.w2q = pack_weights_mx(w2, False)
            if self.ws1 is not None and not self.fold_shared:
                self.ws1q = pack_weights_mx(self.ws1_e, True)
                self.ws2q = pack_weights_mx(self.ws2_e, False)
            return
        self.w1p = pack_weights(w1, True)
        self.w2p = pack_weights(w2, False)
        if self.ws1 is not None and not self.fold_shared:
            self.ws1p = pack_weights(self.ws1_e, True)
            self.ws2p = pack_weights(self.ws2_e, False)

    def _alloc_backward(self, dev, dt):
        T, N, d, E, F, k = self.T, self.N, self.d, self.E, self.F, self.k
        f32 = torch.float32
        self.dy_perm = torch.empty((N, d), dtype=dt, device=dev)
        self.d_topk_w = torch.empty((T, k), dtype=f32, device=dev)
        self.dx_perm = torch.empty((N, d), dtype=dt, device=dev)
        self.dx = torch.empty((T, d), dtype=dt, device=dev)
        self.dw1 = torch.zeros((E, 2 * F, d), dtype=f32, device=dev)
        self.dw2 = torch.zeros((E, d, F), dtype=f32, device=dev)
        self.dw_router = torch.zeros((E, d), dtype=f32, device=dev)
        bwd_ws = bwd_workspace_size(N, F, dt, False)
        if self.ws1 is not None:
            Fs = self.ws1.shape[0] // 2
            bwd_ws = max(bwd_ws, bwd_workspace_size(T, Fs, dt, False))
            self.d_gate = torch.empty((T,), dtype=f32, device=dev)
            self.dx_shared = torch.empty((T, d), dtype=dt, device=dev)
            self.dws1 = torch.zeros((1, 2 * Fs, d), dtype=f32, device=dev)
            self.dws2 = torch.zeros((1, d, Fs), dtype=f32, device=dev)
            self.dw_gate = torch.zeros((d,), dtype=f32, device=dev)
        self.bwd_ws = _ws(bwd_ws, dev)
        self.rbwd_ws = _ws(route_backward_workspace_size(T, d, E, k, dt, self.score,
                                                          self.normalize), dev)

    def _shared(self, x, scale, ws):
        if self.fp8:       # x quantised by _routed earlier in the forward
            grouped_swiglu_fwd_mx(self.xq, None, self.ws1q, self.ws2q, self.shared_off,
                                  row_scale=scale, out=self.y_shared, ws=ws)
        elif self.packed:
            grouped_swiglu_fwd_packed(x, None, self.ws1p, self.ws2p, self.shared_off,
                                      row_scale=scale, out=self.y_shared, ws=ws)
        else:
            grouped_swiglu_fwd(x, self.ws1_e, self.ws2_e, self.shared_off, row_scale=scale,
                               out=self.y_shared, gu_out=self.gu_sh if self.train else None,
                               save_gu=self.train, ws=ws)

    def _shared_unscaled(self, x):
        self._shared(x, None, self.shared_ws if self.overlap_shared else self.ffn_ws)

    def _routed(self, x, xp, rtok, off, rs):
        """The routed grouped GEMMs (fc1 gathers x rows by rtok when xp is None);
        with fold_shared, the shared expert's rows ride along as group E."""
        if self.fold_shared:
            rtok, off, rs, out = self.rtok_ext, self.off_ext, self.rw_ext, self.y_perm_ext
            if self.fp8:
                quantize_mx(x, out=self.xq)
                grouped_swiglu_fwd_mx(self.xq, rtok, self.w1q, self.w2q, off, row_scale=rs,
                                      out=out, ws=self.ffn_ws)
            else:
                grouped_swiglu_fwd_packed(x, rtok, self.w1p, self.w2p, off, row_scale=rs,
                                          out=out, ws=self.ffn_ws)
            return
        if self.fp8:
            quantize_mx(x, out=self.xq)
            grouped_swiglu_fwd_mx(self.xq, rtok, self.w1q, self.w2q, off, row_scale=rs,
                                  out=self.y_perm, ws=self.ffn_ws)
        elif self.packed:
            grouped_swiglu_fwd_packed(x if xp is None else xp, rtok if xp is None else None,
                                      self.w1p, self.w2p, off, row_scale=rs, out=self.y_perm,
                                      gu_out=self.gu, save_gu=self.gu is not None,
                                      ws=self.ffn_ws)
        elif xp is None:
            grouped_swiglu_fwd_gather(x, rtok, self.w1, self.w2, off, row_scale=rs,
                                      out=self.y_perm, gu_out=self.gu,
                                      save_gu=self.gu is not None, ws=self.ffn_ws)
        else:
            grouped_swiglu_fwd(xp, self.w1, self.w2, off, row_scale=rs, out=self.y_perm,
                               gu_out=self.gu, save_gu=self.gu is not None, ws=self.ffn_ws)

    def stages(self, x):
        """The inference forward (no overlap) as named stages, run in order on
        the current stream: route, permute, grouped_gemm (routed experts, and
        a folded shared expert), shared (the shared expert's own call, when
        not folded), combine.  forward() runs them back to back; a profiler
        may bracket each."""
        if self.train or self.overlap_shared:
            raise MoEError("stages() covers the inference forward without the overlap")
        st = {}

        def route_():
            st["r"] = route(x, self.w_router, self.k, self.score, self.normalize,
                            self.logit_bias, self.w_gate, out=self.route_out, ws=self.route_ws,
                            selection_bias=self.selection_bias, block_counts=self.block_counts)

        def permute_():
            idx, w, _, _ = st["r"]
            st["p"] = permute(x, idx, w, self.E, out=self.perm_out, ws=self.perm_ws,
                              copy_rows=not self.gather, block_counts=self.block_counts)

        def experts_():
            off, _, rtok, rw, xp = st["p"]
            self._routed(x, None if self.gather else xp, rtok, off, rw)

        def shared_():
            if self.ws1 is not None and not self.fold_shared:
                self._shared(x, st["r"][3], self.ffn_ws)

        def combine_():
            ysh = self.y_shared if self.ws1 is not None else None
            unpermute_combine(self.y_perm, st["p"][1], None, ysh, out=self.y)

        return [("route", route_), ("permute", permute_), ("grouped_gemm", experts_),
                ("shared", shared_), ("combine", combine_)]

    def forward(self, x):
        if not self.train and not self.overlap_shared:
            for _, fn in self.stages(x):
                fn()
            return self.y
        main = torch.cuda.current_stream()
        if self.overlap_shared:
            self.ev_x.record(main)
            self.side.wait_event(self.ev_x)
            with torch.cuda.stream(self.side):
                self._shared_unscaled(x)
                self.ev_sh.record(self.side)
            x.record_stream(self.side)
        idx, w, cnt, gate = route(x, self.w_router, self.k, self.score, self.normalize,
                                  self.logit_bias, self.w_gate, out=self.route_out,
                                  ws=self.route_ws, selection_bias=self.selection_bias,
                                  block_counts=self.block_counts)
        off, slot, rtok, rw, xp = permute(x, idx, w, self.E, out=self.perm_out, ws=self.perm_ws,
                                          copy_rows=not self.gather,
                                          block_counts=self.block_counts)
        rs = None if self.train else rw      # training: weights applied in combine
        self._routed(x, None if self.gather else xp, rtok, off, rs)
        ysh, sgate = None, None
        if self.ws1 is not None:
            if self.overlap_shared:
                main.wait_event(self.ev_sh)
                sgate = gate                   # unscaled shared output: gate in combine
            elif self.train:
                self._shared_unscaled(x)
                sgate = gate
            else:
                self._shared(x, gate, self.ffn_ws)
            ysh = self.y_shared
        if self.train:
            self.x_saved = x
            return unpermute_combine(self.y_perm, slot, w, ysh, out=self.y, shared_gate=sgate)
        return unpermute_combine(self.y_perm, slot, None, ysh, out=self.y, shared_gate=sgate)

    def backward(self, dy, accumulate=False):
        """Gradients of sum(dy * y) for the last forward (``train=True``):
        combine backward -> grouped-GEMM backward (and the shared expert's,
        row scale = gate) -> permute + router backward.  Returns a dict with
        dx, dw_router, dw1, dw2 (+ dws1, dws2, dw_gate with a shared expert);
        weight gradients are fp32 and accumulate into the held buffers when
        ``accumulate``.  Only kernel launches happen here."""
        if not self.train:
            raise MoEError("MoELayer.backward needs train=True")
        x = self.x_saved
        idx, w, _, gate = self.route_out
        off, slot, rtok, _, xp = self.perm_out
        shared = self.ws1 is not None
        combine_backward(dy, self.y_perm, slot, w, self.y_shared if shared else None,
                         dy_perm=self.dy_perm, d_topk_w=self.d_topk_w,
                         d_gate=self.d_gate if shared else None)
        grouped_swiglu_bwd(self.dy_perm, xp, self.w1, self.w2, off, self.gu, None, accumulate,
                           self.dw1, self.dw2, dx_out=self.dx_perm, ws=self.bwd_ws)
        if shared:
            grouped_swiglu_bwd(dy, x, self.ws1_e, self.ws2_e, self.shared_off, self.gu_sh, gate,
                               accumulate, self.dws1, self.dws2, dx_out=self.dx_shared,
                               ws=self.bwd_ws)
        route_backward(x, self.w_router, idx, w, self.d_topk_w, off, slot, rtok, self.score,
                       self.normalize, self.logit_bias, self.w_gate,
                       self.d_gate if shared else None, dx_perm=self.dx_perm,
                       dx_add=self.dx_shared if shared else None, accumulate=accumulate,
                       dx=self.dx, dw_router=self.dw_router,
                       dw_gate=self.dw_gate if shared else None, ws=self.rbwd_ws)
        g = dict(dx=self.dx, dw_router=self.dw_router, dw1=self.dw1, dw2=self.dw2)
        if shared:
            g.update(dws1=self.dws1[0], dws2=self.dws2[0], dw_gate=self.dw_gate)
        return g


def moe_layer_forward(x, w_router, w1, w2, k, score="softmax", normalize=True,
                      logit_bias=None, w_gate=None, ws1=None, ws2=None, gather=True):
    """Functional form of :class:`MoELayer` (allocates per call)."""
    layer = MoELayer(w_router, w1, w2, k, x.shape[0], score, normalize, logit_bias, w_gate,
                     ws1, ws2, gather=gather)
    y = layer.forward(x)
    return y, layer
