"""Plain CPU oracle of the FP8 (MX, microscaled E4M3) grouped SwiGLU forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the entry
module and the benchmark's ``cpu_baseline`` leg may import or run this file.
It shares no code with the HIP library and imports nothing from it.

What it computes, with the passages it follows:

* FP8 E4M3 values ("Megatron-Bridge 深度剖析", section "FP8 训练": FP8
  doubles the matrix throughput of BF16 and halves the bytes moved, the E4M3
  format has a small dynamic range, so scale factors must be managed; the
  grouped GEMM of a many-expert MoE is memory-bound in BF16 and FP8 halves
  its traffic);
* microscaling ("Megatron-Bridge 深度剖析", section on future directions:
  MXFP8 uses finer-grained scale factors than per-tensor FP8): every block
  of 32 consecutive values along the reduction dimension shares one scale;
* the forward of the grouped SwiGLU FFN of ``moe_oracle`` with its three
  GEMM operands (token rows, fc1 weights, the SwiGLU output) and the fc2
  weights quantised that way, accumulated exactly (float64).

Readings where the pages are silent (each listed in the design notes):
  * the element format is OCP E4M3 ("FN"): bias 7, 3 mantissa bits,
    subnormals, largest finite value 448 (the pages round it to ~480),
    code S.1111.111 is NaN, no infinities;
  * the scale is an E8M0 power of two, one per 32 consecutive values along
    K (the OCP Microscaling format): X = 2^(floor(log2 amax) - 8), where 8
    is the exponent of E4M3's largest normal; an all-zero block gets the
    smallest scale (code 0, 2^-127);
  * elements are v / X rounded to nearest, ties to even, saturated to
    +-448 (|v / X| < 512 always, so saturation only catches [448, 512));
  * quantised: the token rows along the hidden dimension, each fc1 weight
    row along the hidden dimension, the SwiGLU output A = silu(G) U per
    row along the ffn dimension (the quantisation decision is taken on the
    float32 value of A, the precision the kernel holds it in), each fc2
    weight row along the ffn dimension;
  * the routing weight scales fc2's output rows as in the bf16 path.
"""
from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "MX_BLOCK", "e4m3_decode", "e4m3_encode", "mx_scale_code",
           "mx_quantize", "mx_dequantize", "grouped_swiglu_fwd_mx"]

E4M3_MAX = 448.0
MX_BLOCK = 32
_E4M3_EMAX = 8          # exponent of the largest normal, 448 = 1.75 * 2^8


def e4m3_decode(codes):
    """E4M3 code bytes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = (m / 8.0) * np.exp2(-6.0)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


_POS_CODES = np.arange(127, dtype=np.int64)          # 0 .. 126: +0 .. 448
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(v):
    """Round to the nearest E4M3 value, ties to the even code, saturating at
    +-448; NaN -> 0x7F.  The sign of zero follows the input."""
    x = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")        # first value >= a
    hi = np.clip(hi, 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (_POS_CODES[lo] % 2 == 0))
    code = np.where(pick_lo, _POS_CODES[lo], _POS_CODES[hi])
    code = np.where(np.signbit(x), code | 0x80, code)
    return np.where(np.isnan(x), 0x7F, code).astype(np.uint8)


def mx_scale_code(amax):
    """E8M0 code of a block's scale: floor(log2 amax) - 8 + 127 (clamped to
    0..254); 0 for an all-zero block."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = f 2^ex, f in [0.5, 1)
    code = (ex - 1) - _E4M3_EMAX + 127
    code = np.clip(code, 0, 254)
    return np.where(a > 0, code, 0).astype(np.uint8)


def mx_quantize(v, block=MX_BLOCK):
    """Quantise along the last axis in blocks of ``block`` values.
    -> (codes uint8, same shape; scale codes uint8, [..., K / block])."""
    x = np.asarray(v, dtype=np.float64)
    K = x.shape[-1]
    if K % block:
        raise ValueError("the last dimension must be a multiple of the block")
    xb = x.reshape(x.shape[:-1] + (K // block, block))
    sc = mx_scale_code(np.abs(xb).max(axis=-1))
    scale = np.exp2(sc.astype(np.float64) - 127.0)
    codes = e4m3_encode(xb / scale[..., None])
    return codes.reshape(x.shape), sc


def mx_dequantize(codes, scale_codes, block=MX_BLOCK):
    """codes [..., K], scale codes [..., K / block] -> float64 values."""
    c = np.asarray(codes)
    K = c.shape[-1]
    v = e4m3_decode(c).reshape(c.shape[:-1] + (K // block, block))
    scale = np.exp2(np.asarray(scale_codes, dtype=np.float64) - 127.0)
    return (v * scale[..., None]).reshape(c.shape)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def grouped_swiglu_fwd_mx(x_perm, w1, w2, offsets, row_scale=None, return_a=False,
                          return_parts=False):
    """The grouped SwiGLU forward with MX-quantised GEMM operands.

    x_perm [N, d], w1 [E, 2F, d] (gate rows first), w2 [E, d, F]: the bf16
    values as float arrays.  Per expert e over rows [offsets[e], offsets[e+1]):
        G, U = Q(X) Q(W1[e, :F])^T, Q(X) Q(W1[e, F:])^T
        A    = silu(G) U;  Aq = Q(float32(A))
        Y    = (Aq Q(W2[e])^T) * row_scale
    with Q = MX quantise + dequantise along the reduction dimension, all sums
    in float64.  -> Y [N, d]; with return_a also the dequantised A [N, F];
    with return_parts also a dict of the intermediates: "xq", "w1q", "w2q"
    (dequantised operands), "g", "u" [N, F], "a32" (A in float32 before its
    quantisation), "codes" [N, F] and "scales" [N, F / 32] (A's MX codes)."""
    N, d = x_perm.shape
    E, twoF, _ = w1.shape
    F = twoF // 2
    xq = mx_dequantize(*mx_quantize(x_perm))
    w1q = mx_dequantize(*mx_quantize(w1))
    w2q = mx_dequantize(*mx_quantize(w2))
    y = np.zeros((N, d))
    a_all = np.zeros((N, F))
    a_codes = np.zeros((N, F), np.uint8)
    a_scales = np.zeros((N, F // MX_BLOCK), np.uint8)
    g_all, u_all, a32_all = np.zeros((N, F)), np.zeros((N, F)), np.zeros((N, F))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        xe = xq[lo:hi]
        g = xe @ w1q[e, :F].T
        u = xe @ w1q[e, F:].T
        a = (_silu(g) * u).astype(np.float32).astype(np.float64)
        g_all[lo:hi], u_all[lo:hi], a32_all[lo:hi] = g, u, a
        codes, scales = mx_quantize(a)
        aq = mx_dequantize(codes, scales)
        a_all[lo:hi] = aq
        a_codes[lo:hi], a_scales[lo:hi] = codes, scales
        y[lo:hi] = aq @ w2q[e].T
    if row_scale is not None:
        y = y * np.asarray(row_scale, dtype=np.float64)[:, None]
    parts = dict(xq=xq, w1q=w1q, w2q=w2q, g=g_all, u=u_all, a32=a32_all, codes=a_codes,
                 scales=a_scales)
    out = (y,) + ((a_all,) if return_a else ()) + ((parts,) if return_parts else ())
    return out if len(out) > 1 else y
