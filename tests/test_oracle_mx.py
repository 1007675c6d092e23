"""Pins of the MX (microscaled FP8 E4M3) oracle: E4M3 values fixed by the
format's definition (sign, 4 exponent bits with bias 7, 3 mantissa bits,
subnormals, S.1111.111 = NaN), nearest-even rounding with saturation checked
against an exhaustive nearest-value search, the block-scale rule on hand-worked
blocks, the quantisation error bound, and the MX forward against a pure-Python
loop and against the exact forward on exactly representable inputs."""
import math

import numpy as np
import pytest

from oracle import mx_oracle as mx
from oracle import moe_oracle as mo

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x30, 0.5), (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0),
    (0x78, 256.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0),
])
def test_e4m3_values(code, value):
    assert mx.e4m3_decode(code) == value


def test_e4m3_specials_and_order():
    assert math.isnan(mx.e4m3_decode(0x7F)) and math.isnan(mx.e4m3_decode(0xFF))
    assert math.copysign(1.0, mx.e4m3_decode(0x80)) == -1.0
    pos = mx.e4m3_decode(np.arange(127))
    assert (np.diff(pos) > 0).all() and len(set(pos)) == 127      # 127 distinct, increasing
    assert (mx.e4m3_decode(np.arange(128, 255)) == -pos).all()


def _nearest_even_search(a):
    """Brute force: the nearest E4M3 value to a >= 0 (a <= 448), ties to the even code."""
    best, bd = 0, None
    for c in range(127):
        dv = abs(float(mx.e4m3_decode(c)) - a)
        if bd is None or dv < bd or (dv == bd and c % 2 == 0 and best % 2 == 1):
            best, bd = c, dv
    return best


def test_e4m3_encode_against_search():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.uniform(0, 448, 600), np.exp2(rng.uniform(-12, 8.8, 600)),
                           mx.e4m3_decode(np.arange(127))])
    codes = mx.e4m3_encode(vals)
    for v, c in zip(vals, codes):
        assert c == _nearest_even_search(float(v)), v


def test_e4m3_ties_saturation_round_trip():
    pos = mx.e4m3_decode(np.arange(127))
    mid = (pos[:-1] + pos[1:]) / 2                      # every tie between neighbours
    got = mx.e4m3_encode(mid)
    want = np.where(np.arange(126) % 2 == 0, np.arange(126), np.arange(1, 127))
    assert (got == want).all()
    assert (mx.e4m3_encode(np.nextafter(mid, np.inf)) == np.arange(1, 127)).all()
    assert (mx.e4m3_encode(np.nextafter(mid, -np.inf)) == np.arange(126)).all()
    assert (mx.e4m3_encode([449.0, 464.0, 480.0, 1e6, np.inf]) == 0x7E).all()
    assert (mx.e4m3_encode([-449.0, -1e30]) == 0xFE).all()
    assert mx.e4m3_encode(2.0 ** -10) == 0 and mx.e4m3_encode(np.nextafter(2.0 ** -10, 1)) == 1
    assert mx.e4m3_encode(-0.0) == 0x80 and mx.e4m3_encode(np.nan) == 0x7F
    c = np.arange(256)
    finite = ~np.isnan(mx.e4m3_decode(c))
    assert (mx.e4m3_encode(mx.e4m3_decode(c[finite])) == c[finite]).all()


def test_mx_block_scale_hand_worked():
    # amax 1.0: scale 2^(0 - 8) (code 119); 1.0 -> 256 = code 0x78; 0.5 -> 128 = 0x70
    blk = np.zeros(32); blk[0], blk[1] = 1.0, -0.5
    codes, sc = mx.mx_quantize(blk)
    assert sc.tolist() == [119] and codes[0] == 0x78 and codes[1] == 0xF0
    assert (codes[2:] == 0).all()
    # amax 448: scale 1 (code 127), the element itself; amax 500 saturates
    assert mx.mx_quantize(np.full(32, 448.0))[1].tolist() == [127]
    c, s = mx.mx_quantize(np.r_[500.0, np.ones(31)])
    assert s.tolist() == [127] and c[0] == 0x7E and c[1] == 0x38
    # all-zero block: smallest scale, zero codes; two blocks scale independently
    c, s = mx.mx_quantize(np.r_[np.zeros(32), np.full(32, 3.0)])
    assert s.tolist() == [0, 128 - 8] and (c[:32] == 0).all()
    assert mx.mx_dequantize(c, s)[32] == 3.0


def test_mx_error_bound():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    d = mx.mx_dequantize(*mx.mx_quantize(v))
    blocks = np.abs(v).reshape(64, 8, 32).max(-1)
    X = np.exp2(np.floor(np.log2(blocks)) - 8)          # the block scale
    Xe = np.repeat(X, 32, axis=1)
    sat = np.abs(v) > 448.0 * Xe                        # |v / X| in (448, 512): clamped
    normal = (np.abs(v) >= Xe * 2.0 ** -6) & ~sat       # element in E4M3's normal range
    rel = np.abs(d - v)[normal] / np.abs(v)[normal]
    assert rel.max() <= 2.0 ** -4 + 1e-12                # half an ulp of 3 mantissa bits
    sub = ~normal & ~sat
    assert (np.abs(d - v)[sub] <= Xe[sub] * 2.0 ** -10 + 1e-300).all()
    assert sat.any() and (d[sat] == np.sign(v[sat]) * 448.0 * Xe[sat]).all()
    assert (np.abs(d - v)[sat] / np.abs(v)[sat]).max() < 1.0 / 8


def _loop_forward_mx(x, w1, w2, off, rs):
    """Pure-Python MX forward: block scales and codes by the brute-force search."""
    def q(row):
        out = []
        for b in range(0, len(row), 32):
            blk = row[b:b + 32]
            amax = max(abs(float(t)) for t in blk)
            if amax == 0:
                out += [0.0] * 32
                continue
            X = 2.0 ** (math.floor(math.log2(amax)) - 8)
            for t in blk:
                a = min(abs(float(t)) / X, 448.0)
                c = _nearest_even_search(a)
                out.append(math.copysign(float(mx.e4m3_decode(c)), t) * X)
        return out
    N, d = x.shape
    E, twoF, _ = w1.shape
    F = twoF // 2
    y = [[0.0] * d for _ in range(N)]
    for e in range(E):
        W1 = [q(w1[e, r]) for r in range(twoF)]
        W2 = [q(w2[e, r]) for r in range(d)]
        for r in range(off[e], off[e + 1]):
            xr = q(x[r])
            a = []
            for f in range(F):
                g = sum(xr[i] * W1[f][i] for i in range(d))
                u = sum(xr[i] * W1[F + f][i] for i in range(d))
                a.append(float(np.float32(g / (1.0 + math.exp(-g)) * u)))
            aq = q(np.array(a))
            for c in range(d):
                y[r][c] = sum(aq[f] * W2[c][f] for f in range(F)) * rs[r]
    return np.array(y)


def test_forward_mx_against_loops():
    rng = np.random.default_rng(2)
    E, d, F = 2, 64, 32
    off = np.array([0, 3, 5])
    x = rng.standard_normal((5, d))
    w1 = rng.standard_normal((E, 2 * F, d)) * 0.3
    w2 = rng.standard_normal((E, d, F)) * 0.3
    rs = rng.random(5) + 0.5
    ref = _loop_forward_mx(x, w1, w2, off, rs)
    got, a, parts = mx.grouped_swiglu_fwd_mx(x, w1, w2, off, rs, return_a=True,
                                             return_parts=True)
    assert np.abs(got - ref).max() <= 1e-9 * np.abs(ref).max()
    # the returned codes and scales are A's quantisation, of a32 = float32(silu(g) u)
    assert (mx.mx_dequantize(parts["codes"], parts["scales"]) == a).all()
    assert parts["scales"].shape == (5, 1)
    assert (mx.mx_quantize(parts["a32"])[0] == parts["codes"]).all()
    sil = parts["g"] / (1.0 + np.exp(-parts["g"]))
    assert np.allclose(parts["a32"], sil * parts["u"], rtol=2.0 ** -23, atol=0)


def test_forward_mx_exact_inputs_equal_unquantised():
    """Inputs that MX represents exactly give the unquantised GEMMs: E4M3 values
    of mantissa <= 1.75 keep every block's amax / scale <= 448, so nothing
    rounds or saturates.  fc2 then equals the exact product with the oracle's
    own quantised A, and A is the float32 SwiGLU within one E4M3 rounding."""
    rng = np.random.default_rng(3)
    E, d, F = 2, 64, 32
    off = np.array([0, 4, 7])
    codes = [c for c in range(0x38, 0x47) if (c & 7) <= 6]          # 1 .. 3.5
    vals = mx.e4m3_decode(np.array(codes))
    x = rng.choice(vals, (7, d)) * rng.choice([-1, 1], (7, d))
    w1 = rng.choice(vals, (E, 2 * F, d)) * 2.0 ** -7
    w2 = rng.choice(vals, (E, d, F)) * 2.0 ** -7
    for arr in (x, w1, w2):
        assert (mx.mx_dequantize(*mx.mx_quantize(arr)) == arr).all()
    y, a = mx.grouped_swiglu_fwd_mx(x, w1, w2, off, None, return_a=True)
    y_ref = np.concatenate([a[off[e]:off[e + 1]] @ w2[e].T for e in range(E)])
    assert np.abs(y - y_ref).max() <= 1e-12 * np.abs(y_ref).max()
    g = np.concatenate([x[off[e]:off[e + 1]] @ w1[e, :F].T for e in range(E)])
    u = np.concatenate([x[off[e]:off[e + 1]] @ w1[e, F:].T for e in range(E)])
    a_exact = mo.silu(g) * u
    blocks = np.abs(a_exact).reshape(7, F // 32, 32).max(-1)
    X = np.repeat(np.exp2(np.floor(np.log2(blocks)) - 8), 32, axis=1)
    aa = np.abs(a_exact)
    bound = np.where(aa > 448.0 * X, aa - 448.0 * X, np.maximum(aa * 2.0 ** -4, X * 2.0 ** -10))
    assert (np.abs(a - a_exact) <= bound * (1 + 1e-9) + aa * 2.0 ** -23).all()
