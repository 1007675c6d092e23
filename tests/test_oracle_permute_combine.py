"""Pins of the oracle's permutation and combine (CPU only).

  * a hand-worked counting sort (tests/golden/permute_worked.json);
  * nested-loop brute force vs the stable-argsort oracle;
  * invariants: each token appears exactly k times, counts sum to T*k,
    offsets are monotone, token order ascends inside a segment, and
    unpermute(permute(x)) == x bit for bit;
  * combine: one-hot weights give an exact gather, equal rows give
    row * sum(w), and a permutation round trip with unit weights.
"""
import json
import os

import numpy as np
import pytest

from oracle import brute
from oracle import moe_oracle as mo

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_permute():
    with open(os.path.join(GOLD, "permute_worked.json")) as f:
        g = json.load(f)
    idx = np.array(g["topk_idx"], dtype=np.int32)
    p = mo.permute(None, idx, None, g["E"])
    assert p.offsets.tolist() == g["offsets"]
    assert p.row_token.tolist() == g["row_token"]
    assert p.slot_of.tolist() == g["slot_of"]


def _random_idx(rng, T, E, k):
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 3, 2), (33, 8, 8), (50, 16, 4)])
def test_permute_matches_brute_force(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    idx = _random_idx(rng, T, E, k)
    p = mo.permute(None, idx, None, E)
    off_b, slot_b, tok_b = brute.permute(idx.tolist(), E)
    assert p.offsets.tolist() == off_b
    assert p.slot_of.tolist() == slot_b
    assert p.row_token.tolist() == tok_b


def test_permute_invariants_and_roundtrip():
    rng = np.random.default_rng(9)
    T, E, k, d = 300, 20, 6, 5
    # draw from every expert except 3, so expert 3 is empty
    pool = np.array([e for e in range(E) if e != 3])
    idx = np.stack([rng.choice(pool, size=k, replace=False)
                    for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k))
    x = rng.standard_normal((T, d)).astype(np.float32)
    p = mo.permute(x, idx, w, E)
    N = T * k
    assert np.bincount(p.row_token, minlength=T).tolist() == [k] * T
    assert p.offsets[0] == 0 and p.offsets[-1] == N
    assert (np.diff(p.offsets) >= 0).all()
    assert p.offsets[4] - p.offsets[3] == 0   # expert 3 is empty
    for e in range(E):
        seg = p.row_token[p.offsets[e]:p.offsets[e + 1]]
        assert (np.diff(seg) > 0).all()
    assert sorted(p.slot_of.reshape(-1).tolist()) == list(range(N))
    for t in range(T):
        for j in range(k):
            r = p.slot_of[t, j]
            assert p.row_token[r] == t
            assert p.offsets[idx[t, j]] <= r < p.offsets[idx[t, j] + 1]
            assert p.row_w[r] == w[t, j]
    # unpermute(permute(x)) == x, bit for bit, for every copy
    for j in range(k):
        assert np.array_equal(p.x_perm[p.slot_of[:, j]].view(np.uint32),
                              x.view(np.uint32))


def test_combine_one_hot_is_exact_gather():
    rng = np.random.default_rng(4)
    T, k, d = 10, 3, 6
    y_perm = rng.standard_normal((T * k, d))
    slot_of = rng.permutation(T * k).reshape(T, k)
    w = np.zeros((T, k))
    pick = rng.integers(0, k, T)
    w[np.arange(T), pick] = 1.0
    y = mo.unpermute_combine(y_perm, slot_of, w)
    assert np.array_equal(y, y_perm[slot_of[np.arange(T), pick]])


def test_combine_equal_rows_scale_by_weight_sum():
    rng = np.random.default_rng(6)
    T, k, d = 8, 4, 5
    row = rng.standard_normal(d)
    y_perm = np.tile(row, (T * k, 1))
    slot_of = np.arange(T * k).reshape(T, k)
    w = rng.random((T, k))
    y = mo.unpermute_combine(y_perm, slot_of, w)
    np.testing.assert_allclose(y, w.sum(axis=1)[:, None] * row[None, :], rtol=1e-14)


def test_combine_adds_shared_rows_and_prescaled_rows():
    rng = np.random.default_rng(8)
    T, k, d = 5, 2, 3
    y_perm = rng.standard_normal((T * k, d))
    slot_of = np.arange(T * k).reshape(T, k)
    ysh = rng.standard_normal((T, d))
    y = mo.unpermute_combine(y_perm, slot_of, None, ysh)
    np.testing.assert_allclose(y, y_perm[0::2] + y_perm[1::2] + ysh, rtol=1e-14)
