"""Helpers shared by the GPU parity tests: host<->device transfer of the
seeded inputs, poison fills, and the tolerance measures the tests apply.

Tolerances (normwise max relative error ||a - r||_inf / ||r||_inf, the
reading of "max relative error" this build takes):
  * fp32 path: 1e-5;  bf16 outputs: 2e-2;  bf16 gradients: 3e-2;
  * routing weights and gates are fp32 on both sides: 1e-5 absolute;
  * routing indices, permutation maps, counts, offsets and the permuted
    rows are compared bit for bit.
"""
import numpy as np
import torch

TOL_F32 = 1e-5
TOL_BF16 = 2e-2
TOL_BF16_GRAD = 3e-2
TOL_ROUTE_W = 1e-5
NEAR_TIE = 1e-5


def dev():
    return torch.device("cuda", 0)


def to_gpu(a: np.ndarray) -> torch.Tensor:
    """uint16 arrays are bf16 bit patterns; everything else keeps its type."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def poison(shape, dtype) -> torch.Tensor:
    t = torch.empty(shape, dtype=dtype, device=dev())
    if dtype.is_floating_point:
        t.fill_(float("nan"))
    else:
        t.fill_(-1)
    return t


def normwise(a: np.ndarray, r: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = np.abs(r).max()
    if den == 0:
        return float(np.abs(a).max())
    return float(np.abs(a - r).max() / den)


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def check_routing(gpu_idx: np.ndarray, gpu_w: np.ndarray, ref, k: int):
    """Compare the GPU's routing with the oracle's RouteResult ``ref``.

    Non-excluded tokens: the chosen expert sets must be identical and the
    order must match where consecutive chosen scores differ by >= NEAR_TIE.
    Excluded tokens (k-th/(k+1)-th margin < NEAR_TIE): the choice must be a
    legal near-tie choice.  Returns (n_excluded, n_excluded_differing).
    """
    T = gpu_idx.shape[0]
    excl = ref.excluded(NEAR_TIE)
    keep = ~excl
    g_sorted = np.sort(gpu_idx, axis=1)
    o_sorted = np.sort(ref.topk_idx, axis=1)
    bad = np.nonzero(keep & (g_sorted != o_sorted).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} non-excluded tokens differ, e.g. token {bad[:5]}"
    # order inside the top-k where the oracle's scores are clearly apart
    s = ref.s32.astype(np.float64)
    rows = np.arange(T)[:, None]
    os_ = s[rows, ref.topk_idx]
    gaps_ok = (os_[:, :-1] - os_[:, 1:] >= NEAR_TIE).all(axis=1) if k > 1 else np.ones(T, bool)
    sel = keep & gaps_ok
    assert (gpu_idx[sel] == ref.topk_idx[sel]).all()
    # excluded tokens: each chosen expert scores within NEAR_TIE of the k-th
    kth = os_[:, -1]
    chosen = s[rows, gpu_idx]
    assert (chosen[excl] >= kth[excl, None] - NEAR_TIE).all()
    assert all(len(set(r)) == k for r in gpu_idx.tolist())
    differing = int((excl & (g_sorted != o_sorted).any(axis=1)).sum())
    # weights on tokens with identical sets (compare by expert)
    same = (g_sorted == o_sorted).all(axis=1)
    if same.any():
        ow = np.zeros((T, ref.s.shape[1]))
        gw = np.zeros_like(ow)
        np.put_along_axis(ow, ref.topk_idx.astype(np.int64), ref.topk_w, axis=1)
        np.put_along_axis(gw, gpu_idx.astype(np.int64), gpu_w.astype(np.float64), axis=1)
        err = np.abs(ow[same] - gw[same]).max()
        assert err <= TOL_ROUTE_W, f"routing weights off by {err}"
    return int(excl.sum()), differing


class Bf16Experts:
    """Read-only view of a stacked bf16 weight tensor [E, ...] (uint16 bit
    patterns) that hands out one expert at a time as float32, so that the
    oracle's per-expert loops can run at full size without a float copy of
    every expert at once.  Supports what the oracle uses: ``shape`` and
    integer indexing."""

    def __init__(self, bits: np.ndarray):
        self.bits = bits
        self.shape = bits.shape
        self.dtype = np.float32

    def __len__(self):
        return self.shape[0]

    def __getitem__(self, e):
        if not isinstance(e, (int, np.integer)):
            raise TypeError("expert index only")
        b = self.bits[e]
        return b.astype(np.float32) if b.dtype != np.uint16 else (
            b.astype(np.uint32) << 16).view(np.float32)


def expert_weights_view(inp, name):
    """The workload's expert tensor as the oracle takes it: float32 arrays
    unchanged, bf16 bit arrays through Bf16Experts."""
    a = getattr(inp, name)
    if a is None or a.dtype != np.uint16:
        return a
    return Bf16Experts(a)


def normwise_per_expert(a, r, offsets=None):
    """Largest normwise error over the experts of stacked gradients [E, ...]
    (experts with no rows, when ``offsets`` is given, must be exactly 0 on
    both sides and are left out of the maximum)."""
    worst = 0.0
    for e in range(r.shape[0]):
        if offsets is not None and offsets[e + 1] == offsets[e]:
            assert not np.any(a[e]), f"expert {e} has no rows but a nonzero gradient"
            continue
        worst = max(worst, normwise(a[e], r[e]))
    return worst
