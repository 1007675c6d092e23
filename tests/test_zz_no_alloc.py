"""moe_permute_noalloc (the permute with the library's static scratch instead
of a caller workspace) against moe_permute, through the C ABI: bit-identical
maps and row copies on two calls in a row, the second with a smaller input
(the static scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import moe_workloads as mw
import gpu_helpers as gh

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("mixture_experts_layer_05_amd")


def _case(T, d, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    x = mw.make_small_layer_inputs(seed, T=T, d=d, E=1, F=8, dtype="bf16").x
    return gh.to_gpu(x), gh.to_gpu(idx), gh.to_gpu(w)


def test_permute_noalloc_matches_permute():
    # the first call fills more of the static scratch than the second reads
    for T, d, E, k, seed in ((4096, 2048, 256, 8, 11), (300, 64, 16, 4, 12)):
        x, gi, gw = _case(T, d, E, k, seed)
        ref = moe.permute(x, gi, gw, E)
        got = moe.permute_noalloc(x, gi, gw, E)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert gh.bits_equal(a, b), (T, E, k)
