"""nvfp4_quantize_noalloc (the entry point that allocates nothing, for
callers under graph capture or in serving loops) against nvfp4_quantize on
the same inputs: codes, scales, global scale and tile partials bit-exact, on
two calls in a row, the second on a smaller tensor (the scratch keeps the
first call's partial maxima, which the second must not see)."""

import numpy as np
import pytest
import torch

import precision_gemm_nvfp4_amd as P
import synth

pytestmark = pytest.mark.gpu


def _both(x, amax_in=None):
    c0, s0, g0, t0 = P.nvfp4_quantize(x, amax_in=amax_in, tile_partials=True)
    m, k = x.shape
    c1 = torch.full((m, k // 2), 0xAB, dtype=torch.uint8, device=x.device)
    s1 = torch.full((m, k // 16), 0xCD, dtype=torch.uint8, device=x.device)
    g1 = torch.full((1,), -1.0, dtype=torch.float32, device=x.device)
    t1 = torch.full(((m + 127) // 128, k), -1.0, dtype=torch.float32, device=x.device)
    P.nvfp4_quantize_noalloc(x, c1, s1, g1, amax_in=amax_in, tile_partials=t1)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1)
    assert torch.equal(s0, s1)
    assert torch.equal(g0.view(torch.int32), g1.view(torch.int32))
    assert torch.equal(t0.view(torch.int32), t1.view(torch.int32))
    return g1.item()


def test_noalloc_matches_quantize_two_calls_second_smaller():
    P.load()
    dev = torch.device("cuda:0")
    big = synth.activations(3000, 1024, seed=31, heavy_frac=0.01).to(dev)
    # the second tensor's amax is far below the first's: a stale partial
    # maximum left in the scratch would change its global scale
    small = (synth.activations(200, 512, seed=32, heavy_frac=0.0).float() * 1e-3).to(torch.bfloat16).to(dev)
    g_big = _both(big)
    g_small = _both(small)
    assert g_small < g_big / 100
    # fp32 input and a given amax take the other paths of the same launcher
    _both(small.float())
    amax = torch.tensor([5.0], dtype=torch.float32, device=dev)
    _both(small, amax_in=amax)


def test_noalloc_empty_tensor_sets_g_to_one():
    dev = torch.device("cuda:0")
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    c = torch.empty(0, 32, dtype=torch.uint8, device=dev)
    s = torch.empty(0, 4, dtype=torch.uint8, device=dev)
    g = torch.zeros(1, dtype=torch.float32, device=dev)
    P.nvfp4_quantize_noalloc(x, c, s, g)
    torch.cuda.synchronize()
    assert g.item() == 1.0
