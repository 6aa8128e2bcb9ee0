"""Pins of the oracle's dense-mask residual compensation (QUADS section 2.2B:
a binary channel mask keeps the top k% of channels, 50% in the pages'
example; the masked residual is quantized a second time and its GEMM term is
added back).

Each test checks the oracle against something other than itself: an
invariant of the mask, the special cases that reduce to the already pinned
quantizer and compact selection, brute force with independently decoded
operands on tiny inputs, and the size and sign of the correction.  None
needs a GPU.
"""

import numpy as np
import torch

from oracle import gemm as G
from oracle import nvfp4 as Q

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _units(rows_per_unit):
    return np.concatenate([[0], np.cumsum(rows_per_unit)]).astype(np.int64)


def test_mask_zero_outside_selection():
    """Every masked channel dequantizes to exactly 0, and every row has some
    nonzero correction on the selected ones."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((70, 128)).astype(np.float32)
    c, s, g = Q.quantize(x)
    offs = _units([30, 0, 40])
    sel, mc, ms, mg = Q.resq_mask_select_and_requant(x, c, s, g, offs, 64)
    dq = Q.dequantize(mc, ms, 1.0)
    for u in range(3):
        a, b = offs[u], offs[u + 1]
        off = np.setdiff1d(np.arange(128), sel[u])
        assert np.all(dq[a:b][:, off] == 0)
        if b > a:
            assert np.all(np.any(dq[a:b][:, sel[u]] != 0, axis=1))
    assert np.array_equal(sel[1], np.arange(64)) and mg[1] == 1.0


def test_full_mask_is_plain_quantizer_of_residual():
    """k = K: the mask keeps everything, so the correction is the NVFP4
    quantization of R (global scale from the unit's amax of |R|)."""
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((48, 64)) * np.exp(rng.standard_normal((1, 64)))).astype(np.float32)
    c, s, g = Q.quantize(x)
    offs = _units([20, 28])
    sel, mc, ms, mg = Q.resq_mask_select_and_requant(x, c, s, g, offs, 64)
    r = Q.residual(x, c, s, g)
    for u in range(2):
        a, b = offs[u], offs[u + 1]
        rc, rs, rg = Q.quantize(r[a:b])
        assert np.array_equal(sel[u], np.arange(64))
        assert np.array_equal(mc[a:b], rc) and np.array_equal(ms[a:b], rs) and mg[u] == rg


def test_aligned_selection_matches_compact_form():
    """When the selected channels are whole 16-aligned blocks, the masked
    blocks are exactly the compact form's blocks: same codes, block scales
    and global scale, placed at the selected blocks; the other blocks are
    zero codes with zero scales."""
    rng = np.random.default_rng(13)
    x = np.zeros((40, 96), dtype=np.float32)
    hot = [1, 4]                                  # channels 16..31 and 64..79
    for bl in hot:
        x[:, 16 * bl:16 * bl + 16] = rng.standard_normal((40, 16))
    c, s, g = Q.quantize(x)
    r = Q.residual(x, c, s, g)
    assert np.all(np.abs(r[:, 16:32]).sum(0) > 0) and np.all(np.abs(r[:, 64:80]).sum(0) > 0)
    offs = _units([40])
    sel, mc, ms, mg = Q.resq_mask_select_and_requant(x, c, s, g, offs, 32)
    sel_c, rc, rs, rg = Q.resq_select_and_requant(x, c, s, g, offs, 32)
    assert np.array_equal(sel[0], np.r_[16:32, 64:80]) and np.array_equal(sel, sel_c)
    assert mg[0] == rg[0]
    for j, bl in enumerate(hot):
        assert np.array_equal(mc[:, 8 * bl:8 * bl + 8], rc[:, 8 * j:8 * j + 8])
        assert np.array_equal(ms[:, bl], rs[:, j])
    cold = [b for b in range(6) if b not in hot]
    for bl in cold:
        assert np.all(mc[:, 8 * bl:8 * bl + 8] == 0) and np.all(ms[:, bl] == 0)


def _dq_brute(codes, scales, g):
    """Dequantize with a literal E2M1 table and torch's E4M3 decoder; the
    effective block scale is the fp32 product of the E4M3 scale and the
    global scale, and the element times it is rounded once to fp32 (the
    NVFP4 decode rule of the TRACE prerequisites: block scale, then global
    scale, fp32 arithmetic)."""
    m, kh = codes.shape
    sc = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn).double().numpy()
    out = np.zeros((m, 2 * kh))
    for i in range(m):
        for j in range(2 * kh):
            nib = (int(codes[i, j // 2]) >> (4 * (j % 2))) & 15
            v = E2M1[nib & 7] * (-1.0 if nib & 8 else 1.0)
            eff = np.float32(sc[i, j // 16] * np.float32(g))
            out[i, j] = float(np.float32(v * float(eff)))
    return out


def test_masked_gemm_brute_force():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((6, 32)).astype(np.float32)
    w = rng.standard_normal((5, 32)).astype(np.float32)
    xc, xs, xg = Q.quantize(x)
    wc, ws, wg = Q.quantize(w)
    sel, mc, ms, mg = Q.resq_mask_select_and_requant(x, xc, xs, xg, _units([6]), 16)
    y = G.gemm_masked_comp(xc, xs, xg, wc, ws, wg, mc, ms, mg[0])
    a, b, m = _dq_brute(xc, xs, xg), _dq_brute(wc, ws, wg), _dq_brute(mc, ms, mg[0])
    ref = np.zeros((6, 5))
    for i in range(6):
        for n in range(5):
            ref[i, n] = sum((a[i, t] + m[i, t]) * b[n, t] for t in range(32))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_correction_shrinks_activation_error():
    """DQ(Q(X)) + DQ(Q(R*M)) is much closer to X than DQ(Q(X)) on the masked
    channels, and leaves the others untouched: a flipped sign or a
    transposed mask fails this."""
    rng = np.random.default_rng(15)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    c, s, g = Q.quantize(x)
    sel, mc, ms, mg = Q.resq_mask_select_and_requant(x, c, s, g, _units([64]), 64)
    base = Q.dequantize(c, s, g).astype(np.float64)
    fixed = base + Q.dequantize(mc, ms, mg[0]).astype(np.float64)
    on = sel[0]
    off = np.setdiff1d(np.arange(128), on)
    e0 = np.linalg.norm(x[:, on] - base[:, on])
    e1 = np.linalg.norm(x[:, on] - fixed[:, on])
    assert e1 < 0.2 * e0
    assert np.array_equal(fixed[:, off], base[:, off])
    # the top half by residual score carries more than half of the error
    assert e0 ** 2 > 0.5 * np.linalg.norm(x - base) ** 2
