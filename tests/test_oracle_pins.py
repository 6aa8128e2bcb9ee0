"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/worked_example.json), a library implementation of
the same format (torch.float8_e4m3fn), brute force with exact rational
arithmetic on tiny inputs, closed forms and invariants.  None needs a GPU.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import gemm as G
from oracle import nvfp4 as Q

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


# ---------------------------------------------------------------------------
# brute-force helpers (exact rationals; independent of the oracle's code)
# ---------------------------------------------------------------------------

def torch_e4m3_values():
    """E4M3FN values of bytes 0x00..0x7E decoded by torch (a library decoder)."""
    b = torch.arange(0x7F, dtype=torch.uint8)
    return [Fraction(float(v)) for v in b.view(torch.float8_e4m3fn).float()]


E4M3_TORCH = torch_e4m3_values()
E2M1_PAGE = [Fraction(v) for v in GOLDEN["e2m1_levels"]["value"]]


def nearest_even(q, table):
    """Index of the entry of an increasing table nearest to the rational q;
    ties to the even index; beyond the table saturates to the last entry."""
    best = min(range(len(table)), key=lambda i: (abs(table[i] - q), i % 2))
    return best


def bf_fp32(q):
    """The fp32 value nearest to rational q (ties to even), by search."""
    f = np.float32(float(q))          # within an ulp
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


def brute_quantize_block(xs, g):
    """Quantize one 16-element block exactly: returns (scale byte, codes)."""
    amax = max(abs(Fraction(float(v))) for v in xs)
    q = amax / (6 * Fraction(float(g)))
    s_byte = nearest_even(q, E4M3_TORCH) if q < 448 else 0x7E
    S = bf_fp32(E4M3_TORCH[s_byte] * Fraction(float(g)))
    codes = []
    for v in xs:
        fv = Fraction(float(v))
        idx = 0 if S == 0 else nearest_even(abs(fv) / Fraction(float(S)), E2M1_PAGE)
        sign = 1 if np.signbit(np.float32(v)) else 0
        codes.append(sign << 3 | idx)
    return s_byte, codes


# ---------------------------------------------------------------------------
# formats
# ---------------------------------------------------------------------------

def test_e2m1_levels_match_pages():
    lv = GOLDEN["e2m1_levels"]
    assert list(F.E2M1_LEVELS) == lv["value"]
    assert len(F.E2M1_LEVELS) == lv["levels_per_sign"]
    vals = F.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == lv["value"]
    assert list(vals[8:]) == [-v for v in lv["value"]]
    assert np.all(np.diff(vals[:8]) > 0)


def test_e4m3_decode_matches_library():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    ours = F.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert len(F.E4M3_VALUES) == 127 and F.E4M3_VALUES[-1] == 448.0
    assert F.E4M3_VALUES[1] == 2.0 ** -9 and np.all(np.diff(F.E4M3_VALUES) > 0)


def test_e4m3_rounding_matches_library_cast():
    """Nearest-even E4M3 of fp32 values up to 464 equals torch's RNE cast
    (torch turns values that round past 448 into NaN; the scale saturates)."""
    rng = np.random.default_rng(0)
    q = np.concatenate([
        np.exp(rng.uniform(np.log(1e-4), np.log(470), 200000)),
        F.E4M3_MIDPOINTS,                                          # exact ties
        np.nextafter(F.E4M3_MIDPOINTS.astype(np.float32), np.float32(0)),
        np.nextafter(F.E4M3_MIDPOINTS.astype(np.float32), np.float32(1e9)),
        [0.0, 2.0 ** -10, 2.0 ** -11, 448.0, 464.0],
    ]).astype(np.float32)
    q = q[q <= 464.0]
    ours = F.e4m3_code_nearest(q.astype(np.float64), 1.0)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    assert F.e4m3_code_nearest(np.array([480.0, 1e6]), 1.0).tolist() == [0x7E, 0x7E]


def test_e4m3_rounding_of_quotients_brute_force():
    rng = np.random.default_rng(1)
    for _ in range(3000):
        a = np.float32(rng.choice([rng.uniform(0, 10), rng.uniform(0, 1e-3), 2688.0 * rng.uniform(0, 1)]))
        g = np.float32(np.exp(rng.uniform(-12, 2)))
        q = Fraction(float(a)) / (6 * Fraction(float(g)))
        ref = nearest_even(q, E4M3_TORCH) if q < 448 else 0x7E
        assert F.e4m3_code_nearest(np.array([a], np.float64), 6.0 * np.float64(g))[0] == ref


def test_e2m1_rounding_exhaustive_bf16_brute_force():
    """All 65536 bf16 inputs under several scales against exact nearest-of-levels."""
    bits = np.arange(65536, dtype=np.uint16)
    x = F.bf16_bits_to_f32(bits)
    finite = np.isfinite(x)
    x = x[finite]
    for S in [np.float32(1.0), np.float32(24.0), np.float32(0.375), np.float32(1.0 / 3.0)]:
        idx = F.e2m1_index_nearest(np.abs(x).astype(np.float64), np.float64(S))
        # brute force on a subset (all values near the codebook range) with Fractions
        sel = np.flatnonzero((np.abs(x) < 8 * S) & (np.abs(x) > 0.1 * S))
        for i in sel[:: max(1, sel.size // 4000)]:
            ref = nearest_even(abs(Fraction(float(x[i]))) / Fraction(float(S)), E2M1_PAGE)
            assert idx[i] == ref, (x[i], S)
        # ties: exact midpoints times S round to the even index
        for j, m in enumerate(F.E2M1_MIDPOINTS):
            t = np.float64(m) * np.float64(S)
            if np.float32(t) == t:
                got = F.e2m1_index_nearest(np.array([t]), np.float64(S))[0]
                assert got == (j if j % 2 == 0 else j + 1)


# ---------------------------------------------------------------------------
# scales and quantize
# ---------------------------------------------------------------------------

def test_global_scale_closed_forms():
    assert Q.global_scale(np.float32(2688.0)) == np.float32(1.0)
    assert Q.global_scale(np.float32(0.0)) == np.float32(1.0)
    rng = np.random.default_rng(2)
    for a in np.float32(np.exp(rng.uniform(-20, 20, 500))):
        assert Q.global_scale(a) == bf_fp32(Fraction(float(a)) / 2688)


def test_worked_example_rounding_boundary():
    """60.24 and 59.76 under a shared scale of 24 round to 3 and 2; the
    dequantized values differ by 24 (TRACE summary, research motivation)."""
    ex = GOLDEN["rounding_boundary_example"]
    x = np.zeros((2, 32), dtype=np.float32)
    x[0, 16] = x[1, 16] = 2688.0                       # g = 1
    x[0, 0] = x[1, 0] = np.float32(ex["implied_scale"] * 6)   # block amax 144 -> s = 24
    x[0, 1] = np.float32(ex["x_train"])
    x[1, 1] = np.float32(ex["x_rollout"])
    codes, scales, g = Q.quantize(x)
    assert g == 1.0
    assert F.E4M3_VALUES[scales[0, 0]] == ex["implied_scale"] and scales[0, 0] == 0x5C
    nib = Q.unpack_nibbles(codes)
    assert F.e2m1_decode(nib[0, 1]) == ex["code_train"]
    assert F.e2m1_decode(nib[1, 1]) == ex["code_rollout"]
    dq = Q.dequantize(codes, scales, g)
    assert dq[0, 1] - dq[1, 1] == ex["dequantized_difference"]
    assert round(float(x[0, 1]) / ex["implied_scale"], 2) == ex["scaled_train"]
    assert round(float(x[1, 1]) / ex["implied_scale"], 2) == ex["scaled_rollout"]
    # the bf16-rounded activations (60.25, 59.75) sit on the same sides
    xb = F.bf16_bits_to_f32(F.f32_to_bf16_bits(x))
    nb = Q.unpack_nibbles(Q.quantize(xb)[0])
    assert nb[0, 1] == 5 and nb[1, 1] == 4


def test_quantize_brute_force_tiny():
    rng = np.random.default_rng(3)
    for trial in range(12):
        x = (rng.standard_normal((3, 32)) * np.exp(rng.uniform(-3, 3))).astype(np.float32)
        if trial % 3 == 0:
            x[0, :16] = 0
            x[1, 3] = -0.0
        codes, scales, g = Q.quantize(x)
        amax = np.abs(x).max()
        assert g == (bf_fp32(Fraction(float(amax)) / 2688) if amax > 0 else 1.0)
        nib = Q.unpack_nibbles(codes)
        for r in range(3):
            for b in range(2):
                s_byte, cs = brute_quantize_block(x[r, 16 * b:16 * b + 16], g)
                assert scales[r, b] == s_byte
                assert list(nib[r, 16 * b:16 * b + 16]) == cs


def test_zero_tensor_and_signed_zero():
    x = np.zeros((2, 16), dtype=np.float32)
    x[1] = -0.0
    codes, scales, g = Q.quantize(x)
    assert g == 1.0 and np.all(scales == 0)
    nib = Q.unpack_nibbles(codes)
    assert np.all(nib[0] == 0) and np.all(nib[1] == 8)
    # a tiny negative value that rounds to zero keeps its sign
    y = np.zeros((1, 16), dtype=np.float32)
    y[0, 0] = 6.0
    y[0, 1] = -0.1
    assert Q.unpack_nibbles(Q.quantize(y)[0])[0, 1] == 0x8


def test_packing_and_storage_size():
    nib = np.arange(64, dtype=np.uint8).reshape(2, 32) % 16
    packed = Q.pack_nibbles(nib)
    assert packed.shape == (2, 16)
    assert packed[0, 0] == (nib[0, 0] | nib[0, 1] << 4)
    assert np.array_equal(Q.unpack_nibbles(packed), nib)
    # NVFP4 storage: K/2 code bytes + K/16 scale bytes per row = 4.5 bit/element;
    # a 1-bit record plus an amortized E4M3 scale per 16 values is 1.5 bit,
    # which gives the TRACE summary's 2048 x 20 x 1.5 = 61440 bit per token.
    k = 4096
    assert (k // 2 + k // 16) * 8 / k == 4.5
    rec = GOLDEN["record_arithmetic"]
    assert (1 + 8 / 16) == rec["bits_per_value"]
    assert rec["width"] * rec["layers"] * rec["bits_per_value"] == rec["bits_per_token"]


def test_residual_exact_and_code_zero():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 256)) * 3).astype(np.float32)
    x[:, 7] *= 40
    codes, scales, g = Q.quantize(x)
    r = Q.residual(x, codes, scales, g)            # asserts exactness itself
    nib = Q.unpack_nibbles(codes)
    zero = (nib & 7) == 0
    assert np.array_equal(r[zero], x[zero])
    # |R| is at most half a level spacing of the block scale, bounded by S_b
    S = np.repeat(Q.effective_scales(scales, g), 16, axis=1)
    assert np.all(np.abs(r) <= S * 1.0 + 1e-30)


def test_requantized_representable_input_gives_zero_residual():
    """A block whose values are exactly NVFP4 values (g = 1) quantizes to
    itself, so R = 0, r_global = 1 and all residual codes/scales are 0."""
    x = np.zeros((4, 32), dtype=np.float32)
    x[0, 0] = 2688.0
    lv = F.E2M1_LEVELS
    rng = np.random.default_rng(5)
    for r in range(4):
        for b in range(2):
            s = 448.0 if r == b == 0 else F.E4M3_VALUES[rng.integers(40, 100)]
            vals = rng.choice(lv, 16) * rng.choice([-1, 1], 16)
            vals[0] = 6.0                 # block amax 6 * s: the scale is s
            x[r, 16 * b:16 * b + 16] = vals * s
    codes, scales, g = Q.quantize(x)      # tensor amax 2688: g = 1
    assert g == 1.0
    assert np.array_equal(Q.dequantize(codes, scales, g), x)
    sel, rc, rs, rg = Q.resq_select_and_requant(x, codes, scales, g, [0, 4], 16)
    assert list(sel[0]) == list(range(16))      # all scores 0: lowest indices
    assert rg[0] == 1.0 and np.all(rs == 0) and np.all(rc == 0)


# ---------------------------------------------------------------------------
# scores and top-k
# ---------------------------------------------------------------------------

def test_channel_scores_order_and_value():
    rng = np.random.default_rng(6)
    a = np.abs(rng.standard_normal((300, 48))).astype(np.float32)
    s = Q.channel_scores(a)
    # the fixed order: sequential within 128-row tiles, then over tiles
    parts = [np.add.accumulate(a[t:t + 128], axis=0, dtype=np.float32)[-1] for t in range(0, 300, 128)]
    ref = np.add.accumulate(np.stack(parts), axis=0, dtype=np.float32)[-1]
    assert np.array_equal(s, ref)
    assert np.allclose(s, a.astype(np.float64).sum(axis=0), rtol=1e-5)
    b = np.abs(rng.standard_normal((100, 8))).astype(np.float32)
    assert np.array_equal(Q.channel_scores(b), np.add.accumulate(b, axis=0, dtype=np.float32)[-1])
    b[:, 3] = b[:, 5]
    sb = Q.channel_scores(b)
    assert sb[3] == sb[5]


def test_topk_brute_force_and_ties():
    rng = np.random.default_rng(7)
    for _ in range(200):
        kk = 32
        sc = rng.integers(0, 6, kk).astype(np.float32)      # many ties
        k = int(rng.integers(1, kk))
        ref = sorted(sorted(range(kk), key=lambda c: (-sc[c], c))[:k])
        assert list(Q.topk_channels(sc, k)) == ref
    assert list(Q.topk_channels(np.ones(64, np.float32), 16)) == list(range(16))


def test_resq_brute_force_small():
    """Selection by full sort of |R| sums and requantization of the compact residual."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((20, 64)).astype(np.float32)
    x[:, [3, 40]] *= 12
    codes, scales, g = Q.quantize(x)
    offs = [0, 5, 5, 20]                     # second unit empty
    rows = rng.permutation(20)
    sel, rc, rs, rg = Q.resq_select_and_requant(x, codes, scales, g, offs, 16, row_index=rows)
    dq = Q.dequantize(codes, scales, g).astype(np.float64)
    for u in range(3):
        a, b = offs[u], offs[u + 1]
        if a == b:
            assert rg[u] == 1.0
            continue
        absr = np.abs(x[rows[a:b]].astype(np.float64) - dq[rows[a:b]])
        tot = absr.sum(axis=0)
        ref = sorted(sorted(range(64), key=lambda c: (-tot[c], c))[:16])
        assert list(sel[u]) == ref
        rs_ref = (x[rows[a:b]].astype(np.float64) - dq[rows[a:b]])[:, ref].astype(np.float32)
        c2, s2, g2 = Q.quantize(rs_ref)
        assert rg[u] == g2 and np.array_equal(rc[a:b], c2) and np.array_equal(rs[a:b], s2)
    # the blocks holding an outlier channel carry the largest residuals
    assert np.mean((sel[2] < 16) | ((sel[2] >= 32) & (sel[2] < 48))) > 0.5


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def _exact_value_matrix(codes, scales, g):
    nib = Q.unpack_nibbles(codes)
    m, k = nib.shape
    S = Q.effective_scales(scales, g)
    return [[Fraction(float(F.e2m1_decode(nib[i, j]))) * Fraction(float(S[i, j // 16]))
             for j in range(k)] for i in range(m)]


def test_gemm_brute_force_tiny():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 32)).astype(np.float32)
    w = (rng.standard_normal((3, 32)) * 0.02).astype(np.float32)
    xc, xs, xg = Q.quantize(x)
    wc, ws, wg = Q.quantize(w)
    sel, rc, rs, rg = Q.resq_select_and_requant(x, xc, xs, xg, [0, 2], 16)
    y = G.gemm_comp(xc, xs, xg, wc, ws, wg, sel[0], rc, rs, rg[0])
    A = _exact_value_matrix(xc, xs, xg)
    W = _exact_value_matrix(wc, ws, wg)
    R = _exact_value_matrix(rc, rs, rg[0])
    for i in range(2):
        for n in range(3):
            ref = sum(A[i][j] * W[n][j] for j in range(32))
            ref += sum(R[i][j] * W[n][int(sel[0][j])] for j in range(16))
            assert abs(float(ref) - y[i, n]) <= 1e-6 * max(1.0, abs(float(ref)))
    y0 = G.gemm_comp(xc, xs, xg, wc, ws, wg)
    assert not np.allclose(y0, y, rtol=0, atol=0)


def test_compensation_linearity_identity():
    """Adding the correction to the output equals adding the scattered
    quantized residual to the quantized activation (QUADS section 2.2B says
    the correction is added back to the quantized output; the yfxerp digest
    says into the result)."""
    rng = np.random.default_rng(10)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    x[:, 9] *= 20
    w = (rng.standard_normal((24, 128)) * 0.02).astype(np.float32)
    xc, xs, xg = Q.quantize(x)
    wc, ws, wg = Q.quantize(w)
    sel, rc, rs, rg = Q.resq_select_and_requant(x, xc, xs, xg, [0, 16], 32)
    y = G.gemm_comp(xc, xs, xg, wc, ws, wg, sel[0], rc, rs, rg[0])
    xa = Q.dequantize(xc, xs, xg).astype(np.float64)
    xa[:, sel[0]] += Q.dequantize(rc, rs, rg[0]).astype(np.float64)
    y2 = xa @ Q.dequantize(wc, ws, wg).astype(np.float64).T
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-12)


def test_compensation_reduces_error_all_channels():
    """With every channel selected, the compensated output is closer to
    X @ DQ(W)^T than the uncompensated one (on several seeds)."""
    for seed in range(4):
        rng = np.random.default_rng(100 + seed)
        x = rng.standard_normal((32, 256)).astype(np.float32)
        x[:, rng.choice(256, 3, replace=False)] *= 16
        w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
        xc, xs, xg = Q.quantize(x)
        wc, ws, wg = Q.quantize(w)
        wd = Q.dequantize(wc, ws, wg).astype(np.float64)
        exact = x.astype(np.float64) @ wd.T
        err0 = np.linalg.norm(G.gemm_comp(xc, xs, xg, wc, ws, wg) - exact)
        errs = []
        for k in (32, 256):
            sel, rc, rs, rg = Q.resq_select_and_requant(x, xc, xs, xg, [0, 32], k)
            errs.append(np.linalg.norm(G.gemm_comp(xc, xs, xg, wc, ws, wg, sel[0], rc, rs, rg[0]) - exact))
        assert errs[1] < errs[0] < err0


# ---------------------------------------------------------------------------
# MoE layer
# ---------------------------------------------------------------------------

def _small_moe(seed, n_exp=4, tokens=24, hidden=64, inter=32, top_k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, hidden)).astype(np.float32)
    x[:, 5] *= 10
    wgu = (rng.standard_normal((n_exp, 2 * inter, hidden)) * 0.1).astype(np.float32)
    wd = (rng.standard_normal((n_exp, hidden, inter)) * 0.1).astype(np.float32)
    _, gc, gs, gg = Q.qdq_weights(wgu)
    _, dc, ds, dg = Q.qdq_weights(wd)
    logits = rng.standard_normal((tokens, n_exp))
    p = np.exp(logits) / np.exp(logits).sum(1, keepdims=True)
    top = np.argsort(-p, axis=1, kind="stable")[:, :top_k]
    tok = np.repeat(np.arange(tokens), top_k)
    ex = top.reshape(-1)
    order = np.lexsort((tok, ex))
    routing = dict(slot_token=tok[order], slot_weight=p[tok[order], ex[order]].astype(np.float32),
                   offsets=np.concatenate([[0], np.cumsum(np.bincount(ex, minlength=n_exp))]))
    return x, routing, (gc, gs, gg), (dc, ds, dg), top, p


def test_moe_single_expert_reduces_to_dense():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((10, 64)).astype(np.float32)
    wgu = (rng.standard_normal((1, 64, 64)) * 0.1).astype(np.float32)
    wd = (rng.standard_normal((1, 64, 32)) * 0.1).astype(np.float32)
    _, gc, gs, gg = Q.qdq_weights(wgu)
    _, dc, ds, dg = Q.qdq_weights(wd)
    routing = dict(slot_token=np.arange(10), slot_weight=np.ones(10, np.float32), offsets=[0, 10])
    st = G.moe_layer(x, routing, (gc, gs, gg), (dc, ds, dg), 16)
    xc, xs, xg = Q.quantize(x)
    sel, rc, rs, rg = Q.resq_select_and_requant(x, xc, xs, xg, [0, 10], 16)
    gu = G.gemm_comp(xc, xs, xg, gc[0], gs[0], gg[0], sel[0], rc, rs, rg[0])
    g, u = gu[:, :32], gu[:, 32:]
    h = F.f64_to_bf16_bits(g / (1 + np.exp(-g)) * u)
    assert np.array_equal(st["h"], h)
    h32 = F.bf16_bits_to_f32(h)
    hc, hs, hg = Q.quantize(h32)
    sel2, rc2, rs2, rg2 = Q.resq_select_and_requant(h32, hc, hs, hg, [0, 10], 16)
    y = G.gemm_comp(hc, hs, hg, dc[0], ds[0], dg[0], sel2[0], rc2, rs2, rg2[0])
    assert np.allclose(st["y"], y, rtol=1e-12, atol=1e-12)


def test_moe_expert_permutation_invariance():
    x, routing, wgu, wd, top, p = _small_moe(12)
    st = G.moe_layer(x, routing, wgu, wd, 16)
    n_exp = len(routing["offsets"]) - 1
    perm = np.random.default_rng(0).permutation(n_exp)          # new id of each expert
    inv = np.argsort(perm)
    wgu_p = tuple(a[inv] for a in wgu)
    wd_p = tuple(a[inv] for a in wd)
    tokens = x.shape[0]
    tok = np.repeat(np.arange(tokens), top.shape[1])
    ex = perm[top.reshape(-1)]
    order = np.lexsort((tok, ex))
    routing_p = dict(slot_token=tok[order], slot_weight=p[tok[order], inv[ex[order]]].astype(np.float32),
                     offsets=np.concatenate([[0], np.cumsum(np.bincount(ex, minlength=n_exp))]))
    st_p = G.moe_layer(x, routing_p, wgu_p, wd_p, 16)
    assert np.allclose(st["y"], st_p["y"], rtol=1e-12, atol=1e-12)


def test_silu_swiglu_closed_form():
    z = np.array([0.0, 1.0, -1.0, 20.0])
    assert np.allclose(G.silu(z), [0.0, 1 / (1 + np.exp(-1)), -1 / (1 + np.exp(1)), 20 / (1 + np.exp(-20))])
    gu = np.array([[0.0, 2.0, 3.0, 5.0]])
    h = F.bf16_bits_to_f32(G.swiglu_bf16(gu, 2))
    assert h[0, 0] == 0.0 and abs(h[0, 1] - 2 / (1 + np.exp(-2)) * 5) < 2 ** -6 * 8


def test_bf16_rounding_helpers():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 60.24, -59.76, 2 ** -130], dtype=np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.uint16).numpy()
    assert np.array_equal(F.f32_to_bf16_bits(x.astype(np.float32)), ref)
    assert np.array_equal(F.f64_to_bf16_bits(x), ref)
    # double rounding case: 1 + 2^-8 + 2^-30 must round up once from float64
    y = np.array([1.0 + 2 ** -8 + 2 ** -30])
    assert F.bf16_bits_to_f32(F.f64_to_bf16_bits(y))[0] == np.float32(1.0 + 2 ** -7)


# ---------------------------------------------------------------------------
# trainer side
# ---------------------------------------------------------------------------

def test_qdq_representable_is_identity_and_brute_force():
    rng = np.random.default_rng(13)
    w = np.zeros((2, 4, 32), dtype=np.float32)
    for i in range(2):
        for r in range(4):
            for b in range(2):
                s = 448.0 if r == b == 0 else F.E4M3_VALUES[rng.integers(30, 110)]
                v = rng.choice(F.E2M1_LEVELS, 16) * rng.choice([-1, 1], 16)
                v[0] = 6.0
                w[i, r, 16 * b:16 * b + 16] = v * s
    w = F.bf16_bits_to_f32(F.f32_to_bf16_bits(w))   # values already bf16-exact
    out, codes, scales, g = Q.qdq_weights(w)
    assert np.all(g == 1.0)
    assert np.array_equal(F.bf16_bits_to_f32(out), w)
    wr = (rng.standard_normal((1, 2, 32)) * 0.02).astype(np.float32)
    out, codes, scales, g = Q.qdq_weights(wr)
    for r in range(2):
        for b in range(2):
            s_byte, cs = brute_quantize_block(wr[0, r, 16 * b:16 * b + 16], g[0])
            S = bf_fp32(E4M3_TORCH[s_byte] * Fraction(float(g[0])))
            for j, c in enumerate(cs):
                v = bf_fp32(Fraction(float(F.e2m1_decode(c))) * Fraction(float(S)))
                if c == 0x8:
                    v = np.float32(-0.0)          # IEEE: -0 times a scale is -0
                ref = F.f32_to_bf16_bits(np.array([v], np.float32))[0]
                assert out[0, r, 16 * b + j] == ref


def _guided_brute(xt, roll_nib, S):
    """Exact guided rounding of one element (rationals)."""
    levels = sorted(set([-v for v in E2M1_PAGE] + E2M1_PAGE))
    if S == 0:
        return (8 if np.signbit(np.float32(xt)) else 0)
    v = Fraction(float(xt)) / Fraction(float(S))
    lo = max([l for l in levels if l <= v], default=levels[0])
    hi = min([l for l in levels if l >= v], default=levels[-1])
    qr = Fraction(float(F.e2m1_decode(roll_nib)))
    q = hi if abs(hi - qr) < abs(lo - qr) else lo
    neg = q < 0 or (q == 0 and np.signbit(np.float32(xt)))
    return (8 if neg else 0) | E2M1_PAGE.index(abs(q))


def test_guided_worked_example():
    """TRACE research motivation: trainer 60.24 vs rollout 59.76 under scale
    24.  Round-to-nearest gives 3 vs 2; guided rounding picks the rollout's 2."""
    ex = GOLDEN["rounding_boundary_example"]
    xr = np.zeros((1, 32), np.float32)
    xr[0, 16] = 2688.0
    xr[0, 0] = 144.0
    xr[0, 1] = ex["x_rollout"]
    xt = xr.copy()
    xt[0, 1] = ex["x_train"]
    rc, rs, rg = Q.quantize(xr)
    gc, fq, hist = Q.guided_round(xt, rc, rs, rg)
    tc = Q.unpack_nibbles(Q.quantize(xt)[0])
    assert F.e2m1_decode(tc[0, 1]) == ex["code_train"]              # RTN: 3
    assert F.e2m1_decode(Q.unpack_nibbles(gc)[0, 1]) == ex["code_rollout"]  # guided: 2
    assert F.bf16_bits_to_f32(fq)[0, 1] == 48.0
    assert hist.tolist() == [31, 1, 0]


def test_guided_invariant_and_brute_force():
    rng = np.random.default_rng(14)
    xr = (rng.standard_normal((64, 64)) * 2).astype(np.float32)
    xr[:, 7] *= 30
    rc, rs, rg = Q.quantize(xr)
    for rel in (1e-3, 8e-3, 0.1):
        xt = (xr + rng.standard_normal(xr.shape).astype(np.float32) * rel * np.abs(xr)).astype(np.float32)
        gc, fq, hist = Q.guided_round(xt, rc, rs, rg)
        S = np.repeat(Q.effective_scales(rs, rg), 16, axis=1)
        rtn = F.e2m1_index_nearest(np.abs(xt).astype(np.float64), S.astype(np.float64))
        rtn_s = np.where(np.signbit(xt), -rtn, rtn)
        g_s = Q.signed_index(Q.unpack_nibbles(gc))
        r_s = Q.signed_index(Q.unpack_nibbles(rc))
        lv = np.concatenate([-F.E2M1_LEVELS[:0:-1], F.E2M1_LEVELS])
        val = lambda si: lv[si + 7]
        # TRACE Eq. (3): never farther from the rollout level than RTN
        assert np.all(np.abs(val(g_s) - val(r_s)) <= np.abs(val(rtn_s) - val(r_s)))
        assert np.all(np.abs(g_s - rtn_s) <= 1)
        assert hist.sum() == xt.size
        gn = Q.unpack_nibbles(gc)
        rn = Q.unpack_nibbles(rc)
        for (i, j) in zip(rng.integers(0, 64, 300), rng.integers(0, 64, 300)):
            assert gn[i, j] == _guided_brute(xt[i, j], rn[i, j], S[i, j])
    # identical trainer input: guided == RTN == rollout codes
    gc, _, hist = Q.guided_round(xr, rc, rs, rg)
    assert np.array_equal(gc, rc) and hist[1] == 0 and hist[2] == 0


# ---------------------------------------------------------------------------
# mantissa-only guidance record
# ---------------------------------------------------------------------------

def test_guidance_record_layout_and_size():
    """One bit per element (the low code bit), element 8i + j in bit j of
    byte i; with the block scales that is the TRACE summary's 1.5 bits per
    value: 61440 bits (7.5 KB) per token for 2048 values x 20 layers, about 6x
    less than the full 4.5-bit codes and scales of all 40 layers (about 50 KB)."""
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, (5, 48), dtype=np.uint8)
    rec = Q.guidance_record(codes)
    nib = Q.unpack_nibbles(codes)
    assert rec.shape == (5, 12)
    for r in range(5):
        for e in range(96):
            assert (rec[r, e // 8] >> (e % 8)) & 1 == nib[r, e] & 1
    k = 4096
    assert (k // 8 + k // 16) * 8 / k == GOLDEN["record_arithmetic"]["bits_per_value"]
    cmp = GOLDEN["record_compression"]
    width = GOLDEN["record_arithmetic"]["width"]
    rec_bytes = width * cmp["layers_kept"] * 1.5 / 8
    full_bytes = width * cmp["layers_all"] * 4.5 / 8
    assert rec_bytes * 8 == GOLDEN["record_arithmetic"]["bits_per_token"]
    assert rec_bytes / 1024 == cmp["record_kb_per_token_about"]
    assert abs(full_bytes / 1024 - cmp["full_kb_per_token_about"]) / cmp["full_kb_per_token_about"] < 0.15
    assert round(full_bytes / rec_bytes) == cmp["compression_about"]


def _guided_record_brute(xt, bit, S):
    """Exact guided rounding of one element from the record bit (rationals)."""
    levels = sorted(set([-v for v in E2M1_PAGE] + E2M1_PAGE))
    if S == 0:
        return (8 if np.signbit(np.float32(xt)) else 0)
    v = Fraction(float(xt)) / Fraction(float(S))
    lo = max([l for l in levels if l <= v], default=levels[0])
    hi = min([l for l in levels if l >= v], default=levels[-1])
    q = hi if E2M1_PAGE.index(abs(hi)) % 2 == bit else lo
    neg = q < 0 or (q == 0 and np.signbit(np.float32(xt)))
    return (8 if neg else 0) | E2M1_PAGE.index(abs(q))


def test_guided_record_worked_example():
    """TRACE research motivation: the rollout's 59.76 rounds to 2 (index 4,
    low bit 0) under scale 24; the trainer's 60.24 has candidates 2 and 3,
    and the record bit picks 2 where round-to-nearest gives 3."""
    ex = GOLDEN["rounding_boundary_example"]
    xr = np.zeros((1, 32), np.float32)
    xr[0, 16] = 2688.0
    xr[0, 0] = 144.0
    xr[0, 1] = ex["x_rollout"]
    xt = xr.copy()
    xt[0, 1] = ex["x_train"]
    rc, rs, rg = Q.quantize(xr)
    rec = Q.guidance_record(rc)
    assert (rec[0, 0] >> 1) & 1 == 0
    gc, fq, moved = Q.guided_round_record(xt, rec, rs, rg)
    assert F.e2m1_decode(Q.unpack_nibbles(gc)[0, 1]) == ex["code_rollout"]
    assert F.bf16_bits_to_f32(fq)[0, 1] == 48.0
    assert moved.tolist() == [31, 1]


def test_guided_record_brute_force_and_agreement():
    """Brute force on sampled elements; the output is always q- or q+ (one
    code from round-to-nearest at most); wherever the rollout level is one of
    the candidates it equals full-code guided rounding; identical inputs give
    the rollout codes back."""
    rng = np.random.default_rng(15)
    xr = (rng.standard_normal((64, 64)) * 2).astype(np.float32)
    xr[:, 9] *= 30
    rc, rs, rg = Q.quantize(xr)
    rec = Q.guidance_record(rc)
    S = np.repeat(Q.effective_scales(rs, rg), 16, axis=1)
    levels = sorted(set([-v for v in E2M1_PAGE] + E2M1_PAGE))
    for rel in (1e-3, 8e-3, 0.1):
        xt = (xr + rng.standard_normal(xr.shape).astype(np.float32) * rel * np.abs(xr)).astype(np.float32)
        gc, fq, moved = Q.guided_round_record(xt, rec, rs, rg)
        gfull, _, _ = Q.guided_round(xt, rc, rs, rg)
        gn, fn, rn = Q.unpack_nibbles(gc), Q.unpack_nibbles(gfull), Q.unpack_nibbles(rc)
        rtn = F.e2m1_index_nearest(np.abs(xt).astype(np.float64), S.astype(np.float64))
        rtn_s = np.where(np.signbit(xt), -rtn, rtn)
        assert np.all(np.abs(Q.signed_index(gn) - rtn_s) <= 1)
        assert moved.sum() == xt.size and moved[1] == np.sum(Q.signed_index(gn) != rtn_s)
        agree = 0
        for (i, j) in zip(rng.integers(0, 64, 400), rng.integers(0, 64, 400)):
            bit = (rec[i, j // 8] >> (j % 8)) & 1
            assert gn[i, j] == _guided_record_brute(xt[i, j], bit, S[i, j])
            v = Fraction(float(xt[i, j])) / Fraction(float(S[i, j]))
            lo = max([l for l in levels if l <= v], default=levels[0])
            hi = min([l for l in levels if l >= v], default=levels[-1])
            if Fraction(float(F.e2m1_decode(rn[i, j]))) in (lo, hi):
                assert gn[i, j] == fn[i, j]
                agree += 1
        assert agree > 300
    gc, _, moved = Q.guided_round_record(xr, rec, rs, rg)
    assert np.array_equal(gc, rc) and moved[1] == 0
