"""Pin of the oracle's MoE combine: every slot's down-projection row is
weighted by its gate weight p and the rows of a token are summed,
y[t] = sum over t's slots of p * Down_e(h_slot).

TRACE summary, "Prerequisites" (MoE routing: the router sends each token to
a few experts whose outputs are mixed by the gate); the gate weight is read
as the softmax probability over all experts at each chosen expert, not
renormalised over the token's top-k.

The reference here is exact rational arithmetic over operands decoded
independently of the oracle (a literal E2M1 table and torch's E4M3 decoder),
on a tiny layer with gate weights that are distinct, not 1, and whose sum
over a token's slots is below 1.  Dropping, squaring or renormalising the
gate weight, or adding a slot into the wrong token, fails it.  No GPU.
"""

from fractions import Fraction

import numpy as np
import torch

from oracle import gemm as G
from oracle import nvfp4 as Q

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _decode(codes, scales, g):
    """Exact values of an NVFP4 tensor as Fractions: the effective block
    scale is the fp32 product of the E4M3 byte's value and g, and the element
    times it is rounded once to fp32 (the decode rule of the TRACE
    prerequisites: block scale, then global scale, fp32 arithmetic)."""
    m, kh = codes.shape
    sc = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn).double().numpy()
    out = [[Fraction(0)] * (2 * kh) for _ in range(m)]
    for i in range(m):
        for j in range(2 * kh):
            nib = (int(codes[i, j // 2]) >> (4 * (j % 2))) & 15
            v = E2M1[nib & 7] * (-1.0 if nib & 8 else 1.0)
            eff = np.float32(sc[i, j // 16] * np.float32(g))
            out[i][j] = Fraction(float(np.float32(v * float(eff))))
    return out


def _tiny_layer(seed=21, tokens=3, experts=3, top_k=2, inter=32, hidden=16, k=16):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((tokens, experts)) * 1.5
    prob = np.exp(logits) / np.exp(logits).sum(1, keepdims=True)
    top = np.argsort(-prob, axis=1, kind="stable")[:, :top_k]
    tok = np.repeat(np.arange(tokens), top_k)
    ex = top.reshape(-1)
    order = np.lexsort((tok, ex))                     # slots sorted by (expert, token)
    slot_token = tok[order]
    slot_expert = ex[order]
    slot_weight = prob[slot_token, slot_expert].astype(np.float32)
    offsets = np.concatenate([[0], np.cumsum(np.bincount(ex, minlength=experts))]).astype(np.int64)
    h = rng.standard_normal((tokens * top_k, inter)).astype(np.float32)
    h[:, 3] *= 9.0                                    # a channel with a large residual
    wd = (rng.standard_normal((experts, hidden, inter)) * 0.05).astype(np.float32)
    return dict(slot_token=slot_token, slot_expert=slot_expert, slot_weight=slot_weight,
                offsets=offsets, h=h, wd=wd, tokens=tokens, k=k)


def _exact_down(L, hc, hs, hg, dc, ds, dg, sel, rc, rs, rg, weight_fn):
    """y[t][n] as Fractions: sum over t's slots of weight_fn(slot) times the
    slot's compensated down-projection row."""
    tokens, hidden = L["tokens"], dc.shape[1]
    a = _decode(hc, hs, hg)
    y = [[Fraction(0)] * hidden for _ in range(tokens)]
    offs = L["offsets"]
    for e in range(len(offs) - 1):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        w = _decode(dc[e], ds[e], dg[e])
        r = _decode(rc[lo:hi], rs[lo:hi], rg[e])      # the unit's own g_R
        for s in range(lo, hi):
            t = int(L["slot_token"][s])
            for n in range(hidden):
                acc = sum(a[s][c] * w[n][c] for c in range(len(a[s])))
                acc += sum(r[s - lo][j] * w[n][int(sel[e][j])] for j in range(len(sel[e])))
                y[t][n] += weight_fn(s) * acc
    return y


def test_moe_down_gate_weight_exact():
    L = _tiny_layer()
    hc, hs, hg = Q.quantize(L["h"])
    sel, rc, rs, rg = Q.resq_select_and_requant(L["h"], hc, hs, hg, L["offsets"], L["k"])
    dc, ds, dg = [], [], []
    for e in range(L["wd"].shape[0]):
        c, s, g = Q.quantize(L["wd"][e])
        dc.append(c), ds.append(s), dg.append(g)
    dc, ds, dg = np.stack(dc), np.stack(ds), np.array(dg, dtype=np.float32)
    p = L["slot_weight"]
    assert len(set(p.tolist())) == len(p) and np.all(p < 1.0) and np.all(p > 0.0)
    tok_sum = np.bincount(L["slot_token"], weights=p.astype(np.float64))
    assert np.all(tok_sum < 0.999)                    # renormalising would change y

    y = G.moe_down(hc, hs, hg, L["offsets"], dc, ds, dg, L["slot_token"], p, L["tokens"],
                   sel_idx=sel, r_codes=rc, r_scales=rs, r_g=rg)
    fp = lambda s: Fraction(float(p[s]))
    ref = _exact_down(L, hc, hs, hg, dc, ds, dg, sel, rc, rs, rg, fp)
    ref_f = np.array([[float(v) for v in row] for row in ref])
    scale = np.abs(ref_f).max()
    assert scale > 0
    np.testing.assert_allclose(y, ref_f, rtol=0, atol=1e-12 * scale)

    # the pin is sensitive to the plausible mistakes in the weighting
    wrong = {
        "no gate weight": lambda s: Fraction(1),
        "squared gate weight": lambda s: fp(s) * fp(s),
        "renormalised gate weight": lambda s: fp(s) / Fraction(float(tok_sum[L["slot_token"][s]])),
    }
    for name, fn in wrong.items():
        alt = np.array([[float(v) for v in row] for row in
                        _exact_down(L, hc, hs, hg, dc, ds, dg, sel, rc, rs, rg, fn)])
        assert np.abs(alt - ref_f).max() > 1e-3 * scale, name


def test_moe_down_slot_goes_to_its_token():
    """Moving one slot's row to another token changes y there by exactly
    p * row (the oracle adds each slot into slot_token's row only)."""
    L = _tiny_layer(seed=22)
    hc, hs, hg = Q.quantize(L["h"])
    dc, ds, dg = [], [], []
    for e in range(L["wd"].shape[0]):
        c, s, g = Q.quantize(L["wd"][e])
        dc.append(c), ds.append(s), dg.append(g)
    dc, ds, dg = np.stack(dc), np.stack(ds), np.array(dg, dtype=np.float32)
    p = L["slot_weight"]
    y = G.moe_down(hc, hs, hg, L["offsets"], dc, ds, dg, L["slot_token"], p, L["tokens"])
    zero = np.zeros_like(p)
    for s in range(len(p)):
        only = zero.copy()
        only[s] = p[s]
        y_s = G.moe_down(hc, hs, hg, L["offsets"], dc, ds, dg, L["slot_token"], only, L["tokens"])
        t = int(L["slot_token"][s])
        others = np.delete(np.arange(L["tokens"]), t)
        assert np.all(y_s[others] == 0.0) and np.any(y_s[t] != 0.0)
    # summing the single-slot layers gives the layer (linearity in p)
    total = sum(G.moe_down(hc, hs, hg, L["offsets"], dc, ds, dg, L["slot_token"],
                           np.where(np.arange(len(p)) == s, p, 0).astype(np.float32), L["tokens"])
                for s in range(len(p)))
    np.testing.assert_allclose(total, y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
