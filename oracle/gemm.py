"""Compensated W4A4 GEMM and the MoE FFN layer: plain CPU definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The reference result of a GEMM is the float64 product of the dequantized
operands (numpy matmul as the library primitive); fp32-accumulating kernels
are compared against it with a relative tolerance.
"""

import numpy as np

from .formats import f64_to_bf16_bits, bf16_bits_to_f32
from .nvfp4 import dequantize, quantize, resq_select_and_requant


def gemm_comp(a_codes, a_scales, a_g, w_codes, w_scales, w_g,
              sel_idx=None, r_codes=None, r_scales=None, r_g=None):
    """Y = DQ(A) DQ(W)^T + DQ(R_S) DQ(W)[:, S]^T, in float64.

    QUADS section 2.2B: the FP4 GEMM over the quantized activation, plus the
    residual correction of the selected channels added back into the result
    (the yfxerp digest says the second FP4 quantization is added back into
    the result).  Reading of the weight side of the correction: the stored
    NVFP4 weight restricted to the selected input channels (each element keeps
    its block scale and the matrix's global scale), so that the correction
    equals quantizing (Q(X) + scatter(Q(R_S))) against the same weights.

    a_*: [M, K] activation codes/scales and fp32 global scale.
    w_*: [N, K] weight codes/scales and global scale.
    sel_idx: [k] selected channels (ascending) or None for no compensation;
    r_*: [M, k] requantized compact residual and its global scale.
    Returns Y [M, N] float64.
    """
    a = dequantize(a_codes, a_scales, a_g).astype(np.float64)
    w = dequantize(w_codes, w_scales, w_g).astype(np.float64)
    y = a @ w.T
    if sel_idx is not None:
        r = dequantize(r_codes, r_scales, r_g).astype(np.float64)
        y = y + r @ w[:, np.asarray(sel_idx, dtype=np.int64)].T
    return y



def gemm_masked_comp(a_codes, a_scales, a_g, w_codes, w_scales, w_g, m_codes, m_scales, m_g):
    """Y = DQ(A) DQ(W)^T + DQ(Q(R * M)) DQ(W)^T in float64: the dense-mask
    compensation of QUADS section 2.2B as a second GEMM of the same shape over
    the masked, requantized residual (m_* [M, K] from
    nvfp4.resq_mask_select_and_requant, global scale m_g)."""
    w = dequantize(w_codes, w_scales, w_g).astype(np.float64)
    a = dequantize(a_codes, a_scales, a_g).astype(np.float64)
    m = dequantize(m_codes, m_scales, m_g).astype(np.float64)
    return a @ w.T + m @ w.T


def silu(z):
    """z / (1 + exp(-z)) in float64 (SwiGLU gate activation)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu_bf16(gu, inter):
    """h = bf16(silu(G) * U) for gate/up output gu [rows, 2*inter]: columns
    0..inter-1 are the gate G, inter..2*inter-1 the up projection U
    (reading of the SwiGLU layout, which the pages leave open).  Rounded
    once from float64 to bf16.  Returns bf16 bit patterns [rows, inter]."""
    g = gu[:, :inter]
    u = gu[:, inter:2 * inter]
    return f64_to_bf16_bits(silu(g) * u)


def moe_gate_up(x_codes, x_scales, x_g, slot_token, offsets,
                wgu_codes, wgu_scales, wgu_g, inter,
                sel_idx=None, r_codes=None, r_scales=None, r_g=None):
    """Gate/up projection of every routed slot, one expert at a time.

    The activation is quantized once as a tensor before routing; expert e's
    rows are the tokens of slots offsets[e]..offsets[e+1]-1 (slot_token maps
    a slot to its token).  Returns (gu float64 [slots, 2*inter],
    h bf16 bits [slots, inter]).
    """
    slots = int(offsets[-1])
    gu = np.zeros((slots, 2 * inter), dtype=np.float64)
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        rows = np.asarray(slot_token[a:b], dtype=np.int64)
        comp = {} if sel_idx is None else dict(
            sel_idx=sel_idx[e], r_codes=r_codes[a:b], r_scales=r_scales[a:b], r_g=r_g[e])
        gu[a:b] = gemm_comp(x_codes[rows], x_scales[rows], x_g,
                            wgu_codes[e], wgu_scales[e], wgu_g[e], **comp)
    return gu, swiglu_bf16(gu, inter)


def moe_down(h_codes, h_scales, h_g, offsets, wd_codes, wd_scales, wd_g,
             slot_token, slot_weight, n_tokens,
             sel_idx=None, r_codes=None, r_scales=None, r_g=None):
    """Down projection of every slot, weighted by its gate weight and summed
    per token: y[t] = sum over t's slots of p_slot * Down_e(h_slot).
    Returns y float64 [n_tokens, H]."""
    hidden = wd_codes.shape[1]
    y = np.zeros((n_tokens, hidden), dtype=np.float64)
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        comp = {} if sel_idx is None else dict(
            sel_idx=sel_idx[e], r_codes=r_codes[a:b], r_scales=r_scales[a:b], r_g=r_g[e])
        out = gemm_comp(h_codes[a:b], h_scales[a:b], h_g,
                        wd_codes[e], wd_scales[e], wd_g[e], **comp)
        out = out * np.asarray(slot_weight[a:b], dtype=np.float64)[:, None]
        np.add.at(y, np.asarray(slot_token[a:b], dtype=np.int64), out)
    return y


def moe_layer(x, routing, w_gu, w_d, k, compensate=True):
    """The rollout-side MoE FFN layer with residual activation compensation,
    every stage computed by the oracle (used on small shapes).

    x: [T, H] fp32 values (bf16 inputs).  routing: dict with slot_token,
    offsets, slot_weight (sorted slot order).  w_gu = (codes [E, 2I, H/2],
    scales, g [E]); w_d = (codes [E, H, I/2], scales, g [E]).
    Returns a dict of every stage's result.
    """
    slot_token = routing["slot_token"]
    offsets = routing["offsets"]
    inter = w_gu[0].shape[1] // 2
    xc, xs, xg = quantize(x)
    st = dict(x_codes=xc, x_scales=xs, x_g=xg)
    comp1 = {}
    if compensate:
        sel1, rc1, rs1, rg1 = resq_select_and_requant(x, xc, xs, xg, offsets, k, row_index=slot_token)
        comp1 = dict(sel_idx=sel1, r_codes=rc1, r_scales=rs1, r_g=rg1)
        st.update(sel1=sel1, rc1=rc1, rs1=rs1, rg1=rg1)
    gu, h = moe_gate_up(xc, xs, xg, slot_token, offsets, *w_gu, inter, **comp1)
    h32 = bf16_bits_to_f32(h)
    hc, hs, hg = quantize(h32)
    st.update(gu=gu, h=h, h_codes=hc, h_scales=hs, h_g=hg)
    comp2 = {}
    if compensate:
        sel2, rc2, rs2, rg2 = resq_select_and_requant(h32, hc, hs, hg, offsets, k)
        comp2 = dict(sel_idx=sel2, r_codes=rc2, r_scales=rs2, r_g=rg2)
        st.update(sel2=sel2, rc2=rc2, rs2=rs2, rg2=rg2)
    y = moe_down(hc, hs, hg, offsets, *w_d, slot_token, routing["slot_weight"], x.shape[0], **comp2)
    st["y"] = y
    return st
