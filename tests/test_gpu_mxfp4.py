"""GPU parity of the MXFP4 variant: the HIP library (through its C ABI)
against the MXFP4 oracle on identical seeded inputs.

Bar: codes, E8M0 scales, tile partials, selected channels and requantized
residuals bit-exact; GEMM outputs within max|Y_gpu - Y_ref| / max|Y_ref| <=
1e-3 per output tensor (per expert for grouped GEMMs) against the float64
product of the same quantized operands.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import mxfp4 as MX
from oracle import nvfp4 as OQ

pytestmark = pytest.mark.gpu

GEMM_TOL = 1e-3


def np32(t):
    return t.detach().float().cpu().numpy()


def npu8(t):
    return t.detach().cpu().numpy()


def rel_err(y, ref):
    den = np.abs(ref).max()
    return float(np.abs(y - ref).max() / (den if den > 0 else 1.0))


# ---------------------------------------------------------------------------
# quantize
# ---------------------------------------------------------------------------

def test_mx_quantize_exhaustive_bf16(gpu_lib):
    """Every finite bf16 value in blocks of mixed magnitudes, and every value
    again in blocks whose scale is fixed (amax 6 * 2^X) so that each one is
    rounded at X = 0, 9 and -20, ties included."""
    P = gpu_lib
    bits = np.arange(65536, dtype=np.uint16)
    vals = F.bf16_bits_to_f32(bits)
    vals = vals[np.isfinite(vals)]
    rng = np.random.default_rng(0)
    mixed = np.concatenate([vals, np.zeros((-vals.size) % 128, np.float32)])
    x_np = mixed[rng.permutation(mixed.size)].reshape(-1, 128)
    codes, scales, _ = P.mxfp4_quantize(torch.from_numpy(x_np).to(torch.bfloat16).cuda())
    c_ref, s_ref = MX.quantize(x_np)
    assert np.array_equal(npu8(scales), s_ref)
    assert np.array_equal(npu8(codes), c_ref)
    for X in (0, 9, -20):
        d = np.float32(2.0 ** X)
        v = vals[np.abs(vals.astype(np.float64)) < 6.0 * 2.0 ** X]
        n = (v.size + 30) // 31 * 31
        blocks = np.zeros((n // 31, 32), np.float32)
        blocks[:, 0] = 6 * d
        blocks[:, 1:] = np.pad(v, (0, n - v.size)).reshape(-1, 31)
        blocks = np.concatenate([blocks, np.zeros(((-blocks.shape[0]) % 4, 32), np.float32)])
        xb = blocks.reshape(-1, 128)
        codes, scales, _ = P.mxfp4_quantize(torch.from_numpy(xb).to(torch.bfloat16).cuda())
        c_ref, s_ref = MX.quantize(xb)
        assert np.array_equal(npu8(scales), s_ref), f"X={X}"
        assert np.array_equal(npu8(codes), c_ref), f"X={X}"


def test_mx_quantize_scale_boundaries(gpu_lib):
    """Block maxima on and one fp32 ulp either side of every power of two the
    shared exponent changes at, from the subnormal range to 2^127, in fp32."""
    P = gpu_lib
    p2 = np.ldexp(np.float32(1.0), np.arange(-149, 128)).astype(np.float32)
    amax = np.concatenate([p2, np.nextafter(p2, np.float32(0)), np.nextafter(p2, np.float32(np.inf))])
    amax = amax[np.isfinite(amax) & (amax > 0)]
    amax = np.concatenate([amax, np.zeros((-amax.size) % 4, np.float32)])
    rng = np.random.default_rng(4)
    x = (amax[:, None] * rng.uniform(-1, 1, (amax.size, 32))).astype(np.float32)
    x[:, 5] = amax
    x_np = x.reshape(-1, 128)
    codes, scales, _ = P.mxfp4_quantize(torch.from_numpy(x_np).cuda())
    c_ref, s_ref = MX.quantize(x_np)
    assert np.array_equal(npu8(scales), s_ref)
    assert np.array_equal(npu8(codes), c_ref)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("m,k", [(128, 512), (300, 4096), (1, 32), (7, 96)])
def test_mx_quantize_random_with_tile_partials(gpu_lib, dtype, m, k):
    P = gpu_lib
    x = synth.activations(m, k, seed=5, heavy_frac=0.01).to(dtype)
    if dtype == torch.float32:
        x = x + torch.randn(x.shape, generator=torch.Generator().manual_seed(1)) * 1e-3
    x_np = x.float().numpy()
    codes, scales, tp = P.mxfp4_quantize(x.cuda(), tile_partials=True)
    c_ref, s_ref = MX.quantize(x_np)
    assert np.array_equal(npu8(scales), s_ref)
    assert np.array_equal(npu8(codes), c_ref)
    r = np.abs(MX.residual(x_np, c_ref, s_ref))
    tp_ref = np.stack([OQ.channel_scores(r[t:t + 128]) for t in range(0, m, 128)])
    assert np.array_equal(np32(tp), tp_ref)


# ---------------------------------------------------------------------------
# residual selection
# ---------------------------------------------------------------------------

def test_mx_resq_tile_units(gpu_lib):
    """Units = 128-token tiles with the quantizer's fused tile partials."""
    P = gpu_lib
    x = synth.activations(300, 1024, seed=7, heavy_frac=0.01)
    xc = x.cuda()
    codes, scales, tp = P.mxfp4_quantize(xc, tile_partials=True)
    sel, rc, rs = P.mxfp4_resq_select_and_requant(xc, codes, scales, 128, tile_partials=tp)
    x_np = x.float().numpy()
    c_ref, s_ref = MX.quantize(x_np)
    offs = [0, 128, 256, 300]
    sel_r, rc_r, rs_r = MX.resq_select_and_requant(x_np, c_ref, s_ref, offs, 128)
    assert np.array_equal(npu8(sel), sel_r)
    assert np.array_equal(npu8(rs), rs_r)
    assert np.array_equal(npu8(rc), rc_r)


@pytest.mark.parametrize("k", [32, 64])
def test_mx_resq_gathered_expert_units(gpu_lib, k):
    """Units = experts' routed tokens through the slot->token map, with skewed
    loads, an empty expert and units longer than one 128-row tile."""
    P = gpu_lib
    tokens, hidden, n_exp = 400, 256, 6
    x = synth.activations(tokens, hidden, seed=8, heavy_frac=0.02)
    rt = synth.route(tokens, n_exp, seed=8, top_k=2, zipf_s=1.5)
    offs = rt["offsets"].copy()
    offs[4] = offs[3]
    xc = x.cuda()
    codes, scales, _ = P.mxfp4_quantize(xc)
    sel, rc, rs = P.mxfp4_resq_select_and_requant(
        xc, codes, scales, k, unit_offsets=torch.from_numpy(offs).cuda(), rows_total=int(offs[-1]),
        row_index=torch.from_numpy(rt["slot_token"]).cuda())
    x_np = x.float().numpy()
    c_ref, s_ref = MX.quantize(x_np)
    sel_r, rc_r, rs_r = MX.resq_select_and_requant(x_np, c_ref, s_ref, offs, k,
                                                   row_index=rt["slot_token"])
    assert np.diff(offs).max() > 128
    assert np.array_equal(npu8(sel), sel_r)
    assert np.array_equal(npu8(rs), rs_r)
    assert np.array_equal(npu8(rc), rc_r)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def _mx_weights(P, w):
    """MXFP4 codes and scales of w [E, N, K] (each row independently)."""
    e, n, k = w.shape
    c, s, _ = P.mxfp4_quantize(w.reshape(e * n, k).cuda())
    return c.reshape(e, n, k // 2), s.reshape(e, n, k // 32)


def _gemm_ref(a_c, a_s, w_c, w_s, sel=None, rc=None, rs=None):
    return MX.gemm_comp(a_c, a_s, w_c, w_s, sel, rc, rs)


# The oracle never takes an input from the GPU: each stage's oracle operands
# are computed from the seeded inputs by the oracle itself, after checking
# that the GPU's result of that stage is identical.
def ref_mx(x_np, codes, scales, fp8=False):
    c_r, s_r = (MX.quantize_fp8 if fp8 else MX.quantize)(x_np)
    assert np.array_equal(npu8(codes), c_r) and np.array_equal(npu8(scales), s_r)
    return c_r, s_r


def ref_mx_weights(w, wc, ws):
    c_r, s_r = MX.quantize_weights(w.float().numpy())
    assert np.array_equal(npu8(wc), c_r) and np.array_equal(npu8(ws), s_r)
    return c_r, s_r


def ref_mx_resq(x_np, c_r, s_r, offs, k, row_index, sel, rc, rs):
    out = MX.resq_select_and_requant(x_np, c_r, s_r, offs, k, row_index=row_index)
    for got, want in zip((npu8(sel), npu8(rc), npu8(rs)), out):
        assert np.array_equal(got, want)
    return out


@pytest.mark.parametrize("spread", [False, True])
def test_mx_dense_linear_compensated(gpu_lib, spread):
    """Single dense linear 128 x 512 -> 1024 with top-32 compensation over all
    128 tokens (E = 1).  With spread, some weight blocks are scaled by 2^-12, so
    weight rows span more than 8 binades and the compensation's smallest W_S
    elements are rounded to E4M3 on the GPU."""
    P = gpu_lib
    wl = synth.WORKLOADS["dense_T128_K512_N1024_k32"]
    x = synth.activations(wl.tokens, wl.hidden, seed=wl.seed, outlier_channels=wl.outliers)
    w = synth.weights(1, wl.n_out, wl.hidden, seed=wl.seed, tensor_id=synth.WDENSE_ID)
    if spread:
        w = w.clone()
        w[0, :, 32:96] *= 2.0 ** -12
    xc = x.cuda()
    codes, scales, _ = P.mxfp4_quantize(xc)
    offs = torch.tensor([0, wl.tokens], dtype=torch.int64, device="cuda")
    sel, rc, rs = P.mxfp4_resq_select_and_requant(xc, codes, scales, wl.k, unit_offsets=offs,
                                                  rows_total=wl.tokens)
    wc, ws_ = _mx_weights(P, w)
    y = P.moe_mxfp4_grouped_gemm(codes, scales, offs, wl.tokens, wc, ws_, sel_idx=sel, r_codes=rc,
                                 r_scales=rs)
    y0 = P.moe_mxfp4_grouped_gemm(codes, scales, offs, wl.tokens, wc, ws_)
    x_np = x.float().numpy()
    c_r, s_r = ref_mx(x_np, codes, scales)
    sel_r, rc_r, rs_r = ref_mx_resq(x_np, c_r, s_r, [0, wl.tokens], wl.k, None, sel, rc, rs)
    wc_r, ws_r = ref_mx_weights(w, wc, ws_)
    ref = _gemm_ref(c_r, s_r, wc_r[0], ws_r[0], sel_r[0], rc_r, rs_r)
    ref0 = _gemm_ref(c_r, s_r, wc_r[0], ws_r[0])
    e_comp, e_plain = rel_err(np32(y), ref), rel_err(np32(y0), ref0)
    assert e_comp <= GEMM_TOL and e_plain <= GEMM_TOL, (e_comp, e_plain)
    if not spread:
        exact = x.float().numpy().astype(np.float64) @ MX.dequantize(
            wc_r[0], ws_r[0]).astype(np.float64).T
        assert np.linalg.norm(np32(y) - exact) < np.linalg.norm(np32(y0) - exact)


def _comp_rounding_bound(wc, ws, sel, rc, rs):
    """Elementwise bound on how far the GPU's compensation term may be from
    the exact one (the kernel's stated error bound).  The kernel runs the
    correction on the FP8 form of the scaled MFMA, with E4M3 operands under
    one power-of-two scale per operand row:
      W_S[n, j] = e2m1 * 2^(X - Xmax(n)), Xmax(n) the largest block scale of
        weight row n, is exact in E4M3 when X - Xmax(n) >= -8 and otherwise
        rounded to E4M3's subnormal grid: error <= 2^(Xmax(n) - 10);
      Q(R_S)[r, j] likewise against the larger block scale of its 64-wide
        K-step: error <= 2^(Xr(r, step) - 10) when more than 8 binades apart.
    So |dY[r, n]| <= sum_j |R[r, j]| dW[n, j] + dR[r, j] (|W[n, S_j]| + dW[n, j])."""
    w = MX.dequantize(wc, ws).astype(np.float64)
    xw = ws.astype(np.int64) - 127
    xmax = xw.max(axis=1)
    sel = np.asarray(sel, dtype=np.int64)
    xsel = xw[:, sel // 32]
    dw = np.where(xsel - xmax[:, None] < -8, 2.0 ** (xmax[:, None] - 10), 0.0)
    r = MX.dequantize(rc, rs).astype(np.float64)
    xr = rs.astype(np.int64) - 127
    kc = r.shape[1]
    xstep = np.stack([xr[:, 2 * s:2 * s + 2].max(axis=1) for s in range((kc + 63) // 64)], axis=1)
    xr_el = xr[:, np.arange(kc) // 32]
    xs_el = xstep[:, np.arange(kc) // 64]
    dr = np.where(xr_el - xs_el < -8, 2.0 ** (xs_el - 10), 0.0)
    return np.abs(r) @ dw.T + dr @ (np.abs(w[:, sel]) + dw).T, dw, dr


def test_mx_comp_rounding_bound(gpu_lib):
    """The compensation's stated error bound, exercised on both operands: 32
    outlier channels at the lowest indices (their residuals fill the first
    32-block of the compact R_S) and every other channel 2^-12 smaller (the
    second block, 10+ binades below the first in the same 64-wide K-step),
    with weight rows whose blocks span 12 binades.  The GPU result stays
    within the bound plus fp32 accumulation slack, elementwise."""
    P = gpu_lib
    rng = np.random.default_rng(81)
    tokens, k_dim, n_out, kc = 128, 512, 256, 64
    x = (rng.standard_normal((tokens, k_dim)) * 2.0 ** -12).astype(np.float32)
    x[:, :32] = (rng.standard_normal((tokens, 32)) * 16.0).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    w = synth.weights(1, n_out, k_dim, seed=82, tensor_id=synth.WDENSE_ID).clone()
    w[0, :, 64:192] *= 2.0 ** -12
    xc = xb.cuda()
    codes, scales, _ = P.mxfp4_quantize(xc)
    offs = torch.tensor([0, tokens], dtype=torch.int64, device="cuda")
    sel, rc, rs = P.mxfp4_resq_select_and_requant(xc, codes, scales, kc, unit_offsets=offs,
                                                  rows_total=tokens)
    wc, ws_ = _mx_weights(P, w)
    y = P.moe_mxfp4_grouped_gemm(codes, scales, offs, tokens, wc, ws_, sel_idx=sel, r_codes=rc,
                                 r_scales=rs)
    x_np = xb.float().numpy()
    c_r, s_r = ref_mx(x_np, codes, scales)
    sel_r, rc_r, rs_r = ref_mx_resq(x_np, c_r, s_r, [0, tokens], kc, None, sel, rc, rs)
    assert np.array_equal(sel_r[0][:32], np.arange(32))
    wc_r, ws_r = ref_mx_weights(w, wc, ws_)
    ref = _gemm_ref(c_r, s_r, wc_r[0], ws_r[0], sel_r[0], rc_r, rs_r)
    bound, dw, dr = _comp_rounding_bound(wc_r[0], ws_r[0], sel_r[0], rc_r, rs_r)
    assert dw.max() > 0 and dr.max() > 0, "both operands take the rounding path"
    a = np.abs(MX.dequantize(c_r, s_r).astype(np.float64))
    wa = np.abs(MX.dequantize(wc_r[0], ws_r[0]).astype(np.float64))
    s_abs = a @ wa.T + np.abs(MX.dequantize(rc_r, rs_r).astype(np.float64)) @ wa[:, sel_r[0]].T
    slack = (k_dim + kc) * 2.0 ** -24 * s_abs
    err = np.abs(np32(y) - ref)
    assert np.all(err <= bound + slack), float((err - bound - slack).max())
    assert rel_err(np32(y), ref) <= GEMM_TOL


def _route_setup(tokens, hidden, n_exp, inter, seed, zipf, top_k, empty_expert=None):
    x = synth.activations(tokens, hidden, seed=seed, heavy_frac=0.01)
    rt = synth.route(tokens, n_exp, seed=seed, top_k=top_k, zipf_s=zipf)
    offs = rt["offsets"].copy()
    if empty_expert is not None:
        offs[empty_expert + 1] = offs[empty_expert]
    wgu = synth.weights(n_exp, 2 * inter, hidden, seed=seed, tensor_id=synth.WGU_ID)
    wd = synth.weights(n_exp, hidden, inter, seed=seed, tensor_id=synth.WD_ID)
    return x, rt, offs, wgu, wd


def _gate_up_ref(codes, scales, slot_token, offs, gc, gs, sel=None, rc=None, rs=None):
    rows = int(offs[-1])
    out = np.zeros((rows, gc.shape[1]), np.float64)
    for e in range(len(offs) - 1):
        a, b = int(offs[e]), int(offs[e + 1])
        if a == b:
            continue
        tok = slot_token[a:b]
        comp = (sel[e], rc[a:b], rs[a:b]) if sel is not None else (None, None, None)
        out[a:b] = _gemm_ref(codes[tok], scales[tok], gc[e], gs[e], *comp)
    return out


@pytest.mark.parametrize("tokens,n_exp,top_k,zipf", [
    (600, 2, 2, 0.0),     # 600 rows per expert: 256-row tiles, last one 88 rows
    (340, 4, 2, 0.3),     # ~170 rows per expert: one 256-row tile
    (300, 4, 2, 0.5),     # 150 rows per expert: 128-row tiles
    (200, 8, 2, 1.0),     # 50 rows per expert: 64-row tiles
    (64, 16, 4, 0.0),     # 16 rows per expert: 32-row tiles
])
def test_mx_grouped_gemm_tile_variants(gpu_lib, tokens, n_exp, top_k, zipf):
    """Every tile shape (chosen from the average rows per expert) with
    compensation, F32 and SwiGLU epilogues, K = 384 (three 128-K stages) and
    N = 2 x 160 (a partial N tile)."""
    P = gpu_lib
    hidden, inter, k = 384, 160, 64
    x, rt, offs, wgu, _ = _route_setup(tokens, hidden, n_exp, inter, 21, zipf, top_k)
    xc = x.cuda()
    rows = int(offs[-1])
    offs_t = torch.from_numpy(offs).cuda()
    slot_tok = torch.from_numpy(rt["slot_token"]).cuda()
    codes, scales, _ = P.mxfp4_quantize(xc)
    sel, rc, rs = P.mxfp4_resq_select_and_requant(xc, codes, scales, k, unit_offsets=offs_t,
                                                  rows_total=rows, row_index=slot_tok)
    gc, gs = _mx_weights(P, wgu)
    comp = dict(sel_idx=sel, r_codes=rc, r_scales=rs)
    gu = P.moe_mxfp4_grouped_gemm(codes, scales, offs_t, rows, gc, gs, a_row_index=slot_tok, **comp)
    h = P.moe_mxfp4_grouped_gemm(codes, scales, offs_t, rows, gc, gs, a_row_index=slot_tok,
                                 epilogue=P.EPI_SWIGLU_BF16, **comp)
    x_np = x.float().numpy()
    c_r, s_r = ref_mx(x_np, codes, scales)
    sel_r, rc_r, rs_r = ref_mx_resq(x_np, c_r, s_r, offs, k, rt["slot_token"], sel, rc, rs)
    gc_r, gs_r = ref_mx_weights(wgu, gc, gs)
    gu_ref = _gate_up_ref(c_r, s_r, rt["slot_token"], offs, gc_r, gs_r, sel_r, rc_r, rs_r)
    gu_np = np32(gu)
    for e in range(n_exp):
        a, b = offs[e], offs[e + 1]
        if a < b:
            assert rel_err(gu_np[a:b], gu_ref[a:b]) <= GEMM_TOL, f"expert {e}"
    g_, u_ = gu_ref[:, :inter], gu_ref[:, inter:]
    h_r = F.bf16_bits_to_f32(F.f64_to_bf16_bits(g_ / (1 + np.exp(-g_)) * u_))
    tol = np.abs(h_r) * 2.0 ** -7 + GEMM_TOL * np.abs(h_r).max()
    assert np.all(np.abs(np32(h) - h_r) <= tol)


@pytest.mark.parametrize("comp", [True, False])
def test_mx_moe_layer(gpu_lib, comp):
    """The MXFP4 MoE layer stage by stage:
    quantize X, select + requantize per expert, gate/up with SwiGLU and the
    amax of h, quantize h, select per expert, down with the scatter-add."""
    P = gpu_lib
    tokens, hidden, n_exp, inter, k = 200, 256, 8, 256, 64
    x, rt, offs, wgu, wd = _route_setup(tokens, hidden, n_exp, inter, 9, 1.2, 4, empty_expert=5)
    xc = x.cuda()
    rows = int(offs[-1])
    offs_t = torch.from_numpy(offs).cuda()
    slot_tok = torch.from_numpy(rt["slot_token"]).cuda()
    codes, scales, _ = P.mxfp4_quantize(xc)
    comp1, comp1_ref = {}, (None, None, None)
    if comp:
        sel, rc, rs = P.mxfp4_resq_select_and_requant(xc, codes, scales, k, unit_offsets=offs_t,
                                                      rows_total=rows, row_index=slot_tok)
        comp1 = dict(sel_idx=sel, r_codes=rc, r_scales=rs)
    x_np = x.float().numpy()
    c_r, s_r = ref_mx(x_np, codes, scales)
    if comp:
        comp1_ref = ref_mx_resq(x_np, c_r, s_r, offs, k, rt["slot_token"], sel, rc, rs)
    gc, gs = _mx_weights(P, wgu)
    gc_r, gs_r = ref_mx_weights(wgu, gc, gs)
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    h = P.moe_mxfp4_grouped_gemm(codes, scales, offs_t, rows, gc, gs, a_row_index=slot_tok,
                                 epilogue=P.EPI_SWIGLU_BF16, out_amax=amax, **comp1)
    gu_ref = _gate_up_ref(c_r, s_r, rt["slot_token"], offs, gc_r, gs_r, *comp1_ref)
    g_, u_ = gu_ref[:, :inter], gu_ref[:, inter:]
    h_bits = F.f64_to_bf16_bits(g_ / (1 + np.exp(-g_)) * u_)
    h_r = F.bf16_bits_to_f32(h_bits)
    h_np = np32(h)
    tol = np.abs(h_r) * 2.0 ** -7 + GEMM_TOL * np.abs(h_r).max()
    assert np.all(np.abs(h_np - h_r) <= tol)
    assert np32(amax)[0] == np.abs(h_np).max()
    # down projection: both sides on the oracle's h (the GPU's h matched it
    # above within the GEMM tolerance)
    h = torch.from_numpy(h_bits.view(np.int16)).view(torch.bfloat16).cuda()
    h_np = h_r
    hq_c, hq_s, _ = P.mxfp4_quantize(h)
    hc_r, hs_r = ref_mx(h_np, hq_c, hq_s)
    comp2, comp2_ref = {}, None
    if comp:
        sel2, rc2, rs2 = P.mxfp4_resq_select_and_requant(h, hq_c, hq_s, k, unit_offsets=offs_t,
                                                         rows_total=rows)
        s2r = ref_mx_resq(h_np, hc_r, hs_r, offs, k, None, sel2, rc2, rs2)
        comp2, comp2_ref = dict(sel_idx=sel2, r_codes=rc2, r_scales=rs2), s2r
    dc, ds = _mx_weights(P, wd)
    y = torch.zeros(tokens, hidden, dtype=torch.float32, device="cuda")
    P.moe_mxfp4_grouped_gemm(hq_c, hq_s, offs_t, rows, dc, ds, epilogue=P.EPI_SCATTER_ADD_F32,
                             row_weight=torch.from_numpy(rt["slot_weight"]).cuda(),
                             scatter_index=slot_tok, out=y, **comp2)
    y_ref = np.zeros((tokens, hidden), np.float64)
    dc_n, ds_n = ref_mx_weights(wd, dc, ds)
    for e in range(n_exp):
        a, b = int(offs[e]), int(offs[e + 1])
        if a == b:
            continue
        c2 = (comp2_ref[0][e], comp2_ref[1][a:b], comp2_ref[2][a:b]) if comp else (None, None, None)
        out = _gemm_ref(hc_r[a:b], hs_r[a:b], dc_n[e], ds_n[e], *c2)
        np.add.at(y_ref, rt["slot_token"][a:b], out * rt["slot_weight"][a:b, None].astype(np.float64))
    assert rel_err(np32(y), y_ref) <= GEMM_TOL


# ---------------------------------------------------------------------------
# W4A8: MXFP8 activations x MXFP4 weights
# ---------------------------------------------------------------------------

def test_mx8_quantize_exhaustive_bf16(gpu_lib):
    """Every finite bf16 value in mixed-magnitude blocks, and again in blocks
    whose scale is fixed at X = 0, 5 and -20 (amax 448 * 2^X), so that every
    value is rounded (ties and saturation included) at those scales."""
    P = gpu_lib
    bits = np.arange(65536, dtype=np.uint16)
    vals = F.bf16_bits_to_f32(bits)
    vals = vals[np.isfinite(vals)]
    rng = np.random.default_rng(2)
    mixed = np.concatenate([vals, np.zeros((-vals.size) % 128, np.float32)])
    x_np = mixed[rng.permutation(mixed.size)].reshape(-1, 128)
    codes, scales = P.mxfp8_quantize(torch.from_numpy(x_np).to(torch.bfloat16).cuda())
    c_ref, s_ref = MX.quantize_fp8(x_np)
    assert np.array_equal(npu8(scales), s_ref)
    assert np.array_equal(npu8(codes), c_ref)
    for X in (0, 5, -20):
        v = vals[np.abs(vals.astype(np.float64)) <= 480.0 * 2.0 ** X]
        n = (v.size + 30) // 31 * 31
        blocks = np.zeros((n // 31, 32), np.float32)
        blocks[:, 0] = np.float32(448.0 * 2.0 ** X)
        blocks[:, 1:] = np.pad(v, (0, n - v.size)).reshape(-1, 31)
        blocks = np.concatenate([blocks, np.zeros(((-blocks.shape[0]) % 4, 32), np.float32)])
        xb = blocks.reshape(-1, 128)
        codes, scales = P.mxfp8_quantize(torch.from_numpy(xb).to(torch.bfloat16).cuda())
        c_ref, s_ref = MX.quantize_fp8(xb)
        assert np.array_equal(npu8(scales), s_ref), f"X={X}"
        assert np.array_equal(npu8(codes), c_ref), f"X={X}"


@pytest.mark.parametrize("m,k", [(300, 4096), (7, 96)])
def test_mx8_quantize_random_f32(gpu_lib, m, k):
    P = gpu_lib
    x = synth.activations(m, k, seed=6, heavy_frac=0.01).float()
    x = x + torch.randn(x.shape, generator=torch.Generator().manual_seed(3)) * 1e-3
    codes, scales = P.mxfp8_quantize(x.cuda())
    c_ref, s_ref = MX.quantize_fp8(x.numpy())
    assert np.array_equal(npu8(scales), s_ref)
    assert np.array_equal(npu8(codes), c_ref)


@pytest.mark.parametrize("tokens,n_exp,top_k,zipf", [
    (600, 2, 2, 0.0),     # 256-row tiles
    (300, 4, 2, 0.5),     # 128-row tiles
    (200, 8, 2, 1.0),     # 64-row tiles
    (64, 16, 4, 0.0),     # 32-row tiles
])
def test_w4a8_grouped_gemm_tile_variants(gpu_lib, tokens, n_exp, top_k, zipf):
    """Every tile shape of the W4A8 GEMM against the float64 product of the
    same quantized operands: F32 and SwiGLU epilogues, K = 384, N = 2 x 160."""
    P = gpu_lib
    hidden, inter = 384, 160
    x, rt, offs, wgu, _ = _route_setup(tokens, hidden, n_exp, inter, 22, zipf, top_k)
    rows = int(offs[-1])
    offs_t = torch.from_numpy(offs).cuda()
    slot_tok = torch.from_numpy(rt["slot_token"]).cuda()
    ac, asc = P.mxfp8_quantize(x.cuda())
    gc, gs = _mx_weights(P, wgu)
    gu = P.moe_mxfp4_w4a8_grouped_gemm(ac, asc, offs_t, rows, gc, gs, a_row_index=slot_tok)
    h = P.moe_mxfp4_w4a8_grouped_gemm(ac, asc, offs_t, rows, gc, gs, a_row_index=slot_tok,
                                      epilogue=P.EPI_SWIGLU_BF16)
    ac_n, as_n = ref_mx(x.float().numpy(), ac, asc, fp8=True)
    gc_n, gs_n = ref_mx_weights(wgu, gc, gs)
    ref = np.zeros((rows, 2 * inter))
    for e in range(n_exp):
        a, b = int(offs[e]), int(offs[e + 1])
        if a < b:
            tok = rt["slot_token"][a:b]
            ref[a:b] = MX.gemm_w4a8(ac_n[tok], as_n[tok], gc_n[e], gs_n[e])
            assert rel_err(np32(gu)[a:b], ref[a:b]) <= GEMM_TOL, f"expert {e}"
    g_, u_ = ref[:, :inter], ref[:, inter:]
    h_r = F.bf16_bits_to_f32(F.f64_to_bf16_bits(g_ / (1 + np.exp(-g_)) * u_))
    tol = np.abs(h_r) * 2.0 ** -7 + GEMM_TOL * np.abs(h_r).max()
    assert np.all(np.abs(np32(h) - h_r) <= tol)


def test_w4a8_down_scatter(gpu_lib):
    """Down projection with the scatter-add epilogue (K = 256)."""
    P = gpu_lib
    tokens, hidden, n_exp, inter = 160, 256, 8, 256
    _, rt, offs, _, wd = _route_setup(tokens, hidden, n_exp, inter, 24, 1.0, 4)
    rows = int(offs[-1])
    hrows = torch.from_numpy(np.random.default_rng(4).standard_normal((rows, inter)).astype(np.float32))
    hc, hs = P.mxfp8_quantize(hrows.to(torch.bfloat16).cuda())
    dc, ds = _mx_weights(P, wd)
    y = torch.zeros(tokens, hidden, dtype=torch.float32, device="cuda")
    P.moe_mxfp4_w4a8_grouped_gemm(hc, hs, torch.from_numpy(offs).cuda(), rows, dc, ds,
                                  epilogue=P.EPI_SCATTER_ADD_F32,
                                  row_weight=torch.from_numpy(rt["slot_weight"]).cuda(),
                                  scatter_index=torch.from_numpy(rt["slot_token"]).cuda(), out=y)
    y_ref = np.zeros((tokens, hidden))
    hc_n, hs_n = ref_mx(hrows.to(torch.bfloat16).float().numpy(), hc, hs, fp8=True)
    dc_n, ds_n = ref_mx_weights(wd, dc, ds)
    for e in range(n_exp):
        a, b = int(offs[e]), int(offs[e + 1])
        if a < b:
            out = MX.gemm_w4a8(hc_n[a:b], hs_n[a:b], dc_n[e], ds_n[e])
            np.add.at(y_ref, rt["slot_token"][a:b], out * rt["slot_weight"][a:b, None].astype(np.float64))
    assert rel_err(np32(y), y_ref) <= GEMM_TOL



def test_w4a8_down_scatter_overwrite(gpu_lib):
    """EPI_SCATTER_F32 on the MXFP4 path: the add-into-zeros sums bit for bit
    over an out full of NaN, and zeros from a launch with no rows."""
    P = gpu_lib
    tokens, hidden, n_exp, inter = 160, 256, 8, 256
    _, rt, offs, _, wd = _route_setup(tokens, hidden, n_exp, inter, 24, 1.0, 4)
    rows = int(offs[-1])
    hrows = torch.from_numpy(np.random.default_rng(5).standard_normal((rows, inter)).astype(np.float32))
    hc, hs = P.mxfp8_quantize(hrows.to(torch.bfloat16).cuda())
    dc, ds = _mx_weights(P, wd)
    kw = dict(row_weight=torch.from_numpy(rt["slot_weight"]).cuda(),
              scatter_index=torch.from_numpy(rt["slot_token"]).cuda())
    offs_t = torch.from_numpy(offs).cuda()
    y_add = torch.zeros(tokens, hidden, dtype=torch.float32, device="cuda")
    P.moe_mxfp4_w4a8_grouped_gemm(hc, hs, offs_t, rows, dc, ds, epilogue=P.EPI_SCATTER_ADD_F32,
                                  out=y_add, **kw)
    y_ow = torch.full((tokens, hidden), float("nan"), dtype=torch.float32, device="cuda")
    P.moe_mxfp4_w4a8_grouped_gemm(hc, hs, offs_t, rows, dc, ds, epilogue=P.EPI_SCATTER_F32,
                                  out=y_ow, **kw)
    assert np.array_equal(np32(y_add).view(np.uint32), np32(y_ow).view(np.uint32))
    y_none = torch.full((tokens, hidden), float("nan"), dtype=torch.float32, device="cuda")
    P.moe_mxfp4_w4a8_grouped_gemm(hc, hs, torch.zeros(n_exp + 1, dtype=torch.int64, device="cuda"), 0,
                                  dc, ds, epilogue=P.EPI_SCATTER_F32, out=y_none, **kw)
    assert np.all(np32(y_none) == 0.0)

def test_mx_scatter_256_row_tiles_graph_replays(gpu_lib):
    """Groups of 256 rows and more take 256-row tiles, and with the scatter
    epilogue the plan of the row lists runs on the library's second stream
    when eager (on the capturing stream under capture): the call captured in
    a HIP graph and replayed, with eager work in between, gives the eager
    result bit for bit; the eager result matches the oracle."""
    P = gpu_lib
    rng = np.random.default_rng(23)
    counts = np.array([300, 280, 512, 261], dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows, n_exp, K, N, tokens = int(offs[-1]), len(counts), 256, 256, 700
    x = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32)).to(torch.bfloat16)
    w = synth.weights(n_exp, N, K, seed=23, tensor_id=synth.WD_ID)
    slot_token = rng.integers(0, tokens, size=rows).astype(np.int32)
    slot_weight = rng.uniform(0.05, 1.0, size=rows).astype(np.float32)
    xc, xs, _ = P.mxfp4_quantize(x.cuda())
    wc, ws = _mx_weights(P, w)
    kw = dict(epilogue=P.EPI_SCATTER_F32, row_weight=torch.from_numpy(slot_weight).cuda(),
              scatter_index=torch.from_numpy(slot_token).cuda(), out_rows=tokens)
    offs_t = torch.from_numpy(offs).cuda()
    y0 = P.moe_mxfp4_grouped_gemm(xc, xs, offs_t, rows, wc, ws, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y = P.moe_mxfp4_grouped_gemm(xc, xs, offs_t, rows, wc, ws, **kw)
    for _ in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y0.view(torch.int32))
    xc_r, xs_r = ref_mx(x.float().numpy(), xc, xs)
    wc_r, ws_r = ref_mx_weights(w, wc, ws)
    y_ref = np.zeros((tokens, N))
    for e in range(n_exp):
        a, b = int(offs[e]), int(offs[e + 1])
        out = _gemm_ref(xc_r[a:b], xs_r[a:b], wc_r[e], ws_r[e])
        np.add.at(y_ref, slot_token[a:b], out * slot_weight[a:b, None].astype(np.float64))
    assert rel_err(np32(y0), y_ref) <= GEMM_TOL


# ---------------------------------------------------------------------------
# trainer side: MXFP4 weight QDQ and guided rounding
# ---------------------------------------------------------------------------

def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def test_mx_qdq_weights_magnitudes(gpu_lib):
    """bf16(DQ), codes and scales bit-exact, with rows spanning 2^-133 (bf16
    subnormals, the E8M0 floor) to 2^120, zero rows and zero blocks."""
    P = gpu_lib
    g = torch.Generator().manual_seed(51)
    nmat, n, k = 3, 64, 512
    w = torch.randn(nmat, n, k, generator=g)
    expo = torch.randint(-133, 121, (nmat, n, 1), generator=g).float()
    w = (w * torch.exp2(expo)).to(torch.bfloat16)
    w[1, 5] = 0
    w[2, 7, 64:96] = 0
    out, codes, scales = P.mxfp4_qdq_weights(w.cuda())
    out_r, codes_r, scales_r = MX.qdq_weights(w.float().numpy())
    assert np.array_equal(npu8(scales), scales_r)
    assert np.array_equal(npu8(codes), codes_r)
    assert np.array_equal(_bits(out), out_r)
    out2, c2, s2 = P.mxfp4_qdq_weights(w.cuda(), want_codes=False)
    assert c2 is None and s2 is None and torch.equal(out2, out)


def test_mx_qdq_weights_expert_shapes(gpu_lib):
    """Expert-shaped matrices (gate/up 2 x 192 by 256, down 256 by 192)."""
    P = gpu_lib
    for n, k, tid in [(384, 256, synth.WGU_ID), (256, 192, synth.WD_ID)]:
        w = synth.weights(4, n, k, seed=52, tensor_id=tid)
        out, codes, scales = P.mxfp4_qdq_weights(w.cuda())
        out_r, codes_r, scales_r = MX.qdq_weights(w.float().numpy())
        assert np.array_equal(npu8(scales), scales_r)
        assert np.array_equal(npu8(codes), codes_r)
        assert np.array_equal(_bits(out), out_r)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rel", [1e-3, 2e-2, 0.2])
def test_mx_guided_round(gpu_lib, dtype, rel):
    """Guided codes, x_fq and the distance histogram bit-exact against the
    oracle, rollout codes from the MXFP4 quantizer."""
    P = gpu_lib
    x_roll = synth.activations(257, 512, seed=53, heavy_frac=0.01)
    x_train = synth.guided_noise(x_roll, seed=53, rel=rel).to(dtype)
    rc, rs, _ = P.mxfp4_quantize(x_roll.cuda())
    gc, fq, hist = P.mxfp4_guided_round(x_train.cuda(), rc, rs)
    rc_r, rs_r = ref_mx(x_roll.float().numpy(), rc, rs)
    gc_r, fq_r, hist_r = MX.guided_round(x_train.float().numpy(), rc_r, rs_r)
    assert np.array_equal(npu8(gc), gc_r)
    assert np.array_equal(_bits(fq), fq_r)
    assert np.array_equal(hist.cpu().numpy(), hist_r)


def test_mx_guided_round_tiny_scales(gpu_lib):
    """Rollout blocks whose 2^X is subnormal or near the E8M0 floor (the exact
    rounding path) and a padded row stride."""
    P = gpu_lib
    g = torch.Generator().manual_seed(54)
    x_roll = (torch.randn(64, 256, generator=g)
              * torch.exp2(torch.randint(-140, -100, (64, 1), generator=g).float())).to(torch.bfloat16)
    x_train = (x_roll.float() * (1 + 0.05 * torch.randn(64, 256, generator=g))).to(torch.bfloat16)
    rc, rs, _ = P.mxfp4_quantize(x_roll.cuda())
    pad = torch.zeros(64, 320, dtype=torch.bfloat16)
    pad[:, :256] = x_train
    xt = pad.cuda()[:, :256]
    gc, fq, hist = P.mxfp4_guided_round(xt, rc, rs)
    rc_r, rs_r = ref_mx(x_roll.float().numpy(), rc, rs)
    gc_r, fq_r, hist_r = MX.guided_round(x_train.float().numpy(), rc_r, rs_r)
    assert np.array_equal(npu8(gc), gc_r)
    assert np.array_equal(_bits(fq), fq_r)
    assert np.array_equal(hist.cpu().numpy(), hist_r)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rel", [1e-3, 2e-2, 0.2])
def test_mx_guided_round_record(gpu_lib, dtype, rel):
    """Mantissa-only record of MXFP4 rollout codes (packed by the format-free
    record packer), then guided rounding from it: codes, x_fq and the
    kept/moved counts bit-exact."""
    P = gpu_lib
    x_roll = synth.activations(257, 1024, seed=55, heavy_frac=0.01)
    x_train = synth.guided_noise(x_roll, seed=55, rel=rel).to(dtype)
    rc, rs, _ = P.mxfp4_quantize(x_roll.cuda())
    rc_r, rs_r = ref_mx(x_roll.float().numpy(), rc, rs)
    rec = P.guidance_record_pack(rc)
    rec_r = OQ.guidance_record(rc_r)
    assert np.array_equal(npu8(rec), rec_r)
    gc, fq, moved = P.mxfp4_guided_round_record(x_train.cuda(), rec, rs)
    gc_r, fq_r, moved_r = MX.guided_round_record(x_train.float().numpy(), rec_r, rs_r)
    assert np.array_equal(npu8(gc), gc_r)
    assert np.array_equal(_bits(fq), fq_r)
    assert np.array_equal(moved.cpu().numpy(), moved_r)
