"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
identical seeded inputs.

Bar: codes, scales, global scales, selected channels, requantized residuals,
QDQ output and guided codes bit-exact; GEMM outputs within
max|Y_gpu - Y_ref| / max|Y_ref| <= 1e-3 per output tensor (per expert for
grouped GEMMs) against the float64 reference on the same quantized operands.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import gemm as OG
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


# The oracle never takes an input from the GPU: each stage's oracle operands
# are computed from the seeded inputs by the oracle itself, after checking
# that the GPU's result of that stage is identical.
def ref_quant(x, codes, scales, g):
    c_r, s_r, g_r = OQ.quantize(x.float().numpy() if torch.is_tensor(x) else x)
    assert np.array_equal(npu8(codes), c_r) and np.array_equal(npu8(scales), s_r)
    assert np32(g)[0] == g_r
    return c_r, s_r, g_r


def ref_resq(x_np, c_r, s_r, g_r, offs, k, row_index, sel, rc, rs, rg):
    out = OQ.resq_select_and_requant(x_np, c_r, s_r, g_r, offs, k, row_index=row_index)
    for got, want in zip((npu8(sel), npu8(rc), npu8(rs), np32(rg)), out):
        assert np.array_equal(got, want)
    return out


def ref_weights(w, wc, ws, wg):
    _, c_r, s_r, g_r = OQ.qdq_weights(w.float().numpy())
    assert np.array_equal(npu8(wc), c_r) and np.array_equal(npu8(ws), s_r)
    assert np.array_equal(np32(wg), g_r)
    return c_r, s_r, g_r


# ---------------------------------------------------------------------------
# quantize
# ---------------------------------------------------------------------------

def test_quantize_exhaustive_bf16_many_scales(gpu_lib):
    """Every finite bf16 value, under global scales forced through amax_in."""
    P = gpu_lib
    bits = np.arange(65536, dtype=np.uint16)
    vals = F.bf16_bits_to_f32(bits)
    vals = vals[np.isfinite(vals)]
    vals = np.concatenate([vals, np.zeros((-vals.size) % 128, np.float32)])
    rng = np.random.default_rng(0)
    x_np = vals[rng.permutation(vals.size)].reshape(-1, 16 * 8)   # blocks mix magnitudes
    x = torch.from_numpy(x_np).to(torch.bfloat16).cuda()
    for amax in [np.float32(2688.0), np.float32(1.0), np.float32(3.0e38), np.float32(7.5e-3),
                 np.float32(1e-30), np.float32(123.456)]:
        amax_t = torch.tensor([amax], device="cuda")
        codes, scales, g, _ = P.nvfp4_quantize(x, amax_in=amax_t)
        g_ref = OQ.global_scale(amax)
        c_ref, s_ref, _ = OQ.quantize(x_np, g=g_ref)
        assert np32(g)[0] == g_ref
        assert np.array_equal(npu8(scales), s_ref), f"scales differ at amax={amax}"
        assert np.array_equal(npu8(codes), c_ref), f"codes differ at amax={amax}"


def _e4m3_midpoints():
    v = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    return 0.5 * (v[:-1] + v[1:])                      # between bytes b and b + 1


@pytest.mark.parametrize("amax", [2688.0, 2688.0 * 1.37, 2.0 ** -85, 2.0 ** -90])
def test_quantize_scale_rounding_boundaries(gpu_lib, amax):
    """Blocks whose amax sits on every E4M3 rounding boundary of amax_b / (6g)
    and one fp32 ulp either side: exact ties (g = 1, so 6 m g is exact),
    a g with a full mantissa, a tiny g, and a g below 2^-100."""
    P = gpu_lib
    g = OQ.global_scale(np.float32(amax))
    targets = (6.0 * _e4m3_midpoints() * np.float64(g)).astype(np.float32)
    block_amax = np.concatenate([targets, np.nextafter(targets, np.float32(0)),
                                 np.nextafter(targets, np.float32(np.inf))])
    block_amax = block_amax[block_amax <= np.float32(amax)]
    rng = np.random.default_rng(31)
    nblk = block_amax.size + (-(block_amax.size + 1)) % 32 + 1
    x = np.zeros((nblk, 16), np.float32)
    x[0, 0] = np.float32(amax)                         # fixes the global amax
    x[1:block_amax.size + 1] = block_amax[:, None] * rng.uniform(0, 1, (block_amax.size, 16))
    x[1:block_amax.size + 1, 0] = block_amax
    x *= np.where(rng.uniform(size=x.shape) < 0.5, -1, 1).astype(np.float32)
    x_np = x.reshape(-1, 32 * 16)
    codes, scales, g_d, _ = P.nvfp4_quantize(torch.from_numpy(x_np).cuda())
    c_ref, s_ref, g_ref = OQ.quantize(x_np)
    assert np32(g_d)[0] == g_ref == g
    assert np.array_equal(npu8(scales), s_ref)
    assert np.array_equal(npu8(codes), c_ref)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("m,k", [(128, 512), (300, 4096), (1, 16), (7, 48)])
def test_quantize_random_with_tile_partials(gpu_lib, dtype, m, k):
    P = gpu_lib
    x = synth.activations(m, k, seed=5, heavy_frac=0.01).to(dtype)
    if dtype == torch.float32:
        x = x + torch.randn(x.shape, generator=torch.Generator().manual_seed(1)) * 1e-3
    x_np = x.float().numpy()
    codes, scales, g, tp = P.nvfp4_quantize(x.cuda(), tile_partials=True)
    c_ref, s_ref, g_ref = OQ.quantize(x_np)
    assert np32(g)[0] == g_ref
    assert np.array_equal(npu8(scales), s_ref)
    assert np.array_equal(npu8(codes), c_ref)
    r = np.abs(OQ.residual(x_np, c_ref, s_ref, g_ref))
    tp_ref = np.stack([OQ.channel_scores(r[t:t + 128]) for t in range(0, m, 128)])
    assert np.array_equal(np32(tp), tp_ref)


def test_quantize_zero_and_ragged_stride(gpu_lib):
    P = gpu_lib
    z = torch.zeros(5, 32, dtype=torch.bfloat16, device="cuda")
    z[1] = -0.0
    codes, scales, g, _ = P.nvfp4_quantize(z)
    assert np32(g)[0] == 1.0 and int(scales.sum()) == 0
    nib = OQ.unpack_nibbles(npu8(codes))
    assert np.all(nib[0] == 0) and np.all(nib[1] == 8)
    # a strided view (row stride 96 elements, K = 64)
    base = synth.activations(40, 96, seed=6).cuda()
    view = base[:, :64]
    codes, scales, g, _ = P.nvfp4_quantize(view)
    c_ref, s_ref, g_ref = OQ.quantize(view.float().cpu().numpy())
    assert np.array_equal(npu8(codes), c_ref) and np.array_equal(npu8(scales), s_ref)


def test_quantize_worked_example(gpu_lib):
    """TRACE research motivation: 60.25 (train) and 59.75 (rollout) in bf16
    under scale 24 round to 3 and 2."""
    P = gpu_lib
    x = torch.zeros(2, 32, dtype=torch.bfloat16)
    x[:, 16] = 2688.0
    x[:, 0] = 144.0
    x[0, 1] = 60.25
    x[1, 1] = 59.75
    codes, scales, g, _ = P.nvfp4_quantize(x.cuda())
    nib = OQ.unpack_nibbles(npu8(codes))
    assert np32(g)[0] == 1.0 and npu8(scales)[0, 0] == 0x5C
    assert nib[0, 1] == 5 and nib[1, 1] == 4


# ---------------------------------------------------------------------------
# residual selection and requantization
# ---------------------------------------------------------------------------

def test_resq_tile_units(gpu_lib):
    P = gpu_lib
    m, k_dim, k = 300, 1024, 128
    x = synth.activations(m, k_dim, seed=7, heavy_frac=0.01)
    xc = x.cuda()
    codes, scales, g, tp = P.nvfp4_quantize(xc, tile_partials=True)
    sel, rc, rs, rg = P.resq_select_and_requant(xc, codes, scales, g, k, tile_partials=tp)
    x_np = x.float().numpy()
    c_ref, s_ref, g_ref = OQ.quantize(x_np)
    offs = list(range(0, m, 128)) + [m]
    sel_r, rc_r, rs_r, rg_r = OQ.resq_select_and_requant(x_np, c_ref, s_ref, g_ref, offs, k)
    assert np.array_equal(npu8(sel), sel_r)
    assert np.array_equal(np32(rg), rg_r)
    assert np.array_equal(npu8(rs), rs_r)
    assert np.array_equal(npu8(rc), rc_r)


@pytest.mark.parametrize("k_dim,k", [(512, 400), (1536, 128), (4096, 128), (6144, 64), (8208, 128)])
def test_resq_select_widths_and_ties(gpu_lib, k_dim, k):
    """Selection at each channel count the select kernel distinguishes (keys
    in registers up to 8192 channels, in LDS beyond), with exact score ties:
    all-zero 16-blocks (score +0) and copied 16-blocks (equal scores); ties
    go to the lower channel.  With k = 400 of 512 the threshold itself is +0."""
    P = gpu_lib
    m = 200
    x = synth.activations(m, k_dim, seed=14, heavy_frac=0.01).float()
    x[:, 16:176] = 0.0                    # ten zero blocks
    x[:, 192:256] = x[:, 320:384]         # four copied blocks
    x = x.to(torch.bfloat16)
    xc = x.cuda()
    codes, scales, g, tp = P.nvfp4_quantize(xc, tile_partials=True)
    sel, rc, rs, rg = P.resq_select_and_requant(xc, codes, scales, g, k, tile_partials=tp)
    x_np = x.float().numpy()
    c_ref, s_ref, g_ref = OQ.quantize(x_np)
    offs = list(range(0, m, 128)) + [m]
    sel_r, rc_r, rs_r, rg_r = OQ.resq_select_and_requant(x_np, c_ref, s_ref, g_ref, offs, k)
    assert np.array_equal(npu8(sel), sel_r)
    assert np.array_equal(np32(rg), rg_r)
    assert np.array_equal(npu8(rs), rs_r)
    assert np.array_equal(npu8(rc), rc_r)


@pytest.mark.parametrize("k", [16, 64])
def test_resq_gathered_expert_units(gpu_lib, k):
    """Units = experts' routed tokens (gather through the slot->token map),
    with skewed loads, an empty expert and units longer than one 128-row tile."""
    P = gpu_lib
    tokens, hidden, n_exp = 400, 256, 6
    x = synth.activations(tokens, hidden, seed=8, heavy_frac=0.02)
    rt = synth.route(tokens, n_exp, seed=8, top_k=2, zipf_s=1.5)
    offs = rt["offsets"].copy()
    # make expert 3 empty by moving its slots to expert 4 (offsets stay sorted)
    offs[4] = offs[3]
    xc = x.cuda()
    codes, scales, g, _ = P.nvfp4_quantize(xc)
    sel, rc, rs, rg = P.resq_select_and_requant(
        xc, codes, scales, g, k, unit_offsets=torch.from_numpy(offs).cuda(),
        rows_total=int(offs[-1]), row_index=torch.from_numpy(rt["slot_token"]).cuda())
    x_np = x.float().numpy()
    c_ref, s_ref, g_ref = OQ.quantize(x_np)
    sel_r, rc_r, rs_r, rg_r = OQ.resq_select_and_requant(x_np, c_ref, s_ref, g_ref, offs, k,
                                                         row_index=rt["slot_token"])
    assert np.diff(offs).max() > 128
    assert np.array_equal(npu8(sel), sel_r)
    assert np.array_equal(np32(rg), rg_r)
    assert np.array_equal(npu8(rs), rs_r)
    assert np.array_equal(npu8(rc), rc_r)


@pytest.mark.parametrize("hidden,k", [(768, 64), (2048, 16), (2048, 64), (3072, 64)])
def test_resq_small_units(gpu_lib, hidden, k):
    """Decode-sized units (at most 32 routed rows per unit on average), which
    the library handles in one launch with one workgroup per unit: 64 experts,
    many of them empty, and a hot expert of 381 rows (scores over three
    128-row tiles; with k = 64 its R_S is computed a second time for the
    requantization instead of being kept on chip)."""
    P = gpu_lib
    tokens, n_exp = 512, 64
    x = synth.activations(tokens, hidden, seed=21, heavy_frac=0.02)
    rt = synth.route(tokens, n_exp, seed=21, top_k=2, zipf_s=1.1)
    offs = rt["offsets"]
    assert offs[-1] <= 32 * n_exp and np.diff(offs).max() > 2 * 128 and (np.diff(offs) == 0).any()
    xc = x.cuda()
    codes, scales, g, _ = P.nvfp4_quantize(xc)
    sel, rc, rs, rg = P.resq_select_and_requant(
        xc, codes, scales, g, k, unit_offsets=torch.from_numpy(offs).cuda(),
        rows_total=int(offs[-1]), row_index=torch.from_numpy(rt["slot_token"]).cuda())
    x_np = x.float().numpy()
    c_ref, s_ref, g_ref = OQ.quantize(x_np)
    sel_r, rc_r, rs_r, rg_r = OQ.resq_select_and_requant(x_np, c_ref, s_ref, g_ref, offs, k,
                                                         row_index=rt["slot_token"])
    assert np.array_equal(npu8(sel), sel_r)
    assert np.array_equal(np32(rg), rg_r)
    assert np.array_equal(npu8(rs), rs_r)
    assert np.array_equal(npu8(rc), rc_r)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def _quant_weights(P, w):
    _, c, s, g = P.qdq_weights(w.cuda())
    return c, s, g


def test_dense_linear_compensated(gpu_lib):
    """Single dense linear 128 x 512 -> 1024 with top-32 compensation over
    all 128 tokens (E = 1)."""
    P = gpu_lib
    wl = synth.WORKLOADS["dense_T128_K512_N1024_k32"]
    x = synth.activations(wl.tokens, wl.hidden, seed=wl.seed, outlier_channels=wl.outliers)
    w = synth.weights(1, wl.n_out, wl.hidden, seed=wl.seed, tensor_id=synth.WDENSE_ID)
    xc = x.cuda()
    codes, scales, g, _ = P.nvfp4_quantize(xc)
    offs = torch.tensor([0, wl.tokens], dtype=torch.int64, device="cuda")
    sel, rc, rs, rg = P.resq_select_and_requant(xc, codes, scales, g, wl.k, unit_offsets=offs,
                                                rows_total=wl.tokens)
    wc, ws_, wg = _quant_weights(P, w)
    y = P.moe_w4a4_grouped_gemm(codes, scales, g, offs, wl.tokens, wc, ws_, wg,
                                sel_idx=sel, r_codes=rc, r_scales=rs, r_global=rg)
    y0 = P.moe_w4a4_grouped_gemm(codes, scales, g, offs, wl.tokens, wc, ws_, wg)
    c_r, s_r, g_r = ref_quant(x, codes, scales, g)
    sel_r, rc_r, rs_r, rg_r = ref_resq(x.float().numpy(), c_r, s_r, g_r, [0, wl.tokens], wl.k,
                                       None, sel, rc, rs, rg)
    wc_r, ws_r, wg_r = ref_weights(w, wc, ws_, wg)
    ref = OG.gemm_comp(c_r, s_r, g_r, wc_r[0], ws_r[0], wg_r[0], sel_r[0], rc_r, rs_r, rg_r[0])
    ref0 = OG.gemm_comp(c_r, s_r, g_r, wc_r[0], ws_r[0], wg_r[0])
    assert rel_err(np32(y), ref) <= GEMM_TOL
    assert rel_err(np32(y0), ref0) <= GEMM_TOL
    # compensation moves the result toward the unquantized product
    exact = x.float().numpy().astype(np.float64) @ OQ.dequantize(
        wc_r[0], ws_r[0], wg_r[0]).astype(np.float64).T
    assert np.linalg.norm(np32(y) - exact) < np.linalg.norm(np32(y0) - exact)


def _moe_setup(P, tokens, hidden, n_exp, inter, k, seed, zipf=0.0, top_k=8, empty_expert=None):
    x = synth.activations(tokens, hidden, seed=seed, heavy_frac=0.01)
    rt = synth.route(tokens, n_exp, seed=seed, top_k=top_k, zipf_s=zipf)
    offs = rt["offsets"].copy()
    if empty_expert is not None:
        offs[empty_expert + 1] = offs[empty_expert]
    wgu = synth.weights(n_exp, 2 * inter, hidden, seed=seed, tensor_id=synth.WGU_ID)
    wd = synth.weights(n_exp, hidden, inter, seed=seed, tensor_id=synth.WD_ID)
    return x, rt, offs, wgu, wd


@pytest.mark.parametrize("comp", [True, False])
def test_grouped_gemm_swiglu_and_scatter(gpu_lib, comp):
    _check_moe_layer(gpu_lib, 200, 256, 8, 192, 32, seed=9, zipf=1.2, top_k=4, empty_expert=5,
                     comp=comp)


@pytest.mark.parametrize("hidden,inter", [(64, 64), (128, 192), (192, 128), (1024, 320)])
def test_grouped_gemm_32row_tiles(gpu_lib, hidden, inter):
    """16 rows per expert (the 32-row tile, which moves 128 K per stage): K a
    multiple of 128, K with a half-full last stage (192, 320), and K = 64
    (served by the 64-row tile); gate/up with SwiGLU, down with scatter-add,
    both compensated."""
    _check_moe_layer(gpu_lib, 64, hidden, 16, inter, 32, seed=23, zipf=0.0, top_k=4,
                     empty_expert=3, comp=True)


def _check_moe_layer(P, tokens, hidden, n_exp, inter, k, seed, zipf, top_k, empty_expert, comp):
    x, rt, offs, wgu, wd = _moe_setup(P, tokens, hidden, n_exp, inter, k, seed=seed, zipf=zipf,
                                      top_k=top_k, empty_expert=empty_expert)
    xc = x.cuda()
    rows = int(offs[-1])
    offs_t = torch.from_numpy(offs).cuda()
    slot_tok = torch.from_numpy(rt["slot_token"]).cuda()
    codes, scales, g, _ = P.nvfp4_quantize(xc)
    comp1 = {}
    if comp:
        sel, rc, rs, rg = P.resq_select_and_requant(xc, codes, scales, g, k, unit_offsets=offs_t,
                                                    rows_total=rows, row_index=slot_tok)
        comp1 = dict(sel_idx=sel, r_codes=rc, r_scales=rs, r_global=rg)
    gc, gs, gg = _quant_weights(P, wgu)
    # F32 epilogue of gate/up (reference GEMM check per expert)
    gu = P.moe_w4a4_grouped_gemm(codes, scales, g, offs_t, rows, gc, gs, gg, a_row_index=slot_tok,
                                 **comp1)
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    h = P.moe_w4a4_grouped_gemm(codes, scales, g, offs_t, rows, gc, gs, gg, a_row_index=slot_tok,
                                epilogue=P.EPI_SWIGLU_BF16, out_amax=amax, **comp1)
    x_np = x.float().numpy()
    c_r, s_r, g_r = ref_quant(x_np, codes, scales, g)
    gc_r, gs_r, gg_r = ref_weights(wgu, gc, gs, gg)
    comp_ref = {}
    if comp:
        sel_r, rc_r, rs_r, rg_r = ref_resq(x_np, c_r, s_r, g_r, offs, k, rt["slot_token"],
                                           sel, rc, rs, rg)
        comp_ref = dict(sel_idx=sel_r, r_codes=rc_r, r_scales=rs_r, r_g=rg_r)
    gu_ref, h_ref = OG.moe_gate_up(c_r, s_r, g_r, rt["slot_token"], offs,
                                   gc_r, gs_r, gg_r, inter, **comp_ref)
    gu_np = np32(gu)
    for e in range(n_exp):
        a, b = offs[e], offs[e + 1]
        if a < b:
            assert rel_err(gu_np[a:b], gu_ref[a:b]) <= GEMM_TOL, f"expert {e}"
    # h: bf16 of silu(G)*U -- within one bf16 ulp plus the GEMM tolerance
    h_np = np32(h)
    h_r = F.bf16_bits_to_f32(h_ref)
    tol = np.abs(h_r) * 2.0 ** -7 + GEMM_TOL * np.abs(h_r).max()
    assert np.all(np.abs(h_np - h_r) <= tol)
    assert np32(amax)[0] == np.abs(h_np).max()
    # down projection with scatter-add, both sides on the oracle's h (the
    # GPU's h matched it above within the GEMM tolerance; the quantizer's
    # amax_in path gets the amax of that h)
    h_in = torch.from_numpy(h_ref.view(np.int16)).view(torch.bfloat16).cuda()
    h_r32 = F.bf16_bits_to_f32(h_ref)
    h_amax = torch.tensor([np.abs(h_r32).max()], dtype=torch.float32, device="cuda")
    hq_c, hq_s, hq_g, _ = P.nvfp4_quantize(h_in, amax_in=h_amax)
    hc_r, hs_r, hg_r = ref_quant(h_r32, hq_c, hq_s, hq_g)
    h = h_in
    h_np = h_r32
    comp2, comp2_ref = {}, {}
    if comp:
        sel2, rc2, rs2, rg2 = P.resq_select_and_requant(h, hq_c, hq_s, hq_g, k, unit_offsets=offs_t,
                                                        rows_total=rows)
        s2r = ref_resq(h_np, hc_r, hs_r, hg_r, offs, k, None, sel2, rc2, rs2, rg2)
        comp2 = dict(sel_idx=sel2, r_codes=rc2, r_scales=rs2, r_global=rg2)
        comp2_ref = dict(sel_idx=s2r[0], r_codes=s2r[1], r_scales=s2r[2], r_g=s2r[3])
    dc, ds, dg = _quant_weights(P, wd)
    dc_r, ds_r, dg_r = ref_weights(wd, dc, ds, dg)
    y = torch.zeros(tokens, hidden, dtype=torch.float32, device="cuda")
    P.moe_w4a4_grouped_gemm(hq_c, hq_s, hq_g, offs_t, rows, dc, ds, dg,
                            epilogue=P.EPI_SCATTER_ADD_F32,
                            row_weight=torch.from_numpy(rt["slot_weight"]).cuda(),
                            scatter_index=slot_tok, out=y, **comp2)
    y_ref = OG.moe_down(hc_r, hs_r, hg_r, offs, dc_r, ds_r, dg_r, rt["slot_token"],
                        rt["slot_weight"], tokens, **comp2_ref)
    assert rel_err(np32(y), y_ref) <= GEMM_TOL


# ---------------------------------------------------------------------------
# trainer side
# ---------------------------------------------------------------------------

def _check_qdq(P, w, want_codes=True):
    wq, c, s, g = P.qdq_weights(w.cuda(), want_codes=want_codes)
    wq_r, c_r, s_r, g_r = OQ.qdq_weights(w.float().numpy())
    assert np.array_equal(np32(g), g_r)
    if want_codes:
        assert np.array_equal(npu8(c), c_r) and np.array_equal(npu8(s), s_r)
    assert np.array_equal(wq.cpu().view(torch.int16).numpy().view(np.uint16), wq_r)


def test_qdq_weights(gpu_lib):
    P = gpu_lib
    w = synth.weights(3, 96, 256, seed=10, tensor_id=synth.WGU_ID)
    w[1, 5, 7] = 3.0                      # one outlier per matrix changes g
    _check_qdq(P, w)


@pytest.mark.parametrize("nmat,n,k,mag,want_codes", [
    (5, 40, 160, 1e-36, True),    # g, S and the outputs are fp32 subnormals
    (2, 64, 128, 1e30, True),     # large values
    (7, 33, 96, 1.0, False),      # odd sizes, no codes out
    (4, 300, 512, 1.0, True),     # several blocks per thread
])
def test_qdq_weights_magnitudes(gpu_lib, nmat, n, k, mag, want_codes):
    """Weight QDQ bit-exact at extreme magnitudes (subnormal global and block
    scales and subnormal bf16 outputs), with zero matrices and zero blocks."""
    P = gpu_lib
    w = synth.weights(nmat, n, k, seed=12, tensor_id=synth.WGU_ID).float() * (mag / 0.02)
    w[0] = 0.0                            # all-zero matrix: g = 1
    w[-1, :, :16] = 0.0                   # zero blocks next to nonzero ones
    _check_qdq(P, w.to(torch.bfloat16), want_codes)


def test_qdq_weights_large_matrix(gpu_lib):
    """One large matrix (512 x 24608, 12.6M elements): its amax is gathered
    from many workgroups and its blocks are quantized by many more."""
    P = gpu_lib
    w = synth.weights(1, 512, 24608, seed=13, tensor_id=synth.WD_ID)
    _check_qdq(P, w)


@pytest.mark.parametrize("nmat,n,k", [
    (9, 2048, 1536),     # 196608 blocks a matrix: four matrices a step, the last step partial
    (5, 3000, 1536),     # two matrices a step, each past one block per thread, last step partial
    (3, 3000, 3072),     # one matrix a step, three blocks per thread, the last ragged
    (2, 3072, 4096),     # one matrix a step, four blocks per thread
])
def test_qdq_weights_one_pass(gpu_lib, nmat, n, k):
    """Weight QDQ of matrices large enough (3.1 M to 12.6 M elements on 256
    CUs) for the one-pass kernel, which holds each matrix on chip from its
    amax to its quantization: every global scale against the oracle's from
    the matrix's amax, the first and last matrices (the last one in a
    partial step) bit-exact, and the give-up flag of its gathers clear."""
    P = gpu_lib
    lib = P.load()
    w = synth.weights(nmat, n, k, seed=14, tensor_id=synth.WGU_ID)
    w[1, 7, 9] = 5.0                                  # one outlier sets a matrix's g
    w[-1] = w[-1] * 1e-20                             # a tiny matrix last
    wc = w.cuda()
    wq = torch.empty_like(wc)
    codes = torch.empty(nmat, n, k // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(nmat, n, k // 16, dtype=torch.uint8, device="cuda")
    g = torch.empty(nmat, dtype=torch.float32, device="cuda")
    ws_bytes = lib.qdq_weights_workspace_size(nmat, n, k)
    ws = torch.full((ws_bytes,), 0x55, dtype=torch.uint8, device="cuda")
    assert lib.qdq_weights(P._ptr(wc), nmat, n, k, P._ptr(wq), P._ptr(codes), P._ptr(scales), P._ptr(g),
                           P._ptr(ws), ws_bytes, P._stream()) == 0
    torch.cuda.synchronize()
    wf = w.float().numpy()
    g_ref = np.array([OQ.global_scale(np.abs(wf[m]).max()) for m in range(nmat)], dtype=np.float32)
    assert np.array_equal(np32(g), g_ref)
    for m in (0, nmat - 1):
        wq_r, c_r, s_r, g_r = OQ.qdq_weights(wf[m:m + 1])
        assert np.array_equal(npu8(codes[m]), c_r[0]) and np.array_equal(npu8(scales[m]), s_r[0])
        assert np.array_equal(wq[m].cpu().view(torch.int16).numpy().view(np.uint16), wq_r[0])
    # the one-pass kernel's give-up flag (the word after 4 x 4 x 1024 slot
    # words), when this device takes the one-pass kernel for the shape
    per = torch.cuda.get_device_properties(0).multi_processor_count * 768
    nb = n * k // 16
    kb = -(-nb // per)
    if nb >= per and kb <= 4 and nmat >= 2 * (4 // kb):
        assert int(ws[16384 * 4:16384 * 4 + 4].view(torch.int32).item()) == 0


@pytest.mark.parametrize("rel", [1e-3, 8e-3, 0.2])
def test_guided_round(gpu_lib, rel):
    P = gpu_lib
    x_roll = synth.activations(257, 512, seed=11, heavy_frac=0.01)
    x_train = synth.guided_noise(x_roll, seed=11, rel=rel)
    rc, rs, rg, _ = P.nvfp4_quantize(x_roll.cuda())
    gc, fq, hist = P.guided_round(x_train.cuda(), rc, rs, rg)
    c_r, s_r, g_r = ref_quant(x_roll, rc, rs, rg)
    gc_r, fq_r, hist_r = OQ.guided_round(x_train.float().numpy(), c_r, s_r, g_r)
    assert np.array_equal(npu8(gc), gc_r)
    assert np.array_equal(fq.cpu().view(torch.int16).numpy().view(np.uint16), fq_r)
    assert np.array_equal(hist.cpu().numpy(), hist_r)


@pytest.mark.parametrize("rel", [1e-3, 8e-3, 0.2])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_guided_round_record(gpu_lib, rel, dtype):
    """Mantissa-only record: the packed low code bits, then guided rounding
    from them (codes, fake-quant values, kept/moved counts), bit-exact."""
    P = gpu_lib
    x_roll = synth.activations(257, 1024, seed=12, heavy_frac=0.01)
    x_train = synth.guided_noise(x_roll, seed=12, rel=rel).to(dtype)
    if dtype == torch.float32:
        x_train = x_train + torch.randn(x_train.shape, generator=torch.Generator().manual_seed(2)) * 1e-4
    rc, rs, rg, _ = P.nvfp4_quantize(x_roll.cuda())
    rec = P.guidance_record_pack(rc)
    c_r, s_r, g_r = ref_quant(x_roll, rc, rs, rg)
    rec_r = OQ.guidance_record(c_r)
    assert np.array_equal(npu8(rec), rec_r)
    gc, fq, moved = P.guided_round_record(x_train.cuda(), rec, rs, rg)
    gc_r, fq_r, moved_r = OQ.guided_round_record(x_train.float().numpy(), rec_r, s_r, g_r)
    assert np.array_equal(npu8(gc), gc_r)
    assert np.array_equal(fq.cpu().view(torch.int16).numpy().view(np.uint16), fq_r)
    assert np.array_equal(moved.cpu().numpy(), moved_r)
    if rel < 0.1:
        assert moved_r[1] > 0


def test_guided_round_grid_stride_and_stride(gpu_lib):
    """2100 x 2048 with a padded row stride: 537600 eight-element items, more
    than one grid's worth (512 workgroups of 1024 lanes), so lanes take a
    second, ragged trip with their prefetched item; codes, fake-quant values,
    histogram and record form bit-exact against the oracle."""
    P = gpu_lib
    m, k, ld = 2100, 2048, 2056
    x_roll = synth.activations(m, k, seed=41, heavy_frac=0.01)
    x_train = synth.guided_noise(x_roll, seed=41, rel=8e-3)
    buf = torch.zeros(m, ld, dtype=x_train.dtype)
    buf[:, :k] = x_train
    xt = buf.cuda()[:, :k]
    assert xt.stride(0) == ld and m * k // 8 > 512 * 1024
    rc, rs, rg, _ = P.nvfp4_quantize(x_roll.cuda())
    c_r, s_r, g_r = ref_quant(x_roll, rc, rs, rg)
    xt_np = x_train.float().numpy()
    gc, fq, hist = P.guided_round(xt, rc, rs, rg)
    gc_r, fq_r, hist_r = OQ.guided_round(xt_np, c_r, s_r, g_r)
    assert np.array_equal(npu8(gc), gc_r) and np.array_equal(hist.cpu().numpy(), hist_r)
    assert np.array_equal(fq.cpu().view(torch.int16).numpy().view(np.uint16), fq_r)
    rec = P.guidance_record_pack(rc)
    gc2, fq2, moved = P.guided_round_record(xt, rec, rs, rg)
    gc2_r, fq2_r, moved_r = OQ.guided_round_record(xt_np, OQ.guidance_record(c_r), s_r, g_r)
    assert np.array_equal(npu8(gc2), gc2_r) and np.array_equal(moved.cpu().numpy(), moved_r)
    assert np.array_equal(fq2.cpu().view(torch.int16).numpy().view(np.uint16), fq2_r)


@pytest.mark.parametrize("padded", [False, True])
def test_kv_cache_quantize_and_guided(gpu_lib, padded):
    """KV-cache shapes: a key cache [300 tokens, 4 heads, 128] viewed as 1200
    rows of head_dim (blocks along head_dim), quantized under a calibrated
    global scale (amax_in above the data's amax), then guided rounding of the
    trainer's cache from the full codes and from the mantissa-only record; with
    and without a padded row stride (a cache laid out [tokens, heads, 136])."""
    P = gpu_lib
    t, h, d = 300, 4, 128
    k_roll = synth.kv_cache(t, h, d, seed=31)
    k_train = synth.guided_noise(k_roll, seed=31, rel=8e-3)
    amax = np.float32(float(k_roll.float().abs().max()) * 1.25)
    g_ref = OQ.global_scale(amax)

    def dev_rows(x):
        if not padded:
            return x.reshape(t * h, d).cuda()
        buf = torch.zeros(t, h, d + 8, dtype=x.dtype)
        buf[:, :, :d] = x
        return buf.cuda().reshape(t * h, d + 8)[:, :d]

    xr, xt = dev_rows(k_roll), dev_rows(k_train)
    assert xr.stride(0) == (d + 8 if padded else d)
    rc, rs, rg, _ = P.nvfp4_quantize(xr, amax_in=torch.tensor([amax], device="cuda"))
    xr_np = k_roll.reshape(t * h, d).float().numpy()
    xt_np = k_train.reshape(t * h, d).float().numpy()
    c_ref, s_ref, _ = OQ.quantize(xr_np, g=g_ref)
    assert np32(rg)[0] == g_ref
    assert np.array_equal(npu8(rc), c_ref) and np.array_equal(npu8(rs), s_ref)
    gc, fq, hist = P.guided_round(xt, rc, rs, rg)
    gc_r, fq_r, hist_r = OQ.guided_round(xt_np, c_ref, s_ref, g_ref)
    assert np.array_equal(npu8(gc), gc_r) and np.array_equal(hist.cpu().numpy(), hist_r)
    assert np.array_equal(fq.cpu().view(torch.int16).numpy().view(np.uint16), fq_r)
    rec = P.guidance_record_pack(rc)
    gc2, fq2, moved = P.guided_round_record(xt, rec, rs, rg)
    gc2_r, fq2_r, moved_r = OQ.guided_round_record(xt_np, OQ.guidance_record(c_ref), s_ref, g_ref)
    assert np.array_equal(npu8(gc2), gc2_r) and np.array_equal(moved.cpu().numpy(), moved_r)
    assert np.array_equal(fq2.cpu().view(torch.int16).numpy().view(np.uint16), fq2_r)


def test_guidance_record_pack_exhaustive_bytes(gpu_lib):
    """Every code byte value in every position of a 16-element group."""
    P = gpu_lib
    codes = torch.arange(256, dtype=torch.int32).repeat(8 * 16).reshape(-1, 64).to(torch.uint8)
    codes = codes[torch.randperm(codes.shape[0], generator=torch.Generator().manual_seed(4))]
    rec = P.guidance_record_pack(codes.cuda())
    assert np.array_equal(npu8(rec), OQ.guidance_record(codes.numpy()))


@pytest.mark.parametrize("tokens,n_exp,top_k,zipf", [
    (600, 2, 2, 0.0),     # 600 rows per expert: 256-row tiles, last one 88 rows
    (340, 4, 2, 0.3),     # ~170 rows per expert: one 256-row tile, waves with 2-4 live fragments
    (300, 4, 2, 0.5),     # 150 rows per expert: 128-row tiles
    (200, 8, 2, 1.0),     # 50 rows per expert: 64-row tiles
    (64, 16, 4, 0.0),     # 16 rows per expert: 32-row tiles
])
def test_grouped_gemm_tile_variants(gpu_lib, tokens, n_exp, top_k, zipf):
    """Every tile shape of the grouped GEMM (chosen from the average rows per
    expert) against the reference, with compensation, F32 and SwiGLU epilogues,
    K = 320 (a K-step count that is not a power of two) and N = 2 x 160 (a
    partial N tile)."""
    P = gpu_lib
    hidden, inter, k = 320, 160, 32
    x, rt, offs, wgu, _ = _moe_setup(P, tokens, hidden, n_exp, inter, k, seed=21, zipf=zipf,
                                     top_k=top_k)
    xc = x.cuda()
    rows = int(offs[-1])
    offs_t = torch.from_numpy(offs).cuda()
    slot_tok = torch.from_numpy(rt["slot_token"]).cuda()
    codes, scales, g, _ = P.nvfp4_quantize(xc)
    sel, rc, rs, rg = P.resq_select_and_requant(xc, codes, scales, g, k, unit_offsets=offs_t,
                                                rows_total=rows, row_index=slot_tok)
    gc, gs, gg = _quant_weights(P, wgu)
    comp = dict(sel_idx=sel, r_codes=rc, r_scales=rs, r_global=rg)
    gu = P.moe_w4a4_grouped_gemm(codes, scales, g, offs_t, rows, gc, gs, gg, a_row_index=slot_tok,
                                 **comp)
    h = P.moe_w4a4_grouped_gemm(codes, scales, g, offs_t, rows, gc, gs, gg, a_row_index=slot_tok,
                                epilogue=P.EPI_SWIGLU_BF16, **comp)
    x_np = x.float().numpy()
    c_r, s_r, g_r = ref_quant(x_np, codes, scales, g)
    sel_r, rc_r, rs_r, rg_r = ref_resq(x_np, c_r, s_r, g_r, offs, k, rt["slot_token"],
                                       sel, rc, rs, rg)
    gc_r, gs_r, gg_r = ref_weights(wgu, gc, gs, gg)
    gu_ref, h_ref = OG.moe_gate_up(c_r, s_r, g_r, rt["slot_token"], offs, gc_r, gs_r, gg_r, inter,
                                   sel_idx=sel_r, r_codes=rc_r, r_scales=rs_r, r_g=rg_r)
    gu_np = np32(gu)
    for e in range(n_exp):
        a, b = offs[e], offs[e + 1]
        if a < b:
            assert rel_err(gu_np[a:b], gu_ref[a:b]) <= GEMM_TOL, f"expert {e}"
    h_r = F.bf16_bits_to_f32(h_ref)
    tol = np.abs(h_r) * 2.0 ** -7 + GEMM_TOL * np.abs(h_r).max()
    assert np.all(np.abs(np32(h) - h_r) <= tol)


def test_scatter_add_fixed_order_and_ragged_n(gpu_lib):
    """Scatter-add epilogue: each output row receives its rows in increasing
    row order on top of the caller's initial values, for an N that is not a
    multiple of 4; two runs are bit-identical."""
    P = gpu_lib
    tokens, hidden, n_exp, inter = 96, 100, 5, 64
    rng = np.random.default_rng(3)
    h = torch.from_numpy(rng.standard_normal((tokens * 3, inter)).astype(np.float32)).to(torch.bfloat16)
    rt = synth.route(tokens, n_exp, seed=13, top_k=3)
    offs = rt["offsets"]
    rows = int(offs[-1])
    wd = synth.weights(n_exp, hidden, inter, seed=13, tensor_id=synth.WD_ID)
    hc, hs, hg, _ = P.nvfp4_quantize(h.cuda())
    dc, ds, dg = _quant_weights(P, wd)
    y0 = torch.from_numpy(rng.standard_normal((tokens, hidden)).astype(np.float32))
    outs = []
    for _ in range(2):
        y = y0.clone().cuda()
        P.moe_w4a4_grouped_gemm(hc, hs, hg, torch.from_numpy(offs).cuda(), rows, dc, ds, dg,
                                epilogue=P.EPI_SCATTER_ADD_F32,
                                row_weight=torch.from_numpy(rt["slot_weight"]).cuda(),
                                scatter_index=torch.from_numpy(rt["slot_token"]).cuda(), out=y)
        outs.append(np32(y))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    hc_r, hs_r, hg_r = ref_quant(h, hc, hs, hg)
    dc_r, ds_r, dg_r = ref_weights(wd, dc, ds, dg)
    y_gemm = OG.moe_down(hc_r, hs_r, hg_r, offs, dc_r, ds_r, dg_r, rt["slot_token"],
                         rt["slot_weight"], tokens)
    y_ref = y0.numpy().astype(np.float64) + y_gemm
    assert rel_err(outs[0], y_ref) <= GEMM_TOL
    # the added part alone, so that the initial values (about 10x the GEMM's
    # magnitude here) do not loosen the tolerance on it; subtracting y0 in
    # float64 from the fp32 output adds at most half an fp32 ulp of |y|
    assert rel_err(outs[0].astype(np.float64) - y0.numpy().astype(np.float64), y_gemm) <= GEMM_TOL


@pytest.mark.gpu
def test_scatter_overwrite_equals_add_into_zeros(gpu_lib):
    """EPI_SCATTER_F32 writes the same sums as EPI_SCATTER_ADD_F32 into a
    zeroed out, bit for bit; output rows that no slot names (here the five
    past the tokens) and an out full of NaN before the call end as zeros; a
    launch with no rows writes zeros everywhere."""
    P = gpu_lib
    tokens, hidden, n_exp, inter = 96, 100, 5, 64
    rng = np.random.default_rng(4)
    h = torch.from_numpy(rng.standard_normal((tokens * 3, inter)).astype(np.float32)).to(torch.bfloat16)
    rt = synth.route(tokens, n_exp, seed=14, top_k=3)
    offs = torch.from_numpy(rt["offsets"]).cuda()
    rows = int(rt["offsets"][-1])
    wd = synth.weights(n_exp, hidden, inter, seed=14, tensor_id=synth.WD_ID)
    hc, hs, hg, _ = P.nvfp4_quantize(h.cuda())
    dc, ds, dg = _quant_weights(P, wd)
    kw = dict(row_weight=torch.from_numpy(rt["slot_weight"]).cuda(),
              scatter_index=torch.from_numpy(rt["slot_token"]).cuda())
    out_rows = tokens + 5
    y_add = torch.zeros(out_rows, hidden, dtype=torch.float32, device="cuda")
    P.moe_w4a4_grouped_gemm(hc, hs, hg, offs, rows, dc, ds, dg, epilogue=P.EPI_SCATTER_ADD_F32,
                            out=y_add, **kw)
    y_ow = torch.full((out_rows, hidden), float("nan"), dtype=torch.float32, device="cuda")
    P.moe_w4a4_grouped_gemm(hc, hs, hg, offs, rows, dc, ds, dg, epilogue=P.EPI_SCATTER_F32,
                            out=y_ow, **kw)
    a, b = np32(y_add), np32(y_ow)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.all(b[tokens:] == 0.0) and np.all(np.abs(b[:tokens]).sum(axis=1) > 0)
    y_alloc = P.moe_w4a4_grouped_gemm(hc, hs, hg, offs, rows, dc, ds, dg, epilogue=P.EPI_SCATTER_F32,
                                      out_rows=out_rows, **kw)
    assert np.array_equal(np32(y_alloc).view(np.uint32), a.view(np.uint32))
    y_none = torch.full((out_rows, hidden), float("nan"), dtype=torch.float32, device="cuda")
    P.moe_w4a4_grouped_gemm(hc, hs, hg, torch.zeros(n_exp + 1, dtype=torch.int64, device="cuda"), 0,
                            dc, ds, dg, epilogue=P.EPI_SCATTER_F32, out=y_none, **kw)
    assert np.all(np32(y_none) == 0.0)


@pytest.mark.gpu
def test_grouped_gemm_tail_split_graph_replays(gpu_lib):
    """Groups of 256 rows and more take 256-row tiles plus a launch of 32-row
    tiles for their ragged remainders (on the library's second stream when
    eager, on the capturing stream under capture); the call captured in a HIP
    graph and replayed (eager work in between) gives the eager result bit for
    bit every time."""
    P = gpu_lib
    rng = np.random.default_rng(21)
    counts = np.array([300, 280, 512, 261], dtype=np.int64)          # remainders 44, 24, 0, 5
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows, n_exp, K, N = int(offs[-1]), len(counts), 256, 512
    x = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32)).to(torch.bfloat16).cuda()
    w = synth.weights(n_exp, N, K, seed=21, tensor_id=synth.WD_ID)
    xc, xs, xg, _ = P.nvfp4_quantize(x)
    wc, ws, wg = _quant_weights(P, w)
    offs_t = torch.from_numpy(offs).cuda()
    y0 = P.moe_w4a4_grouped_gemm(xc, xs, xg, offs_t, rows, wc, ws, wg)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y = P.moe_w4a4_grouped_gemm(xc, xs, xg, offs_t, rows, wc, ws, wg)
    for _ in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y0.view(torch.int32))
    # and the eager result against the oracle
    xc_r, xs_r, xg_r = ref_quant(x.cpu(), xc, xs, xg)
    wc_r, ws_r, wg_r = ref_weights(w, wc, ws, wg)
    for e in range(n_exp):
        a, b = int(offs[e]), int(offs[e + 1])
        ref = OG.gemm_comp(xc_r[a:b], xs_r[a:b], xg_r, wc_r[e], ws_r[e], wg_r[e])
        assert rel_err(np32(y0)[a:b], ref) <= GEMM_TOL, f"group {e}"
