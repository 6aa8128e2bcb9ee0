"""GPU parity of the dense binary-mask compensation (QUADS section 2.2B: the
top k% of channels by residual magnitude, 50% in the pages' example, are
quantized a second time and their GEMM term added back) against the oracle.

The masked residual step is compared bit for bit (selection, codes, block
scales, global scales); the GEMM within GEMM_TOL of the oracle's float64
product, as the other GEMM tests.
"""

import numpy as np
import pytest
import torch

import synth
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


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("hidden,frac", [(256, 0.5), (512, 0.25), (1536, 0.5)])
def test_mask_resq_gathered_expert_units(gpu_lib, dtype, hidden, frac):
    """Units = experts' routed tokens through the slot->token map, skewed
    loads, an empty expert, units longer than a 128-row tile."""
    P = gpu_lib
    tokens, n_exp = 300, 5
    k = int(hidden * frac)
    x = synth.activations(tokens, hidden, seed=31, heavy_frac=0.02).to(dtype)
    rt = synth.route(tokens, n_exp, seed=31, top_k=2, zipf_s=1.2)
    offs = rt["offsets"].copy()
    offs[3] = offs[2]                                   # expert 2 empty
    xc = x.cuda()
    codes, scales, g, _ = P.nvfp4_quantize(xc)
    sel, mc, ms, mg = P.resq_mask_select_and_requant(
        xc, codes, scales, g, k, unit_offsets=torch.from_numpy(offs).cuda(),
        rows_total=int(offs[-1]), row_index=torch.from_numpy(rt["slot_token"]).cuda())
    x_np = x.float().numpy()
    c_ref, s_ref, g_ref = OQ.quantize(x_np)
    assert np.array_equal(npu8(codes), c_ref)
    sel_r, mc_r, ms_r, mg_r = OQ.resq_mask_select_and_requant(x_np, c_ref, s_ref, g_ref, offs, k,
                                                              row_index=rt["slot_token"])
    assert np.diff(offs).max() > 128
    assert np.array_equal(npu8(sel), sel_r)
    assert np.array_equal(np32(mg), mg_r)
    assert np.array_equal(npu8(ms), ms_r)
    assert np.array_equal(npu8(mc), mc_r)


@pytest.mark.parametrize("m,k_dim,k", [(300, 4096, 2048), (129, 512, 512), (40, 2048, 16)])
def test_mask_resq_tile_units(gpu_lib, m, k_dim, k):
    """Units = the 128-row tiles of x, scores from the quantizer's partials;
    the full mask (k = K) and a ragged last tile."""
    P = gpu_lib
    x = synth.activations(m, k_dim, seed=32, heavy_frac=0.01)
    xc = x.cuda()
    codes, scales, g, part = P.nvfp4_quantize(xc, tile_partials=True)
    sel, mc, ms, mg = P.resq_mask_select_and_requant(xc, codes, scales, g, k, tile_partials=part)
    x_np = x.float().numpy()
    c_ref, s_ref, g_ref = OQ.quantize(x_np)
    offs = np.minimum(np.arange(0, m + 128, 128), m)
    offs = np.unique(np.r_[offs, m])
    sel_r, mc_r, ms_r, mg_r = OQ.resq_mask_select_and_requant(x_np, c_ref, s_ref, g_ref, offs, k)
    assert np.array_equal(npu8(sel), sel_r)
    assert np.array_equal(np32(mg), mg_r)
    assert np.array_equal(npu8(ms), ms_r)
    assert np.array_equal(npu8(mc), mc_r)


@pytest.mark.parametrize("tokens,n_exp,top_k,zipf", [
    (600, 2, 2, 0.0),     # 256-row tiles, ragged last
    (300, 4, 2, 0.5),     # 128-row tiles
    (200, 8, 2, 1.0),     # 64-row tiles
    (64, 16, 4, 0.0),     # 32-row tiles
])
def test_masked_comp_gemm_tile_variants(gpu_lib, tokens, n_exp, top_k, zipf):
    """Main product (F32) then the masked term accumulated into it, for
    every tile shape, with a 50% mask, K = 320 and a partial N tile."""
    P = gpu_lib
    hidden, inter = 320, 160
    k = hidden // 2
    x = synth.activations(tokens, hidden, seed=33, heavy_frac=0.01)
    rt = synth.route(tokens, n_exp, seed=33, top_k=top_k, zipf_s=zipf)
    offs = rt["offsets"]
    wgu = synth.weights(n_exp, 2 * inter, hidden, seed=33, tensor_id=synth.WGU_ID)
    xc = x.cuda()
    rows = int(offs[-1])
    offs_t = torch.from_numpy(offs).cuda()
    slot_tok = torch.from_numpy(rt["slot_token"]).cuda()
    codes, scales, g, _ = P.nvfp4_quantize(xc)
    sel, mc, ms, mg = P.resq_mask_select_and_requant(xc, codes, scales, g, k, unit_offsets=offs_t,
                                                     rows_total=rows, row_index=slot_tok)
    _, gc, gs, gg = P.qdq_weights(wgu.cuda())
    y = P.moe_w4a4_grouped_gemm(codes, scales, g, offs_t, rows, gc, gs, gg, a_row_index=slot_tok)
    y0 = y.clone()
    P.moe_w4a4_masked_comp_gemm(mc, ms, mg, offs_t, rows, gc, gs, gg, out=y)
    y_np, y0_np = np32(y), np32(y0)
    # the oracle's own operands, after checking the GPU's are identical
    x_np = x.float().numpy()
    c_np, s_np, g_np = OQ.quantize(x_np)
    assert np.array_equal(npu8(codes), c_np) and np32(g)[0] == g_np
    _, mc_np, ms_np, mg_np = OQ.resq_mask_select_and_requant(x_np, c_np, s_np, g_np, offs, k,
                                                             row_index=rt["slot_token"])
    assert np.array_equal(npu8(mc), mc_np) and np.array_equal(np32(mg), mg_np)
    _, gc_np, gs_np, gg_np = OQ.qdq_weights(wgu.float().numpy())
    assert np.array_equal(npu8(gc), gc_np) and np.array_equal(np32(gg), gg_np)
    for e in range(n_exp):
        a, b = offs[e], offs[e + 1]
        if a == b:
            continue
        tok = rt["slot_token"][a:b]
        ref = OG.gemm_masked_comp(c_np[tok], s_np[tok], g_np, gc_np[e], gs_np[e], gg_np[e],
                                  mc_np[a:b], ms_np[a:b], mg_np[e])
        ref0 = OG.gemm_comp(c_np[tok], s_np[tok], g_np, gc_np[e], gs_np[e], gg_np[e])
        assert rel_err(y_np[a:b], ref) <= GEMM_TOL, f"expert {e}"
        assert rel_err(y0_np[a:b], ref0) <= GEMM_TOL, f"expert {e}"


def test_masked_comp_moves_toward_exact(gpu_lib):
    """With a 50% mask the compensated product is closer to the product of
    the unquantized activation with the stored weight than the plain one, and
    closer than the 32-channel compact form."""
    P = gpu_lib
    tokens, hidden, n_out = 256, 1024, 512
    x = synth.activations(tokens, hidden, seed=34, heavy_frac=0.01)
    w = synth.weights(1, n_out, hidden, seed=34, tensor_id=synth.WDENSE_ID)
    xc = x.cuda()
    codes, scales, g, _ = P.nvfp4_quantize(xc)
    offs = torch.tensor([0, tokens], dtype=torch.int64, device="cuda")
    _, wc, ws_, wg = P.qdq_weights(w.cuda())
    y0 = P.moe_w4a4_grouped_gemm(codes, scales, g, offs, tokens, wc, ws_, wg)
    sel, rc, rs, rg = P.resq_select_and_requant(xc, codes, scales, g, 32, unit_offsets=offs,
                                                rows_total=tokens)
    yc = P.moe_w4a4_grouped_gemm(codes, scales, g, offs, tokens, wc, ws_, wg, sel_idx=sel,
                                 r_codes=rc, r_scales=rs, r_global=rg)
    _, mc, ms, mg = P.resq_mask_select_and_requant(xc, codes, scales, g, hidden // 2,
                                                   unit_offsets=offs, rows_total=tokens)
    ym = y0.clone()
    P.moe_w4a4_masked_comp_gemm(mc, ms, mg, offs, tokens, wc, ws_, wg, out=ym)
    _, wc_r, ws_r, wg_r = OQ.qdq_weights(w.float().numpy())
    assert np.array_equal(npu8(wc), wc_r)
    exact = x.float().numpy().astype(np.float64) @ OQ.dequantize(
        wc_r[0], ws_r[0], wg_r[0]).astype(np.float64).T
    e0, ec, em = (np.linalg.norm(np32(t) - exact) for t in (y0, yc, ym))
    assert em < ec < e0
