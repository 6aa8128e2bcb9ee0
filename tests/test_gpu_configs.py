"""Parity at the shapes of the three workloads between the dense linear and the
8192-token layer, in the launch configurations the bench times:

  * the quantizer + residual-selection workload (X [16384 x 4096], 1% heavy
    channels, top-128 per 128-token tile),
  * the decode-shaped MoE layer (256 tokens, H 2048, 128 experts, I 768,
    top-8, k 64), whose grouped GEMMs run the 32-row tile,
  * the Zipf(1.1)-skewed prefill layer (16384 tokens, same dimensions): about
    15.9k routed rows on expert 0 (one selection unit of about 124 score
    tiles) and experts with only a few rows.

The GPU runs the bench's own input builder and step; the oracle recomputes
sampled outputs from the seeded inputs alone (never from a GPU result):
global scales from its own amax of the whole tensor, codes, scales,
selections and Q(R_S) bit-exact, GEMM rows within max|dY| / max|Y| <= 1e-3.
The down projection runs at full size on seeded activations of its own, as
the oracle cannot recompute amax(h) of a whole gate/up output it only
samples.

Also here: the compensation's combination of global scales when the
residual's global scale is tiny next to the activation's (a unit that is
representable but for one tiny element).
"""

import numpy as np
import pytest
import torch

import bench
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


def bits32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _layer(P, name):
    wl = synth.WORKLOADS[name]
    inp, _ = bench.build_inputs(torch, P, synth, wl, torch.device("cuda"))
    out = bench.run_step(P, inp, wl, bench.Timeline(torch), trainer=False)
    torch.cuda.synchronize()
    return wl, inp, out


def _check_expert_rollout(P, wl, inp, out, x, g, e, n_rows_h):
    """Expert e of a MoE layer: the codes and scales of its token rows, its
    selection and Q(R_S) bit-exact; its weights' codes bit-exact; n_rows_h
    sampled rows of the SwiGLU output against the oracle's compensated GEMM."""
    offs = inp["routing"]["offsets"]
    a, b = int(offs[e]), int(offs[e + 1])
    tok = inp["routing"]["slot_token"][a:b]
    xq_c, xq_s, _ = out["xq"]
    sel, rc, rs, rg = out["sel1"]
    c_r, s_r, _ = OQ.quantize(x[tok], g=g)
    idx = torch.from_numpy(tok.astype(np.int64)).cuda()
    assert np.array_equal(npu8(xq_c[idx]), c_r), f"expert {e} codes"
    assert np.array_equal(npu8(xq_s[idx]), s_r), f"expert {e} scales"
    sel_r, rc_r, rs_r, rg_r = OQ.resq_select_and_requant(x[tok], c_r, s_r, g, [0, b - a], wl.k)
    assert np.array_equal(npu8(sel[e]), sel_r[0]), f"expert {e} selection"
    assert np32(rg)[e] == rg_r[0]
    assert np.array_equal(npu8(rc[a:b]), rc_r) and np.array_equal(npu8(rs[a:b]), rs_r)
    _, wc, ws, wg = OQ.qdq_weights(np32(inp["wgu"][e:e + 1]))
    assert np.array_equal(npu8(inp["gc"][e]), wc[0]) and np.array_equal(npu8(inp["gs"][e]), ws[0])
    assert np32(inp["gg"])[e] == wg[0]
    rng = np.random.default_rng(100 + e)
    rows = np.arange(b - a) if b - a <= n_rows_h else np.sort(rng.choice(b - a, n_rows_h, replace=False))
    gu = OG.gemm_comp(c_r[rows], s_r[rows], g, wc[0], ws[0], wg[0], sel_r[0], rc_r[rows], rs_r[rows],
                      rg_r[0])
    h_r = F.bf16_bits_to_f32(OG.swiglu_bf16(gu, wl.inter))
    h_g = np32(out["h"][torch.from_numpy(a + rows).cuda()])
    tol = np.abs(h_r) * 2.0 ** -7 + GEMM_TOL * np.abs(h_r).max()
    assert np.all(np.abs(h_g - h_r) <= tol), f"expert {e} SwiGLU rows"


def _check_down_tokens(P, wl, tokens, seed):
    """The down projection of a whole layer (all routed rows, compensated,
    fixed-order scatter-add) on seeded activations, against the oracle for
    the given tokens, each summing its top-8 slots from their own experts."""
    rt = synth.route(wl.tokens, wl.experts, seed=wl.seed, top_k=wl.top_k, zipf_s=wl.zipf_s)
    offs = rt["offsets"]
    rows = int(offs[-1])
    h = synth.activations(rows, wl.inter, seed=seed, device="cuda", heavy_frac=0.01)
    wd = synth.weights(wl.experts, wl.hidden, wl.inter, seed=wl.seed, tensor_id=synth.WD_ID,
                       device="cuda")
    _, dc, ds, dg = P.qdq_weights(wd)
    offs_t = torch.from_numpy(offs).cuda()
    hq_c, hq_s, hq_g, _ = P.nvfp4_quantize(h)
    sel, rc, rs, rg = P.resq_select_and_requant(h, hq_c, hq_s, hq_g, wl.k, unit_offsets=offs_t,
                                                rows_total=rows)
    y = torch.zeros(wl.tokens, wl.hidden, dtype=torch.float32, device="cuda")
    P.moe_w4a4_grouped_gemm(hq_c, hq_s, hq_g, offs_t, rows, dc, ds, dg,
                            epilogue=P.EPI_SCATTER_ADD_F32, sel_idx=sel, r_codes=rc, r_scales=rs,
                            r_global=rg, row_weight=torch.from_numpy(rt["slot_weight"]).cuda(),
                            scatter_index=torch.from_numpy(rt["slot_token"]).cuda(), out=y)
    y_np, h_np = np32(y), np32(h)
    g = OQ.global_scale(np.abs(h_np).max())
    assert np32(hq_g)[0] == g
    slot_expert = np.repeat(np.arange(wl.experts), np.diff(offs))
    cache = {}
    for t in tokens:
        slots = np.nonzero(rt["slot_token"] == t)[0]
        assert slots.size == wl.top_k
        ref = np.zeros(wl.hidden)
        for s in slots:
            e = int(slot_expert[s])
            a, b = int(offs[e]), int(offs[e + 1])
            if e not in cache:
                c_ref, s_ref, _ = OQ.quantize(h_np[a:b], g=g)
                assert np.array_equal(npu8(hq_c[a:b]), c_ref)
                sel_r, rc_r, rs_r, rg_r = OQ.resq_select_and_requant(h_np[a:b], c_ref, s_ref, g,
                                                                     [0, b - a], wl.k)
                assert np.array_equal(npu8(sel[e]), sel_r[0]) and np32(rg)[e] == rg_r[0]
                _, wc, ws, wg = OQ.qdq_weights(np32(wd[e:e + 1]))
                cache[e] = (c_ref, s_ref, sel_r[0], rc_r, rs_r, rg_r[0], wc[0], ws[0], wg[0])
            c_ref, s_ref, sel_e, rc_r, rs_r, rg_e, wc, ws, wg = cache[e]
            r = s - a
            row = OG.gemm_comp(c_ref[r:r + 1], s_ref[r:r + 1], g, wc, ws, wg, sel_e,
                               rc_r[r:r + 1], rs_r[r:r + 1], rg_e)[0]
            ref += float(rt["slot_weight"][s]) * row
        err = np.abs(y_np[t] - ref).max() / np.abs(ref).max()
        assert err <= GEMM_TOL, f"token {t}: {err}"
    return rt


# ---------------------------------------------------------------------------
# quantizer + residual selection, 16384 x 4096, 128-token tiles, k = 128
# ---------------------------------------------------------------------------

def test_quant_select_full_shape(gpu_lib):
    """Sampled tiles (the first, two inner, the last) of the 128 tile units:
    codes, scales, the fused score partials, the selected channels and the
    requantized residual bit-exact; the global scale from the oracle's amax
    of the whole tensor."""
    P = gpu_lib
    wl = synth.WORKLOADS["quant_select_T16384_K4096_k128"]
    x = synth.activations(wl.tokens, wl.hidden, seed=wl.seed, device="cuda",
                          heavy_frac=wl.heavy_frac)
    c, s, g, tp = P.nvfp4_quantize(x, tile_partials=True)
    sel, rc, rs, rg = P.resq_select_and_requant(x, c, s, g, wl.k, tile_partials=tp)
    torch.cuda.synchronize()
    x_np = np32(x)
    g_r = OQ.global_scale(np.abs(x_np).max())
    assert np32(g)[0] == g_r
    n_tiles = wl.tokens // 128
    assert sel.shape[0] == n_tiles
    for t in (0, 37, 90, n_tiles - 1):
        rows = slice(128 * t, 128 * t + 128)
        c_r, s_r, _ = OQ.quantize(x_np[rows], g=g_r)
        assert np.array_equal(npu8(c[rows]), c_r), f"tile {t} codes"
        assert np.array_equal(npu8(s[rows]), s_r), f"tile {t} scales"
        part = OQ.channel_scores(np.abs(OQ.residual(x_np[rows], c_r, s_r, g_r)))
        assert np.array_equal(bits32(np32(tp[t])), bits32(part)), f"tile {t} score partials"
        sel_r, rc_r, rs_r, rg_r = OQ.resq_select_and_requant(x_np[rows], c_r, s_r, g_r,
                                                             [0, 128], wl.k)
        assert np.array_equal(npu8(sel[t]), sel_r[0]), f"tile {t} selection"
        assert np32(rg)[t] == rg_r[0]
        assert np.array_equal(npu8(rc[rows]), rc_r) and np.array_equal(npu8(rs[rows]), rs_r)


# ---------------------------------------------------------------------------
# decode-shaped MoE layer: 256 tokens, H 2048, 128 experts, I 768, k 64
# ---------------------------------------------------------------------------

def test_decode_layer_full_shape(gpu_lib):
    """The whole X quantization and every expert's selection and Q(R_S)
    bit-exact; every row of the largest, the smallest non-empty and four other
    experts through the gate/up GEMM (32-row tile, K 2048, N 1536,
    compensated) and SwiGLU; the down projection (K 768) on two tokens."""
    P = gpu_lib
    wl, inp, out = _layer(P, "moe_decode_T256_H2048_E128_I768_k64")
    assert inp["rows"] // wl.experts < 24          # the library picks its 32-row tile
    x = np32(inp["x"])
    g = OQ.global_scale(np.abs(x).max())
    xq_c, xq_s, xq_g = out["xq"]
    assert np32(xq_g)[0] == g
    c_r, s_r, _ = OQ.quantize(x, g=g)
    assert np.array_equal(npu8(xq_c), c_r) and np.array_equal(npu8(xq_s), s_r)
    offs = inp["routing"]["offsets"]
    sel, rc, rs, rg = out["sel1"]
    sel_r, rc_r, rs_r, rg_r = OQ.resq_select_and_requant(x, c_r, s_r, g, offs, wl.k,
                                                         row_index=inp["routing"]["slot_token"])
    assert np.array_equal(npu8(sel), sel_r) and np.array_equal(bits32(np32(rg)), bits32(rg_r))
    assert np.array_equal(npu8(rc), rc_r) and np.array_equal(npu8(rs), rs_r)
    counts = np.diff(offs)
    live = np.nonzero(counts)[0]
    sample = sorted({int(live[np.argmax(counts[live])]), int(live[np.argmin(counts[live])]),
                     int(live[0]), int(live[len(live) // 3]), int(live[2 * len(live) // 3]),
                     int(live[-1])})
    for e in sample:
        _check_expert_rollout(P, wl, inp, out, x, g, e, n_rows_h=64)
    _check_down_tokens(P, wl, tokens=(3, 200), seed=66)


# ---------------------------------------------------------------------------
# Zipf-skewed prefill layer: 16384 tokens, same dimensions
# ---------------------------------------------------------------------------

def test_prefill_zipf_full_shape(gpu_lib):
    """The hot expert's selection over its ~15.9k rows (about 124 score
    tiles in one unit) and its Q(R_S) bit-exact, with 24 sampled SwiGLU rows;
    a tail expert with fewer than 16 rows in full; the down projection on two
    tokens, one of them routed to the hot expert."""
    P = gpu_lib
    wl, inp, out = _layer(P, "moe_prefill_T16384_H2048_E128_I768_zipf1.1_k64")
    offs = inp["routing"]["offsets"]
    counts = np.diff(offs)
    hot = int(np.argmax(counts))
    assert counts[hot] > 15000, "the Zipf bias puts about 15.9k rows on one expert"
    tail = [e for e in range(wl.experts) if 0 < counts[e] < 16]
    assert tail, "some experts get fewer than 16 rows"
    x = np32(inp["x"])
    g = OQ.global_scale(np.abs(x).max())
    assert np32(out["xq"][2])[0] == g
    _check_expert_rollout(P, wl, inp, out, x, g, hot, n_rows_h=24)
    _check_expert_rollout(P, wl, inp, out, x, g, tail[0], n_rows_h=16)
    # a token whose slots include the hot expert, and one more
    rt = inp["routing"]
    hot_tokens = rt["slot_token"][offs[hot]:offs[hot + 1]]
    _check_down_tokens(P, wl, tokens=(int(hot_tokens[7]), 12345), seed=67)


# ---------------------------------------------------------------------------
# compensation with a residual global scale far below the activation's
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows0,rows1", [(40, 72), (12, 20), (300, 260)])
def test_comp_tiny_residual_global_scale(gpu_lib, rows0, rows1):
    """Expert 1's rows are exactly representable in NVFP4 (E2M1 levels under
    block scale 1 and global scale 1) except one element of 2^-120 that
    quantizes to 0, so its residual, and the global scale of its Q(R_S),
    are about 2^-131 while the activation's global scale is 1: the ratio of
    the two is about 2^131.  Expert 0 holds the tensor's amax 2688.  The
    result must stay finite and within the GEMM tolerance of the oracle, for
    rows per expert that select the 64-, 32- and 256-row tiles."""
    P = gpu_lib
    rng = np.random.default_rng(71)
    levels = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    k_dim, n_out, kc = 256, 192, 32
    x = torch.from_numpy((rng.standard_normal((rows0 + rows1, k_dim)) * 0.5).astype(np.float32))
    x = x.to(torch.bfloat16).float().numpy()                 # bf16 values
    x[3, 17] = 2688.0                                        # tensor amax: g = 1
    rep = rng.choice(levels, size=(rows1, k_dim)) * rng.choice([-1.0, 1.0], size=(rows1, k_dim))
    rep[:, ::16] = 6.0                                       # every block's amax is 6: scale 1
    rep[5, 35] = 2.0 ** -120                                 # the one non-representable element
    x[rows0:] = rep
    xb = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(xb.float().numpy(), x)
    w = synth.weights(2, n_out, k_dim, seed=72, tensor_id=synth.WDENSE_ID)
    xc = xb.cuda()
    codes, scales, g, _ = P.nvfp4_quantize(xc)
    offs_np = np.array([0, rows0, rows0 + rows1], dtype=np.int64)
    offs = torch.from_numpy(offs_np).cuda()
    sel, rc, rs, rg = P.resq_select_and_requant(xc, codes, scales, g, kc, unit_offsets=offs,
                                                rows_total=rows0 + rows1)
    _, wc, ws_, wg = P.qdq_weights(w.cuda())
    y = torch.empty(rows0 + rows1, n_out, dtype=torch.float32, device="cuda")
    P.moe_w4a4_grouped_gemm(codes, scales, g, offs, rows0 + rows1, wc, ws_, wg, sel_idx=sel,
                            r_codes=rc, r_scales=rs, r_global=rg, out=y)
    torch.cuda.synchronize()
    y_np = np32(y)
    assert np.all(np.isfinite(y_np))
    g_r = OQ.global_scale(np.abs(x).max())
    assert g_r == 1.0 and np32(g)[0] == 1.0
    c_r, s_r, _ = OQ.quantize(x, g=g_r)
    sel_r, rc_r, rs_r, rg_r = OQ.resq_select_and_requant(x, c_r, s_r, g_r, offs_np, kc)
    assert np.array_equal(npu8(sel), sel_r) and np.array_equal(bits32(np32(rg)), bits32(rg_r))
    assert rg_r[1] < 2.0 ** -100 * g_r
    _, wc_r, ws_r, wg_r = OQ.qdq_weights(w.float().numpy())
    for e in range(2):
        lo, hi = offs_np[e], offs_np[e + 1]
        ref = OG.gemm_comp(c_r[lo:hi], s_r[lo:hi], g_r, wc_r[e], ws_r[e], wg_r[e], sel_r[e],
                           rc_r[lo:hi], rs_r[lo:hi], rg_r[e])
        err = np.abs(y_np[lo:hi] - ref).max() / np.abs(ref).max()
        assert err <= GEMM_TOL, f"expert {e}: {err}"
