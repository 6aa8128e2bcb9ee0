"""Parity at the full size of the 8192-token MoE layer (T 8192, H 4096, 256
experts, I 1536, top-8 routing, k 64), in the launch configuration the bench
times: the bench's own input builder and step run on the GPU, and the oracle
recomputes sampled outputs one by one.

Every oracle input comes from the seeded generators, never from the GPU's
results: global scales from the oracle's own amax of the whole tensor, the
selection of a sampled expert from the oracle's quantization of that
expert's rows, and the GEMM rows from those.  Outputs that depend on a whole
tensor the oracle cannot recompute at this size (amax(h) of the gate/up
output) are checked through properties instead: the down projection runs at
full size on seeded inputs of its own.
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
WL = synth.WORKLOADS["moe_T8192_H4096_E256_I1536_k64_trainer"]
SAMPLE_EXPERTS = (0, 173)
ROWS_PER_EXPERT = 24


def npu8(t):
    return t.detach().cpu().numpy()


def np32(t):
    return t.detach().float().cpu().numpy()


def bf16_bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.fixture(scope="module")
def step(gpu_lib):
    P = gpu_lib
    inp, _ = bench.build_inputs(torch, P, synth, WL, torch.device("cuda"))
    out = bench.run_step(P, inp, WL, bench.Timeline(torch), trainer=True)
    torch.cuda.synchronize()
    yield P, inp, out
    del inp, out
    torch.cuda.empty_cache()


def _expert_rows(inp, e):
    offs = inp["routing"]["offsets"]
    return int(offs[e]), int(offs[e + 1])


def test_full_quantize_and_selection(step):
    """X's global scale, the codes and scales of the sampled experts' token
    rows, and those experts' selections and requantized residuals, all
    bit-exact."""
    P, inp, out = step
    x = np32(inp["x"])
    g = OQ.global_scale(np.abs(x).max())
    xq_c, xq_s, xq_g = out["xq"]
    sel, rc, rs, rg = out["sel1"]
    assert np32(xq_g)[0] == g
    slot_token = inp["routing"]["slot_token"]
    for e in SAMPLE_EXPERTS:
        a, b = _expert_rows(inp, e)
        assert b - a > 128, "sampled expert spans several 128-row tiles"
        tok = slot_token[a:b]
        c_ref, s_ref, _ = OQ.quantize(x[tok], g=g)
        assert np.array_equal(npu8(xq_c[torch.from_numpy(tok).cuda()]), c_ref)
        assert np.array_equal(npu8(xq_s[torch.from_numpy(tok).cuda()]), s_ref)
        sel_r, rc_r, rs_r, rg_r = OQ.resq_select_and_requant(x[tok], c_ref, s_ref, g,
                                                             [0, b - a], WL.k)
        assert np.array_equal(npu8(sel[e]), sel_r[0])
        assert np32(rg)[e] == rg_r[0]
        assert np.array_equal(npu8(rc[a:b]), rc_r)
        assert np.array_equal(npu8(rs[a:b]), rs_r)


def test_full_weight_qdq(step):
    """The trainer-side weight QDQ of the sampled experts' gate/up matrices:
    codes, scales, global scale and bf16 output bit-exact."""
    P, inp, _ = step
    w_qdq, codes, scales, g = P.qdq_weights(inp["wgu"])
    for e in SAMPLE_EXPERTS:
        out_r, c_r, s_r, g_r = OQ.qdq_weights(np32(inp["wgu"][e:e + 1]))
        assert np32(g)[e] == g_r[0]
        assert np.array_equal(npu8(codes[e]), c_r[0])
        assert np.array_equal(npu8(scales[e]), s_r[0])
        assert np.array_equal(bf16_bits(w_qdq[e]), out_r[0])
        assert np.array_equal(npu8(inp["gc"][e]), c_r[0])


def test_full_gate_up_rows(step):
    """SwiGLU output h of sampled rows of the sampled experts against the
    oracle's compensated GEMM over the oracle's own operands; amax(h) is the
    largest |h| of the whole output."""
    P, inp, out = step
    x = np32(inp["x"])
    g = OQ.global_scale(np.abs(x).max())
    h = out["h"]
    slot_token = inp["routing"]["slot_token"]
    rng = np.random.default_rng(61)
    for e in SAMPLE_EXPERTS:
        a, b = _expert_rows(inp, e)
        tok = slot_token[a:b]
        c_ref, s_ref, _ = OQ.quantize(x[tok], g=g)
        sel_r, rc_r, rs_r, rg_r = OQ.resq_select_and_requant(x[tok], c_ref, s_ref, g,
                                                             [0, b - a], WL.k)
        _, wc, ws, wg = OQ.qdq_weights(np32(inp["wgu"][e:e + 1]))
        rows = np.sort(rng.choice(b - a, ROWS_PER_EXPERT, replace=False))
        gu = OG.gemm_comp(c_ref[rows], s_ref[rows], g, wc[0], ws[0], wg[0], sel_r[0],
                          rc_r[rows], rs_r[rows], rg_r[0])
        h_r = F.bf16_bits_to_f32(OG.swiglu_bf16(gu, WL.inter))
        h_g = np32(h[torch.from_numpy(a + rows).cuda()])
        tol = np.abs(h_r) * 2.0 ** -7 + GEMM_TOL * np.abs(h_r).max()
        assert np.all(np.abs(h_g - h_r) <= tol), f"expert {e}"
    assert np32(inp["amax"])[0] == float(h.float().abs().max())


def test_full_guided_rows(step):
    """Guided rounding of sampled token rows against the oracle, with the
    rollout codes from the oracle's quantization; the histogram counts every
    element."""
    P, inp, out = step
    x = np32(inp["x"])
    g = OQ.global_scale(np.abs(x).max())
    gc, fq, hist = out["guided"]
    rows = np.sort(np.random.default_rng(62).choice(WL.tokens, 48, replace=False))
    c_ref, s_ref, _ = OQ.quantize(x[rows], g=g)
    gc_r, fq_r, _ = OQ.guided_round(np32(inp["x_train"][rows]), c_ref, s_ref, g)
    idx = torch.from_numpy(rows).cuda()
    assert np.array_equal(npu8(gc[idx]), gc_r)
    assert np.array_equal(bf16_bits(fq[idx]), fq_r)
    assert int(hist.sum()) == WL.tokens * WL.hidden


def test_full_down_projection(gpu_lib):
    """The down projection at full size (65536 routed rows of I = 1536 into
    H = 4096, 256 experts, compensated, fixed-order scatter-add of the top-8
    slots) on seeded activations, against the oracle for sampled tokens: each
    token's output sums its 8 slots, each from its own expert's selection."""
    P = gpu_lib
    rt = synth.route(WL.tokens, WL.experts, seed=WL.seed, top_k=WL.top_k, zipf_s=WL.zipf_s)
    offs = rt["offsets"]
    rows = int(offs[-1])
    h = synth.activations(rows, WL.inter, seed=63, device="cuda", heavy_frac=0.01)
    wd = synth.weights(WL.experts, WL.hidden, WL.inter, seed=WL.seed, tensor_id=synth.WD_ID,
                       device="cuda")
    _, dc, ds, dg = P.qdq_weights(wd)
    offs_t = torch.from_numpy(offs).cuda()
    hq_c, hq_s, hq_g, _ = P.nvfp4_quantize(h)
    sel, rc, rs, rg = P.resq_select_and_requant(h, hq_c, hq_s, hq_g, WL.k, unit_offsets=offs_t,
                                                rows_total=rows)
    y = torch.zeros(WL.tokens, WL.hidden, dtype=torch.float32, device="cuda")
    P.moe_w4a4_grouped_gemm(hq_c, hq_s, hq_g, offs_t, rows, dc, ds, dg,
                            epilogue=P.EPI_SCATTER_ADD_F32, sel_idx=sel, r_codes=rc, r_scales=rs,
                            r_global=rg, row_weight=torch.from_numpy(rt["slot_weight"]).cuda(),
                            scatter_index=torch.from_numpy(rt["slot_token"]).cuda(), out=y)
    y_np = np32(y)
    h_np = np32(h)
    g = OQ.global_scale(np.abs(h_np).max())
    assert np32(hq_g)[0] == g
    slot_expert = np.repeat(np.arange(WL.experts), np.diff(offs))
    cache = {}
    for t in (5, 4097):
        slots = np.nonzero(rt["slot_token"] == t)[0]
        assert slots.size == WL.top_k
        ref = np.zeros(WL.hidden)
        for s in slots:
            e = int(slot_expert[s])
            a, b = int(offs[e]), int(offs[e + 1])
            if e not in cache:
                c_ref, s_ref, _ = OQ.quantize(h_np[a:b], g=g)
                sel_r, rc_r, rs_r, rg_r = OQ.resq_select_and_requant(h_np[a:b], c_ref, s_ref, g,
                                                                     [0, b - a], WL.k)
                _, wc, ws, wg = OQ.qdq_weights(np32(wd[e:e + 1]))
                cache[e] = (c_ref, s_ref, sel_r[0], rc_r, rs_r, rg_r[0], wc[0], ws[0], wg[0])
            c_ref, s_ref, sel_e, rc_r, rs_r, rg_e, wc, ws, wg = cache[e]
            r = s - a
            row = OG.gemm_comp(c_ref[r:r + 1], s_ref[r:r + 1], g, wc, ws, wg, sel_e,
                               rc_r[r:r + 1], rs_r[r:r + 1], rg_e)[0]
            ref += float(rt["slot_weight"][s]) * row
        err = np.abs(y_np[t] - ref).max() / np.abs(ref).max()
        assert err <= GEMM_TOL, f"token {t}: {err}"


# ---------------------------------------------------------------------------
# the same layer in MXFP4 (the bench's MXFP4 workload with the trainer side)
# ---------------------------------------------------------------------------
MX_WL = synth.WORKLOADS["mx_moe_T8192_H4096_E256_I1536_k64_trainer"]


@pytest.fixture(scope="module")
def mx_step(gpu_lib):
    P = gpu_lib
    inp, _ = bench.build_inputs(torch, P, synth, MX_WL, torch.device("cuda"))
    out = bench.run_step(P, inp, MX_WL, bench.Timeline(torch), trainer=True)
    torch.cuda.synchronize()
    yield P, inp, out
    del inp, out
    torch.cuda.empty_cache()


def test_full_mx_rollout_rows(mx_step):
    """MXFP4 codes and scales of the sampled experts' token rows, their
    selections and requantized residuals bit-exact, and sampled rows of the
    SwiGLU output against the oracle's compensated GEMM."""
    from oracle import mxfp4 as MX
    P, inp, out = mx_step
    x = np32(inp["x"])
    xq_c, xq_s = out["xq"]
    sel, rc, rs = out["sel1"]
    h = out["h"]
    slot_token = inp["routing"]["slot_token"]
    rng = np.random.default_rng(64)
    for e in SAMPLE_EXPERTS:
        a, b = _expert_rows(inp, e)
        tok = slot_token[a:b]
        c_ref, s_ref = MX.quantize(x[tok])
        idx = torch.from_numpy(tok).cuda()
        assert np.array_equal(npu8(xq_c[idx]), c_ref)
        assert np.array_equal(npu8(xq_s[idx]), s_ref)
        sel_r, rc_r, rs_r = MX.resq_select_and_requant(x[tok], c_ref, s_ref, [0, b - a], MX_WL.k)
        assert np.array_equal(npu8(sel[e]), sel_r[0])
        assert np.array_equal(npu8(rc[a:b]), rc_r)
        assert np.array_equal(npu8(rs[a:b]), rs_r)
        wc, ws = MX.quantize_weights(np32(inp["wgu"][e:e + 1]))
        assert np.array_equal(npu8(inp["gc"][e]), wc[0])
        rows = np.sort(rng.choice(b - a, ROWS_PER_EXPERT, replace=False))
        gu = MX.gemm_comp(c_ref[rows], s_ref[rows], wc[0], ws[0], sel_r[0], rc_r[rows], rs_r[rows])
        h_r = F.bf16_bits_to_f32(OG.swiglu_bf16(gu, MX_WL.inter))
        h_g = np32(h[torch.from_numpy(a + rows).cuda()])
        tol = np.abs(h_r) * 2.0 ** -7 + GEMM_TOL * np.abs(h_r).max()
        assert np.all(np.abs(h_g - h_r) <= tol), f"expert {e}"


def test_full_mx_trainer_rows(mx_step):
    """MXFP4 weight QDQ of the sampled experts' gate/up matrices and guided
    rounding of sampled token rows, bit-exact."""
    from oracle import mxfp4 as MX
    P, inp, out = mx_step
    w_qdq, codes, scales = P.mxfp4_qdq_weights(inp["wgu"])
    for e in SAMPLE_EXPERTS:
        out_r, c_r, s_r = MX.qdq_weights(np32(inp["wgu"][e:e + 1]))
        assert np.array_equal(npu8(codes[e]), c_r[0])
        assert np.array_equal(npu8(scales[e]), s_r[0])
        assert np.array_equal(bf16_bits(w_qdq[e]), out_r[0])
    x = np32(inp["x"])
    gc, fq, hist = out["guided"]
    rows = np.sort(np.random.default_rng(65).choice(MX_WL.tokens, 48, replace=False))
    c_ref, s_ref = MX.quantize(x[rows])
    gc_r, fq_r, _ = MX.guided_round(np32(inp["x_train"][rows]), c_ref, s_ref)
    idx = torch.from_numpy(rows).cuda()
    assert np.array_equal(npu8(gc[idx]), gc_r)
    assert np.array_equal(bf16_bits(fq[idx]), fq_r)
    assert int(hist.sum()) == MX_WL.tokens * MX_WL.hidden
