#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 MoE hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole hot path over one batch of synthetic input:
  rollout side   nvfp4_quantize(X) -> resq_select_and_requant(X, expert units)
                 -> gate/up grouped GEMM (+comp, SwiGLU, amax) -> nvfp4_quantize(h)
                 -> resq_select_and_requant(h) -> down grouped GEMM (+comp, scatter-add)
  trainer side   qdq_weights(all expert matrices) -> guided_round(X_train vs rollout codes)
Inputs are resident in HBM before the timed region; weights are pre-quantized
to NVFP4 (the rollout holds NVFP4 weights) outside it.

Prints ONE JSON line.  value = algorithmic FLOPs of the compensated expert
GEMMs per step / step time.  Per-part times come from HIP events recorded on
the stream the kernels run on; the roofline object is for the kernel that
takes most of the step, and "parts" gives every part's own rate.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_PEAK_TFLOPS = 2500.0        # dense fp16 / bf16 MFMA, MI355X
FP4_PEAK_TFLOPS = 10100.0


def profiled_traffic(workload, kernel, summary=None):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 summary (profiles/<summary>.md, by default the grouped-GEMM one
    of the workload), or None when there is none or the kernel's sources have
    changed since the counters were taken (hash of its files)."""
    import hashlib
    import re
    name = summary or f"grouped_gemm_{workload.replace('_trainer', '')}"
    path = os.path.join(ROOT, "profiles", f"{name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    fields = dict(re.findall(r"^(traffic_kernel|traffic_bytes_per_launch|source_sha256_16|source_files): (.*)$",
                             text, re.M))
    if len(fields) != 4 or kernel not in fields["traffic_kernel"]:
        return None
    h = hashlib.sha256()
    for f in fields["source_files"].split():
        with open(os.path.join(ROOT, "precision_gemm_nvfp4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != fields["source_sha256_16"].strip():
        return None
    return float(fields["traffic_bytes_per_launch"])


def traffic_int(t):
    return None if t is None else int(t)


def gemm_kernel_name(rows, experts, epilogue, fmt="nvfp4", k=4096, kc=64):
    """Name of the grouped-GEMM kernel instance the library picks: rows per
    tile from the average rows per expert (>= 160: 256, >= 64: 128,
    >= 24: 64, else 32), the LDS slots, epilogue 1 = SwiGLU, 2 = scatter, and
    the gather width (8 when the 128-K stages hold more than 3 selected
    channels on average, else 4)."""
    avg = rows // max(experts, 1)
    cfg = "4, 4, 2, 2" if avg >= 160 else "2, 4, 2, 2" if avg >= 64 else \
          "1, 4, 2, 2" if avg >= 24 else "1, 2, 1, 4"
    if fmt == "mxfp4":     # compensated (the bench always compensates)
        return f"nvfp4::mxg::mx_grouped_gemm_kernel<{cfg}, {epilogue}, true, false>"
    # <MI, NJ, WM, WN, LDS slots, epilogue, compensation substeps, gather width>;
    # the 32-row tile keeps two slots when two workgroups then fit a CU (k <= 64, K <= 4096)
    gw = 8 if kc * 128 > 3 * k else 4
    slots = 2 if cfg == "1, 2, 1, 4" and kc <= 64 and k <= 4096 else 3
    return f"nvfp4::nvg::grouped_gemm_kernel<{cfg}, {slots}, {epilogue}, {4 if kc <= 64 else 8}, {gw}>"


def gemm_flops(rows, n, k, kc):
    return 2.0 * rows * n * (k + kc)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="moe_T8192_H4096_E256_I1536_k64_trainer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the brief runs of the four smaller workloads after the headline one")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="calibration: time a plain device copy of this many bytes instead "
                         "(its FETCH_SIZE / WRITE_SIZE per dispatch scale the traffic counters)")
    return ap.parse_args()


def copy_calibration(args, torch):
    """A plain device-to-device copy of known size (torch's copy kernel), for
    scaling the HBM traffic counters: FETCH_SIZE and WRITE_SIZE of one
    dispatch should read copy_bytes each."""
    n = args.copy_bytes // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    print(json.dumps({"calibration": "device copy", "bytes_read": n * 4, "bytes_written": n * 4,
                      "ms": round(ms, 4), "gbs": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}))


class NoMarks:
    """A timeline that records nothing: the timed steps carry no events
    between their parts (each costs a few microseconds of GPU time)."""

    def mark(self, name):
        pass


class Timeline:
    """HIP events recorded on the current stream between the parts of a step."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []

    def mark(self, name):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record(self.torch.cuda.current_stream())
        self.marks.append((name, ev))

    def durations(self):
        out = {}
        for (n0, e0), (n1, e1) in zip(self.marks[:-1], self.marks[1:]):
            out[n1] = out.get(n1, 0.0) + e0.elapsed_time(e1)
        return out


def build_inputs(torch, P, synth, wl, dev):
    t_gen = time.time()
    x = synth.activations(wl.tokens, wl.hidden, seed=wl.seed, device=dev.type,
                          heavy_frac=wl.heavy_frac)
    rt = synth.route(wl.tokens, wl.experts, seed=wl.seed, top_k=wl.top_k, zipf_s=wl.zipf_s)
    wgu = synth.weights(wl.experts, 2 * wl.inter, wl.hidden, seed=wl.seed, tensor_id=synth.WGU_ID,
                        device=dev.type)
    wd = synth.weights(wl.experts, wl.hidden, wl.inter, seed=wl.seed, tensor_id=synth.WD_ID,
                       device=dev.type)
    x_train = synth.guided_noise(x, seed=wl.seed, rel=wl.guided_rel) if wl.trainer else None
    # rollout-side FP4 weights (pre-quantized outside the timed region)
    if wl.fmt == "mxfp4":
        E = wl.experts
        gc, gs, _ = P.mxfp4_quantize(wgu.reshape(E * 2 * wl.inter, wl.hidden))
        dc, ds, _ = P.mxfp4_quantize(wd.reshape(E * wl.hidden, wl.inter))
        gc, gs = gc.reshape(E, 2 * wl.inter, -1), gs.reshape(E, 2 * wl.inter, -1)
        dc, ds = dc.reshape(E, wl.hidden, -1), ds.reshape(E, wl.hidden, -1)
        gg = dg = None
    else:
        _, gc, gs, gg = P.qdq_weights(wgu)
        _, dc, ds, dg = P.qdq_weights(wd)
    torch.cuda.synchronize()
    inp = dict(
        x=x, x_train=x_train, wgu=wgu, wd=wd, gc=gc, gs=gs, gg=gg, dc=dc, ds=ds, dg=dg,
        offs=torch.from_numpy(rt["offsets"]).to(dev),
        slot_token=torch.from_numpy(rt["slot_token"]).to(dev),
        slot_weight=torch.from_numpy(rt["slot_weight"]).to(dev),
        rows=int(rt["offsets"][-1]), routing=rt,
        y=torch.zeros(wl.tokens, wl.hidden, dtype=torch.float32, device=dev),
        amax=torch.empty(1, dtype=torch.float32, device=dev),
    )
    return inp, time.time() - t_gen


def run_step_mx(P, inp, wl, tl, trainer=True):
    """One pass of the MXFP4 path (same steps as run_step)."""
    tl.mark("start")
    xq_c, xq_s, _ = P.mxfp4_quantize(inp["x"])
    tl.mark("quantize_x")
    sel1, rc1, rs1 = P.mxfp4_resq_select_and_requant(
        inp["x"], xq_c, xq_s, wl.k, unit_offsets=inp["offs"], rows_total=inp["rows"],
        row_index=inp["slot_token"])
    tl.mark("resq_x")
    h = P.moe_mxfp4_grouped_gemm(xq_c, xq_s, inp["offs"], inp["rows"], inp["gc"], inp["gs"],
                                 epilogue=P.EPI_SWIGLU_BF16, a_row_index=inp["slot_token"],
                                 sel_idx=sel1, r_codes=rc1, r_scales=rs1, out_amax=inp["amax"])
    tl.mark("gemm_gate_up")
    hq_c, hq_s, _ = P.mxfp4_quantize(h)
    tl.mark("quantize_h")
    sel2, rc2, rs2 = P.mxfp4_resq_select_and_requant(h, hq_c, hq_s, wl.k, unit_offsets=inp["offs"],
                                                     rows_total=inp["rows"])
    tl.mark("resq_h")
    P.moe_mxfp4_grouped_gemm(hq_c, hq_s, inp["offs"], inp["rows"], inp["dc"], inp["ds"],
                             epilogue=P.EPI_SCATTER_F32, sel_idx=sel2, r_codes=rc2,
                             r_scales=rs2, row_weight=inp["slot_weight"],
                             scatter_index=inp["slot_token"], out=inp["y"])
    tl.mark("gemm_down")
    out = dict(xq=(xq_c, xq_s), sel1=(sel1, rc1, rs1), h=h, hq=(hq_c, hq_s), sel2=(sel2, rc2, rs2))
    if trainer and inp["x_train"] is not None:
        P.mxfp4_qdq_weights(inp["wgu"], want_codes=False)
        P.mxfp4_qdq_weights(inp["wd"], want_codes=False)
        tl.mark("qdq")
        out["guided"] = P.mxfp4_guided_round(inp["x_train"], xq_c, xq_s, want_fq=True)
        tl.mark("guided")
    return out


def run_step(P, inp, wl, tl, trainer=True):
    if wl.fmt == "mxfp4":
        return run_step_mx(P, inp, wl, tl, trainer)
    tl.mark("start")
    xq_c, xq_s, xq_g, _ = P.nvfp4_quantize(inp["x"])
    tl.mark("quantize_x")
    sel1, rc1, rs1, rg1 = P.resq_select_and_requant(
        inp["x"], xq_c, xq_s, xq_g, wl.k, unit_offsets=inp["offs"], rows_total=inp["rows"],
        row_index=inp["slot_token"])
    tl.mark("resq_x")
    h = P.moe_w4a4_grouped_gemm(xq_c, xq_s, xq_g, inp["offs"], inp["rows"], inp["gc"], inp["gs"],
                                inp["gg"], epilogue=P.EPI_SWIGLU_BF16, a_row_index=inp["slot_token"],
                                sel_idx=sel1, r_codes=rc1, r_scales=rs1, r_global=rg1,
                                out_amax=inp["amax"])
    tl.mark("gemm_gate_up")
    hq_c, hq_s, hq_g, _ = P.nvfp4_quantize(h, amax_in=inp["amax"])
    tl.mark("quantize_h")
    sel2, rc2, rs2, rg2 = P.resq_select_and_requant(h, hq_c, hq_s, hq_g, wl.k,
                                                    unit_offsets=inp["offs"], rows_total=inp["rows"])
    tl.mark("resq_h")
    P.moe_w4a4_grouped_gemm(hq_c, hq_s, hq_g, inp["offs"], inp["rows"], inp["dc"], inp["ds"],
                            inp["dg"], epilogue=P.EPI_SCATTER_F32, sel_idx=sel2, r_codes=rc2,
                            r_scales=rs2, r_global=rg2, row_weight=inp["slot_weight"],
                            scatter_index=inp["slot_token"], out=inp["y"])
    tl.mark("gemm_down")
    out = dict(xq=(xq_c, xq_s, xq_g), sel1=(sel1, rc1, rs1, rg1), h=h, hq=(hq_c, hq_s, hq_g),
               sel2=(sel2, rc2, rs2, rg2))
    if trainer and inp["x_train"] is not None:
        P.qdq_weights(inp["wgu"], want_codes=False)
        P.qdq_weights(inp["wd"], want_codes=False)
        tl.mark("qdq")
        out["guided"] = P.guided_round(inp["x_train"], xq_c, xq_s, xq_g, want_fq=True)
        tl.mark("guided")
    return out


def part_work(wl, rows):
    """Algorithmic bytes / flops of each part of one step."""
    T, H, I, E, k = wl.tokens, wl.hidden, wl.inter, wl.experts, wl.k
    sb = 32 if wl.fmt == "mxfp4" else 16
    nv = lambda n: n * (0.5 + 1 / sb)                       # FP4 bytes of n elements (codes + scales)
    w = {}
    w["quantize_x"] = dict(bytes=T * H * 2 + nv(T * H), unit="GB/s")
    w["resq_x"] = dict(bytes=rows * H * 2 + nv(rows * H) + nv(rows * k) + E * k * 4, unit="GB/s")
    w["gemm_gate_up"] = dict(flops=gemm_flops(rows, 2 * I, H, k),
                             bytes=E * nv(2 * I * H) + nv(rows * H) + nv(rows * k) + rows * I * 2,
                             unit="TFLOP/s")
    w["quantize_h"] = dict(bytes=rows * I * 2 + nv(rows * I), unit="GB/s")
    w["resq_h"] = dict(bytes=rows * I * 2 + nv(rows * I) + nv(rows * k) + E * k * 4, unit="GB/s")
    w["gemm_down"] = dict(flops=gemm_flops(rows, H, I, k),
                          bytes=E * nv(H * I) + nv(rows * I) + nv(rows * k) + T * H * 4,
                          unit="TFLOP/s")
    if wl.trainer:
        n_w = E * (2 * I * H + H * I)
        w["qdq"] = dict(bytes=n_w * 2 * 2, unit="GB/s")
        w["guided"] = dict(bytes=T * H * 2 + nv(T * H) + T * H / 2 + T * H * 2, unit="GB/s")
    return w


def cpu_baseline(wl, inp, budget_s):
    """The oracle (as it stands) on a bounded sample of the same workload:
    compensated gate/up and down GEMMs of whole experts, taken in expert order
    until the time budget is spent.  Returns GEMM TFLOP/s on the host."""
    import torch
    from oracle import gemm as OG
    from oracle import mxfp4 as OM
    from oracle import nvfp4 as OQ
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    offs = inp["routing"]["offsets"]
    tok = inp["routing"]["slot_token"]
    xs = inp["x"].float().cpu().numpy()
    flops = 0.0
    done = 0
    t0 = time.time()
    mx = wl.fmt == "mxfp4"
    if mx:
        xc, xsc = OM.quantize(xs)
    else:
        xc, xsc, xg = OQ.quantize(xs)
    for e in range(wl.experts):
        a, b = int(offs[e]), int(offs[e + 1])
        if b == a:
            continue
        wgu = inp["wgu"][e:e + 1].float().cpu().numpy()
        if mx:
            sel, rc, rs = OM.resq_select_and_requant(xs, xc, xsc, [0, b - a], wl.k, row_index=tok[a:b])
            gc, gs = OM.quantize_weights(wgu)
            OM.gemm_comp(xc[tok[a:b]], xsc[tok[a:b]], gc[0], gs[0], sel[0], rc, rs)
        else:
            sel, rc, rs, rg = OQ.resq_select_and_requant(xs, xc, xsc, xg, [0, b - a], wl.k,
                                                         row_index=tok[a:b])
            _, gc, gs, gg = OQ.qdq_weights(wgu)
            OG.gemm_comp(xc[tok[a:b]], xsc[tok[a:b]], xg, gc[0], gs[0], gg[0], sel[0], rc, rs, rg[0])
        flops += gemm_flops(b - a, 2 * wl.inter, wl.hidden, wl.k)
        done += 1
        if time.time() - t0 > budget_s:
            break
    dt = time.time() - t0
    # the same oracle on one thread, on the first expert only (a bounded sample)
    one = None
    try:
        from threadpoolctl import threadpool_limits
        e = next(i for i in range(wl.experts) if offs[i + 1] > offs[i])
        a, b = int(offs[e]), int(offs[e + 1])
        with threadpool_limits(limits=1):
            t1 = time.time()
            wgu = inp["wgu"][e:e + 1].float().cpu().numpy()
            if mx:
                sel, rc, rs = OM.resq_select_and_requant(xs, xc, xsc, [0, b - a], wl.k, row_index=tok[a:b])
                gc, gs = OM.quantize_weights(wgu)
                OM.gemm_comp(xc[tok[a:b]], xsc[tok[a:b]], gc[0], gs[0], sel[0], rc, rs)
            else:
                sel, rc, rs, rg = OQ.resq_select_and_requant(xs, xc, xsc, xg, [0, b - a], wl.k,
                                                             row_index=tok[a:b])
                _, gc, gs, gg = OQ.qdq_weights(wgu)
                OG.gemm_comp(xc[tok[a:b]], xsc[tok[a:b]], xg, gc[0], gs[0], gg[0], sel[0], rc, rs, rg[0])
            dt1 = time.time() - t1
        one = dict(value=gemm_flops(b - a, 2 * wl.inter, wl.hidden, wl.k) / dt1 / 1e12, unit="TFLOP/s",
                   cores=1, seconds=round(dt1, 2),
                   sample=f"expert {e} of the gate/up projection ({b - a} rows), as above, one thread")
    except Exception as exc:                       # threadpoolctl missing or no BLAS to limit
        one = dict(error=str(exc))
    model, ncpu = host_cpu()
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"{wl.fmt.upper()} quantization of X, then {done} expert(s) of the gate/up projection "
                       f"({wl.hidden}->{2 * wl.inter}, k={wl.k}) in expert order, each with residual "
                       f"selection, weight quantization and the fp64 compensated GEMM; {dt:.1f} s",
                seconds=round(dt, 2), host_cpu=model, host_logical_cpus=ncpu,
                threads_note="cores = the BLAS thread count numpy used (the GEMM step is the "
                             "multithreaded part; the quantizer and selection run on one thread)",
                one_thread=one)


def timed_steps(torch, step, steps):
    """(ms per step, {part: ms}): `steps` steps timed with no events between
    their parts, then one untimed step, then as many again (at least 3, at
    most 10) with an event at each part boundary for the per-part times."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        step(NoMarks())
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    n = max(3, min(steps, 10))
    # One unmarked step first, with no synchronisation after it: the host
    # enqueues the marked steps while the GPU runs it, so a part's events
    # time the GPU's work rather than the host's launches of the first parts.
    step(NoMarks())
    tls = []
    for _ in range(n):
        tl = Timeline(torch)
        step(tl)
        tls.append(tl)
    torch.cuda.synchronize()
    parts = {}
    for tl in tls:
        for k, v in tl.durations().items():
            parts[k] = parts.get(k, 0.0) + v / n
    return ms, parts


def time_call(torch, fn, n=10, warm=2):
    """Mean ms of fn() over n calls, HIP events on the current stream."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / n


def host_cpu():
    """CPU model and logical core count of the host that runs the bench."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def comp_overhead(torch, P, inp, wl, sel1, sel2, hq, n=5):
    """Time of each grouped GEMM with and without the compensation term on
    the step's own operands, and the selection that feeds it: the cost of
    residual compensation next to the pages' 5-9% (QUADS section 4)."""
    xq_c, xq_s, xq_g = sel1["xq"]
    hq_c, hq_s, hq_g = hq
    h = sel2["h"]
    gu = dict(a_row_index=inp["slot_token"], out_amax=inp["amax"], epilogue=P.EPI_SWIGLU_BF16)
    dn = dict(epilogue=P.EPI_SCATTER_F32, row_weight=inp["slot_weight"],
              scatter_index=inp["slot_token"], out=inp["y"])
    s1, s2 = sel1["sel"], sel2["sel"]
    t = {}
    t["gate_up_plain"] = time_call(torch, lambda: P.moe_w4a4_grouped_gemm(
        xq_c, xq_s, xq_g, inp["offs"], inp["rows"], inp["gc"], inp["gs"], inp["gg"], **gu), n)
    t["gate_up_comp"] = time_call(torch, lambda: P.moe_w4a4_grouped_gemm(
        xq_c, xq_s, xq_g, inp["offs"], inp["rows"], inp["gc"], inp["gs"], inp["gg"], sel_idx=s1[0],
        r_codes=s1[1], r_scales=s1[2], r_global=s1[3], **gu), n)
    t["resq_x"] = time_call(torch, lambda: P.resq_select_and_requant(
        inp["x"], xq_c, xq_s, xq_g, wl.k, unit_offsets=inp["offs"], rows_total=inp["rows"],
        row_index=inp["slot_token"]), n)
    t["down_plain"] = time_call(torch, lambda: P.moe_w4a4_grouped_gemm(
        hq_c, hq_s, hq_g, inp["offs"], inp["rows"], inp["dc"], inp["ds"], inp["dg"], **dn), n)
    t["down_comp"] = time_call(torch, lambda: P.moe_w4a4_grouped_gemm(
        hq_c, hq_s, hq_g, inp["offs"], inp["rows"], inp["dc"], inp["ds"], inp["dg"], sel_idx=s2[0],
        r_codes=s2[1], r_scales=s2[2], r_global=s2[3], **dn), n)
    t["resq_h"] = time_call(torch, lambda: P.resq_select_and_requant(
        h, hq_c, hq_s, hq_g, wl.k, unit_offsets=inp["offs"], rows_total=inp["rows"]), n)
    plain = t["gate_up_plain"] + t["down_plain"]
    return dict(
        ms={k: round(v, 4) for k, v in t.items()},
        gemm_only=round((t["gate_up_comp"] + t["down_comp"]) / plain - 1, 4),
        with_selection=round((t["gate_up_comp"] + t["down_comp"] + t["resq_x"] + t["resq_h"]) / plain - 1, 4),
        flop_fraction=round(wl.k * (2 * wl.inter + wl.hidden) / (wl.hidden * 2 * wl.inter + wl.inter * wl.hidden), 4),
        pages="5-9% slower than plain NVFP4 W4A4 rollout (QUADS section 4, NVIDIA Blackwell)")


def moe_summary(torch, P, synth, wl, dev, steps=5):
    """One MoE workload timed briefly: step time, per-part times, the gate/up
    GEMM's rate against the fp16 MFMA peak (prefill) or the weights' HBM
    stream (decode), and the compensation overhead."""
    inp, _ = build_inputs(torch, P, synth, wl, dev)
    for _ in range(2):
        run_step(P, inp, wl, Timeline(torch), trainer=False)
    torch.cuda.synchronize()
    res_out = {}

    def step(tl):
        res_out["out"] = run_step(P, inp, wl, tl, trainer=False)

    ms, parts = timed_steps(torch, step, steps)
    out = res_out["out"]
    work = part_work(wl, inp["rows"])
    gflop = work["gemm_gate_up"]["flops"] + work["gemm_down"]["flops"]
    T, H, I, E = wl.tokens, wl.hidden, wl.inter, wl.experts
    w_bytes = E * (2 * I * H + H * I) * (0.5 + 1 / 16)
    gu_tf = work["gemm_gate_up"]["flops"] / (parts["gemm_gate_up"] * 1e-3) / 1e12
    res = dict(workload=wl.name, ms_per_step=round(ms, 4),
               parts_ms={k: round(v, 4) for k, v in parts.items() if k in work},
               gemm_tflops=round(gflop / ((parts["gemm_gate_up"] + parts["gemm_down"]) * 1e-3) / 1e12, 2),
               gate_up=dict(ms=round(parts["gemm_gate_up"], 4), tflops=round(gu_tf, 2),
                            frac_fp16_peak=round(gu_tf / FP16_PEAK_TFLOPS, 4),
                            frac_fp4_peak=round(gu_tf / FP4_PEAK_TFLOPS, 4)))
    if inp["rows"] // E < 24:            # decode: the GEMMs stream the expert weights
        gbs = w_bytes / ((parts["gemm_gate_up"] + parts["gemm_down"]) * 1e-3) / 1e9
        res["weights_stream"] = dict(bytes=int(w_bytes), gbs=round(gbs, 1),
                                     frac_hbm=round(gbs / HBM_PEAK_GBS, 4), bound="hbm")
    res["comp_overhead"] = comp_overhead(
        torch, P, inp, wl, dict(xq=out["xq"], sel=out["sel1"]),
        dict(h=out["h"], sel=out["sel2"]), out["hq"])
    del inp, out
    torch.cuda.empty_cache()
    return res


def dense_summary(torch, P, synth, wl, dev, n=20):
    """The single dense linear (E = 1): the whole path (quantize, select,
    compensated GEMM) and the GEMM with and without compensation."""
    x = synth.activations(wl.tokens, wl.hidden, seed=wl.seed, device=dev.type,
                          outlier_channels=wl.outliers)
    w = synth.weights(1, wl.n_out, wl.hidden, seed=wl.seed, tensor_id=synth.WDENSE_ID, device=dev.type)
    _, wc, ws, wg = P.qdq_weights(w)
    offs = torch.tensor([0, wl.tokens], dtype=torch.int64, device=dev)

    def path():
        c, sc, g, _ = P.nvfp4_quantize(x)
        sel = P.resq_select_and_requant(x, c, sc, g, wl.k, unit_offsets=offs, rows_total=wl.tokens)
        return P.moe_w4a4_grouped_gemm(c, sc, g, offs, wl.tokens, wc, ws, wg, sel_idx=sel[0],
                                       r_codes=sel[1], r_scales=sel[2], r_global=sel[3])
    c, sc, g, _ = P.nvfp4_quantize(x)
    sel = P.resq_select_and_requant(x, c, sc, g, wl.k, unit_offsets=offs, rows_total=wl.tokens)
    t_path = time_call(torch, path, n)
    t_comp = time_call(torch, lambda: P.moe_w4a4_grouped_gemm(
        c, sc, g, offs, wl.tokens, wc, ws, wg, sel_idx=sel[0], r_codes=sel[1], r_scales=sel[2],
        r_global=sel[3]), n)
    t_plain = time_call(torch, lambda: P.moe_w4a4_grouped_gemm(c, sc, g, offs, wl.tokens, wc, ws, wg), n)
    return dict(workload=wl.name, bound="launch latency (142.6 MFLOP)",
                us_path=round(t_path * 1e3, 1), us_gemm_comp=round(t_comp * 1e3, 1),
                us_gemm_plain=round(t_plain * 1e3, 1),
                comp_overhead_gemm=round(t_comp / t_plain - 1, 4))


def config_summaries(args, torch, P, synth, dev):
    """The four smaller workloads, each timed briefly after the headline one
    (outside its timed region)."""
    out = {}
    wl = synth.WORKLOADS["dense_T128_K512_N1024_k32"]
    out["dense"] = dense_summary(torch, P, synth, wl, dev)
    wl = synth.WORKLOADS["quant_select_T16384_K4096_k128"]
    qargs = argparse.Namespace(**vars(args))
    qargs.steps, qargs.warmup, qargs.no_cpu_baseline = 10, 2, True
    q = quant_select_bench(qargs, torch, P, synth, wl, dev)
    out["quant_select"] = dict(workload=wl.name, ms_per_step=q["ms_per_step"], gbs=q["value"],
                               frac_hbm=round(q["value"] / HBM_PEAK_GBS, 4), parts=q["parts"],
                               bound="hbm")
    for key, name in (("decode", "moe_decode_T256_H2048_E128_I768_k64"),
                      ("prefill", "moe_prefill_T16384_H2048_E128_I768_zipf1.1_k64")):
        out[key] = moe_summary(torch, P, synth, synth.WORKLOADS[name], dev)
    return out


def quant_select_bench(args, torch, P, synth, wl, dev):
    """Quantizer + residual select only (bandwidth-bound): per step,
    nvfp4_quantize with fused 128-row tile scores, then resq_select_and_requant
    over the 128-token tiles.  value = algorithmic GB/s."""
    x = synth.activations(wl.tokens, wl.hidden, seed=wl.seed, device=dev.type,
                          heavy_frac=wl.heavy_frac)
    torch.cuda.synchronize()

    def step(tl):
        tl.mark("start")
        c, s, g, tp = P.nvfp4_quantize(x, tile_partials=True)
        tl.mark("quantize")
        out = P.resq_select_and_requant(x, c, s, g, wl.k, tile_partials=tp)
        tl.mark("resq")
        return out

    for _ in range(args.warmup):
        step(Timeline(torch))
    torch.cuda.synchronize()
    ms, parts_ms = timed_steps(torch, step, args.steps)
    T, K, k = wl.tokens, wl.hidden, wl.k
    tiles = (T + 127) // 128
    nv = lambda n: n * (0.5 + 1 / 16)
    b_quant = T * K * 2 + nv(T * K)
    b_resq = tiles * k * 4 + nv(T * k) + tiles * 4
    parts = {n: dict(ms=round(v, 4)) for n, v in parts_ms.items()}
    parts["quantize"]["gbs"] = round(b_quant / (parts_ms["quantize"] * 1e-3) / 1e9, 1)
    total_bytes = b_quant + b_resq
    value = total_bytes / (ms * 1e-3) / 1e9
    ach = b_quant / (parts_ms["quantize"] * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import nvfp4 as OQ
        rows = 1024
        xs = x[:rows].float().cpu().numpy()
        t0 = time.time()
        c, sc, g = OQ.quantize(xs)
        OQ.resq_select_and_requant(xs, c, sc, g, list(range(0, rows, 128)) + [rows], k)
        dt = time.time() - t0
        cpu = dict(value=round(rows * K * (2 + 0.5625) / dt / 1e9, 4), unit="GB/s", cores=1,
                   kind="oracle", sample=f"first {rows} of {T} rows (8 tiles): quantize + select + "
                                         f"requant, {dt:.1f} s")
    return dict(
        metric="compensated W4A4 MoE GEMM TFLOPS (% FP4 peak); quantizer GB/s (% HBM)",
        value=round(value, 1), unit="GB/s", ms_per_step=round(ms, 4),
        config={"workload": wl.name, "tokens": T, "hidden": K, "k_comp": k,
                "units": "128-token tiles", "parallelism": "single GPU"},
        algorithmic_bytes=int(total_bytes), parts=parts,
        roofline=dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(ach / HBM_PEAK_GBS, 4),
                      traffic=traffic_int(profiled_traffic(
                          wl.name, "amax_partials_kernel + quantize_tile_kernel",
                          "quantizer_quant_select_T16384_K4096_k128")),
                      kernel="amax_partials_kernel + quantize_tile_kernel<SCORES>"),
        frac_hbm=round(value / HBM_PEAK_GBS, 4), cpu_baseline=cpu)


def guidance_bench(args, torch, P, synth, wl, dev):
    """Mantissa-only guidance record (bandwidth-bound): per step, the rollout
    side packs the low code bits of Q(X_roll) (guidance_record_pack), and the
    trainer side rounds X_train from that record (guided_round_record, with the
    bf16 fake-quant output).  Q(X_roll) itself belongs to the rollout forward and
    is made once outside the timed region.  value = algorithmic GB/s."""
    x_roll = synth.activations(wl.tokens, wl.hidden, seed=wl.seed, device=dev.type,
                               heavy_frac=wl.heavy_frac)
    x_train = synth.guided_noise(x_roll, seed=wl.seed, rel=wl.guided_rel)
    rc, rs, rg, _ = P.nvfp4_quantize(x_roll)
    torch.cuda.synchronize()

    def step(tl):
        tl.mark("start")
        rec = P.guidance_record_pack(rc)
        tl.mark("pack")
        out = P.guided_round_record(x_train, rec, rs, rg, want_fq=True)
        tl.mark("guided_record")
        return out

    for _ in range(args.warmup):
        step(Timeline(torch))
    torch.cuda.synchronize()
    ms, parts_ms = timed_steps(torch, step, args.steps)
    n = wl.tokens * wl.hidden
    b_pack = n * (0.5 + 0.125)                              # codes in, record out
    b_guided = n * (2 + 0.125 + 1 / 16 + 0.5 + 2)           # x, record, scales in; codes, x_fq out
    parts = {nm: dict(ms=round(v, 4)) for nm, v in parts_ms.items()}
    for nm, b in (("pack", b_pack), ("guided_record", b_guided)):
        gbs = b / (parts_ms[nm] * 1e-3) / 1e9
        parts[nm].update(gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
    value = (b_pack + b_guided) / (ms * 1e-3) / 1e9
    ach = b_guided / (parts_ms["guided_record"] * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import nvfp4 as OQ
        rows = 256
        xr = x_roll[:rows].float().cpu().numpy()
        xt = x_train[:rows].float().cpu().numpy()
        c, sc, g = OQ.quantize(xr)
        t0 = time.time()
        rec = OQ.guidance_record(c)
        OQ.guided_round_record(xt, rec, sc, g)
        dt = time.time() - t0
        cpu = dict(value=round(rows * wl.hidden * (0.625 + 4.6875) / dt / 1e9, 4), unit="GB/s",
                   cores=1, kind="oracle",
                   sample=f"first {rows} of {wl.tokens} rows: record pack + guided rounding from "
                          f"the record, {dt:.1f} s")
    return dict(
        metric="compensated W4A4 MoE GEMM TFLOPS (% FP4 peak); quantizer GB/s (% HBM)",
        value=round(value, 1), unit="GB/s", ms_per_step=round(ms, 4),
        config={"workload": wl.name, "tokens": wl.tokens, "hidden": wl.hidden,
                "record_bits_per_value": 1.5, "parallelism": "single GPU"},
        algorithmic_bytes=int(b_pack + b_guided), parts=parts,
        roofline=dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic_int(profiled_traffic(
                          wl.name, "guided_kernel", "guidance_record_T8192_K4096")),
                      kernel="guided_kernel<bf16, record>"),
        frac_hbm=round(value / HBM_PEAK_GBS, 4), cpu_baseline=cpu)


def mask_bench(args, torch, P, synth, wl, dev):
    """Dense 50% binary-mask compensation of the 8192-token layer's two
    projections (F32 outputs): per projection the main grouped GEMM, the
    masked residual of the top half of the channels per expert
    (resq_mask_select_and_requant, k = K/2) and the second GEMM accumulated
    into the product (moe_w4a4_masked_comp_gemm).  Gate/up reads X through
    the routing; down reads seeded activations of the routed rows.
    value = main-product GEMM TFLOP/s (the compensation counted as cost)."""
    T, H, E, I = wl.tokens, wl.hidden, wl.experts, wl.inter
    x = synth.activations(T, H, seed=wl.seed, device=dev.type, heavy_frac=wl.heavy_frac)
    rt = synth.route(T, E, seed=wl.seed, top_k=wl.top_k, zipf_s=wl.zipf_s)
    rows = int(rt["offsets"][-1])
    offs = torch.from_numpy(rt["offsets"]).to(dev)
    tok = torch.from_numpy(rt["slot_token"]).to(dev)
    h = synth.activations(rows, I, seed=wl.seed + 1, device=dev.type, heavy_frac=wl.heavy_frac)
    wgu = synth.weights(E, 2 * I, H, seed=wl.seed, tensor_id=synth.WGU_ID, device=dev.type)
    wd = synth.weights(E, H, I, seed=wl.seed, tensor_id=synth.WD_ID, device=dev.type)
    _, gc, gs, gg = P.qdq_weights(wgu)
    _, dc, ds, dg = P.qdq_weights(wd)
    del wgu, wd
    y_gu = torch.empty(rows, 2 * I, dtype=torch.float32, device=dev)
    y_d = torch.empty(rows, H, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(tl):
        tl.mark("start")
        xc, xs, xg, _ = P.nvfp4_quantize(x)
        tl.mark("quantize_x")
        P.moe_w4a4_grouped_gemm(xc, xs, xg, offs, rows, gc, gs, gg, a_row_index=tok, out=y_gu)
        tl.mark("gemm_gate_up")
        _, mc, ms, mg = P.resq_mask_select_and_requant(x, xc, xs, xg, H // 2, unit_offsets=offs,
                                                       rows_total=rows, row_index=tok)
        tl.mark("mask_select_x")
        P.moe_w4a4_masked_comp_gemm(mc, ms, mg, offs, rows, gc, gs, gg, out=y_gu)
        tl.mark("mask_gemm_gate_up")
        hc, hs, hg, _ = P.nvfp4_quantize(h)
        tl.mark("quantize_h")
        P.moe_w4a4_grouped_gemm(hc, hs, hg, offs, rows, dc, ds, dg, out=y_d)
        tl.mark("gemm_down")
        _, mc2, ms2, mg2 = P.resq_mask_select_and_requant(h, hc, hs, hg, I // 2, unit_offsets=offs,
                                                          rows_total=rows)
        tl.mark("mask_select_h")
        P.moe_w4a4_masked_comp_gemm(mc2, ms2, mg2, offs, rows, dc, ds, dg, out=y_d)
        tl.mark("mask_gemm_down")

    for _ in range(args.warmup):
        step(Timeline(torch))
    torch.cuda.synchronize()
    ms, parts_ms = timed_steps(torch, step, args.steps)
    f_gu, f_d = 2.0 * rows * 2 * I * H, 2.0 * rows * H * I
    parts = {nm: dict(ms=round(v, 4)) for nm, v in parts_ms.items()}
    for nm, f in (("gemm_gate_up", f_gu), ("mask_gemm_gate_up", f_gu), ("gemm_down", f_d),
                  ("mask_gemm_down", f_d)):
        parts[nm]["tflops"] = round(f / (parts_ms[nm] * 1e-3) / 1e12, 2)
    overhead = {
        "gate_up": round((parts_ms["mask_select_x"] + parts_ms["mask_gemm_gate_up"])
                         / parts_ms["gemm_gate_up"], 3),
        "down": round((parts_ms["mask_select_h"] + parts_ms["mask_gemm_down"])
                      / parts_ms["gemm_down"], 3)}
    ach = f_gu / (parts_ms["mask_gemm_gate_up"] * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import gemm as OG
        from oracle import nvfp4 as OQ
        xn = x.float().cpu().numpy()
        g = OQ.global_scale(np.abs(xn).max())
        w_all = synth.weights(E, 2 * I, H, seed=wl.seed, tensor_id=synth.WGU_ID, device=dev.type)
        t0, dt, n_rows, n_exp = time.time(), 0.0, 0, 0
        for e in range(E):                      # whole experts until about 10 s
            a, b = int(rt["offsets"][e]), int(rt["offsets"][e + 1])
            sub = xn[rt["slot_token"][a:b]]
            we = w_all[e:e + 1].float().cpu().numpy()
            t1 = time.time()
            c, sc, _ = OQ.quantize(sub, g=g)
            _, mcn, msn, mgn = OQ.resq_mask_select_and_requant(sub, c, sc, g, [0, b - a], H // 2)
            _, wc, ws, wgn = OQ.qdq_weights(we)
            OG.gemm_masked_comp(c, sc, g, wc[0], ws[0], wgn[0], mcn, msn, mgn[0])
            dt += time.time() - t1
            n_rows, n_exp = n_rows + (b - a), n_exp + 1
            if time.time() - t0 > 10.0:
                break
        del w_all
        cpu = dict(value=round(2.0 * n_rows * 2 * I * H / dt / 1e12, 5), unit="TFLOP/s",
                   cores=torch.get_num_threads(), kind="oracle",
                   sample=f"{n_exp} expert(s) ({n_rows} routed rows) of the gate/up projection in "
                          f"expert order: quantize, masked residual (k = {H // 2}), weight "
                          f"quantization, fp64 main + masked GEMM; {dt:.1f} s")
    return dict(
        metric="compensated W4A4 MoE GEMM TFLOPS (% FP4 peak); quantizer GB/s (% HBM)",
        value=round((f_gu + f_d) / (ms * 1e-3) / 1e12, 2), unit="TFLOP/s",
        ms_per_step=round(ms, 4),
        config={"workload": wl.name, "tokens": T, "hidden": H, "experts": E, "inter": I,
                "top_k": wl.top_k, "mask_fraction": 0.5, "routed_rows": rows,
                "parallelism": "single GPU"},
        dtype="nvfp4 (e2m1 + e4m3 scales) operands, fp16 MFMA (exact products), fp32 accumulate",
        parts=parts, mask_overhead_vs_main_gemm=overhead,
        roofline=dict(bound="mfma", achieved=round(ach, 2), peak=2500.0, unit="TFLOP/s",
                      frac=round(ach / 2500.0, 4), traffic=None, mfma_dtype="fp16",
                      kernel="nvfp4::nvg::grouped_gemm_kernel<4, 4, 2, 2, 3, 0, 0, 4> (masked second GEMM)"),
        cpu_baseline=cpu)


def kv_bench(args, torch, P, synth, wl, dev):
    """NVFP4 KV cache with guided KV rounding (bandwidth-bound): per step, for
    the key and the value cache [tokens, heads, head_dim] (blocks along
    head_dim, one calibrated global scale per cache passed as amax), the
    rollout side quantizes the cache and packs its mantissa-only record, and
    the trainer side rounds its own cache from that record (with the bf16
    fake-quant output).  The calibration amax is taken once outside the timed
    region.  value = algorithmic GB/s."""
    T, H, D = wl.tokens, wl.extra["heads"], wl.hidden
    roll = [synth.kv_cache(T, H, D, seed=wl.seed + i, device=dev.type, heavy_frac=wl.heavy_frac)
            for i in range(2)]
    train = [synth.guided_noise(r, seed=wl.seed + i, rel=wl.guided_rel) for i, r in enumerate(roll)]
    rows = [r.reshape(T * H, D) for r in roll]
    trows = [t.reshape(T * H, D) for t in train]
    amax = [r.abs().max().float().reshape(1) for r in rows]
    torch.cuda.synchronize()

    def step(tl):
        tl.mark("start")
        q = [P.nvfp4_quantize(rows[i], amax_in=amax[i]) for i in range(2)]
        tl.mark("quantize_kv")
        rec = [P.guidance_record_pack(q[i][0]) for i in range(2)]
        tl.mark("record_pack")
        out = [P.guided_round_record(trows[i], rec[i], q[i][1], q[i][2], want_fq=True)
               for i in range(2)]
        tl.mark("guided_kv")
        return out

    for _ in range(args.warmup):
        step(Timeline(torch))
    torch.cuda.synchronize()
    ms, parts_ms = timed_steps(torch, step, args.steps)
    n = 2 * T * H * D                                      # key and value elements
    b = {"quantize_kv": n * (2 + 0.5625), "record_pack": n * (0.5 + 0.125),
         "guided_kv": n * (2 + 0.125 + 1 / 16 + 0.5 + 2)}
    parts = {nm: dict(ms=round(v, 4)) for nm, v in parts_ms.items()}
    for nm, nb in b.items():
        gbs = nb / (parts_ms[nm] * 1e-3) / 1e9
        parts[nm].update(gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
    total = sum(b.values())
    value = total / (ms * 1e-3) / 1e9
    ach = b["guided_kv"] / (parts_ms["guided_kv"] * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import nvfp4 as OQ
        r_n = 4096
        xr = rows[0][:r_n].float().cpu().numpy()
        xt = trows[0][:r_n].float().cpu().numpy()
        t0 = time.time()
        c, sc, g = OQ.quantize(xr, g=OQ.global_scale(amax[0].cpu().numpy()[0]))
        rec = OQ.guidance_record(c)
        OQ.guided_round_record(xt, rec, sc, g)
        dt = time.time() - t0
        cpu = dict(value=round(r_n * D * (2.5625 + 0.625 + 4.6875) / dt / 1e9, 4), unit="GB/s",
                   cores=1, kind="oracle",
                   sample=f"first {r_n} of {T * H} key rows: quantize + record pack + guided "
                          f"rounding from the record, {dt:.1f} s")
    return dict(
        metric="compensated W4A4 MoE GEMM TFLOPS (% FP4 peak); quantizer GB/s (% HBM)",
        value=round(value, 1), unit="GB/s", ms_per_step=round(ms, 4),
        config={"workload": wl.name, "tokens": T, "kv_heads": H, "head_dim": D,
                "caches": "key and value", "parallelism": "single GPU"},
        algorithmic_bytes=int(total), parts=parts,
        roofline=dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic_int(profiled_traffic(
                          wl.name, "guided_kernel", "kv_T65536_H4_D128")),
                      kernel="guided_kernel<bf16, record>"),
        frac_hbm=round(value / HBM_PEAK_GBS, 4), cpu_baseline=cpu)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); nothing in this "
              "library uses a second GPU.", file=sys.stderr)
        sys.exit(2)
    import torch
    import precision_gemm_nvfp4_amd as P
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_bytes:
        copy_calibration(args, torch)
        return
    P.load()
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    if wl.kind in ("quant_select", "guidance", "kv", "mask"):
        fn = {"quant_select": quant_select_bench, "guidance": guidance_bench,
              "kv": kv_bench, "mask": mask_bench}[wl.kind]
        res = fn(args, torch, P, synth, wl, dev)
        line = {"metric": res.pop("metric"), "value": res.pop("value"), "unit": res.pop("unit"),
                "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in, nvfp4 out",
                "data": "synthetic (seeded; N(0,1) with 1% Student-t(3) x8 channels)"}
        line.update(res)
        print(json.dumps(line))
        return
    assert wl.kind == "moe", "bench.py runs MoE, quantizer, guidance-record and KV workloads"
    print(f"[bench] workload {wl.name}: generating inputs", file=sys.stderr, flush=True)
    inp, gen_s = build_inputs(torch, P, synth, wl, dev)
    print(f"[bench] inputs ready in {gen_s:.1f}s; rows={inp['rows']}; warmup {args.warmup}",
          file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        run_step(P, inp, wl, Timeline(torch))
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        run_step(P, inp, wl, NoMarks())
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # the parts: the same steps again, after the timed region, with events
    # between the parts
    part_steps = max(3, min(args.steps, 10))
    timelines = []
    for _ in range(part_steps):
        tl = Timeline(torch)
        run_step(P, inp, wl, tl)
        timelines.append(tl)
    torch.cuda.synchronize()
    parts_ms = {}
    for tl in timelines:
        for k, v in tl.durations().items():
            parts_ms[k] = parts_ms.get(k, 0.0) + v / part_steps
    work = part_work(wl, inp["rows"])
    parts = {}
    for name, ms in parts_ms.items():
        if name not in work:
            continue
        w = work[name]
        d = dict(ms=round(ms, 4))
        if "flops" in w:
            d["tflops"] = round(w["flops"] / (ms * 1e-3) / 1e12, 2)
            d["frac_fp16_peak"] = round(d["tflops"] / FP16_PEAK_TFLOPS, 4)
            d["frac_fp4_peak"] = round(d["tflops"] / FP4_PEAK_TFLOPS, 4)
        d["gbs"] = round(w["bytes"] / (ms * 1e-3) / 1e9, 1)
        d["frac_hbm"] = round(d["gbs"] / HBM_PEAK_GBS, 4)
        parts[name] = d

    gemm_flops_step = work["gemm_gate_up"]["flops"] + work["gemm_down"]["flops"]
    value = gemm_flops_step / (ms_per_step * 1e-3) / 1e12
    gemm_ms = parts_ms["gemm_gate_up"] + parts_ms["gemm_down"]
    # Dominant kernel: the gate/up grouped GEMM (one launch per step, the
    # largest single kernel of the step).  Its part also holds the 1-thread
    # fill that zeroes out_amax (about 2 us).
    ach = work["gemm_gate_up"]["flops"] / (parts_ms["gemm_gate_up"] * 1e-3) / 1e12
    kname = gemm_kernel_name(inp["rows"], wl.experts, 1, wl.fmt, k=wl.hidden, kc=wl.k)
    traffic = profiled_traffic(wl.name, kname)
    mx = wl.fmt == "mxfp4"
    peak = FP4_PEAK_TFLOPS if mx else FP16_PEAK_TFLOPS
    roofline = dict(bound="mfma", achieved=round(ach, 2), peak=peak, unit="TFLOP/s",
                    frac=round(ach / peak, 4),
                    traffic=None if traffic is None else int(traffic),
                    kernel=kname, mfma_dtype="fp4 (block-scaled)" if mx else "fp16",
                    launch_ms=round(parts_ms["gemm_gate_up"], 4),
                    flops_per_launch=work["gemm_gate_up"]["flops"],
                    frac_fp4_peak=round(ach / FP4_PEAK_TFLOPS, 4))

    comp = None
    configs = None
    if not args.no_configs and not mx:
        print("[bench] compensation overhead and the four smaller workloads", file=sys.stderr, flush=True)
        out = run_step(P, inp, wl, Timeline(torch), trainer=False)
        comp = comp_overhead(torch, P, inp, wl, dict(xq=out["xq"], sel=out["sel1"]),
                             dict(h=out["h"], sel=out["sel2"]), out["hq"])
        del out
        configs = config_summaries(args, torch, P, synth, dev)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, inp, args.cpu_budget_s)

    line = {
        "metric": "compensated W4A4 MoE GEMM TFLOPS (% FP4 peak); quantizer GB/s (% HBM)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp4 (e2m1 + e8m0 scales) operands, block-scaled fp4 MFMA, fp32 accumulate"
                  if mx else
                  "nvfp4 (e2m1 + e4m3 scales) operands, fp16 MFMA (exact products), fp32 accumulate"),
        "data": "synthetic (seeded; Gaussian activations with 1% Student-t(3) x8 channels, "
                "N(0,0.02) weights, top-8 softmax routing)",
        "config": {"workload": wl.name, "tokens": wl.tokens, "hidden": wl.hidden,
                   "experts": wl.experts, "inter": wl.inter, "top_k": wl.top_k, "k_comp": wl.k,
                   "routed_rows": inp["rows"], "parallelism": "single GPU"},
        "gemm_tflops": round(gemm_flops_step / (gemm_ms * 1e-3) / 1e12, 2),
        "parts": parts,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    if comp is not None:
        line["comp_overhead"] = comp
    if configs is not None:
        line["configs"] = configs
    print(json.dumps(line))


if __name__ == "__main__":
    main()
