"""Seeded synthetic inputs for the NVFP4 W4A4 MoE compensation path.

This module only draws inputs and builds routing metadata.  It holds none of
the quantization, selection or GEMM arithmetic, and it is the only code that
both the CPU oracle and the HIP path use.

Inputs stand in for the pages' workload: rollouts of a MoE language model
whose routed-expert activations are quantized to NVFP4 (QUADS summary,
section 4; TRACE summary, "Method steps").  The pages' models, datasets and
weights are not available; shapes, value distributions (Gaussian bulk plus a
few heavy-tailed or outlier channels, which is what makes residual
compensation matter) and routing skew are synthetic.

Random streams: every tensor is drawn from its own torch.Generator seeded
with seed * 1000 + tensor_id (tensor ids: 0 activations, 1 heavy-channel
choice, 2 Student-t draws, 3 gate/up weights, 4 down weights, 5 router
logits, 6 guided-rounding noise, 7 dense weight).  Values are drawn in fp32
and rounded to bf16 (round-to-nearest-even).  torch's CPU and GPU generators
produce different streams, so a tensor is defined by (seed, tensor id,
device kind); tests that compare the two sides hand the very same bytes to
both.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

X_ID, HEAVY_ID, STUDENT_ID, WGU_ID, WD_ID, LOGIT_ID, NOISE_ID, WDENSE_ID = range(8)


def _gen(seed, tensor_id, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(tensor_id))
    return g


def activations(rows, cols, seed, device="cpu", heavy_frac=0.0, heavy_scale=8.0,
                outlier_channels=(), outlier_scale=16.0):
    """bf16 [rows, cols]: N(0, 1) entries; round(heavy_frac * cols) channels
    (chosen without replacement) replaced by Student-t(nu=3) * heavy_scale;
    the listed outlier channels multiplied by outlier_scale."""
    x = torch.randn(rows, cols, generator=_gen(seed, X_ID, device), device=device,
                    dtype=torch.float32)
    n_heavy = int(round(heavy_frac * cols))
    if n_heavy:
        heavy = torch.randperm(cols, generator=_gen(seed, HEAVY_ID, device), device=device)[:n_heavy]
        z = torch.randn(4, rows, n_heavy, generator=_gen(seed, STUDENT_ID, device),
                        device=device, dtype=torch.float32)
        # Student-t with 3 degrees of freedom: z0 / sqrt(chi2_3 / 3)
        t3 = z[0] / torch.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3.0)
        x[:, heavy] = t3 * heavy_scale
    for c in outlier_channels:
        x[:, c] *= outlier_scale
    return x.to(torch.bfloat16)


def kv_cache(tokens, heads, head_dim, seed, device="cpu", heavy_frac=0.01):
    """bf16 [tokens, heads, head_dim] key or value cache: the activations
    recipe over the tokens x (heads * head_dim) matrix (N(0, 1) bulk with
    round(heavy_frac * heads * head_dim) Student-t(3) x 8 channels).  Rows of
    the [tokens * heads, head_dim] view are the NVFP4 rows, so blocks run along
    head_dim."""
    return activations(tokens, heads * head_dim, seed, device=device,
                       heavy_frac=heavy_frac).reshape(tokens, heads, head_dim)


def weights(n_mat, rows, cols, seed, tensor_id, device="cpu", std=0.02):
    """bf16 [n_mat, rows, cols] with N(0, std^2) entries, drawn one matrix at
    a time (bounded fp32 scratch for large expert stacks)."""
    out = torch.empty(n_mat, rows, cols, dtype=torch.bfloat16, device=device)
    gen = _gen(seed, tensor_id, device)
    for i in range(n_mat):
        out[i] = (torch.randn(rows, cols, generator=gen, device=device,
                              dtype=torch.float32) * std).to(torch.bfloat16)
    return out


def guided_noise(x_roll, seed, rel=1e-3):
    """X_train = bf16(fp32(X_roll) + z * rel * |X_roll|), z ~ N(0, 1): a
    trainer-side activation that differs slightly from the rollout's."""
    xr = x_roll.float()
    z = torch.randn(xr.shape, generator=_gen(seed, NOISE_ID, xr.device.type),
                    device=xr.device, dtype=torch.float32)
    return (xr + z * rel * xr.abs()).to(torch.bfloat16)


def route(n_tokens, n_experts, seed, top_k=8, zipf_s=0.0):
    """Top-k routing of softmax(router logits), logits ~ N(0, 1) minus
    zipf_s * ln(e + 1) for expert e (skewed expert loads when zipf_s > 0).

    Gate weights are the softmax probabilities of the chosen experts, not
    renormalized; ties pick the lower expert id.  Slots (token t, choice j)
    are sorted stably by (expert, token).  Returns numpy arrays:
      slot_token [n_tokens*top_k] int32  token of each sorted slot,
      slot_weight [n_tokens*top_k] fp32  its gate weight,
      offsets [n_experts+1] int64        expert e owns sorted slots offsets[e]..offsets[e+1]-1,
      topk_experts [n_tokens, top_k] int32.
    """
    logits = torch.randn(n_tokens, n_experts, generator=_gen(seed, LOGIT_ID, "cpu"),
                         dtype=torch.float32).numpy().astype(np.float64)
    if zipf_s:
        logits = logits - zipf_s * np.log(np.arange(n_experts, dtype=np.float64) + 1.0)
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    top = np.argsort(-p, axis=1, kind="stable")[:, :top_k].astype(np.int32)
    token = np.repeat(np.arange(n_tokens, dtype=np.int64), top_k)
    expert = top.reshape(-1).astype(np.int64)
    order = np.lexsort((token, expert))
    counts = np.bincount(expert, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return dict(
        slot_token=token[order].astype(np.int32),
        slot_weight=p[token[order], expert[order]].astype(np.float32),
        offsets=offsets,
        topk_experts=top,
    )


@dataclass
class Workload:
    """One synthetic workload: its name, sizes and generator settings."""
    name: str
    kind: str                 # "dense", "quant_select", "moe", "guidance", "kv"
    seed: int
    tokens: int
    hidden: int
    k: int                    # compensated channels per selection unit
    n_out: int = 0            # dense: output features
    experts: int = 0
    inter: int = 0
    top_k: int = 8
    zipf_s: float = 0.0
    heavy_frac: float = 0.0
    outliers: tuple = ()
    trainer: bool = False     # also run weight QDQ and guided rounding
    guided_rel: float = 1e-3
    fmt: str = "nvfp4"        # FP4 format of the rollout path: "nvfp4" or "mxfp4"
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    w.name: w for w in [
        Workload("dense_T128_K512_N1024_k32", "dense", seed=0, tokens=128, hidden=512,
                 n_out=1024, k=32, outliers=(5, 133, 270, 411)),
        Workload("quant_select_T16384_K4096_k128", "quant_select", seed=1, tokens=16384,
                 hidden=4096, k=128, heavy_frac=0.01),
        Workload("moe_decode_T256_H2048_E128_I768_k64", "moe", seed=2, tokens=256, hidden=2048,
                 experts=128, inter=768, k=64, heavy_frac=0.01),
        Workload("moe_prefill_T16384_H2048_E128_I768_zipf1.1_k64", "moe", seed=3, tokens=16384,
                 hidden=2048, experts=128, inter=768, k=64, heavy_frac=0.01, zipf_s=1.1),
        Workload("moe_T8192_H4096_E256_I1536_k64_trainer", "moe", seed=4, tokens=8192,
                 hidden=4096, experts=256, inter=1536, k=64, heavy_frac=0.01, trainer=True),
        Workload("mx_moe_decode_T256_H2048_E128_I768_k64", "moe", seed=2, tokens=256,
                 hidden=2048, experts=128, inter=768, k=64, heavy_frac=0.01, fmt="mxfp4"),
        Workload("mx_moe_prefill_T16384_H2048_E128_I768_zipf1.1_k64", "moe", seed=3,
                 tokens=16384, hidden=2048, experts=128, inter=768, k=64, heavy_frac=0.01,
                 zipf_s=1.1, fmt="mxfp4"),
        Workload("mx_moe_T8192_H4096_E256_I1536_k64", "moe", seed=4, tokens=8192, hidden=4096,
                 experts=256, inter=1536, k=64, heavy_frac=0.01, fmt="mxfp4"),
        Workload("mx_moe_T8192_H4096_E256_I1536_k64_trainer", "moe", seed=4, tokens=8192,
                 hidden=4096, experts=256, inter=1536, k=64, heavy_frac=0.01, fmt="mxfp4",
                 trainer=True),
        Workload("mask_moe_T8192_H4096_E256_I1536_k50pct", "mask", seed=4, tokens=8192,
                 hidden=4096, experts=256, inter=1536, k=0, heavy_frac=0.01),
        Workload("guidance_record_T8192_K4096", "guidance", seed=4, tokens=8192, hidden=4096,
                 k=0, heavy_frac=0.01),
        Workload("kv_T65536_H4_D128", "kv", seed=5, tokens=65536, hidden=128, k=0,
                 heavy_frac=0.01, extra={"heads": 4}),
    ]
}
