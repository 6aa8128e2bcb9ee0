"""MXFP4: the microscaling FP4 format, its quantization, the residual channel
selection and the compensated GEMM in that format -- plain CPU definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The TRACE summary validates its method in two FP4 rollout formats, NVFP4 and
MXFP4 (its novelty paragraph, the results paragraph and Table 4: MXFP4 W4A8
and W4A4 rollouts of the 35B-A3B model).  The pages name MXFP4 but give none
of its rules.  Reading: the OCP Microscaling (MX) v1.0 format, the public
definition that name refers to --

  * blocks are 32 consecutive elements of a row;
  * each block has one shared scale 2^X stored as an E8M0 byte X + 127
    (X in [-127, 127]; byte 0xFF is NaN and is never produced);
  * X = floor(log2(amax_b)) - 2, where 2 is the exponent of the largest
    E2M1 level (6 = 1.5 * 2^2), clamped to [-127, 127]; an all-zero block
    takes X = -127 (byte 0);
  * an element's code is the E2M1 index nearest to |x| / 2^X (exact real
    quotient, ties to the even index, values above 6 saturating to 6), with
    the sign bit copying the sign bit of x -- the same element rule as the
    NVFP4 oracle;
  * there is no per-tensor scale.

Layout conventions (shared with the C ABI by specification, not by code):
codes as in NVFP4 (element 2j in the low nibble of byte j, K/2 bytes a row);
scales one E8M0 byte per (row, 32-block), row-major [M, K/32].

The residual compensation follows the NVFP4 oracle step for step (QUADS
section 2.2B): R = x - DQ(Q(x)), channel scores in the fixed 128-row tile
order, top-k with ties to the lower index, and Q(R_S) of the compact residual
-- here in MXFP4, blocks of 32 along the compact axis, so k is a multiple of
32.  The weight side of the correction is the stored MXFP4 weight restricted
to the selected channels, each element keeping its own block scale.
"""

import numpy as np

from .formats import (E2M1_LEVELS, E4M3_VALUES, bf16_bits_to_f32, e2m1_decode, e2m1_index_nearest,
                      e4m3_code_nearest, f32_to_bf16_bits)
from .nvfp4 import (channel_scores, guided_round_record_under, guided_round_under, pack_nibbles,
                    topk_channels, unpack_nibbles)

BLOCK = 32
#: Exponent of the largest E2M1 level: 6 = 1.5 * 2^2.
E2M1_EMAX = 2
E8M0_BIAS = 127
E8M0_XMIN, E8M0_XMAX = -127, 127


def e8m0_decode(scales):
    """Value 2^(byte - 127) of E8M0 scale bytes (float64; NaN for 0xFF)."""
    b = np.asarray(scales).astype(np.int64) & 0xFF
    return np.where(b == 0xFF, np.nan, np.ldexp(1.0, b - E8M0_BIAS))


def shared_exponents(x):
    """X of every 32-block of x [M, K] (fp32 values): floor(log2 amax) - 2,
    clamped to [-127, 127]; -127 for an all-zero block.

    floor(log2 a) for a > 0 is read off np.frexp exactly: a = f * 2^e with
    f in [0.5, 1) gives floor(log2 a) = e - 1 (subnormal inputs included)."""
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    amax = np.abs(x.reshape(m, k // BLOCK, BLOCK)).max(axis=2).astype(np.float64)
    _, e = np.frexp(amax)
    xe = np.where(amax > 0, e - 1 - E2M1_EMAX, E8M0_XMIN)
    return np.clip(xe, E8M0_XMIN, E8M0_XMAX).astype(np.int64)


def quantize(x):
    """MXFP4 quantization of x [M, K] (fp32 values; bf16 inputs are exact).

    Per block: X from shared_exponents, scale byte X + 127; per element the
    E2M1 index nearest to |x| / 2^X (2^X is exact in float64 and so is every
    midpoint times it, so the comparison decides the exact quotient), ties to
    the even index, saturating at 6; sign bit from x.

    Returns (codes [M, K/2] uint8, scales [M, K/32] uint8)."""
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    assert k % BLOCK == 0
    xe = shared_exponents(x)
    d = np.repeat(np.ldexp(1.0, xe), BLOCK, axis=1)
    idx = e2m1_index_nearest(np.abs(x).astype(np.float64), d)
    sign = np.signbit(x).astype(np.int64)
    nib = ((sign << 3) | idx).astype(np.uint8)
    return pack_nibbles(nib), (xe + E8M0_BIAS).astype(np.uint8)


def dequantize(codes, scales):
    """DQ = value(code) * 2^X as fp32 [M, K].

    The product has at most 2 significant bits and |X| <= 127, so it is exact
    in fp32 (2^-128 is an fp32 subnormal; 6 * 2^127 would overflow, but
    finite fp32 inputs give X <= 125)."""
    nib = unpack_nibbles(codes)
    s = np.repeat(e8m0_decode(scales), BLOCK, axis=1)
    v = e2m1_decode(nib) * s
    out = v.astype(np.float32)
    assert np.array_equal(out.astype(np.float64), v), "MXFP4 dequantization not exact in fp32"
    return out


def residual(x, codes, scales):
    """R = fp32(x) - DQ(Q(x)), exact in fp32 (Sterbenz: a nonzero code puts
    DQ within a factor of two of x, a zero code gives R = x); checked here."""
    x = np.asarray(x, dtype=np.float32)
    dq = dequantize(codes, scales)
    r = (x - dq).astype(np.float32)
    assert np.array_equal(r.astype(np.float64), x.astype(np.float64) - dq.astype(np.float64)), \
        "residual subtraction not exact"
    return r


def resq_select_and_requant(x, codes, scales, unit_offsets, k, row_index=None):
    """Residual activation compensation in MXFP4 (QUADS section 2.2B).

    As the NVFP4 oracle's step of the same name: units are ranges of unit
    rows (unit row r reads tensor row row_index[r]); per unit the channel
    scores of |R| (128-row tile order), the top-k channels in ascending
    order, and the compact residual R_S quantized to MXFP4 with 32-blocks
    along the compact axis (k % 32 == 0).  A unit without rows gets
    sel_idx = 0..k-1 and no rows.

    Returns (sel_idx [U, k] int32, r_codes [rows, k/2], r_scales [rows, k/32])."""
    assert k % BLOCK == 0
    x = np.asarray(x, dtype=np.float32)
    unit_offsets = np.asarray(unit_offsets, dtype=np.int64)
    n_units = unit_offsets.size - 1
    rows_total = int(unit_offsets[-1])
    if row_index is None:
        row_index = np.arange(rows_total)
    row_index = np.asarray(row_index, dtype=np.int64)
    r_full = residual(x, codes, scales)
    sel = np.zeros((n_units, k), dtype=np.int32)
    r_codes = np.zeros((rows_total, k // 2), dtype=np.uint8)
    r_scales = np.zeros((rows_total, k // BLOCK), dtype=np.uint8)
    for u in range(n_units):
        a, b = int(unit_offsets[u]), int(unit_offsets[u + 1])
        if b == a:
            sel[u] = np.arange(k, dtype=np.int32)
            continue
        r_unit = r_full[row_index[a:b]]
        sel[u] = topk_channels(channel_scores(np.abs(r_unit)), k)
        r_codes[a:b], r_scales[a:b] = quantize(r_unit[:, sel[u]])
    return sel, r_codes, r_scales


def gemm_comp(a_codes, a_scales, w_codes, w_scales, sel_idx=None, r_codes=None, r_scales=None):
    """Y = DQ(A) DQ(W)^T + DQ(R_S) DQ(W)[:, S]^T in float64 (numpy matmul of
    the exactly dequantized operands), as the NVFP4 oracle's compensated GEMM
    with MXFP4 operands and no global scales."""
    a = dequantize(a_codes, a_scales).astype(np.float64)
    w = dequantize(w_codes, w_scales).astype(np.float64)
    y = a @ w.T
    if sel_idx is not None:
        r = dequantize(r_codes, r_scales).astype(np.float64)
        y = y + r @ w[:, np.asarray(sel_idx, dtype=np.int64)].T
    return y


def quantize_weights(w):
    """MXFP4 of every matrix of w [nmat, N, K] along K (no global scale, so
    matrices are independent).  Returns (codes [nmat, N, K/2], scales
    [nmat, N, K/32])."""
    w = np.asarray(w, dtype=np.float32)
    nmat, n, k = w.shape
    c, s = quantize(w.reshape(nmat * n, k))
    return c.reshape(nmat, n, k // 2), s.reshape(nmat, n, k // BLOCK)


# ---------------------------------------------------------------------------
# trainer side in MXFP4 (QUADS section 2.2A weight QDQ; TRACE core method and
# method step four, guided rounding), with the MXFP4 scale rule above
# ---------------------------------------------------------------------------

def qdq_weights(w):
    """MXFP4 fake quantization of weights w [nmat, N, K] (fp32 values, bf16
    inputs): the trainer's forward sees the rollout's MXFP4 weights as BF16.
    Blocks of 32 along K; there is no global scale, so the matrices are
    independent.  DQ = value * 2^X is exact in fp32 and, having at most two
    significant bits, also in bf16, so w_qdq is DQ itself.

    Returns (w_qdq bf16 bits [nmat, N, K] uint16, codes [nmat, N, K/2],
    scales [nmat, N, K/32])."""
    w = np.asarray(w, dtype=np.float32)
    nmat, n, k = w.shape
    codes, scales = quantize(w.reshape(nmat * n, k))
    dq = dequantize(codes, scales)
    bits = f32_to_bf16_bits(dq)
    assert np.array_equal(bf16_bits_to_f32(bits), dq), "MXFP4 DQ not exact in bf16"
    return (bits.reshape(nmat, n, k), codes.reshape(nmat, n, k // 2),
            scales.reshape(nmat, n, k // BLOCK))


def guided_round(x_train, roll_codes, roll_scales):
    """Rollout-guided rounding against MXFP4 rollout codes: the rule of the
    NVFP4 oracle's guided_round (candidates q- <= x/S <= q+, the one closer
    to the rollout level, zero keeps x's sign bit) with S = 2^X of the
    element's 32-block.  Returns (guided codes [M, K/2], x_fq bf16 bits
    [M, K], dist_hist int64[3])."""
    S_all = np.repeat(e8m0_decode(roll_scales), BLOCK, axis=1).astype(np.float64)
    return guided_round_under(x_train, unpack_nibbles(roll_codes), S_all)


def guided_round_record(x_train, record, roll_scales):
    """Guided rounding from the mantissa-only record of MXFP4 rollout codes
    (TRACE method steps two and four): the record is the low code bit per
    element (nvfp4.guidance_record, the same for both formats), with the E8M0
    scales of the rollout beside it (1 + 8/32 = 1.25 bits per element); the
    rule of the NVFP4 oracle's guided_round_record with S = 2^X.  Returns
    (guided codes [M, K/2], x_fq bf16 bits [M, K], moved int64[2])."""
    S_all = np.repeat(e8m0_decode(roll_scales), BLOCK, axis=1).astype(np.float64)
    return guided_round_record_under(x_train, record, S_all)


# ---------------------------------------------------------------------------
# W4A8: MXFP8 activations (the TRACE summary's MXFP4 W4A8 rollout, Table 4)
# ---------------------------------------------------------------------------
#: Exponent of the largest E4M3 value: 448 = 1.75 * 2^8.
E4M3_EMAX = 8


def shared_exponents_fp8(x):
    """X of every 32-block for MXFP8 elements: floor(log2 amax) - 8, clamped
    to [-127, 127]; -127 for an all-zero block (OCP MX, read as for MXFP4)."""
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    amax = np.abs(x.reshape(m, k // BLOCK, BLOCK)).max(axis=2).astype(np.float64)
    _, e = np.frexp(amax)
    xe = np.where(amax > 0, e - 1 - E4M3_EMAX, E8M0_XMIN)
    return np.clip(xe, E8M0_XMIN, E8M0_XMAX).astype(np.int64)


def quantize_fp8(x):
    """MXFP8 quantization of activations x [M, K]: per 32-block the shared
    exponent above; per element the E4M3 value nearest to |x| / 2^X (exact
    real quotient, ties to the even byte, values above 448 saturating to 448),
    sign bit from x.  Returns (codes [M, K] uint8 E4M3 bytes, scales [M, K/32])."""
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    assert k % BLOCK == 0
    xe = shared_exponents_fp8(x)
    codes = np.zeros((m, k), dtype=np.uint8)
    for b in range(k // BLOCK):
        cols = slice(BLOCK * b, BLOCK * b + BLOCK)
        blk = x[:, cols]
        for r in range(m):
            mag = e4m3_code_nearest(np.abs(blk[r]).astype(np.float64), np.ldexp(1.0, int(xe[r, b])))
            codes[r, cols] = mag | (np.signbit(blk[r]).astype(np.uint8) << 7)
    return codes, (xe + E8M0_BIAS).astype(np.uint8)


def dequantize_fp8(codes, scales):
    """value(E4M3 byte) * 2^X as float64 (exact)."""
    c = np.asarray(codes).astype(np.int64)
    mag = E4M3_VALUES[c & 0x7F]
    v = np.where(c & 0x80, -mag, mag)
    return v * np.repeat(e8m0_decode(scales), BLOCK, axis=1)


def gemm_w4a8(a_codes, a_scales, w_codes, w_scales):
    """Y = DQ(A8) DQ(W4)^T in float64: MXFP8 activations times MXFP4 weights."""
    return dequantize_fp8(a_codes, a_scales) @ dequantize(w_codes, w_scales).astype(np.float64).T


__all__ = ["qdq_weights", "guided_round", "guided_round_record", "shared_exponents_fp8", "quantize_fp8", "dequantize_fp8", "gemm_w4a8",
           "BLOCK", "E2M1_LEVELS", "e8m0_decode", "shared_exponents", "quantize", "dequantize",
           "residual", "resq_select_and_requant", "gemm_comp", "quantize_weights"]
