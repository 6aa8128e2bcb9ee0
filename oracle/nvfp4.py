"""NVFP4 quantization, residual channel selection, weight QDQ and
rollout-guided rounding: the plain CPU definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Layout conventions (shared with the C ABI by specification, not by code):
  * tensors are row-major [M, K]; blocks are 16 consecutive elements of a row;
  * codes: byte j of a row holds element 2j in the low nibble and element
    2j+1 in the high nibble; a row has K/2 bytes;
  * scales: one E4M3 byte per (row, block), row-major [M, K/16];
  * the global scale g is one fp32 per tensor (per unit for residuals).

Readings of what the pages leave open are stated in each function.
"""

import numpy as np

from .formats import (
    E2M1_LEVELS,
    E4M3_VALUES,
    e2m1_decode,
    e2m1_index_nearest,
    e4m3_code_nearest,
    f32_to_bf16_bits,
)

BLOCK = 16
#: Largest representable magnitude of a block: E2M1 max (6) times E4M3 max (448).
FP4_TIMES_E4M3_MAX = np.float32(6.0 * 448.0)
#: Rows per tile of the fixed residual-score summation order.
SCORE_TILE_ROWS = 128


# ---------------------------------------------------------------------------
# packing
# ---------------------------------------------------------------------------

def pack_nibbles(nib):
    """[M, K] codes 0..15 -> [M, K/2] bytes, element 2j in the low nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """[M, K/2] bytes -> [M, K] codes 0..15 (inverse of pack_nibbles)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


# ---------------------------------------------------------------------------
# scales
# ---------------------------------------------------------------------------

def global_scale(amax):
    """Global (per-tensor) decode scale g.

    The pages name a global scale next to the per-block scale (TRACE summary,
    "Prerequisites: NVFP4 and the E2M1 codebook") but give no formula.
    Reading: g maps the largest block of the tensor onto the largest
    representable block, g = RNE32(amax / (6 * 448)) -- a correctly rounded
    fp32 division.  A zero tensor (or a quotient that underflows to 0) takes
    g = 1.
    """
    g = np.float32(amax) / FP4_TIMES_E4M3_MAX
    return np.float32(1.0) if g == 0 else np.float32(g)


def block_scales(x, g):
    """E4M3 block-scale bytes of x [M, K] (fp32 values) under global scale g.

    s_b = E4M3 value nearest to amax_b / (6 g) (exact real quotient; ties to
    even; saturating at 448; at or below 2^-10 giving 0).  Reading of the
    per-block scale that the TRACE prerequisites name: the decode scale that
    puts the block's largest magnitude on the largest E2M1 level.
    """
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    amax_b = np.abs(x.reshape(m, k // BLOCK, BLOCK)).max(axis=2).astype(np.float64)
    return e4m3_code_nearest(amax_b, 6.0 * np.float64(g))


def effective_scales(scales, g):
    """S_b = RNE32(s_b * g): the fp32 decode scale of every block."""
    s = E4M3_VALUES[np.asarray(scales, dtype=np.int64)].astype(np.float32)
    return (s * np.float32(g)).astype(np.float32)


# ---------------------------------------------------------------------------
# quantize / dequantize
# ---------------------------------------------------------------------------

def quantize(x, g=None):
    """NVFP4 quantization of x [M, K] (fp32 values; bf16 inputs are exact in fp32).

    Follows the TRACE prerequisites (global scale plus per-block scale, then
    round-to-nearest onto the E2M1 codebook) and the pages' worked example in
    the TRACE summary ("Research motivation"): 60.24 and 59.76 under a shared
    scale give 2.51 and 2.49, which round to 3 and 2.

    Per element: magnitude index = E2M1 index nearest to |x| / S_b (exact
    real quotient, ties to even index, saturating at 6; S_b == 0 gives 0);
    the code's sign bit copies the sign bit of x (so -0.1 and -0.0 give
    0x8 when their magnitude rounds to 0).

    Returns (codes [M, K/2] uint8, scales [M, K/16] uint8, g float32).
    g, when given, is used instead of the tensor's own global scale.
    """
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    assert k % BLOCK == 0
    if g is None:
        g = global_scale(np.abs(x).max() if x.size else np.float32(0))
    g = np.float32(g)
    scales = block_scales(x, g)
    S = np.repeat(effective_scales(scales, g), BLOCK, axis=1).astype(np.float64)
    idx = e2m1_index_nearest(np.abs(x).astype(np.float64), S)
    sign = np.signbit(x).astype(np.int64)
    nib = ((sign << 3) | idx).astype(np.uint8)
    return pack_nibbles(nib), scales, g


def dequantize(codes, scales, g):
    """DQ = RNE32(value(code) * S_b) as fp32 [M, K].

    value * S_b is exact in float64 (<= 3 + 24 significant bits); the cast to
    fp32 is the single rounding."""
    nib = unpack_nibbles(codes)
    S = np.repeat(effective_scales(scales, g), BLOCK, axis=1).astype(np.float64)
    return (e2m1_decode(nib) * S).astype(np.float32)


def residual(x, codes, scales, g):
    """R = fp32(x) - DQ(Q(x)) (QUADS section 2.2B: the residual between the
    activation and its FP4 quantization).

    The subtraction is exact in fp32: for a nonzero code, DQ and x are within
    a factor of two of each other (Sterbenz), and a zero code gives R = x.
    The oracle checks that exactness in float64."""
    x = np.asarray(x, dtype=np.float32)
    dq = dequantize(codes, scales, g)
    r = (x - dq).astype(np.float32)
    assert np.array_equal(r.astype(np.float64), x.astype(np.float64) - dq.astype(np.float64)), \
        "residual subtraction not exact"
    return r


# ---------------------------------------------------------------------------
# residual activation compensation: channel scores, top-k, requantization
# ---------------------------------------------------------------------------

def channel_scores(abs_r):
    """score[c] = sum over the unit's rows of |R[row, c]|, in fp32.

    QUADS section 2.2B ranks channels by residual magnitude.  Reading of
    the order (the pages fix none): the unit's rows, in unit order, are cut
    into consecutive tiles of 128 rows; each tile is summed sequentially in
    increasing row order in fp32 (starting from 0); the tile sums are then
    added sequentially in tile order (starting from 0).  For units of at most
    128 rows this is the plain sequential sum.

    abs_r: [rows, K] fp32 absolute residuals in unit order.
    """
    abs_r = np.asarray(abs_r, dtype=np.float32)
    rows, k = abs_r.shape
    total = np.zeros(k, dtype=np.float32)
    for t0 in range(0, rows, SCORE_TILE_ROWS):
        part = np.zeros(k, dtype=np.float32)
        for r in range(t0, min(t0 + SCORE_TILE_ROWS, rows)):
            part = (part + abs_r[r]).astype(np.float32)
        total = (total + part).astype(np.float32)
    return total


def topk_channels(scores, k):
    """Indices of the k highest-scoring channels, returned in ascending order.

    QUADS section 2.2B: a binary channel mask keeps the channels of largest
    residual magnitude.  Ties go to the lower channel index (total order:
    score descending, then index ascending).  Returned ascending so that the
    compact residual's columns follow channel order.
    """
    scores = np.asarray(scores, dtype=np.float32)
    order = np.lexsort((np.arange(scores.size), -scores.astype(np.float64)))
    return np.sort(order[:k]).astype(np.int32)


def resq_select_and_requant(x, codes, scales, g, unit_offsets, k, row_index=None):
    """Residual activation compensation, selection and second quantization.

    QUADS section 2.2B (and the yfxerp digest): pick the high-residual
    channels online, quantize their residual to FP4 a second time; the
    correction is added back to the result by the GEMM.

    x, codes, scales, g: the activation tensor [rows_x, K] and its NVFP4
    quantization.  Units are consecutive ranges of "unit rows"
    (unit_offsets[u]..unit_offsets[u+1]); unit row r reads tensor row
    row_index[r] (identity when row_index is None).  Per unit u:
      * scores from R of the unit's rows (channel_scores order),
      * sel_idx[u] = topk_channels(scores, k),
      * R_S = R[rows, sel_idx[u]] as a compact fp32 [rows_u, k] tensor,
      * Q(R_S) with its own global scale r_global[u] (reading: one global
        scale per unit, since each unit has its own channel set), blocks of
        16 along the compact axis.
    A unit without rows gets sel_idx = 0..k-1, r_global = 1 and no rows.

    Returns (sel_idx [U, k] int32, r_codes [rows, k/2], r_scales [rows, k/16],
    r_global [U] float32).
    """
    x = np.asarray(x, dtype=np.float32)
    unit_offsets = np.asarray(unit_offsets, dtype=np.int64)
    n_units = unit_offsets.size - 1
    rows_total = int(unit_offsets[-1])
    if row_index is None:
        row_index = np.arange(rows_total)
    row_index = np.asarray(row_index, dtype=np.int64)
    r_full = residual(x, codes, scales, g)
    sel = np.zeros((n_units, k), dtype=np.int32)
    r_codes = np.zeros((rows_total, k // 2), dtype=np.uint8)
    r_scales = np.zeros((rows_total, k // BLOCK), dtype=np.uint8)
    r_global = np.ones(n_units, dtype=np.float32)
    for u in range(n_units):
        a, b = int(unit_offsets[u]), int(unit_offsets[u + 1])
        if b == a:
            sel[u] = np.arange(k, dtype=np.int32)
            continue
        r_unit = r_full[row_index[a:b]]
        sel[u] = topk_channels(channel_scores(np.abs(r_unit)), k)
        r_s = r_unit[:, sel[u]]
        rc, rs, rg = quantize(r_s)
        r_codes[a:b], r_scales[a:b], r_global[u] = rc, rs, rg
    return sel, r_codes, r_scales, r_global


def resq_mask_select_and_requant(x, codes, scales, g, unit_offsets, k, row_index=None):
    """Dense-mask form of the residual compensation (QUADS section 2.2B: a
    binary channel mask keeps the top k% of channels by residual magnitude,
    50% in the pages' example, and those channels are quantized a second
    time).

    Reading: the mask M_u of unit u is 1 on the k channels that
    resq_select_and_requant selects (same scores, same tie rule) and 0
    elsewhere; the correction is Q(R * M_u), an ordinary NVFP4 tensor of the
    full width K (blocks of 16 consecutive input channels, zeros outside the
    mask), with one global scale per unit from the largest |R * M_u| of the
    unit's rows.  Its GEMM term is Q(R * M) Q(W)^T over all K channels, the
    masked channels contributing nothing.

    Returns (sel_idx [U, k] int32, m_codes [rows, K/2], m_scales [rows, K/16],
    m_global [U] float32); a unit without rows gets sel_idx = 0..k-1,
    m_global = 1 and no rows.
    """
    x = np.asarray(x, dtype=np.float32)
    unit_offsets = np.asarray(unit_offsets, dtype=np.int64)
    n_units = unit_offsets.size - 1
    rows_total = int(unit_offsets[-1])
    kdim = x.shape[1]
    if row_index is None:
        row_index = np.arange(rows_total)
    row_index = np.asarray(row_index, dtype=np.int64)
    r_full = residual(x, codes, scales, g)
    sel = np.zeros((n_units, k), dtype=np.int32)
    m_codes = np.zeros((rows_total, kdim // 2), dtype=np.uint8)
    m_scales = np.zeros((rows_total, kdim // BLOCK), dtype=np.uint8)
    m_global = np.ones(n_units, dtype=np.float32)
    for u in range(n_units):
        a, b = int(unit_offsets[u]), int(unit_offsets[u + 1])
        if b == a:
            sel[u] = np.arange(k, dtype=np.int32)
            continue
        r_unit = r_full[row_index[a:b]]
        sel[u] = topk_channels(channel_scores(np.abs(r_unit)), k)
        masked = np.zeros_like(r_unit)
        masked[:, sel[u]] = r_unit[:, sel[u]]
        m_codes[a:b], m_scales[a:b], m_global[u] = quantize(masked)
    return sel, m_codes, m_scales, m_global


# ---------------------------------------------------------------------------
# trainer side
# ---------------------------------------------------------------------------

def qdq_weights(w):
    """Weight quantize-dequantize of the asymmetric W4A16 QAT (QUADS section
    2.2A): every forward pass of the trainer sees the NVFP4 weights the
    rollout uses, as BF16 values.

    w: [nmat, N, K] fp32 values (bf16 inputs).  Reading: one global scale per
    matrix, blocks along K (the input dimension), output bf16 of the fp32 DQ
    (fp32 rounding, then bf16 rounding).

    Returns (w_qdq bf16 bits [nmat, N, K] uint16, codes [nmat, N, K/2],
    scales [nmat, N, K/16], g [nmat] float32).
    """
    w = np.asarray(w, dtype=np.float32)
    nmat, n, k = w.shape
    out = np.empty((nmat, n, k), dtype=np.uint16)
    codes = np.empty((nmat, n, k // 2), dtype=np.uint8)
    scales = np.empty((nmat, n, k // BLOCK), dtype=np.uint8)
    gs = np.empty(nmat, dtype=np.float32)
    for i in range(nmat):
        c, s, g = quantize(w[i])
        out[i] = f32_to_bf16_bits(dequantize(c, s, g))
        codes[i], scales[i], gs[i] = c, s, g
    return out, codes, scales, gs


#: Signed E2M1 levels in increasing order, with signed index -7..7.
_SIGNED_LEVELS = np.concatenate([-E2M1_LEVELS[:0:-1], E2M1_LEVELS])   # -6 .. 6
_SIGNED_INDEX = np.arange(-7, 8)


def signed_index(codes):
    """Signed level index of 4-bit codes: -7..7 with +0 and -0 both 0."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    i = c & 7
    return np.where((c & 8) != 0, -i, i)


def guided_round(x_train, roll_codes, roll_scales, roll_g):
    """Rollout-guided rounding (TRACE summary, "Core method" and step four).

    Under the rollout side's scale S = RNE32(s_roll * g_roll) of each
    element's block, v = x_train / S (exact real).  q- is the largest signed
    E2M1 level <= v and q+ the smallest >= v (both clamped to +-6; equal
    when v sits on a level).  The guided level is whichever of q-, q+ is
    closer to the rollout level q_roll, instead of round-to-nearest.  The
    two candidates are adjacent levels and q_roll is a level, so they are
    never equidistant unless equal.  A zero result takes x_train's sign bit
    (reading).  S == 0 gives magnitude 0.

    Returns (guided codes [M, K/2], x_fq bf16 bits [M, K]: the guided code's
    value times S, RNE32 then bf16 (the value of code 0x8 is -0, as in DQ), dist_hist int64[3] = counts of |signed index of RTN(v)
    - signed index of q_roll| equal to 0, 1 and >= 2).
    """
    S_all = np.repeat(effective_scales(roll_scales, roll_g), BLOCK, axis=1).astype(np.float64)
    return guided_round_under(x_train, unpack_nibbles(roll_codes), S_all)


def guided_round_under(x_train, roll_nib, S_all):
    """The guided rule of guided_round with the rollout scale of every
    element given directly (S_all float64 [M, K], each an fp32 value):
    candidates q- <= x/S <= q+ among the signed E2M1 levels, the one closer to
    the rollout level, codes, x_fq = bf16(RNE32(value * S)) and the histogram.
    Shared by the NVFP4 and MXFP4 forms, which differ only in S."""
    x = np.asarray(x_train, dtype=np.float32)
    m, k = x.shape
    nib = np.empty((m, k), dtype=np.uint8)
    x_fq = np.empty((m, k), dtype=np.uint16)
    hist = np.zeros(3, dtype=np.int64)
    for r0 in range(0, m, 64):                  # row chunks bound the memory
        r1 = min(r0 + 64, m)
        xs = x[r0:r1]
        xd = xs.astype(np.float64)
        S = S_all[r0:r1]
        # Exact comparison of x with level * S (level <= 3 significant bits).
        t = _SIGNED_LEVELS[None, None, :] * S[..., None]          # exact
        le = t <= xd[..., None]
        ge = t >= xd[..., None]
        lo = np.clip(le.sum(axis=2) - 1, 0, 14)                   # q-, clamped at -6
        hi = np.where(ge.any(axis=2), ge.argmax(axis=2), 14)      # q+, clamped at +6
        lo = np.minimum(lo, hi)
        q_lo, q_hi = _SIGNED_LEVELS[lo], _SIGNED_LEVELS[hi]
        q_roll = e2m1_decode(roll_nib[r0:r1])
        q = np.where(np.abs(q_hi - q_roll) < np.abs(q_lo - q_roll), q_hi, q_lo)
        q = np.where(S == 0, 0.0, q)
        mag_idx = np.searchsorted(E2M1_LEVELS, np.abs(q))
        neg = (q < 0) | ((q == 0) & np.signbit(xs))
        nib[r0:r1] = (neg.astype(np.int64) << 3) | mag_idx
        x_fq[r0:r1] = f32_to_bf16_bits((e2m1_decode(nib[r0:r1]) * S).astype(np.float32))
        # distance between round-to-nearest under the rollout scale and q_roll
        rtn_idx = e2m1_index_nearest(np.abs(xd), S)
        rtn_signed = np.where(np.signbit(xs), -rtn_idx, rtn_idx)
        dist = np.abs(rtn_signed - signed_index(roll_nib[r0:r1]))
        hist += [(dist == 0).sum(), (dist == 1).sum(), (dist >= 2).sum()]
    return pack_nibbles(nib), x_fq, hist


# ---------------------------------------------------------------------------
# mantissa-only guidance record
# ---------------------------------------------------------------------------

def guidance_record(roll_codes):
    """Mantissa-only guidance record of the rollout codes (TRACE summary, "Core
    method", second innovation, and method step two).

    One bit per element: the low bit of its 4-bit rollout code, which is the
    low bit of the level's magnitude index (the E2M1 mantissa bit).
    Neighbouring signed levels always differ in that bit, so together with
    the candidates {q-, q+} of the training side it names the rollout level
    whenever that level is one of them.  The rollout block scales (and g)
    travel beside it unchanged, one byte per 16 elements, so the record costs
    1 + 8/16 = 1.5 bits per element.

    Layout (reading; the pages fix none): row-major [M, K/8] bytes; bit j of
    byte i of a row is the bit of element 8i + j (low bit first, the order of
    the code nibbles).
    """
    nib = unpack_nibbles(roll_codes).astype(np.uint32)
    m, k = nib.shape
    bits = (nib & 1).reshape(m, k // 8, 8)
    weights = (1 << np.arange(8, dtype=np.uint32))[None, None, :]
    return (bits * weights).sum(axis=2).astype(np.uint8)


def guided_round_record(x_train, record, roll_scales, roll_g):
    """Rollout-guided rounding from the mantissa-only record (TRACE summary,
    method steps two and four).

    S, v = x_train / S and the neighbouring levels q- <= v <= q+ (clamped to
    +-6) are those of guided_round.  Only the low code bit b of q_roll is
    known; q- and q+ differ in it, so the output is the candidate whose
    magnitude index has low bit b, and q- when q- == q+.  When q_roll is q- or
    q+ this is guided_round's choice (the pages find more than 99% of the
    training/rollout mismatches one code apart).  A zero result takes
    x_train's sign bit (reading, as in guided_round); S == 0 gives magnitude 0.

    Returns (guided codes [M, K/2], x_fq bf16 bits [M, K] (the guided code's
    value times S, RNE32 then bf16), moved int64[2] = numbers of elements
    whose signed level index equals round-to-nearest's under S, and differs
    from it).
    """
    S_all = np.repeat(effective_scales(roll_scales, roll_g), BLOCK, axis=1).astype(np.float64)
    return guided_round_record_under(x_train, record, S_all)


def guided_round_record_under(x_train, record, S_all):
    """The record rule of guided_round_record with the rollout scale of every
    element given directly (S_all float64 [M, K], each an fp32 value); shared
    by the NVFP4 and MXFP4 forms, which differ only in S."""
    x = np.asarray(x_train, dtype=np.float32)
    m, k = x.shape
    rec = np.asarray(record, dtype=np.uint8)
    bits = ((rec[:, :, None] >> np.arange(8, dtype=np.uint8)[None, None, :]) & 1).reshape(m, k)
    nib = np.empty((m, k), dtype=np.uint8)
    x_fq = np.empty((m, k), dtype=np.uint16)
    moved = np.zeros(2, dtype=np.int64)
    mag_of_pos = np.abs(np.arange(_SIGNED_LEVELS.size) - (_SIGNED_LEVELS.size // 2))
    for r0 in range(0, m, 64):                  # row chunks bound the memory
        r1 = min(r0 + 64, m)
        xs = x[r0:r1]
        xd = xs.astype(np.float64)
        S = S_all[r0:r1]
        t = _SIGNED_LEVELS[None, None, :] * S[..., None]          # exact
        le = t <= xd[..., None]
        ge = t >= xd[..., None]
        lo = np.clip(le.sum(axis=2) - 1, 0, 14)                   # q-, clamped at -6
        hi = np.where(ge.any(axis=2), ge.argmax(axis=2), 14)      # q+, clamped at +6
        lo = np.minimum(lo, hi)
        pick = np.where((mag_of_pos[hi] & 1) == bits[r0:r1], hi, lo)
        q = np.where(S == 0, 0.0, _SIGNED_LEVELS[pick])
        mag_idx = np.searchsorted(E2M1_LEVELS, np.abs(q))
        neg = (q < 0) | ((q == 0) & np.signbit(xs))
        nib[r0:r1] = (neg.astype(np.int64) << 3) | mag_idx
        x_fq[r0:r1] = f32_to_bf16_bits((e2m1_decode(nib[r0:r1]) * S).astype(np.float32))
        rtn_idx = e2m1_index_nearest(np.abs(xd), S)
        rtn_signed = np.where(np.signbit(xs), -rtn_idx, rtn_idx)
        same = signed_index(nib[r0:r1]) == rtn_signed
        moved += [same.sum(), (~same).sum()]
    return pack_nibbles(nib), x_fq, moved
