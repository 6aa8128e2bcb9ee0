"""E2M1 (FP4) and E4M3 codebooks with exact round-to-nearest-even.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

E2M1: the FP4 element format of NVFP4.  The TRACE summary ("Prerequisites:
NVFP4 and the E2M1 codebook") says an E2M1 value has 2 exponent bits and one
mantissa bit, takes only a finite set of codebook values, and that real
inputs are mapped by round-to-nearest onto the nearest codeword after the
global and per-block scales are applied.  The QUADS summary (section 1,
"Problem Statement") counts 8 levels per sign.  The non-negative levels are
0, 0.5, 1, 1.5, 2, 3, 4, 6 (index 0..7).  A 4-bit code is sign<<3 | index;
index = exponent<<1 | mantissa with exponent bias 1 (exponent 0 is the
subnormal range 0, 0.5).

E4M3: the per-16-element block-scale format.  Reading (the pages only name
"block scale"): OCP E4M3FN -- bias 7, no infinities, max 448, subnormals
m * 2^-9, bytes 0x7F/0xFF are NaN and are never produced.  There are 127
finite non-negative values (bytes 0x00..0x7E).

Rounding rule for both: nearest value to an EXACT real quotient a/d; a tie
goes to the code whose least significant bit is 0 ("even"); values above the
largest finite value saturate to it.  The decision is made by comparing a
against midpoint*d, where midpoint*d is exact in float64 (see each function).
"""

import numpy as np

# ---------------------------------------------------------------------------
# E2M1
# ---------------------------------------------------------------------------

#: Non-negative E2M1 magnitudes by index (QUADS section 1 / TRACE prerequisites).
E2M1_LEVELS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

#: Midpoints between consecutive E2M1 magnitudes; midpoint j lies between
#: index j and j+1.  Each has at most 3 significant bits.
E2M1_MIDPOINTS = (E2M1_LEVELS[:-1] + E2M1_LEVELS[1:]) / 2.0


def e2m1_decode(codes):
    """Value of 4-bit E2M1 codes (any integer array, low nibble used)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = E2M1_LEVELS[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e2m1_index_nearest(ax, d):
    """Index 0..7 of the E2M1 magnitude nearest to the real ax/d.

    ax >= 0 and d > 0 are float64 arrays (broadcastable) holding exact fp32
    values.  ax is compared with midpoint_j * d; midpoint_j has <= 3
    significant bits and d (an fp32 value) <= 24, so the product is exact in
    float64 and the comparison decides the exact real quotient.  A tie
    (ax == midpoint_j * d) goes to the even index.  ax/d > 6 gives 7 (6.0).
    Entries with d == 0 give index 0.
    """
    ax = np.asarray(ax, dtype=np.float64)
    d = np.asarray(d, dtype=np.float64)
    ax, d = np.broadcast_arrays(ax, d)
    idx = np.zeros(ax.shape, dtype=np.int64)
    for j, mid in enumerate(E2M1_MIDPOINTS):
        t = mid * d                       # exact
        above = ax > t
        tie = ax == t
        # past midpoint j the nearest index is >= j+1; on the midpoint the
        # even one of (j, j+1) wins: j+1 exactly when j is odd.
        idx += above | (tie & (j % 2 == 1))
    idx[d == 0] = 0
    return idx


# ---------------------------------------------------------------------------
# E4M3 (OCP E4M3FN)
# ---------------------------------------------------------------------------

def _e4m3_value(byte):
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0:
        v = m * 2.0 ** -9
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if byte & 0x80 else v


#: Finite non-negative E4M3 values, indexed by code byte 0x00..0x7E.
E4M3_VALUES = np.array([_e4m3_value(b) for b in range(0x7F)], dtype=np.float64)

#: Midpoints between consecutive E4M3 values (126 of them); each has <= 5
#: significant bits.
E4M3_MIDPOINTS = (E4M3_VALUES[:-1] + E4M3_VALUES[1:]) / 2.0

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Value of E4M3FN bytes (NaN for 0x7F/0xFF)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    mag = np.where((c & 0x7F) == 0x7F, np.nan, E4M3_VALUES[np.minimum(c & 0x7F, 0x7E)])
    return np.where((c & 0x80) != 0, -mag, mag)


def e4m3_code_nearest(a, d):
    """E4M3 byte (0x00..0x7E) nearest to the non-negative real a/d.

    a >= 0 is a float64 array of exact fp32 values; d > 0 is one float64
    number with d*midpoint exact in float64: callers pass d = 6*g with g an
    fp32 value, so d has <= 26 significant bits and d*midpoint <= 31.
    The code is the number of midpoints below a/d, plus one when a/d sits
    exactly on a midpoint whose upper neighbour is the even byte.  Hence ties
    go to the even byte, a/d above 448 saturates to 448 (0x7E) and a/d at or
    below 2^-10 rounds to 0.
    """
    a = np.asarray(a, dtype=np.float64)
    t = E4M3_MIDPOINTS * float(d)          # exact, increasing
    below = np.searchsorted(t, a, side="left")          # count of t < a
    on_mid = (below < t.size) & (a == t[np.minimum(below, t.size - 1)])
    tie_up = on_mid & (below % 2 == 1)
    return (below + tie_up).astype(np.uint8)


# ---------------------------------------------------------------------------
# bf16 helpers (storage format of activations and weights)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x):
    """Round fp32 values to bf16 (RNE) and return the uint16 bit patterns.

    Inputs are finite (non-finite values are outside the contract)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact fp32 values of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f64_to_bf16_bits(x):
    """Round float64 values directly (once) to bf16, RNE, as bit patterns.

    Used where a stored bf16 is defined as the rounding of a real result
    (the SwiGLU output of the MoE layer).  |x| = m * 2^e with m in [0.5, 1);
    bf16 keeps 8 significant bits, so its spacing at |x| is 2^(e-8), and
    2^-133 in the subnormal range.  Scaling by a power of two is exact and
    np.rint rounds half to even."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(np.abs(x))
    shift = np.maximum(e - 8, -133)
    n = np.rint(np.ldexp(np.abs(x), -shift))
    r = np.copysign(np.ldexp(n, shift), x)
    return f32_to_bf16_bits(r.astype(np.float32))
