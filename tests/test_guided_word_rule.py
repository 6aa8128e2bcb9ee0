"""The guided-rounding kernel's word arithmetic, restated in Python.

The kernel (csrc/trainer.hip, guided_kernel) takes per element only the sign
of level*S - |x| and then makes the rollout-guided choice of the TRACE summary
("Core method", method step four) on eight 4-bit codes at once.  This test
mirrors those word formulas and checks them against the per-element rule:
the candidates are the round-to-nearest index i and its neighbour on x's side
(i + 1 up to 7 when the level lies below |x|, i - 1 when above, none on the
level); the full-code rule keeps the candidate on the rollout level's side in
signed index order, the record rule the candidate whose index has the recorded
low bit; S == 0 keeps every code.  The histogram counts the signed-index
distance 0, 1 or more between round-to-nearest and the rollout code.  The GPU
tests check the kernel itself against the oracle.
"""
import random

M32 = 0xFFFFFFFF


def nibble_zero3(t):
    return ~(t + 0x77777777) & 0x88888888 & M32


def nibble_zero4(t):
    return ~(t | ((t & 0x77777777) + 0x77777777)) & 0x88888888 & M32


def nibble_spread8(b):
    b = (b | (b << 12)) & 0x000F000F
    b = (b | (b << 6)) & 0x03030303
    return (b | (b << 3)) & 0x11111111


def word_rule(w, lt, gt, rw, rbits, live, record):
    """The kernel's choice for the eight codes of w.  lt / gt: bit 3 of
    nibble j set when level*S - |x| of element j is below / above zero."""
    i_, sgn = w & 0x77777777, w & 0x88888888
    inc = (lt & ~(i_ + 0x11111111) & 0x88888888) >> 3
    dec = gt >> 3
    if record:
        flip = ((i_ ^ nibble_spread8(rbits & 0xFF)) & 0x11111111) if live else 0
        pick = (i_ + (flip & inc) - (flip & dec)) & M32
        return sgn | pick, bin(flip & (inc | dec)).count("1"), None
    r_, rs = rw & 0x77777777, rw & 0x88888888
    same = ((~(rs ^ sgn) & M32) | (~(r_ + 0x77777777) & M32)) & 0x88888888
    hi = i_ + inc
    ge = ((r_ | 0x88888888) - hi) & 0x88888888
    sel = ((same & ge) >> 3) if live else 0
    pick = (i_ - dec + (sel & (inc | dec))) & M32
    ad = ((r_ | 0x88888888) - i_) & M32
    e0 = same & nibble_zero3(r_ ^ i_)
    e1 = (same & (nibble_zero4(ad ^ 0x99999999) | nibble_zero4(ad ^ 0x77777777))) | \
        ((~same & M32) & nibble_zero4((r_ + i_) ^ 0x11111111))
    return sgn | pick, bin(e0).count("1"), bin(e1).count("1")


def signed_index(code):
    return -(code & 7) if code & 8 else code & 7


def element_rule(code, dsign, rcode, rbit, live, record):
    """(guided code, moved or distance == 0, distance == 1) of one element."""
    i, sgn = code & 7, code & 8
    if dsign < 0:
        other = i + 1 if i < 7 else i
    elif dsign > 0:
        other = i - 1
    else:
        other = i
    if not live:
        pick = i
    elif record:
        pick = other if (i ^ rbit) & 1 else i
    else:
        # of the two adjacent candidates (in signed index order, both with
        # x's sign), the one on the rollout code's side
        sgn_f = -1 if sgn else 1
        lo, hi = sorted({i, other}, key=lambda m: sgn_f * m)[0], sorted({i, other}, key=lambda m: sgn_f * m)[-1]
        pick = hi if signed_index(rcode) >= sgn_f * hi else lo
    dist = abs(signed_index(code) - signed_index(rcode))
    if record:
        return sgn | pick, int(pick != i), None
    return sgn | pick, int(dist == 0), int(dist == 1)


def consistent_cases():
    for code in range(16):
        for dsign in (-1, 0, 1):
            if dsign > 0 and code & 7 == 0:      # level 0 never lies above |x|
                continue
            for rcode in range(16):
                for rbit in (0, 1):
                    yield code, dsign, rcode, rbit


def test_word_rule_matches_element_rule():
    rng = random.Random(1)
    cases = list(consistent_cases())
    for record in (False, True):
        for live in (True, False):
            # S == 0: every round-to-nearest code has magnitude 0 and level*S - |x| <= 0
            pool = [c for c in cases if live or (c[0] & 7 == 0 and c[1] <= 0)]
            for pos in range(8):
                for case in pool:
                    els = [rng.choice(pool) for _ in range(8)]
                    els[pos] = case
                    w = rw = lt = gt = rbits = 0
                    want_g, want_a, want_b = 0, 0, 0
                    for j, (code, dsign, rcode, rbit) in enumerate(els):
                        w |= code << (4 * j)
                        rw |= rcode << (4 * j)
                        rbits |= rbit << j
                        lt |= (8 << (4 * j)) if dsign < 0 else 0
                        gt |= (8 << (4 * j)) if dsign > 0 else 0
                        g, a, b = element_rule(code, dsign, rcode, rbit, live, record)
                        want_g |= g << (4 * j)
                        want_a += a
                        want_b += b or 0
                    got_g, got_a, got_b = word_rule(w, lt, gt, rw, rbits, live, record)
                    assert got_g == want_g, (record, live, els)
                    assert got_a == want_a, (record, live, els)
                    if not record:
                        assert got_b == want_b, (record, live, els)
