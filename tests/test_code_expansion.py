"""CPU check of the byte arithmetic the low-bit decode kernels use to turn a
row of packed two's-complement codes into fp16 A-fragment slots: the row's
8-nibble window is split into even and odd nibbles (each in the upper half
of a byte), v_perm places nibble k in the slot of the k-th set bit of the
row's mask byte (selector 0x0C gives a zero byte for a clear bit), a xor
with 0x80 turns the nibble q into q + 8, and 0x54 in the high byte makes the
fp16 value 64 + (q + 8) = q + 72.  2-bit codes are placed in the top two
bits of their byte instead, so a code c becomes 4c + 72 (the kernels scale
the corrected sums by 1/4).  The expected values come from the mask and the
codes alone: slot p holds its code (times 4 for 2-bit) + 72 when bit p is
set, else 72.  No kernel is launched."""
import numpy as np


def v_perm(s0, s1, sel):
    """v_perm_b32 for the selector bytes used here: 0-7 pick byte s of the
    64-bit value s0:s1 (s1 the low dword), 0x0C gives 0."""
    src = (int(s0) << 32) | int(s1)
    out = 0
    for i in range(4):
        s = (sel >> (8 * i)) & 0xFF
        b = (src >> (8 * s)) & 0xFF if s < 8 else (0 if s == 0x0C else None)
        assert b is not None
        out |= b << (8 * i)
    return out


def row_selectors(b):
    """Byte selectors for mask byte b: slot p takes nibble k = set bits of b
    below p when bit p is set; nibble k is byte k/2 of lo4 (k even, bytes
    0-3) or of hi4 (k odd, bytes 4-7)."""
    sel = [0, 0]
    for p in range(8):
        v = 0x0C
        if (b >> p) & 1:
            k = bin(b & ((1 << p) - 1)).count("1")
            v = 4 + (k >> 1) if k & 1 else k >> 1
        sel[p // 4] |= v << (8 * (p % 4))
    return sel


def split4(codes):
    """The 4-bit window of a row's codes, split as the kernels do."""
    win = 0
    for k, q in enumerate(codes):
        win |= (q & 0xF) << (4 * k)
    return (win << 4) & 0xF0F0F0F0, win & 0xF0F0F0F0


def split2(codes):
    """The 2-bit window (16 bits) spread to one code per nibble, then each
    code moved to the top two bits of its byte, even codes in lo4 and odd
    codes in hi4."""
    t = 0
    for k, c in enumerate(codes):
        t |= (c & 0x3) << (2 * k)
    t = (t | (t << 8)) & 0x00FF00FF
    t = (t | (t << 4)) & 0x0F0F0F0F
    t = (t | (t << 2)) & 0x33333333
    return (t << 6) & 0xC0C0C0C0, (t << 2) & 0xC0C0C0C0


def expand(codes, b, bits=4):
    """fp16 slots of a row: codes are the row's kept values in order."""
    lo4, hi4 = (split4 if bits == 4 else split2)(codes)
    sx, sy = row_selectors(b)
    e0 = v_perm(hi4, lo4, sx) ^ 0x80808080
    e1 = v_perm(hi4, lo4, sy) ^ 0x80808080
    dw = [v_perm(0x54545454, e0, 0x04010400), v_perm(0x54545454, e0, 0x04030402),
          v_perm(0x54545454, e1, 0x04010400), v_perm(0x54545454, e1, 0x04030402)]
    return np.array(dw, dtype=np.uint32).view(np.float16).astype(np.float64)


def test_every_mask_byte_and_code():
    rng = np.random.default_rng(5)
    for b in range(256):
        n = bin(b).count("1")
        for _ in range(4):
            codes = [int(c) for c in rng.integers(-8, 8, size=n)]
            slots = expand(codes, b)
            want = np.full(8, 72.0)
            k = 0
            for p in range(8):
                if (b >> p) & 1:
                    want[p] += codes[k]
                    k += 1
            assert np.array_equal(slots, want), (b, codes, slots, want)


def test_extreme_codes_are_exact():
    for q in range(-8, 8):
        assert np.array_equal(expand([q] * 8, 0xFF), np.full(8, 72.0 + q))
    # the offset form is exact: 64 + u for every nibble u
    for u in range(16):
        h = np.array([0x5400 | (u << 4)], dtype=np.uint16).view(np.float16)[0]
        assert float(h) == 64.0 + u


def test_two_bit_codes_every_mask_byte():
    rng = np.random.default_rng(6)
    for b in range(256):
        n = bin(b).count("1")
        for _ in range(4):
            codes = [int(c) for c in rng.integers(-2, 2, size=n)]
            slots = expand(codes, b, bits=2)
            want = np.full(8, 72.0)
            k = 0
            for p in range(8):
                if (b >> p) & 1:
                    want[p] += 4 * codes[k]
                    k += 1
            assert np.array_equal(slots, want), (b, codes, slots, want)
