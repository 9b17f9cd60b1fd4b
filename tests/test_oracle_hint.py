"""Pins for the oracle's page-order hint (oracle.page_kmax): the largest bf16 exponent field of
each (sequence, kv head, logical page)'s K values.

The hint is not part of the pages' method; the attention only uses it to choose which page
each wave visits first.  Its pin is independent of bit manipulation: the expected exponent
field of every value comes from math.frexp of the float (biased exponent e + 126 for a normal
value m 2^e with m in [0.5, 1), 0 for zeros and subnormals, 255 for infinities and NaNs), over
tokens chosen so that a mistake in the token range (values past seq_lens, the page past the
end), in the K / V choice or in the head index changes the answer.
"""
import math
import struct

import numpy as np

import oracle

T, H, D = 4, 2, 64


def bf16(x: float) -> int:
    """bf16 bits of x (x exactly representable: its low 16 float bits are zero)."""
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    assert b & 0xFFFF == 0 or math.isnan(x), x
    return b >> 16


def field(x: float) -> int:
    if math.isnan(x) or math.isinf(x):
        return 255
    if x == 0.0 or abs(x) < 2.0 ** -126:
        return 0
    return math.frexp(x)[1] + 126


def test_page_kmax_against_frexp():
    P = 5
    pages = np.zeros((P, H, 2, T, D), np.uint16)
    vals = {}  # (page, head, kv, slot, dim) -> float

    def put(p, h, kv, t, d, x):
        pages[p, h, kv, t, d] = bf16(x)
        vals[(p, h, kv, t, d)] = x

    # sequence 0: 6 tokens on pages 3 (tokens 0-3) and 1 (tokens 4, 5); page 1's slots 2, 3
    # are past the end and hold larger values
    put(3, 0, 0, 0, 5, 3.0)
    put(3, 0, 0, 2, 63, -1000.0)
    put(3, 0, 1, 1, 0, 2.0 ** 100)        # V: never counted
    put(3, 1, 0, 3, 7, 2.0 ** -100)
    put(3, 1, 0, 0, 0, 2.0 ** -130)       # subnormal
    put(1, 0, 0, 1, 1, 0.375)
    put(1, 0, 0, 2, 1, 2.0 ** 90)         # past seq_lens
    put(1, 1, 0, 0, 9, -7.0)
    put(1, 1, 0, 3, 9, float("inf"))      # past seq_lens
    # sequence 1: 3 tokens on page 0, with an infinity and a NaN; page 4 listed, never used
    put(0, 0, 0, 2, 3, float("-inf"))
    put(0, 1, 0, 1, 4, float("nan"))
    put(4, 0, 0, 0, 0, 2.0 ** 120)
    lens = np.array([6, 3], np.int32)
    pt = np.array([[3, 1, 2], [0, 4, -1]], np.int32)

    want = np.zeros((2, H, 3), np.int64)
    for (p, h, kv, t, d), x in vals.items():
        for b in range(2):
            for lp in range(3):
                if pt[b, lp] == p and kv == 0 and lp * T + t < lens[b]:
                    want[b, h, lp] = max(want[b, h, lp], field(x))
    got = oracle.page_kmax(pages, lens, pt)
    assert got.dtype == np.uint32 and got.shape == (2, H, 3)
    assert np.array_equal(got.astype(np.int64), want)
    # spelled out: the fields the sweep above found
    assert want[0, 0, 0] == 136 and want[0, 1, 0] == 27      # -1000 (2^9.97), 2^-100
    assert want[0, 0, 1] == 125 and want[0, 1, 1] == 129     # 0.375, -7
    assert want[1, 0, 0] == 255 and want[1, 1, 0] == 255     # -inf, NaN
    assert not want[0, :, 2].any() and not want[1, :, 1:].any()


def test_page_kmax_of_random_pages_is_the_largest_magnitude_field():
    """On random pages the field of the largest |k| of each page (found with numpy on the
    float values) is the hint."""
    rng = np.random.default_rng(5)
    P, B, maxp = 12, 3, 4
    f = (rng.standard_normal((P, H, 2, T, D)) * np.exp2(rng.integers(-20, 20, (P, H, 2, T, 1)))).astype(np.float32)
    pages = (f.view(np.uint32) >> 16).astype(np.uint16)
    vals = (pages.astype(np.uint32) << 16).view(np.float32)
    pt = rng.permutation(P)[: B * maxp].reshape(B, maxp).astype(np.int32)
    lens = np.array([16, 5, 0], np.int32)
    got = oracle.page_kmax(pages, lens, pt)
    for b in range(B):
        for p in range(maxp):
            n = max(0, min(T, int(lens[b]) - p * T))
            for h in range(H):
                want = field(float(np.abs(vals[pt[b, p], h, 0, :n]).max())) if n else 0
                assert got[b, h, p] == want, (b, h, p)
