"""The decode GEMV reads 3-, 5- and 6-bit codes as window pairs: pair
(c1, c2) of a 32-code half comes from the 32-bit window of the half's words
that starts at bit s, with one AND-OR of a mask and of the magic exponents
2^(10-o) (o = the code's bit offset in its 16-bit half).  This CPU test reads
the tables from the kernel source and emulates the two instructions on words
packed by the oracle: every pair must decode, as fp16, to exactly
(2^(10-o1) + q[c1], 2^(10-o2) + q[c2]), and the pairs must cover each half
once.  (The kernel source also checks coverage and offsets at compile time;
this checks the masks, magics and windows against the packing itself.)"""
import os
import re

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(__file__), "..", "quantized_matmul_qgemv_amd", "csrc", "qgemv.hip")


def window_pairs(bits):
    src = open(SRC).read()
    m = re.search(r"struct WinPairs<%d> \{\s*static constexpr WinPair p\[16\] = \{(.*?)\};" % bits, src, re.S)
    assert m, f"no WinPairs<{bits}> table in the GEMV source"
    pairs = [tuple(map(int, t)) for t in re.findall(r"\{(\d+), (\d+), (\d+)\}", m.group(1))]
    assert len(pairs) == 16
    return pairs


def window(words, s, bits):
    """Bits s .. s+31 of the half's `bits` words (0 past the end), as the
    kernel forms them: the word itself, a funnel shift of two words, or a
    shift of the last word."""
    j, r = divmod(s, 32)
    if r == 0:
        return int(words[j])
    hi = int(words[j + 1]) if j + 1 < bits else 0
    return ((hi << 32) | int(words[j])) >> r & 0xFFFFFFFF


@pytest.mark.parametrize("bits", [3, 5, 6])
def test_window_pairs_decode_the_oracle_packing(bits):
    pairs = window_pairs(bits)
    assert sorted(c for _, c1, c2 in pairs for c in (c1, c2)) == list(range(32))
    r = np.random.default_rng(bits)
    codes = r.integers(0, 1 << bits, (9, 256), dtype=np.uint8)
    codes[0] = (1 << bits) - 1            # all ones: every mask bit set
    codes[1] = 0
    words = oracle.pack(codes, bits).view(np.uint32)
    mask_all = (1 << bits) - 1
    for row in range(codes.shape[0]):
        for half in range(codes.shape[1] // 32):
            w = words[row, half * bits:(half + 1) * bits]
            for s, c1, c2 in pairs:
                o1, o2 = bits * c1 - s, bits * c2 - s - 16
                assert 0 <= o1 and o1 + bits <= 10 and 0 <= o2 and o2 + bits <= 10, (bits, s, c1, c2)
                mask = (mask_all << o1) | (mask_all << (16 + o2))
                magic = ((25 - o1) << 10) | ((25 - o2) << 26)
                v = (window(w, s, bits) & mask) | magic
                lo, hi = np.array([v & 0xFFFF, v >> 16], dtype=np.uint16).view(np.float16).astype(np.float64)
                assert lo - 2.0 ** (10 - o1) == codes[row, half * 32 + c1], (bits, row, half, s, c1)
                assert hi - 2.0 ** (10 - o2) == codes[row, half * 32 + c2], (bits, row, half, s, c2)


@pytest.mark.parametrize("bits", [3, 5, 6])
def test_planted_table_mistake_is_caught(bits):
    """A window start one bit off must fail the emulation (the check above is
    not vacuous)."""
    pairs = window_pairs(bits)
    s, c1, c2 = next(p for p in pairs if p[0] % 32)   # a shifted window
    codes = np.arange(64, dtype=np.uint8)[None] % (1 << bits)
    words = oracle.pack(codes, bits).view(np.uint32)
    w = words[0, :bits]
    o1, o2 = bits * c1 - s, bits * c2 - s - 16
    mask = (((1 << bits) - 1) << o1) | (((1 << bits) - 1) << (16 + o2))
    magic = ((25 - o1) << 10) | ((25 - o2) << 26)
    v = (window(w, s + 1, bits) & mask) | magic
    lo, hi = np.array([v & 0xFFFF, v >> 16], dtype=np.uint16).view(np.float16).astype(np.float64)
    assert (lo - 2.0 ** (10 - o1), hi - 2.0 ** (10 - o2)) != (codes[0, c1], codes[0, c2])
