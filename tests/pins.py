"""Pins of the CPU oracle against facts that do not come from the oracle.

Every check takes the oracle module as an argument, so the same checks can
run against the real oracle (test_oracle_pins.py) and against copies with a
planted mistake (test_oracle_mutants.py), which must fail at least one.

Sources of truth used here, none of them the oracle's own formulas:
  * hand-worked fixtures in golden/hand_cases.json;
  * exact rational arithmetic (fractions.Fraction) for rounding and dots;
  * closed forms (one-hot and all-ones activations, unit-scale integer codes);
  * exhaustive enumeration (all codes of a group, all byte patterns);
  * mathematical invariants (nearest quantization level, error bounds).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ------------------------------------------------------ exact fp helpers --

def exact(v) -> Fraction:
    """Exact rational value of a finite binary float."""
    return Fraction(float(v))


def rne_to_binary(v: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round a rational to the nearest binary float with `mant_bits`
    fraction bits, minimum normal exponent emin, max exponent emax, ties
    to even; returns the rounded value (inf as Fraction not supported, so
    callers stay in range).  Written from the IEEE-754 definition."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix floating log2 off-by-one
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)                       # subnormal range shares emin's ulp
    ulp = Fraction(2) ** (e - mant_bits)
    q = a / ulp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    assert r <= Fraction(2) ** (emax + 1), "overflow"
    return sign * r


def rne_f16(v: Fraction) -> Fraction:
    return rne_to_binary(v, 10, -14, 15)


def rne_f32(v: Fraction) -> Fraction:
    return rne_to_binary(v, 23, -126, 127)


# ------------------------------------------------------------- fp16 pins --

def check_f16_rounding(o, seed=0):
    """oracle.f16_bits / round_to_f16_bits / round_to_f32 equal exact
    round-to-nearest-even, on random values, on every fp16 halfway point of
    a few binades, and on float64 values where rounding through float32
    first would give a different (double-rounded) fp16."""
    r = np.random.default_rng(seed)
    vals = list(r.standard_normal(2000) * 10.0 ** r.integers(-7, 4, 2000))
    # halfway points between consecutive fp16 values (normal and subnormal)
    for e in (-24, -20, -15, -14, -3, 0, 7, 14):
        ulp = Fraction(2) ** (e - 10) if e >= -14 else Fraction(2) ** -24
        for m in (1024, 1025, 1500, 2047):
            base = m * ulp if e >= -14 else (m % 1024) * ulp
            vals.append(float(base + ulp / 2))
            vals.append(-float(base + ulp / 2))
    # double-rounding traps: just above a fp16 halfway point by less than a
    # float32 ulp, so RN32 lands exactly on the halfway point
    for m in (1025, 1026, 1027, 1701):
        half = (Fraction(m) + Fraction(1, 2)) * Fraction(2) ** -10
        vals.append(float(half + Fraction(2) ** -40))
        vals.append(float(half - Fraction(2) ** -40))
    vals = np.array(vals, dtype=np.float64)
    got16 = o.round_to_f16_bits(vals).view(np.float16).astype(np.float64)
    for v, g in zip(vals, got16):
        assert exact(g) == rne_f16(exact(v)), (v, g)
    got32 = o.round_to_f32(vals).astype(np.float64)
    for v, g in zip(vals, got32):
        assert exact(g) == rne_f32(exact(v)), (v, g)
    v32 = vals.astype(np.float32)
    g = o.f16_bits(v32).view(np.float16).astype(np.float64)
    for v, gg in zip(v32, g):
        assert exact(gg) == rne_f16(exact(v)), (v, gg)


# --------------------------------------------------------- packing pins --

def check_pack_golden(o):
    for case in golden()["pack"]:
        bits = case["bits"]
        codes = np.array([case["codes"]], dtype=np.uint8)
        want = np.array([[int(w, 16) for w in case["words"]]], dtype=np.uint32)
        got = o.pack(codes, bits)
        assert got.dtype == np.uint32 and got.shape == want.shape, (bits, got.shape)
        assert np.array_equal(got, want), (bits, [hex(x) for x in got[0]])
        assert np.array_equal(o.unpack(want, bits, codes.shape[1]), codes), bits


def check_pack_roundtrip(o, seed=1):
    """unpack(pack(q)) == q for every code pattern: for each width, one row
    per byte value 0..255 laid over the first codes, plus random rows."""
    r = np.random.default_rng(seed)
    for bits in (2, 3, 4, 5, 6, 8):
        k = 64
        levels = 1 << bits
        rows = []
        for byte in range(256):
            row = np.zeros(k, dtype=np.uint8)
            # spread the byte's bits over consecutive codes
            stream = [(byte >> j) & 1 for j in range(8)]
            for i in range(k):
                c = 0
                for j in range(bits):
                    c |= stream[(i * bits + j) % 8] << j
                row[i] = c
            rows.append(row)
        rows.append(r.integers(0, levels, k, dtype=np.uint8))
        rows.append(np.full(k, levels - 1, dtype=np.uint8))
        codes = np.stack(rows)
        words = o.pack(codes, bits)
        assert words.shape == (codes.shape[0], k * bits // 32)
        assert np.array_equal(o.unpack(words, bits, k), codes), bits
        # independent bit-level check of the stream on the random row
        row, wrow = codes[-2], words[-2]
        acc = 0
        for i, c in enumerate(row):
            acc |= int(c) << (bits * i)
        for j, w in enumerate(wrow):
            assert int(w) == (acc >> (32 * j)) & 0xFFFFFFFF, (bits, j)


# ------------------------------------------------------- quantizer pins --

def _h1_w():
    return (np.arange(64) % 16 / 64.0).astype(np.float32)[None, :]


def check_quantize_golden(o):
    g = {c["name"].split()[0]: c for c in golden()["quantize"]}
    # H1
    w = _h1_w()
    q, s, b = o.quantize(w, 4)
    assert s[0, 0] == int(g["H1"]["s_bits"], 16) and b[0, 0] == int(g["H1"]["b_bits"], 16)
    assert np.array_equal(q[0], np.arange(64) % 16)
    words = o.pack(q, 4)
    ones = np.ones((1, 64), dtype=np.float16)
    assert o.qmatmul_f64(words, s, b, ones, 4)[0, 0] == g["H1"]["y_ones"]
    first8 = np.zeros((1, 64), dtype=np.float16)
    first8[0, :8] = 1
    assert o.qmatmul_f64(words, s, b, first8, 4)[0, 0] == g["H1"]["y_first8"]
    assert np.array_equal(o.dequant_f64(q, s, b), w.astype(np.float64))
    # H2
    qv = np.concatenate([np.arange(0, 252, 4), [255]])
    w = (-1.0 + qv / 128.0).astype(np.float32)[None, :]
    q, s, b = o.quantize(w, 8)
    assert s[0, 0] == int(g["H2"]["s_bits"], 16) and b[0, 0] == int(g["H2"]["b_bits"], 16)
    assert np.array_equal(q[0], qv)
    # H3
    w = _h1_w()
    w[0, 1:4] = np.array([0.5, 1.5, 2.5], dtype=np.float32) / np.float32(64)
    q, s, b = o.quantize(w, 4)
    assert list(q[0, 1:4]) == g["H3"]["codes_1_3"]
    # H4
    w = np.full((1, 64), 0.3, dtype=np.float32)
    q, s, b = o.quantize(w, 4)
    assert s[0, 0] == int(g["H4"]["s_bits"], 16) and b[0, 0] == int(g["H4"]["b_bits"], 16)
    assert not q.any()
    # H5
    w = (np.float32(0.3) + np.float32(1e-7) * np.arange(64, dtype=np.float32))[None, :]
    q, s, b = o.quantize(w, 4)
    assert s[0, 0] == int(g["H5"]["s_bits"], 16) and b[0, 0] == int(g["H5"]["b_bits"], 16)
    assert not q.any()
    err = np.abs(o.dequant_f64(q, s, b) - w.astype(np.float64)).max()
    assert err < g["H5"]["max_abs_err_below"]


def check_quantize_nearest_level(o, seed=2):
    """Brute force on 4x64 matrices: every chosen code is (one of) the
    nearest of the 2**bits levels s*c + b to w, and codes are in range.
    Equidistant levels (within a float32 rounding slop) may go either way."""
    r = np.random.default_rng(seed)
    for bits in (2, 3, 4, 5, 6, 8):
        levels = (1 << bits) - 1
        w = (r.standard_normal((4, 64)) * 0.02).astype(np.float32)
        w[3] = r.uniform(-3, 5, 64).astype(np.float32)
        q, s, b = o.quantize(w, bits)
        assert q.dtype == np.uint8 and q.max() <= levels
        sv = o.f16_value(s)[:, 0]
        bv = o.f16_value(b)[:, 0]
        for n in range(4):
            lv = sv[n] * np.arange(levels + 1) + bv[n]
            for kk in range(64):
                d = np.abs(lv - float(w[n, kk]))
                slop = 2.0 ** -20 * (abs(float(w[n, kk])) + abs(bv[n]) + sv[n] * levels)
                assert d[q[n, kk]] <= d.min() + slop, (bits, n, kk)


def check_quantize_error_bound(o, seed=3):
    """|w - W_hat| <= s/2 + |b - mn| + L*|s - (mx-mn)/L| + 2^-20*(|mn|+|mx|),
    the half step plus the fp16 rounding of b and s and fp32 slop."""
    r = np.random.default_rng(seed)
    for bits in (2, 3, 4, 5, 6, 8):
        levels = (1 << bits) - 1
        w = (r.standard_normal((16, 256)) * 0.02).astype(np.float32)
        q, s, b = o.quantize(w, bits)
        w_hat = o.dequant_f64(q, s, b)
        wg = w.astype(np.float64).reshape(16, 4, 64)
        mn, mx = wg.min(axis=2), wg.max(axis=2)
        sv, bv = o.f16_value(s), o.f16_value(b)
        bound = sv / 2 + np.abs(bv - mn) + levels * np.abs(sv - (mx - mn) / levels) \
            + 2.0 ** -20 * (np.abs(mn) + np.abs(mx))
        err = np.abs(w_hat - w.astype(np.float64)).reshape(16, 4, 64).max(axis=2)
        assert np.all(err <= bound), bits
        # min and max of each group are reconstructed to within the bound too
        assert np.all(np.abs(w_hat.reshape(16, 4, 64).min(axis=2) - mn) <= bound)


# ---------------------------------------------------------- matmul pins --

def check_dot_exact_rational(o, seed=4):
    """4x64 brute force: y from the oracle equals the exact rational
    sum_k x_k * (s*q_k + b) within gamma_K * sum|x * W_hat|."""
    r = np.random.default_rng(seed)
    for bits in (2, 3, 4, 5, 6, 8):
        w = (r.standard_normal((4, 64)) * 0.02).astype(np.float32)
        x = r.standard_normal((2, 64)).astype(np.float16)
        q, s, b = o.quantize(w, bits)
        y = o.qmatmul_f64(o.pack(q, bits), s, b, x, bits)
        assert y.shape == (2, 4)
        gamma = 64 * 2.0 ** -53 / (1 - 64 * 2.0 ** -53)
        for m in range(2):
            for n in range(4):
                sv, bv = exact(o.f16_value(s[n, 0])), exact(o.f16_value(b[n, 0]))
                terms = [exact(x[m, kk]) * (sv * int(q[n, kk]) + bv) for kk in range(64)]
                ex = sum(terms)
                mag = sum(abs(t) for t in terms)
                assert abs(exact(y[m, n]) - ex) <= Fraction(gamma) * mag, (bits, m, n)


def check_closed_forms(o, seed=5):
    """one-hot x gives a column of W_hat; x = 1 gives
    sum_g (s_g * sum_{k in g} q_k + 64 * b_g); unit scale and zero bias give
    an integer matmul; scaling x by 2 scales y by 2 exactly."""
    r = np.random.default_rng(seed)
    n, k = 8, 192
    for bits in (2, 3, 4, 5, 6, 8):
        w = (r.standard_normal((n, k)) * 0.02).astype(np.float32)
        q, s, b = o.quantize(w, bits)
        words = o.pack(q, bits)
        sv, bv = o.f16_value(s), o.f16_value(b)
        for kk in (0, 1, 63, 64, 100, k - 1):
            e = np.zeros((1, k), dtype=np.float16)
            e[0, kk] = 1
            col = o.qmatmul_f64(words, s, b, e, bits)[0]
            want = sv[:, kk // 64] * q[:, kk].astype(np.float64) + bv[:, kk // 64]
            assert np.array_equal(col, want), (bits, kk)
        ones = np.ones((1, k), dtype=np.float16)
        want = (sv * q.reshape(n, 3, 64).sum(axis=2) + 64 * bv).sum(axis=1)
        assert np.allclose(o.qmatmul_f64(words, s, b, ones, bits)[0], want, rtol=1e-14, atol=1e-14)
        x = r.standard_normal((3, k)).astype(np.float16)
        y1 = o.qmatmul_f64(words, s, b, x, bits)
        y2 = o.qmatmul_f64(words, s, b, (x.astype(np.float32) * 2).astype(np.float16), bits)
        assert np.array_equal(y2, 2 * y1)
        # integer special case: s = 1.0 (0x3C00), b = 0, small-integer x
        one = np.full(s.shape, 0x3C00, dtype=np.uint16)
        zero = np.zeros(b.shape, dtype=np.uint16)
        xi = r.integers(-8, 9, (3, k))
        yi = o.qmatmul_f64(words, one, zero, xi.astype(np.float16), bits)
        assert np.array_equal(yi, (xi @ q.astype(np.int64).T).astype(np.float64))


def check_gemm_rows_are_gemvs(o, seed=6):
    """Row m of the M>1 product equals the M=1 product of x[m]; the output
    has shape [M, N] with N the weight's row count (not a transposition)."""
    r = np.random.default_rng(seed)
    w = (r.standard_normal((5, 128)) * 0.02).astype(np.float32)
    q, s, b = o.quantize(w, 4)
    words = o.pack(q, 4)
    x = r.standard_normal((3, 128)).astype(np.float16)
    y = o.qmatmul_f64(words, s, b, x, 4)
    assert y.shape == (3, 5)
    for m in range(3):
        assert np.allclose(y[m], o.qmatmul_f64(words, s, b, x[m:m + 1], 4)[0], rtol=1e-15, atol=0)


# --------------------------------------------------------- grouped pins --

def check_grouped(o, seed=7):
    """Grouped product: each output row equals the dense product of its own
    expert and A row (token row pair // top_k, or the pair's own row);
    a single expert equals the dense product; rows of unused experts are
    never touched; empty input gives an empty output."""
    r = np.random.default_rng(seed)
    e_count, n, k, t, top_k = 5, 6, 128, 7, 3
    ws = (r.standard_normal((e_count, n, k)) * 0.02).astype(np.float32)
    qs, ss, bs = zip(*(o.quantize(ws[e], 4) for e in range(e_count)))
    words = np.stack([o.pack(q, 4) for q in qs])
    s = np.stack(ss)
    b = np.stack(bs)
    ids = np.stack([r.choice(e_count - 1, top_k, replace=False) for _ in range(t)]).astype(np.int32)
    x = r.standard_normal((t, k)).astype(np.float16)
    h = r.standard_normal((t * top_k, k)).astype(np.float16)
    yx = o.grouped_f64(words, s, b, x, ids, 4, a_row_per_pair=False)
    yh = o.grouped_f64(words, s, b, h, ids, 4, a_row_per_pair=True)
    assert yx.shape == (t * top_k, n) and yh.shape == (t * top_k, n)
    for p in range(t * top_k):
        e = ids.flat[p]
        want_x = o.qmatmul_f64(words[e], s[e], b[e], x[p // top_k:p // top_k + 1], 4)[0]
        want_h = o.qmatmul_f64(words[e], s[e], b[e], h[p:p + 1], 4)[0]
        assert np.array_equal(yx[p], want_x), p
        assert np.array_equal(yh[p], want_h), p
    one = np.zeros((t, 1), dtype=np.int32) + 2
    y1 = o.grouped_f64(words, s, b, x, one, 4, a_row_per_pair=False)
    assert np.array_equal(y1, o.qmatmul_f64(words[2], s[2], b[2], x, 4))
    empty = o.grouped_f64(words, s, b, x[:0], ids[:0], 4, a_row_per_pair=False)
    assert empty.shape == (0, n)


def check_route(o, seed=8):
    """Routing: ids are the top-k logits (softmax is monotone) as found by a
    plain sort of the logits, distinct, probabilities descending; weights
    sum to one and their ratios are exp(logit differences)."""
    r = np.random.default_rng(seed)
    logits = r.standard_normal((64, 16))
    logits[0, 3] = logits[0, 5]          # an exact tie: lower index first
    ids, wts = o.route(logits, 4)
    assert ids.dtype == np.int32 and ids.shape == (64, 4)
    assert np.array_equal(ids, synth.topk_ids(logits, 4))
    for i in range(64):
        assert len(set(ids[i])) == 4
        assert np.all(np.diff(wts[i]) <= 0)
        assert abs(wts[i].sum() - 1) < 1e-12
        ratio = wts[i, 1:] / wts[i, 0]
        assert np.allclose(ratio, np.exp(logits[i, ids[i, 1:]] - logits[i, ids[i, 0]]), rtol=1e-12)


def check_group_sizes(o, seed=9):
    """Groups of 32 and 128 codes.
    * Per-group error bound (as check_quantize_error_bound) on rows whose
      32-code slices have ranges a thousand times apart, so quantizing with
      any other grouping breaks the bound on the narrow slices.
    * Equivalence: when both halves of every 2*gs-code span share their min
      and max, groups of gs and of 2*gs give the same codes, and the finer
      scales and biases are the coarser ones repeated; the products agree.
    * The matmul with groups of 32 equals the one with groups of 64 when the
      two halves of each 64-group carry the same scale and bias."""
    r = np.random.default_rng(seed)
    for gs in (32, 128):
        for bits in (2, 3, 4, 5, 6, 8):
            levels = (1 << bits) - 1
            w = (r.standard_normal((8, 256)) * 0.02).astype(np.float32)
            w[:, 32:64] *= 1000.0  # slices of very different range
            w[:, 160:192] *= 1000.0
            q, s, b = o.quantize(w, bits, gs)
            assert s.shape == (8, 256 // gs) and q.max() <= levels
            w_hat = o.dequant_f64(q, s, b, gs)
            wg = w.astype(np.float64).reshape(8, 256 // gs, gs)
            mn, mx = wg.min(axis=2), wg.max(axis=2)
            sv, bv = o.f16_value(s), o.f16_value(b)
            bound = sv / 2 + np.abs(bv - mn) + levels * np.abs(sv - (mx - mn) / levels) \
                + 2.0 ** -20 * (np.abs(mn) + np.abs(mx))
            err = np.abs(w_hat - w.astype(np.float64)).reshape(8, 256 // gs, gs).max(axis=2)
            assert np.all(err <= bound), (gs, bits)
    for fine, coarse in ((32, 64), (64, 128)):
        for bits in (3, 4, 8):
            w = (r.standard_normal((4, 256)) * 0.02).astype(np.float32)
            wc = w.reshape(4, 256 // coarse, 2, fine)
            lo = np.minimum(wc[:, :, 0].min(axis=2), wc[:, :, 1].min(axis=2))
            hi = np.maximum(wc[:, :, 0].max(axis=2), wc[:, :, 1].max(axis=2))
            for half in (0, 1):  # both halves hold the span's min at 0 and max at 1
                wc[:, :, half, 0] = lo
                wc[:, :, half, 1] = hi
            w = wc.reshape(4, 256)
            qf, sf, bf = o.quantize(w, bits, fine)
            qc, sc, bc = o.quantize(w, bits, coarse)
            assert np.array_equal(qf, qc), (fine, bits)
            assert np.array_equal(sf, np.repeat(sc, 2, axis=1)) and np.array_equal(bf, np.repeat(bc, 2, axis=1))
            x = r.standard_normal((3, 256)).astype(np.float16)
            yf = o.qmatmul_f64(o.pack(qf, bits), sf, bf, x, bits, fine)
            yc = o.qmatmul_f64(o.pack(qc, bits), sc, bc, x, bits, coarse)
            assert np.array_equal(yf, yc), (fine, bits)


def check_fp16_weights(o, seed=10):
    """Unquantized fp16 weights: an identity weight returns x exactly; unit
    scale, zero bias and integer codes (exact in fp16) give the same product
    through the quantized path and through the fp16-weight path; a weight
    matrix with one nonzero column picks that column of x times the weight."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((3, 64)).astype(np.float16)
    eye = np.eye(64, dtype=np.float16).view(np.uint16)
    assert np.array_equal(o.hmatmul_f64(eye, x), x.astype(np.float64))
    for bits in (2, 4, 8):
        codes = r.integers(0, 1 << bits, (5, 128), dtype=np.uint8)
        s = np.full((5, 2), 0x3C00, dtype=np.uint16)
        b = np.zeros((5, 2), dtype=np.uint16)
        xx = r.standard_normal((2, 128)).astype(np.float16)
        yq = o.qmatmul_f64(o.pack(codes, bits), s, b, xx, bits)
        yh = o.hmatmul_f64(codes.astype(np.float16).view(np.uint16), xx)
        assert np.array_equal(yq, yh), bits
    w = np.zeros((4, 64), dtype=np.float16)
    w[2, 17] = np.float16(-0.375)
    y = o.hmatmul_f64(w.view(np.uint16), x)
    assert np.array_equal(y[:, 2], -0.375 * x[:, 17].astype(np.float64))
    assert not y[:, [0, 1, 3]].any()


def check_moe_ffn(o, seed=11):
    """SwiGLU and the weighted combine.
    * silu: silu(0) = 0; silu(1) = 1/(1 + e^-1) = 0.7310585786300049 (the
      textbook logistic value); silu(x) - silu(-x) = x; silu(40) = 40 and
      silu(-40) = -40 e^-40 to double precision.
    * one-hot activation (x = e_j): g and u are column j of the expert's
      dequantized gate and up weights, so h = silu(W_g[:, j]) * W_u[:, j].
    * combine: one-hot routing weights pick one pair row; weights summing to
      one over identical rows return that row; the slot order matters."""
    assert o.silu_f64(0.0) == 0.0
    assert abs(o.silu_f64(1.0) - 0.7310585786300049) < 1e-15
    xs = np.linspace(-6, 6, 25)
    assert np.allclose(o.silu_f64(xs) - o.silu_f64(-xs), xs, rtol=0, atol=1e-14)
    assert abs(o.silu_f64(40.0) - 40.0) < 1e-12 and abs(o.silu_f64(-40.0) + 40.0 * np.exp(-40.0)) < 1e-28
    r = np.random.default_rng(seed)
    e, n, k, t, top_k = 3, 5, 64, 4, 2
    ids = np.array([[0, 2], [1, 0], [2, 1], [0, 1]], dtype=np.int32)
    mats = []
    for which in range(2):
        ws = [o.quantize((r.standard_normal((n, k)) * 0.5).astype(np.float32), 4) for _ in range(e)]
        mats.append((np.stack([o.pack(q, 4) for q, _, _ in ws]), np.stack([s_ for _, s_, _ in ws]),
                     np.stack([b_ for _, _, b_ in ws]), [o.dequant_f64(q, s_, b_) for q, s_, b_ in ws]))
    for j in (0, 17, 63):
        x = np.zeros((t, k), dtype=np.float16)
        x[:, j] = 1.0
        h = o.moe_swiglu_f64(mats[0][:3], mats[1][:3], x, ids, 4)
        for p_ in range(t * top_k):
            ex = ids.reshape(-1)[p_]
            g = mats[0][3][ex][:, j]
            u = mats[1][3][ex][:, j]
            assert np.allclose(h[p_], g / (1 + np.exp(-g)) * u, rtol=1e-15, atol=0)
    yp = r.standard_normal((t * top_k, 7))
    w1 = np.zeros((t, top_k)); w1[:, 1] = 1.0
    assert np.array_equal(o.moe_combine_f64(yp, w1), yp[1::top_k])
    same = np.repeat(r.standard_normal((t, 1, 7)), top_k, axis=1).reshape(t * top_k, 7)
    assert np.allclose(o.moe_combine_f64(same, np.full((t, top_k), 1.0 / top_k)), same[::top_k], rtol=1e-15)


def check_bf16_to_f16(o):
    """bf16 -> fp16 conversion of weights: hand-worked patterns (1.0, -2.0,
    0.125, 65280 = largest bf16 below fp16's max, 65536 -> inf, NaN), the
    two subnormal rounding cases at 2^-25 (a tie, to even: 0) and 1.5 * 2^-25
    (up to the smallest subnormal 2^-24), and exactness of every bf16 whose
    magnitude lies in fp16's normal range."""
    cases = {0x3F80: 0x3C00, 0xC000: 0xC000, 0x3E00: 0x3000, 0x477F: 0x7BF8, 0x4780: 0x7C00,
             0xC780: 0xFC00, 0x3300: 0x0000, 0x3340: 0x0001, 0x0000: 0x0000, 0x8000: 0x8000}
    got = o.bf16_to_f16_bits(np.array(list(cases), dtype=np.uint16))
    assert [int(v) for v in got] == list(cases.values()), [hex(v) for v in got]
    nan = int(o.bf16_to_f16_bits(np.array([0x7FC0], dtype=np.uint16))[0])
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x03FF) != 0
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # NaN patterns
        val = (allb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    normal = np.isfinite(val) & (np.abs(val) >= 2.0 ** -14) & (np.abs(val) <= 65504.0)
    out = o.f16_value(o.bf16_to_f16_bits(allb[normal]))
    assert np.array_equal(out, val[normal])


ALL_CHECKS = (
    check_f16_rounding, check_pack_golden, check_pack_roundtrip,
    check_quantize_golden, check_quantize_nearest_level, check_quantize_error_bound,
    check_dot_exact_rational, check_closed_forms, check_gemm_rows_are_gemvs,
    check_grouped, check_route, check_group_sizes, check_fp16_weights, check_moe_ffn,
    check_bf16_to_f16,
)
