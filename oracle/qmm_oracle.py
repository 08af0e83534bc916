"""Plain, slow, obviously-correct float64 oracle (numpy).

Test infrastructure only; see the package docstring for what it follows and
what pins it.  Conventions used throughout:

* A dense weight is W[n, k] (out x in, row-major); y = x @ W_hat.T.
* fp16 scale/bias arrays are carried as their uint16 bit patterns, shape
  [n, k // group_size], so that "bit-exact" comparisons are comparisons of
  integers.
* Codes are uint8 [n, k] in 0 .. 2**bits - 1.
* Packed words are uint32 [n, k * bits // 32]: a little-endian bit stream
  along k in which code k occupies bits [bits*k, bits*k + bits).
"""
from __future__ import annotations

import numpy as np

SUPPORTED_BITS = (2, 3, 4, 5, 6, 8)


# ------------------------------------------------------------------ fp16 --

def f16_bits(a) -> np.ndarray:
    """Round float32/float64 values to fp16 (IEEE round-to-nearest-even, via
    numpy's direct conversion) and return the uint16 bit patterns."""
    return np.asarray(a).astype(np.float16).view(np.uint16)


def f16_value(bits) -> np.ndarray:
    """fp16 bit patterns -> their exact values as float64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_to_f32(a64: np.ndarray) -> np.ndarray:
    """float64 -> float32, round-to-nearest-even (single rounding)."""
    return np.asarray(a64, dtype=np.float64).astype(np.float32)


def round_to_f16_bits(a64: np.ndarray) -> np.ndarray:
    """float64 -> fp16 bit patterns with ONE rounding (numpy converts
    float64 to float16 directly, not through float32)."""
    return np.asarray(a64, dtype=np.float64).astype(np.float16).view(np.uint16)


# ------------------------------------------------------------- quantizer --

def quantize(w, bits: int, group_size: int = 64):
    """Asymmetric min/max quantization per group of `group_size` along k.

    Steps for each row n and group g (k in [g*gs, (g+1)*gs)), L = 2**bits - 1,
    all arithmetic in IEEE float32:
      1. mn = min(w), mx = max(w) over the group;
      2. s32 = (mx - mn) / L            (true division);
      3. s = fp16(s32), b = fp16(mn)    (round-to-nearest-even);
      4. if s == 0 (constant group, or s32 underflows fp16) every code is 0;
      5. else q = clamp(rint((w - b) / s), 0, L), where rint rounds half to
         even and (w - b) / s uses the stored fp16 s and b widened to fp32.
    Returns (codes uint8 [n, k], s_bits uint16 [n, G], b_bits uint16 [n, G]).
    """
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"bits must be one of {SUPPORTED_BITS}")
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [n, k]")
    n, k = w.shape
    if k % group_size != 0:
        raise ValueError("k must be a multiple of group_size")
    if not np.all(np.isfinite(w)):
        raise ValueError("w must be finite")
    levels = np.float32(2 ** bits - 1)
    wg = w.reshape(n, k // group_size, group_size)
    mn = wg.min(axis=2)
    mx = wg.max(axis=2)
    s32 = (mx - mn) / levels
    s16 = s32.astype(np.float16)
    b16 = mn.astype(np.float16)
    if not (np.all(np.isfinite(s16)) and np.all(np.isfinite(b16))):
        raise ValueError("group range does not fit fp16 scale/bias")
    s = s16.astype(np.float32)[:, :, None]
    b = b16.astype(np.float32)[:, :, None]
    zero = s == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (wg - b) / np.where(zero, np.float32(1), s)
    q = np.clip(np.rint(t), 0, levels)
    q = np.where(zero, np.float32(0), q)
    codes = q.astype(np.uint8).reshape(n, k)
    return codes, s16.view(np.uint16), b16.view(np.uint16)


# --------------------------------------------------------------- packing --

def packed_words_per_row(k: int, bits: int) -> int:
    if (k * bits) % 32 != 0:
        raise ValueError("k * bits must be a multiple of 32")
    return k * bits // 32


def pack(codes, bits: int) -> np.ndarray:
    """Codes uint8 [..., k] -> uint32 [..., k*bits/32].

    Writes each code's `bits` low bits, least significant first, into a
    little-endian bit stream (bit j of code k -> stream bit bits*k + j;
    stream bit i -> bit i % 32 of word i // 32)."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.size and codes.max() >= (1 << bits):
        raise ValueError("code out of range")
    *lead, k = codes.shape
    wpr = packed_words_per_row(k, bits)
    shifts = np.arange(bits, dtype=np.uint8)
    stream = ((codes[..., :, None] >> shifts) & 1).astype(np.uint8)   # [..., k, bits]
    stream = stream.reshape(*lead, k * bits)
    as_bytes = np.packbits(stream, axis=-1, bitorder="little")         # [..., k*bits/8]
    return np.ascontiguousarray(as_bytes).view("<u4").reshape(*lead, wpr).astype(np.uint32)


def unpack(words, bits: int, k: int) -> np.ndarray:
    """Inverse of `pack`: uint32 [..., k*bits/32] -> codes uint8 [..., k]."""
    words = np.ascontiguousarray(np.asarray(words, dtype="<u4"))
    *lead, wpr = words.shape
    if wpr != packed_words_per_row(k, bits):
        raise ValueError("word count does not match k and bits")
    stream = np.unpackbits(words.view(np.uint8), axis=-1, bitorder="little")
    stream = stream.reshape(*lead, k, bits).astype(np.uint16)
    weights = (1 << np.arange(bits, dtype=np.uint16))
    return (stream * weights).sum(axis=-1).astype(np.uint8)


# ---------------------------------------------------------------- dequant --

def dequant_f64(codes, s_bits, b_bits, group_size: int = 64) -> np.ndarray:
    """W_hat[n, k] = s[n, k // gs] * q[n, k] + b[n, k // gs] in float64.

    This is exact: s and b are fp16 (11 significant bits, multiples of
    2**-24), q has at most 8 bits, so s*q needs at most 19 significant bits
    and the sum at most 49, inside float64's 53."""
    q = np.asarray(codes).astype(np.float64)
    s = np.repeat(f16_value(s_bits), group_size, axis=-1)
    b = np.repeat(f16_value(b_bits), group_size, axis=-1)
    return s * q + b


# ---------------------------------------------------------------- matmul --

def matmul_f64(x16, w_hat64) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * W_hat[n, k] in float64 (x given as fp16)."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    return x @ np.asarray(w_hat64, dtype=np.float64).T


def qmatmul_f64(words, s_bits, b_bits, x16, bits: int, group_size: int = 64):
    """Reference quantized matmul: unpack -> dequantize (fp64) -> matmul.
    GEMV is the m = 1 case."""
    x16 = np.atleast_2d(np.asarray(x16, dtype=np.float16))
    k = x16.shape[1]
    w_hat = dequant_f64(unpack(words, bits, k), s_bits, b_bits, group_size)
    return matmul_f64(x16, w_hat)


def bf16_to_f16_bits(b_bits) -> np.ndarray:
    """bf16 bit patterns -> fp16 bit patterns of the same value, rounded to
    nearest even (the bf16 value is exact in float32; numpy converts float32
    to float16 with one rounding).  Beyond fp16's range: +-inf; NaN stays NaN."""
    f32 = (np.asarray(b_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    with np.errstate(over="ignore"):
        return f32.astype(np.float16).view(np.uint16)


def hmatmul_f64(w_bits, x16) -> np.ndarray:
    """Unquantized fp16 weights (the 16-bit format next to Q2..Q8): y[m, n] =
    sum_k x[m, k] * W[n, k] with W given as fp16 bit patterns [n, k], each
    taken at its exact value."""
    return matmul_f64(np.atleast_2d(np.asarray(x16, dtype=np.float16)), f16_value(w_bits))


def grouped_f64(words, s_bits, b_bits, a16, ids, bits: int, a_row_per_pair: bool,
                group_size: int = 64) -> np.ndarray:
    """Mixture-of-experts grouped matmul.

    ids[t, j] (int, [T, top_k]) names the expert of pair p = t*top_k + j.
    The A row of pair p is a16[p // top_k] (token rows, a16 [T, k]) or, with
    a_row_per_pair, a16[p] (a16 [T*top_k, k]).  Output row p is
        y[p, n] = sum_k A[row(p), k] * W_hat[ids.flat[p], n, k]
    for the expert's own weights words[e], s_bits[e], b_bits[e]."""
    ids = np.asarray(ids)
    t, top_k = ids.shape
    a16 = np.asarray(a16, dtype=np.float16)
    k = a16.shape[1]
    e_count, n = words.shape[0], words.shape[1]
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= e_count):
        raise ValueError("expert id out of range")
    y = np.zeros((t * top_k, n), dtype=np.float64)
    for e in np.unique(flat):
        pairs = np.nonzero(flat == e)[0]
        rows = pairs if a_row_per_pair else pairs // top_k
        w_hat = dequant_f64(unpack(words[e], bits, k), s_bits[e], b_bits[e], group_size)
        y[pairs] = matmul_f64(a16[rows], w_hat)
    return y


# ------------------------------------------------------- MoE FFN block --

def silu_f64(g) -> np.ndarray:
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g)), in float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def moe_swiglu_f64(gate, up, x16, ids, bits: int, group_size: int = 64) -> np.ndarray:
    """SwiGLU input of the down projection, per pair p (token row p // top_k):
        h[p, c] = silu(g[p, c]) * u[p, c]
    where g and u are the grouped products of the token row with the pair's
    expert's gate and up weights (each given as (words, s_bits, b_bits))."""
    g = grouped_f64(*gate, x16, ids, bits, False, group_size)
    u = grouped_f64(*up, x16, ids, bits, False, group_size)
    return silu_f64(g) * u


def moe_combine_f64(y_pairs, weights) -> np.ndarray:
    """y[t, c] = sum_j weights[t, j] * y_pairs[t * top_k + j, c] in float64."""
    w = np.asarray(weights, dtype=np.float64)
    t, top_k = w.shape
    yp = np.asarray(y_pairs, dtype=np.float64).reshape(t, top_k, -1)
    return np.einsum("tj,tjc->tc", w, yp)


# --------------------------------------------------------------- routing --

def route(logits, top_k: int):
    """Router of the MoE workload: softmax over experts (float64, max
    subtracted), the top_k experts by probability in descending order with
    ties to the lower index, and their probabilities renormalised to sum to
    one.  Returns (ids int32 [T, top_k], weights float64 [T, top_k])."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    t, e = p.shape
    ids = np.empty((t, top_k), dtype=np.int32)
    wts = np.empty((t, top_k), dtype=np.float64)
    for i in range(t):
        chosen = sorted(range(e), key=lambda j: (-p[i, j], j))[:top_k]
        ids[i] = chosen
        wts[i] = p[i, chosen] / p[i, chosen].sum()
    return ids, wts
