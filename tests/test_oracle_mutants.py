"""Each pin set must catch a planted mistake.

A fresh copy of the oracle module gets one function replaced by a
plausible wrong version (a dropped term, a wrong index, a wrong rounding,
a transposed operand ...); running every pin against that copy must fail.
The real oracle is never modified."""
import importlib.util
import os

import numpy as np
import pytest

import pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "qmm_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("oracle_mutant_copy", ORACLE_SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def m_dequant_no_bias(o):
    def dequant_f64(codes, s_bits, b_bits, group_size=64):
        s = np.repeat(o.f16_value(s_bits), group_size, axis=-1)
        return s * np.asarray(codes).astype(np.float64)
    o.dequant_f64 = dequant_f64


def m_dequant_wrong_group(o):
    def dequant_f64(codes, s_bits, b_bits, group_size=64):
        reps = np.asarray(codes).shape[-1] // np.asarray(s_bits).shape[-1]
        s = np.tile(o.f16_value(s_bits), reps)
        b = np.tile(o.f16_value(b_bits), reps)
        return s * np.asarray(codes).astype(np.float64) + b
    o.dequant_f64 = dequant_f64


def m_quantize_ignores_group_size(o):
    real_quant = o.quantize

    def quantize(w, bits, group_size=64):
        q, s, b = real_quant(w, bits, 64)   # always groups of 64
        f = 64 // group_size if group_size < 64 else 1
        c = group_size // 64 if group_size > 64 else 1
        return q, np.repeat(s, f, axis=1)[:, ::c], np.repeat(b, f, axis=1)[:, ::c]
    o.quantize = quantize


def m_silu_is_sigmoid(o):
    o.silu_f64 = lambda g: 1.0 / (1.0 + np.exp(-np.asarray(g, dtype=np.float64)))


def m_combine_slots_reversed(o):
    real = o.moe_combine_f64
    o.moe_combine_f64 = lambda y_pairs, weights: real(y_pairs, np.asarray(weights)[:, ::-1])


def m_pack_high_first(o):
    real_pack, real_unpack = o.pack, o.unpack

    def rev(c, bits):
        c = np.asarray(c, dtype=np.uint8)
        out = np.zeros_like(c)
        for j in range(bits):
            out |= ((c >> j) & 1) << (bits - 1 - j)
        return out
    o.pack = lambda codes, bits: real_pack(rev(codes, bits), bits)
    o.unpack = lambda words, bits, k: rev(real_unpack(words, bits, k), bits)


def m_unpack_skips_word(o):
    real_unpack = o.unpack

    def unpack(words, bits, k):
        w = np.asarray(words).copy()
        if w.shape[-1] > 1:
            w[..., 1] = w[..., 0]
        return real_unpack(w, bits, k)
    o.unpack = unpack


def _patch_quantize(o, fn):
    o.quantize = fn


def m_quantize_floor(o):
    real = o.np

    class NP:
        def __getattr__(self, name):
            return getattr(real, name)
        rint = staticmethod(real.floor)
    o.np = NP()


def m_quantize_ties_up(o):
    real = o.np

    class NP:
        def __getattr__(self, name):
            return getattr(real, name)

        @staticmethod
        def rint(t):
            return real.floor(t + real.float32(0.5))
    o.np = NP()


def m_quantize_bias_max(o):
    real_quant = o.quantize

    def quantize(w, bits, group_size=64):
        w = np.asarray(w, dtype=np.float32)
        return real_quant(-w, bits, group_size)[0], *real_quant(w, bits, group_size)[1:]
    o.quantize = quantize


def m_quantize_unrounded_scale(o):
    def quantize(w, bits, group_size=64):
        w = np.asarray(w, dtype=np.float32)
        n, k = w.shape
        levels = np.float32(2 ** bits - 1)
        wg = w.reshape(n, k // group_size, group_size)
        mn, mx = wg.min(axis=2), wg.max(axis=2)
        s32 = (mx - mn) / levels
        s16, b16 = s32.astype(np.float16), mn.astype(np.float16)
        with np.errstate(divide="ignore", invalid="ignore"):
            t = (wg - b16.astype(np.float32)[:, :, None]) / np.where(s32 == 0, 1, s32)[:, :, None]
        q = np.clip(np.rint(t), 0, levels).astype(np.uint8).reshape(n, k)
        return q, s16.view(np.uint16), b16.view(np.uint16)
    o.quantize = quantize


def m_quantize_no_clamp(o):
    real = o.np

    class NP:
        def __getattr__(self, name):
            return getattr(real, name)

        @staticmethod
        def clip(a, lo, hi):
            return real.mod(a, hi + 1)
    o.np = NP()


def m_quantize_levels_off_by_one(o):
    real_quant = o.quantize

    def quantize(w, bits, group_size=64):
        w = np.asarray(w, dtype=np.float32)
        q, s, b = real_quant(w, bits, group_size)
        s2 = (o.f16_value(s) * (2 ** bits - 1) / (2 ** bits)).astype(np.float16).view(np.uint16)
        return q, s2, b
    o.quantize = quantize


def m_matmul_transposed(o):
    def matmul_f64(x16, w_hat64):
        x = np.asarray(x16, dtype=np.float16).astype(np.float64)
        w = np.asarray(w_hat64, dtype=np.float64)
        return (w[:, :x.shape[0]].T @ (x @ w.T)[:, :]) if w.shape[0] != x.shape[0] else x @ w
    o.matmul_f64 = matmul_f64


def m_matmul_f32(o):
    def matmul_f64(x16, w_hat64):
        x = np.asarray(x16, dtype=np.float16).astype(np.float32)
        return (x @ np.asarray(w_hat64, dtype=np.float32).T).astype(np.float64)
    o.matmul_f64 = matmul_f64


def m_grouped_wrong_row(o):
    real = o.grouped_f64

    def grouped_f64(words, s_bits, b_bits, a16, ids, bits, a_row_per_pair, group_size=64):
        if not a_row_per_pair:
            a16 = np.repeat(np.asarray(a16), np.asarray(ids).shape[1], axis=0)
            return real(words, s_bits, b_bits, a16[::-1].copy(), ids, bits, True, group_size)
        return real(words, s_bits, b_bits, a16, ids, bits, a_row_per_pair, group_size)
    o.grouped_f64 = grouped_f64


def m_grouped_expert_off_by_one(o):
    real = o.grouped_f64

    def grouped_f64(words, s_bits, b_bits, a16, ids, bits, a_row_per_pair, group_size=64):
        return real(words, s_bits, b_bits, a16, (np.asarray(ids) + 1) % words.shape[0],
                    bits, a_row_per_pair, group_size)
    o.grouped_f64 = grouped_f64


def m_route_no_renorm(o):
    real = o.route

    def route(logits, top_k):
        ids, w = real(logits, top_k)
        z = np.exp(logits - logits.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        return ids, np.take_along_axis(p, ids.astype(np.int64), axis=1)
    o.route = route


def m_route_ascending(o):
    real = o.route

    def route(logits, top_k):
        ids, w = real(-np.asarray(logits), top_k)
        return ids, w
    o.route = route


def m_f16_double_rounding(o):
    o.round_to_f16_bits = lambda a: np.asarray(a, dtype=np.float64).astype(np.float32).astype(
        np.float16).view(np.uint16)


def m_f16_truncate(o):
    def f16_bits(a):
        a32 = np.asarray(a, dtype=np.float32)
        bits = a32.view(np.uint32)
        trunc = (bits & np.uint32(0xFFFFE000)).view(np.float32)
        return trunc.astype(np.float16).view(np.uint16)
    o.f16_bits = f16_bits
    o.round_to_f16_bits = lambda a: f16_bits(np.asarray(a, dtype=np.float64).astype(np.float32))


MUTANTS = [
    m_dequant_no_bias, m_dequant_wrong_group, m_pack_high_first, m_unpack_skips_word,
    m_quantize_floor, m_quantize_ties_up, m_quantize_bias_max, m_quantize_unrounded_scale,
    m_quantize_no_clamp, m_quantize_levels_off_by_one, m_matmul_transposed, m_matmul_f32,
    m_grouped_wrong_row, m_grouped_expert_off_by_one, m_route_no_renorm, m_route_ascending,
    m_f16_double_rounding, m_f16_truncate, m_quantize_ignores_group_size, m_silu_is_sigmoid,
    m_combine_slots_reversed,
]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda m: m.__name__)
def test_pins_catch_mutant(mutate):
    o = fresh_oracle()
    mutate(o)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(o)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(exc).__name__))
    assert caught, f"no pin caught {mutate.__name__}"
