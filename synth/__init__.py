"""Seeded synthetic inputs for the weight-quantized GEMV/GEMM workloads.

This module is shared by the tests, the benchmark and the oracle-side
fixtures.  It draws random tensors and lists workload shapes; it holds none
of the quantized-matmul arithmetic (no quantizer, no packing, no dequant,
no dot products).  Every draw is keyed by a tuple of small integers so that
any tensor can be regenerated on its own:

    key = (workload_id, layer, projection_index, stream)

with stream 0 = weights, 1 = activations, 2 = router logits.

The shapes are those of the models the BaseRT paper (native-Metal LLM
inference on Apple Silicon, Fig. 1 and §4.1) and the MetalRT article (§2.1)
evaluate: Qwen3-0.6B, Llama-3.2-3B and Qwen3-4B as dense decoders and
Qwen3-30B-A3B as the mixture-of-experts model.  Trained weights are not
available, so weights are drawn N(0, 0.02) and activations N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

STREAM_W = 0
STREAM_X = 1
STREAM_LOGITS = 2

WEIGHT_STD = 0.02


def rng(*key: int) -> np.random.Generator:
    """A numpy Generator seeded by a tuple of non-negative integers."""
    return np.random.default_rng([int(k) for k in key])


def draw_weight(key, n: int, k: int) -> np.ndarray:
    """Dense weight W[n, k] (out x in), float32, N(0, 0.02)."""
    w = rng(*key).standard_normal((n, k), dtype=np.float32)
    w *= np.float32(WEIGHT_STD)
    return w


def draw_act(key, m: int, k: int) -> np.ndarray:
    """Activations x[m, k] as float16: float32 N(0, 1) cast to fp16."""
    return rng(*key).standard_normal((m, k), dtype=np.float32).astype(np.float16)


def draw_logits(key, m: int, e: int) -> np.ndarray:
    """Router logits [m, e], float64 N(0, 1)."""
    return rng(*key).standard_normal((m, e))


def topk_ids(logits: np.ndarray, k: int) -> np.ndarray:
    """Expert ids of the k largest logits per row, largest first, ties to
    the lower index.  Softmax is strictly increasing, so these are also the
    top-k experts by routing probability.  Returns int32 [m, k]."""
    order = np.argsort(-logits, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :k].astype(np.int32))


# ---------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Proj:
    name: str
    k: int  # input features
    n: int  # output features


@dataclass(frozen=True)
class DenseWorkload:
    wid: int                 # key prefix for every draw of this workload
    name: str
    bits: int
    layers: int
    projs: tuple             # tuple[Proj, ...] repeated per layer
    extra: tuple = ()        # projections applied once (e.g. lm_head)
    ms: tuple = (1,)         # activation rows (1 = decode)
    group_size: int = 64

    def problems(self):
        """(layer, proj_index, Proj) for every matmul of one pass; extra
        projections get layer = self.layers."""
        out = []
        for layer in range(self.layers):
            for i, p in enumerate(self.projs):
                out.append((layer, i, p))
        for i, p in enumerate(self.extra):
            out.append((self.layers, len(self.projs) + i, p))
        return out

    def weight_count(self) -> int:
        return sum(p.k * p.n for _, _, p in self.problems())


@dataclass(frozen=True)
class MoEWorkload:
    wid: int
    name: str
    bits: int
    hidden: int
    inter: int
    experts: int
    top_k: int
    ms: tuple
    group_size: int = 64


SINGLE_Q4 = DenseWorkload(
    wid=1, name="q4-gemv-1x1024x1024", bits=4, layers=1,
    projs=(Proj("w", 1024, 1024),))

QWEN3_0_6B_Q4_DECODE = DenseWorkload(
    wid=2, name="qwen3-0.6b-q4-decode", bits=4, layers=28,
    projs=(Proj("q", 1024, 2048), Proj("k", 1024, 1024), Proj("v", 1024, 1024),
           Proj("o", 2048, 1024), Proj("gate", 1024, 3072), Proj("up", 1024, 3072),
           Proj("down", 3072, 1024)),
    extra=(Proj("lm_head", 1024, 151936),))

LLAMA32_3B_Q8_DECODE = DenseWorkload(
    wid=3, name="llama-3.2-3b-q8-decode", bits=8, layers=28,
    projs=(Proj("q", 3072, 3072), Proj("k", 3072, 1024), Proj("v", 3072, 1024),
           Proj("o", 3072, 3072), Proj("gate", 3072, 8192), Proj("up", 3072, 8192),
           Proj("down", 8192, 3072)))

QWEN3_4B_Q4_PREFILL = DenseWorkload(
    wid=4, name="qwen3-4b-q4-prefill", bits=4, layers=36,
    projs=(Proj("q", 2560, 4096), Proj("k", 2560, 1024), Proj("v", 2560, 1024),
           Proj("o", 4096, 2560), Proj("gate", 2560, 9728), Proj("up", 2560, 9728),
           Proj("down", 9728, 2560)),
    ms=(128, 256, 512, 1024, 2048))

QWEN3_30B_A3B_Q4_MOE = MoEWorkload(
    wid=5, name="qwen3-30b-a3b-q4-moe-prefill", bits=4, hidden=2048, inter=768,
    experts=128, top_k=8, ms=(512, 2048))

ALL = (SINGLE_Q4, QWEN3_0_6B_Q4_DECODE, LLAMA32_3B_Q8_DECODE,
       QWEN3_4B_Q4_PREFILL, QWEN3_30B_A3B_Q4_MOE)


def moe_projs(w: MoEWorkload):
    """The three grouped matmuls of one MoE FFN block: gate and up read the
    token row (pair // top_k), down reads the pair's own row."""
    return (("gate", w.hidden, w.inter, 0), ("up", w.hidden, w.inter, 0),
            ("down", w.inter, w.hidden, 1))


def draw_moe_inputs(w: MoEWorkload, m: int, proj_index: int):
    """(A, ids) for one grouped matmul at m tokens.  A is fp16 x[m, hidden]
    for gate/up and fp16 h[m*top_k, inter] for down; ids int32 [m, top_k]
    come from N(0, 1) logits (one draw per m, shared by the three)."""
    name, k, n, per_pair = moe_projs(w)[proj_index]
    logits = draw_logits((w.wid, m, 0, STREAM_LOGITS), m, w.experts)
    ids = topk_ids(logits, w.top_k)
    rows = m * w.top_k if per_pair else m
    a = draw_act((w.wid, m, proj_index, STREAM_X), rows, k)
    return a, ids, logits


def draw_expert_weights(w: MoEWorkload, proj_index: int, experts=None):
    """Dense fp32 weights [E, n, k] of one grouped projection, drawn per
    expert with key (wid, expert, proj_index, STREAM_W)."""
    _, k, n, _ = moe_projs(w)[proj_index]
    es = range(w.experts) if experts is None else experts
    return np.stack([draw_weight((w.wid, e, proj_index, STREAM_W), n, k) for e in es])
