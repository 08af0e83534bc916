#!/usr/bin/env python3
"""Throughput of the weight-quantized matmul hot path on one MI355X.

One step = one decode pass of a Qwen3-0.6B-shaped model with 4-bit weights:
the 197 GEMVs of 28 layers (q 1024->2048, k/v 1024->1024, o 2048->1024,
gate/up 1024->3072, down 3072->1024) plus the lm_head (1024->151936), all in
ONE batched qmm_qgemv_batched launch.  `value` is algorithmic bytes moved
per step (packed codes + fp16 scales/biases + fp16 x + fp32 y, each once)
divided by the step time, in GB/s, with every input resident in HBM.  Two
full copies of the weights alternate between steps, so a step never finds
its weights in the 256 MB last-level cache.

The same JSON line carries, measured in the same run:
  roofline      the batched GEMV kernel against the 8 TB/s HBM peak: the
                timed region between two HIP events on the launch stream,
                divided by the launches in it (one per step), plus the HBM
                traffic rocprofv3 counted for the same kernel;
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same
                workload, on this host's cores;
  prefill       Qwen3-4B-shaped 4-bit GEMMs (36 layers x 7 projections, run
                as 4 batched launches per layer: q+k+v, o, gate+up, down) at
                M = 128 ... 2048, TFLOP/s against the fp16 matrix-core peak;
  moe           Qwen3-30B-A3B-shaped grouped GEMMs (128 experts, top-8) at
                M = 512 and 2048 tokens (one routing pass shared by gate, up
                and down), against their HBM roofline;
  decode_context the lm_head alone, q/k/v as three launches vs one launch over
                the stacked weights, the decode pass as 197 sequential launches
                replayed as one HIP graph, and that graph's per-launch floor;
  decode_q8     the Llama-3.2-3B-shaped 8-bit decode sweep (196 GEMVs);
  decode_formats the Qwen3-0.6B-shaped decode pass with 2-, 3-, 5- and 6-bit
                and unquantized fp16 weights (one batched launch each);
  gemm_formats  one 2048 x 9728 x 2560 prefill GEMM per weight width (and fp16);
  single_gemv   one 1x1024x1024 4-bit GEMV launch (latency).
Inputs are seeded synthetic tensors with the models' shapes (weights
N(0, 0.02) quantized on the GPU by qmm_quantize, activations N(0, 1) fp16).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
FP16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense fp16 matrix cores (256 CU x 2.4 GHz x 4096 flop/clk)

METRIC = "Q4 decode GEMV HBM GB/s (% peak) + prefill qGEMM TFLOP/s (% MFMA peak)"

# HBM traffic of one batched-GEMV launch on the decode workload, from two
# rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) scaled by the same counters
# on a copy of known size; valid only for the kernel sources it was taken on.
TRAFFIC = {
    # rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE on `bench.py --only decode`
    # (KiB per dispatch of qgemv_batched_kernel<4,16,4,64>) and on
    # `bench.py --copy-calib` (a 1 GiB device copy: FETCH_SIZE reads 524,300
    # KiB for 1 GiB read, WRITE_SIZE 1,048,576 KiB for 1 GiB written).
    "fetch_kib": 166755.8, "fetch_scale": 1073741824 / (524301.3 * 1024),
    "write_kib": 1938.6, "write_scale": 1073741824 / (1048576.0 * 1024),
    "sources_sha256": "930899746c41ab2d2905f5f5fa9d8b2f56ec7e532b18d36df56b54d6a11fff14",
}


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for f in ("qgemv.hip", "qmm_api.hip", "qmm_device.h", "qmm_internal.h"):
        with open(os.path.join(ROOT, "quantized_matmul_qgemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ setup --

def prepare_dense(torch, qmm, w: synth.DenseWorkload, copies: int):
    """Quantize each distinct projection once on the GPU, then make `copies`
    x layers device copies.  Returns per copy a list of (W, S, B, X, Y, n, k)."""
    base = {}
    for i, p in enumerate(w.projs + w.extra):
        layer = w.layers if i >= len(w.projs) else 0
        wf = torch.from_numpy(synth.draw_weight((w.wid, layer, i, synth.STREAM_W), p.n, p.k)).cuda()
        if w.bits == 16:  # unquantized fp16 weights: no scales or biases
            words, s, b = wf.half().view(torch.int32), None, None
        else:
            words, s, b = qmm.quantize(wf, w.bits)
        del wf
        base[i] = (words, s, b)
    sets = []
    for c in range(copies):
        probs = []
        for layer, i, p in w.problems():
            words, s, b = base[i]
            if c > 0 or layer > 0 or (i >= len(w.projs)):
                words, s, b = (None if t is None else t.clone() for t in (words, s, b))
            x = torch.from_numpy(synth.draw_act((w.wid, layer, i, synth.STREAM_X), 1, p.k)[0]).cuda()
            y = torch.empty(p.n, dtype=torch.float32, device="cuda")
            probs.append((words, s, b, x, y, p.n, p.k))
        sets.append(probs)
    torch.cuda.synchronize()
    return sets


def gemv_bytes(n, k, bits):
    scales = 0 if bits == 16 else 2 * 2 * n * (k // 64)   # fp16 scale + bias per group of 64
    return n * k * bits // 8 + scales + 2 * k + 4 * n


# ------------------------------------------------------------- measuring --

def time_launches(torch, launch, steps, warmup, stream):
    """Warm up, then time `steps` back-to-back calls between one pair of HIP
    events recorded on the launch stream.  Returns (ms per call, wall s).
    (Events around every single launch would add their own overhead to a
    ~60 us kernel, so the per-launch time is the timed region / steps.)"""
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        launch(warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return t0.elapsed_time(t1) / steps, wall


def bench_decode(torch, qmm, wl, steps, warmup, copies=2):
    sets = prepare_dense(torch, qmm, wl, copies)
    plans = [qmm.qgemv_batched_plan([p[:5] for p in s], wl.bits) for s in sets]
    step_bytes = sum(gemv_bytes(p.n, p.k, wl.bits) for _, _, p in wl.problems())
    stream = torch.cuda.current_stream()
    ms_step, wall = time_launches(
        torch, lambda i: qmm.qgemv_batched(plans[i % copies]), steps, warmup, stream)
    return dict(sets=sets, plans=plans, step_bytes=step_bytes, ms_step=ms_step, wall=wall)


def bench_decode_formats(torch, qmm, wl, bits_list=(2, 3, 5, 6, 16), steps=20, warmup=3):
    """The same decode pass (one batched launch of all its GEMVs) with the
    weights quantized to other widths: streaming rate per format."""
    out = {}
    for bits in bits_list:
        w = dataclasses.replace(wl, bits=bits, name=f"{wl.name}@q{bits}")
        d = bench_decode(torch, qmm, w, steps, warmup)
        gbs = d["step_bytes"] / (d["ms_step"] * 1e-3) / 1e9
        out["f16" if bits == 16 else f"q{bits}"] = {"bytes_per_step": d["step_bytes"], "ms_per_step": round(d["ms_step"], 5),
                           "gb_per_s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del d
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def bench_gemm_formats(torch, qmm, m=2048, n=9728, k=2560, bits_list=(2, 3, 4, 5, 6, 8, 16),
                       steps=20, warmup=3):
    """One M x N x K prefill GEMM (the gate projection at M = 2048) per
    weight width, TFLOP/s against the fp16 matrix-core peak."""
    out = {}
    wf = torch.from_numpy(synth.draw_weight((9, m, n, k), n, k)).cuda()
    x = torch.from_numpy(synth.draw_act((9, m, n, k + 1), m, k)).cuda()
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for bits in bits_list:
        wq = (wf.half().view(torch.int32), None, None) if bits == 16 else qmm.quantize(wf, bits)
        wq = (qmm.repack_tiled(wq[0], bits), wq[1], wq[2])  # tile-interleaved copy, once
        ws = torch.empty(max(qmm.qgemm_workspace_size(m, n, k, bits), 16), dtype=torch.uint8, device="cuda")
        ms_call, _ = time_launches(torch, lambda i: qmm.qgemm(*wq, x, bits, y=y, workspace=ws, tiled=True),
                                   steps, warmup, stream)
        tfl = 2.0 * m * n * k / (ms_call * 1e-3) / 1e12
        out["f16" if bits == 16 else f"q{bits}"] = {"ms_per_call": round(ms_call, 4), "tflops": round(tfl, 1),
                           "frac_of_fp16_peak": round(tfl / FP16_MFMA_PEAK_TFLOPS, 4)}
        del wq, ws
    del wf, x, y
    torch.cuda.empty_cache()
    return out


def bench_single_gemv(torch, qmm, steps=200, warmup=20):
    wl = synth.SINGLE_Q4
    sets = prepare_dense(torch, qmm, wl, 1)
    words, s, b, x, y, n, k = sets[0][0]
    stream = torch.cuda.current_stream()
    ms, _ = time_launches(
        torch, lambda i: qmm.qgemv(words, s, b, x, wl.bits, y=y), steps, warmup, stream)
    return {"workload": wl.name, "us_per_launch": round(ms * 1e3, 2),
            "gb_per_s": round(gemv_bytes(n, k, 4) / (ms * 1e-3) / 1e9, 1)}


def bench_projections(torch, qmm, wl, sets, launches=20):
    """Each distinct projection of the decode pass (layer 0's q, k, v, o,
    gate, up, down and the lm_head) as `launches` back-to-back single GEMV
    launches, in that order (a kernel trace of this run gives each
    projection's kernel duration; the event time here includes the launch
    gaps, which dominate the small projections)."""
    stream = torch.cuda.current_stream()
    names = [p.name for p in wl.projs] + [p.name for p in wl.extra]
    picks = list(range(len(wl.projs))) + [len(sets[0]) - 1]
    out = {}
    for name, idx in zip(names, picks):
        words, s_, b_, x, y, n, k = sets[0][idx]
        ms, _ = time_launches(torch, lambda i: qmm.qgemv(words, s_, b_, x, wl.bits, y=y), launches, 3, stream)
        out[name] = {"n": n, "k": k, "us_per_launch": round(ms * 1e3, 2),
                     "gb_per_s": round(gemv_bytes(n, k, wl.bits) / (ms * 1e-3) / 1e9, 1)}
    return out


def bench_decode_extras(torch, qmm, wl, sets, steps=20, warmup=3):
    """Context for the batched headline, on the same weight copies:
      lm_head      the 1024 -> 151936 projection alone, one qmm_qgemv launch;
      graph_197    the decode pass as 197 sequential qmm_qgemv launches (the
                   order a dependent decode would need) replayed as one HIP graph;
      graph_floor  the same graph shape with 197 one-element kernels: the
                   per-launch floor that the sequential form pays."""
    stream = torch.cuda.current_stream()
    copies = len(sets)
    out = {}
    lm = [st[-1] for st in sets]
    ms, _ = time_launches(torch, lambda i: qmm.qgemv(*lm[i % copies][:4], wl.bits, y=lm[i % copies][4]),
                          steps, warmup, stream)
    nb = gemv_bytes(lm[0][5], lm[0][6], wl.bits)
    out["lm_head"] = {"n": lm[0][5], "k": lm[0][6], "us_per_launch": round(ms * 1e3, 2),
                      "gb_per_s": round(nb / (ms * 1e-3) / 1e9, 1)}
    # q, k, v of layer 0 (same activations): three launches vs one launch over
    # the weights stacked along n (2048 + 1024 + 1024 rows)
    q, kk, v = sets[0][0], sets[0][1], sets[0][2]
    ms3, _ = time_launches(torch, lambda i: [qmm.qgemv(*t[:4], wl.bits, y=t[4]) for t in (q, kk, v)],
                           steps, warmup, stream)
    cat = [torch.cat([t[j] for t in (q, kk, v)]) for j in range(3)]
    ycat = torch.empty(cat[0].shape[0], dtype=torch.float32, device="cuda")
    ms1, _ = time_launches(torch, lambda i: qmm.qgemv(*cat, q[3], wl.bits, y=ycat), steps, warmup, stream)
    out["qkv"] = {"n": int(cat[0].shape[0]), "k": q[6], "us_three_launches": round(ms3 * 1e3, 2),
                  "us_fused": round(ms1 * 1e3, 2)}

    def capture(body):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            body()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=side):
                body()
        torch.cuda.synchronize()
        return g

    def seq(st):
        def body():
            for (w, s_, b, x, y, n, k) in st:
                qmm.qgemv(w, s_, b, x, wl.bits, y=y)
        return body
    graphs = [capture(seq(st)) for st in sets]
    ms_g, _ = time_launches(torch, lambda i: graphs[i % copies].replay(), steps, warmup, stream)
    step_bytes = sum(gemv_bytes(p.n, p.k, wl.bits) for _, _, p in wl.problems())
    out["graph_197"] = {"launches": len(sets[0]), "ms_per_pass": round(ms_g, 4),
                        "gb_per_s": round(step_bytes / (ms_g * 1e-3) / 1e9, 1)}
    tiny = torch.zeros(1, device="cuda")

    def empty():
        for _ in range(len(sets[0])):
            tiny.add_(1.0)
    g0 = capture(empty)
    ms_0, _ = time_launches(torch, lambda i: g0.replay(), steps, warmup, stream)
    out["graph_floor"] = {"launches": len(sets[0]), "us_per_launch": round(ms_0 * 1e3 / len(sets[0]), 3)}
    del graphs, g0
    return out


# Projections of one layer that read the same activations run as one batched
# launch: q, k and v; o; gate and up; down.
PREFILL_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


PREFILL_WEIGHTS = "tile-interleaved copy (qmm_repack_tiled, once at load)"


def bench_prefill(torch, qmm, ms, steps=3, warmup=1, batched=True):
    wl = synth.QWEN3_4B_Q4_PREFILL
    out = {}
    base = {}
    for i, p in enumerate(wl.projs):
        wf = torch.from_numpy(synth.draw_weight((wl.wid, 0, i, synth.STREAM_W), p.n, p.k)).cuda()
        words, s_, b_ = qmm.quantize(wf, wl.bits)
        # the batched launches read the tile-interleaved copy (repacked once,
        # as a model would at load time); the per-projection path row-major
        base[i] = (qmm.repack_tiled(words, wl.bits), s_, b_) if batched else (words, s_, b_)
        del wf, words
    layers = [[tuple(t.clone() for t in base[i]) if layer else base[i]
               for i in range(len(wl.projs))] for layer in range(wl.layers)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for m in ms:
        xs = [torch.from_numpy(synth.draw_act((wl.wid, m, i, synth.STREAM_X), m, p.k)).cuda()
              for i, p in enumerate(wl.projs)]
        ys = [torch.empty((m, p.n), dtype=torch.float32, device="cuda") for p in wl.projs]
        if batched:
            names = [p.name for p in wl.projs]
            plans = [[qmm.qgemm_batched_plan(
                [(*L[names.index(nm)], xs[names.index(nm)], ys[names.index(nm)]) for nm in grp],
                wl.bits, tiled=True) for grp in PREFILL_GROUPS] for L in layers]

            def step(_):
                for lp in plans:
                    for plan in lp:
                        qmm.qgemm_batched(plan)
        else:
            def step(_):
                for L in layers:
                    for i, (words, s, b) in enumerate(L):
                        qmm.qgemm(words, s, b, xs[i], wl.bits, y=ys[i])
        ms_step, _ = time_launches(torch, step, steps, warmup, stream)
        flops = 2.0 * m * sum(p.n * p.k for p in wl.projs) * wl.layers
        tfl = flops / (ms_step * 1e-3) / 1e12
        out[str(m)] = {"ms_per_step": round(ms_step, 3), "tflops": round(tfl, 1),
                       "frac_of_fp16_peak": round(tfl / FP16_MFMA_PEAK_TFLOPS, 4)}
        if batched:
            out[str(m)]["tiles"] = {"+".join(g): "{bm}x{n}/S{splits}".format(n=pl.header["nb"] * 128, **pl.header)
                                    for g, pl in zip(PREFILL_GROUPS, plans[0])}
            del plans
        del xs, ys
    del layers, base
    torch.cuda.synchronize()
    return out


def bench_moe(torch, qmm, steps=10, warmup=2):
    wl = synth.QWEN3_30B_A3B_Q4_MOE
    out = {}
    weights = []
    for pi, (name, k, n, per_pair) in enumerate(synth.moe_projs(wl)):
        ws, ss, bs = [], [], []
        for e in range(wl.experts):
            wf = torch.from_numpy(synth.draw_weight((wl.wid, e, pi, synth.STREAM_W), n, k)).cuda()
            w_, s_, b_ = qmm.quantize(wf, wl.bits)
            ws.append(w_); ss.append(s_); bs.append(b_)
        # tile-interleaved copy of the stacked expert words (once, at load)
        weights.append((qmm.repack_tiled(torch.stack(ws), wl.bits), torch.stack(ss), torch.stack(bs),
                        n, k, per_pair))
        del ws, ss, bs
    stream = torch.cuda.current_stream()
    for m in wl.ms:
        calls = []
        step_bytes = 0
        flops = 0
        for pi, (W, S, B, n, k, per_pair) in enumerate(weights):
            a, ids, _ = synth.draw_moe_inputs(wl, m, pi)
            A = torch.from_numpy(a).cuda()
            I = torch.from_numpy(ids).cuda()
            pairs = m * wl.top_k
            Y = torch.empty((pairs, n), dtype=torch.float32, device="cuda")
            wsz = qmm.qgemm_grouped_workspace_size(m, wl.top_k, wl.experts, n, k, wl.bits)
            WS = torch.empty(wsz, dtype=torch.uint8, device="cuda")
            used = np.unique(ids).size
            step_bytes += used * (n * k * wl.bits // 8 + 4 * n * (k // 64)) + A.numel() * 2 \
                + pairs * n * 4 + ids.size * 4
            flops += 2 * pairs * n * k
            calls.append((W, S, B, A, I, per_pair, Y, WS))

        # the three projections share the routing: bucket once per step
        ids0 = calls[0][4]
        plan = qmm.moe_route(ids0, wl.experts)

        def step(_):
            qmm.moe_route(ids0, wl.experts, plan=plan)
            for (W, S, B, A, I, per_pair, Y, WS) in calls:
                qmm.qgemm_grouped(W, S, B, A, I, wl.bits, per_pair, y=Y, plan=plan, tiled=True)

        def step_unshared(_):
            for (W, S, B, A, I, per_pair, Y, WS) in calls:
                qmm.qgemm_grouped(W, S, B, A, I, wl.bits, per_pair, y=Y, workspace=WS, tiled=True)
        ms_step, _ = time_launches(torch, step, steps, warmup, stream)
        ms_unshared, _ = time_launches(torch, step_unshared, steps, warmup, stream)
        t = ms_step * 1e-3
        roof = max(step_bytes / (HBM_PEAK_GBS * 1e9), flops / (FP16_MFMA_PEAK_TFLOPS * 1e12))
        out[str(m)] = {"ms_per_step": round(ms_step, 4), "gb_per_s": round(step_bytes / t / 1e9, 1),
                       "tflops": round(flops / t / 1e12, 2), "frac_of_roofline": round(roof / t, 4),
                       "launches": "1 routing + 3 grouped GEMMs",
                       "ms_per_step_bucketing_each_gemm": round(ms_unshared, 4)}
        # the whole FFN block: routing, fused gate+up with SwiGLU (fp16 h),
        # down from h, routing-weighted combine into y [M, hidden]
        (Wg, Sg, Bg, X, _, _, _, _), (Wu, Su, Bu, _, _, _, _, _), (Wd, Sd, Bd, _, _, _, Yd, _) = calls
        pairs = m * wl.top_k
        H = torch.empty((pairs, wl.inter), dtype=torch.float16, device="cuda")
        logits = synth.draw_logits((wl.wid, m, 0, synth.STREAM_LOGITS), m, wl.experts)
        p_ = np.exp(logits - logits.max(axis=1, keepdims=True))
        p_ = p_ / p_.sum(axis=1, keepdims=True)
        wts = np.take_along_axis(p_, calls[0][4].cpu().numpy().astype(np.int64), axis=1)
        Wts = torch.from_numpy((wts / wts.sum(axis=1, keepdims=True)).astype(np.float32)).cuda()
        Yout = torch.empty((m, wl.hidden), dtype=torch.float32, device="cuda")

        def block(_):
            qmm.moe_route(ids0, wl.experts, plan=plan)
            qmm.moe_gate_up_swiglu((Wg, Sg, Bg), (Wu, Su, Bu), X, ids0, plan, wl.bits, h=H, tiled=True)
            qmm.qgemm_grouped(Wd, Sd, Bd, H, ids0, wl.bits, True, y=Yd, plan=plan, tiled=True)
            qmm.moe_combine(Yd, Wts, y=Yout)
        ms_block, _ = time_launches(torch, block, steps, warmup, stream)
        used = np.unique(calls[0][4].cpu().numpy()).size
        wbytes = sum(used * (n * k * wl.bits // 8 + 4 * n * (k // 64)) for (_, k, n, _) in synth.moe_projs(wl))
        bbytes = wbytes + m * wl.hidden * 2 + 2 * pairs * wl.inter * 2 + 2 * pairs * wl.hidden * 4 \
            + m * wl.hidden * 4 + m * wl.top_k * 8
        tb = ms_block * 1e-3
        broof = max(bbytes / (HBM_PEAK_GBS * 1e9), flops / (FP16_MFMA_PEAK_TFLOPS * 1e12))
        out[str(m)]["ffn_block"] = {
            "launches": "routing + fused gate/up SwiGLU + down + combine",
            "ms_per_block": round(ms_block, 4), "bytes": int(bbytes),
            "tflops": round(flops / tb / 1e12, 2), "frac_of_roofline": round(broof / tb, 4)}
        del calls
    del weights
    torch.cuda.synchronize()
    return out


def cpu_baseline(wl, budget_s=15.0):
    """The float64 oracle (unpack -> dequantize -> matmul) on a bounded
    sample of the decode workload: whole layers in order, then lm_head row
    slices, until about `budget_s` seconds of oracle time."""
    import oracle
    try:
        import threadpoolctl
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    done_bytes = 0
    spent = 0.0
    items = 0
    problems = wl.problems()
    order = [p for p in problems if p[0] < wl.layers] + \
        [(wl.layers, len(wl.projs), synth.Proj("lm_head", 1024, 4096))] * 8
    for layer, i, p in order:
        if spent >= budget_s:
            break
        w = synth.draw_weight((wl.wid, min(layer, wl.layers), i, synth.STREAM_W), p.n, p.k)
        codes, s, b = oracle.quantize(w, wl.bits)
        words = oracle.pack(codes, wl.bits)
        x = synth.draw_act((wl.wid, layer, i, synth.STREAM_X), 1, p.k)
        t0 = time.perf_counter()
        oracle.qmatmul_f64(words, s, b, x, wl.bits)
        spent += time.perf_counter() - t0
        done_bytes += gemv_bytes(p.n, p.k, wl.bits)
        items += 1
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{items} GEMVs of the decode workload ({done_bytes / 1e6:.1f} MB algorithmic, "
                      f"{spent:.1f} s of float64 unpack+dequant+matmul; lm_head as 4096-row slices)"}


# ------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", choices=["all", "decode", "decode_extras", "projections", "prefill", "moe"],
                    default="all",
                    help="run one workload only (for profiling); prefill and moe print "
                         "their own section as the JSON line")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--gemm", metavar="M,N,K",
                    help="run only qmm_qgemm on one 4-bit shape, --steps times (for counters), and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_matmul_qgemv_amd as qmm
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    qmm.lib()  # fail loudly if the HIP library is missing

    if args.copy_calib:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "launches": 5}))
        return

    if args.gemm:
        m, n, k = (int(v) for v in args.gemm.split(","))
        wq = qmm.quantize(torch.from_numpy(synth.draw_weight((9, m, n, k), n, k)).cuda(), 4)
        x = torch.from_numpy(synth.draw_act((9, m, n, k + 1), m, k)).cuda()
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(qmm.qgemm_workspace_size(m, n, k, 4), 16), dtype=torch.uint8, device="cuda")
        ms_call, _ = time_launches(torch, lambda i: qmm.qgemm(*wq, x, 4, y=y, workspace=ws),
                                   args.steps, args.warmup, torch.cuda.current_stream())
        print(json.dumps({"gemm": [m, n, k], "ms_per_call": round(ms_call, 4),
                          "tflops": round(2.0 * m * n * k / (ms_call * 1e-3) / 1e12, 1)}), flush=True)
        return

    if args.only in ("prefill", "moe"):
        if args.only == "prefill":
            out = {"workload": synth.QWEN3_4B_Q4_PREFILL.name, "peak_tflops": FP16_MFMA_PEAK_TFLOPS,
                   "weights": PREFILL_WEIGHTS,
                   "by_m": bench_prefill(torch, qmm, synth.QWEN3_4B_Q4_PREFILL.ms)}
        else:
            out = {"workload": synth.QWEN3_30B_A3B_Q4_MOE.name, "weights": PREFILL_WEIGHTS,
                   "by_m": bench_moe(torch, qmm)}
        print(json.dumps(out), flush=True)
        return

    wl = synth.QWEN3_0_6B_Q4_DECODE
    log("decode: preparing", wl.name)
    d = bench_decode(torch, qmm, wl, args.steps, args.warmup)
    # one step is one launch of the batched kernel, so the kernel's average
    # launch time is the timed region divided by the steps
    value = d["step_bytes"] / (d["ms_step"] * 1e-3) / 1e9
    achieved = value
    log(f"decode: {value:.1f} GB/s")
    traffic = None
    if TRAFFIC["sources_sha256"] == kernel_sources_sha256():
        traffic = round(TRAFFIC["fetch_kib"] * 1024 * TRAFFIC["fetch_scale"]
                        + TRAFFIC["write_kib"] * 1024 * TRAFFIC["write_scale"])
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "gemvs_per_step": len(wl.problems()),
                   "bits": wl.bits, "group_size": wl.group_size,
                   "weights_per_step": wl.weight_count(), "bytes_per_step": d["step_bytes"],
                   "launch": "one qmm_qgemv_batched launch per step",
                   "weight_copies_alternated": 2},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "qgemv_batched_kernel<4,16,4,64>",
                     "bytes_per_launch": d["step_bytes"],
                     "launch_ms_mean": round(d["ms_step"], 5)},
    }
    if args.only in ("all", "decode_extras"):
        log("decode extras")
        result["decode_context"] = bench_decode_extras(torch, qmm, wl, d["sets"])
    if args.only == "projections":
        result["projections"] = bench_projections(torch, qmm, wl, d["sets"])
    del d
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if args.only == "all":
        log("single GEMV")
        result["single_gemv"] = bench_single_gemv(torch, qmm)
        log("decode Q8")
        q8 = bench_decode(torch, qmm, synth.LLAMA32_3B_Q8_DECODE, 10, 3)
        gbs = q8["step_bytes"] / (q8["ms_step"] * 1e-3) / 1e9
        result["decode_q8"] = {"workload": synth.LLAMA32_3B_Q8_DECODE.name,
                               "bytes_per_step": q8["step_bytes"], "ms_per_step": round(q8["ms_step"], 4),
                               "gb_per_s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del q8
        torch.cuda.empty_cache()
        log("decode formats")
        result["decode_formats"] = {"workload": wl.name + " shapes", **bench_decode_formats(torch, qmm, wl)}
        log("prefill")
        result["prefill"] = {"workload": synth.QWEN3_4B_Q4_PREFILL.name,
                             "peak_tflops": FP16_MFMA_PEAK_TFLOPS, "weights": PREFILL_WEIGHTS,
                             "by_m": bench_prefill(torch, qmm, synth.QWEN3_4B_Q4_PREFILL.ms)}
        torch.cuda.empty_cache()
        log("gemm formats")
        result["gemm_formats"] = {"shape": [2048, 9728, 2560], "weights": PREFILL_WEIGHTS,
                                  **bench_gemm_formats(torch, qmm)}
        log("moe")
        result["moe"] = {"workload": synth.QWEN3_30B_A3B_Q4_MOE.name, "weights": PREFILL_WEIGHTS,
                         "by_m": bench_moe(torch, qmm)}
    if not args.no_cpu:
        log("cpu baseline")
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
