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
LLC_EVICT_BYTES = 320 << 20     # more than the 256 MB last-level cache (MALL)
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
    "fetch_kib": 171951.3, "fetch_scale": 1073741824 / (524301.3 * 1024),
    "write_kib": 1937.5, "write_scale": 1073741824 / (1048576.0 * 1024),
    "sources_sha256": "ea51f520baa2af36c0ee180ce6299d4b0cda6ce07b3a48f84671f36ce5f2fcc1",
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


def time_steps(torch, step, steps, warmup, stream):
    """Warm up, then time each of `steps` calls between its own pair of HIP
    events on the launch stream (a step here is a whole prefill or MoE pass,
    milliseconds long, so per-step events cost nothing measurable).  Returns
    the per-step times in ms."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(warmup + i)
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def step_stats(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"ms_per_step_median": round(float(np.median(a)), 4), "ms_per_step_min": round(float(a.min()), 4),
            "ms_per_step_mean": round(float(a.mean()), 4), "steps_timed": int(a.size)}


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
    weight width, TFLOP/s against the fp16 matrix-core peak.  Consecutive
    calls rotate over enough device copies of the weights (more than the
    256 MB last-level cache holds) that no call finds its weights cached."""
    out = {}
    wf = torch.from_numpy(synth.draw_weight((9, m, n, k), n, k)).cuda()
    x = torch.from_numpy(synth.draw_act((9, m, n, k + 1), m, k)).cuda()
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for bits in bits_list:
        wq = (wf.half().view(torch.int32), None, None) if bits == 16 else qmm.quantize(wf, bits)
        stiled = PREFILL_SCALES_TILED and bits != 16
        # tile-interleaved copy (and interleaved scales), once
        wq = (qmm.repack_tiled(wq[0], bits), qmm.repack_scales_tiled(wq[1], wq[2]) if stiled else wq[1],
              None if stiled else wq[2])
        wbytes = sum(t.numel() * t.element_size() for t in wq if t is not None)
        copies = max(2, -(-LLC_EVICT_BYTES // wbytes))
        sets = [wq] + [tuple(None if t is None else t.clone() for t in wq) for _ in range(copies - 1)]
        ws = torch.empty(max(qmm.qgemm_workspace_size(m, n, k, bits), 16), dtype=torch.uint8, device="cuda")
        ms_call, _ = time_launches(
            torch, lambda i: qmm.qgemm(*sets[i % copies], x, bits, y=y, workspace=ws, tiled=True,
                                       scales_tiled=stiled),
            steps, warmup, stream)
        tfl = 2.0 * m * n * k / (ms_call * 1e-3) / 1e12
        out["f16" if bits == 16 else f"q{bits}"] = {"ms_per_call": round(ms_call, 4), "tflops": round(tfl, 1),
                           "frac_of_fp16_peak": round(tfl / FP16_MFMA_PEAK_TFLOPS, 4),
                           "weight_copies_rotated": copies}
        del wq, ws, sets
        torch.cuda.empty_cache()
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


def bench_streaming_reference(torch, nbytes):
    """Plain streaming rates of the same GPU, for scale: the best of a
    read-only kernel over `nbytes` (16-byte loads, several grid sizes, with
    ordinary and with non-temporal loads, two buffers alternating so every
    launch reads HBM; the stand-alone harness stream_probe.hip, no library
    code), and a 1 GiB device-to-device copy (read + write) through torch."""
    import subprocess
    out = {}
    exe = os.path.join(ROOT, "quantized_matmul_qgemv_amd", "qmm_stream_probe")
    if os.path.exists(exe):
        r = subprocess.run([exe, str(nbytes)], capture_output=True, text=True, timeout=300)
        if r.returncode == 0:
            out["read_only_kernel"] = json.loads(r.stdout.strip().splitlines()[-1])
        else:
            log("stream probe failed:", r.stderr.strip()[-500:])
    stream = torch.cuda.current_stream()
    src = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    ms_copy, _ = time_launches(torch, lambda i: dst.copy_(src), 10, 2, stream)
    del src, dst
    torch.cuda.empty_cache()
    out["copy_1gib"] = {"bytes_moved": 2 << 30, "ms": round(ms_copy, 4),
                        "gb_per_s": round((2 << 30) / (ms_copy * 1e-3) / 1e9, 1)}
    return out


def bench_decode_extras(torch, qmm, wl, sets, steps=20, warmup=3):
    """Context for the batched headline, on the same weight copies:
      lm_head      the 1024 -> 151936 projection alone, one qmm_qgemv launch;
      graph_197    the decode pass as 197 sequential qmm_qgemv launches (the
                   order a dependent decode would need) replayed as one HIP graph;
      graph_floor  the same graph shape with 197 one-element kernels: the
                   per-launch floor that the sequential form pays;
      graph_layer_batched  a dependent decode step batched only where one
                   step allows it: per layer q+k+v as one GEMV over the
                   weights stacked along n, o, gate+up likewise stacked, down
                   (the projections that read the same activations share a
                   launch), then the lm_head: 4 x 28 + 1 = 113 launches
                   replayed as one HIP graph (the stacked q+k+v and gate+up
                   read the first projection's activations)."""
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

    names = [p.name for p in wl.projs]
    groups = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    if all(nm in names for grp in groups for nm in grp):
        def layer_launches(st):
            seq_l = []
            for layer in range(wl.layers):
                base = layer * len(names)
                for grp in groups:
                    parts = [st[base + names.index(nm)] for nm in grp]
                    if len(parts) == 1:
                        w, s_, b, x, y, n, k = parts[0]
                    else:
                        w, s_, b = (torch.cat([t[j] for t in parts]) for j in range(3))
                        x, k = parts[0][3], parts[0][6]
                        n = int(w.shape[0])
                        y = torch.empty(n, dtype=torch.float32, device="cuda")
                    seq_l.append((w, s_, b, x, y))
            w, s_, b, x, y, n, k = st[-1]   # lm_head
            seq_l.append((w, s_, b, x, y))
            return seq_l
        stacked = [layer_launches(st) for st in sets]

        def seq_layers(lst):
            def body():
                for (w, s_, b, x, y) in lst:
                    qmm.qgemv(w, s_, b, x, wl.bits, y=y)
            return body
        graphs = [capture(seq_layers(lst)) for lst in stacked]
        ms_l, _ = time_launches(torch, lambda i: graphs[i % copies].replay(), steps, warmup, stream)
        out["graph_layer_batched"] = {"launches": len(stacked[0]), "ms_per_pass": round(ms_l, 4),
                                      "gb_per_s": round(step_bytes / (ms_l * 1e-3) / 1e9, 1)}
        del graphs, stacked
    return out


# Projections of one layer that read the same activations run as one batched
# launch: q, k and v; o; gate and up; down.
PREFILL_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


# The prefill and MoE GEMMs read interleaved scales and biases
# (qmm_repack_scales_tiled) unless --row-major-scales is given.
PREFILL_SCALES_TILED = True
PREFILL_WEIGHTS = ("tile-interleaved copy (qmm_repack_tiled, once at load) with interleaved scales and "
                   "biases (qmm_repack_scales_tiled, once at load)")


def prefill_layers(torch, qmm, wl, batched=True):
    """Per-layer weights of the prefill workload: each distinct projection
    quantized once on the GPU, then device copies for every layer (36 x 57 MB
    at 4 bits, far more than the last-level cache).  Batched launches read
    the tile-interleaved copy (repacked once, as a model would at load time);
    the per-projection path reads row-major words."""
    base = {}
    for i, p in enumerate(wl.projs):
        wf = torch.from_numpy(synth.draw_weight((wl.wid, 0, i, synth.STREAM_W), p.n, p.k)).cuda()
        words, s_, b_ = qmm.quantize(wf, wl.bits)
        if not batched:
            base[i] = (words, s_, b_)
        elif PREFILL_SCALES_TILED:
            base[i] = (qmm.repack_tiled(words, wl.bits), qmm.repack_scales_tiled(s_, b_), None)
        else:
            base[i] = (qmm.repack_tiled(words, wl.bits), s_, b_)
        del wf, words
    layers = [[tuple(None if t is None else t.clone() for t in base[i]) if layer else base[i]
               for i in range(len(wl.projs))] for layer in range(wl.layers)]
    torch.cuda.synchronize()
    return layers


def prefill_io(torch, wl, m):
    xs = [torch.from_numpy(synth.draw_act((wl.wid, m, i, synth.STREAM_X), m, p.k)).cuda()
          for i, p in enumerate(wl.projs)]
    ys = [torch.empty((m, p.n), dtype=torch.float32, device="cuda") for p in wl.projs]
    return xs, ys


def prefill_plans(qmm, wl, layers, xs, ys, groups=PREFILL_GROUPS):
    names = [p.name for p in wl.projs]
    return [[qmm.qgemm_batched_plan(
        [(*L[names.index(nm)], xs[names.index(nm)], ys[names.index(nm)]) for nm in grp],
        wl.bits, tiled=True, scales_tiled=PREFILL_SCALES_TILED) for grp in groups] for L in layers]


def prefill_work(wl, m):
    """Algorithmic bytes (x, packed codes, fp16 scales and biases, y, each
    once) and flops of one prefill step (all layers) at m rows."""
    per_layer = sum(m * p.k * 2 + p.n * p.k * wl.bits // 8 + 4 * p.n * (p.k // 64) + 4 * m * p.n
                    for p in wl.projs)
    flops = 2.0 * m * sum(p.n * p.k for p in wl.projs) * wl.layers
    return per_layer * wl.layers, flops


def bench_prefill(torch, qmm, ms, steps=20, warmup=3, batched=True):
    """Each step: 36 layers x 4 batched launches (q+k+v, o, gate+up, down).
    Per-step HIP events; median and minimum over `steps` timed steps.
    Roofline per M: min(fp16 matrix-core peak, intensity x HBM bandwidth)."""
    wl = synth.QWEN3_4B_Q4_PREFILL
    out = {}
    layers = prefill_layers(torch, qmm, wl, batched)
    stream = torch.cuda.current_stream()
    for m in ms:
        xs, ys = prefill_io(torch, wl, m)
        if batched:
            plans = prefill_plans(qmm, wl, layers, xs, ys)

            def step(_):
                for lp in plans:
                    for plan in lp:
                        qmm.qgemm_batched(plan)
        else:
            def step(_):
                for L in layers:
                    for i, (words, s, b) in enumerate(L):
                        qmm.qgemm(words, s, b, xs[i], wl.bits, y=ys[i])
        st = step_stats(time_steps(torch, step, steps, warmup, stream))
        nbytes, flops = prefill_work(wl, m)
        roof_s = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (FP16_MFMA_PEAK_TFLOPS * 1e12))
        roof_tfl = flops / roof_s / 1e12
        tfl = flops / (st["ms_per_step_median"] * 1e-3) / 1e12
        out[str(m)] = {**st, "tflops": round(tfl, 1),
                       "tflops_at_min": round(flops / (st["ms_per_step_min"] * 1e-3) / 1e12, 1),
                       "frac_of_fp16_peak": round(tfl / FP16_MFMA_PEAK_TFLOPS, 4),
                       "bytes_per_step": int(nbytes), "flops_per_step": flops,
                       "roofline_tflops": round(roof_tfl, 1),
                       "roofline_bound": "mfma" if roof_tfl >= FP16_MFMA_PEAK_TFLOPS - 1e-6 else "hbm",
                       "frac_of_roofline": round(tfl / roof_tfl, 4)}
        if batched:
            out[str(m)]["tiles"] = {"+".join(g): "{bm}x{n}/S{splits}/K{kw}".format(n=pl.header["nb"] * 128, **pl.header)
                                    for g, pl in zip(PREFILL_GROUPS, plans[0])}
            del plans
        del xs, ys
    del layers
    torch.cuda.synchronize()
    return out


def prefill_roofline_block(by_m):
    """The prefill half of the metric: achieved TFLOP/s (median step) against
    min(fp16 matrix-core peak, arithmetic intensity x HBM bandwidth) per M."""
    return {"unit": "TFLOP/s", "peak": FP16_MFMA_PEAK_TFLOPS, "hbm_peak_gbs": HBM_PEAK_GBS,
            "kernel": "qgemm_batched_kernel (4 launches per layer)",
            "by_m": {m: {"achieved": v["tflops"], "roofline": v["roofline_tflops"], "bound": v["roofline_bound"],
                         "frac": v["frac_of_roofline"], "frac_of_peak": v["frac_of_fp16_peak"],
                         "ms_per_step_median": v["ms_per_step_median"], "ms_per_step_min": v["ms_per_step_min"]}
                     for m, v in by_m.items()}}


def moe_weights(torch, qmm, wl, copies=2):
    """Expert weights of gate, up and down (quantized once on the GPU, then
    repacked to the tile-interleaved layout), `copies` device copies so that
    consecutive steps never find them in the last-level cache (340 MB each)."""
    sets = [[] for _ in range(copies)]
    for pi, (name, k, n, per_pair) in enumerate(synth.moe_projs(wl)):
        ws, ss, bs = [], [], []
        for e in range(wl.experts):
            wf = torch.from_numpy(synth.draw_weight((wl.wid, e, pi, synth.STREAM_W), n, k)).cuda()
            w_, s_, b_ = qmm.quantize(wf, wl.bits)
            ws.append(w_); ss.append(s_); bs.append(b_)
        W = qmm.repack_tiled(torch.stack(ws), wl.bits)
        S, B = torch.stack(ss), torch.stack(bs)
        if PREFILL_SCALES_TILED:  # interleaved scales and biases, one array
            S, B = qmm.repack_scales_tiled(S, B), None
        del ws, ss, bs
        for c in range(copies):
            sets[c].append((W, S, B, n, k, per_pair) if c == 0 else
                           (W.clone(), S.clone(), None if B is None else B.clone(), n, k, per_pair))
    torch.cuda.synchronize()
    return sets


def bench_moe(torch, qmm, steps=20, warmup=3, copies=2):
    wl = synth.QWEN3_30B_A3B_Q4_MOE
    out = {}
    wsets = moe_weights(torch, qmm, wl, copies)
    stream = torch.cuda.current_stream()
    for m in wl.ms:
        ins = []
        step_bytes = 0
        flops = 0
        pairs = m * wl.top_k
        for pi, (W, S, B, n, k, per_pair) in enumerate(wsets[0]):
            a, ids, _ = synth.draw_moe_inputs(wl, m, pi)
            A = torch.from_numpy(a).cuda()
            I = torch.from_numpy(ids).cuda()
            Y = torch.empty((pairs, n), dtype=torch.float32, device="cuda")
            wsz = qmm.qgemm_grouped_workspace_size(m, wl.top_k, wl.experts, n, k, wl.bits)
            WS = torch.empty(wsz, dtype=torch.uint8, device="cuda")
            used = np.unique(ids).size
            step_bytes += used * (n * k * wl.bits // 8 + 4 * n * (k // 64)) + A.numel() * 2 \
                + pairs * n * 4 + ids.size * 4
            flops += 2 * pairs * n * k
            ins.append((A, I, per_pair, Y, WS))
        # the three projections share the routing: bucket once per step
        ids0 = ins[0][1]
        plan = qmm.moe_route(ids0, wl.experts)

        def step(i):
            ws = wsets[i % copies]
            qmm.moe_route(ids0, wl.experts, plan=plan)
            for (W, S, B, n, k, _), (A, I, per_pair, Y, WS) in zip(ws, ins):
                qmm.qgemm_grouped(W, S, B, A, I, wl.bits, per_pair, y=Y, plan=plan, tiled=True,
                                  scales_tiled=PREFILL_SCALES_TILED)

        def step_unshared(i):
            ws = wsets[i % copies]
            for (W, S, B, n, k, _), (A, I, per_pair, Y, WS) in zip(ws, ins):
                qmm.qgemm_grouped(W, S, B, A, I, wl.bits, per_pair, y=Y, workspace=WS, tiled=True,
                                  scales_tiled=PREFILL_SCALES_TILED)
        st = step_stats(time_steps(torch, step, steps, warmup, stream))
        st_un = step_stats(time_steps(torch, step_unshared, steps, warmup, stream))
        t = st["ms_per_step_median"] * 1e-3
        roof = max(step_bytes / (HBM_PEAK_GBS * 1e9), flops / (FP16_MFMA_PEAK_TFLOPS * 1e12))
        out[str(m)] = {**st, "gb_per_s": round(step_bytes / t / 1e9, 1),
                       "tflops": round(flops / t / 1e12, 2), "bytes_per_step": int(step_bytes),
                       "flops_per_step": int(flops), "roofline_ms": round(roof * 1e3, 4),
                       "frac_of_roofline": round(roof / t, 4),
                       "launches": "1 routing + 3 grouped GEMMs",
                       "ms_per_step_bucketing_each_gemm": st_un["ms_per_step_median"]}
        # the whole FFN block: routing, fused gate+up with SwiGLU (fp16 h),
        # down from h, routing-weighted combine into y [M, hidden]
        (A, _, _, _, _), _, (_, _, _, Yd, _) = ins
        H = torch.empty((pairs, wl.inter), dtype=torch.float16, device="cuda")
        logits = synth.draw_logits((wl.wid, m, 0, synth.STREAM_LOGITS), m, wl.experts)
        p_ = np.exp(logits - logits.max(axis=1, keepdims=True))
        p_ = p_ / p_.sum(axis=1, keepdims=True)
        wts = np.take_along_axis(p_, ids0.cpu().numpy().astype(np.int64), axis=1)
        Wts = torch.from_numpy((wts / wts.sum(axis=1, keepdims=True)).astype(np.float32)).cuda()
        Yout = torch.empty((m, wl.hidden), dtype=torch.float32, device="cuda")

        def block(i):
            (Wg, Sg, Bg, *_), (Wu, Su, Bu, *_), (Wd, Sd, Bd, *_) = wsets[i % copies]
            qmm.moe_route(ids0, wl.experts, plan=plan)
            qmm.moe_gate_up_swiglu((Wg, Sg, Bg), (Wu, Su, Bu), A, ids0, plan, wl.bits, h=H, tiled=True,
                                   scales_tiled=PREFILL_SCALES_TILED)
            qmm.qgemm_grouped(Wd, Sd, Bd, H, ids0, wl.bits, True, y=Yd, plan=plan, tiled=True,
                              scales_tiled=PREFILL_SCALES_TILED)
            qmm.moe_combine(Yd, Wts, y=Yout)
        stb = step_stats(time_steps(torch, block, steps, warmup, stream))
        used = np.unique(ids0.cpu().numpy()).size
        wbytes = sum(used * (n * k * wl.bits // 8 + 4 * n * (k // 64)) for (_, k, n, _) in synth.moe_projs(wl))
        bbytes = wbytes + m * wl.hidden * 2 + 2 * pairs * wl.inter * 2 + 2 * pairs * wl.hidden * 4 \
            + m * wl.hidden * 4 + m * wl.top_k * 8
        tb = stb["ms_per_step_median"] * 1e-3
        broof = max(bbytes / (HBM_PEAK_GBS * 1e9), flops / (FP16_MFMA_PEAK_TFLOPS * 1e12))
        out[str(m)]["ffn_block"] = {
            "launches": "routing + fused gate/up SwiGLU + down + combine",
            "ms_per_block_median": stb["ms_per_step_median"], "ms_per_block_min": stb["ms_per_step_min"],
            "bytes": int(bbytes), "tflops": round(flops / tb / 1e12, 2),
            "frac_of_roofline": round(broof / tb, 4)}
        del ins
    del wsets
    torch.cuda.synchronize()
    return out


def host_info():
    """Cores and CPU of the host the oracle runs on."""
    try:
        import threadpoolctl
        blas = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = 1
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "nproc": len(os.sched_getaffinity(0)),
            "blas_threads": int(blas), "cpu_model": model}


def _oracle_gemm(oracle, wl, layer, i, p, m, rows=None):
    """Inputs of one projection (quantized by the oracle, not timed) and the
    timed oracle call; rows limits the output rows (a row slice)."""
    n = p.n if rows is None else min(rows, p.n)
    w = synth.draw_weight((wl.wid, layer, i, synth.STREAM_W), n, p.k)
    codes, s, b = oracle.quantize(w, wl.bits)
    words = oracle.pack(codes, wl.bits)
    x = synth.draw_act((wl.wid, m, i, synth.STREAM_X), m, p.k)
    t0 = time.perf_counter()
    oracle.qmatmul_f64(words, s, b, x, wl.bits)
    return time.perf_counter() - t0, n


def cpu_baseline(wl, budget_s=8.0):
    """The float64 oracle (unpack -> dequantize -> matmul, numpy: the unpack
    and dequantize steps run on one thread, the matmul on the BLAS threads)
    on a bounded sample of the decode workload: whole layers in order, then
    lm_head row slices, until about `budget_s` seconds of oracle time."""
    import oracle
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
    info = host_info()
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": info["blas_threads"],
            "kind": "oracle", **info,
            "sample": f"{items} GEMVs of the decode workload ({done_bytes / 1e6:.1f} MB algorithmic, "
                      f"{spent:.1f} s of float64 unpack+dequant+matmul; lm_head as 4096-row slices)"}


def cpu_baseline_configs(rows=2048, experts=16):
    """The oracle on bounded samples of the other workloads, each scaled to
    the whole workload and labelled as such:
      single GEMV 1x1024x1024 (timed in full, best of 3);
      Llama-3.2-3B Q8 decode: layer 0, the first `rows` output rows of each
        projection, scaled by weight count to the 196-GEMV pass (every layer
        has the same shapes);
      Qwen3-4B Q4 prefill at each M: layer 0, the first `rows` output rows of
        each projection, scaled by weight count to 36 layers;
      Qwen3-30B-A3B MoE at each M: gate, up and down for the pairs of the
        first `experts` experts, scaled by the number of experts (the
        oracle's time is dominated by unpacking and dequantizing each
        expert's weights once)."""
    import oracle
    out = {}
    single = synth.SINGLE_Q4
    p = single.projs[0]
    best = min(_oracle_gemm(oracle, single, 0, 0, p, 1)[0] for _ in range(3))
    out["q4-gemv-1x1024x1024"] = {"ms": round(best * 1e3, 3),
                                  "gb_per_s": round(gemv_bytes(p.n, p.k, 4) / best / 1e9, 4),
                                  "sample": "whole GEMV, best of 3"}
    q8 = synth.LLAMA32_3B_Q8_DECODE
    spent, wsample, bsample = 0.0, 0, 0
    for i, p in enumerate(q8.projs):
        dt, n = _oracle_gemm(oracle, q8, 0, i, p, 1, rows)
        spent += dt
        wsample += n * p.k
        bsample += gemv_bytes(n, p.k, q8.bits)
    scale = q8.weight_count() / wsample
    out[q8.name] = {"ms_per_step_extrapolated": round(spent * scale * 1e3, 1),
                    "gb_per_s": round(bsample / spent / 1e9, 4),
                    "sample": f"layer 0, first {rows} rows of each projection ({spent:.1f} s); "
                              f"x{scale:.1f} by weight count, extrapolated (identical shapes per layer)"}
    pf = synth.QWEN3_4B_Q4_PREFILL
    by_m = {}
    for m in pf.ms:
        spent, wsample, fl = 0.0, 0, 0.0
        for i, p in enumerate(pf.projs):
            dt, n = _oracle_gemm(oracle, pf, 0, i, p, m, rows)
            spent += dt
            wsample += n * p.k
        scale = pf.weight_count() / wsample
        _, flops = prefill_work(pf, m)
        t_full = spent * scale
        by_m[str(m)] = {"ms_per_step_extrapolated": round(t_full * 1e3, 1),
                        "tflops": round(flops / t_full / 1e12, 5),
                        "sample_s": round(spent, 2)}
    out[pf.name] = {"by_m": by_m, "sample": f"layer 0, first {rows} rows of each projection at each M; "
                                            "scaled by weight count to 36 layers, extrapolated"}
    moe = synth.QWEN3_30B_A3B_Q4_MOE
    by_m = {}
    for m in moe.ms:
        spent, fl = 0.0, 0.0
        for pi, (name, k, n, per_pair) in enumerate(synth.moe_projs(moe)):
            a, ids, _ = synth.draw_moe_inputs(moe, m, pi)
            ws = [oracle.quantize(synth.draw_weight((moe.wid, e, pi, synth.STREAM_W), n, k), moe.bits)
                  for e in range(experts)]
            words = np.stack([oracle.pack(c, moe.bits) for c, _, _ in ws])
            s_ = np.stack([s for _, s, _ in ws])
            b_ = np.stack([b for _, _, b in ws])
            # exactly the pairs routed to the sampled experts, each as its
            # own one-slot token (row(p) = p), with its A row
            flat = ids.reshape(-1)
            sel = np.nonzero(flat < experts)[0]
            a_sub = a[sel] if per_pair else a[sel // moe.top_k]
            t0 = time.perf_counter()
            oracle.grouped_f64(words, s_, b_, a_sub, flat[sel][:, None].astype(np.int32), moe.bits, True)
            spent += time.perf_counter() - t0
            fl += 2.0 * m * moe.top_k * n * k
        t_full = spent * moe.experts / experts
        by_m[str(m)] = {"ms_per_step_extrapolated": round(t_full * 1e3, 1),
                        "tflops": round(fl / t_full / 1e12, 5), "sample_s": round(spent, 2)}
    out[moe.name] = {"by_m": by_m, "sample": f"gate, up and down over experts 0..{experts - 1} and the tokens "
                                             f"routed to them; x{moe.experts // experts} by expert count, "
                                             "extrapolated"}
    return {"kind": "oracle", **host_info(), "by_workload": out}


def dispatch_cost():
    """Host microseconds per call of each entry point, from the C++ harness
    (no Python in the loop); None if it was not built."""
    import subprocess
    exe = os.path.join(ROOT, "quantized_matmul_qgemv_amd", "qmm_dispatch_cost")
    if not os.path.exists(exe):
        return None
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        log("dispatch harness failed:", r.stderr.strip()[-500:])
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def python_dispatch_cost(torch, qmm, calls=200):
    """Host microseconds per call through the Python binding (ctypes
    marshalling + the C call) for qgemv and a batched GEMM launch."""
    wl = synth.SINGLE_Q4
    words, s, b, x, y, n, k = prepare_dense(torch, qmm, wl, 1)[0][0]
    X = torch.zeros((64, k), dtype=torch.float16, device="cuda")
    Y = torch.empty((64, n), dtype=torch.float32, device="cuda")
    plan = qmm.qgemm_batched_plan([(words, s, b, X, Y)], 4)
    out = {}
    for name, fn in (("qgemv", lambda: qmm.qgemv(words, s, b, x, 4, y=y)),
                     ("qgemm_batched", lambda: qmm.qgemm_batched(plan))):
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        reps = []
        for _ in range(5):
            t0 = time.perf_counter()
            for _ in range(calls):
                fn()
            reps.append((time.perf_counter() - t0) / calls * 1e6)
            torch.cuda.synchronize()
        out[name] = round(float(np.median(reps)), 3)
    return {"unit": "us host time per call", **out}


_PROFILE_CACHE = {}
PROFILE_LAYERS = 8


def profile_launch(torch, qmm, spec, reps):
    """One launch of the benchmark, repeated `reps` times, for profilers and
    tile sweeps: spec = "prefill:M:GROUP" (GROUP = qkv, o, gateup or down;
    the batched launch over tile-interleaved weights, rotating over the
    weights of PROFILE_LAYERS layers, 8 x 57 MB, so that every launch reads
    its weights from HBM as in a full prefill step rather than from the
    last-level cache) or "moe:M:PROJ" (PROJ = gate, up, down or swiglu;
    routed, over tile-interleaved weights, rotating over 3 copies of the
    expert weights for the same reason)."""
    kind, m, what = spec.split(":")
    m = int(m)
    stream = torch.cuda.current_stream()
    if kind == "prefill":
        wl = synth.QWEN3_4B_Q4_PREFILL
        wl1 = dataclasses.replace(wl, layers=PROFILE_LAYERS)
        if "prefill" not in _PROFILE_CACHE:
            _PROFILE_CACHE["prefill"] = prefill_layers(torch, qmm, wl1)
        layers = _PROFILE_CACHE["prefill"]
        if ("io", m) not in _PROFILE_CACHE:
            _PROFILE_CACHE[("io", m)] = prefill_io(torch, wl1, m)
        xs, ys = _PROFILE_CACHE[("io", m)]
        gi = {"qkv": 0, "o": 1, "gateup": 2, "down": 3}[what]
        plans = [pl[0] for pl in prefill_plans(qmm, wl1, layers, xs, ys, (PREFILL_GROUPS[gi],))]
        ms, _ = time_launches(torch, lambda i: qmm.qgemm_batched(plans[i % len(plans)]), reps, 2, stream)
        _, flops1 = prefill_work(dataclasses.replace(wl, layers=1, projs=tuple(
            p for p in wl.projs if p.name in PREFILL_GROUPS[gi])), m)
        h = plans[0].header
        return {"launch": spec, "ms_per_launch": round(ms, 5), "tflops": round(flops1 / (ms * 1e-3) / 1e12, 1),
                "tiles": "{bm}x{n}/S{splits}/K{kw}".format(n=h["nb"] * 128, **h)}
    wl = synth.QWEN3_30B_A3B_Q4_MOE
    if "moe" not in _PROFILE_CACHE:
        _PROFILE_CACHE["moe"] = moe_weights(torch, qmm, wl, 3)
    wsets = _PROFILE_CACHE["moe"]
    pi = {"gate": 0, "up": 1, "down": 2, "swiglu": 0}[what]
    a, ids, _ = synth.draw_moe_inputs(wl, m, pi)
    A, I = torch.from_numpy(a).cuda(), torch.from_numpy(ids).cuda()
    plan = qmm.moe_route(I, wl.experts)
    _, _, _, n, k, per_pair = wsets[0][pi]
    if what == "swiglu":
        H = torch.empty((m * wl.top_k, n), dtype=torch.float16, device="cuda")
        fn = lambda i: qmm.moe_gate_up_swiglu(wsets[i % 3][0][:3], wsets[i % 3][1][:3], A, I, plan, wl.bits,
                                              h=H, tiled=True, scales_tiled=PREFILL_SCALES_TILED)
        flops = 2 * 2.0 * m * wl.top_k * n * k
    else:
        Y = torch.empty((m * wl.top_k, n), dtype=torch.float32, device="cuda")
        fn = lambda i: qmm.qgemm_grouped(*wsets[i % 3][pi][:3], A, I, wl.bits, per_pair, y=Y, plan=plan, tiled=True,
                                         scales_tiled=PREFILL_SCALES_TILED)
        flops = 2.0 * m * wl.top_k * n * k
    ms, _ = time_launches(torch, fn, reps, 2, stream)
    return {"launch": spec, "ms_per_launch": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}


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
    ap.add_argument("--launch", metavar="SPEC",
                    help="run benchmark launches --steps times each and exit (for profilers): a "
                         "comma-separated list of prefill:M:{qkv,o,gateup,down} and moe:M:{gate,up,down,swiglu}")
    ap.add_argument("--ms", metavar="M[,M...]", help="prefill/moe: only these M")
    ap.add_argument("--decode-bits", type=int, choices=[2, 3, 4, 5, 6, 8, 16], default=4,
                    help="with --only decode: the decode pass at another weight width (for counters)")
    ap.add_argument("--row-major-scales", action="store_true",
                    help="prefill and MoE GEMMs read row-major scales and biases instead of the "
                         "interleaved copy (for comparisons)")
    ap.add_argument("--forces", metavar="F;F...",
                    help="with --launch: time every launch under each forced tile: QMM_GEMM_FORCE "
                         "for prefill launches (bm,nb,splits[,kw]), QMM_MOE_FORCE for moe launches "
                         "(bm,nb); empty = the planner's or the routing rule's choice")
    args = ap.parse_args()
    if args.row_major_scales:
        global PREFILL_SCALES_TILED, PREFILL_WEIGHTS
        PREFILL_SCALES_TILED = False
        PREFILL_WEIGHTS = "tile-interleaved copy (qmm_repack_tiled, once at load); row-major scales and biases"
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

    if args.launch:
        forces = args.forces.split(";") if args.forces else [None]
        for spec in args.launch.split(","):
            for f in forces:
                if f is not None:
                    var = "QMM_MOE_FORCE" if spec.startswith("moe") else "QMM_GEMM_FORCE"
                    if f:
                        os.environ[var] = f
                    else:
                        os.environ.pop(var, None)
                r = profile_launch(torch, qmm, spec, args.steps)
                if f is not None:
                    r["force"] = f
                print(json.dumps(r), flush=True)
        return

    if args.only in ("prefill", "moe"):
        if args.only == "prefill":
            ms = tuple(int(v) for v in args.ms.split(",")) if args.ms else synth.QWEN3_4B_Q4_PREFILL.ms
            by_m = bench_prefill(torch, qmm, ms)
            out = {"workload": synth.QWEN3_4B_Q4_PREFILL.name, "peak_tflops": FP16_MFMA_PEAK_TFLOPS,
                   "weights": PREFILL_WEIGHTS, "by_m": by_m, "prefill_roofline": prefill_roofline_block(by_m)}
        else:
            out = {"workload": synth.QWEN3_30B_A3B_Q4_MOE.name, "weights": PREFILL_WEIGHTS,
                   "by_m": bench_moe(torch, qmm)}
        print(json.dumps(out), flush=True)
        return

    wl = synth.QWEN3_0_6B_Q4_DECODE
    if args.decode_bits != wl.bits:
        if args.only != "decode":
            print("--decode-bits needs --only decode", file=sys.stderr)
            sys.exit(2)
        wl = dataclasses.replace(wl, bits=args.decode_bits, name=f"{wl.name}@q{args.decode_bits}")
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
                     "traffic": traffic if wl.bits == 4 else None,
                     "kernel": "qgemv_batched_kernel<4,16,4,64>" if wl.bits == 4 else "qgemv_batched_kernel",
                     "bytes_per_launch": d["step_bytes"],
                     "launch_ms_mean": round(d["ms_step"], 5)},
    }
    if args.only in ("all", "decode_extras"):
        log("decode extras")
        result["decode_context"] = bench_decode_extras(torch, qmm, wl, d["sets"])
        result["decode_context"]["host_dispatch_c"] = dispatch_cost()
        result["decode_context"]["host_dispatch_python"] = python_dispatch_cost(torch, qmm)
        result["decode_context"]["streaming_reference"] = bench_streaming_reference(torch, d["step_bytes"])
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
        by_m = bench_prefill(torch, qmm, synth.QWEN3_4B_Q4_PREFILL.ms)
        result["prefill_roofline"] = prefill_roofline_block(by_m)
        result["prefill"] = {"workload": synth.QWEN3_4B_Q4_PREFILL.name,
                             "peak_tflops": FP16_MFMA_PEAK_TFLOPS, "weights": PREFILL_WEIGHTS,
                             "by_m": by_m}
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
        if args.only == "all":
            log("cpu baseline, other workloads")
            result["cpu_baseline"]["other_workloads"] = cpu_baseline_configs()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
