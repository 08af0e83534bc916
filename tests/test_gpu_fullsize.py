"""Parity at the workloads' full sizes, in the launch configuration that
bench.py times, on sampled outputs the oracle computes one by one.

Weights are quantized on the GPU here (as in the benchmark); the oracle
quantizes the sampled rows from the same seeded fp32 weights itself, so the
test also checks the GPU quantizer bit for bit at full size."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from qmm_testlib import assert_close, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bench  # noqa: E402
import quantized_matmul_qgemv_amd as qmm  # noqa: E402


def sample_rows(n, count, seed):
    r = np.random.default_rng(seed)
    rows = set(r.choice(n, size=min(count, n), replace=False).tolist())
    rows.update({0, n - 1})
    return np.array(sorted(rows))


def _decode_at(bits):
    """The Qwen3-0.6B-shaped decode pass with its weights at another width,
    as bench.py's decode_formats times it."""
    wl = synth.QWEN3_0_6B_Q4_DECODE
    return dataclasses.replace(wl, bits=bits, name=f"{wl.name}@q{bits}")


@pytest.mark.parametrize("wl", [synth.QWEN3_0_6B_Q4_DECODE, synth.LLAMA32_3B_Q8_DECODE] +
                         [_decode_at(b) for b in (2, 3, 5, 6)], ids=lambda w: w.name)
def test_decode_sweep_batched_sampled(wl):
    say("full decode sweep", wl.name)
    sets = bench.prepare_dense(torch, qmm, wl, 1)
    plan = qmm.qgemv_batched_plan([p[:5] for p in sets[0]], wl.bits)
    qmm.qgemv_batched(plan)
    torch.cuda.synchronize()
    probs = wl.problems()
    for idx, (layer, i, p) in enumerate(probs):
        # every projection of the first and the last layer, and the lm_head
        if layer not in (0, wl.layers - 1, wl.layers):
            continue
        words_d, s_d, b_d, x_d, y_d, n, k = sets[0][idx]
        rows = sample_rows(n, 48, idx)
        w_layer = wl.layers if i >= len(wl.projs) else 0
        w = synth.draw_weight((wl.wid, w_layer, i, synth.STREAM_W), n, k)[rows]
        codes, s, b = oracle.quantize(w, wl.bits)
        words = oracle.pack(codes, wl.bits)
        assert np.array_equal(host(words_d, np.uint32)[rows], words), (p.name, "codes")
        assert np.array_equal(host(s_d, np.uint16)[rows], s) and np.array_equal(host(b_d, np.uint16)[rows], b)
        x = synth.draw_act((wl.wid, layer, i, synth.STREAM_X), 1, k)
        want = oracle.qmatmul_f64(words, s, b, x, wl.bits)[0]
        assert_close(host(y_d)[rows], want, f"{wl.name} layer {layer} {p.name}")


@pytest.mark.parametrize("m", synth.QWEN3_4B_Q4_PREFILL.ms)
def test_prefill_layer_sampled(m):
    """One layer as bench.py runs it (q+k+v, o, gate+up, down as four batched
    launches with the planner's tiles and splits), and every projection
    again through the single-GEMM entry point."""
    wl = synth.QWEN3_4B_Q4_PREFILL
    names = [p.name for p in wl.projs]
    wfs, dev_w, xs, ys = [], [], [], []
    for i, p in enumerate(wl.projs):
        wf = synth.draw_weight((wl.wid, 0, i, synth.STREAM_W), p.n, p.k)
        wfs.append(wf)
        dev_w.append(qmm.quantize(torch.from_numpy(wf).cuda(), wl.bits))
        xs.append(synth.draw_act((wl.wid, m, i, synth.STREAM_X), m, p.k))
        ys.append(torch.full((m, p.n), float("nan"), dtype=torch.float32, device="cuda"))
    xd = [torch.from_numpy(x).cuda() for x in xs]
    for grp in bench.PREFILL_GROUPS:
        say("full prefill batched", m, "+".join(grp))
        plan = qmm.qgemm_batched_plan(
            [(*dev_w[names.index(nm)], xd[names.index(nm)], ys[names.index(nm)]) for nm in grp], wl.bits)
        qmm.qgemm_batched(plan)
    # as bench.py runs it: tile-interleaved weights, bit-identical outputs
    yt = [torch.full_like(y, float("nan")) for y in ys]
    wt = [qmm.repack_tiled(w[0], wl.bits) for w in dev_w]
    for grp in bench.PREFILL_GROUPS:
        say("full prefill batched tiled", m, "+".join(grp))
        idx = [names.index(nm) for nm in grp]
        plan = qmm.qgemm_batched_plan([(wt[i], dev_w[i][1], dev_w[i][2], xd[i], yt[i]) for i in idx],
                                      wl.bits, tiled=True)
        qmm.qgemm_batched(plan)
    torch.cuda.synchronize()
    for i, p in enumerate(wl.projs):
        assert torch.equal(yt[i], ys[i]), f"prefill m={m} {p.name}: tiled weights differ"
    for i, p in enumerate(wl.projs):
        say("full prefill single", m, p.name)
        y1 = qmm.qgemm(*dev_w[i], xd[i], wl.bits)
        torch.cuda.synchronize()
        cols = sample_rows(p.n, 32, 7 * m + i)
        rows = sample_rows(m, 32, 11 * m + i)
        codes, s, b = oracle.quantize(wfs[i][cols], wl.bits)
        want = oracle.qmatmul_f64(oracle.pack(codes, wl.bits), s, b, xs[i][rows], wl.bits)
        assert_close(host(ys[i])[np.ix_(rows, cols)], want, f"prefill batched m={m} {p.name}")
        assert_close(host(y1)[np.ix_(rows, cols)], want, f"prefill single m={m} {p.name}")
        assert not torch.isnan(ys[i]).any(), f"prefill batched m={m} {p.name}: unwritten outputs"


@pytest.mark.parametrize("m", synth.QWEN3_30B_A3B_Q4_MOE.ms)
def test_moe_sampled(m):
    wl = synth.QWEN3_30B_A3B_Q4_MOE
    for pi, (name, k, n, per_pair) in enumerate(synth.moe_projs(wl)):
        say("full moe", m, name)
        wf = synth.draw_expert_weights(wl, pi)                        # [E, n, k] fp32
        q = [qmm.quantize(torch.from_numpy(wf[e]).cuda(), wl.bits) for e in range(wl.experts)]
        W = torch.stack([t[0] for t in q])
        S = torch.stack([t[1] for t in q])
        B = torch.stack([t[2] for t in q])
        a, ids, logits = synth.draw_moe_inputs(wl, m, pi)
        y = qmm.qgemm_grouped(W, S, B, torch.from_numpy(a).cuda(), torch.from_numpy(ids).cuda(),
                              wl.bits, bool(per_pair))
        torch.cuda.synchronize()
        yh = host(y)
        r = np.random.default_rng(m + pi)
        pairs = r.choice(m * wl.top_k, size=24, replace=False)
        cols = sample_rows(n, 24, m + pi)
        for p in pairs:
            e = ids.flat[p]
            codes, s, b = oracle.quantize(wf[e][cols], wl.bits)
            row = a[p] if per_pair else a[p // wl.top_k]
            want = oracle.qmatmul_f64(oracle.pack(codes, wl.bits), s, b, row[None, :], wl.bits)[0]
            assert_close(yh[p, cols], want, f"moe m={m} {name} pair {p}")
        # routing from the oracle agrees with the ids the kernel was given
        ids_o, _ = oracle.route(logits[:64], wl.top_k)
        assert np.array_equal(ids_o, ids[:64])
        del W, S, B, q


_MOE_DEV = {}


def _moe_device_weights(wl):
    """Every expert of gate, up and down quantized on the GPU, as bench.py
    holds them (drawn once per test module)."""
    if not _MOE_DEV:
        for pi, (name, k, n, _) in enumerate(synth.moe_projs(wl)):
            ws, ss, bs = [], [], []
            for e in range(wl.experts):
                wf = torch.from_numpy(synth.draw_weight((wl.wid, e, pi, synth.STREAM_W), n, k)).cuda()
                w_, s_, b_ = qmm.quantize(wf, wl.bits)
                ws.append(w_); ss.append(s_); bs.append(b_)
            _MOE_DEV[name] = (torch.stack(ws), torch.stack(ss), torch.stack(bs))
    return _MOE_DEV


@pytest.mark.parametrize("m", synth.QWEN3_30B_A3B_Q4_MOE.ms)
def test_moe_ffn_block_sampled(m):
    """The FFN block as bench.py times it (routing plan, fused gate/up with
    SwiGLU to fp16 h, routed down from h, routing-weighted combine) on
    sampled tokens: h over all intermediate columns of each of the token's
    pairs, and the combined output on sampled hidden columns."""
    wl = synth.QWEN3_30B_A3B_Q4_MOE
    dw = _moe_device_weights(wl)
    x, ids, logits = synth.draw_moe_inputs(wl, m, 0)
    ids_o, wts = oracle.route(logits, wl.top_k)
    assert np.array_equal(ids_o, ids)
    say("full moe ffn block", m)
    I = torch.from_numpy(ids).cuda()
    plan = qmm.moe_route(I, wl.experts)
    h = qmm.moe_gate_up_swiglu(dw["gate"], dw["up"], torch.from_numpy(x).cuda(), I, plan, wl.bits)
    yd = qmm.qgemm_grouped(*dw["down"], h, I, wl.bits, True, plan=plan)
    y = qmm.moe_combine(yd, torch.from_numpy(wts.astype(np.float32)).cuda())
    # as bench.py runs it: tile-interleaved expert weights, bit-identical
    tw = {nm: (qmm.repack_tiled(dw[nm][0], wl.bits), dw[nm][1], dw[nm][2]) for nm in dw}
    h_t = qmm.moe_gate_up_swiglu(tw["gate"], tw["up"], torch.from_numpy(x).cuda(), I, plan, wl.bits,
                                 tiled=True)
    yd_t = qmm.qgemm_grouped(*tw["down"], h_t, I, wl.bits, True, plan=plan, tiled=True)
    torch.cuda.synchronize()
    assert torch.equal(h_t, h) and torch.equal(yd_t, yd), f"moe ffn m={m}: tiled weights differ"
    del tw, h_t, yd_t
    hh, yh = host(h), host(y)
    tokens = sorted({0, m - 1, int(np.random.default_rng(m).integers(1, m - 1))})
    cols = sample_rows(wl.hidden, 32, 5 * m)
    for t in tokens:
        y_pairs = np.zeros((wl.top_k, cols.size))
        for slot in range(wl.top_k):
            p, e = t * wl.top_k + slot, int(ids[t, slot])
            proj = {}
            for pi, name in ((0, "gate"), (1, "up")):
                wf = synth.draw_weight((wl.wid, e, pi, synth.STREAM_W), wl.inter, wl.hidden)
                codes, s, b = oracle.quantize(wf, wl.bits)
                proj[name] = oracle.qmatmul_f64(oracle.pack(codes, wl.bits), s, b, x[t][None, :], wl.bits)[0]
            h_want = oracle.silu_f64(proj["gate"]) * proj["up"]
            assert_close(hh[p].astype(np.float64), h_want, f"moe ffn m={m} h of pair {p}")
            wd = synth.draw_weight((wl.wid, e, 2, synth.STREAM_W), wl.hidden, wl.inter)[cols]
            codes, s, b = oracle.quantize(wd, wl.bits)
            y_pairs[slot] = oracle.qmatmul_f64(oracle.pack(codes, wl.bits), s, b,
                                               h_want.astype(np.float16)[None, :], wl.bits)[0]
        want = oracle.moe_combine_f64(y_pairs, wts[t:t + 1].astype(np.float32))[0]
        assert_close(yh[t, cols], want, f"moe ffn m={m} token {t}")
