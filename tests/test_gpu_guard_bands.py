"""Guard bands around every output of the hot path, on the GPU.

Each entry point writes into the middle of a buffer whose bytes start as a
sentinel (4 KiB on either side, and the output region itself), at ragged
shapes that leave partial tiles in every dimension: the sentinels on both
sides must survive, and the output must still match the oracle (bit-exact
for codes, dequantized values, quantizer output and repacked words; within
the stated tolerance for the products).  Covered: codes, dequant (fp32 and
fp16), quantizer words/scales/biases, tile-interleaved repack, bf16
conversion, GEMV, batched GEMV, GEMM and batched GEMM with their split-k
partial workspaces, the grouped GEMM with its bucket workspace, the routing
plan, the routed product, the fused SwiGLU output and the combine."""
import numpy as np
import pytest

import oracle
import synth
from qmm_testlib import Guarded, assert_close, dev, host, quantized, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import quantized_matmul_qgemv_amd as qmm  # noqa: E402


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_guard_codes_dequant_quantize(bits):
    say("guard codes/dequant/quantize", bits)
    n, k = 37, 320
    w, codes, words, s, b = quantized((970, bits), n, k, bits)
    W, S, B = dev(words), dev(s), dev(b)
    g = Guarded((n, k), torch.uint8)
    qmm.unpack_codes(W, k, bits, out=g.t)
    gd = Guarded((n, k), torch.float32)
    qmm.dequant(W, S, B, k, bits, out_f16=False, out=gd.t)
    gh = Guarded((n, k), torch.int16)
    qmm.dequant(W, S, B, k, bits, out_f16=True, out=gh.t)
    gw = Guarded(words.shape, torch.int32)
    gs_ = Guarded(s.shape, torch.int16)
    gb = Guarded(b.shape, torch.int16)
    qmm.quantize(torch.from_numpy(w).cuda(), bits, out=(gw.t, gs_.t, gb.t))
    torch.cuda.synchronize()
    for gg, what in ((g, "codes"), (gd, "dequant f32"), (gh, "dequant f16"), (gw, "words"),
                     (gs_, "scales"), (gb, "biases")):
        gg.check(what)
    assert np.array_equal(host(g.t), codes)
    exact = oracle.dequant_f64(codes, s, b)
    assert np.array_equal(host(gd.t), oracle.round_to_f32(exact))
    assert np.array_equal(host(gh.t).view(np.uint16), oracle.round_to_f16_bits(exact))
    assert np.array_equal(host(gw.t, np.uint32), words)
    assert np.array_equal(host(gs_.t).view(np.uint16), s) and np.array_equal(host(gb.t).view(np.uint16), b)


@pytest.mark.parametrize("bits", [3, 4, 16])
def test_guard_repack_and_bf16(bits):
    say("guard repack/bf16", bits)
    n, k = 96, 320
    r = np.random.default_rng([971, bits])
    words = r.integers(0, 2**32, size=(n, k * bits // 32), dtype=np.uint64).astype(np.uint32)
    g = Guarded(words.shape, torch.int32)
    qmm.repack_tiled(dev(words.view(np.int32)), bits, out=g.t)
    src = r.integers(0, 2**16, size=(33, 70), dtype=np.uint64).astype(np.uint16)
    gbf = Guarded((33, 35), torch.int32)
    qmm.convert_bf16(dev(src.view(np.int16)), out=gbf.t)
    torch.cuda.synchronize()
    g.check("repack")
    gbf.check("bf16")
    wpg = 2 * bits
    want = np.ascontiguousarray(words.reshape(n // 32, 32, k // 64, wpg).transpose(0, 2, 1, 3)).reshape(n, -1)
    assert np.array_equal(host(g.t, np.uint32), want)
    got16 = host(gbf.t, np.uint32).view(np.uint16).reshape(33, 70)
    w16 = oracle.bf16_to_f16_bits(src)
    isnan = ((w16 & 0x7C00) == 0x7C00) & ((w16 & 0x03FF) != 0)
    assert np.array_equal(got16[~isnan], w16[~isnan])


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_guard_gemv_and_batched(bits):
    say("guard gemv", bits)
    shapes = [(1, 64), (37, 192), (300, 1024), (513, 3072), (64, 8192)]
    probs, wants, guards = [], [], []
    for i, (n, k) in enumerate(shapes):
        _, _, words, s, b = quantized((972, bits, i), n, k, bits)
        x = synth.draw_act((972, bits, i, 1), 1, k)
        W, S, B, X = dev(words), dev(s), dev(b), dev(x[0])
        g = Guarded((n,), torch.float32)
        qmm.qgemv(W, S, B, X, bits, y=g.t)
        torch.cuda.synchronize()
        g.check(f"gemv n={n} k={k}")
        want = oracle.qmatmul_f64(words, s, b, x, bits)[0]
        assert_close(host(g.t), want, f"guarded gemv n={n} k={k}")
        gb = Guarded((n,), torch.float32)
        probs.append((W, S, B, X, gb.t))
        guards.append(gb)
        wants.append(want)
    qmm.qgemv_batched(qmm.qgemv_batched_plan(probs, bits))
    torch.cuda.synchronize()
    for g, want, (n, k) in zip(guards, wants, shapes):
        g.check(f"batched gemv n={n} k={k}")
        assert_close(host(g.t), want, f"guarded batched gemv n={n} k={k}")


@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("force", ["256,2,2", "128,2,3", "64,1,4", "32,2,1", "32,1,5",
                                   "128,1,1,2", "64,2,2,2", "64,1,2,2", "32,1,1,2"])
def test_guard_gemm_and_batched(bits, force, monkeypatch):
    """y and the split-k partial workspace of qmm_qgemm and of a batched
    plan, every tile family (one or two k halves per workgroup), with and
    without k split, at ragged m and n."""
    say("guard gemm", bits, force)
    shapes = [(70, 520, 1280), (300, 224, 768), (1, 64, 256)]
    monkeypatch.setenv("QMM_GEMM_FORCE", force)
    probs, wants, guards = [], [], []
    for i, (m, n, k) in enumerate(shapes):
        _, _, words, s, b = quantized((973, bits, i), n, k, bits)
        x = synth.draw_act((973, bits, i, 1), m, k)
        W, S, B, X = dev(words), dev(s), dev(b), dev(x)
        want = oracle.qmatmul_f64(words, s, b, x, bits)
        g = Guarded((m, n), torch.float32)
        wsz = qmm.qgemm_workspace_size(m, n, k, bits)
        gw = Guarded((max(wsz, 16),), torch.uint8)
        qmm.qgemm(W, S, B, X, bits, y=g.t, workspace=gw.t)
        torch.cuda.synchronize()
        g.check(f"gemm y m={m} n={n} k={k}")
        gw.check(f"gemm workspace m={m} n={n} k={k}")
        assert_close(host(g.t), want, f"guarded gemm {force} m={m} n={n} k={k}")
        gb = Guarded((m, n), torch.float32)
        probs.append((W, S, B, X, gb.t))
        guards.append(gb)
        wants.append(want)
    plan = qmm.qgemm_batched_plan(probs, bits)
    monkeypatch.delenv("QMM_GEMM_FORCE")
    gws = Guarded((plan.workspace.numel(),), torch.uint8)
    plan.workspace = gws.t
    qmm.qgemm_batched(plan)
    torch.cuda.synchronize()
    gws.check("batched workspace")
    for g, want, (m, n, k) in zip(guards, wants, shapes):
        g.check(f"batched gemm y m={m} n={n} k={k}")
        assert_close(host(g.t), want, f"guarded batched gemm {force} m={m} n={n} k={k}")


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("bm,nb", [(32, 2), (64, 1), (128, 2), (160, 1)])
def test_guard_moe(bits, bm, nb, monkeypatch):
    """Grouped GEMM y and bucket workspace, the routing plan, the routed
    product, the fused SwiGLU h and the combine y, on an expert mix with
    ragged buckets and ragged columns."""
    say("guard moe", bits, bm, nb)
    e, hidden, inter, t, top_k = 6, 192, 300, 75, 4
    r = np.random.default_rng([974, bits])
    ids = np.ascontiguousarray(synth.topk_ids(r.standard_normal((t, e)), top_k), dtype=np.int32)
    x = synth.draw_act((974, bits, 1), t, hidden)
    qs = [quantized((975, bits, i), inter, hidden, bits) for i in range(e)]
    gate = tuple(np.stack([q[j] for q in qs]) for j in (2, 3, 4))
    qs = [quantized((976, bits, i), inter, hidden, bits) for i in range(e)]
    up = tuple(np.stack([q[j] for q in qs]) for j in (2, 3, 4))
    G = tuple(dev(v) for v in gate)
    U = tuple(dev(v) for v in up)
    I, X = dev(ids), dev(x)
    pairs = t * top_k
    monkeypatch.setenv("QMM_MOE_FORCE", f"{bm},{nb}")
    gy = Guarded((pairs, inter), torch.float32)
    gws = Guarded((qmm.qgemm_grouped_workspace_size(t, top_k, e, inter, hidden, bits),), torch.uint8)
    qmm.qgemm_grouped(*G, X, I, bits, False, y=gy.t, workspace=gws.t)
    gplan = Guarded((qmm.moe_route_size(t, top_k, e),), torch.uint8)
    qmm.moe_route(I, e, plan=gplan.t)
    gy2 = Guarded((pairs, inter), torch.float32)
    qmm.qgemm_grouped(*G, X, I, bits, False, y=gy2.t, plan=gplan.t)
    gh = Guarded((pairs, inter), torch.float16)
    qmm.moe_gate_up_swiglu(G, U, X, I, gplan.t, bits, h=gh.t)
    torch.cuda.synchronize()
    monkeypatch.delenv("QMM_MOE_FORCE")
    for g, what in ((gy, "grouped y"), (gws, "grouped workspace"), (gplan, "routing plan"),
                    (gy2, "routed y"), (gh, "swiglu h")):
        g.check(what)
    want = oracle.grouped_f64(*gate, x, ids, bits, False)
    assert_close(host(gy.t), want, f"guarded grouped {bm}x{nb}")
    assert torch.equal(gy.t, gy2.t)
    assert_close(host(gh.t).astype(np.float64), oracle.moe_swiglu_f64(gate, up, x, ids, bits),
                 f"guarded swiglu {bm}x{nb}")
    wts = r.random((t, top_k)).astype(np.float32)
    gc = Guarded((t, inter), torch.float32)
    qmm.moe_combine(gy.t, torch.from_numpy(wts).cuda(), y=gc.t)
    torch.cuda.synchronize()
    gc.check("combine y")
    assert_close(host(gc.t), oracle.moe_combine_f64(host(gy.t), wts), "guarded combine")
