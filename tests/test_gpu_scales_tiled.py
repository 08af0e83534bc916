"""Interleaved scales and biases (qmm_repack_scales_tiled, QMM_SCALES_TILED)
for the prefill GEMM over tile-interleaved weights: the repack is checked
word for word against the layout written out with numpy, and every GEMM
that reads it must equal the same call over row-major scales bit for bit
(only the addressing of the scale loads differs), and the oracle within
tolerance.  Covered: every quantized width, the quad scale loads and the
per-group loads (a k split whose ranges are not whole quads), the 256 x 256
tile, two k halves per workgroup, split k, several problems per plan, and
the grouped MoE calls and the fused gate/up SwiGLU over stacked experts."""
import numpy as np
import pytest

import oracle
import synth
from qmm_testlib import assert_close, dev, host, quantized, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import quantized_matmul_qgemv_amd as qmm  # noqa: E402

BITS = (2, 3, 4, 5, 6, 8)


def _tiled_scales(s, b):
    """The interleaved layout written out with numpy: for every 32-column
    block and quad of groups, the 32 columns' {s[4q..4q+3], b[4q..4q+3]}."""
    n, g = s.shape
    s4 = np.asarray(s).reshape(n // 32, 32, g // 4, 4).transpose(0, 2, 1, 3)
    b4 = np.asarray(b).reshape(n // 32, 32, g // 4, 4).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(np.concatenate([s4, b4], axis=3)).reshape(-1)


@pytest.mark.parametrize("n,k", [(32, 256), (96, 512), (224, 1024)])
def test_repack_scales_tiled_bit_exact(n, k):
    say("repack scales tiled", n, k)
    r = np.random.default_rng([970, n, k])
    s = r.integers(0, 2**16, size=(n, k // 64), dtype=np.uint16)
    b = r.integers(0, 2**16, size=(n, k // 64), dtype=np.uint16)
    got = qmm.repack_scales_tiled(dev(s.view(np.int16)), dev(b.view(np.int16)))
    torch.cuda.synchronize()
    assert np.array_equal(host(got).view(np.uint16), _tiled_scales(s, b))


@pytest.mark.parametrize("bits", BITS)
def test_gemm_scales_tiled_every_format(bits, monkeypatch):
    """qmm_qgemm and a one-problem batched plan over interleaved scales equal
    the calls over row-major scales bit for bit, for tiles that take the
    quad scale loads (128x256, 64x128 split 4, 256x256 split 2, 32x256) and
    ones whose split ranges are not whole quads (per-group scale loads:
    128x128 split 8, 64x128 split 16), and a two-half tile."""
    m, n, k = 150, 224, 1024
    _, _, words, s16, b16 = quantized((971, bits), n, k, bits)
    x = synth.draw_act((971, bits, 1), m, k)
    want = oracle.qmatmul_f64(words, s16, b16, x, bits)
    W, S, B, X = dev(words), dev(s16), dev(b16), dev(x)
    Wt = qmm.repack_tiled(W, bits)
    St = qmm.repack_scales_tiled(S, B)
    for force in ("128,2,1", "64,1,4", "256,2,2", "32,2,1", "128,1,8", "64,1,16", "64,1,2,2"):
        say("gemm scales tiled", bits, force)
        monkeypatch.setenv("QMM_GEMM_FORCE", force)
        single = force.count(",") == 2
        if single:
            y0 = qmm.qgemm(Wt, S, B, X, bits, tiled=True)
            y1 = qmm.qgemm(Wt, St, None, X, bits, tiled=True, scales_tiled=True)
        yb0 = torch.full((m, n), float("nan"), device="cuda")
        yb1 = torch.full((m, n), float("nan"), device="cuda")
        p0 = qmm.qgemm_batched_plan([(Wt, S, B, X, yb0)], bits, tiled=True)
        p1 = qmm.qgemm_batched_plan([(Wt, St, None, X, yb1)], bits, tiled=True, scales_tiled=True)
        monkeypatch.delenv("QMM_GEMM_FORCE")
        assert p1.header["stiled"] == 1 and p0.header["stiled"] == 0
        assert (p0.header["bm"], p0.header["splits"], p0.header["kw"]) == \
               (p1.header["bm"], p1.header["splits"], p1.header["kw"])
        qmm.qgemm_batched(p0)
        qmm.qgemm_batched(p1)
        torch.cuda.synchronize()
        if single:
            assert torch.equal(y0, y1), f"qgemm scales tiled differs: bits={bits} {force}"
            assert_close(host(y1), want, f"qgemm scales tiled bits={bits} {force}")
        assert torch.equal(yb0, yb1), f"batched scales tiled differs: bits={bits} {force}"
        assert_close(host(yb1), want, f"batched scales tiled bits={bits} {force}")


@pytest.mark.parametrize("force", [None, "64,2,3", "32,1,2,2", "128,2,1"])
def test_gemm_batched_scales_tiled_several_problems(force, monkeypatch):
    """A plan over three problems of different k (768, 2048 and 256: 12, 32
    and 4 groups) and an empty one, interleaved against row-major scales."""
    bits = 4
    shapes = [(70, 512, 768), (300, 224, 2048), (1, 64, 256), (0, 96, 512)]
    row, til, wants = [], [], []
    for i, (m, n, k) in enumerate(shapes):
        _, _, words, s16, b16 = quantized((972, i), n, k, bits)
        x = synth.draw_act((972, i, 1), m, k)
        wants.append(oracle.qmatmul_f64(words, s16, b16, x, bits) if m else None)
        W = qmm.repack_tiled(dev(words), bits)
        S, B = dev(s16), dev(b16)
        X = dev(x) if m else torch.zeros((0, k), dtype=torch.float16, device="cuda")
        row.append((W, S, B, X, torch.full((m, n), float("nan"), device="cuda")))
        til.append((W, qmm.repack_scales_tiled(S, B), None, X, torch.full((m, n), float("nan"), device="cuda")))
    say("gemm batched scales tiled", force)
    if force:
        monkeypatch.setenv("QMM_GEMM_FORCE", force)
    p0 = qmm.qgemm_batched_plan(row, bits, tiled=True)
    p1 = qmm.qgemm_batched_plan(til, bits, tiled=True, scales_tiled=True)
    if force:
        monkeypatch.delenv("QMM_GEMM_FORCE")
    qmm.qgemm_batched(p0)
    qmm.qgemm_batched(p1)
    torch.cuda.synchronize()
    for (m, n, k), a, c, want in zip(shapes, row, til, wants):
        assert torch.equal(a[4], c[4]), f"differs: {force} m={m} n={n} k={k}"
        if m:
            assert_close(host(c[4]), want, f"scales tiled {force} m={m} n={n} k={k}")


def _experts(key, e, n, k, bits):
    qs = [quantized(key + (ei,), n, k, bits) for ei in range(e)]
    return dev(np.stack([q[2] for q in qs])), dev(np.stack([q[3] for q in qs])), dev(np.stack([q[4] for q in qs]))


@pytest.mark.parametrize("bits", [4, 3, 8])
@pytest.mark.parametrize("bm,nb", [(32, 1), (64, 2), (64, 1), (128, 1), (160, 1), (None, None)])
def test_moe_scales_tiled(bits, bm, nb, monkeypatch):
    """Grouped GEMMs (self-bucketing, routed and allocation-free) and the
    fused gate/up SwiGLU over tile-interleaved expert weights with
    interleaved expert scales (the stacked [E, n, k/64] arrays repacked as
    one) equal the runs over row-major scales bit for bit, for every row
    tile, at k = 256 and 768.  Unforced (100 pairs per expert), the grouped
    GEMMs over interleaved scales take 64 x 256 tiles, and must equal the
    row-major run forced to that tile."""
    e, inter, t, top_k = 6, 320, 150, 4
    for hidden in (256, 768):
        say("moe scales tiled", bits, bm, nb, hidden)
        r = np.random.default_rng([973, bits, hidden])
        ids = np.ascontiguousarray(synth.topk_ids(r.standard_normal((t, e)), top_k), dtype=np.int32)
        x = dev(synth.draw_act((973, bits, hidden), t, hidden))
        gw, gs_, gb = _experts((974, bits, hidden), e, inter, hidden, bits)
        uw, us, ub = _experts((975, bits, hidden), e, inter, hidden, bits)
        gate = (qmm.repack_tiled(gw, bits), gs_, gb)
        up = (qmm.repack_tiled(uw, bits), us, ub)
        gate_s = (gate[0], qmm.repack_scales_tiled(gs_, gb), None)
        up_s = (up[0], qmm.repack_scales_tiled(us, ub), None)
        if bm is not None:
            monkeypatch.setenv("QMM_MOE_FORCE", f"{bm},{nb}")
        I = dev(ids)
        plan = qmm.moe_route(I, e)
        if bm is None:
            monkeypatch.setenv("QMM_MOE_FORCE", "64,2")
        y0 = qmm.qgemm_grouped(*gate, x, I, bits, False, plan=plan, tiled=True)
        if bm is None:
            monkeypatch.delenv("QMM_MOE_FORCE")
        y1 = qmm.qgemm_grouped(*gate_s, x, I, bits, False, plan=plan, tiled=True, scales_tiled=True)
        y2 = qmm.qgemm_grouped(*gate_s, x, I, bits, False, tiled=True, scales_tiled=True)
        y3 = torch.full_like(y0, float("nan"))
        qmm.qgemm_grouped_noalloc(*gate_s, x, I, bits, False, y3, tiled=True, scales_tiled=True)
        h0 = qmm.moe_gate_up_swiglu(gate, up, x, I, plan, bits, tiled=True)
        h1 = qmm.moe_gate_up_swiglu(gate_s, up_s, x, I, plan, bits, tiled=True, scales_tiled=True)
        torch.cuda.synchronize()
        monkeypatch.delenv("QMM_MOE_FORCE", raising=False)
        assert torch.equal(y0, y1) and torch.equal(y0, y2) and torch.equal(y0, y3), \
            f"grouped scales tiled differs bits={bits} {bm}x{nb} k={hidden}"
        assert torch.equal(h0, h1), f"swiglu scales tiled differs bits={bits} {bm}x{nb} k={hidden}"
        assert not torch.isnan(y0).any()
