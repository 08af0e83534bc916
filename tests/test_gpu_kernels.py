"""GPU parity of every kernel against the CPU oracle, through the C ABI, for
2-, 3-, 4-, 5-, 6- and 8-bit weights.

Bit-exact: code unpack, dequantization (fp32 and fp16) and the quantizer.
Within tolerance (relative L2 <= 1e-3, max |err| <= 1e-2 against float64):
GEMV, batched GEMV, GEMM and the grouped MoE GEMM, on shapes that span
several tiles with ragged tails, plus edge and degenerate cases."""
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


# ------------------------------------------------------------ bit-exact --

@pytest.mark.parametrize("bits", BITS)
def test_unpack_codes_bit_exact(bits):
    say("unpack", bits)
    r = np.random.default_rng(100 + bits)
    n, k = 37, 320
    codes = r.integers(0, 1 << bits, (n, k), dtype=np.uint8)
    codes[0] = (1 << bits) - 1
    codes[1] = 0
    words = oracle.pack(codes, bits)
    got = host(qmm.unpack_codes(dev(words), k, bits))
    torch.cuda.synchronize()
    assert np.array_equal(got, codes)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("f16", [False, True])
def test_dequant_bit_exact(bits, f16):
    say("dequant", bits, f16)
    w, codes, words, s, b = quantized((900, bits, 0, 0), 45, 256, bits)
    # add rows with extreme scale/bias: large, tiny and subnormal fp16 values
    extra = np.stack([np.linspace(-60000, 60000, 256), np.linspace(-1e-3, 1e-3, 256),
                      np.linspace(0, 2e-6, 256)]).astype(np.float32)
    c2, s2, b2 = oracle.quantize(extra, bits)
    codes = np.concatenate([codes, c2])
    s = np.concatenate([s, s2])
    b = np.concatenate([b, b2])
    words = oracle.pack(codes, bits)
    exact = oracle.dequant_f64(codes, s, b)
    got = host(qmm.dequant(dev(words), dev(s), dev(b), 256, bits, out_f16=f16))
    if f16:
        assert np.array_equal(got.view(np.uint16), oracle.round_to_f16_bits(exact))
    else:
        assert np.array_equal(got, oracle.round_to_f32(exact))


def quantize_cases():
    r = np.random.default_rng(7)
    rows = [synth.draw_weight((901, 0, 0, 0), 60, 512)]
    special = np.zeros((8, 512), dtype=np.float32)
    special[0] = (np.arange(512) % 16 / 64.0)                 # exact grid
    special[1, :64] = 0.3                                     # constant group
    special[2] = np.float32(0.3) + np.float32(1e-7) * np.arange(512, dtype=np.float32)
    special[3] = r.uniform(-1000, 1000, 512)                  # wide range
    special[4] = r.standard_normal(512) * 1e-5                # tiny values
    special[5, ::2] = 1.0
    special[6] = np.repeat([-1.0, 1.0], 256)
    special[7] = r.standard_normal(512).astype(np.float32) * 0.02
    special[7, 1:4] = np.array([0.5, 1.5, 2.5], dtype=np.float32) * (special[7, :64].max() -
                                                                    special[7, :64].min()) / 15
    rows.append(special.astype(np.float32))
    return np.concatenate(rows)


@pytest.mark.parametrize("bits", BITS)
def test_quantize_bit_exact(bits):
    say("quantize", bits)
    w = quantize_cases()
    codes, s, b = oracle.quantize(w, bits)
    words, gs, gb = qmm.quantize(dev(w), bits)
    assert np.array_equal(host(gs, np.uint16), s)
    assert np.array_equal(host(gb, np.uint16), b)
    assert np.array_equal(host(words, np.uint32), oracle.pack(codes, bits))


# ------------------------------------------------------------------ GEMV --

GEMV_SHAPES = [(1, 64), (3, 128), (37, 192), (100, 320), (1000, 1024), (1024, 1024),
               (300, 2048), (129, 2560), (513, 3072), (64, 8192), (7, 9728)]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("n,k", GEMV_SHAPES)
def test_gemv_parity(bits, n, k):
    say("gemv", bits, n, k)
    _, _, words, s, b = quantized((902, bits, n, k), n, k, bits)
    x = synth.draw_act((902, bits, n, 1), 1, k)
    want = oracle.qmatmul_f64(words, s, b, x, bits)[0]
    y = qmm.qgemv(dev(words), dev(s), dev(b), dev(x[0]), bits)
    assert_close(host(y), want, f"gemv bits={bits} n={n} k={k}")


def test_gemv_deterministic_and_overwrites():
    say("gemv determinism")
    n, k, bits = 777, 1024, 4
    _, _, words, s, b = quantized((903, 0, 0, 0), n, k, bits)
    x = dev(synth.draw_act((903, 0, 0, 1), 1, k)[0])
    y1 = torch.full((n,), float("nan"), device="cuda")
    y2 = torch.full((n,), 123.0, device="cuda")
    qmm.qgemv(dev(words), dev(s), dev(b), x, bits, y=y1)
    qmm.qgemv(dev(words), dev(s), dev(b), x, bits, y=y2)
    assert torch.equal(y1, y2)


def test_gemv_integer_closed_form():
    """Unit scale, zero bias and integer activations: the exact result is an
    integer matmul, representable in fp32, so the GPU must hit it exactly."""
    say("gemv integer")
    r = np.random.default_rng(5)
    for bits in BITS:
        n, k = 96, 512
        codes = r.integers(0, 1 << bits, (n, k), dtype=np.uint8)
        words = oracle.pack(codes, bits)
        s = np.full((n, k // 64), 0x3C00, dtype=np.uint16)
        b = np.zeros((n, k // 64), dtype=np.uint16)
        xi = r.integers(-4, 5, k)
        y = host(qmm.qgemv(dev(words), dev(s), dev(b), dev(xi.astype(np.float16)), bits))
        assert np.array_equal(y.astype(np.float64), (codes.astype(np.int64) @ xi).astype(np.float64))


@pytest.mark.parametrize("bits", BITS)
def test_gemv_batched_mixed_shapes(bits):
    say("gemv batched", bits)
    shapes = [(2048, 1024), (1024, 1024), (1024, 2048), (3072, 1024), (1024, 3072), (999, 1024)]
    probs, wants, ys = [], [], []
    for i, (n, k) in enumerate(shapes):
        _, _, words, s, b = quantized((904, i, 0, 0), n, k, bits)
        x = synth.draw_act((904, i, 0, 1), 1, k)
        y = torch.full((n,), float("nan"), device="cuda")
        probs.append((dev(words), dev(s), dev(b), dev(x[0]), y))
        wants.append(oracle.qmatmul_f64(words, s, b, x, bits)[0])
        ys.append(y)
    plan = qmm.qgemv_batched_plan(probs, bits)
    qmm.qgemv_batched(plan)
    for (n, k), y, want in zip(shapes, ys, wants):
        assert_close(host(y), want, f"batched n={n} k={k}")
    first = [y.clone() for y in ys]
    qmm.qgemv_batched(plan)
    for a, b in zip(first, ys):
        assert torch.equal(a, b)
    for (w, s, b, x, _), y in zip(probs, ys):
        single = qmm.qgemv(w, s, b, x, bits)
        assert_close(host(single), host(y), "single vs batched")


# ------------------------------------------------------------------ GEMM --

GEMM_SHAPES = [(1, 32, 64), (2, 100, 128), (3, 256, 192), (17, 300, 320), (33, 1024, 128),
               (64, 512, 256), (65, 96, 512), (127, 384, 256), (128, 1024, 2560),
               (129, 640, 512), (300, 1000, 1024), (513, 257, 640),
               # few tiles and long k: split over k with an ordered reduction
               (1, 4096, 4096), (16, 2048, 8192), (64, 4096, 4096), (200, 1024, 2560)]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
def test_gemm_parity(bits, m, n, k):
    say("gemm", bits, m, n, k)
    _, _, words, s, b = quantized((905, bits, n, k), n, k, bits)
    x = synth.draw_act((905, bits, m, 1), m, k)
    want = oracle.qmatmul_f64(words, s, b, x, bits)
    y = qmm.qgemm(dev(words), dev(s), dev(b), dev(x), bits)
    assert_close(host(y), want, f"gemm bits={bits} m={m} n={n} k={k}")


def test_gemm_split_k_workspace_and_determinism():
    say("gemm split-k")
    m, n, k, bits = 16, 2048, 8192, 4
    need = qmm.qgemm_workspace_size(m, n, k, bits)
    assert need >= 2 * m * n * 4, "this shape is expected to split k"
    _, _, words, s, b = quantized((911, 0, 0, 0), n, k, bits)
    x = synth.draw_act((911, 0, 0, 1), m, k)
    W, S, B, X = dev(words), dev(s), dev(b), dev(x)
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")   # garbage is fine
    y1 = qmm.qgemm(W, S, B, X, bits, workspace=ws)
    y2 = qmm.qgemm(W, S, B, X, bits, workspace=ws)
    assert torch.equal(y1, y2)
    assert_close(host(y1), oracle.qmatmul_f64(words, s, b, x, bits), "split-k")
    with pytest.raises(qmm.QmmError):
        qmm.qgemm(W, S, B, X, bits, workspace=ws[: need - 1])


# ---------------------------------------------------------- batched GEMM --

BATCH_SHAPES = [(70, 520, 1024), (33, 256, 256), (300, 200, 192), (1, 64, 64), (0, 128, 128),
                (257, 384, 512)]
BATCH_CFGS = [(256, 2), (128, 2), (128, 1), (64, 2), (64, 1), (32, 2), (32, 1)]


def _batch_inputs(bits, shapes, seed):
    ins, wants = [], []
    for i, (m, n, k) in enumerate(shapes):
        _, _, words, s, b = quantized((seed, bits, i, 0), n, k, bits)
        x = synth.draw_act((seed, bits, i, 1), m, k)
        wants.append(oracle.qmatmul_f64(words, s, b, x, bits) if m else np.zeros((0, n)))
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        ins.append((dev(words), dev(s), dev(b), dev(x) if m else torch.zeros((0, k), dtype=torch.float16, device="cuda"), y))
    return ins, wants


@pytest.mark.parametrize("bits", BITS)
def test_gemm_batched_parity(bits):
    say("gemm batched", bits)
    ins, wants = _batch_inputs(bits, BATCH_SHAPES, 921)
    plan = qmm.qgemm_batched_plan(ins, bits)
    qmm.qgemm_batched(plan)
    for (m, n, k), t, want in zip(BATCH_SHAPES, ins, wants):
        assert_close(host(t[4]), want, f"batched bits={bits} m={m} n={n} k={k} {plan.header}")


@pytest.mark.parametrize("bits", [4, 3, 5, 6])
@pytest.mark.parametrize("bm,nb", BATCH_CFGS)
@pytest.mark.parametrize("splits", [1, 3])
def test_gemm_batched_forced_tiles_and_split_k(bits, bm, nb, splits, monkeypatch):
    """Every tile shape, with and without k split: parity and identical
    results on a second call over a dirtied workspace."""
    say("gemm batched forced", bits, bm, nb, splits)
    shapes = [(70, 520, 1024), (300, 200, 768), (1, 64, 256)]
    ins, wants = _batch_inputs(bits, shapes, 922)
    monkeypatch.setenv("QMM_GEMM_FORCE", f"{bm},{nb},{splits}")
    plan = qmm.qgemm_batched_plan(ins, bits)
    monkeypatch.delenv("QMM_GEMM_FORCE")
    h = plan.header
    assert (h["bm"], h["nb"], h["splits"]) == (bm, nb, splits), h
    qmm.qgemm_batched(plan)
    first = [t[4].clone() for t in ins]
    for (m, n, k), y, want in zip(shapes, first, wants):
        assert_close(host(y), want, f"forced {bm}x{nb} S={splits} m={m} n={n} k={k}")
    for t in ins:
        t[4].fill_(float("nan"))
    plan.workspace.fill_(0xAB)
    qmm.qgemm_batched(plan)
    torch.cuda.synchronize()
    for y0, t in zip(first, ins):
        assert torch.equal(y0, t[4])


BATCH_KW_CFGS = [(128, 1), (64, 2), (64, 1), (32, 1)]


@pytest.mark.parametrize("bits", [4, 3, 8])
@pytest.mark.parametrize("bm,nb", BATCH_KW_CFGS)
@pytest.mark.parametrize("splits", [1, 3])
def test_gemm_batched_two_k_halves(bits, bm, nb, splits, monkeypatch):
    """Tiles whose 8 waves split each record's k range in two halves that
    meet in LDS: parity, identical results on a second call, and the same
    result over tile-interleaved weights.  k = 256 with quad scale loads
    leaves the second half empty; k = 768 splits its 12 groups 8 + 4."""
    say("gemm batched two k halves", bits, bm, nb, splits)
    shapes = [(70, 512, 1024), (300, 224, 768), (33, 96, 512)] + ([(1, 64, 256)] if splits == 1 else [])
    ins, wants = _batch_inputs(bits, shapes, 923)
    monkeypatch.setenv("QMM_GEMM_FORCE", f"{bm},{nb},{splits},2")
    plan = qmm.qgemm_batched_plan(ins, bits)
    tiled = [(qmm.repack_tiled(w, bits), s_, b_, x, torch.full_like(y, float("nan")))
             for (w, s_, b_, x, y) in ins]
    plan_t = qmm.qgemm_batched_plan(tiled, bits, tiled=True)
    monkeypatch.delenv("QMM_GEMM_FORCE")
    h = plan.header
    assert (h["bm"], h["nb"], h["splits"], h["kw"]) == (bm, nb, splits, 2), h
    qmm.qgemm_batched(plan)
    first = [t[4].clone() for t in ins]
    for (m, n, k), y, want in zip(shapes, first, wants):
        assert_close(host(y), want, f"two halves {bm}x{nb} S={splits} m={m} n={n} k={k}")
    for t in ins:
        t[4].fill_(float("nan"))
    plan.workspace.fill_(0xAB)
    qmm.qgemm_batched(plan)
    torch.cuda.synchronize()
    for y0, t in zip(first, ins):
        assert torch.equal(y0, t[4])
    assert plan_t.header["kw"] == 2
    qmm.qgemm_batched(plan_t)
    torch.cuda.synchronize()
    for (m, n, k), y0, t1 in zip(shapes, first, tiled):
        assert torch.equal(y0, t1[4]), f"tiled differs: {bm}x{nb} S={splits} m={m} k={k}"


def _tiled_words(words, n, k, bits):
    """The tile-interleaved layout written out with numpy: group g of
    column c goes to ((c // 32) * G * 32 + g * 32 + c % 32) * WPG."""
    g, wpg = k // 64, 2 * bits
    w = np.asarray(words, dtype=np.uint32).reshape(n // 32, 32, g, wpg)
    return np.ascontiguousarray(w.transpose(0, 2, 1, 3)).reshape(n, g * wpg)


@pytest.mark.parametrize("bits", [4, 3, 8, 16])
def test_repack_tiled_bit_exact(bits):
    say("repack tiled", bits)
    n, k = 96, 320
    r = np.random.default_rng([960, bits])
    words = r.integers(0, 2**32, size=(n, k * bits // 32), dtype=np.uint64).astype(np.uint32)
    got = qmm.repack_tiled(dev(words.view(np.int32)), bits)
    assert np.array_equal(host(got, np.uint32), _tiled_words(words, n, k, bits))


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("bm,nb", BATCH_CFGS)
@pytest.mark.parametrize("splits", [1, 3])
def test_gemm_batched_tiled_weights(bits, bm, nb, splits, monkeypatch):
    """Batched GEMM over tile-interleaved weights: bit-identical to the same
    plan over row-major weights (only the addressing differs), and within
    tolerance of the oracle."""
    say("gemm batched tiled", bits, bm, nb, splits)
    shapes = [(70, 512, 1024), (300, 224, 768), (1, 64, 256)]
    ins, wants = _batch_inputs(bits, shapes, 961)
    tiled = [(qmm.repack_tiled(w, bits), s_, b_, x, torch.full_like(y, float("nan")))
             for (w, s_, b_, x, y) in ins]
    monkeypatch.setenv("QMM_GEMM_FORCE", f"{bm},{nb},{splits}")
    plan = qmm.qgemm_batched_plan(ins, bits)
    plan_t = qmm.qgemm_batched_plan(tiled, bits, tiled=True)
    monkeypatch.delenv("QMM_GEMM_FORCE")
    assert plan_t.header["wtiled"] == 1 and plan.header["wtiled"] == 0
    assert (plan_t.header["bm"], plan_t.header["nb"], plan_t.header["splits"]) == (bm, nb, splits)
    qmm.qgemm_batched(plan)
    qmm.qgemm_batched(plan_t)
    torch.cuda.synchronize()
    for (m, n, k), t0, t1, want in zip(shapes, ins, tiled, wants):
        assert torch.equal(t0[4], t1[4]), f"tiled differs from row-major: {bm}x{nb} S={splits} m={m}"
        assert_close(host(t1[4]), want, f"tiled {bm}x{nb} S={splits} m={m} n={n} k={k}")


@pytest.mark.parametrize("bits", [4, 16])
@pytest.mark.parametrize("force", ["256,2,2", "128,2,1", "128,1,4", "64,1,1", "32,2,2"])
def test_gemm_tiled_weights(bits, force, monkeypatch):
    """qmm_qgemm over tile-interleaved weights is bit-identical to the
    row-major call (every tile family, with and without k split)."""
    say("gemm tiled", bits, force)
    m, n, k = 300, 224, 1024
    if bits == 16:
        w = dev(fp16_weight((965, 0), n, k)[1])
        s_ = b_ = None
    else:
        _, _, words, s16, b16 = quantized((965, bits), n, k, bits)
        w, s_, b_ = dev(words), dev(s16), dev(b16)
    x = dev(synth.draw_act((965, 1), m, k))
    wt = qmm.repack_tiled(w, bits)
    monkeypatch.setenv("QMM_GEMM_FORCE", force)
    y0 = qmm.qgemm(w, s_, b_, x, bits)
    y1 = qmm.qgemm(wt, s_, b_, x, bits, tiled=True)
    torch.cuda.synchronize()
    monkeypatch.delenv("QMM_GEMM_FORCE")
    assert torch.equal(y0, y1), force


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("gs", [32, 64, 128])
def test_gemm_tiled_every_format(bits, gs, monkeypatch):
    """Tile-interleaved weights for every width and scale-group size (the
    6-bit 8-byte and 8-bit 32-byte half-group loads, and the scale index of
    groups of 32 and 128 under the tiled group stride): qmm_qgemm and a
    batched plan over the repacked words are bit-identical to the row-major
    calls with the same tile and split, and within tolerance of the oracle."""
    m, n, k = 150, 224, 1024
    w32, _, words, s16, b16 = quantized_gs((966, bits, gs), n, k, bits, gs)
    x = synth.draw_act((966, bits, gs, 1), m, k)
    want = oracle.qmatmul_f64(words, s16, b16, x, bits, gs)
    W, S, B, X = dev(words), dev(s16), dev(b16), dev(x)
    Wt = qmm.repack_tiled(W, bits)
    for force in ("128,2,1", "64,1,4", "256,2,2", "32,2,1"):
        say("gemm tiled format", bits, gs, force)
        monkeypatch.setenv("QMM_GEMM_FORCE", force)
        y0 = qmm.qgemm(W, S, B, X, bits, group_size=gs)
        y1 = qmm.qgemm(Wt, S, B, X, bits, group_size=gs, tiled=True)
        yb0 = torch.full((m, n), float("nan"), device="cuda")
        yb1 = torch.full((m, n), float("nan"), device="cuda")
        p0 = qmm.qgemm_batched_plan([(W, S, B, X, yb0)], bits, group_size=gs)
        p1 = qmm.qgemm_batched_plan([(Wt, S, B, X, yb1)], bits, group_size=gs, tiled=True)
        monkeypatch.delenv("QMM_GEMM_FORCE")
        qmm.qgemm_batched(p0)
        qmm.qgemm_batched(p1)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1), f"qgemm tiled differs: bits={bits} gs={gs} {force}"
        assert torch.equal(yb0, yb1), f"batched tiled differs: bits={bits} gs={gs} {force}"
        assert_close(host(y1), want, f"qgemm tiled bits={bits} gs={gs} {force}")
        assert_close(host(yb1), want, f"batched tiled bits={bits} gs={gs} {force}")


@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_unaligned_scales_take_per_group_path(bits, monkeypatch):
    """Scales and biases that are 2-byte but not 8-byte aligned (a slice at
    an odd fp16 offset) make the GEMMs load the scales group by group: the
    plan records sbq = 0 and the products equal the aligned run bit for bit."""
    say("gemm unaligned scales", bits)
    m, n, k = 200, 256, 2048
    _, _, words, s16, b16 = quantized((967, bits), n, k, bits)
    x = dev(synth.draw_act((967, bits, 1), m, k))
    W = dev(words)
    S, B = dev(s16), dev(b16)
    flat_s = torch.empty(S.numel() + 1, dtype=S.dtype, device="cuda")
    flat_b = torch.empty(B.numel() + 3, dtype=B.dtype, device="cuda")
    Su = flat_s[1:].view(S.shape)
    Bu = flat_b[3:].view(B.shape)
    Su.copy_(S)
    Bu.copy_(B)
    assert Su.data_ptr() % 8 and Bu.data_ptr() % 8
    y0 = qmm.qgemm(W, S, B, x, bits)
    y1 = qmm.qgemm(W, Su, Bu, x, bits)
    ya = torch.empty((m, n), device="cuda")
    yu = torch.empty((m, n), device="cuda")
    monkeypatch.setenv("QMM_GEMM_FORCE", "128,2,1")
    pa = qmm.qgemm_batched_plan([(W, S, B, x, ya)], bits)
    pu = qmm.qgemm_batched_plan([(W, Su, Bu, x, yu)], bits)
    monkeypatch.delenv("QMM_GEMM_FORCE")
    assert pa.header["sbq"] == 1 and pu.header["sbq"] == 0
    qmm.qgemm_batched(pa)
    qmm.qgemm_batched(pu)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert torch.equal(ya, yu)
    assert_close(host(y1), oracle.qmatmul_f64(words, s16, b16, host(x), bits), "unaligned scales")


def test_gemm_rows_equal_gemv_and_deterministic():
    say("gemm rows")
    m, n, k, bits = 70, 520, 1024, 4
    _, _, words, s, b = quantized((906, 0, 0, 0), n, k, bits)
    x = synth.draw_act((906, 0, 0, 1), m, k)
    W, S, B, X = dev(words), dev(s), dev(b), dev(x)
    y = qmm.qgemm(W, S, B, X, bits)
    y2 = qmm.qgemm(W, S, B, X, bits)
    assert torch.equal(y, y2)
    for row in (0, 31, 32, 69):
        g = qmm.qgemv(W, S, B, X[row].contiguous(), bits)
        assert_close(host(y[row]), host(g), f"row {row}")


# --------------------------------------------------------------- grouped --

def grouped_inputs(key, e, n, k, bits, t, top_k, ids=None):
    r = np.random.default_rng(list(key))
    ws = [quantized(key + (ei,), n, k, bits) for ei in range(e)]
    words = np.stack([q[2] for q in ws])
    s = np.stack([q[3] for q in ws])
    b = np.stack([q[4] for q in ws])
    if ids is None:
        ids = synth.topk_ids(r.standard_normal((t, e)), top_k)
    x = synth.draw_act(key + (1000,), t, k)
    h = synth.draw_act(key + (1001,), t * top_k, k)
    return words, s, b, np.ascontiguousarray(ids, dtype=np.int32), x, h


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("e,n,k,t,top_k", [(8, 96, 128, 37, 3), (16, 300, 256, 100, 4),
                                           (128, 64, 128, 512, 8), (5, 520, 640, 64, 2)])
def test_grouped_parity(bits, e, n, k, t, top_k):
    say("grouped", bits, e, n, k, t, top_k)
    words, s, b, ids, x, h = grouped_inputs((907, bits, e, n), e, n, k, bits, t, top_k)
    W, S, B, I = dev(words), dev(s), dev(b), dev(ids)
    for per_pair, a in ((False, x), (True, h)):
        want = oracle.grouped_f64(words, s, b, a, ids, bits, per_pair)
        y = qmm.qgemm_grouped(W, S, B, dev(a), I, bits, per_pair)
        assert_close(host(y), want, f"grouped per_pair={per_pair}")


def test_grouped_edge_cases():
    bits, e, n, k, t, top_k = 4, 6, 200, 192, 50, 2
    cases = {
        "all on one expert": np.tile(np.array([[3, 3]]), (t, 1)),
        "unused experts": np.stack([np.array([0, 5])] * t),
        "skewed": np.stack([[i % 2, 2 + (i % 3 == 0)] for i in range(t)]),
    }
    for name, ids in cases.items():
        say("grouped edge", name)
        words, s, b, ids, x, h = grouped_inputs((908, 0, 0, 0), e, n, k, bits, t, top_k, ids=ids)
        want = oracle.grouped_f64(words, s, b, x, ids, bits, False)
        y = qmm.qgemm_grouped(dev(words), dev(s), dev(b), dev(x), dev(ids), bits, False)
        assert_close(host(y), want, name)
    # a single expert equals the dense GEMM, bit for bit (same tile core)
    say("grouped E=1")
    words, s, b, ids, x, h = grouped_inputs((909, 0, 0, 0), 1, n, k, bits, 64, 1,
                                            ids=np.zeros((64, 1)))
    y = qmm.qgemm_grouped(dev(words), dev(s), dev(b), dev(x), dev(ids), bits, False)
    want = oracle.qmatmul_f64(words[0], s[0], b[0], x, bits)
    assert_close(host(y), want, "E=1")
    # determinism across runs
    words, s, b, ids, x, h = grouped_inputs((910, 0, 0, 0), 16, 256, 256, bits, 200, 4)
    args = (dev(words), dev(s), dev(b), dev(h), dev(ids), bits, True)
    assert torch.equal(qmm.qgemm_grouped(*args), qmm.qgemm_grouped(*args))
    # zero tokens: nothing launched, output untouched
    y = torch.full((0, 256), 1.0, device="cuda")
    qmm.qgemm_grouped(dev(words), dev(s), dev(b), dev(h[:0]), dev(ids[:0]), bits, True, y=y)


# ----------------------------------------------------------- group sizes --

GROUP_SIZES = (32, 128)


def quantized_gs(key, n, k, bits, gs):
    w = synth.draw_weight(key, n, k)
    codes, s, b = oracle.quantize(w, bits, gs)
    return w, codes, oracle.pack(codes, bits), s, b


@pytest.mark.parametrize("gs", GROUP_SIZES)
@pytest.mark.parametrize("bits", BITS)
def test_group_size_quantize_dequant_bit_exact(bits, gs):
    say("group size quantize/dequant", bits, gs)
    w = synth.draw_weight((930, bits, gs, 0), 37, 512)
    w[0, :gs] *= 1000.0   # a wide group next to narrow ones
    w[1] = 0.25           # constant row: zero scale
    codes, s, b = oracle.quantize(w, bits, gs)
    words, gsc, gbi = qmm.quantize(dev(w), bits, group_size=gs)
    assert np.array_equal(host(gsc, np.uint16), s)
    assert np.array_equal(host(gbi, np.uint16), b)
    assert np.array_equal(host(words, np.uint32), oracle.pack(codes, bits))
    exact = oracle.dequant_f64(codes, s, b, gs)
    got = host(qmm.dequant(words, dev(s), dev(b), 512, bits, out_f16=False, group_size=gs))
    assert np.array_equal(got, oracle.round_to_f32(exact))
    got = host(qmm.dequant(words, dev(s), dev(b), 512, bits, out_f16=True, group_size=gs))
    assert np.array_equal(got.view(np.uint16), oracle.round_to_f16_bits(exact))


@pytest.mark.parametrize("gs", GROUP_SIZES)
@pytest.mark.parametrize("bits", BITS)
def test_group_size_gemv_and_gemm(bits, gs):
    say("group size gemv/gemm", bits, gs)
    for n, k in ((1, 128), (300, 512), (1024, 1024), (64, 8192)):
        _, _, words, s, b = quantized_gs((931, bits, gs, n), n, k, bits, gs)
        x = synth.draw_act((931, bits, gs, n + 1), 1, k)
        want = oracle.qmatmul_f64(words, s, b, x, bits, gs)[0]
        y = qmm.qgemv(dev(words), dev(s), dev(b), dev(x[0]), bits, group_size=gs)
        assert_close(host(y), want, f"gemv bits={bits} gs={gs} n={n} k={k}")
    probs, wants = [], []
    for i, (n, k) in enumerate(((2048, 1024), (999, 3072), (4096, 512))):
        _, _, words, s, b = quantized_gs((932, bits, gs, i), n, k, bits, gs)
        x = synth.draw_act((932, bits, gs, i + 10), 1, k)
        probs.append((dev(words), dev(s), dev(b), dev(x[0]), torch.full((n,), float("nan"), device="cuda")))
        wants.append(oracle.qmatmul_f64(words, s, b, x, bits, gs)[0])
    qmm.qgemv_batched(qmm.qgemv_batched_plan(probs, bits, group_size=gs))
    for t, want in zip(probs, wants):
        assert_close(host(t[4]), want, f"batched gemv bits={bits} gs={gs}")
    for m, n, k in ((1, 32, 128), (70, 520, 1024), (300, 1000, 1024), (16, 2048, 8192)):
        _, _, words, s, b = quantized_gs((933, bits, gs, m), n, k, bits, gs)
        x = synth.draw_act((933, bits, gs, m + 1), m, k)
        want = oracle.qmatmul_f64(words, s, b, x, bits, gs)
        y = qmm.qgemm(dev(words), dev(s), dev(b), dev(x), bits, group_size=gs)
        assert_close(host(y), want, f"gemm bits={bits} gs={gs} m={m} n={n} k={k}")


@pytest.mark.parametrize("gs", GROUP_SIZES)
@pytest.mark.parametrize("bits", [3, 4, 8])
def test_group_size_batched_gemm_every_tile(bits, gs, monkeypatch):
    shapes = [(70, 520, 1024), (300, 200, 768 if gs == 32 else 896), (1, 64, 256)]
    ins, wants = [], []
    for i, (m, n, k) in enumerate(shapes):
        _, _, words, s, b = quantized_gs((934, bits, gs, i), n, k, bits, gs)
        x = synth.draw_act((934, bits, gs, i + 10), m, k)
        wants.append(oracle.qmatmul_f64(words, s, b, x, bits, gs))
        ins.append((dev(words), dev(s), dev(b), dev(x), torch.full((m, n), float("nan"), device="cuda")))
    for bm, nb, kw in [(bm, nb, 1) for bm, nb in BATCH_CFGS] + [(bm, nb, 2) for bm, nb in BATCH_KW_CFGS]:
        for splits in ((1, 3) if kw == 1 else (1, 2)):  # k = 256 has 4 groups: at most 2 x 2
            say("group size batched", bits, gs, bm, nb, splits, kw)
            monkeypatch.setenv("QMM_GEMM_FORCE", f"{bm},{nb},{splits},{kw}")
            plan = qmm.qgemm_batched_plan(ins, bits, group_size=gs)
            monkeypatch.delenv("QMM_GEMM_FORCE")
            assert (plan.header["bm"], plan.header["nb"], plan.header["splits"], plan.header["kw"]) == \
                (bm, nb, splits, kw)
            assert plan.header["sbq"] == 0
            qmm.qgemm_batched(plan)
            for (m, n, k), t, want in zip(shapes, ins, wants):
                assert_close(host(t[4]), want, f"batched bits={bits} gs={gs} {bm}x{nb} S={splits} m={m}")
                t[4].fill_(float("nan"))


@pytest.mark.parametrize("gs", GROUP_SIZES)
@pytest.mark.parametrize("bits", [3, 4, 8])
def test_group_size_grouped(bits, gs):
    say("group size grouped", bits, gs)
    e, n, k, t, top_k = 16, 300, 256, 100, 4
    r = np.random.default_rng([935, bits, gs])
    ws = [quantized_gs((935, bits, gs, ei), n, k, bits, gs) for ei in range(e)]
    words = np.stack([q[2] for q in ws])
    s = np.stack([q[3] for q in ws])
    b = np.stack([q[4] for q in ws])
    ids = np.ascontiguousarray(synth.topk_ids(r.standard_normal((t, e)), top_k), dtype=np.int32)
    x = synth.draw_act((935, bits, gs, 1000), t, k)
    want = oracle.grouped_f64(words, s, b, x, ids, bits, False, gs)
    y = qmm.qgemm_grouped(dev(words), dev(s), dev(b), dev(x), dev(ids), bits, False, group_size=gs)
    assert_close(host(y), want, f"grouped bits={bits} gs={gs}")


# --------------------------------------------- unquantized fp16 weights --

def fp16_weight(key, n, k):
    """Seeded N(0, 0.02) weights rounded to fp16: (bit patterns [n, k] uint16,
    packed words [n, k/2] uint32 with the lower-k half in the low bits)."""
    w16 = synth.draw_weight(key, n, k).astype(np.float16).view(np.uint16)
    return w16, np.ascontiguousarray(w16).view(np.uint32)


def test_fp16_weights_gemv():
    for n, k in ((1, 64), (37, 192), (1000, 1024), (300, 2048), (513, 3072), (64, 8192)):
        say("fp16 gemv", n, k)
        w16, words = fp16_weight((940, n, k), n, k)
        x = synth.draw_act((940, n, k + 1), 1, k)
        y = qmm.qgemv(dev(words), None, None, dev(x[0]), 16)
        assert_close(host(y), oracle.hmatmul_f64(w16, x)[0], f"fp16 gemv n={n} k={k}")
    say("fp16 gemv batched")
    probs, wants = [], []
    for i, (n, k) in enumerate(((2048, 1024), (1024, 3072), (999, 1024))):
        w16, words = fp16_weight((941, i, n), n, k)
        x = synth.draw_act((941, i, n + 1), 1, k)
        probs.append((dev(words), None, None, dev(x[0]), torch.full((n,), float("nan"), device="cuda")))
        wants.append(oracle.hmatmul_f64(w16, x)[0])
    qmm.qgemv_batched(qmm.qgemv_batched_plan(probs, 16))
    for t, want in zip(probs, wants):
        assert_close(host(t[4]), want, "fp16 batched gemv")


@pytest.mark.parametrize("bits", [4, 8, 16])
def test_gemv_split_lanes_every_lane_count(bits):
    """The split-group lanes (a lane reads a half, quarter or eighth of two,
    four or eight groups per step and partner lanes join the parts) at every
    lanes-per-row count they apply to: k = 128, 256, 512, 1024 and 2560 give
    2, 4, 8, 16 and 8 lanes per row (fewer lanes than parts per group fall
    back to whole groups), with and without the in-workgroup k split (small
    n), single and batched launches."""
    shapes = [(3, 128), (5, 256), (33, 512), (130, 1024), (7, 2560), (600, 256), (41, 8192)]
    probs, wants = [], []
    for i, (n, k) in enumerate(shapes):
        say("gemv split lanes", bits, n, k)
        x = synth.draw_act((944, bits, i), 1, k)
        if bits == 16:
            w16, words = fp16_weight((943, i, n), n, k)
            W, S, B = dev(words), None, None
            want = oracle.hmatmul_f64(w16, x)[0]
        else:
            _, _, words, s16, b16 = quantized((943, bits, i), n, k, bits)
            W, S, B = dev(words), dev(s16), dev(b16)
            want = oracle.qmatmul_f64(words, s16, b16, x, bits)[0]
        y = qmm.qgemv(W, S, B, dev(x[0]), bits)
        assert_close(host(y), want, f"split lanes bits={bits} n={n} k={k}")
        probs.append((W, S, B, dev(x[0]), torch.full((n,), float("nan"), device="cuda")))
        wants.append(want)
    qmm.qgemv_batched(qmm.qgemv_batched_plan(probs, bits))
    for (n, k), t, want in zip(shapes, probs, wants):
        assert_close(host(t[4]), want, f"split lanes batched bits={bits} n={n} k={k}")


def test_fp16_weights_gemm(monkeypatch):
    for m, n, k in ((1, 32, 64), (17, 300, 320), (128, 1024, 2560), (300, 1000, 1024), (16, 2048, 8192)):
        say("fp16 gemm", m, n, k)
        w16, words = fp16_weight((942, m, n), n, k)
        x = synth.draw_act((942, m, n + 1), m, k)
        y = qmm.qgemm(dev(words), None, None, dev(x), 16)
        assert_close(host(y), oracle.hmatmul_f64(w16, x), f"fp16 gemm m={m} n={n} k={k}")
    shapes = [(70, 520, 1024), (300, 200, 768), (1, 64, 256)]
    ins, wants = [], []
    for i, (m, n, k) in enumerate(shapes):
        w16, words = fp16_weight((943, i, n), n, k)
        x = synth.draw_act((943, i, n + 1), m, k)
        wants.append(oracle.hmatmul_f64(w16, x))
        ins.append((dev(words), None, None, dev(x), torch.full((m, n), float("nan"), device="cuda")))
    plan = qmm.qgemm_batched_plan(ins, 16)
    assert plan.header["nb"] == 1 and plan.header["sbq"] == 0
    for bm in (128, 64, 32):
        for splits, kw in ((1, 1), (3, 1), (1, 2), (2, 2)):
            say("fp16 gemm batched", bm, splits, kw)
            monkeypatch.setenv("QMM_GEMM_FORCE", f"{bm},1,{splits},{kw}")
            plan = qmm.qgemm_batched_plan(ins, 16)
            monkeypatch.delenv("QMM_GEMM_FORCE")
            assert (plan.header["bm"], plan.header["nb"], plan.header["splits"], plan.header["kw"]) == \
                (bm, 1, splits, kw)
            qmm.qgemm_batched(plan)
            for (m, n, k), t, want in zip(shapes, ins, wants):
                assert_close(host(t[4]), want, f"fp16 batched {bm} S={splits} m={m}")
                t[4].fill_(float("nan"))


def test_fp16_weights_grouped():
    e, n, k, t, top_k = 16, 300, 256, 100, 4
    say("fp16 grouped")
    r = np.random.default_rng(944)
    w16s, wordss = zip(*[fp16_weight((944, ei, n), n, k) for ei in range(e)])
    words = np.stack(wordss)
    ids = np.ascontiguousarray(synth.topk_ids(r.standard_normal((t, e)), top_k), dtype=np.int32)
    x = synth.draw_act((944, 1000), t, k)
    h = synth.draw_act((944, 1001), t * top_k, k)
    for per_pair, a in ((False, x), (True, h)):
        want = np.zeros((t * top_k, n))
        for p, ex in enumerate(ids.reshape(-1)):
            want[p] = oracle.hmatmul_f64(w16s[ex], a[p if per_pair else p // top_k][None])[0]
        y = qmm.qgemm_grouped(dev(words), None, None, dev(a), dev(ids), 16, per_pair)
        assert_close(host(y), want, f"fp16 grouped per_pair={per_pair}")


def test_fused_qkv_gemv_equals_separate():
    """Decode q, k and v projections read the same activation vector; with
    their weights stacked along n ([Wq; Wk; Wv], Qwen3-0.6B: 2048 + 1024 +
    1024 rows over k = 1024) one GEMV launch gives exactly the three
    separate results (rows are computed independently)."""
    k = 1024
    for bits in (4, 8, 16):
        say("fused qkv", bits)
        parts, sep = [], []
        x = dev(synth.draw_act((945, bits), 1, k)[0])
        for i, n in enumerate((2048, 1024, 1024)):
            if bits == 16:
                _, words = fp16_weight((945, bits, i), n, k)
                s = b = None
            else:
                _, _, words, s, b = quantized((945, bits, i, 0), n, k, bits)
            parts.append((words, s, b))
            sep.append(qmm.qgemv(dev(words), None if s is None else dev(s), None if b is None else dev(b), x, bits))
        cat = lambda j: None if parts[0][j] is None else dev(np.concatenate([p[j] for p in parts]))
        fused = qmm.qgemv(cat(0), cat(1), cat(2), x, bits)
        assert torch.equal(fused, torch.cat(sep)), bits


def test_routed_grouped_equals_grouped():
    """One routing plan serves gate, up and down (and any width or group
    size); results are bit-identical to the self-bucketing call.  A plan
    built for other expert counts is refused on the device: the whole
    output becomes NaN."""
    t, top_k, e, hidden, inter = 96, 4, 16, 384, 256
    r = np.random.default_rng(946)
    ids = np.ascontiguousarray(synth.topk_ids(r.standard_normal((t, e)), top_k), dtype=np.int32)
    I = dev(ids)
    plan = qmm.moe_route(I, e)
    x = dev(synth.draw_act((946, 1), t, hidden))
    h = dev(synth.draw_act((946, 2), t * top_k, inter))
    for bits, gs in ((4, 64), (3, 32), (8, 128)):
        for (k, n, per_pair, a) in ((hidden, inter, False, x), (inter, hidden, True, h)):
            say("routed grouped", bits, gs, k, n)
            words, s_, b_, *_ = grouped_inputs((946, bits, k, n), e, n, k, bits, t, top_k, ids=ids)
            if gs != 64:
                qs = [quantized_gs((946, bits, gs, ei), n, k, bits, gs) for ei in range(e)]
                words = np.stack([q[2] for q in qs]); s_ = np.stack([q[3] for q in qs]); b_ = np.stack([q[4] for q in qs])
            W, S, B = dev(words), dev(s_), dev(b_)
            y0 = qmm.qgemm_grouped(W, S, B, a, I, bits, per_pair, group_size=gs)
            y1 = qmm.qgemm_grouped(W, S, B, a, I, bits, per_pair, group_size=gs, plan=plan)
            assert torch.equal(y0, y1), (bits, gs, per_pair)
    say("routed grouped: foreign plan")
    other = qmm.moe_route(I, e + 1)
    y = torch.full((t * top_k, inter), 7.0, device="cuda")
    words, s_, b_, *_ = grouped_inputs((947, 4, 0, 0), e, inter, hidden, 4, t, top_k, ids=ids)
    qmm.qgemm_grouped(dev(words), dev(s_), dev(b_), x, I, 4, False, y=y, plan=other)
    hh = torch.zeros((t * top_k, inter), dtype=torch.float16, device="cuda")
    qmm.moe_gate_up_swiglu((dev(words), dev(s_), dev(b_)), (dev(words), dev(s_), dev(b_)), x, I, other, 4, h=hh)
    torch.cuda.synchronize()
    assert bool(torch.isnan(y).all()), "grouped output over a foreign plan must be all NaN"
    assert bool(torch.isnan(hh).all()), "SwiGLU output over a foreign plan must be all NaN"


@pytest.mark.parametrize("bits,t", [(4, 40), (8, 40), (4, 1200)])
def test_moe_out_of_range_ids_nan_and_counted(bits, t):
    """Pairs whose expert id lies outside [0, E) (here -1, E, E + 100 and a
    large negative id) are not computed: their output rows are NaN in the
    self-bucketing, routed and fused SwiGLU products, every other row matches
    the oracle, and the plan header (byte offset 16) counts them.  At t = 1200
    the 4800 pairs are bucketed in several chunks, with bad ids in three."""
    say("moe out-of-range ids", bits, t)
    top_k, e, hidden, inter = 4, 8, 128, 160
    r = np.random.default_rng([948, bits, t])
    ids = np.ascontiguousarray(synth.topk_ids(r.standard_normal((t, e)), top_k), dtype=np.int32)
    flat = ids.reshape(-1)
    bad_at = [0, 5, 6, 17, 63, t * top_k - 1] + ([2700, 2701] if t * top_k > 4096 else [])
    for i, v in zip(bad_at, (-1, e, e + 100, -(1 << 30), e, -1, e + 1, -5)):
        flat[i] = v
    bad = np.zeros(t * top_k, dtype=bool)
    bad[bad_at] = True
    ok_ids = np.where(bad.reshape(ids.shape), 0, ids)   # oracle rows for the valid pairs
    x = synth.draw_act((948, bits, 1), t, hidden)
    gate, _ = _expert_set((948, bits, 2), e, inter, hidden, bits)
    up, _ = _expert_set((948, bits, 3), e, inter, hidden, bits)
    I = dev(ids)
    ws = torch.empty(qmm.qgemm_grouped_workspace_size(t, top_k, e, inter, hidden, bits), dtype=torch.uint8,
                     device="cuda")
    y0 = qmm.qgemm_grouped(*_to_dev(gate), dev(x), I, bits, False, workspace=ws)
    plan = qmm.moe_route(I, e)
    y1 = qmm.qgemm_grouped(*_to_dev(gate), dev(x), I, bits, False, plan=plan)
    h = qmm.moe_gate_up_swiglu(_to_dev(gate), _to_dev(up), dev(x), I, plan, bits)
    torch.cuda.synchronize()
    assert qmm.moe_plan_dropped(ws) == len(bad_at)
    assert qmm.moe_plan_dropped(plan) == len(bad_at)
    want = oracle.grouped_f64(*gate, x, ok_ids, bits, False)
    hw = oracle.moe_swiglu_f64(gate, up, x, ok_ids, bits)
    for name, got in (("self-bucketing", host(y0)), ("routed", host(y1)),
                      ("swiglu", host(h).astype(np.float64))):
        assert np.isnan(got[bad]).all(), f"{name}: rows of out-of-range pairs must be NaN"
        assert not np.isnan(got[~bad]).any(), f"{name}: valid rows must be finite"
        assert_close(got[~bad], (hw if name == "swiglu" else want)[~bad], f"{name} valid rows")
    assert torch.equal(torch.nan_to_num(y0, nan=-7.0), torch.nan_to_num(y1, nan=-7.0)), \
        "routed differs from self-bucketing"


@pytest.mark.parametrize("t,top_k,e", [(2048, 8, 128), (37, 3, 5), (512, 8, 128), (700, 8, 1000)])
def test_moe_route_plan_is_a_bucketing(t, top_k, e):
    """The routing plan is checked for what is unique about it: the header
    words, a sorted pair list that is a permutation of the pairs with each
    expert's pairs contiguous and the buckets in expert order (out-of-range
    pairs last), and a tile list that covers every bucket in order with
    tiles of at most the header's row count.  The order of pairs inside a
    bucket is not fixed (atomic placement) and is not compared."""
    say("moe route plan", t, top_k, e)
    r = np.random.default_rng([947, t, e])
    ids = np.ascontiguousarray(synth.topk_ids(r.standard_normal((t, e)), min(top_k, e)), dtype=np.int32)
    flat = ids.reshape(-1)
    bad = r.choice(flat.size, size=min(9, flat.size // 4), replace=False)
    flat[bad] = np.where(np.arange(bad.size) % 2 == 0, -1, e + 3)
    plan = qmm.moe_route(dev(ids), e)
    torch.cuda.synchronize()
    words = host(plan.view(torch.int32)).astype(np.int64)
    pairs = flat.size
    ntiles, bm, hp, he, nbad = (int(v) for v in words[:5])
    assert (hp, he, nbad) == (pairs, e, bad.size) and list(words[5:8]) == [0, 0, 0]
    sorted_ = words[8:8 + pairs]
    assert np.array_equal(np.sort(sorted_), np.arange(pairs)), "sorted list is not a permutation"
    key = np.where((flat >= 0) & (flat < e), flat, e)   # out-of-range pairs sort last
    assert np.all(np.diff(key[sorted_]) >= 0), "buckets are not contiguous in expert order"
    tiles = words[8 + pairs:8 + pairs + 3 * ntiles].reshape(ntiles, 3)
    pos = 0
    for ex, start, rows in tiles:
        assert start == pos and 1 <= rows <= bm, (ex, start, rows, pos)
        seg = key[sorted_[start:start + rows]]
        assert np.all(seg == (e if ex < 0 else ex)), (ex, start, rows)
        pos += rows
    assert pos == pairs, "tiles do not cover the pair list"


# ---------------------------------------------------- MoE FFN block (fused) --

def _expert_set(key, e, n, k, bits, gs=64):
    if bits == 16:
        ws = [fp16_weight(key + (ei,), n, k) for ei in range(e)]
        return (np.stack([w[1] for w in ws]), None, None), [w[0] for w in ws]
    qs = [quantized_gs(key + (ei,), n, k, bits, gs) for ei in range(e)]
    return (np.stack([q[2] for q in qs]), np.stack([q[3] for q in qs]), np.stack([q[4] for q in qs])), None


def _to_dev(triple):
    return tuple(None if v is None else dev(v) for v in triple)


@pytest.mark.parametrize("bits,gs", [(4, 64), (3, 64), (8, 64), (4, 32), (16, 64)])
def test_moe_gate_up_swiglu(bits, gs):
    say("swiglu", bits, gs)
    e, hidden, inter, t, top_k = 16, 256, 300, 100, 4
    r = np.random.default_rng([950, bits, gs])
    ids = np.ascontiguousarray(synth.topk_ids(r.standard_normal((t, e)), top_k), dtype=np.int32)
    x = synth.draw_act((950, bits, gs), t, hidden)
    gate, g16 = _expert_set((951, bits, gs), e, inter, hidden, bits, gs)
    up, u16 = _expert_set((952, bits, gs), e, inter, hidden, bits, gs)
    I = dev(ids)
    plan = qmm.moe_route(I, e)
    h = qmm.moe_gate_up_swiglu(_to_dev(gate), _to_dev(up), dev(x), I, plan, bits, group_size=gs)
    if bits == 16:
        g = np.stack([oracle.hmatmul_f64(g16[ids.reshape(-1)[p]], x[p // top_k][None])[0] for p in range(t * top_k)])
        u = np.stack([oracle.hmatmul_f64(u16[ids.reshape(-1)[p]], x[p // top_k][None])[0] for p in range(t * top_k)])
        want = oracle.silu_f64(g) * u
    else:
        want = oracle.moe_swiglu_f64(gate, up, x, ids, bits, gs)
    assert_close(host(h).astype(np.float64), want, f"swiglu bits={bits} gs={gs}")


@pytest.mark.parametrize("bits", [4, 3, 8])
@pytest.mark.parametrize("bm,nb", [(32, 1), (32, 2), (64, 1), (64, 2), (128, 1), (128, 2), (160, 1)])
def test_moe_forced_tiles(bits, bm, nb, monkeypatch):
    """Every MoE row tile and column width, forced: self-bucketing and
    routed grouped GEMMs and the fused gate/up SwiGLU on ragged shapes
    (experts with more pairs than one row tile, columns past the last
    full 128- or 256-wide tile)."""
    say("moe forced tile", bits, bm, nb)
    e, hidden, inter, t, top_k = 6, 192, 300, 150, 4   # 100 pairs per expert on average
    r = np.random.default_rng([957, bits])
    ids = np.ascontiguousarray(synth.topk_ids(r.standard_normal((t, e)), top_k), dtype=np.int32)
    x = synth.draw_act((957, bits, 1), t, hidden)
    gate, _ = _expert_set((958, bits), e, inter, hidden, bits)
    up, _ = _expert_set((959, bits), e, inter, hidden, bits)
    monkeypatch.setenv("QMM_MOE_FORCE", f"{bm},{nb}")
    I = dev(ids)
    plan = qmm.moe_route(I, e)
    y0 = qmm.qgemm_grouped(*_to_dev(gate), dev(x), I, bits, False)
    y1 = qmm.qgemm_grouped(*_to_dev(gate), dev(x), I, bits, False, plan=plan)
    h = qmm.moe_gate_up_swiglu(_to_dev(gate), _to_dev(up), dev(x), I, plan, bits)
    torch.cuda.synchronize()
    monkeypatch.delenv("QMM_MOE_FORCE")
    assert_close(host(y0), oracle.grouped_f64(*gate, x, ids, bits, False), f"grouped {bm}x{nb}")
    assert torch.equal(y0, y1), "routed differs from self-bucketing"
    assert_close(host(h).astype(np.float64), oracle.moe_swiglu_f64(gate, up, x, ids, bits),
                 f"swiglu {bm}x{nb}")


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("bm,nb", [(32, 1), (64, 2), (128, 1), (160, 1)])
def test_moe_tiled_weights(bits, bm, nb, monkeypatch):
    """Grouped GEMMs (self-bucketing and routed) and the fused SwiGLU over
    tile-interleaved expert weights are bit-identical to the row-major run."""
    say("moe tiled", bits, bm, nb)
    e, hidden, inter, t, top_k = 6, 192, 320, 150, 4
    r = np.random.default_rng([962, bits])
    ids = np.ascontiguousarray(synth.topk_ids(r.standard_normal((t, e)), top_k), dtype=np.int32)
    x = dev(synth.draw_act((962, bits, 1), t, hidden))
    gate = _to_dev(_expert_set((963, bits), e, inter, hidden, bits)[0])
    up = _to_dev(_expert_set((964, bits), e, inter, hidden, bits)[0])
    gate_t = (qmm.repack_tiled(gate[0], bits), gate[1], gate[2])
    up_t = (qmm.repack_tiled(up[0], bits), up[1], up[2])
    monkeypatch.setenv("QMM_MOE_FORCE", f"{bm},{nb}")
    I = dev(ids)
    plan = qmm.moe_route(I, e)
    y0 = qmm.qgemm_grouped(*gate, x, I, bits, False)
    y1 = qmm.qgemm_grouped(*gate_t, x, I, bits, False, tiled=True)
    y2 = qmm.qgemm_grouped(*gate_t, x, I, bits, False, plan=plan, tiled=True)
    h0 = qmm.moe_gate_up_swiglu(gate, up, x, I, plan, bits)
    h1 = qmm.moe_gate_up_swiglu(gate_t, up_t, x, I, plan, bits, tiled=True)
    torch.cuda.synchronize()
    monkeypatch.delenv("QMM_MOE_FORCE")
    assert torch.equal(y0, y1) and torch.equal(y0, y2), f"grouped tiled differs {bm}x{nb}"
    assert torch.equal(h0, h1), f"swiglu tiled differs {bm}x{nb}"


def test_moe_ffn_block_chain():
    """route -> fused gate/up SwiGLU -> routed down -> weighted combine equals
    the float64 chain; the combine alone is checked on random rows too."""
    say("moe ffn chain")
    e, hidden, inter, t, top_k, bits = 16, 256, 192, 64, 4, 4
    r = np.random.default_rng(953)
    logits = r.standard_normal((t, e))
    ids, wts = oracle.route(logits, top_k)
    x = synth.draw_act((953, 1), t, hidden)
    gate, _ = _expert_set((954,), e, inter, hidden, bits)
    up, _ = _expert_set((955,), e, inter, hidden, bits)
    down, _ = _expert_set((956,), e, hidden, inter, bits)
    I = dev(np.ascontiguousarray(ids))
    plan = qmm.moe_route(I, e)
    h = qmm.moe_gate_up_swiglu(_to_dev(gate), _to_dev(up), dev(x), I, plan, bits)
    yd = qmm.qgemm_grouped(*_to_dev(down), h, I, bits, True, plan=plan)
    W = torch.from_numpy(wts.astype(np.float32)).cuda()
    y = qmm.moe_combine(yd, W)
    h_want = oracle.moe_swiglu_f64(gate, up, x, ids, bits)
    yd_want = oracle.grouped_f64(*down, host(h).astype(np.float16), ids, bits, True)
    assert_close(host(yd), yd_want, "down from the GPU's h")
    y_want = oracle.moe_combine_f64(oracle.grouped_f64(*down, h_want.astype(np.float16), ids, bits, True),
                                    wts.astype(np.float32))
    assert_close(host(y), y_want, "moe ffn block")
    yp = r.standard_normal((t * top_k, 333)).astype(np.float32)
    got = qmm.moe_combine(torch.from_numpy(yp).cuda(), W)
    assert_close(host(got), oracle.moe_combine_f64(yp, wts.astype(np.float32)), "combine")
    # the four-column kernel (n a multiple of 4, 16-byte aligned rows) and the
    # one-column kernel (the same rows 4 bytes further on) give identical bits
    yp4 = torch.from_numpy(r.standard_normal((t * top_k, 336)).astype(np.float32)).cuda()
    buf = torch.empty(yp4.numel() + 1, dtype=torch.float32, device="cuda")
    buf[1:].copy_(yp4.reshape(-1))
    shifted = buf[1:].view(t * top_k, 336)
    assert shifted.data_ptr() % 16 != 0
    y4 = qmm.moe_combine(yp4, W)
    assert torch.equal(y4, qmm.moe_combine(shifted, W)), "combine: vector and scalar kernels differ"
    assert_close(host(y4), oracle.moe_combine_f64(host(yp4), wts.astype(np.float32)), "combine n=336")



def test_convert_bf16_bit_exact_all_patterns():
    """Every one of the 65536 bf16 bit patterns converts to the oracle's fp16
    (NaN payloads compared as NaN); then a GEMV over converted bf16 weights
    matches the float64 product of the bf16 values (exact in fp16 here)."""
    say("bf16 -> fp16")
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = host(qmm.convert_bf16(dev(allb.view(np.int16))), np.uint32).view(np.uint16)
    want = oracle.bf16_to_f16_bits(allb)
    nan = (want & 0x7C00) == 0x7C00
    nan &= (want & 0x03FF) != 0
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all(((got[nan] & 0x7C00) == 0x7C00) & ((got[nan] & 0x03FF) != 0))
    n, k = 300, 1024
    wb = torch.from_numpy(synth.draw_weight((960, n, k), n, k)).to(torch.bfloat16)
    w16 = oracle.bf16_to_f16_bits(wb.view(torch.int16).numpy().view(np.uint16))
    x = synth.draw_act((960, 1), 1, k)
    y = qmm.qgemv(qmm.convert_bf16(wb.cuda()), None, None, dev(x[0]), 16)
    assert_close(host(y), oracle.hmatmul_f64(w16, x)[0], "bf16 weights via fp16")
