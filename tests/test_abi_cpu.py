"""The C ABI without a GPU: the library loads, exports every entry point
declared in include/qmm.h, and rejects every bad argument on the host with
the documented status and a message, before any HIP call."""
import ctypes as C
import os
import re

import pytest

from quantized_matmul_qgemv_amd import _lib
from quantized_matmul_qgemv_amd._lib import GemmProblem, GemvProblem

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qmm.h")

INV, UNS, WSP = _lib.QMM_ERR_INVALID_ARG, _lib.QMM_ERR_UNSUPPORTED, _lib.QMM_ERR_WORKSPACE
A = 0x10000          # a fake, 64-byte aligned, never dereferenced device address
MIS = 0x10002        # misaligned for 16-byte operands


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert "qmm_qgemv" in names and "qmm_qgemm_grouped" in names and len(names) >= 12
    for name in names:
        assert hasattr(L, name), name
        assert name in _lib.SIGNATURES, f"binding misses {name}"


def test_version_and_empty_error(L):
    assert L.qmm_version() >= 100
    L.qmm_qgemm(A, A, A, A, A, 0, 64, 64, 4, 64, None, 0, None)   # m = 0: valid no-op
    assert _lib.last_error() == ""


def expect(status, code, fragment):
    assert status == code, (status, _lib.last_error())
    assert fragment in _lib.last_error(), _lib.last_error()


def test_gemv_errors(L):
    expect(L.qmm_qgemv(A, A, A, A, A, 8, 64, 7, 64, None), UNS, "bits=7")
    expect(L.qmm_qgemv(A, A, A, A, A, 8, 64, 1, 64, None), UNS, "bits=1")
    expect(L.qmm_qgemv(A, A, A, A, A, 8, 64, 12, 64, None), UNS, "bits=12")
    # 16 = unquantized fp16 weights: matmul entry points only, scales may be NULL
    expect(L.qmm_qgemv(A, None, None, MIS, A, 8, 64, 16, 64, None), INV, "x is not 16-byte aligned")
    expect(L.qmm_quantize(A, A, A, A, 8, 64, 16, 64, None), UNS, "bits=16")
    expect(L.qmm_dequant(A, A, A, A, 1, 8, 64, 16, 64, None), UNS, "bits=16")
    expect(L.qmm_qgemv(A, A, A, A, A, 8, 64, 4, 16, None), UNS, "group_size=16")
    expect(L.qmm_qgemv(A, A, A, A, A, 8, 64, 4, 256, None), UNS, "group_size=256")
    expect(L.qmm_qgemv(A, A, A, A, A, 8, 64, 4, 128, None), INV, "multiple of group_size 128")
    expect(L.qmm_qgemv(A, A, A, A, A, 0, 64, 4, 64, None), INV, "n=0")
    expect(L.qmm_qgemv(A, A, A, A, A, 8, 100, 4, 64, None), INV, "k=100")
    expect(L.qmm_qgemv(A, A, A, A, A, 8, 0, 4, 64, None), INV, "k=0")
    expect(L.qmm_qgemv(A, A, A, A, A, 8, 64 * 1024, 4, 64, None), INV, "exceeds")
    expect(L.qmm_qgemv(None, A, A, A, A, 8, 64, 4, 64, None), INV, "null pointer w")
    expect(L.qmm_qgemv(MIS, A, A, A, A, 8, 64, 4, 64, None), INV, "w is not 16-byte aligned")
    expect(L.qmm_qgemv(A, A, A, MIS, A, 8, 64, 4, 64, None), INV, "x is not 16-byte aligned")
    expect(L.qmm_qgemv(A, A + 1, A, A, A, 8, 64, 4, 64, None), INV, "scales is not 2-byte aligned")
    expect(L.qmm_qgemv(A, A, A, A, None, 8, 64, 4, 64, None), INV, "null pointer y")


def test_gemm_errors(L):
    expect(L.qmm_qgemm(A, A, A, A, A, -1, 8, 64, 4, 64, None, 0, None), INV, "m=-1")
    expect(L.qmm_qgemm(A, A, A, A, A, 4, 8, 96, 4, 64, None, 0, None), INV, "k=96")
    expect(L.qmm_qgemm(A, A, A, A, A, 4, 8, 64, 7, 64, None, 0, None), UNS, "bits=7")
    expect(L.qmm_qgemm(A, A, A, MIS, A, 4, 8, 64, 4, 64, None, 0, None), INV, "x is not")
    assert L.qmm_qgemm_workspace_size(2048, 9728, 2560, 4, 64) == 0
    expect(L.qmm_qgemm(A, A, A, A, A, 4, 8, 192, 4, 128, None, 0, None), INV, "multiple of group_size 128")
    expect(L.qmm_qgemm(A, A, A, A, A, 4, 8, 64, 4, 48, None, 0, None), UNS, "group_size=48")


def test_grouped_errors(L):
    ws = L.qmm_qgemm_grouped_workspace_size(512, 8, 128, 768, 2048, 4, 64)
    assert ws >= 4 * 512 * 8
    expect(L.qmm_qgemm_grouped(A, A, A, A, 0, A, A, 512, 8, 128, 768, 2048, 4, 64, A, ws - 1, None),
           WSP, "workspace")
    expect(L.qmm_qgemm_grouped(A, A, A, A, 0, A, A, 512, 8, 128, 768, 2048, 4, 64, None, ws, None),
           WSP, "workspace")
    expect(L.qmm_qgemm_grouped(A, A, A, A, 0, A, A, 512, 8, 2000, 768, 2048, 4, 64, A, ws, None),
           INV, "e=2000")
    expect(L.qmm_qgemm_grouped(A, A, A, A, 2, A, A, 512, 8, 128, 768, 2048, 4, 64, A, ws, None),
           INV, "a_row_per_pair")
    expect(L.qmm_qgemm_grouped(A, A, A, A, 0, A, A, 512, 0, 128, 768, 2048, 4, 64, A, ws, None),
           INV, "top_k=0")
    expect(L.qmm_qgemm_grouped(A, A, A, A, 0, A + 2, A, 512, 8, 128, 768, 2048, 4, 64, A, ws, None),
           INV, "expert_ids is not 4-byte aligned")
    expect(L.qmm_qgemm_grouped(A, A, A, A, 0, A, A, 512, 8, 128, 768, 2048, 7, 64, A, ws, None),
           UNS, "bits=7")


def test_route_errors(L):
    need = L.qmm_moe_route_size(512, 8, 128)
    assert need >= 4 * 512 * 8
    assert L.qmm_moe_route_size(512, 0, 128) == 0 and L.qmm_moe_route_size(512, 8, 2000) == 0
    expect(L.qmm_moe_route(A, 512, 8, 128, A, need - 1, None), WSP, "plan of")
    expect(L.qmm_moe_route(A, 512, 8, 128, None, need, None), WSP, "plan of")
    expect(L.qmm_moe_route(A + 2, 512, 8, 128, A, need, None), INV, "expert_ids is not 4-byte aligned")
    expect(L.qmm_moe_route(A, 512, 8, 0, A, need, None), INV, "e=0")
    assert L.qmm_moe_route(A, 0, 8, 128, None, 0, None) == 0            # no tokens: no-op
    expect(L.qmm_qgemm_grouped_routed(A, A, A, A, 0, None, need, A, 512, 8, 128, 768, 2048, 4, 64, None),
           INV, "null pointer plan")
    expect(L.qmm_qgemm_grouped_routed(A, A, A, A, 3, A, need, A, 512, 8, 128, 768, 2048, 4, 64, None),
           INV, "a_row_per_pair")
    expect(L.qmm_qgemm_grouped_routed(A, A, A, A, 0, A, need, A, 512, 8, 128, 768, 2048, 7, 64, None),
           UNS, "bits=7")
    # a plan buffer smaller than the routing plan for these counts is refused
    # on the host (a plan for other counts of the same size is caught on the
    # device, where the output becomes NaN)
    expect(L.qmm_qgemm_grouped_routed(A, A, A, A, 0, A, need - 1, A, 512, 8, 128, 768, 2048, 4, 64, None),
           WSP, "routing plan for t=512")
    expect(L.qmm_moe_gate_up_swiglu(A, A, A, A, A, A, A, A, need - 1, A, 512, 8, 128, 768, 2048, 4, 64, None),
           WSP, "routing plan for t=512")
    small = L.qmm_moe_route_size(256, 8, 128)
    expect(L.qmm_qgemm_grouped_routed(A, A, A, A, 0, A, small, A, 512, 8, 128, 768, 2048, 4, 64, None),
           WSP, "plan of")


def test_grouped_noalloc_errors(L):
    """The allocation-free grouped call validates like qmm_qgemm_grouped and
    refuses, before any HIP call, a problem whose bucket lists exceed its
    1 MiB static scratch."""
    assert _lib.QMM_GROUPED_SCRATCH_BYTES == 1 << 20
    ok = L.qmm_qgemm_grouped_workspace_size(28900, 8, 128, 768, 2048, 4, 64)
    assert ok <= _lib.QMM_GROUPED_SCRATCH_BYTES
    big = L.qmm_qgemm_grouped_workspace_size(40000, 8, 128, 768, 2048, 4, 64)
    assert big > _lib.QMM_GROUPED_SCRATCH_BYTES
    expect(L.qmm_qgemm_grouped_noalloc(A, A, A, A, 0, A, A, 40000, 8, 128, 768, 2048, 4, 64, None),
           WSP, "static scratch holds 1048576")
    expect(L.qmm_qgemm_grouped_noalloc(A, A, A, A, 0, None, A, 512, 8, 128, 768, 2048, 4, 64, None),
           INV, "null pointer expert_ids")
    expect(L.qmm_qgemm_grouped_noalloc(A, A, A, A, 2, A, A, 512, 8, 128, 768, 2048, 4, 64, None),
           INV, "a_row_per_pair")
    expect(L.qmm_qgemm_grouped_noalloc(A, A, A, A, 0, A, A, 512, 8, 128, 768, 2048, 7, 64, None),
           UNS, "bits=7")
    expect(L.qmm_qgemm_grouped_noalloc(A, A, A, A, 0, A, A, 8, 2, 4, 200, 128, 4 | _lib.QMM_WEIGHTS_TILED,
                                       64, None), INV, "multiple of 32")
    assert L.qmm_qgemm_grouped_noalloc(A, A, A, A, 0, A, A, 0, 8, 128, 768, 2048, 4, 64, None) == 0


def test_route_size_counts_out_of_range_bucket(L):
    """The plan has an 8-word header, one word per pair and three per row
    tile; the row-tile bound counts the E valid buckets plus one for pairs
    whose expert id is out of range (every tile holds at least one pair, so
    never more tiles than pairs).  After them come E + 1 counts per chunk of
    the pair list: one chunk up to 4096 pairs, else chunks of at least 256
    pairs, at most 64 chunks and at most 32768 counts."""
    for t, top_k, e in ((512, 8, 128), (2048, 8, 128), (1, 1, 1), (3, 2, 1000), (5, 8, 4),
                        (40000, 8, 128), (300, 8, 1000)):
        pairs = t * top_k
        tiles = min((pairs + 31) // 32 + e + 1, pairs)
        g = max(1, min(64, 32768 // (e + 1)))
        chunk = max(256, -(-pairs // g))
        chunks = 1 if pairs <= 4096 else -(-pairs // chunk)
        want = -(-(8 + pairs + 3 * tiles + chunks * (e + 1)) * 4 // 256) * 256
        assert L.qmm_moe_route_size(t, top_k, e) == want, (t, top_k, e)
        assert L.qmm_qgemm_grouped_workspace_size(t, top_k, e, 768, 2048, 4, 64) == want


def test_workspace_size_ignores_layout_flag(L):
    """The split-k workspace does not depend on the weight layout: the size
    query gives the same answer with QMM_WEIGHTS_TILED on the bits."""
    tiled = _lib.QMM_WEIGHTS_TILED
    for (m, n, k) in ((128, 2560, 9728), (64, 512, 4096), (2048, 9728, 2560), (1, 64, 64)):
        for bits in (2, 3, 4, 5, 6, 8, 16):
            plain = L.qmm_qgemm_workspace_size(m, n, k, bits, 64)
            assert L.qmm_qgemm_workspace_size(m, n, k, bits | tiled, 64) == plain, (m, n, k, bits)
    assert L.qmm_qgemm_workspace_size(128, 2560, 9728, 4, 64) > 0


def test_convert_bf16_errors(L):
    expect(L.qmm_convert_bf16(A, A, 7, None), INV, "must be even")
    expect(L.qmm_convert_bf16(A + 2, A, 8, None), INV, "src is not 4-byte aligned")
    expect(L.qmm_convert_bf16(A, None, 8, None), INV, "null pointer dst")
    assert L.qmm_convert_bf16(None, None, 0, None) == 0


def test_other_errors(L):
    expect(L.qmm_quantize(MIS, A, A, A, 8, 64, 4, 64, None), INV, "w_f32 is not 16-byte aligned")
    expect(L.qmm_unpack_codes(A, A, 8, 65, 4, None), INV, "k=65")
    expect(L.qmm_dequant(A, A, A, A, 2, 8, 64, 4, 64, None), INV, "out_is_f16")
    expect(L.qmm_dequant(A, A, A, A, 1, 8, 64, 7, 64, None), UNS, "bits=7")


def check_gemv_plan_covers(buf, shapes):
    """Block records of a GEMV plan image: pointers and row ranges tile every
    problem (problem i has w = A * (i + 1)) exactly once, in whole passes
    except for each problem's last block."""
    hdr = (C.c_int32 * 16).from_buffer(buf)
    lpr, rows, blocks, max_groups = hdr[4], hdr[5], hdr[6], hdr[7]
    assert max_groups == max(k for _, k in shapes) // 64
    assert all((k // 64) % lpr == 0 for _, k in shapes)
    rec = (C.c_int64 * (8 * blocks)).from_buffer(buf, 64)
    seen = {}
    for bi in range(blocks):
        r = rec[8 * bi: 8 * bi + 8]
        n_k = r[5] & 0xFFFFFFFFFFFFFFFF
        n, k = n_k & 0xFFFFFFFF, n_k >> 32
        rr = r[6] & 0xFFFFFFFFFFFFFFFF
        row0, nrows = rr & 0xFFFFFFFF, rr >> 32
        seen.setdefault(r[0], []).append((row0, nrows, n, k))
    assert len(seen) == len(shapes)
    for i, (n, k) in enumerate(shapes):
        recs = sorted(seen[A * (i + 1)])
        assert all(x[2] == n and x[3] == k and x[1] > 0 for x in recs)
        assert recs[0][0] == 0 and all(a[0] + a[1] == b[0] for a, b in zip(recs, recs[1:]))
        assert recs[-1][0] + recs[-1][1] == n
        assert all(x[1] % rows == 0 for x in recs[:-1])


def test_batched_plan_host_only(L):
    probs = (GemvProblem * 3)()
    shapes = [(2048, 1024), (1024, 3072), (151936, 1024)]
    for i, (n, k) in enumerate(shapes):
        probs[i] = GemvProblem(A * (i + 1), A, A, A, A, n, k)
    need = C.c_size_t(0)
    expect(L.qmm_qgemv_batched_plan(probs, 3, 4, 64, None, 0, C.byref(need)), WSP, "plan buffer")
    assert need.value > 64
    buf = (C.c_uint8 * need.value)()
    assert L.qmm_qgemv_batched_plan(probs, 3, 4, 64, buf, need.value, C.byref(need)) == 0
    hdr = (C.c_int32 * 16).from_buffer(buf)
    assert hdr[0] == 0x504D4D51 and hdr[2] == 4 and hdr[3] == 64
    lpr, rows, blocks, max_groups, count = hdr[4], hdr[5], hdr[6], hdr[7], hdr[8]
    assert lpr == 16 and max_groups == 48 and count == 3 and rows == 64
    assert need.value == 64 + 64 * blocks
    check_gemv_plan_covers(buf, shapes)
    # corrupt header / bad problem
    bad = (C.c_uint8 * 64)()
    expect(L.qmm_qgemv_batched(A, bad, None), INV, "not a plan image")
    probs[1] = GemvProblem(A, A, A, A, A, 1024, 3000)
    expect(L.qmm_qgemv_batched_plan(probs, 3, 4, 64, buf, need.value, C.byref(need)), INV, "problem 1")
    probs[1] = GemvProblem(A, A, A, MIS, A, 1024, 3072)
    expect(L.qmm_qgemv_batched_plan(probs, 3, 4, 64, buf, need.value, C.byref(need)), INV, "misaligned")


def gemm_batch_plan(L, shapes, bits=4, env=None, gs=64):
    """Build a batched-GEMM plan on the host for (m, n, k) shapes; decode it."""
    import struct
    old = os.environ.pop("QMM_GEMM_FORCE", None)
    if env:
        os.environ["QMM_GEMM_FORCE"] = env
    try:
        probs = (GemmProblem * len(shapes))()
        for i, (m, n, k) in enumerate(shapes):
            probs[i] = GemmProblem(A * (i + 1), A, A, A, A * (i + 1) + 0x1000, m, n, k)
        need, ws = C.c_size_t(0), C.c_size_t(0)
        expect(L.qmm_qgemm_batched_plan(probs, len(shapes), bits, gs, None, 0, C.byref(need),
                                        C.byref(ws)), WSP, "plan buffer")
        buf = (C.c_uint8 * need.value)()
        assert L.qmm_qgemm_batched_plan(probs, len(shapes), bits, gs, buf, need.value,
                                        C.byref(need), C.byref(ws)) == 0
    finally:
        os.environ.pop("QMM_GEMM_FORCE", None)
        if old is not None:
            os.environ["QMM_GEMM_FORCE"] = old
    raw = bytes(buf)
    f = struct.unpack_from("<IIiiiiiiiiiiQii", raw, 0)
    hdr = dict(zip(["magic", "version", "bits", "gs", "bm", "nb", "sbq", "count", "num_tiles",
                    "split_tiles", "splits", "wtiled", "ws", "kw", "stiled"], f))
    off = 64 + 64 * len(shapes)
    recs = [struct.unpack_from("<8i", raw, off + 32 * i) for i in range(hdr["num_tiles"])]
    off2 = off + 32 * hdr["num_tiles"]
    hdr["split_recs"] = [struct.unpack_from("<4i", raw, off2 + 16 * i)[:3] for i in range(hdr["split_tiles"])]
    assert need.value == off2 + 16 * hdr["split_tiles"] and ws.value == hdr["ws"]
    return hdr, recs


def check_gemm_plan_covers(hdr, recs, shapes):
    """Every output tile of every problem is covered by S records whose k
    ranges split [0, G) in order; split tiles have one GemmSplitTile each;
    the workspace holds every partial tile."""
    assert hdr["magic"] == 0x424D4D51 and hdr["count"] == len(shapes)
    bm, bn, S = hdr["bm"], hdr["nb"] * 128, hdr["splits"]
    assert bm in (32, 64, 128, 256) and hdr["num_tiles"] % 8 == 0
    live = [r for r in recs if r[0] >= 0]
    tiles = {}
    for p, m0, n0, g0, g1, sp, sps, sid in live:
        assert sps == S and 0 <= sp < S and g0 < g1
        if hdr["sbq"]:
            assert g0 % 4 == 0 and g1 % 4 == 0
        tiles.setdefault((p, m0, n0), []).append((sp, g0, g1, sid))
    want = 0
    sids = set()
    for p, (m, n, k) in enumerate(shapes):
        G = k // 64
        for m0 in range(0, m, bm):
            for n0 in range(0, n, bn):
                want += 1
                parts = sorted(tiles.pop((p, m0, n0)))
                assert [x[0] for x in parts] == list(range(S))
                assert parts[0][1] == 0 and parts[-1][2] == G
                assert all(a[2] == b[1] for a, b in zip(parts, parts[1:]))
                assert len({x[3] for x in parts}) == 1
                sids.add(parts[0][3])
                if S > 1:
                    assert hdr["split_recs"][parts[0][3]] == (p, m0, n0)
    assert not tiles, "records outside the problems"
    assert len(live) == want * S
    if S > 1:
        assert sids == set(range(hdr["split_tiles"])) and hdr["split_tiles"] == want
        assert hdr["ws"] == hdr["split_tiles"] * S * bm * bn * 4
    else:
        assert hdr["ws"] == 0


def test_gemm_plan_two_k_halves(L):
    """A forced two-half tile (8 waves, the k range of every record split
    again inside the workgroup) is recorded in the header, still covers
    every tile once, and needs at least two groups per half-split; the
    planner's own choices use one half unless a two-half tile is cheaper."""
    shapes = [(70, 520, 1024), (300, 200, 768), (1, 64, 256)]
    for env, want in (("64,1,1,2", (64, 1, 1, 2)), ("32,1,2,2", (32, 1, 2, 2)),
                      ("128,1,2,2", (128, 1, 2, 2)), ("64,2,1,2", (64, 2, 1, 2)),
                      ("64,1,3", (64, 1, 3, 1))):
        hdr, recs = gemm_batch_plan(L, shapes, env=env)
        assert (hdr["bm"], hdr["nb"], hdr["splits"], hdr["kw"]) == want, (env, hdr)
        check_gemm_plan_covers(hdr, recs, shapes)
    # no two-half tile with 256 rows or with two column blocks of 32 rows, and
    # no third half: such forces are ignored (the planner's own choice stands)
    own, _ = gemm_batch_plan(L, shapes)
    for env in ("256,2,1,2", "32,2,1,2", "64,1,1,3"):
        hdr, _ = gemm_batch_plan(L, shapes, env=env)
        assert {k: hdr[k] for k in ("bm", "nb", "splits", "kw")} == \
            {k: own[k] for k in ("bm", "nb", "splits", "kw")}, (env, hdr)
    # a k of 4 groups cannot be split into 4 x 2 halves: the force is ignored
    hdr, _ = gemm_batch_plan(L, [(64, 128, 256)], env="64,1,4,2")
    assert (hdr["splits"], hdr["kw"]) != (4, 2)




@pytest.mark.parametrize("shapes", [
    [(2048, 4096, 2560), (2048, 1024, 2560), (2048, 1024, 2560)],   # q, k, v
    [(2048, 9728, 2560), (2048, 9728, 2560)],                         # gate, up
    [(128, 2560, 9728)],                                              # down at M=128
    [(128, 4096, 2560), (128, 1024, 2560), (128, 1024, 2560)],
    [(70, 520, 1024), (1, 64, 64), (0, 128, 128), (300, 200, 192)],   # ragged, m=0, k=3 groups
])
def test_batched_gemm_plan_covers_every_tile(L, shapes):
    hdr, recs = gemm_batch_plan(L, shapes)
    check_gemm_plan_covers(hdr, recs, shapes)


def test_batched_plans_random(L):
    """Seeded random problem lists (ragged and empty problems, every width
    and group size, planner choices and forced tiles and splits): both plan
    builders cover every output exactly once."""
    import numpy as np
    r = np.random.default_rng(2024)
    cfgs = [(256, 2), (128, 2), (128, 1), (64, 2), (64, 1), (32, 2), (32, 1)]
    for trial in range(60):
        bits = int(r.choice([2, 3, 4, 5, 6, 8, 16]))
        gs = 64 if bits == 16 else int(r.choice([32, 64, 128]))
        step = max(64, gs)
        count = int(r.integers(1, 5))
        shapes = []
        for _ in range(count):
            m = int(r.choice([0, 1, int(r.integers(2, 700))]))
            shapes.append((m, int(r.integers(1, 1500)), step * int(r.integers(1, 40))))
        env = None
        if trial % 2:
            bm, nb = cfgs[int(r.integers(len(cfgs)))]
            env = f"{bm},{nb},{int(r.choice([1, 2, 3, 4, 5, 8]))}"
        hdr, recs = gemm_batch_plan(L, shapes, bits=bits, env=env, gs=gs)
        assert hdr["bits"] == bits and hdr["gs"] == gs
        check_gemm_plan_covers(hdr, recs, shapes)

        vshapes = [(int(r.integers(1, 5000)), step * int(r.integers(1, 4096 // step + 1)))
                   for _ in range(int(r.integers(1, 7)))]
        probs = (GemvProblem * len(vshapes))()
        for i, (n, k) in enumerate(vshapes):
            probs[i] = GemvProblem(A * (i + 1), A, A, A, A, n, k)
        need = C.c_size_t(0)
        expect(L.qmm_qgemv_batched_plan(probs, len(vshapes), bits, gs, None, 0, C.byref(need)), WSP,
               "plan buffer")
        buf = (C.c_uint8 * need.value)()
        assert L.qmm_qgemv_batched_plan(probs, len(vshapes), bits, gs, buf, need.value, C.byref(need)) == 0
        hv = (C.c_int32 * 16).from_buffer(buf)
        assert hv[2] == bits and hv[3] == gs and hv[8] == len(vshapes)
        assert need.value == 64 + 64 * hv[6]
        check_gemv_plan_covers(buf, vshapes)


def test_repack_tiled_errors_and_plan_flag(L):
    """qmm_repack_tiled checks shapes, width and overlap on the host; a
    batched plan with QMM_WEIGHTS_TILED records the flag and needs n % 32 == 0."""
    B = A + (1 << 24)
    expect(L.qmm_repack_tiled(A, B, 48, 128, 4, None), INV, "multiple of 32")
    expect(L.qmm_repack_tiled(A, B, 64, 100, 4, None), INV, "k=100")
    expect(L.qmm_repack_tiled(A, B, 64, 128, 7, None), UNS, "bits=7")
    expect(L.qmm_repack_tiled(None, B, 64, 128, 4, None), INV, "null pointer")
    expect(L.qmm_repack_tiled(A, MIS, 64, 128, 4, None), INV, "aligned")
    expect(L.qmm_repack_tiled(A, A + 64, 64, 128, 4, None), INV, "overlap")
    tiled = _lib.QMM_WEIGHTS_TILED
    hdr, recs = gemm_batch_plan(L, [(70, 512, 1024), (300, 224, 768)], bits=4 | tiled)
    assert hdr["bits"] == 4 and hdr["wtiled"] == 1
    check_gemm_plan_covers(hdr, recs, [(70, 512, 1024), (300, 224, 768)])
    hdr, _ = gemm_batch_plan(L, [(70, 512, 1024)], bits=4)
    assert hdr["wtiled"] == 0
    probs = (GemmProblem * 1)()
    probs[0] = GemmProblem(A, A, A, A, A, 64, 200, 128)
    need, ws = C.c_size_t(0), C.c_size_t(0)
    expect(L.qmm_qgemm_batched_plan(probs, 1, 4 | tiled, 64, None, 0, C.byref(need), C.byref(ws)), INV,
           "n % 32")
    expect(L.qmm_qgemm(A, A, A, A, A, 8, 200, 128, 4 | tiled, 64, A, 1 << 20, None), INV, "multiple of 32")
    expect(L.qmm_qgemm_grouped(A, A, A, A, 0, A, A, 8, 2, 4, 200, 128, 4 | tiled, 64, A, 1 << 20, None),
           INV, "multiple of 32")
    expect(L.qmm_qgemm_grouped_routed(A, A, A, A, 0, A, 1 << 20, A, 8, 2, 4, 200, 128, 4 | tiled, 64, None),
           INV, "multiple of 32")
    expect(L.qmm_moe_gate_up_swiglu(A, A, A, A, A, A, A, A, 1 << 20, A, 8, 2, 4, 200, 128, 4 | tiled, 64,
                                    None),
           INV, "multiple of 32")
    # entry points that read row-major weights only refuse the flag
    expect(L.qmm_qgemv(A, A, A, A, A, 64, 128, 4 | tiled, 64, None), UNS, "bits")
    expect(L.qmm_dequant(A, A, A, A, 0, 64, 128, 4 | tiled, 64, None), UNS, "bits")
    expect(L.qmm_repack_tiled(A, B, 64, 128, 4 | tiled, None), UNS, "bits")


def test_scales_tiled_host_checks(L):
    """QMM_SCALES_TILED (interleaved scales from qmm_repack_scales_tiled)
    needs tile-interleaved weights, quantized codes, groups of 64, k % 256
    == 0 and 16-byte aligned scales; biases may be NULL; plans record the
    flag; entry points without the layout refuse it; the repack checks its
    shapes, pointers and overlap on the host."""
    B = A + (1 << 24)
    st, wt = _lib.QMM_SCALES_TILED, _lib.QMM_WEIGHTS_TILED
    expect(L.qmm_qgemm(A, A, None, A, A, 8, 64, 256, 4 | st, 64, A, 1 << 20, None), INV, "QMM_WEIGHTS_TILED")
    expect(L.qmm_qgemm(A, A, None, A, A, 8, 64, 320, 4 | st | wt, 64, A, 1 << 20, None), INV, "k % 256")
    expect(L.qmm_qgemm(A, A, None, A, A, 8, 64, 256, 4 | st | wt, 32, A, 1 << 20, None), INV, "group_size 64")
    expect(L.qmm_qgemm(A, A, None, A, A, 8, 64, 256, 16 | st | wt, 64, A, 1 << 20, None), INV, "fp16")
    expect(L.qmm_qgemm(A, A + 8, None, A, A, 8, 64, 256, 4 | st | wt, 64, A, 1 << 20, None), INV, "aligned")
    hdr, recs = gemm_batch_plan(L, [(70, 512, 1024), (300, 224, 768)], bits=4 | wt | st)
    assert hdr["stiled"] == 1 and hdr["wtiled"] == 1 and hdr["bits"] == 4
    check_gemm_plan_covers(hdr, recs, [(70, 512, 1024), (300, 224, 768)])
    assert gemm_batch_plan(L, [(70, 512, 1024)], bits=4 | wt)[0]["stiled"] == 0
    probs = (GemmProblem * 1)()
    need, ws = C.c_size_t(0), C.c_size_t(0)
    probs[0] = GemmProblem(A, A, 0, A, A, 64, 256, 320)
    expect(L.qmm_qgemm_batched_plan(probs, 1, 4 | wt | st, 64, None, 0, C.byref(need), C.byref(ws)), INV,
           "k % 256")
    probs[0] = GemmProblem(A, A + 8, 0, A, A, 64, 256, 512)
    expect(L.qmm_qgemm_batched_plan(probs, 1, 4 | wt | st, 64, None, 0, C.byref(need), C.byref(ws)), INV,
           "misaligned")
    expect(L.qmm_qgemm_batched_plan(probs, 1, 4 | st, 64, None, 0, C.byref(need), C.byref(ws)), INV,
           "QMM_WEIGHTS_TILED")
    assert L.qmm_qgemm_workspace_size(128, 2560, 9728, 4 | wt | st, 64) == \
        L.qmm_qgemm_workspace_size(128, 2560, 9728, 4, 64)
    # the grouped MoE calls check the flag the same way
    expect(L.qmm_qgemm_grouped(A, A, A, A, 0, A, A, 8, 2, 4, 256, 256, 4 | st, 64, A, 1 << 20, None),
           INV, "QMM_WEIGHTS_TILED")
    expect(L.qmm_qgemm_grouped_noalloc(A, A, A, A, 0, A, A, 8, 2, 4, 256, 320, 4 | wt | st, 64, None),
           INV, "k % 256")
    expect(L.qmm_qgemm_grouped_routed(A, A + 8, None, A, 0, A, 1 << 20, A, 8, 2, 4, 256, 256, 4 | wt | st,
                                      64, None), INV, "aligned")
    expect(L.qmm_moe_gate_up_swiglu(A, A, A, A, A, A, A, A, 1 << 20, A, 8, 2, 4, 256, 256, 4 | wt | st, 32,
                                    None), INV, "group_size 64")
    # entry points without the interleaved scale layout refuse the flag
    expect(L.qmm_qgemv(A, A, A, A, A, 64, 256, 4 | st, 64, None), UNS, "bits")
    expect(L.qmm_dequant(A, A, A, A, 0, 64, 256, 4 | st, 64, None), UNS, "bits")
    # the repack
    expect(L.qmm_repack_scales_tiled(A, A, B, 48, 256, None), INV, "multiple of 32")
    expect(L.qmm_repack_scales_tiled(A, A, B, 64, 320, None), INV, "multiple of 256")
    expect(L.qmm_repack_scales_tiled(A, A, B, 64, 100, None), INV, "k=100")
    expect(L.qmm_repack_scales_tiled(None, A, B, 64, 256, None), INV, "null pointer")
    expect(L.qmm_repack_scales_tiled(A, A, MIS, 64, 256, None), INV, "aligned")
    expect(L.qmm_repack_scales_tiled(A, A + (1 << 20), A + 64, 64, 256, None), INV, "overlap")
    expect(L.qmm_repack_scales_tiled(A, A + (1 << 20), A + (1 << 20) + 64, 64, 256, None), INV, "overlap")


def test_batched_gemm_plan_group_sizes(L):
    """Quad scale loads (sbq) only for groups of 64; the header records the group size."""
    for gs in (32, 64, 128):
        hdr, _ = gemm_batch_plan(L, [(2048, 2560, 9728)], env="256,2,4", gs=gs)
        assert hdr["gs"] == gs and hdr["sbq"] == (1 if gs == 64 else 0), (gs, hdr)


def test_batched_gemm_plan_sbq_needs_aligned_scales(L):
    """Quad scale loads are 8-byte loads: a plan whose scales or biases are
    only 2- or 4-byte aligned takes the per-group path (sbq = 0)."""
    for s_ptr, b_ptr, want in ((A, A, 1), (A + 2, A, 0), (A, A + 4, 0), (A + 8, A + 16, 1)):
        probs = (GemmProblem * 2)()
        probs[0] = GemmProblem(A, A, A, A, A, 2048, 2560, 9728)
        probs[1] = GemmProblem(A, s_ptr, b_ptr, A, A, 2048, 2560, 9728)
        need, ws = C.c_size_t(0), C.c_size_t(0)
        os.environ["QMM_GEMM_FORCE"] = "128,2,1"
        try:
            assert L.qmm_qgemm_batched_plan(probs, 2, 4, 64, None, 0, C.byref(need), C.byref(ws)) == WSP
            buf = (C.c_uint8 * need.value)()
            assert L.qmm_qgemm_batched_plan(probs, 2, 4, 64, buf, need.value, C.byref(need),
                                            C.byref(ws)) == 0
        finally:
            os.environ.pop("QMM_GEMM_FORCE", None)
        assert C.cast(buf, C.POINTER(C.c_int32))[6] == want, (s_ptr, b_ptr)


def test_batched_gemm_plan_force_and_errors(L):
    hdr, _ = gemm_batch_plan(L, [(2048, 2560, 9728)], env="256,2,4")
    assert (hdr["bm"], hdr["nb"], hdr["splits"], hdr["sbq"]) == (256, 2, 4, 1)
    hdr, _ = gemm_batch_plan(L, [(64, 512, 192)], env="64,1,3")
    assert (hdr["bm"], hdr["splits"], hdr["sbq"]) == (64, 3, 0)
    probs = (GemmProblem * 2)()
    probs[0] = GemmProblem(A, A, A, A, A, 64, 128, 128)
    probs[1] = GemmProblem(A, A, A, A, A, 64, 128, 100)
    need, ws = C.c_size_t(0), C.c_size_t(0)
    expect(L.qmm_qgemm_batched_plan(probs, 2, 4, 64, None, 0, C.byref(need), C.byref(ws)), INV,
           "problem 1")
    probs[1] = GemmProblem(A, A, A, MIS, A, 64, 128, 128)
    expect(L.qmm_qgemm_batched_plan(probs, 2, 4, 64, None, 0, C.byref(need), C.byref(ws)), INV,
           "misaligned")
    probs[1] = GemmProblem(A, A, A, A, A, -1, 128, 128)
    expect(L.qmm_qgemm_batched_plan(probs, 2, 4, 64, None, 0, C.byref(need), C.byref(ws)), INV,
           "problem 1")
    expect(L.qmm_qgemm_batched_plan(probs, 0, 4, 64, None, 0, C.byref(need), C.byref(ws)), INV,
           "count=0")
    expect(L.qmm_qgemm_batched_plan(probs, 2, 7, 64, None, 0, C.byref(need), C.byref(ws)), UNS,
           "bits=7")
    bad = (C.c_uint8 * 64)()
    expect(L.qmm_qgemm_batched(A, bad, None, 0, None), INV, "not a batched-GEMM plan")
    # a split plan refuses a missing or short workspace before any launch
    probs1 = (GemmProblem * 1)()
    probs1[0] = GemmProblem(A, A, A, A, A, 64, 512, 4096)
    os.environ["QMM_GEMM_FORCE"] = "64,1,4"
    try:
        assert L.qmm_qgemm_batched_plan(probs1, 1, 4, 64, None, 0, C.byref(need), C.byref(ws)) == WSP
        buf = (C.c_uint8 * need.value)()
        assert L.qmm_qgemm_batched_plan(probs1, 1, 4, 64, buf, need.value, C.byref(need),
                                        C.byref(ws)) == 0
    finally:
        os.environ.pop("QMM_GEMM_FORCE", None)
    assert ws.value > 0
    expect(L.qmm_qgemm_batched(A, buf, None, 0, None), WSP, "workspace")
    expect(L.qmm_qgemm_batched(A, buf, A, ws.value - 1, None), WSP, "workspace")
    # a header whose k-halves field names no kernel is refused before any launch
    for kw in (0, 3, -1):
        C.cast(buf, C.POINTER(C.c_int32))[14] = kw
        expect(L.qmm_qgemm_batched(A, buf, A, ws.value, None), INV, "corrupt plan header")
