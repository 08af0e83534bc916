"""The C ABI without a GPU: the library loads, exports every entry point
declared in include/qmm.h, and rejects every bad argument on the host with
the documented status and a message, before any HIP call."""
import ctypes as C
import os
import re

import pytest

from quantized_matmul_qgemv_amd import _lib
from quantized_matmul_qgemv_amd._lib import GemvProblem

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
    expect(L.qmm_qgemv(A, A, A, A, A, 8, 64, 3, 64, None), UNS, "bits=3")
    expect(L.qmm_qgemv(A, A, A, A, A, 8, 64, 4, 32, None), UNS, "group_size=32")
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
    expect(L.qmm_qgemm(A, A, A, A, A, 4, 8, 64, 5, 64, None, 0, None), UNS, "bits=5")
    expect(L.qmm_qgemm(A, A, A, MIS, A, 4, 8, 64, 4, 64, None, 0, None), INV, "x is not")
    assert L.qmm_qgemm_workspace_size(2048, 9728, 2560, 4, 64) == 0


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
    expect(L.qmm_qgemm_grouped(A, A, A, A, 0, A, A, 512, 8, 128, 768, 2048, 6, 64, A, ws, None),
           UNS, "bits=6")


def test_other_errors(L):
    expect(L.qmm_quantize(MIS, A, A, A, 8, 64, 4, 64, None), INV, "w_f32 is not 16-byte aligned")
    expect(L.qmm_unpack_codes(A, A, 8, 65, 4, None), INV, "k=65")
    expect(L.qmm_dequant(A, A, A, A, 2, 8, 64, 4, 64, None), INV, "out_is_f16")
    expect(L.qmm_dequant(A, A, A, A, 1, 8, 64, 7, 64, None), UNS, "bits=7")


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
    # block records: pointers and row ranges tile every problem exactly once
    rec = (C.c_int64 * (8 * blocks)).from_buffer(buf, 64)
    seen = {}
    for bi in range(blocks):
        r = rec[8 * bi: 8 * bi + 8]
        n_k = r[5] & 0xFFFFFFFFFFFFFFFF
        n, k = n_k & 0xFFFFFFFF, n_k >> 32
        rr = r[6] & 0xFFFFFFFFFFFFFFFF
        row0, nrows = rr & 0xFFFFFFFF, rr >> 32
        seen.setdefault(r[0], []).append((row0, nrows, n, k))
    for i, (n, k) in enumerate(shapes):
        recs = sorted(seen[A * (i + 1)])
        assert all(x[2] == n and x[3] == k for x in recs)
        assert recs[0][0] == 0 and all(a[0] + a[1] == b[0] for a, b in zip(recs, recs[1:]))
        assert recs[-1][0] + recs[-1][1] == n
        assert all(x[1] % rows == 0 for x in recs[:-1])
    # corrupt header / bad problem
    bad = (C.c_uint8 * 64)()
    expect(L.qmm_qgemv_batched(A, bad, None), INV, "not a plan image")
    probs[1] = GemvProblem(A, A, A, A, A, 1024, 3000)
    expect(L.qmm_qgemv_batched_plan(probs, 3, 4, 64, buf, need.value, C.byref(need)), INV, "problem 1")
    probs[1] = GemvProblem(A, A, A, MIS, A, 1024, 3072)
    expect(L.qmm_qgemv_batched_plan(probs, 3, 4, 64, buf, need.value, C.byref(need)), INV, "misaligned")
