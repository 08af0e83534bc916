"""The allocation-free grouped product (qmm_qgemm_grouped_noalloc) against
the workspace entry point it varies (qmm_qgemm_grouped), through the C ABI.

Two calls in a row on one GPU, the second on a smaller problem (fewer
tokens, experts, columns and k) so that the static scratch still holds the
first call's bucket lists when the second runs: each result must equal the
workspace call's bit for bit (the same kernels over the same bucketing) and
the oracle within tolerance, with guard bands around y.  A problem too
large for the scratch is refused."""
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
from quantized_matmul_qgemv_amd import _lib  # noqa: E402


def _case(key, t, top_k, e, n, k, bits):
    r = np.random.default_rng(list(key))
    ids = np.ascontiguousarray(synth.topk_ids(r.standard_normal((t, e)), top_k), dtype=np.int32)
    qs = [quantized(key + (i,), n, k, bits) for i in range(e)]
    words, s, b = (np.stack([q[j] for q in qs]) for j in (2, 3, 4))
    x = synth.draw_act(key + (1000,), t, k)
    h = synth.draw_act(key + (1001,), t * top_k, k)
    return words, s, b, ids, x, h


@pytest.mark.parametrize("bits", [4, 3])
def test_noalloc_matches_workspace_call_twice(bits):
    cases = [((980, bits), 300, 8, 32, 320, 256), ((981, bits), 37, 4, 8, 96, 128)]
    for key, t, top_k, e, n, k in cases:
        words, s, b, ids, x, h = _case(key, t, top_k, e, n, k, bits)
        W, S, B, I = dev(words), dev(s), dev(b), dev(ids)
        for per_pair, a in ((False, x), (True, h)):
            say("noalloc grouped", bits, t, top_k, e, n, k, per_pair)
            A = dev(a)
            ref = qmm.qgemm_grouped(W, S, B, A, I, bits, per_pair)
            g = Guarded((t * top_k, n), torch.float32)
            qmm.qgemm_grouped_noalloc(W, S, B, A, I, bits, per_pair, g.t)
            torch.cuda.synchronize()
            g.check("noalloc y")
            assert torch.equal(g.t, ref), f"noalloc differs from the workspace call: t={t} per_pair={per_pair}"
            assert_close(host(g.t), oracle.grouped_f64(words, s, b, a, ids, bits, per_pair),
                         f"noalloc t={t} e={e} per_pair={per_pair}")


def test_noalloc_refuses_oversized_problem():
    say("noalloc oversized")
    t, top_k, e = 40000, 8, 128
    assert qmm.qgemm_grouped_workspace_size(t, top_k, e, 64, 64, 4) > _lib.QMM_GROUPED_SCRATCH_BYTES
    w = torch.zeros((e, 64, 8), dtype=torch.int32, device="cuda")
    sb = torch.zeros((e, 64, 1), dtype=torch.int16, device="cuda")
    a = torch.zeros((t, 64), dtype=torch.float16, device="cuda")
    ids = torch.zeros((t, top_k), dtype=torch.int32, device="cuda")
    y = torch.zeros((t * top_k, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.QmmError) as ei:
        qmm.qgemm_grouped_noalloc(w, sb, sb, a, ids, 4, False, y)
    assert ei.value.status == _lib.QMM_ERR_WORKSPACE and "static scratch" in str(ei.value)
