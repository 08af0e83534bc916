"""Python binding over the C ABI, with torch tensors as device buffers.

Every function passes `tensor.data_ptr()` and the current HIP stream to the
matching qmm_* entry point; all arithmetic happens in the HIP kernels.
Tensor conventions (device tensors, contiguous):
  packed words  int32 [n, k*bits/32]   (or [E, n, k*bits/32] for experts)
  scales/biases int16 or float16 [n, k/64], fp16 bit patterns
  activations   float16 [m, k] (or [k] for the GEMV)
  outputs       float32
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import GemmProblem, GemvProblem, check, lib

GROUP = 64


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t: torch.Tensor, name: str, dtypes) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _sb(t, name: str, bits: int) -> int:
    """Scale or bias array; fp16 weights (bits = 16) have none (None -> NULL)."""
    if t is None and bits == 16:
        return 0
    return _dev(t, name, _SB)


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def moe_plan_dropped(plan: torch.Tensor) -> int:
    """Pairs whose expert id lay outside [0, E) when `plan` was built (the
    int32 at byte offset 16 of a routing plan or grouped workspace); their
    output rows are NaN.  Reads device memory, so it synchronizes."""
    return int(plan[16:20].view(torch.int32).item())


_W = (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)
_SB = (torch.int16, torch.float16) + ((torch.uint16,) if hasattr(torch, "uint16") else ())
_X = (torch.float16,)
_Y = (torch.float32,)


def qgemv(w, scales, biases, x, bits: int, y=None, group_size: int = GROUP, stream=None):
    """y[n] = sum_k x[k] * W_hat[n, k] via qmm_qgemv."""
    n, k = w.shape[0], x.shape[-1]
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=w.device)
    check(lib().qmm_qgemv(_dev(w, "w", _W), _sb(scales, "scales", bits), _sb(biases, "biases", bits),
                          _dev(x, "x", _X), _dev(y, "y", _Y), n, k, bits, group_size, _stream(stream)))
    return y


@dataclass
class GemvPlan:
    host: C.Array          # host image (header + block records)
    device: torch.Tensor   # device copy of the image
    keep: tuple            # tensors the plan points into

    def __len__(self):
        return len(self.keep)


def qgemv_batched_plan(problems, bits: int, group_size: int = GROUP) -> GemvPlan:
    """Build a batched-GEMV plan for a list of (w, scales, biases, x, y)."""
    arr = (GemvProblem * len(problems))()
    for i, (w, s, b, x, y) in enumerate(problems):
        arr[i] = GemvProblem(_dev(w, "w", _W), _sb(s, "scales", bits), _sb(b, "biases", bits),
                             _dev(x, "x", _X), _dev(y, "y", _Y), w.shape[0], x.shape[-1])
    need = C.c_size_t(0)
    st = lib().qmm_qgemv_batched_plan(arr, len(problems), bits, group_size, None, 0, C.byref(need))
    if st not in (_lib.QMM_OK, _lib.QMM_ERR_WORKSPACE):
        check(st)
    host = (C.c_uint8 * need.value)()
    check(lib().qmm_qgemv_batched_plan(arr, len(problems), bits, group_size, host, need.value,
                                       C.byref(need)))
    device = torch.frombuffer(bytearray(host), dtype=torch.uint8).to(problems[0][0].device)
    return GemvPlan(host=host, device=device, keep=tuple(problems))


def qgemv_batched(plan: GemvPlan, stream=None) -> None:
    check(lib().qmm_qgemv_batched(plan.device.data_ptr(), C.addressof(plan.host), _stream(stream)))


def qgemm_workspace_size(m, n, k, bits, group_size=GROUP) -> int:
    return lib().qmm_qgemm_workspace_size(m, n, k, bits, group_size)


def qgemm(w, scales, biases, x, bits: int, y=None, group_size: int = GROUP, workspace=None,
          stream=None, tiled: bool = False, scales_tiled: bool = False):
    """y[m, n] = sum_k x[m, k] * W_hat[n, k] via qmm_qgemm (tiled=True when w
    comes from repack_tiled; scales_tiled=True when scales comes from
    repack_scales_tiled, which then holds the biases too)."""
    m, k = x.shape
    n = w.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=w.device)
    ws_bytes = qgemm_workspace_size(m, n, k, bits, group_size)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=w.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(lib().qmm_qgemm(_dev(w, "w", _W), _sb(scales, "scales", bits),
                          None if scales_tiled else _sb(biases, "biases", bits),
                          _dev(x, "x", _X), _dev(y, "y", _Y), m, n, k,
                          bits | (_lib.QMM_WEIGHTS_TILED if tiled else 0)
                          | (_lib.QMM_SCALES_TILED if scales_tiled else 0), group_size,
                          ws_ptr, ws_len, _stream(stream)))
    return y


@dataclass
class GemmBatchPlan:
    host: C.Array              # host image (header, problems, tile records)
    device: torch.Tensor       # device copy of the image
    workspace: torch.Tensor    # split-k partial tiles
    keep: tuple                # tensors the plan points into

    def __len__(self):
        return len(self.keep)

    @property
    def header(self) -> dict:
        """Tile choice recorded in the image (for logs and tests)."""
        raw = bytes(self.host)[:64]
        f = __import__("struct").unpack("<IIiiiiiiiiiiQii", raw)
        return {"bits": f[2], "bm": f[4], "nb": f[5], "sbq": f[6], "count": f[7],
                "num_tiles": f[8], "split_tiles": f[9], "splits": f[10], "wtiled": f[11],
                "kw": f[13], "stiled": f[14]}


def qgemm_batched_plan(problems, bits: int, group_size: int = GROUP, tiled: bool = False,
                       scales_tiled: bool = False) -> GemmBatchPlan:
    """Plan one launch for a list of (w, scales, biases, x, y) GEMM problems;
    tiled=True when every w comes from repack_tiled, scales_tiled=True when
    every scales comes from repack_scales_tiled (biases then unused)."""
    flag_bits = bits | (_lib.QMM_WEIGHTS_TILED if tiled else 0) | (_lib.QMM_SCALES_TILED if scales_tiled else 0)
    arr = (GemmProblem * len(problems))()
    for i, (w, s, b, x, y) in enumerate(problems):
        arr[i] = GemmProblem(_dev(w, "w", _W), _sb(s, "scales", bits),
                             None if scales_tiled else _sb(b, "biases", bits),
                             _dev(x, "x", _X), _dev(y, "y", _Y), x.shape[0], w.shape[0],
                             x.shape[1])
    need, ws = C.c_size_t(0), C.c_size_t(0)
    st = lib().qmm_qgemm_batched_plan(arr, len(problems), flag_bits, group_size, None, 0,
                                      C.byref(need), C.byref(ws))
    if st not in (_lib.QMM_OK, _lib.QMM_ERR_WORKSPACE):
        check(st)
    host = (C.c_uint8 * need.value)()
    check(lib().qmm_qgemm_batched_plan(arr, len(problems), flag_bits, group_size, host, need.value,
                                       C.byref(need), C.byref(ws)))
    dev_ = problems[0][0].device
    device = torch.frombuffer(bytearray(host), dtype=torch.uint8).to(dev_)
    workspace = torch.empty(max(ws.value, 16), dtype=torch.uint8, device=dev_)
    return GemmBatchPlan(host=host, device=device, workspace=workspace, keep=tuple(problems))


def qgemm_batched(plan: GemmBatchPlan, stream=None) -> None:
    check(lib().qmm_qgemm_batched(plan.device.data_ptr(), C.addressof(plan.host),
                                  plan.workspace.data_ptr(),
                                  plan.workspace.numel() * plan.workspace.element_size(),
                                  _stream(stream)))


def qgemm_grouped_workspace_size(t, top_k, e, n, k, bits, group_size=GROUP) -> int:
    return lib().qmm_qgemm_grouped_workspace_size(t, top_k, e, n, k, bits, group_size)


def qgemm_grouped(w, scales, biases, a, expert_ids, bits: int, a_row_per_pair: bool,
                  y=None, group_size: int = GROUP, workspace=None, stream=None, plan=None,
                  tiled: bool = False, scales_tiled: bool = False):
    """Grouped MoE product via qmm_qgemm_grouped; returns y [T*top_k, n].
    With `plan` (from moe_route on the same expert_ids) it calls
    qmm_qgemm_grouped_routed and skips the bucketing.  tiled=True when w
    comes from repack_tiled (of the stacked [E*n, ...] words); scales_tiled=True
    when scales comes from repack_scales_tiled (biases then unused)."""
    flag_bits = bits | (_lib.QMM_WEIGHTS_TILED if tiled else 0) | (_lib.QMM_SCALES_TILED if scales_tiled else 0)
    if scales_tiled:
        biases = None
    e, n = w.shape[0], w.shape[1]
    t, top_k = expert_ids.shape
    k = a.shape[1]
    if y is None:
        y = torch.empty((t * top_k, n), dtype=torch.float32, device=w.device)
    if plan is not None:
        check(lib().qmm_qgemm_grouped_routed(_dev(w, "w", _W), _sb(scales, "scales", bits),
                                             (None if scales_tiled else _sb(biases, "biases", bits)), _dev(a, "a", _X),
                                             int(bool(a_row_per_pair)), plan.data_ptr(), _nbytes(plan),
                                             _dev(y, "y", _Y),
                                             t, top_k, e, n, k, flag_bits, group_size, _stream(stream)))
        return y
    ws_bytes = qgemm_grouped_workspace_size(t, top_k, e, n, k, bits, group_size)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=w.device)
    check(lib().qmm_qgemm_grouped(_dev(w, "w", _W), _sb(scales, "scales", bits),
                                  (None if scales_tiled else _sb(biases, "biases", bits)), _dev(a, "a", _X),
                                  int(bool(a_row_per_pair)), _dev(expert_ids, "expert_ids", (torch.int32,)),
                                  _dev(y, "y", _Y), t, top_k, e, n, k, flag_bits, group_size,
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream(stream)))
    return y


def qgemm_grouped_noalloc(w, scales, biases, a, expert_ids, bits: int, a_row_per_pair: bool, y,
                          group_size: int = GROUP, stream=None, tiled: bool = False,
                          scales_tiled: bool = False):
    """qmm_qgemm_grouped_noalloc: the grouped product into a caller-given y
    [T*top_k, n] with the library's static device scratch instead of a
    workspace (nothing is allocated; calls on one GPU must not overlap)."""
    flag_bits = bits | (_lib.QMM_WEIGHTS_TILED if tiled else 0) | (_lib.QMM_SCALES_TILED if scales_tiled else 0)
    e, n = w.shape[0], w.shape[1]
    t, top_k = expert_ids.shape
    k = a.shape[1]
    check(lib().qmm_qgemm_grouped_noalloc(_dev(w, "w", _W), _sb(scales, "scales", bits),
                                          (None if scales_tiled else _sb(biases, "biases", bits)), _dev(a, "a", _X),
                                          int(bool(a_row_per_pair)),
                                          _dev(expert_ids, "expert_ids", (torch.int32,)),
                                          _dev(y, "y", _Y), t, top_k, e, n, k, flag_bits, group_size,
                                          _stream(stream)))
    return y


def moe_route_size(t: int, top_k: int, e: int) -> int:
    """Bytes of the routing plan qmm_moe_route writes for (t, top_k, e)."""
    return lib().qmm_moe_route_size(t, top_k, e)


def moe_route(expert_ids, e: int, plan=None, stream=None):
    """Bucket expert_ids [T, top_k] once (qmm_moe_route); returns the plan
    tensor that qgemm_grouped(..., plan=...) reuses for every projection."""
    t, top_k = expert_ids.shape
    need = lib().qmm_moe_route_size(t, top_k, e)
    if plan is None:
        plan = torch.empty(max(need, 16), dtype=torch.uint8, device=expert_ids.device)
    check(lib().qmm_moe_route(_dev(expert_ids, "expert_ids", (torch.int32,)), t, top_k, e,
                              plan.data_ptr(), plan.numel() * plan.element_size(), _stream(stream)))
    return plan


def moe_gate_up_swiglu(gate, up, x, expert_ids, plan, bits: int, h=None, group_size: int = GROUP,
                       stream=None, tiled: bool = False, scales_tiled: bool = False):
    """h [T*top_k, n] fp16 = silu(x W_gate^T) * (x W_up^T) per pair, via
    qmm_moe_gate_up_swiglu; gate and up are (words, scales, biases), both
    from repack_tiled when tiled=True; their scales from repack_scales_tiled
    when scales_tiled=True (biases then unused)."""
    flag_bits = bits | (_lib.QMM_WEIGHTS_TILED if tiled else 0) | (_lib.QMM_SCALES_TILED if scales_tiled else 0)
    wg, sg, bg = gate
    wu, su, bu = up
    e, n = wg.shape[0], wg.shape[1]
    t, top_k = expert_ids.shape
    k = x.shape[1]
    if h is None:
        h = torch.empty((t * top_k, n), dtype=torch.float16, device=wg.device)
    check(lib().qmm_moe_gate_up_swiglu(_dev(wg, "w_gate", _W), _sb(sg, "s_gate", bits), (None if scales_tiled else _sb(bg, "b_gate", bits)),
                                       _dev(wu, "w_up", _W), _sb(su, "s_up", bits), (None if scales_tiled else _sb(bu, "b_up", bits)),
                                       _dev(x, "x", _X), plan.data_ptr(), _nbytes(plan), _dev(h, "h", _X),
                                       t, top_k, e, n, k, flag_bits, group_size, _stream(stream)))
    return h


def moe_combine(y_pairs, weights, y=None, stream=None):
    """y [T, n] = sum_j weights[t, j] * y_pairs[t*top_k + j] (slot order), via qmm_moe_combine."""
    t, top_k = weights.shape
    n = y_pairs.shape[1]
    if y is None:
        y = torch.empty((t, n), dtype=torch.float32, device=y_pairs.device)
    check(lib().qmm_moe_combine(_dev(y_pairs, "y_pairs", _Y), _dev(weights, "weights", _Y),
                                _dev(y, "y", _Y), t, top_k, n, _stream(stream)))
    return y


def convert_bf16(w_bf16, out=None, stream=None):
    """bf16 weights (torch.bfloat16, or int16 bit patterns) -> fp16 weights as
    int32 words [.., k/2] for bits = 16, via qmm_convert_bf16."""
    src = w_bf16.view(torch.int16) if w_bf16.dtype == torch.bfloat16 else w_bf16
    if not src.is_contiguous() or src.shape[-1] % 2:
        raise ValueError("w_bf16 must be contiguous with an even last dimension")
    if out is None:
        out = torch.empty(src.shape[:-1] + (src.shape[-1] // 2,), dtype=torch.int32, device=src.device)
    check(lib().qmm_convert_bf16(_dev(src, "w_bf16", _SB), out.data_ptr(), src.numel(), _stream(stream)))
    return out


def repack_tiled(w, bits: int, out=None, stream=None):
    """Tile-interleaved copy of packed weights w [n, k*bits/32] (int32) for
    the batched prefill GEMM with tiled=True, via qmm_repack_tiled."""
    n = w.numel() // w.shape[-1]  # stacked experts [E, n, words] repack as one [E*n, words]
    k = w.shape[-1] * 32 // bits
    if out is None:
        out = torch.empty_like(w)
    check(lib().qmm_repack_tiled(_dev(w, "w", _W), _dev(out, "out", _W), n, k, bits, _stream(stream)))
    return out


def repack_scales_tiled(scales, biases, out=None, stream=None):
    """Interleaved scales and biases [n, k/64] (fp16 bits, groups of 64) for
    the prefill GEMM with scales_tiled=True, via qmm_repack_scales_tiled:
    one array of 2 * n * k/64 fp16 holding both."""
    n = scales.numel() // scales.shape[-1]
    k = scales.shape[-1] * 64
    if out is None:
        out = torch.empty(2 * scales.numel(), dtype=scales.dtype, device=scales.device)
    check(lib().qmm_repack_scales_tiled(_dev(scales, "scales", _SB), _dev(biases, "biases", _SB),
                                        _dev(out, "out", _SB), n, k, _stream(stream)))
    return out


def quantize(w_f32, bits: int, group_size: int = GROUP, stream=None, out=None):
    """Quantize fp32 W [n, k] on the device -> (words int32, scales int16, biases int16);
    `out` = (words, scales, biases) writes into given tensors."""
    n, k = w_f32.shape
    if out is None:
        words = torch.empty((n, k * bits // 32), dtype=torch.int32, device=w_f32.device)
        s = torch.empty((n, k // group_size), dtype=torch.int16, device=w_f32.device)
        b = torch.empty_like(s)
    else:
        words, s, b = out
    check(lib().qmm_quantize(_dev(w_f32, "w_f32", (torch.float32,)), _dev(words, "words", _W),
                             _dev(s, "scales", _SB), _dev(b, "biases", _SB), n, k, bits, group_size,
                             _stream(stream)))
    return words, s, b


def unpack_codes(w, k: int, bits: int, stream=None, out=None):
    n = w.shape[0]
    codes = torch.empty((n, k), dtype=torch.uint8, device=w.device) if out is None else out
    check(lib().qmm_unpack_codes(_dev(w, "w", _W), _dev(codes, "codes", (torch.uint8,)), n, k, bits,
                                 _stream(stream)))
    return codes


def dequant(w, scales, biases, k: int, bits: int, out_f16: bool, group_size: int = GROUP,
            stream=None, out=None):
    n = w.shape[0]
    if out is None:
        out = torch.empty((n, k), dtype=torch.int16 if out_f16 else torch.float32, device=w.device)
    check(lib().qmm_dequant(_dev(w, "w", _W), _dev(scales, "scales", _SB), _dev(biases, "biases", _SB),
                            _dev(out, "out", (torch.int16,) if out_f16 else (torch.float32,)), int(out_f16),
                            n, k, bits, group_size, _stream(stream)))
    return out
