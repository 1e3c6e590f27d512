"""Python binding of libstq, the STQ1_0 sparse-ternary matmul library for MI355X.

Thin ctypes marshalling over the C ABI in ``include/stq.h``: every function
takes torch tensors that already live on the GPU, passes their device
pointers and the current HIP stream, and checks the returned status.  All
computation happens in the HIP kernels of ``libstq.so``; there is no
fallback.  If the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "QK", "BLOCK_BYTES", "ENC_WLS", "ENC_AMAX", "StqError", "lib", "lib_path",
    "row_bytes", "quantize_rows", "dequantize_rows", "gemv", "gemv_noalloc", "gemv_plan", "grouped_gemm",
    "moe_ffn_decode",
    "moe_ffn_workspace", "layer_errors", "layer_errors_workspace", "q2_roundtrip", "greedy_allocation",
    "stream_read_probe", "mfma_loop_probe", "lds_read_probe", "MFMA_PROBE_FLOP_PER_ROUND",
    "LDS_PROBE_READS_PER_ROUND",
]

QK = 256
BLOCK_BYTES = 42
ENC_WLS, ENC_AMAX = 0, 1
X_F32, X_BF16 = 0, 1
# work of one round of the measurement probes (include/stq.h)
MFMA_PROBE_FLOP_PER_ROUND = 2147483648.0
LDS_PROBE_READS_PER_ROUND = 131072

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libstq.so")
_lib = None

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_vp = ctypes.c_void_p


class StqError(RuntimeError):
    """A libstq entry point returned a status other than STQ_OK."""

    def __init__(self, func: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{func} failed with status {status}: {detail}")


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libstq.so (built in-tree by ``python -m sparse_ternary_bit_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m sparse_ternary_bit_amd.build` first")
    L = ctypes.CDLL(_LIB_PATH)
    L.stq_row_bytes.argtypes = [_c_i64]
    L.stq_row_bytes.restype = _c_i64
    L.stq_status_string.argtypes = [_c_int]
    L.stq_status_string.restype = ctypes.c_char_p
    L.stq_last_error.argtypes = []
    L.stq_last_error.restype = ctypes.c_char_p
    L.stq_quantize_rows.argtypes = [_c_vp, _c_vp, _c_i64, _c_i64, _c_int, _c_int, _c_vp, _c_vp]
    L.stq_quantize_rows.restype = _c_int
    L.stq_dequantize_rows.argtypes = [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp]
    L.stq_dequantize_rows.restype = _c_int
    L.stq_gemv.argtypes = [_c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_int, _c_i64, _c_i64,
                           _c_vp, _c_vp, _c_i64, _c_vp, _c_vp, _c_i64, _c_vp]
    L.stq_gemv.restype = _c_int
    L.stq_gemv_noalloc.argtypes = [_c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_int, _c_i64, _c_i64,
                                   _c_vp, _c_vp, _c_i64, _c_vp, _c_vp]
    L.stq_gemv_noalloc.restype = _c_int
    L.stq_gemv_plan.argtypes = [_c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(_c_i64)]
    L.stq_gemv_plan.restype = _c_int
    L.stq_grouped_gemm.argtypes = [_c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_i64, _c_vp, _c_vp]
    L.stq_grouped_gemm.restype = _c_int
    L.stq_moe_ffn_decode.argtypes = [_c_vp, _c_i64, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_i64,
                                     _c_vp, _c_vp, _c_i64, _c_vp, _c_vp, _c_i64, _c_vp]
    L.stq_moe_ffn_decode.restype = _c_int
    L.stq_moe_ffn_workspace.argtypes = [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_int32,
                                        ctypes.POINTER(_c_i64)]
    L.stq_moe_ffn_workspace.restype = _c_int
    L.stq_layer_errors.argtypes = [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_vp, _c_vp, _c_i64,
                                   _c_vp]
    L.stq_layer_errors.restype = _c_int
    L.stq_layer_errors_workspace.argtypes = [_c_i64, _c_i64, _c_i64, ctypes.POINTER(_c_i64)]
    L.stq_layer_errors_workspace.restype = _c_int
    L.stq_q2_roundtrip.argtypes = [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp]
    L.stq_q2_roundtrip.restype = _c_int
    L.stq_greedy_allocation.argtypes = [_c_vp, _c_vp, _c_i64, ctypes.c_double, _c_vp]
    L.stq_greedy_allocation.restype = _c_int
    L.stq_stream_read_probe.argtypes = [_c_vp, _c_i64, _c_vp, _c_vp]
    L.stq_stream_read_probe.restype = _c_int
    L.stq_mfma_loop_probe.argtypes = [_c_i64, _c_vp, _c_vp]
    L.stq_mfma_loop_probe.restype = _c_int
    L.stq_lds_read_probe.argtypes = [_c_int, _c_i64, _c_vp, _c_vp]
    L.stq_lds_read_probe.restype = _c_int
    _lib = L
    return L


def _check(func: str, status: int) -> None:
    if status != 0:
        raise StqError(func, status, lib().stq_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


_CUS: dict = {}


def _device_cus(device) -> int:
    """Compute units of a GPU tensor's device, the count the library plans the GEMV for."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if idx not in _CUS:
        _CUS[idx] = torch.cuda.get_device_properties(idx).multi_processor_count
    return _CUS[idx]


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _on_gpu(name: str, t: torch.Tensor, dtype: torch.dtype) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _holds(name: str, t: torch.Tensor, n: int) -> None:
    """The kernels index raw pointers: a buffer smaller than the shapes say would be read or
    written past its end, so it is refused here."""
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n}")


def _workspace(ws: torch.Tensor | None, need: int, device) -> torch.Tensor | None:
    """A caller's workspace (checked) or a new one from torch's caching allocator; its memory
    is ordered on the current stream, like every other tensor the call takes."""
    if ws is None:
        return torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return ws


def _ws_args(ws: torch.Tensor | None) -> tuple:
    return (None, 0) if ws is None else (ws.data_ptr(), ws.numel() * ws.element_size())


def _table(name: str, t: torch.Tensor, n_experts: int, stride: int, n: int, k: int) -> None:
    if n_experts > 0 and n > 0:
        _holds(name, t, (int(n_experts) - 1) * int(stride) + int(n) * row_bytes(k))


def row_bytes(k: int) -> int:
    rb = lib().stq_row_bytes(int(k))
    if rb < 0:
        raise ValueError("k must be a positive multiple of 256")
    return rb


def quantize_rows(w: torch.Tensor, imatrix: torch.Tensor | None = None, encoder: int = ENC_WLS,
                  rounds: int = 3, out: torch.Tensor | None = None) -> torch.Tensor:
    """Encode fp32 rows [n, k] on the GPU into a packed matrix (flat uint8, n*k/256*42 bytes,
    64-row tiles, block-major inside a tile)."""
    _on_gpu("w", w, torch.float32)
    n, k = w.shape
    if imatrix is not None:
        _on_gpu("imatrix", imatrix, torch.float32)
        _holds("imatrix", imatrix, k)
    if out is None:
        out = torch.empty(n * row_bytes(k), dtype=torch.uint8, device=w.device)
    _on_gpu("out", out, torch.uint8)
    if out.numel() < n * row_bytes(k):
        raise ValueError("out must hold n*k/256*42 bytes")
    _check("stq_quantize_rows", lib().stq_quantize_rows(w.data_ptr(), _ptr(imatrix), n, k, int(encoder),
                                                        int(rounds), out.data_ptr(), _stream()))
    return out


def dequantize_rows(q: torch.Tensor, n: int, k: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Decode a packed matrix of n rows to fp32 [n, k]."""
    _on_gpu("q", q, torch.uint8)
    if q.numel() < n * row_bytes(k):
        raise ValueError("q must hold n*k/256*42 bytes")
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=q.device)
    _on_gpu("out", out, torch.float32)
    _holds("out", out, n * k)
    _check("stq_dequantize_rows", lib().stq_dequantize_rows(q.data_ptr(), n, k, out.data_ptr(), _stream()))
    return out


def gemv_plan(n_experts: int, n: int, k: int, n_pairs: int, n_cus: int = 0) -> tuple[int, int, int]:
    """(splits, max_parts, scratch_bytes) that gemv takes for these shapes on n_cus
    compute units (0: the current device's); host only."""
    sp, mp, sb = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check("stq_gemv_plan", lib().stq_gemv_plan(int(n_experts), int(n), int(k), int(n_pairs), int(n_cus),
                                                ctypes.byref(sp), ctypes.byref(mp), ctypes.byref(sb)))
    return sp.value, mp.value, sb.value


def gemv(w_table: torch.Tensor, expert_stride: int, n_experts: int, n: int, k: int, x: torch.Tensor,
         pair_expert: torch.Tensor | None = None, pair_token: torch.Tensor | None = None,
         n_pairs: int | None = None, out: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y[i] = W_{pair_expert[i]} x[pair_token[i]] for every pair; x is [n_tokens, k] fp32 or bf16.
    `workspace` (GPU bytes, at least gemv_plan(...)[2]) is allocated here when not given."""
    _on_gpu("w_table", w_table, torch.uint8)
    if x.dtype == torch.bfloat16:
        xd = X_BF16
    elif x.dtype == torch.float32:
        xd = X_F32
    else:
        raise ValueError("x must be float32 or bfloat16")
    _on_gpu("x", x, x.dtype)
    n_tokens = x.shape[0]
    if n_pairs is None:
        if pair_expert is not None:
            n_pairs = pair_expert.numel()
        elif pair_token is not None:
            n_pairs = pair_token.numel()
        else:
            n_pairs = n_tokens
    for nm, t in (("pair_expert", pair_expert), ("pair_token", pair_token)):
        if t is not None:
            _on_gpu(nm, t, torch.int32)
            if t.numel() != n_pairs:
                raise ValueError(f"{nm} must hold n_pairs entries")
    if out is None:
        out = torch.empty((n_pairs, n), dtype=torch.float32, device=x.device)
    _on_gpu("out", out, torch.float32)
    _holds("out", out, int(n_pairs) * int(n))
    if int(n_pairs) > 0:
        _table("w_table", w_table, n_experts, expert_stride, n, k)
    # a one-row view may carry any stride in its first dimension; its rows are k apart
    x_stride = x.stride(0) if n_tokens > 1 else x.shape[1]
    if workspace is None and int(n_pairs) > 0 and int(n) > 0:
        need = gemv_plan(n_experts, n, k, n_pairs, _device_cus(x.device))[2]
        workspace = _workspace(None, need, x.device)
    else:
        workspace = _workspace(workspace, 0, x.device)
    _check("stq_gemv", lib().stq_gemv(w_table.data_ptr(), int(expert_stride), int(n_experts), int(n), int(k),
                                      x.data_ptr(), xd, x_stride, n_tokens, _ptr(pair_expert),
                                      _ptr(pair_token), int(n_pairs), out.data_ptr(), *_ws_args(workspace),
                                      _stream()))
    return out


def gemv_noalloc(w_table: torch.Tensor, expert_stride: int, n_experts: int, n: int, k: int, x: torch.Tensor,
                 pair_expert: torch.Tensor | None, pair_token: torch.Tensor | None, out: torch.Tensor) -> torch.Tensor:
    """gemv without any allocation (neither here nor in the library): the caller passes `out`
    [n_pairs, n] fp32; split outputs use the library's fixed per-GPU scratch, so calls on one
    GPU must not overlap.  Shapes needing more scratch than it holds raise."""
    _on_gpu("w_table", w_table, torch.uint8)
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be float32 or bfloat16")
    _on_gpu("x", x, x.dtype)
    _on_gpu("out", out, torch.float32)
    n_tokens = x.shape[0]
    n_pairs = out.shape[0]
    for nm, t in (("pair_expert", pair_expert), ("pair_token", pair_token)):
        if t is not None:
            _on_gpu(nm, t, torch.int32)
            if t.numel() != n_pairs:
                raise ValueError(f"{nm} must hold out.shape[0] entries")
    _holds("out", out, int(n_pairs) * int(n))
    if int(n_pairs) > 0:
        _table("w_table", w_table, n_experts, expert_stride, n, k)
    x_stride = x.stride(0) if n_tokens > 1 else x.shape[1]
    _check("stq_gemv_noalloc",
           lib().stq_gemv_noalloc(w_table.data_ptr(), int(expert_stride), int(n_experts), int(n), int(k),
                                  x.data_ptr(), X_BF16 if x.dtype == torch.bfloat16 else X_F32, x_stride, n_tokens,
                                  _ptr(pair_expert), _ptr(pair_token), int(n_pairs), out.data_ptr(), _stream()))
    return out


def grouped_gemm(w_table: torch.Tensor, expert_stride: int, n_experts: int, n: int, k: int,
                 x_sorted: torch.Tensor, offsets: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Y[rows of e] = X[rows of e] W_e^T with rows grouped by expert; x_sorted bf16 [total_m, k]."""
    _on_gpu("w_table", w_table, torch.uint8)
    _on_gpu("x_sorted", x_sorted, torch.bfloat16)
    _on_gpu("offsets", offsets, torch.int32)
    if offsets.numel() != n_experts + 1:
        raise ValueError("offsets must hold n_experts + 1 entries")
    if x_sorted.dim() != 2 or x_sorted.shape[1] != k:
        raise ValueError("x_sorted must be [total_m, k]")
    total_m = x_sorted.shape[0]
    if out is None:
        out = torch.empty((total_m, n), dtype=torch.float32, device=x_sorted.device)
    _on_gpu("out", out, torch.float32)
    _holds("out", out, total_m * int(n))
    if total_m > 0:
        _table("w_table", w_table, n_experts, expert_stride, n, k)
    _check("stq_grouped_gemm", lib().stq_grouped_gemm(w_table.data_ptr(), int(expert_stride), int(n_experts),
                                                      int(n), int(k), x_sorted.data_ptr(), offsets.data_ptr(),
                                                      total_m, out.data_ptr(), _stream()))
    return out


def moe_ffn_workspace(n_experts: int, d_model: int, d_ff: int, n_tokens: int, top_k: int, n_cus: int = 0) -> int:
    """Workspace bytes moe_ffn_decode needs for these shapes on n_cus compute units (0: the
    current device's); host only."""
    wb = ctypes.c_int64()
    _check("stq_moe_ffn_workspace", lib().stq_moe_ffn_workspace(int(n_experts), int(d_model), int(d_ff),
                                                                int(n_tokens), int(top_k), int(n_cus),
                                                                ctypes.byref(wb)))
    return wb.value


def moe_ffn_decode(w_gate_up: torch.Tensor, gate_up_stride: int, w_down: torch.Tensor, down_stride: int,
                   n_experts: int, d_model: int, d_ff: int, x: torch.Tensor, pair_expert: torch.Tensor,
                   pair_weight: torch.Tensor, top_k: int, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Routed-expert FFN for decode tokens x bf16 [T, d_model]: per token, the routing-weighted sum
    over its top_k pairs of W_down_e (silu(W_gate_e x) * (W_up_e x)); pairs token-major [T*top_k].
    `workspace` (GPU bytes, at least moe_ffn_workspace(...)) is allocated here when not given."""
    _on_gpu("w_gate_up", w_gate_up, torch.uint8)
    _on_gpu("w_down", w_down, torch.uint8)
    _on_gpu("x", x, torch.bfloat16)
    _on_gpu("pair_expert", pair_expert, torch.int32)
    _on_gpu("pair_weight", pair_weight, torch.float32)
    if x.dim() != 2 or x.shape[1] != d_model:
        raise ValueError("x must be [n_tokens, d_model]")
    n_tokens = x.shape[0]
    if pair_expert.numel() != n_tokens * top_k or pair_weight.numel() != n_tokens * top_k:
        raise ValueError("pair_expert and pair_weight must hold n_tokens*top_k entries")
    if out is None:
        out = torch.empty((n_tokens, d_model), dtype=torch.float32, device=x.device)
    _on_gpu("out", out, torch.float32)
    _holds("out", out, n_tokens * int(d_model))
    if n_tokens > 0:
        _table("w_gate_up", w_gate_up, n_experts, gate_up_stride, 2 * int(d_ff), d_model)
        _table("w_down", w_down, n_experts, down_stride, d_model, d_ff)
    if workspace is None and n_tokens > 0:
        need = moe_ffn_workspace(n_experts, d_model, d_ff, n_tokens, top_k, _device_cus(x.device))
        workspace = _workspace(None, need, x.device)
    else:
        workspace = _workspace(workspace, 0, x.device)
    _check("stq_moe_ffn_decode",
           lib().stq_moe_ffn_decode(w_gate_up.data_ptr(), int(gate_up_stride), w_down.data_ptr(), int(down_stride),
                                    int(n_experts), int(d_model), int(d_ff), x.data_ptr(), n_tokens,
                                    pair_expert.data_ptr(), pair_weight.data_ptr(), int(top_k), out.data_ptr(),
                                    *_ws_args(workspace), _stream()))
    return out


def layer_errors_workspace(n_rows: int, k: int, n_calib: int) -> int:
    """Workspace bytes layer_errors needs for these shapes (host only)."""
    wb = ctypes.c_int64()
    _check("stq_layer_errors_workspace", lib().stq_layer_errors_workspace(int(n_rows), int(k), int(n_calib),
                                                                          ctypes.byref(wb)))
    return wb.value


def layer_errors(w: torch.Tensor, w_hat: torch.Tensor, x_calib: torch.Tensor,
                 out_full: torch.Tensor | None = None, out_diag: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None):
    """Per-row error of w_hat against w under calibration rows x_calib fp32 [N, k]: full-Hessian
    sum_i ((w - w_hat) . x_i)^2 and diagonal sum_c H_cc (w - w_hat)_c^2, both fp64 [n].
    `workspace` (GPU bytes, at least layer_errors_workspace(...)) is allocated here when not given."""
    _on_gpu("w", w, torch.float32)
    _on_gpu("w_hat", w_hat, torch.float32)
    _on_gpu("x_calib", x_calib, torch.float32)
    n, k = w.shape
    if tuple(w_hat.shape) != (n, k) or x_calib.dim() != 2 or x_calib.shape[1] != k:
        raise ValueError("w, w_hat must be [n, k] and x_calib [N, k]")
    if out_full is None:
        out_full = torch.empty(n, dtype=torch.float64, device=w.device)
    if out_diag is None:
        out_diag = torch.empty(n, dtype=torch.float64, device=w.device)
    _on_gpu("out_full", out_full, torch.float64)
    _on_gpu("out_diag", out_diag, torch.float64)
    if out_full.numel() < n or out_diag.numel() < n:
        raise ValueError("outputs must hold n entries")
    if workspace is None and n > 0 and x_calib.shape[0] > 0:
        workspace = _workspace(None, layer_errors_workspace(n, k, x_calib.shape[0]), w.device)
    else:
        workspace = _workspace(workspace, 0, w.device)
    _check("stq_layer_errors", lib().stq_layer_errors(w.data_ptr(), w_hat.data_ptr(), n, k, x_calib.data_ptr(),
                                                      x_calib.shape[0], out_full.data_ptr(), out_diag.data_ptr(),
                                                      *_ws_args(workspace), _stream()))
    return out_full, out_diag


def q2_roundtrip(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Reconstruction of fp32 rows [n, k] through the 2-bit stand-in format (fp16 rms/2 scale per
    256 weights, levels +-s, +-3s)."""
    _on_gpu("w", w, torch.float32)
    n, k = w.shape
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    _on_gpu("out", out, torch.float32)
    if tuple(out.shape) != (n, k):
        raise ValueError("out must be [n, k]")
    _check("stq_q2_roundtrip", lib().stq_q2_roundtrip(w.data_ptr(), n, k, out.data_ptr(), _stream()))
    return out


def greedy_allocation(gain, extra_bytes, budget: float):
    """Layers to move to the larger format, taken by error reduction per added byte within
    `budget` bytes (host function; numpy in, numpy bool mask out)."""
    import numpy as np
    g = np.ascontiguousarray(gain, dtype=np.float64)
    e = np.ascontiguousarray(extra_bytes, dtype=np.float64)
    if g.shape != e.shape or g.ndim != 1:
        raise ValueError("gain and extra_bytes must be 1-D of equal length")
    chosen = np.zeros(g.shape[0], dtype=np.uint8)
    _check("stq_greedy_allocation", lib().stq_greedy_allocation(g.ctypes.data, e.ctypes.data, g.shape[0],
                                                                float(budget), chosen.ctypes.data))
    return chosen.astype(bool)


def stream_read_probe(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Read every byte of the GPU tensor `buf` once (a streaming-read rate
    reference for the HBM roofline); `sink` is a one-element int32 GPU tensor."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    _on_gpu("sink", sink, torch.int32)
    nbytes = buf.numel() * buf.element_size()
    _check("stq_stream_read_probe", lib().stq_stream_read_probe(buf.data_ptr(), nbytes - nbytes % 16,
                                                                sink.data_ptr(), _stream()))


def mfma_loop_probe(rounds: int, sink: torch.Tensor) -> None:
    """Matrix-core reference: MFMA_PROBE_FLOP_PER_ROUND * rounds flops of
    bf16 MFMAs with no memory traffic; `sink` is a one-element float32 GPU tensor."""
    _on_gpu("sink", sink, torch.float32)
    _check("stq_mfma_loop_probe", lib().stq_mfma_loop_probe(int(rounds), sink.data_ptr(), _stream()))


def lds_read_probe(mode: int, rounds: int, sink: torch.Tensor) -> None:
    """LDS read reference: LDS_PROBE_READS_PER_ROUND * rounds wavefront LDS
    reads, 16-byte contiguous (mode 0) or two 4-byte table reads at a code
    (mode 1); `sink` is a one-element int32 GPU tensor."""
    _on_gpu("sink", sink, torch.int32)
    _check("stq_lds_read_probe", lib().stq_lds_read_probe(int(mode), int(rounds), sink.data_ptr(), _stream()))
