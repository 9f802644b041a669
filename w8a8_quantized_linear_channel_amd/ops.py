"""Thin torch binding of the libq8 C ABI, one Python function per C call and
with the same name.  It checks tensor devices/dtypes/shapes, allocates
outputs and the workspace with torch, passes raw device pointers and the
current HIP stream, and turns a non-OK status into an exception.  All
arithmetic happens in the HIP kernels."""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib

_DT = {torch.float32: _lib.Q8_F32, torch.float16: _lib.Q8_F16, torch.bfloat16: _lib.Q8_BF16}
_FMT = {"int8_asym": _lib.Q8_INT8_ASYM, "int8_sym": _lib.Q8_INT8_SYM, "fp8_e4m3": _lib.Q8_FP8_E4M3}
_OP = {"linear": _lib.Q8_OP_LINEAR, "decomp": _lib.Q8_OP_DECOMP, "fp8": _lib.Q8_OP_FP8,
       "static": _lib.Q8_OP_STATIC, "grouped": _lib.Q8_OP_GROUPED}


class _DtypeCodes(dict):
    """torch dtype -> q8_dtype code; an unsupported dtype is a TypeError that
    names the supported ones."""

    def __missing__(self, key):
        raise TypeError(f"unsupported dtype {key}: expected torch.float32, torch.float16 or torch.bfloat16")


_DT = _DtypeCodes(_DT)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, dev=None) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


def q8_workspace_bytes(op: str, M: int, N: int, K: int) -> int:
    return int(_lib.lib().q8_workspace_bytes(_OP[op], M, N, K))


def _workspace(op: str, M: int, N: int, K: int, dev) -> torch.Tensor:
    n = q8_workspace_bytes(op, M, N, K)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=dev)


def q8_quantize_weight(w: torch.Tensor, fmt: str = "int8_asym"):
    """Per-output-channel weight quantization.  Returns (wq, scale, zero_point);
    zero_point is None for "fp8_e4m3" (codes are returned as uint8)."""
    _need(w, "w")
    if w.dim() != 2 or w.dtype not in _DT:
        raise ValueError("w must be 2-D float32/float16/bfloat16")
    N, K = w.shape
    dev = w.device
    if fmt == "int8_asym":
        wq = torch.empty(N, K, dtype=torch.int8, device=dev)
        zp = torch.empty(N, dtype=torch.float32, device=dev)
    elif fmt == "fp8_e4m3":
        wq = torch.empty(N, K, dtype=torch.uint8, device=dev)
        zp = None
    else:
        raise ValueError(f"unsupported weight format {fmt}")
    scale = torch.empty(N, dtype=torch.float32, device=dev)
    st = _lib.lib().q8_quantize_weight(_FMT[fmt], _ptr(w), _DT[w.dtype], N, K, _ptr(wq), _ptr(scale),
                                       _ptr(zp), _stream(dev))
    _lib.check("q8_quantize_weight", st)
    return wq, scale, zp


def q8_quantize_act(x: torch.Tensor, fmt: str = "int8_sym", scale_ub: float = math.inf,
                    rowsum: bool = True, out=None):
    """Dynamic per-token quantization.  Returns (xq, scale, rowsum or None);
    `out` may supply those three tensors preallocated."""
    _need(x, "x")
    if x.dim() != 2 or x.dtype not in _DT:
        raise ValueError("x must be 2-D float32/float16/bfloat16")
    M, K = x.shape
    dev = x.device
    if fmt not in ("int8_sym", "fp8_e4m3"):
        raise ValueError(f"unsupported activation format {fmt}")
    code_dt = torch.int8 if fmt == "int8_sym" else torch.uint8
    if out is not None:
        xq, scale, rs = out
        _need(xq, "xq", code_dt, (M, K), dev)
        _need(scale, "scale", torch.float32, (M,), dev)
        if rs is not None:
            _need(rs, "rowsum", torch.int32, (M,), dev)
    else:
        xq = torch.empty(M, K, dtype=code_dt, device=dev)
        scale = torch.empty(M, dtype=torch.float32, device=dev)
        rs = torch.empty(M, dtype=torch.int32, device=dev) if (rowsum and fmt == "int8_sym") else None
    st = _lib.lib().q8_quantize_act(_FMT[fmt], _ptr(x), _DT[x.dtype], M, K, float(scale_ub), _ptr(xq),
                                    _ptr(scale), _ptr(rs), _stream(dev))
    _lib.check("q8_quantize_act", st)
    return xq, scale, rs


def q8_linear(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor, w_zp: torch.Tensor,
              bias: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
              acc_out: bool = False, workspace: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None):
    """W8A8 linear.  Returns y (and the INT32 accumulator if acc_out)."""
    _need(x, "x")
    dev = x.device
    M, K = x.shape
    N = wq.shape[0]
    _need(wq, "wq", torch.int8, (N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (N,), dev)
    _need(w_zp, "w_zp", torch.float32, (N,), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (N,), dev)
    out_dtype = out_dtype or x.dtype
    y = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=dev)
    _need(y, "y", out_dtype, (M, N), dev)
    acc = torch.empty(M, N, dtype=torch.int32, device=dev) if acc_out else None
    ws = workspace if workspace is not None else _workspace("linear", M, N, K, dev)
    st = _lib.lib().q8_linear(_ptr(x), _DT[x.dtype], M, K, _ptr(wq), _ptr(w_scale), _ptr(w_zp), N,
                              _ptr(bias), _ptr(y), _DT[out_dtype], _ptr(ws), ws.numel(), _ptr(acc),
                              _stream(dev))
    _lib.check("q8_linear", st)
    return (y, acc) if acc_out else y


def q8_linear_noalloc(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor, w_zp: torch.Tensor,
                      bias: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                      acc_out: bool = False, out: Optional[torch.Tensor] = None):
    """q8_linear without a workspace (the library's own scratch array); with
    `out` (and acc_out False) the binding allocates nothing either.  Returns y
    (and the INT32 accumulator if acc_out)."""
    _need(x, "x")
    dev = x.device
    M, K = x.shape
    N = wq.shape[0]
    _need(wq, "wq", torch.int8, (N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (N,), dev)
    _need(w_zp, "w_zp", torch.float32, (N,), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (N,), dev)
    out_dtype = out_dtype or x.dtype
    y = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=dev)
    _need(y, "y", out_dtype, (M, N), dev)
    acc = torch.empty(M, N, dtype=torch.int32, device=dev) if acc_out else None
    st = _lib.lib().q8_linear_noalloc(_ptr(x), _DT[x.dtype], M, K, _ptr(wq), _ptr(w_scale), _ptr(w_zp), N,
                                      _ptr(bias), _ptr(y), _DT[out_dtype], _ptr(acc), _stream(dev))
    _lib.check("q8_linear_noalloc", st)
    return (y, acc) if acc_out else y


def q8_linear_int8_decomp(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                          w_zp: torch.Tensor, threshold: float = 6.0,
                          bias: Optional[torch.Tensor] = None, return_outliers: bool = False,
                          acc_out: bool = False, workspace: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None):
    """LLM.int8() decomposition.  Returns y, plus (outlier_idx, n_outliers)
    device tensors if return_outliers, plus the int8-path accumulator if acc_out."""
    _need(x, "x", torch.float16)
    dev = x.device
    M, K = x.shape
    N = wq.shape[0]
    _need(wq, "wq", torch.int8, (N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (N,), dev)
    _need(w_zp, "w_zp", torch.float32, (N,), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (N,), dev)
    y = out if out is not None else torch.empty(M, N, dtype=torch.float16, device=dev)
    _need(y, "y", torch.float16, (M, N), dev)
    idx = torch.empty(K, dtype=torch.int32, device=dev) if return_outliers else None
    cnt = torch.empty(1, dtype=torch.int32, device=dev) if return_outliers else None
    acc = torch.empty(M, N, dtype=torch.int32, device=dev) if acc_out else None
    ws = workspace if workspace is not None else _workspace("decomp", M, N, K, dev)
    st = _lib.lib().q8_linear_int8_decomp(_ptr(x), M, K, _ptr(wq), _ptr(w_scale), _ptr(w_zp), N,
                                          float(threshold), _ptr(bias), _ptr(y), _ptr(ws), ws.numel(),
                                          _ptr(idx), _ptr(cnt), _ptr(acc), _stream(dev))
    _lib.check("q8_linear_int8_decomp", st)
    res = [y]
    if return_outliers:
        res += [idx, cnt]
    if acc_out:
        res.append(acc)
    return res[0] if len(res) == 1 else tuple(res)


def q8_linear_fp8(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                  scale_ub: float = 1200.0, bias: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """FP8 e4m3 W8A8 rowwise linear (bf16 in, bf16 out)."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    M, K = x.shape
    N = wq.shape[0]
    _need(wq, "wq", torch.uint8, (N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (N,), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (N,), dev)
    y = out if out is not None else torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, (M, N), dev)
    ws = workspace if workspace is not None else _workspace("fp8", M, N, K, dev)
    st = _lib.lib().q8_linear_fp8(_ptr(x), M, K, _ptr(wq), _ptr(w_scale), N, float(scale_ub), _ptr(bias),
                                  _ptr(y), _ptr(ws), ws.numel(), _stream(dev))
    _lib.check("q8_linear_fp8", st)
    return y


def q8_gemm_int8(xq: torch.Tensor, x_scale: torch.Tensor, x_rowsum: torch.Tensor, wq: torch.Tensor,
                 w_scale: torch.Tensor, w_zp: torch.Tensor, bias: Optional[torch.Tensor] = None,
                 out_dtype: torch.dtype = torch.bfloat16, acc_out: bool = False,
                 out: Optional[torch.Tensor] = None):
    """INT8 GEMM + dequantization epilogue on pre-quantized activations."""
    _need(xq, "xq", torch.int8)
    dev = xq.device
    M, K = xq.shape
    N = wq.shape[0]
    _need(x_scale, "x_scale", torch.float32, (M,), dev)
    _need(x_rowsum, "x_rowsum", torch.int32, (M,), dev)
    _need(wq, "wq", torch.int8, (N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (N,), dev)
    _need(w_zp, "w_zp", torch.float32, (N,), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (N,), dev)
    y = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=dev)
    _need(y, "y", out_dtype, (M, N), dev)
    acc = torch.empty(M, N, dtype=torch.int32, device=dev) if acc_out else None
    st = _lib.lib().q8_gemm_int8(_ptr(xq), _ptr(x_scale), _ptr(x_rowsum), M, K, _ptr(wq), _ptr(w_scale),
                                 _ptr(w_zp), N, _ptr(bias), _ptr(y), _DT[out_dtype], _ptr(acc),
                                 _stream(dev))
    _lib.check("q8_gemm_int8", st)
    return (y, acc) if acc_out else y


def q8_gemm_fp8(xq: torch.Tensor, x_scale: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """Rowwise FP8 GEMM on e4m3 codes (bf16 out)."""
    _need(xq, "xq", torch.uint8)
    dev = xq.device
    M, K = xq.shape
    N = wq.shape[0]
    _need(x_scale, "x_scale", torch.float32, (M,), dev)
    _need(wq, "wq", torch.uint8, (N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (N,), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (N,), dev)
    y = out if out is not None else torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, (M, N), dev)
    st = _lib.lib().q8_gemm_fp8(_ptr(xq), _ptr(x_scale), M, K, _ptr(wq), _ptr(w_scale), N, _ptr(bias),
                                _ptr(y), _stream(dev))
    _lib.check("q8_gemm_fp8", st)
    return y


def q8_linear_w8a16(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor, w_zp: torch.Tensor,
                    bias: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                    out: Optional[torch.Tensor] = None):
    """Weight-only W8A16 linear for up to 16 tokens: y = x . (S_w (Wq - Z_w))^T (+ bias),
    x bf16 or fp16, weights from q8_quantize_weight("int8_asym")."""
    dev = x.device
    M, K = x.shape
    N = wq.shape[0]
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q8_linear_w8a16: x must be bfloat16 or float16")
    _need(x, "x", x.dtype, (M, K), dev)
    _need(wq, "wq", torch.int8, (N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (N,), dev)
    _need(w_zp, "w_zp", torch.float32, (N,), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (N,), dev)
    y = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=dev)
    _need(y, "y", out_dtype, (M, N), dev)
    st = _lib.lib().q8_linear_w8a16(_ptr(x), _DT[x.dtype], M, K, _ptr(wq), _ptr(w_scale), _ptr(w_zp), N,
                                    _ptr(bias), _ptr(y), _DT[out_dtype], _stream(dev))
    _lib.check("q8_linear_w8a16", st)
    return y


def q8_quantize_act_static(x: torch.Tensor, x_scale: float, out=None):
    """Static INT8 codes with one calibrated scale: (xq int8 [M,K], rowsum int32 [M])."""
    dev = x.device
    M, K = x.shape
    _need(x, "x", x.dtype, (M, K), dev)
    xq, rs = out if out is not None else (torch.empty(M, K, dtype=torch.int8, device=dev),
                                          torch.empty(M, dtype=torch.int32, device=dev))
    _need(xq, "xq", torch.int8, (M, K), dev)
    _need(rs, "x_rowsum", torch.int32, (M,), dev)
    st = _lib.lib().q8_quantize_act_static(_ptr(x), _DT[x.dtype], M, K, float(x_scale), _ptr(xq), _ptr(rs),
                                           _stream(dev))
    _lib.check("q8_quantize_act_static", st)
    return xq, rs


def q8_linear_static(x: torch.Tensor, x_scale: float, wq: torch.Tensor, w_scale: torch.Tensor,
                     w_zp: torch.Tensor, y_scale: float, bias: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """W8A8 linear with a static activation scale and INT8 output codes (scale y_scale)."""
    dev = x.device
    M, K = x.shape
    N = wq.shape[0]
    _need(x, "x", x.dtype, (M, K), dev)
    _need(wq, "wq", torch.int8, (N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (N,), dev)
    _need(w_zp, "w_zp", torch.float32, (N,), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (N,), dev)
    yq = out if out is not None else torch.empty(M, N, dtype=torch.int8, device=dev)
    _need(yq, "yq", torch.int8, (M, N), dev)
    ws = workspace if workspace is not None else _workspace("static", M, N, K, dev)
    st = _lib.lib().q8_linear_static(_ptr(x), _DT[x.dtype], M, K, float(x_scale), _ptr(wq), _ptr(w_scale),
                                     _ptr(w_zp), N, _ptr(bias), float(y_scale), _ptr(yq), _ptr(ws),
                                     ws.numel(), _stream(dev))
    _lib.check("q8_linear_static", st)
    return yq


def q8_linear_fp8_grouped(x: torch.Tensor, expert_offsets: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                          scale_ub: float = 1200.0, out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None):
    """FP8 expert projection on routed tokens: x bf16 [T,K] grouped by expert,
    expert_offsets int32 [E+1] on the device, wq e4m3 [E,N,K], w_scale [E,N]."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    T, K = x.shape
    E, N = wq.shape[0], wq.shape[1]
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    _need(wq, "wq", torch.uint8, (E, N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (E, N), dev)
    y = out if out is not None else torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, (T, N), dev)
    ws = workspace if workspace is not None else _workspace("fp8", T, N, K, dev)
    st = _lib.lib().q8_linear_fp8_grouped(_ptr(x), T, K, _ptr(expert_offsets), E, _ptr(wq), _ptr(w_scale), N,
                                          float(scale_ub), _ptr(y), _ptr(ws), ws.numel(), _stream(dev))
    _lib.check("q8_linear_fp8_grouped", st)
    return y


def q8_quantize_weight_grouped(w: torch.Tensor, group: int = 128):
    """Per-group asymmetric INT8 weights: returns (wq int8 [N, K], w_scale float32
    [K/group, N], w_zp float32 [K/group, N]), the parameters group-major."""
    dev = w.device
    N, K = w.shape
    if w.dtype not in _DT:
        raise TypeError(f"q8_quantize_weight_grouped: unsupported dtype {w.dtype}")
    _need(w, "w", w.dtype, (N, K), dev)
    G = K // group if group > 0 else 0
    wq = torch.empty(N, K, dtype=torch.int8, device=dev)
    ws = torch.empty(max(G, 1), N, dtype=torch.float32, device=dev)
    wz = torch.empty(max(G, 1), N, dtype=torch.float32, device=dev)
    st = _lib.lib().q8_quantize_weight_grouped(_ptr(w), _DT[w.dtype], N, K, group, _ptr(wq), _ptr(ws), _ptr(wz),
                                               _stream(dev))
    _lib.check("q8_quantize_weight_grouped", st)
    return wq, ws, wz


def q8_linear_grouped(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor, w_zp: torch.Tensor,
                      group: int = 128, bias: Optional[torch.Tensor] = None,
                      out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None):
    """W8A8 linear with per-group weights (from q8_quantize_weight_grouped with the
    same group) and dynamic per-token INT8 activations."""
    dev = x.device
    M, K = x.shape
    N = wq.shape[0]
    G = K // group if group > 0 else 0
    _need(x, "x", x.dtype, (M, K), dev)
    _need(wq, "wq", torch.int8, (N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (G, N), dev)
    _need(w_zp, "w_zp", torch.float32, (G, N), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (N,), dev)
    y = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=dev)
    _need(y, "y", out_dtype, (M, N), dev)
    ws = workspace if workspace is not None else _workspace("grouped", M, N, K, dev)
    st = _lib.lib().q8_linear_grouped(_ptr(x), _DT[x.dtype], M, K, _ptr(wq), _ptr(w_scale), _ptr(w_zp), group, N,
                                      _ptr(bias), _ptr(y), _DT[out_dtype], _ptr(ws), ws.numel(), _stream(dev))
    _lib.check("q8_linear_grouped", st)
    return y


def q8_bench_mfma_loop(fmt: str, iters: int, workgroups: int, sink: torch.Tensor) -> None:
    """Measurement helper (include/q8_bench.h): a register-only MFMA loop,
    fmt "int8_sym" (int8 32x32x32) or "fp8_e4m3" (fp8 32x32x64); sink is a
    device int32 tensor of workgroups * 256 elements."""
    dev = sink.device
    _need(sink, "sink", torch.int32, (workgroups * 256,), dev)
    st = _lib.lib().q8_bench_mfma_loop(_FMT[fmt], iters, workgroups, _ptr(sink), _stream(dev))
    _lib.check("q8_bench_mfma_loop", st)


def q8_probe_fp8_mfma(a: torch.Tensor, b: torch.Tensor, c: torch.Tensor) -> torch.Tensor:
    """Measurement helper (include/q8_bench.h): d = c + a . b^T through one
    FP8 MFMA per problem.  a, b: uint8 e4m3 codes [P, 32, 64]; c: float32
    [P, 32, 32]; returns d float32 [P, 32, 32]."""
    dev = a.device
    P = a.shape[0]
    _need(a, "a", torch.uint8, (P, 32, 64), dev)
    _need(b, "b", torch.uint8, (P, 32, 64), dev)
    _need(c, "c", torch.float32, (P, 32, 32), dev)
    d = torch.empty(P, 32, 32, dtype=torch.float32, device=dev)
    st = _lib.lib().q8_probe_fp8_mfma(_ptr(a), _ptr(b), _ptr(c), _ptr(d), P, _stream(dev))
    _lib.check("q8_probe_fp8_mfma", st)
    return d


def q8_gemm_tile(op: str, M: int, N: int, K: int) -> tuple:
    """Introspection helper (include/q8_bench.h): the (rows, columns) output
    tile of the MFMA GEMM that a call of op ("linear", "static", "decomp",
    "fp8") runs at this shape; (0, 0) where none runs."""
    bm, bn = ctypes.c_int32(0), ctypes.c_int32(0)
    st = _lib.lib().q8_gemm_tile(_OP[op], M, N, K, ctypes.byref(bm), ctypes.byref(bn))
    _lib.check("q8_gemm_tile", st)
    return bm.value, bn.value


def q8_bench_stream_read(src: torch.Tensor, workgroups: int, sink: torch.Tensor) -> None:
    """Measurement helper (include/q8_bench.h): one streaming read of the
    device tensor src (its bytes, a multiple of 16); sink is a device int32
    tensor of workgroups * 256 elements."""
    dev = src.device
    _need(src, "src", None, None, dev)
    _need(sink, "sink", torch.int32, (workgroups * 256,), dev)
    nbytes = src.numel() * src.element_size()
    st = _lib.lib().q8_bench_stream_read(_ptr(src), nbytes, workgroups, _ptr(sink), _stream(dev))
    _lib.check("q8_bench_stream_read", st)
