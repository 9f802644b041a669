"""CPU oracle for the 8-bit quantized linear layer Y = X.W^T.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and imports nothing from it.  It is deliberately plain
and slow: every step is the definition from the pages, written with numpy in
the precision the pages' PyTorch code uses (IEEE binary32 for scales and codes,
exact integers for the INT8 products, float64 for the reported outputs).

Sources (web pages; cited by title and section):
  [LF]   "8-Bit LLM Quantization with Lightning Fabric" (mlqm.cn news 20786)
  [OV]   "大模型量化技术概述" -- LLM quantization overview (devpress.csdn.net)
  [FB]   "Transformers FP8 (W8A8) 量化实战：基于 FBGEMM 的模型压缩与加载" (2kiu.com)
  [BNB]  "Transformers 单 GPU 高效推理：bitsandbytes LLM.int8 8-bit 混合精度量化" (pwwt.cn)
  [NOTE] Xilyfe, "大模型量化" lecture notes (xilyfeaaaa.github.io/posts/quantization)

Readings taken where the pages are silent, garbled or disagree (each one is
listed with its reason in the design notes of the repository):
  R1  signed int8 weight codes, Z = -128 - rne(lo/S)      ([OV] §2.3 min-max with Q_min=-128;
                                                          [NOTE] asymmetric z formula)
  R2  the quantized-matmul identity uses (q - Z), not (Z + q)  ([NOTE] "量化是什么": r = S(q - Z))
  R3  the weight range is widened to contain 0 (lo<=0<=hi)  ([NOTE]: Z is the code of float 0)
  R4  every scale is floored at eps = 1e-8                ([NOTE] QuantInt8 code, clamp(min=eps))
  R5  codes use IEEE binary32 division x/S                ([LF] §3.3 code, [OV] §2.3 code)
  R6  "round" is round-half-to-even (torch.round)         (all code listings on the pages)
  R7  symmetric codes are clamped to [-127, 127]          ([NOTE] QuantInt8 code)
  R8  FP8 is OCP e4m3fn (bias 7, max 448, subnormals kept, no inf; NaN never produced)
  R9  activation_scale_ub bounds the row absmax before the scale is taken ([FB] §1, §4, §6)
  R10 outlier columns: max_m |x[m,k]| >= tau; tau <= 0 disables the decomposition ([BNB] core idea,
      BitsAndBytesConfig table)
  R11 the int8 part of the decomposition takes its per-token scale over the regular columns only
  R12 outlier weights are the fp16 rounding of the dequantized int8 columns (no fp16 copy kept)
  R13 weight-only (W8A16): the dequantized weights S (q - Z) enter the product exactly; the
      pages' "dequantized back to 16 bits" is the storage of an implementation, whose rounding
      (<= 2^-9 relative) the output tolerance covers
  R14 static quantization: one calibrated scale per activation tensor, symmetric (Z_x = 0, as for
      the dynamic codes); the INT8 output is the scaling of the float64 epilogue value by the
      reciprocal of the output scale, rounded half to even and clamped to [-127, 127]
  R15 per-group weights: a group is a run of g consecutive weights along K inside one output row
      (g = 64 or 128, K a multiple of g), quantized as O2 quantizes a row (range widened to 0,
      eps floor, Z = -128 - rne(lo/S)); the activations stay per token; the parameters are stored
      group-major, [K/g, N]
"""
from __future__ import annotations

import numpy as np

EPS = np.float32(1e-8)          # R4
INT8_ASYM_LEVELS = np.float32(255.0)
E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# O1: input decode -- bf16 / fp16 / fp32 -> fp32, exactly
# --------------------------------------------------------------------------
def to_f32(t) -> np.ndarray:
    """Decode an input tensor to float32 without rounding.

    bf16 is the upper half of a binary32 word, so decoding is a 16-bit shift;
    fp16 widens exactly ([NOTE] number formats section: FP32 8e/23m, FP16 5e/10m,
    BF16 8e/7m).  Accepts torch CPU tensors or numpy arrays.
    """
    if isinstance(t, np.ndarray):
        if t.dtype == np.float32:
            return t
        if t.dtype == np.float16:
            return t.astype(np.float32)
        raise TypeError(f"unsupported numpy dtype {t.dtype}")
    import torch  # only for the tensor view; no arithmetic is done in torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.float16:
        return t.numpy().astype(np.float32)
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32)
    raise TypeError(f"unsupported torch dtype {t.dtype}")


# --------------------------------------------------------------------------
# O2: weights, INT8 asymmetric, per output channel
# --------------------------------------------------------------------------
def quantize_weight_int8_asym(w):
    """Per-output-channel asymmetric min-max INT8 quantization of W [N, K].

    [LF] §2.1 (one scale and zero-point per output row) and §3.3 (quantizer:
    scale = (w_max - w_min)/255, q = round(w/scale) + zero_point, clamp to
    [-128, 127]); [OV] §2.3 min-max: S = (R_max - R_min)/(Q_max - Q_min),
    Z = Q_min - round(R_min/S).  With Q_min = -128 (R1) and the range widened
    to contain 0 (R3):
        lo = min(0, min_k w), hi = max(0, max_k w)
        S  = max((hi - lo) / 255, eps)                 binary32
        Z  = -128 - rne(lo / S)                        integer in [-128, 127]
        q  = clamp(rne(w / S) + Z, -128, 127)
    Returns (q int8 [N,K], S float32 [N], Z float32 [N] holding integers).
    """
    w = to_f32(w)
    lo = np.minimum(w.min(axis=1), np.float32(0))
    hi = np.maximum(w.max(axis=1), np.float32(0))
    scale = (hi - lo) / INT8_ASYM_LEVELS
    scale = np.maximum(scale, EPS).astype(np.float32)
    zp = (np.float32(-128) - np.rint(lo / scale)).astype(np.float32)
    q = np.rint(w / scale[:, None]) + zp[:, None]
    q = np.clip(q, -128, 127).astype(np.int8)
    return q, scale, zp


def dequantize_weight_int8(q, scale, zp) -> np.ndarray:
    """r = S (q - Z)  ([NOTE] "量化是什么"; [LF] §3.3 dequantize_weight).  float64."""
    return scale.astype(np.float64)[:, None] * (q.astype(np.float64) - zp.astype(np.float64)[:, None])


# --------------------------------------------------------------------------
# O3: activations, INT8 symmetric, per token (dynamic)
# --------------------------------------------------------------------------
def quantize_symmetric_absmax(x, qmax: int):
    """Row-wise symmetric absmax quantization with qmax = 2^(b-1) - 1.

    [NOTE] symmetric section: alpha = max |x|, scale alpha/qmax; QuantInt8 code:
    scale = (alpha/qmax).clamp(min=eps), q = round(x/scale).clamp(-qmax, qmax).
    Returns (q int64 [M,K], scale float32 [M]).
    """
    x = to_f32(x)
    alpha = np.abs(x).max(axis=1)
    scale = np.maximum(alpha / np.float32(qmax), EPS).astype(np.float32)
    q = np.clip(np.rint(x / scale[:, None]), -qmax, qmax).astype(np.int64)
    return q, scale


def quantize_act_int8_sym(x):
    """Dynamic per-token INT8 quantization of X [M, K] ([NOTE] dynamic
    quantization section; [FB] §5.2 per-row dynamic activations).
    Also returns the per-row code sum Sum_k q[m,k], needed by the zero-point
    correction of the weights (see ``linear_int8``).
    Returns (q int8 [M,K], S float32 [M], rowsum int32 [M]).
    """
    q, scale = quantize_symmetric_absmax(x, 127)
    rowsum = q.sum(axis=1)
    assert np.all(np.abs(rowsum) < 2**31)
    return q.astype(np.int8), scale, rowsum.astype(np.int32)


# --------------------------------------------------------------------------
# O4 / O5: INT8 x INT8 with INT32 accumulation, then the dequant epilogue
# --------------------------------------------------------------------------
def int_gemm(xq, wq) -> np.ndarray:
    """acc[m,n] = Sum_k xq[m,k] * wq[n,k], exact.  ([NOTE] "INT8 这么小的范围不会导致溢出吗？":
    int8 x int8 products summed in an INT32 accumulator.)

    The matrix product is taken in float64 by the library routine: every
    product and every partial sum, in whatever order the routine adds them,
    is an integer of magnitude at most 128 * 128 * K, below 2^53 for any K up
    to 2^39, so every float64 operation is exact and the result equals the
    integer sum.  Returned as int64, checked to fit int32."""
    xq = np.asarray(xq)
    wq = np.asarray(wq)
    assert 128 * 128 * xq.shape[1] < 2**53
    acc = (xq.astype(np.float64) @ wq.astype(np.float64).T).astype(np.int64)
    assert acc.size == 0 or np.abs(acc).max() < 2**31
    return acc


def epilogue(acc, xs, rowsum, ws, wz, bias=None) -> np.ndarray:
    """y[m,n] = S_x[m] S_w[n] (acc[m,n] - Z_w[n] rowsum[m]) (+ b[n]).

    [OV] §2.1 quantized matmul Y = S_x(X_q - Z_x) . S_w(W_q - Z_w)^T with the
    sign read as r = S(q - Z) (R2) and Z_x = 0 (symmetric activations):
    Sum_k q_x (q_w - Z_w) = acc - Z_w Sum_k q_x.  The correction is done in
    exact integers, the scaling in float64.  Bias is fp32, added after the
    scaling ([FB] §5.3).
    """
    c = acc - wz.astype(np.int64)[None, :] * rowsum.astype(np.int64)[:, None]
    y = xs.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :] * c.astype(np.float64)
    if bias is not None:
        y = y + to_f32(bias).astype(np.float64)[None, :]
    return y


def linear_int8(x, wq, ws, wz, bias=None):
    """W8A8 linear: dynamic per-token INT8 X, per-channel asymmetric INT8 W.
    Returns (y float64 [M,N], dict of intermediates)."""
    xq, xs, rs = quantize_act_int8_sym(x)
    acc = int_gemm(xq, wq)
    y = epilogue(acc, xs, rs, ws, wz, bias)
    return y, {"xq": xq, "x_scale": xs, "x_rowsum": rs, "acc": acc}


# --------------------------------------------------------------------------
# O6 / O7: LLM.int8() mixed-precision decomposition
# --------------------------------------------------------------------------
def outlier_columns(x, tau: float) -> np.ndarray:
    """Feature columns that go through the 16-bit flow ([BNB] core idea: the
    systematic outlier features, e.g. in [-60,-6] or [6,60], are computed in
    fp16; the BitsAndBytesConfig table: threshold 6.0).  Reading R10:
    column k is an outlier iff max_m |x[m,k]| >= tau; tau <= 0 selects none.
    Returns ascending int64 column indices."""
    x = to_f32(x)
    if not (tau > 0):
        return np.zeros(0, dtype=np.int64)
    colmax = np.abs(x).max(axis=0)
    return np.nonzero(colmax >= np.float32(tau))[0].astype(np.int64)


def outlier_weights_f16(wq, ws, wz, cols) -> np.ndarray:
    """W_O[n,j] = fp16(fp32(S_w[n] * (q_w[n, O_j] - Z_w[n]))) (reading R12)."""
    d = wq[:, cols].astype(np.float32) - wz[:, None]
    return (ws[:, None] * d).astype(np.float32).astype(np.float16)


def linear_int8_decomp(x_f16, wq, ws, wz, tau: float = 6.0, bias=None):
    """y = int8 path over the regular columns + fp16 path over the outlier columns.

    X_R is X with the outlier columns set to 0; its per-token INT8 scale is
    therefore taken over the regular columns only (R11).  The outlier product
    X_O . W_O^T uses fp16 operands and is summed in float64.
    Returns (y float64 [M,N], dict of intermediates)."""
    x = to_f32(x_f16)
    cols = outlier_columns(x, tau)
    xr = x.copy()
    xr[:, cols] = 0
    xq, xs, rs = quantize_act_int8_sym(xr)
    acc = int_gemm(xq, wq)
    y = epilogue(acc, xs, rs, ws, wz, None)
    w_o = outlier_weights_f16(wq, ws, wz, cols)
    x_o = x[:, cols]          # exact: x is fp16 data
    y = y + x_o.astype(np.float64) @ w_o.astype(np.float64).T
    if bias is not None:
        y = y + to_f32(bias).astype(np.float64)[None, :]
    return y, {"cols": cols, "xq": xq, "x_scale": xs, "x_rowsum": rs, "acc": acc, "w_o": w_o}


# --------------------------------------------------------------------------
# O8 / O9: FP8 e4m3 W8A8 rowwise
# --------------------------------------------------------------------------
def e4m3_decode(codes) -> np.ndarray:
    """OCP FP8 e4m3fn code -> value (float64).  1 sign, 4 exponent (bias 7),
    3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is
    NaN; there are no infinities.  ([FB] §1: float8_e4m3fn, 4-bit exponent +
    3-bit mantissa; the field layout is the OCP 8-bit floating point format.)"""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(r) -> np.ndarray:
    """Round a real value with |r| <= 448 to the nearest e4m3fn code, ties to
    even (R8).  Within a binade [2^e, 2^(e+1)) the spacing is 2^(e-3); below
    the smallest normal 2^-6 it is the subnormal spacing 2^-9.  The sign of
    zero is kept.  Values must already be clamped to [-448, 448]."""
    r = np.asarray(r, dtype=np.float64)
    assert np.all(np.abs(r) <= E4M3_MAX), "clamp to +-448 before encoding"
    a = np.abs(r)
    sign = np.signbit(r).astype(np.int64)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -6)   # binade exponent (subnormals share -6)
    n = np.rint(a / np.exp2((e - 3).astype(np.float64))).astype(np.int64)   # 0..16
    carry = n == 16
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 8, n)
    normal = n >= 8
    field_e = np.where(normal, e + 7, 0)
    field_m = np.where(normal, n - 8, n)
    code = (sign << 7) | (field_e << 3) | field_m
    return code.astype(np.uint8)


def quantize_fp8_rowwise(x, scale_ub=None):
    """Row-wise (per output channel / per token) e4m3 quantization.

    [FB] §5.1: weight stored as float8_e4m3fn with one fp32 weight_scale per
    output channel; §5.2: activations quantized per row at every forward with
    the input_scale_ub bound; §1/§6: the input is truncated at the upper bound
    (default 1200.0) before quantizing.  With reading R9:
        a = max_k |x|,  a = min(a, ub) if a bound is given
        S = max(a / 448, eps);  q = e4m3(clamp(x / S, -448, 448))
    Returns (codes uint8 [R,K], S float32 [R])."""
    x = to_f32(x)
    a = np.abs(x).max(axis=1)
    if scale_ub is not None:
        a = np.minimum(a, np.float32(scale_ub))
    scale = np.maximum(a / np.float32(E4M3_MAX), EPS).astype(np.float32)
    r = np.clip(x / scale[:, None], np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(r), scale


def linear_fp8(x, wq_codes, w_scale, scale_ub=1200.0, bias=None):
    """FP8 W8A8 rowwise linear ([FB] §5.3: both operands fp8 with per-row
    scales, output bf16, fp32 bias added after).  Products of two e4m3 values
    are exact in float64; the sum is taken in float64.
    Returns (y float64 [M,N], dict of intermediates)."""
    xq, xs = quantize_fp8_rowwise(x, scale_ub)
    dot = e4m3_decode(xq) @ e4m3_decode(wq_codes).T
    y = dot * xs.astype(np.float64)[:, None] * w_scale.astype(np.float64)[None, :]
    if bias is not None:
        y = y + to_f32(bias).astype(np.float64)[None, :]
    return y, {"xq": xq, "x_scale": xs}


# --------------------------------------------------------------------------
# O13: FP8 expert projection over routed tokens (grouped by expert)
# --------------------------------------------------------------------------
def linear_fp8_grouped(x, offsets, wq_codes, w_scale, scale_ub=1200.0):
    """Mixture-of-experts FP8 projection ([FB] §5.4, Llama4 experts: the expert
    weights are kept as one FP8 tensor with a per-row scale for each expert;
    every expert's tokens get their own per-token activation quantization and
    the rowwise FP8 product with that expert's weights).  Rows
    offsets[e] .. offsets[e+1]-1 of X belong to expert e; each group is O8 + O9
    with wq_codes[e], w_scale[e].  Returns y float64 [T, N]."""
    offsets = np.asarray(offsets, dtype=np.int64)
    E, N = wq_codes.shape[0], wq_codes.shape[1]
    xf = to_f32(x)
    y = np.zeros((xf.shape[0], N), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y[lo:hi], _ = linear_fp8(xf[lo:hi], wq_codes[e], w_scale[e], scale_ub)
    return y


# --------------------------------------------------------------------------
# O10: weight-only W8A16 (16-bit activations, INT8 asymmetric weights)
# --------------------------------------------------------------------------
def linear_w8a16(x, wq, ws, wz, bias=None):
    """Weight-only linear ([NOTE] PTQ section, weight quantization: the weights
    are stored as INT8, read from memory and dequantized for a product in the
    activations' 16-bit format; the activations are not quantized):
        y[m,n] = Sum_k x[m,k] S_w[n] (q_w[n,k] - Z_w[n])  (+ b[n])
    with the dequantized weights exact (R13: no rounding of S (q - Z) to 16
    bits) and the product in float64.  Returns y float64 [M,N]."""
    y = to_f32(x).astype(np.float64) @ dequantize_weight_int8(wq, ws, wz).T
    if bias is not None:
        y = y + to_f32(bias).astype(np.float64)[None, :]
    return y


# --------------------------------------------------------------------------
# O11 / O12: static activation scale, INT8 requantized output
# --------------------------------------------------------------------------
def quantize_act_int8_static(x, scale):
    """Static INT8 activation quantization ([NOTE] "INT8 这么小的范围不会导致溢出吗？",
    static quantization: the scale comes from calibration run beforehand and is
    applied unchanged at inference): one float32 scale S for the tensor,
    q = clamp(rne(x / S), -127, 127) with the binary32 division (R5, R6, R7),
    and the per-row code sums.  Returns (q int8 [M,K], rowsum int32 [M])."""
    x = to_f32(x)
    s = np.float32(scale)
    q = np.clip(np.rint(x / s), -127, 127).astype(np.int64)
    rowsum = q.sum(axis=1)
    assert np.all(np.abs(rowsum) < 2**31)
    return q.astype(np.int8), rowsum.astype(np.int32)


def requantize_int8(y, y_scale):
    """INT8 output for the next layer ([NOTE] same section, step 4: the INT32
    result is scaled and squeezed back into INT8 before it is passed on):
    q_y = clamp(rne(y * (1 / S_y)), -127, 127), the reciprocal and the product
    in float64 (R14)."""
    inv = 1.0 / np.float64(np.float32(y_scale))
    return np.clip(np.rint(np.asarray(y, dtype=np.float64) * inv), -127, 127).astype(np.int8)


def linear_static(x, x_scale, wq, ws, wz, y_scale, bias=None):
    """W8A8 linear with a static activation scale and an INT8 output:
    codes by O11, exact INT32 product (O4), the O5 epilogue in float64 with
    S_x = x_scale on every row, then O12's requantization.
    Returns (yq int8 [M,N], dict of intermediates)."""
    xq, rs = quantize_act_int8_static(x, x_scale)
    acc = int_gemm(xq, wq)
    xs = np.full(xq.shape[0], np.float32(x_scale), dtype=np.float32)
    y = epilogue(acc, xs, rs, ws, wz, bias)
    return requantize_int8(y, y_scale), {"xq": xq, "x_rowsum": rs, "acc": acc, "y": y}


# --------------------------------------------------------------------------
# O14 / O15: per-group asymmetric INT8 weights
# --------------------------------------------------------------------------
def quantize_weight_int8_grouped(w, group: int):
    """Per-group asymmetric INT8 quantization of W [N, K].

    [OV] §2.2 (granularity table: between per-tensor and per-channel sit
    groups of 64 to 128 parameters, each group with its own quantization
    parameters) and [NOTE] quantization granularity passage (per-group: the
    data is cut into blocks, each with its own scale and zero point).  R15:
    group j of row n is w[n, j g : (j+1) g]; for each group, as O2 for a row,
        lo = min(0, min w), hi = max(0, max w)
        S  = max((hi - lo) / 255, eps)                 binary32
        Z  = -128 - rne(lo / S)
        q  = clamp(rne(w / S) + Z, -128, 127)
    Returns (q int8 [N,K], S float32 [K/g, N], Z float32 [K/g, N]); the
    parameters are group-major: S[j, n] belongs to group j of row n.
    """
    w = to_f32(w)
    N, K = w.shape
    assert group > 0 and K % group == 0
    G = K // group
    q = np.empty((N, K), dtype=np.int8)
    S = np.empty((G, N), dtype=np.float32)
    Z = np.empty((G, N), dtype=np.float32)
    for j in range(G):
        blk = w[:, j * group:(j + 1) * group]
        lo = np.minimum(blk.min(axis=1), np.float32(0))
        hi = np.maximum(blk.max(axis=1), np.float32(0))
        s = np.maximum((hi - lo) / INT8_ASYM_LEVELS, EPS).astype(np.float32)
        z = (np.float32(-128) - np.rint(lo / s)).astype(np.float32)
        q[:, j * group:(j + 1) * group] = np.clip(np.rint(blk / s[:, None]) + z[:, None], -128, 127)
        S[j] = s
        Z[j] = z
    return q, S, Z


def group_code_sums(xq, group: int) -> np.ndarray:
    """Sum of the activation codes over each group of columns:
    gsum[j, m] = Sum_{k in group j} q_x[m, k], group-major [K/g, M], int32."""
    xq = np.asarray(xq).astype(np.int64)
    M, K = xq.shape
    assert K % group == 0
    return xq.reshape(M, K // group, group).sum(axis=2).T.astype(np.int32)


def linear_int8_grouped(x, wq, S, Z, group: int, bias=None):
    """W8A8 linear with per-group asymmetric weights (O14) and dynamic
    per-token INT8 activations (O3).  The quantized-matmul identity of O5
    ([OV] §2.1, R2) taken group by group, since S and Z change with the group:
        C_j[m,n] = Sum_{k in j} q_x[m,k] q_w[n,k] - Z[j,n] Sum_{k in j} q_x[m,k]   (exact integers)
        y[m,n]   = S_x[m] Sum_j S[j,n] C_j[m,n]  (+ b[n])                          (float64)
    Returns (y float64 [M,N], dict of intermediates)."""
    xq, xs, _ = quantize_act_int8_sym(x)
    M, K = xq.shape
    N = wq.shape[0]
    G = K // group
    assert K % group == 0 and S.shape == (G, N) and Z.shape == (G, N)
    gsum = group_code_sums(xq, group)
    t = np.zeros((M, N), dtype=np.float64)
    for j in range(G):
        cols = slice(j * group, (j + 1) * group)
        acc = int_gemm(xq[:, cols], wq[:, cols])
        c = acc - Z[j].astype(np.int64)[None, :] * gsum[j].astype(np.int64)[:, None]
        t += S[j].astype(np.float64)[None, :] * c.astype(np.float64)
    y = xs.astype(np.float64)[:, None] * t
    if bias is not None:
        y = y + to_f32(bias).astype(np.float64)[None, :]
    return y, {"xq": xq, "x_scale": xs, "gsum": gsum}


# --------------------------------------------------------------------------
# Comparison metric used by the parity tests
# --------------------------------------------------------------------------
def max_rel_err(y, y_ref, floor_frac: float = 1e-3) -> float:
    """max_i |y_i - yref_i| / max(|yref_i|, floor_frac * max_j |yref_j|).

    The floor keeps outputs that cancel to almost zero from dominating a
    relative metric (0.1% of the largest reference output)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y_ref.size == 0:
        return 0.0
    floor = floor_frac * np.abs(y_ref).max()
    den = np.maximum(np.abs(y_ref), floor if floor > 0 else 1e-30)
    return float(np.max(np.abs(y - y_ref) / den))
