"""Whole-layer pins of the oracle: every layer's output against the exact
float product X . W^T, within the error bound that rounding to the nearest
code fixes a priori.

The quantizers round to the nearest code, so each activation or weight is off
by at most half a quantization step ("大模型量化技术概述" §2.1: r = S (q - Z),
q = round(r / S) + Z; the lecture notes' quantization-error passage: the error
is the difference between a value and its dequantized code).  For one output

    |y - x . w| <= Sum_k |x_k - x^_k| |w_k| + |x^_k| |w_k - w^_k|

with x^, w^ the dequantized operands.  Every bound below is computed from x,
w and the scales that the quantization rules define, never from the oracle's
own codes or intermediates, so a dropped term, a wrong sign, a transposed
operand or a scale in the wrong place (each of which moves y by many
quantization steps) fails here even though the oracle agrees with itself.

Per-element bounds used:
  * INT8 symmetric activations, S_x = absmax / 127: |x - x^| <= S_x / 2 (plus
    the binary32 rounding of the quotient, < 2^-16 S_x);
  * INT8 asymmetric weights, S_w = (max(0, max w) - min(0, min w)) / 255:
    |w - w^| <= S_w (half a step, plus at most half a step where the top of
    the range meets the clamp at 127 after the zero point is rounded);
  * e4m3 (3 fraction bits): |x - x^| <= 2^-4 |x| + 2^-10 S (half the spacing
    in a binade, or half the subnormal spacing 2^-9 S);
  * LLM.int8 outlier weights, binary16 of the binary32 product:
    |w - W_O| <= S_w + 2^-10 |w^|.
"""
import numpy as np
import pytest

from oracle import q8_oracle as O

SLACK = 1.0 + 1e-6          # binary32 rounding of the scales themselves


def _exact(x, w):
    return x.astype(np.float64) @ w.astype(np.float64).T


def _asym_step(w):
    lo = np.minimum(w.min(axis=1), 0.0).astype(np.float64)
    hi = np.maximum(w.max(axis=1), 0.0).astype(np.float64)
    return (hi - lo) / 255.0 * SLACK


def _sym_step(x, qmax):
    return np.abs(x).max(axis=1).astype(np.float64) / qmax * SLACK


def _bound(ex, ew, x, w):
    """Sum_k ex[m,k] |w[n,k]| + (|x[m,k]| + ex[m,k]) ew[n,k] for every (m, n)."""
    ax, aw = np.abs(x).astype(np.float64), np.abs(w).astype(np.float64)
    return ex @ aw.T + (ax + ex) @ ew.T


def _case(seed, M, N, K, spread=1.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * spread).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.05 + rng.uniform(-0.02, 0.05, (N, 1))).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    return x, w, b


@pytest.mark.parametrize("seed,M,N,K", [(1, 5, 7, 64), (2, 3, 11, 200), (3, 9, 4, 33)])
def test_linear_int8_within_rounding_bound(seed, M, N, K):
    x, w, b = _case(seed, M, N, K)
    wq, ws, wz = O.quantize_weight_int8_asym(w)
    y, _ = O.linear_int8(x, wq, ws, wz, bias=b)
    ex = np.repeat((_sym_step(x, 127) * (0.5 + 2.0 ** -16))[:, None], K, axis=1)
    ew = np.repeat(_asym_step(w)[:, None], K, axis=1)
    err = np.abs(y - (_exact(x, w) + b.astype(np.float64)))
    bound = _bound(ex, ew, x, w) * (1 + 1e-9) + 1e-12
    assert np.all(err <= bound), float((err / bound).max())
    # the bound is not vacuous: it is a small fraction of the outputs' scale
    assert bound.max() < 0.2 * np.abs(_exact(x, w)).max()


@pytest.mark.parametrize("seed,M,N,K", [(4, 6, 5, 96), (5, 2, 9, 300)])
def test_linear_fp8_within_rounding_bound(seed, M, N, K):
    x, w, b = _case(seed, M, N, K, spread=3.0)
    wq, ws = O.quantize_fp8_rowwise(w)
    y, _ = O.linear_fp8(x, wq, ws, scale_ub=None, bias=b)
    sx = _sym_step(x, 448.0)
    sw = _sym_step(w, 448.0)
    ex = 2.0 ** -4 * np.abs(x).astype(np.float64) + 2.0 ** -10 * sx[:, None]
    ew = 2.0 ** -4 * np.abs(w).astype(np.float64) + 2.0 ** -10 * sw[:, None]
    err = np.abs(y - (_exact(x, w) + b.astype(np.float64)))
    bound = _bound(ex, ew, x, w) * (1 + 1e-9) + 1e-12
    assert np.all(err <= bound), float((err / bound).max())
    # about an eighth of Sum |x| |w|: two operands, 2^-4 each
    assert np.all(bound < 0.14 * (np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64).T))


def test_linear_w8a16_within_rounding_bound():
    x, w, b = _case(6, 4, 9, 128)
    wq, ws, wz = O.quantize_weight_int8_asym(w)
    y = O.linear_w8a16(x, wq, ws, wz, bias=b)
    ew = np.repeat(_asym_step(w)[:, None], 128, axis=1)
    err = np.abs(y - (_exact(x, w) + b.astype(np.float64)))
    bound = _bound(np.zeros_like(x, dtype=np.float64), ew, x, w) * (1 + 1e-9) + 1e-12
    assert np.all(err <= bound), float((err / bound).max())


def test_linear_int8_decomp_within_rounding_bound():
    rng = np.random.default_rng(7)
    M, N, K, tau = 12, 10, 80, 6.0
    x = np.clip(rng.standard_normal((M, K)), -3.5, 3.5).astype(np.float32)
    cols = np.array([3, 41, 77])
    x[:, cols] = rng.uniform(6.0, 40.0, (M, 3)).astype(np.float32) * rng.choice([-1, 1], (M, 3))
    x16 = x.astype(np.float16)
    xf = x16.astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    wq, ws, wz = O.quantize_weight_int8_asym(w)
    y, _ = O.linear_int8_decomp(x16, wq, ws, wz, tau, bias=b)
    # the outlier set from its definition: columns whose max |x| reaches tau
    out = np.abs(xf).max(axis=0) >= tau
    assert set(np.flatnonzero(out)) == set(cols)
    xr = np.where(out[None, :], 0.0, xf)
    s_reg = _sym_step(xr, 127) * (0.5 + 2.0 ** -16)
    step_w = _asym_step(w)
    ex = np.where(out[None, :], 0.0, s_reg[:, None])                 # outlier activations are exact
    dq = np.abs(w).astype(np.float64) + step_w[:, None]               # |w^| <= |w| + step
    ew = np.where(out[None, :], step_w[:, None] + 2.0 ** -10 * dq, step_w[:, None])
    err = np.abs(y - (_exact(xf, w) + b.astype(np.float64)))
    bound = _bound(ex, ew, xf, w) * (1 + 1e-9) + 1e-12
    assert np.all(err <= bound), float((err / bound).max())
    # without the outlier flow the error would far exceed the bound
    y_plain, _ = O.linear_int8(xr, wq, ws, wz, bias=b)
    assert np.any(np.abs(y_plain - (_exact(xf, w) + b.astype(np.float64))) > 10 * bound)


@pytest.mark.parametrize("group", [16, 32])
def test_linear_grouped_within_rounding_bound(group):
    x, w, b = _case(8, 5, 6, 96)
    wq, S, Z = O.quantize_weight_int8_grouped(w, group)
    y = O.linear_int8_grouped(x, wq, S, Z, group, bias=b)
    y = y[0] if isinstance(y, tuple) else y
    ex = np.repeat((_sym_step(x, 127) * (0.5 + 2.0 ** -16))[:, None], 96, axis=1)
    ew = np.concatenate([np.repeat(_asym_step(w[:, j:j + group])[:, None], group, axis=1)
                         for j in range(0, 96, group)], axis=1)
    err = np.abs(y - (_exact(x, w) + b.astype(np.float64)))
    bound = _bound(ex, ew, x, w) * (1 + 1e-9) + 1e-12
    assert np.all(err <= bound), float((err / bound).max())


def test_static_requantized_output_within_rounding_bound():
    x, w, b = _case(9, 4, 8, 64)
    xs_static = float(np.abs(x).max()) / 127.0 * 1.3        # calibrated above the data: no saturation
    y_scale = 0.05
    wq, ws, wz = O.quantize_weight_int8_asym(w)
    yq, _ = O.linear_static(x, xs_static, wq, ws, wz, y_scale, bias=b)
    ex = np.full(x.shape, np.float32(xs_static) * (0.5 + 2.0 ** -16), dtype=np.float64)
    ew = np.repeat(_asym_step(w)[:, None], 64, axis=1)
    exact = (_exact(x, w) + b.astype(np.float64)) / np.float64(np.float32(y_scale))
    bound = _bound(ex, ew, x, w) / np.float64(np.float32(y_scale)) + 0.5 + 1e-9
    inside = np.abs(exact) < 127 - bound                      # outputs the clamp does not reach
    assert inside.mean() > 0.5
    assert np.all(np.abs(yq.astype(np.float64) - exact)[inside] <= bound[inside])
    assert np.all(yq[exact > 127 + bound] == 127) and np.all(yq[exact < -127 - bound] == -127)
