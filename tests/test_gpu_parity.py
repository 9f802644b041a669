"""GPU parity: every C-ABI call against the CPU oracle on the same seeded
inputs.  Integer results (codes, scale bit patterns, zero-points, row sums,
INT32 accumulators, outlier sets) must match bit for bit; floating outputs
within max relative error 1e-2 (floored at 0.1% of the largest output).
Large workloads run at full size on the GPU and are compared on every output,
except two that are compared on sampled rows the oracle computes one by one
(every kernel here is row-independent in X): the full-size FP8 GEMM, whose
per-output error bound is built from all K products of each output, and the
largest weight matrix (2^31 - 2^16 elements)."""
import numpy as np
import pytest
import torch

from oracle import q8_oracle as O
from w8a8_quantized_linear_channel_amd import inputs
from w8a8_quantized_linear_channel_amd import ops as q8

import fp8_accum as F

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-2


def log(msg):
    print(msg, flush=True)


def g(t):
    return t.to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.int32)


def assert_equal(got, ref, what):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = np.argwhere(got != ref)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {got[i]} want {ref[i]}")


def out_f64(y):
    return y.detach().float().cpu().numpy().astype(np.float64)


def check_close(y_gpu, y_ref, what):
    err = O.max_rel_err(y_gpu, y_ref)
    log(f"  {what}: max rel err {err:.3e}")
    assert err <= TOL, (what, err)


# The FP8 GEMM runs with the fast accumulation of the page's FP8 GEMM
# ("Transformers FP8 (W8A8) 量化实战…" §5.3, use_fast_accum=True): its matrix
# instruction cuts each product 13 bits below the largest of its group of
# eight (tests/fp8_accum.py, pinned on the instruction by
# test_gpu_fp8_accum.py).  An FP8 output passes if its error is within the
# 1e-2 relative tolerance, or within that tolerance plus the bound B that the
# instruction's cuts and the chain's binary32 roundings can add to the exact
# sum (fp8_accum.gemm_bound, computed from the oracle's codes).
def check_close_fp8(y_gpu, y_ref, x_rows, w, ub, what):
    """y_gpu, y_ref [R, N] for the activation rows x_rows [R, K] (input
    values) and weights w [N, K] (input values)."""
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if y_ref.size == 0:
        return
    plain = O.max_rel_err(y_gpu, y_ref)
    den = np.maximum(np.abs(y_ref), 1e-3 * np.abs(y_ref).max())
    err = np.abs(y_gpu - y_ref)
    over = np.argwhere(err > TOL * den)
    worst = 0.0
    if over.size:
        xq, xs = O.quantize_fp8_rowwise(x_rows, ub)
        wq, wsc = O.quantize_fp8_rowwise(w)
        xv, wv = O.e4m3_decode(xq), O.e4m3_decode(wq)
        for r in np.unique(over[:, 0]):
            cols = over[over[:, 0] == r][:, 1]
            b = F.gemm_bound(xv[r:r + 1], xs[r:r + 1], wv[cols], wsc[cols])[0]
            excess = err[r, cols] - TOL * den[r, cols]
            assert np.all(excess <= b), (what, int(r), int(cols[np.argmax(excess - b)]))
            worst = max(worst, float(np.max(excess / b)))
    log(f"  {what}: max rel err {plain:.3e}; {len(over)} of {y_ref.size} outputs beyond 1e-2, "
        f"their excess at most {worst:.3f} of the fast-accumulation bound")


def sample_rows(M, n=12, seed=0, extra=()):
    rng = np.random.default_rng(seed)
    rows = {0, M - 1, *[r for r in extra if 0 <= r < M]}
    rows |= set(rng.integers(0, M, size=min(n, M)).tolist())
    return np.array(sorted(rows))


# ---------------------------------------------------------------- weights INT8 asym
WEIGHT_CASES = [
    ("tiny_256x256_f32", 256, 256, torch.float32, 0),
    ("ragged_37x48_f32", 37, 48, torch.float32, 1),
    ("f32_overflow_row_9x8208", 9, 8208, torch.float32, 2),
    ("bf16_65x4112", 65, 4112, torch.bfloat16, 3),
    ("f16_overflow_row_5x20032", 5, 20032, torch.float16, 4),
]


@pytest.mark.parametrize("name,N,K,dt,seed", WEIGHT_CASES)
def test_quantize_weight_int8(name, N, K, dt, seed):
    log(f"[weight int8] {name}")
    w = inputs.random_matrix(seed, (N, K), 0.02, dt)
    wq, ws, wz = q8.q8_quantize_weight(g(w), "int8_asym")
    rq, rs, rz = O.quantize_weight_int8_asym(w)
    assert_equal(host(wq), rq, "codes")
    assert_equal(f32_bits(host(ws)), f32_bits(rs), "scale bits")
    assert_equal(host(wz), rz, "zero-points")


def test_quantize_weight_int8_edge_rows():
    log("[weight int8] edge rows")
    K = 64
    rows = [np.zeros(K), np.linspace(0.1, 2.0, K), -np.linspace(0.1, 2.0, K),
            np.r_[[-128.0, 127.0], np.arange(K - 2) - 30.0], np.full(K, 3.0),
            np.r_[[1e-30, -1e-30], np.zeros(K - 2)], np.r_[[-7.5, 2.5, 127.0, -128.0], np.zeros(K - 4)]]
    w = torch.tensor(np.stack(rows), dtype=torch.float32)
    wq, ws, wz = q8.q8_quantize_weight(g(w), "int8_asym")
    rq, rs, rz = O.quantize_weight_int8_asym(w)
    assert_equal(host(wq), rq, "codes")
    assert_equal(f32_bits(host(ws)), f32_bits(rs), "scale bits")
    assert_equal(host(wz), rz, "zero-points")


@pytest.mark.parametrize("which", ["decode_q_proj_4096x4096", "prefill_ffn_up_14336x4096"])
def test_quantize_weight_int8_full_size(which):
    log(f"[weight int8] {which}")
    wl = inputs.decode_qproj() if which.startswith("decode") else inputs.prefill_ffn_up()
    wq, ws, wz = q8.q8_quantize_weight(g(wl.w), "int8_asym")
    rq, rs, rz = O.quantize_weight_int8_asym(wl.w)
    assert_equal(host(wq), rq, "codes")
    assert_equal(f32_bits(host(ws)), f32_bits(rs), "scale bits")
    assert_equal(host(wz), rz, "zero-points")


# ---------------------------------------------------------------- activations INT8 sym
ACT_CASES = [
    ("tiny_16x256_f32", 16, 256, torch.float32, 10),
    ("ragged_33x80_f16", 33, 80, torch.float16, 11),
    ("prefill_2048x4096_bf16", 2048, 4096, torch.bfloat16, 12),
    ("overflow_row_5x20032_bf16", 5, 20032, torch.bfloat16, 13),
    ("f32_overflow_3x8208", 3, 8208, torch.float32, 14),
    # 16-bit rows of up to 4096 values run a two-chunk register cache, longer
    # ones the eight-chunk one: both sides of that boundary
    ("cache_edge_9x4096_f16", 9, 4096, torch.float16, 15),
    ("cache_edge_7x4112_bf16", 7, 4112, torch.bfloat16, 16),
    ("cache_edge_6x4112_f16", 6, 4112, torch.float16, 17),
]


@pytest.mark.parametrize("name,M,K,dt,seed", ACT_CASES)
def test_quantize_act_int8(name, M, K, dt, seed):
    log(f"[act int8] {name}")
    x = inputs.random_matrix(seed, (M, K), 1.0, dt)
    xq, xs, rsum = q8.q8_quantize_act(g(x), "int8_sym")
    rq, rs, rr = O.quantize_act_int8_sym(x)
    assert_equal(host(xq), rq, "codes")
    assert_equal(f32_bits(host(xs)), f32_bits(rs), "scale bits")
    assert_equal(host(rsum), rr, "row sums")


def test_quantize_act_int8_edge_rows():
    log("[act int8] edge rows")
    K = 32
    rows = [np.zeros(K), np.r_[[127.0, 2.5, -3.5, 0.5, -0.5, 126.5], np.zeros(K - 6)],
            np.full(K, -2.0), np.r_[[1e-38], np.zeros(K - 1)], np.arange(K) - 16.0]
    x = torch.tensor(np.stack(rows), dtype=torch.float32)
    xq, xs, rsum = q8.q8_quantize_act(g(x), "int8_sym")
    rq, rs, rr = O.quantize_act_int8_sym(x)
    assert_equal(host(xq), rq, "codes")
    assert_equal(f32_bits(host(xs)), f32_bits(rs), "scale bits")
    assert_equal(host(rsum), rr, "row sums")


# ---------------------------------------------------------------- FP8 quantization
@pytest.mark.parametrize("name,N,K,dt,seed", [("ragged_19x272_f32", 19, 272, torch.float32, 20),
                                              ("bf16_40x1040", 40, 1040, torch.bfloat16, 21)])
def test_quantize_weight_fp8(name, N, K, dt, seed):
    log(f"[weight fp8] {name}")
    w = inputs.random_matrix(seed, (N, K), 0.02, dt)
    wq, ws, wz = q8.q8_quantize_weight(g(w), "fp8_e4m3")
    assert wz is None
    rq, rs = O.quantize_fp8_rowwise(w)
    assert_equal(host(wq), rq, "e4m3 codes")
    assert_equal(f32_bits(host(ws)), f32_bits(rs), "scale bits")


@pytest.mark.parametrize("ub", [1200.0, 1000.0, float("inf")])
def test_quantize_act_fp8_scale_ub(ub):
    log(f"[act fp8] ub={ub}")
    x = inputs.random_matrix(22, (6, 96), 3.0, torch.float32).numpy().copy()
    x[1, 5] = 5000.0           # bound binds for ub = 1000 / 1200
    x[2, :] *= 400.0
    x[3, :] = 0.0
    x[4, 7] = -1100.0
    xt = torch.from_numpy(x).to(torch.bfloat16)
    xq, xs, _ = q8.q8_quantize_act(g(xt), "fp8_e4m3", scale_ub=ub)
    rq, rs = O.quantize_fp8_rowwise(xt, None if ub == float("inf") else ub)
    assert_equal(host(xq), rq, "e4m3 codes")
    assert_equal(f32_bits(host(xs)), f32_bits(rs), "scale bits")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("K", [4096, 4112])
def test_quantize_act_fp8_row_cache_edge(dt, K):
    # 16-bit rows of up to 4096 values run the two-chunk register cache,
    # longer ones the eight-chunk one; rows with the bound binding and not
    log(f"[act fp8] row cache edge K={K} {dt}")
    x = inputs.random_matrix(23, (7, K), 2.0, torch.float32).numpy().copy()
    x[2, K - 1] = 3000.0       # the bound binds on this row
    x[4, :] = 0.0
    xt = torch.from_numpy(x).to(dt)
    xq, xs, _ = q8.q8_quantize_act(g(xt), "fp8_e4m3", scale_ub=1200.0)
    rq, rs = O.quantize_fp8_rowwise(xt, 1200.0)
    assert_equal(host(xq), rq, "e4m3 codes")
    assert_equal(f32_bits(host(xs)), f32_bits(rs), "scale bits")


def test_quantize_fp8_full_size():
    log("[fp8 quant] 4096x14336 activations and weights, every row")
    wl = inputs.fp8_rowwise()
    xq, xs, _ = q8.q8_quantize_act(g(wl.x), "fp8_e4m3", scale_ub=1200.0)
    wq, ws, _ = q8.q8_quantize_weight(g(wl.w), "fp8_e4m3")
    rq, rs = O.quantize_fp8_rowwise(wl.x, 1200.0)
    assert_equal(host(xq), rq, "activation codes")
    assert_equal(f32_bits(host(xs)), f32_bits(rs), "activation scale bits")
    rq, rs = O.quantize_fp8_rowwise(wl.w)
    assert_equal(host(wq), rq, "weight codes")
    assert_equal(f32_bits(host(ws)), f32_bits(rs), "weight scale bits")


# ---------------------------------------------------------------- q8_linear
def oracle_weights(w):
    return O.quantize_weight_int8_asym(w)


def run_linear_case(x, w, out_dtype, rows=None, bias=None, what=""):
    """GPU q8_linear on the full problem; oracle on `rows` (all if None)."""
    wq, ws, wz = q8.q8_quantize_weight(g(w), "int8_asym")
    b = g(bias) if bias is not None else None
    y, acc = q8.q8_linear(g(x), wq, ws, wz, bias=b, out_dtype=out_dtype, acc_out=True)
    rq, rs, rz = oracle_weights(w)
    xr = x if rows is None else x[rows]
    y_ref, inter = O.linear_int8(xr, rq, rs, rz, bias=bias)
    acc_g = host(acc) if rows is None else host(acc)[rows]
    y_g = out_f64(y) if rows is None else out_f64(y)[rows]
    assert_equal(acc_g, inter["acc"].astype(np.int32), f"{what} INT32 accumulator")
    check_close(y_g, y_ref, f"{what} output")
    if x.shape[0] > 10:
        # q8_linear above 10 tokens is q8_quantize_act + q8_gemm_int8, bit for bit
        xq, xs, xr_ = q8.q8_quantize_act(g(x), "int8_sym")
        y2, acc2 = q8.q8_gemm_int8(xq, xs, xr_, wq, ws, wz, bias=b, out_dtype=out_dtype, acc_out=True)
        assert torch.equal(acc, acc2), f"{what}: q8_gemm_int8 accumulator differs"
        assert torch.equal(y.view(torch.uint8), y2.view(torch.uint8)), f"{what}: q8_gemm_int8 differs"
    return y, acc


def test_linear_tiny_config():
    log("[linear] tiny 16x256x256 fp32 -> fp32")
    wl = inputs.tiny_linear()
    run_linear_case(wl.x, wl.w, torch.float32, what="tiny")


def test_linear_every_small_m():
    """M = 1 .. 17 one by one, across the three dispatch regimes (fused decode
    up to 10 tokens, the GEMV on codes for 11 .. 16, the GEMM from 17), on a
    ragged shape: N = 40 (not a multiple of 16 or 32), K = 272 (not a multiple
    of 64), and on the per-group path with K = 384 (three groups of 128)."""
    log("[linear] every M in 1..17, N=40 K=272; per-group N=40 K=384")
    w = inputs.random_matrix(180, (40, 272), 0.02, torch.float32)
    wg = inputs.random_matrix(181, (40, 384), 0.02, torch.float32)
    for M in range(1, 18):
        x = inputs.random_matrix(182 + M, (M, 272), 1.0, torch.bfloat16)
        run_linear_case(x, w, torch.bfloat16, what=f"M={M}")
        xg = inputs.random_matrix(200 + M, (M, 384), 1.0, torch.bfloat16)
        run_grouped_linear_case(xg, wg, 128, torch.float32, what=f"grouped M={M}")


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_linear_decode_qproj_full_size(M):
    log(f"[linear] decode q_proj M={M} N=K=4096 bf16")
    wl = inputs.decode_qproj(M=M)
    wq, ws, wz = q8.q8_quantize_weight(g(wl.w), "int8_asym")
    y, acc = q8.q8_linear(g(wl.x), wq, ws, wz, out_dtype=torch.bfloat16, acc_out=True)
    rq, rs, rz = oracle_weights(wl.w)
    # every output: the oracle's integer product is one float64 BLAS call
    y_ref, inter = O.linear_int8(wl.x, rq, rs, rz)
    assert_equal(host(acc), inter["acc"].astype(np.int32), "INT32 accumulator")
    check_close(out_f64(y), y_ref, "output")


@pytest.mark.parametrize("M,N,K,dt", [(3, 100, 4112, torch.bfloat16),      # fused: two K segments, N tail
                                      (16, 48, 16, torch.float32),          # on codes: smallest K
                                      (7, 33, 208, torch.float16),          # fused: partial MFMA k-step
                                      (14, 33, 208, torch.float16),         # on codes: partial MFMA k-step
                                      (1, 1, 8192, torch.bfloat16),         # fused: one output feature
                                      (11, 100, 4112, torch.bfloat16),      # on codes, just above fused
                                      (16, 37, 8240, torch.float16),        # on codes: two K segments, N tail
                                      (13, 1, 64, torch.float32),           # on codes: one output feature
                                      (10, 40, 4112, torch.float16)])       # fused, largest M
def test_linear_decode_ragged(M, N, K, dt):
    log(f"[linear] decode ragged M={M} N={N} K={K} {dt}")
    x = inputs.random_matrix(30 + M, (M, K), 1.0, dt)
    w = inputs.random_matrix(40 + N, (N, K), 0.02, torch.float32)
    run_linear_case(x, w, torch.float32, what="decode ragged")


# Shapes that the GEMM's tile rule sends to each tile (asserted through
# q8_gemm_tile), with ragged M, N and K: every tile is compared on the whole
# matrix (the whole INT32 accumulator and every output).
GEMM_TILE_SHAPES = [((64, 64), 17, 64, 128),          # just above the decode path
                    ((64, 64), 300, 520, 1040),       # K tail of 16
                    ((64, 128), 500, 3000, 208),
                    ((64, 128), 512, 4096, 4096),     # the LLM.int8 shape through the plain layer
                    ((128, 128), 1000, 3000, 208),
                    ((256, 256), 2040, 6200, 336)]


@pytest.mark.parametrize("tile,M,N,K", GEMM_TILE_SHAPES)
def test_linear_gemm_tiles(tile, M, N, K):
    log(f"[linear] GEMM M={M} N={N} K={K} bf16, tile {tile}")
    assert q8.q8_gemm_tile("linear", M, N, K) == tile
    x = inputs.random_matrix(50 + M, (M, K), 1.0, torch.bfloat16)
    w = inputs.random_matrix(60 + N, (N, K), 0.02, torch.float32)
    bias = inputs.random_matrix(61, (N,), 0.3, torch.float32)
    run_linear_case(x, w, torch.bfloat16, bias=bias, what="gemm")


def test_linear_prefill_full_size():
    log("[linear] prefill FFN-up 2048x14336x4096 bf16, whole matrix")
    wl = inputs.prefill_ffn_up()
    assert q8.q8_gemm_tile("linear", 2048, 14336, 4096) == (256, 256)
    y, acc = run_linear_case(wl.x, wl.w, torch.bfloat16, what="prefill")
    # determinism: a second call gives identical bits
    wq, ws, wz = q8.q8_quantize_weight(g(wl.w), "int8_asym")
    y2, acc2 = q8.q8_linear(g(wl.x), wq, ws, wz, out_dtype=torch.bfloat16, acc_out=True)
    assert torch.equal(acc, acc2) and torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("M", [5, 12, 200])
def test_linear_bias_and_output_dtypes(M):
    log(f"[linear] bias + output dtypes M={M}")
    x = inputs.random_matrix(70, (M, 256), 1.0, torch.bfloat16)
    w = inputs.random_matrix(71, (96, 256), 0.02, torch.float32)
    bias = inputs.random_matrix(72, (96,), 0.5, torch.float32)
    for od in (torch.float32, torch.float16, torch.bfloat16):
        run_linear_case(x, w, od, bias=bias, what=f"bias {od}")


# ---------------------------------------------------------------- LLM.int8 decomposition
def run_decomp_case(x, w, tau, rows=None, bias=None, what=""):
    wq, ws, wz = q8.q8_quantize_weight(g(w), "int8_asym")
    b = g(bias) if bias is not None else None
    y, idx, cnt, acc = q8.q8_linear_int8_decomp(g(x), wq, ws, wz, threshold=tau, bias=b,
                                                return_outliers=True, acc_out=True)
    rq, rs, rz = oracle_weights(w)
    cols = O.outlier_columns(x, tau)
    n = int(host(cnt)[0])
    assert n == len(cols), (what, n, len(cols))
    assert_equal(host(idx)[:n], cols.astype(np.int32), f"{what} outlier columns")
    # the outlier set is a property of all rows; the per-row math is row-local
    xr = x if rows is None else x[rows]
    x_np = O.to_f32(x)
    xm = x_np.copy()
    xm[:, cols] = 0
    rq_x, rs_x, rr_x = O.quantize_act_int8_sym(xm if rows is None else xm[rows])
    acc_ref = O.int_gemm(rq_x, rq)
    y_ref = O.epilogue(acc_ref, rs_x, rr_x, rs, rz, bias)
    w_o = O.outlier_weights_f16(rq, rs, rz, cols)
    y_ref = y_ref + O.to_f32(xr)[:, cols].astype(np.float64) @ w_o.astype(np.float64).T
    acc_g = host(acc) if rows is None else host(acc)[rows]
    y_g = out_f64(y) if rows is None else out_f64(y)[rows]
    assert_equal(acc_g, acc_ref.astype(np.int32), f"{what} INT32 accumulator")
    check_close(y_g, y_ref, f"{what} output")
    if rows is None:
        y_full, _ = O.linear_int8_decomp(x, rq, rs, rz, tau, bias)
        check_close(y_g, y_full, f"{what} output vs oracle.linear_int8_decomp")
    return y


def test_decomp_llm_int8_full_size():
    log("[decomp] 512x4096x4096 fp16, 6 outlier columns, threshold 6.0")
    wl = inputs.llm_int8_outliers()
    run_decomp_case(wl.x, wl.w, 6.0, what="llm.int8")
    assert O.outlier_columns(wl.x, 6.0).tolist() == wl.extra["outlier_cols"].tolist()


@pytest.mark.parametrize("tile,M,N,K,seed", [((64, 128), 512, 4096, 4096, 31),   # the LLM.int8 shape, other seeds
                                             ((64, 128), 512, 4096, 8192, 32),   # two K segments of the outlier list
                                             ((128, 128), 1000, 3000, 208, 35),  # ragged
                                             ((64, 64), 300, 3000, 1024, 33),    # ragged M and N
                                             ((64, 64), 200, 1000, 512, 34)])
def test_decomp_whole_accumulator(tile, M, N, K, seed):
    """Every tile: the whole INT32 accumulator against the exact product of
    the oracle's codes (a float64 matmul of integers below 2^53 is exact), the
    output on sampled rows, and a second call giving the same bits.  (Seed 31
    has an outlier weight S (q - Z) next to a tie of fp16, where a fused
    single-rounding conversion differs from the two roundings.)"""
    log(f"[decomp] whole matrix: M={M} N={N} K={K}, tile {tile}")
    assert q8.q8_gemm_tile("decomp", M, N, K) == tile
    wl = inputs.llm_int8_outliers(seed=seed, M=M, K=K, N=N, n_outlier_cols=5)
    y = run_decomp_case(wl.x, wl.w, 6.0, what="whole")
    wq, ws, wz = q8.q8_quantize_weight(g(wl.w), "int8_asym")
    y1, _, _, acc = q8.q8_linear_int8_decomp(g(wl.x), wq, ws, wz, threshold=6.0, return_outliers=True, acc_out=True)
    y2 = q8.q8_linear_int8_decomp(g(wl.x), wq, ws, wz, threshold=6.0)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "second call differs"
    assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), "acc_out changes the output"
    cols = O.outlier_columns(wl.x, 6.0)
    xm = O.to_f32(wl.x).copy()
    xm[:, cols] = 0
    rq_x, _, _ = O.quantize_act_int8_sym(xm)
    rq, _, _ = oracle_weights(wl.w)
    acc_ref = rq_x.astype(np.float64) @ rq.astype(np.float64).T
    assert_equal(host(acc), acc_ref.astype(np.int64).astype(np.int32), "whole INT32 accumulator")


@pytest.mark.parametrize("K", [4096, 4112])
def test_decomp_row_cache_edge(K):
    # the masked quantizer keeps rows of up to 4096 values in a two-chunk
    # register cache and longer ones in the eight-chunk one
    log(f"[decomp] row cache edge K={K}")
    wl = inputs.llm_int8_outliers(M=40, K=K, N=200, n_outlier_cols=5)
    run_decomp_case(wl.x, wl.w, 6.0, what=f"K={K}")


@pytest.mark.parametrize("tau", [6.0, 0.0, -1.0, 1e-30])
def test_decomp_thresholds(tau):
    log(f"[decomp] threshold {tau}")
    wl = inputs.llm_int8_outliers(M=70, K=96, N=72, n_outlier_cols=3)
    run_decomp_case(wl.x, wl.w, tau, what=f"tau={tau}")


@pytest.mark.parametrize("n_cols,M,N,K", [(16, 200, 520, 1024), (17, 200, 520, 1024), (21, 333, 700, 2048),
                                          (40, 64, 4096, 4096)])
def test_decomp_more_outliers_than_the_panels(n_cols, M, N, K):
    """The first 16 outlier columns reach the GEMM through the quantizer's
    compact fp16 panels and any further ones through its gather path: exactly
    16, one more, and several chunks past the panels, on ragged and tile-
    aligned shapes, with the whole INT32 accumulator and every output."""
    log(f"[decomp] {n_cols} outlier columns: M={M} N={N} K={K}")
    wl = inputs.llm_int8_outliers(seed=40 + n_cols, M=M, K=K, N=N, n_outlier_cols=n_cols)
    run_decomp_case(wl.x, wl.w, 6.0, what=f"{n_cols} outliers")
    assert len(O.outlier_columns(wl.x, 6.0)) == n_cols


def test_decomp_exact_threshold_and_bias():
    log("[decomp] entries exactly at 6.0, bias, ragged shapes")
    x = inputs.random_matrix(80, (45, 2064), 1.0, torch.float32).numpy().clip(-3.5, 3.5)
    x[7, 100] = 6.0
    x[44, 2063] = -6.0
    x[0, 5] = 5.99
    x[3, 2048] = 60.0
    xt = torch.from_numpy(x).to(torch.float16)
    w = inputs.random_matrix(81, (130, 2064), 0.02, torch.float32)
    bias = inputs.random_matrix(82, (130,), 0.5, torch.float32)
    run_decomp_case(xt, w, 6.0, bias=bias, what="exact-6")
    assert O.outlier_columns(xt, 6.0).tolist() == [100, 2048, 2063]


# ---------------------------------------------------------------- FP8 linear
def run_fp8_case(x, w, ub, rows=None, bias=None, what=""):
    wq, ws, _ = q8.q8_quantize_weight(g(w), "fp8_e4m3")
    b = g(bias) if bias is not None else None
    y = q8.q8_linear_fp8(g(x), wq, ws, scale_ub=ub, bias=b)
    rq, rs = O.quantize_fp8_rowwise(w)
    assert_equal(host(wq), rq, f"{what} weight codes")
    xr = x if rows is None else x[rows]
    y_ref, _ = O.linear_fp8(xr, rq, rs, ub, bias)
    y_g = out_f64(y) if rows is None else out_f64(y)[rows]
    check_close_fp8(y_g, y_ref, xr, w, ub, f"{what} output")
    # the two-step form (quantize, then the rowwise GEMM) gives the same bits
    xq, xs, _ = q8.q8_quantize_act(g(x), "fp8_e4m3", scale_ub=ub)
    y2 = q8.q8_gemm_fp8(xq, xs, wq, ws, bias=b)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"{what}: q8_gemm_fp8 differs"
    return y


@pytest.mark.parametrize("tile,M,N,K", [((64, 64), 100, 500, 208),
                                        ((64, 128), 500, 3000, 208),
                                        ((128, 128), 1000, 3000, 208),
                                        ((128, 128), 1024, 4096, 256),
                                        ((256, 256), 2040, 6200, 336)])
def test_fp8_gemm_tiles(tile, M, N, K):
    """Every FP8 tile on the whole matrix, ragged M, N and K."""
    log(f"[fp8] M={M} N={N} K={K}, tile {tile}")
    assert q8.q8_gemm_tile("fp8", M, N, K) == tile
    x = inputs.random_matrix(95 + M, (M, K), 1.0, torch.bfloat16)
    w = inputs.random_matrix(96 + N, (N, K), 0.02, torch.float32)
    bias = inputs.random_matrix(97, (N,), 0.1, torch.float32)
    run_fp8_case(x, w, 1200.0, bias=bias, what="fp8 tile")


@pytest.mark.parametrize("M,N,K", [(200, 300, 1040), (37, 1000, 128), (600, 2100, 256)])
def test_fp8_linear_ragged(M, N, K):
    log(f"[fp8] M={M} N={N} K={K}")
    x = inputs.random_matrix(90 + M, (M, K), 1.0, torch.bfloat16)
    w = inputs.random_matrix(91 + N, (N, K), 0.02, torch.float32)
    bias = inputs.random_matrix(92, (N,), 0.1, torch.float32)
    run_fp8_case(x, w, 1200.0, bias=bias, what="fp8 ragged")


def test_fp8_linear_scale_ub_binds():
    log("[fp8] activation scale bound binds")
    x = inputs.random_matrix(93, (20, 256), 1.0, torch.float32).numpy()
    x[3, 10] = 3000.0
    x[5, :] *= 2000.0
    xt = torch.from_numpy(x).to(torch.bfloat16)
    w = inputs.random_matrix(94, (64, 256), 0.02, torch.float32)
    run_fp8_case(xt, w, 1000.0, what="fp8 ub")


def test_fp8_linear_full_size_sampled():
    log("[fp8] 4096x4096x14336 bf16, sampled rows")
    wl = inputs.fp8_rowwise()
    rows = sample_rows(4096, 8, seed=5, extra=(255, 256))
    run_fp8_case(wl.x, wl.w, 1200.0, rows=rows, what="fp8 full")


# ---------------------------------------------------------------- weight-only W8A16
def run_w8a16_case(x, w, out_dtype, cols=None, bias=None, what=""):
    """GPU q8_linear_w8a16 on the full problem; oracle O10 on output columns
    `cols` (all if None)."""
    wq, ws, wz = q8.q8_quantize_weight(g(w), "int8_asym")
    b = g(bias) if bias is not None else None
    y = q8.q8_linear_w8a16(g(x), wq, ws, wz, bias=b, out_dtype=out_dtype)
    rq, rs, rz = oracle_weights(w)
    if cols is None:
        y_ref = O.linear_w8a16(x, rq, rs, rz, bias=bias)
        y_g = out_f64(y)
    else:
        y_ref = O.linear_w8a16(x, rq[cols], rs[cols], rz[cols], bias=None if bias is None else bias[cols])
        y_g = out_f64(y)[:, cols]
    check_close(y_g, y_ref, f"{what} output")
    return y


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_w8a16_decode_qproj_full_size(M, dt):
    log(f"[w8a16] decode q_proj M={M} N=K=4096 {dt}")
    wl = inputs.decode_qproj(M=M)
    run_w8a16_case(wl.x.to(dt), wl.w, torch.bfloat16, what=f"w8a16 M={M}")


@pytest.mark.parametrize("M,N,K,dt", [(3, 100, 4112, torch.bfloat16),     # two K segments, N tail
                                      (16, 37, 8240, torch.float16),      # two segments, 16 rows
                                      (1, 1, 16, torch.float16),          # smallest K, one feature
                                      (7, 33, 208, torch.bfloat16),       # partial MFMA k-steps
                                      (5, 64, 1024, torch.float16)])
def test_w8a16_ragged(M, N, K, dt):
    log(f"[w8a16] ragged M={M} N={N} K={K} {dt}")
    x = inputs.random_matrix(110 + M, (M, K), 1.0, dt)
    w = inputs.random_matrix(120 + N, (N, K), 0.02, torch.float32)
    run_w8a16_case(x, w, torch.float32, what="w8a16 ragged")


def test_w8a16_one_signed_rows_and_bias():
    """Rows with all-positive or all-negative weights (zero points at the ends
    of the code range) and a bias, for each output dtype."""
    log("[w8a16] one-signed weight rows, bias, output dtypes")
    x = inputs.random_matrix(130, (4, 512), 1.0, torch.bfloat16)
    w = inputs.random_matrix(131, (48, 512), 0.02, torch.float32).numpy().copy()
    w[:8] = np.abs(w[:8])
    w[8:16] = -np.abs(w[8:16])
    w = torch.from_numpy(w)
    bias = inputs.random_matrix(132, (48,), 0.5, torch.float32)
    for od in (torch.float32, torch.float16, torch.bfloat16):
        run_w8a16_case(x, w, od, bias=bias, what=f"w8a16 bias {od}")


# ---------------------------------------------------------------- static scales, INT8 output
@pytest.mark.parametrize("name,M,K,dt,scale", [("bf16_2048x4096", 2048, 4096, torch.bfloat16, 0.021),
                                               ("f32_37x272_saturating", 37, 272, torch.float32, 0.004),
                                               ("f16_5x1040", 5, 1040, torch.float16, 0.0371),
                                               ("bf16_4x4112_cache_edge", 4, 4112, torch.bfloat16, 0.019)])
def test_quantize_act_static_codes(name, M, K, dt, scale):
    log(f"[act static] {name} S={scale}")
    x = inputs.random_matrix(140 + M, (M, K), 1.0, dt)
    xq, rs = q8.q8_quantize_act_static(g(x), scale)
    rq, rr = O.quantize_act_int8_static(x, scale)
    assert_equal(host(xq), rq, "static codes")
    assert_equal(host(rs), rr, "static row sums")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("K", [1024, 4112])
def test_quantize_act_static_every_value(dt, K):
    # Every finite 16-bit value in [-64, 64] against scales that put x / S on
    # half-integers (0.25, 0.5), next to them (0.1, 1/3, 0.0371, 7), far past
    # the clamp (1e-3, 1.5e-38: x / S overflows), and with a reciprocal below
    # the normal range (1e38): the kernel decides most codes from x * RN(1/S)
    # and the ones next to a half-integer by the division; all must equal the
    # binary32 division's codes.
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    if dt == torch.bfloat16:
        vals = (bits.astype(np.uint32) << 16).view(np.float32)
    else:
        vals = bits.view(np.float16).astype(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 64.0)]
    M = (vals.size + K - 1) // K
    flat = np.zeros(M * K, dtype=np.float32)
    flat[:vals.size] = vals
    x = torch.tensor(flat.reshape(M, K)).to(dt)
    for scale in (0.25, 0.5, 0.1, 1.0 / 3.0, 0.0371, 7.0, 1e-3, 1.5e-38, 1e38):
        log(f"[act static] every {dt} value, K={K}, S={scale}")
        xq, rs = q8.q8_quantize_act_static(g(x), scale)
        rq, rr = O.quantize_act_int8_static(x, scale)
        assert_equal(host(xq), rq, f"static codes S={scale}")
        assert_equal(host(rs), rr, f"static row sums S={scale}")


def run_static_case(x, w, x_scale, rows=None, bias=None, clip_frac=0.2, what=""):
    """GPU q8_linear_static on the full problem; oracle O12 on `rows` (all if
    None).  The output scale is set from the oracle's float64 values so that
    about `clip_frac` of the largest outputs saturate."""
    wq, ws, wz = q8.q8_quantize_weight(g(w), "int8_asym")
    rq, rs, rz = oracle_weights(w)
    xr = x if rows is None else x[rows]
    _, inter = O.linear_static(xr, x_scale, rq, rs, rz, 1.0, bias=bias)
    y_scale = float(np.float32(np.quantile(np.abs(inter["y"][::7]), 1.0 - clip_frac) / 127.0))
    yq_ref = O.requantize_int8(inter["y"], y_scale)
    b = g(bias) if bias is not None else None
    yq = q8.q8_linear_static(g(x), x_scale, wq, ws, wz, y_scale, bias=b)
    got = host(yq) if rows is None else host(yq)[rows]
    assert_equal(got, yq_ref, f"{what} int8 output")
    sat = float(np.mean(np.abs(yq_ref.astype(int)) == 127))
    log(f"  {what}: {yq_ref.size} int8 outputs bit-exact, {sat:.1%} saturated")


@pytest.mark.parametrize("tile,M,N,K,sx", [((0, 0), 1, 4096, 4096, 0.03),        # decode: streaming GEMV on codes
                                           ((0, 0), 16, 100, 4112, 0.02),        # decode, N tail, two K segments
                                           ((64, 64), 300, 520, 1040, 0.025),
                                           ((64, 128), 500, 3000, 208, 0.03),
                                           ((128, 128), 1000, 3000, 208, 0.03),
                                           ((256, 256), 2040, 6200, 336, 0.03)])  # ragged M/N
def test_linear_static_int8_output(tile, M, N, K, sx):
    log(f"[linear static] M={M} N={N} K={K} S_x={sx}, tile {tile}")
    assert q8.q8_gemm_tile("static", M, N, K) == tile
    x = inputs.random_matrix(150 + M, (M, K), 1.0, torch.bfloat16)
    w = inputs.random_matrix(160 + N, (N, K), 0.02, torch.float32)
    run_static_case(x, w, sx, what=f"static {M}x{N}x{K}")


def test_linear_static_prefill_full_size_with_bias():
    log("[linear static] prefill 2048x14336x4096 bf16 with bias, whole matrix")
    wl = inputs.prefill_ffn_up()
    bias = inputs.random_matrix(170, (14336,), 0.5, torch.float32)
    run_static_case(wl.x, wl.w, 0.03, bias=bias, what="static prefill")


# ---------------------------------------------------------------- FP8 experts on routed tokens
def run_grouped_case(x, w, offsets, rows_per_expert=None, ub=1200.0, what=""):
    """GPU q8_linear_fp8_grouped; oracle O13 on every row (rows_per_expert None)
    or on a sample of each expert's rows.  Also checks that the grouped call on
    each expert's rows equals the plain FP8 linear of those rows, bit for bit."""
    E, N, K = w.shape
    T = x.shape[0]
    wq, ws, _ = q8.q8_quantize_weight(g(w.reshape(E * N, K)), "fp8_e4m3")
    wq, ws = wq.view(E, N, K), ws.view(E, N)
    off = torch.tensor(np.asarray(offsets), dtype=torch.int32)
    y = q8.q8_linear_fp8_grouped(g(x), g(off), wq, ws, scale_ub=ub)
    rq, rs = O.quantize_fp8_rowwise(w.reshape(E * N, K))
    rq, rs = rq.reshape(E, N, K), rs.reshape(E, N)
    y_g = out_f64(y)
    rows = []
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        r = np.arange(lo, hi) if rows_per_expert is None else \
            np.unique(np.r_[lo, hi - 1, np.random.default_rng(e).integers(lo, hi, rows_per_expert)])
        yr, _ = O.linear_fp8(x[r], rq[e], rs[e], ub)
        rows.append(r)
        check_close_fp8(y_g[r], yr, x[r], w[e], ub, f"{what} expert {e} output ({len(r)} rows)")
        if hi - lo <= 600:
            # the same rows through the plain rowwise FP8 path give the same bits
            y1 = q8.q8_linear_fp8(g(x[lo:hi]), wq[e].contiguous(), ws[e].contiguous(), scale_ub=ub)
            assert torch.equal(y[lo:hi].view(torch.int16), y1.view(torch.int16)), f"{what}: expert {e} differs"
    assert sum(len(r) for r in rows) > 0 or int(offsets[-1]) == 0


def test_fp8_grouped_moe_full_size():
    wl = inputs.moe_fp8()
    off = wl.extra["offsets"].numpy()
    log(f"[fp8 experts] {wl.name}, tokens per expert {np.diff(off).tolist()}")
    E = off.size - 1
    run_grouped_case(wl.x, wl.w.view(E, -1, wl.w.shape[-1]), off, rows_per_expert=8, what="moe full")


@pytest.mark.parametrize("counts,N,K", [([0, 130, 0, 7, 300, 0], 200, 528),     # empty experts, 64x128 tiles
                                        ([513], 256, 256),                       # one expert, 128x128 tiles (mean 513)
                                        ([1, 1, 1, 1], 96, 64),                  # one token each
                                        ([150, 0, 400, 100], 1000, 1040),        # 128x128 tiles (mean 162)
                                        ([900, 0, 411, 300], 520, 576),          # 128x128 tiles (mean 402), N tail
                                        ([1600, 7], 300, 320)])                  # 256x256 tiles (mean 803)
def test_fp8_grouped_ragged(counts, N, K):
    log(f"[fp8 experts] counts={counts} N={N} K={K}")
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    x = inputs.random_matrix(180 + sum(counts), (max(int(offsets[-1]), 1), K), 1.0, torch.bfloat16)
    w = inputs.random_matrix(190 + N, (E, N, K), 0.02, torch.float32)
    run_grouped_case(x[:int(offsets[-1])], w, offsets, what="moe ragged")


def test_fp8_grouped_many_experts_and_malformed_offsets():
    """300 experts, most of them holding a few tokens or none; then offsets
    that decrease, go below 0 and past T.  The kernel reads them as the
    running maximum of max(offsets, 0) capped at T (group e spans c[e] ..
    c[e+1]); rows inside those spans are compared with the oracle for their
    expert, rows outside every span are left alone."""
    log("[fp8 experts] 300 experts; malformed offsets")
    rng = np.random.default_rng(210)
    counts = rng.integers(0, 8, 300)
    counts[rng.random(300) < 0.4] = 0
    run_grouped_case(inputs.random_matrix(211, (int(counts.sum()), 128), 1.0, torch.bfloat16),
                     inputs.random_matrix(212, (300, 96, 128), 0.02, torch.float32),
                     np.concatenate([[0], np.cumsum(counts)]), what="300 experts")
    T, N, K = 800, 160, 192
    raw = np.array([5, -3, 400, 200, 900, 1200, 700])
    E = raw.size - 1
    c = np.minimum(np.maximum.accumulate(np.maximum(raw, 0)), T)
    assert c.tolist() == [5, 5, 400, 400, 800, 800, 800]
    x = inputs.random_matrix(213, (T, K), 1.0, torch.bfloat16)
    w = inputs.random_matrix(214, (E, N, K), 0.02, torch.float32)
    wq, ws, _ = q8.q8_quantize_weight(g(w.reshape(E * N, K)), "fp8_e4m3")
    y = q8.q8_linear_fp8_grouped(g(x), g(torch.tensor(raw, dtype=torch.int32)), wq.view(E, N, K), ws.view(E, N),
                                 scale_ub=1200.0)
    rq, rs = O.quantize_fp8_rowwise(w.reshape(E * N, K))
    rq, rs = rq.reshape(E, N, K), rs.reshape(E, N)
    for e in range(E):
        lo, hi = int(c[e]), int(c[e + 1])
        if hi > lo:
            yr, _ = O.linear_fp8(x[lo:hi], rq[e], rs[e], 1200.0)
            check_close_fp8(out_f64(y[lo:hi]), yr, x[lo:hi], w[e], 1200.0, f"malformed offsets, expert {e} rows {lo}..{hi - 1}")


# ---------------------------------------------------------------- per-group weights (q8_linear_grouped)
def varied_groups(w, group, seed):
    """The same weights with every group scaled by 10^u (u in -1..1) and the
    first two groups of every row made one-signed (Z = -128 and Z = 127), so a
    parameter taken from the wrong group or row changes the output."""
    a = w.float().numpy().copy()
    N, K = a.shape
    rng = np.random.default_rng(seed)
    a *= (10.0 ** rng.integers(-1, 2, (N, K // group))).repeat(group, axis=1).astype(np.float32)
    a[:, :group] = np.abs(a[:, :group])
    if K >= 2 * group:
        a[:, group:2 * group] = -np.abs(a[:, group:2 * group])
    return torch.from_numpy(a).to(w.dtype)


def check_grouped_weights(w, group, what=""):
    wq, ws, wz = q8.q8_quantize_weight_grouped(g(w), group)
    rq, rs, rz = O.quantize_weight_int8_grouped(w, group)
    assert_equal(host(wq), rq, f"{what} grouped weight codes")
    assert_equal(f32_bits(host(ws)), f32_bits(rs), f"{what} grouped scale bits")
    assert_equal(host(wz), rz, f"{what} grouped zero points")
    return (wq, ws, wz), (rq, rs, rz)


def run_grouped_linear_case(x, w, group, out_dtype, rows=None, cols=None, bias=None, what=""):
    """GPU q8_linear_grouped on the full problem; oracle O15 on `rows` x `cols`."""
    (wq, ws, wz), (rq, rs, rz) = check_grouped_weights(w, group, what)
    b = g(bias) if bias is not None else None
    y = q8.q8_linear_grouped(g(x), wq, ws, wz, group, bias=b, out_dtype=out_dtype)
    xr = x if rows is None else x[rows]
    br = bias
    if cols is not None:
        rq, rs, rz = rq[cols], rs[:, cols], rz[:, cols]
        br = None if bias is None else bias[cols]
    y_ref, _ = O.linear_int8_grouped(xr, rq, rs, rz, group, bias=br)
    yg = out_f64(y)
    if rows is not None:
        yg = yg[rows]
    if cols is not None:
        yg = yg[:, cols]
    check_close(yg, y_ref, f"{what} output")
    return y


@pytest.mark.parametrize("name,N,K,group,dt,seed", [("f32_256x256_g128", 256, 256, 128, torch.float32, 90),
                                                    ("f32_37x192_g64", 37, 192, 64, torch.float32, 91),
                                                    ("bf16_65x4224_g128", 65, 4224, 128, torch.bfloat16, 92),
                                                    ("f16_9x8256_g64", 9, 8256, 64, torch.float16, 93)])
def test_quantize_weight_grouped(name, N, K, group, dt, seed):
    log(f"[grouped] weight quantization {name}")
    w = inputs.random_matrix(seed, (N, K), 0.02, dt)
    check_grouped_weights(w, group, name)
    check_grouped_weights(varied_groups(w, group, seed), group, name + " varied")


def test_quantize_weight_grouped_edge_groups():
    log("[grouped] weight quantization: zero, constant and one-signed groups")
    w = inputs.random_matrix(94, (8, 512), 0.02, torch.float32).numpy().copy()
    w[0, :64] = 0.0                 # all-zero group: S = eps, Z = -128, codes -128
    w[1, 64:128] = 0.37             # constant positive group
    w[2, 128:192] = -1e-3           # constant negative group
    w[3, :] = np.abs(w[3, :])
    w[4, :] = -np.abs(w[4, :])
    check_grouped_weights(torch.from_numpy(w), 64, "edge")


@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_linear_grouped_decode_qproj_full_size(M, group):
    log(f"[grouped] decode q_proj M={M} N=K=4096 group={group} bf16")
    wl = inputs.decode_qproj(M=M)
    run_grouped_linear_case(wl.x, wl.w, group, torch.bfloat16, what="decode")


@pytest.mark.parametrize("M,N,K,group,dt", [(3, 100, 4224, 128, torch.bfloat16),   # decode: partial 2nd segment, N tail
                                            (16, 37, 8256, 64, torch.float16),     # decode: 3 segments, N tail
                                            (1, 1, 128, 128, torch.float32),       # one output, one group
                                            (13, 50, 64, 64, torch.bfloat16),      # one group of 64
                                            (17, 64, 128, 128, torch.bfloat16),    # just above the decode path
                                            (300, 520, 1024, 64, torch.bfloat16),  # GEMM: ragged M and N
                                            (1000, 3000, 256, 128, torch.float16), # GEMM: few groups
                                            (130, 4100, 4224, 128, torch.float32), # GEMM: odd group count
                                            (257, 300, 192, 64, torch.bfloat16),   # GEMM: 3 stages, 3 groups
                                            (40, 70, 64, 64, torch.bfloat16),      # GEMM: one stage, one group
                                            (33, 130, 128, 64, torch.float16)])    # GEMM: two stages, two groups
def test_linear_grouped_ragged(M, N, K, group, dt):
    log(f"[grouped] ragged M={M} N={N} K={K} group={group} {dt}")
    x = inputs.random_matrix(100 + M, (M, K), 1.0, dt)
    w = varied_groups(inputs.random_matrix(110 + N, (N, K), 0.02, torch.float32), group, N)
    run_grouped_linear_case(x, w, group, torch.float32, what="ragged")


def test_linear_grouped_prefill_full_size():
    log("[grouped] prefill FFN-up 2048x14336x4096 group=128 bf16, whole matrix")
    wl = inputs.prefill_ffn_up()
    y = run_grouped_linear_case(wl.x, wl.w, 128, torch.bfloat16, what="prefill")
    wq, ws, wz = q8.q8_quantize_weight_grouped(g(wl.w), 128)
    y2 = q8.q8_linear_grouped(g(wl.x), wq, ws, wz, 128, out_dtype=torch.bfloat16)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "second call differs"


@pytest.mark.parametrize("M", [5, 200])
def test_linear_grouped_bias_and_dtypes(M):
    log(f"[grouped] bias + input/output dtypes M={M}")
    w = varied_groups(inputs.random_matrix(120, (96, 512), 0.02, torch.float32), 128, 7)
    bias = inputs.random_matrix(121, (96,), 0.5, torch.float32)
    for xd in (torch.float32, torch.float16, torch.bfloat16):
        x = inputs.random_matrix(122, (M, 512), 1.0, xd)
        for od in (torch.float32, torch.float16, torch.bfloat16):
            run_grouped_linear_case(x, w, 128, od, bias=bias, what=f"x {xd} y {od}")


# ---------------------------------------------------------------- maximum sizes
@pytest.mark.parametrize("M", [1, 16, 33])
def test_linear_max_k_extreme_accumulators(M):
    """K = 65536, the largest accepted, with codes that drive the INT32 sums
    to their extremes: acc = -16256 K and the zero-point-corrected sum
    -32385 K = -2.12e9 (127 * 255 * K, within 1.3 % of the int32 limit), on
    the fused decode (M = 1), the GEMV on codes (M = 16) and the GEMM (M = 33)."""
    log(f"[linear] K = 65536 extreme codes, M={M}")
    wl = inputs.extreme_codes(M=M)
    rq, _, rz = oracle_weights(wl.w)
    assert (rq[0::3] == -128).all() and (rz[0::3] == 127).all()
    assert (rq[1::3] == 127).all() and (rz[1::3] == -128).all()
    y, acc = run_linear_case(wl.x, wl.w, torch.bfloat16, what=f"K=65536 M={M}")
    a = host(acc)
    assert a[:, 0::3].min() == -16256 * 65536 and a[:, 1::3].max() == 16129 * 65536


@pytest.mark.parametrize("path,M", [("fp8", 1), ("fp8", 33), ("decomp", 40), ("w8a16", 1), ("w8a16", 16),
                                    ("grouped128", 1), ("grouped64", 16), ("grouped128", 40), ("static", 33)])
def test_other_paths_at_max_k(path, M):
    """Every other product at K = 65536, the largest accepted (16 K segments
    of the decode kernels, 1024 stages of the GEMM main loops, 512 or 1024
    weight groups)."""
    K, N = 65536, 64
    log(f"[max K] {path} M={M} N={N} K={K}")
    w = inputs.random_matrix(90 + M, (N, K), 0.02, torch.float32)
    if path == "fp8":
        run_fp8_case(inputs.random_matrix(91 + M, (M, K), 1.0, torch.bfloat16), w, 1200.0, what=f"fp8 K={K}")
    elif path == "decomp":
        d = inputs.llm_int8_outliers(seed=92, M=M, K=K, N=N, n_outlier_cols=5)
        run_decomp_case(d.x, d.w, 6.0, what=f"decomp K={K}")
    elif path == "w8a16":
        run_w8a16_case(inputs.random_matrix(93 + M, (M, K), 1.0, torch.bfloat16), w, torch.bfloat16,
                       what=f"w8a16 K={K}")
    elif path == "static":
        run_static_case(inputs.random_matrix(94 + M, (M, K), 1.0, torch.bfloat16), w, 0.02, what=f"static K={K}")
    else:
        group = int(path[len("grouped"):])
        run_grouped_linear_case(inputs.random_matrix(95 + M, (M, K), 1.0, torch.bfloat16), w, group,
                                torch.bfloat16, what=f"grouped g{group} K={K}")


@pytest.mark.parametrize("K", [16, 48])
def test_short_k_every_gemm(K):
    """K below one 64-byte stage: the GEMMs run no DMA stage at all, only the
    register-loaded partial stage (int8, FP8 and LLM.int8 tiles, M above the
    decode sizes), and the decode kernels a single partial k-step."""
    log(f"[short K] K={K}: int8 GEMM, FP8 GEMM, LLM.int8, decode")
    w = inputs.random_matrix(120 + K, (70, K), 0.02, torch.float32)
    for M in (3, 13, 40, 300):
        run_linear_case(inputs.random_matrix(121 + M, (M, K), 1.0, torch.bfloat16), w, torch.bfloat16,
                        what=f"int8 K={K} M={M}")
    run_fp8_case(inputs.random_matrix(125, (300, K), 1.0, torch.bfloat16), w, 1200.0, what=f"fp8 K={K}")
    d = inputs.llm_int8_outliers(seed=126, M=300, K=K, N=70, n_outlier_cols=2)
    run_decomp_case(d.x, d.w, 6.0, what=f"decomp K={K}")
    for M in (1, 16):
        run_w8a16_case(inputs.random_matrix(127 + M, (M, K), 1.0, torch.bfloat16), w, torch.bfloat16,
                       what=f"w8a16 K={K} M={M}")
    run_static_case(inputs.random_matrix(129, (300, K), 1.0, torch.bfloat16), w, 0.02, what=f"static K={K}")


def test_linear_max_weight_elements_sampled():
    """A weight matrix of N * K = 32767 * 65536 = 2^31 - 65536 elements, just
    under the 2^31 limit of the 32-bit offsets (2 GB of int8 codes), through
    the fused decode (M = 1) and the GEMM (M = 64); codes, scales and zero
    points are bit-exact and outputs within tolerance on sampled rows up to
    the last one."""
    N, K = 32767, 65536
    log(f"[linear] {N}x{K} weights (2^31 - 2^16 elements), sampled rows")
    base, rows_of = inputs.tiled_rows(K=K)
    bg = g(base)
    w = torch.empty(N, K, dtype=torch.float32, device=DEV)
    for r0 in range(0, N, 4096):
        r1 = min(N, r0 + 4096)
        w[r0:r1] = rows_of(bg, torch.arange(r0, r1, device=DEV))
    wq, ws, wz = q8.q8_quantize_weight(w, "int8_asym")
    del w, bg
    torch.cuda.empty_cache()
    sel = np.array([0, 1, 256, 16383, 32511, 32640, 32765, N - 1])
    w_sel = rows_of(base, torch.from_numpy(sel))
    rq, rs, rz = O.quantize_weight_int8_asym(w_sel)
    assert_equal(host(wq[torch.from_numpy(sel).to(DEV)]), rq, "codes of the sampled rows")
    assert_equal(host(ws[torch.from_numpy(sel).to(DEV)]).view(np.uint32), rs.view(np.uint32), "scales")
    assert_equal(host(wz[torch.from_numpy(sel).to(DEV)]), rz, "zero points")
    x = inputs.random_matrix(82, (64, K), 1.0, torch.bfloat16)
    for M in (1, 64):
        y = q8.q8_linear(g(x[:M]), wq, ws, wz, out_dtype=torch.bfloat16)
        y_ref, _ = O.linear_int8(x[:M], rq, rs, rz)
        check_close(out_f64(y)[:, sel], y_ref, f"max weight elements M={M}")
    del wq
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- pointer validation
_VALIDATE_CHILD = '''
import torch
from w8a8_quantized_linear_channel_amd import _lib, ops as q8
dev = "cuda:0"
w = torch.randn(64, 64, device=dev)
wq, ws, wz = q8.q8_quantize_weight(w, "int8_asym")
x = torch.randn(4, 64, device=dev, dtype=torch.bfloat16)
y = torch.empty(4, 64, device=dev, dtype=torch.bfloat16)
xh = x.cpu().pin_memory()   # pinned: device-readable, so even an unchecked launch could not fault
L = _lib.lib()
st = torch.cuda.current_stream().cuda_stream
host_x = L.q8_linear(xh.data_ptr(), _lib.Q8_BF16, 4, 64, wq.data_ptr(), ws.data_ptr(), wz.data_ptr(), 64,
                     None, y.data_ptr(), _lib.Q8_BF16, None, 0, None, st)
dev_x = L.q8_linear(x.data_ptr(), _lib.Q8_BF16, 4, 64, wq.data_ptr(), ws.data_ptr(), wz.data_ptr(), 64,
                    None, y.data_ptr(), _lib.Q8_BF16, None, 0, None, st)
torch.cuda.synchronize()
print(host_x, dev_x, flush=True)
'''


def test_debug_pointer_validation():
    """With Q8_DEBUG_VALIDATE=1 every pointer is checked to be device memory
    of the stream's device: a (pinned) host buffer is Q8_ERR_BAD_ARG before
    any launch, device buffers pass.  Run in a child process (the switch is
    read once per process)."""
    import os
    import subprocess
    import sys
    log("[validate] Q8_DEBUG_VALIDATE=1: host pointer rejected, device pointers accepted")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, Q8_DEBUG_VALIDATE="1", PYTHONPATH=root)
    r = subprocess.run([sys.executable, "-c", _VALIDATE_CHILD], env=env, cwd=root, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    host_st, dev_st = map(int, r.stdout.split()[-2:])
    assert host_st == 5 and dev_st == 0, r.stdout


# ---------------------------------------------------------------- concurrent streams
def test_calls_on_two_streams_run_concurrently():
    """The library keeps no state between calls, so calls enqueued on two
    streams at once (each with its own workspace) give the same bits as the
    same calls run one after the other."""
    log("[streams] q8_linear, LLM.int8 and FP8 interleaved on two streams")
    w = g(inputs.random_matrix(140, (512, 1024), 0.02, torch.float32))
    wq, ws, wz = q8.q8_quantize_weight(w, "int8_asym")
    fq, fs = q8.q8_quantize_weight(w, "fp8_e4m3")[:2]
    d = inputs.llm_int8_outliers(seed=141, M=96, K=1024, N=512, n_outlier_cols=4)
    dq, ds, dz = q8.q8_quantize_weight(g(d.w), "int8_asym")
    xd = g(d.x)
    xs = [g(inputs.random_matrix(142 + i, (M, 1024), 1.0, torch.bfloat16)) for i, M in enumerate((1, 16, 700, 300))]

    def calls(i):
        x = xs[i]
        M = x.shape[0]
        y = torch.empty(M, 512, dtype=torch.bfloat16, device=DEV)
        wl = torch.empty(max(1, q8.q8_workspace_bytes("linear", M, 512, 1024)), dtype=torch.uint8, device=DEV)
        yf = torch.empty(M, 512, dtype=torch.bfloat16, device=DEV)
        wf = torch.empty(max(1, q8.q8_workspace_bytes("fp8", M, 512, 1024)), dtype=torch.uint8, device=DEV)
        yd = torch.empty(96, 512, dtype=torch.float16, device=DEV)
        wd = torch.empty(q8.q8_workspace_bytes("decomp", 96, 512, 1024), dtype=torch.uint8, device=DEV)

        def run():
            q8.q8_linear(x, wq, ws, wz, out=y, workspace=wl)
            q8.q8_linear_fp8(x, fq, fs, out=yf, workspace=wf)
            q8.q8_linear_int8_decomp(xd, dq, ds, dz, 6.0, out=yd, workspace=wd)
        return run, (y, yf, yd)

    jobs = [calls(i) for i in range(len(xs))]
    ref = []
    for run, outs in jobs:
        run()
        torch.cuda.synchronize()
        ref.append([o.clone() for o in outs])
        for o in outs:
            o.fill_(0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for i, (run, _) in enumerate(jobs):
            with torch.cuda.stream(streams[i % 2]):
                run()
        torch.cuda.synchronize()
        for i, (_, outs) in enumerate(jobs):
            for o, r in zip(outs, ref[i]):
                assert torch.equal(o.view(torch.int16), r.view(torch.int16)), f"rep {rep}, job {i} differs"
                o.fill_(0)
        torch.cuda.synchronize()


# ---------------------------------------------------------------- empty batch
def test_empty_batch_every_entry_point():
    """An empty batch (M = 0 tokens) gives empty outputs from every call
    that takes activations and enqueues nothing; the LLM.int8 call still
    reports its outlier set as empty (count 0, list untouched).  A call on a
    real batch before and after gives the same bits."""
    from w8a8_quantized_linear_channel_amd import _lib
    log("[empty] M = 0 through every activation entry point")
    K, N = 256, 128
    w = g(inputs.random_matrix(71, (N, K), 0.02, torch.float32))
    wq, ws, wz = q8.q8_quantize_weight(w, "int8_asym")
    fq, fs = q8.q8_quantize_weight(w, "fp8_e4m3")[:2]
    gq, gs, gz = q8.q8_quantize_weight_grouped(w, 128)
    x3 = g(inputs.random_matrix(72, (3, K), 1.0, torch.bfloat16))
    before = q8.q8_linear(x3, wq, ws, wz)
    xb = torch.empty(0, K, dtype=torch.bfloat16, device=DEV)
    xh = torch.empty(0, K, dtype=torch.float16, device=DEV)
    assert q8.q8_linear(xb, wq, ws, wz).shape == (0, N)
    xq, xs, rs = q8.q8_quantize_act(xb)
    assert xq.shape == (0, K) and xs.shape == (0,) and rs.shape == (0,)
    fx, fxs, _ = q8.q8_quantize_act(xb, "fp8_e4m3", scale_ub=1200.0)
    assert fx.shape == (0, K)
    assert q8.q8_gemm_int8(xq, xs, rs, wq, ws, wz).shape == (0, N)
    assert q8.q8_gemm_fp8(fx, fxs, fq, fs).shape == (0, N)
    assert q8.q8_linear_fp8(xb, fq, fs).shape == (0, N)
    assert q8.q8_linear_w8a16(xb, wq, ws, wz).shape == (0, N)
    assert q8.q8_linear_grouped(xb, gq, gs, gz, 128).shape == (0, N)
    sq, srs = q8.q8_quantize_act_static(xb, 0.05)
    assert sq.shape == (0, K) and srs.shape == (0,)
    assert q8.q8_linear_static(xb, 0.05, wq, ws, wz, 0.1).shape == (0, N)
    eq, es = q8.q8_quantize_weight(w.repeat(3, 1), "fp8_e4m3")[:2]
    off = torch.zeros(4, dtype=torch.int32, device=DEV)
    assert q8.q8_linear_fp8_grouped(xb, off, eq.view(3, N, K), es.view(3, N)).shape == (0, N)
    assert q8.q8_linear_int8_decomp(xh, wq, ws, wz, 6.0).shape == (0, N)
    # the count is written even for no rows; the list is left alone
    cnt = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    idx = torch.full((K,), -5, dtype=torch.int32, device=DEV)
    st = _lib.lib().q8_linear_int8_decomp(None, 0, K, wq.data_ptr(), ws.data_ptr(), wz.data_ptr(), N, 6.0, None,
                                          None, None, 0, idx.data_ptr(), cnt.data_ptr(), None,
                                          torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert int(cnt.item()) == 0 and bool((idx == -5).all())
    after = q8.q8_linear(x3, wq, ws, wz)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), after.view(torch.int16))


# ---------------------------------------------------------------- graph capture
def test_graph_capture_replays_match_eager():
    """Every call is asynchronous on the caller's stream and allocates nothing,
    so it can be captured in a HIP graph.  Each captured call is replayed three
    times, with eager work and synchronizations between the replays, and every
    replay must give the eager result bit for bit (no memset nodes, no state
    kept between calls)."""
    log("[graph] capture and replay: decode (fused, on codes), GEMM, LLM.int8, FP8, per-group")
    wl = inputs.decode_qproj(M=16)
    w = g(wl.w[:512, :1024].contiguous())
    wq, ws, wz = q8.q8_quantize_weight(w, "int8_asym")
    gq, gs, gz = q8.q8_quantize_weight_grouped(w, 128)
    fq, fs = q8.q8_quantize_weight(w, "fp8_e4m3")[:2]
    xs = {M: g(inputs.random_matrix(200 + M, (M, 1024), 1.0, torch.bfloat16)) for M in (1, 16, 96)}
    d = inputs.llm_int8_outliers(seed=9, M=96, K=1024, N=512, n_outlier_cols=3)
    dq, ds, dz = q8.q8_quantize_weight(g(d.w), "int8_asym")
    xd = g(d.x)
    calls = []
    for M, x in xs.items():
        y = torch.empty(M, 512, dtype=torch.bfloat16, device=DEV)
        wsp = torch.empty(max(1, q8.q8_workspace_bytes("linear", M, 512, 1024)), dtype=torch.uint8, device=DEV)
        calls.append((f"linear M={M}", y, lambda x=x, y=y, wsp=wsp: q8.q8_linear(x, wq, ws, wz, out=y, workspace=wsp)))
        yg_ = torch.empty(M, 512, dtype=torch.bfloat16, device=DEV)
        wg = torch.empty(max(1, q8.q8_workspace_bytes("grouped", M, 512, 1024)), dtype=torch.uint8, device=DEV)
        calls.append((f"grouped M={M}", yg_,
                      lambda x=x, y=yg_, wg=wg: q8.q8_linear_grouped(x, gq, gs, gz, 128, out=y, workspace=wg)))
    yd = torch.empty(96, 512, dtype=torch.float16, device=DEV)
    wd = torch.empty(q8.q8_workspace_bytes("decomp", 96, 512, 1024), dtype=torch.uint8, device=DEV)
    calls.append(("llm.int8", yd, lambda: q8.q8_linear_int8_decomp(xd, dq, ds, dz, 6.0, out=yd, workspace=wd)))
    yf = torch.empty(96, 512, dtype=torch.bfloat16, device=DEV)
    wf = torch.empty(q8.q8_workspace_bytes("fp8", 96, 512, 1024), dtype=torch.uint8, device=DEV)
    calls.append(("fp8", yf, lambda: q8.q8_linear_fp8(xs[96], fq, fs, out=yf, workspace=wf)))

    eager = {}
    for name, y, fn in calls:
        fn()
        torch.cuda.synchronize()
        eager[name] = y.clone()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for _, _, fn in calls:
                fn()
    torch.cuda.synchronize()
    for rep in range(3):
        for _, y, _ in calls:
            y.fill_(0)                      # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, y, _ in calls:
            assert torch.equal(y.view(torch.int16), eager[name].view(torch.int16)), f"replay {rep}: {name} differs"
