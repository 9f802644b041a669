"""Host-side tests of the C ABI: the library loads, exports every function
include/q8.h declares, and rejects bad arguments before any device work.
Pointers passed here are never dereferenced (validation fails first), so
these run without a GPU."""
import ctypes
import os
import re

import pytest

from w8a8_quantized_linear_channel_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8.h")
BENCH_HEADER = os.path.join(ROOT, "include", "q8_bench.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libq8.so not built")

P = 0x10000           # a fake 16-byte-aligned device address (never dereferenced)
P2 = 0x20000
MIS = 0x10004         # misaligned
INF = float("inf")
NAN = float("nan")


def declared_functions():
    text = open(HEADER).read() + open(BENCH_HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_calls_and_helpers():
    names = declared_functions()
    for f in ["q8_quantize_weight", "q8_quantize_act", "q8_linear", "q8_linear_int8_decomp",
              "q8_linear_fp8", "q8_linear_w8a16", "q8_quantize_act_static", "q8_linear_static",
              "q8_linear_fp8_grouped", "q8_quantize_weight_grouped", "q8_linear_grouped",
              "q8_workspace_bytes", "q8_status_str"]:
        assert f in names
    assert set(names) == set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    h = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(h, name), name


def test_status_strings():
    L = _lib.lib()
    for code, name in _lib.STATUS_NAMES.items():
        assert L.q8_status_str(code).decode() == name


def test_workspace_sizes():
    L = _lib.lib()
    ws = lambda op, M, N, K: L.q8_workspace_bytes(op, M, N, K)  # noqa: E731
    # decode up to 10 tokens: the activation quantization is fused, no workspace
    for M in (1, 2, 4, 10):
        assert ws(_lib.Q8_OP_LINEAR, M, 4096, 4096) == 0
    # 11..16 tokens: codes, scales and code sums for the streaming GEMV
    for M in (11, 16):
        assert ws(_lib.Q8_OP_LINEAR, M, 4096, 4096) == M * 4096 + 2 * 256
    # GEMM path: codes + scale + row sum, each 256-byte aligned
    assert ws(_lib.Q8_OP_LINEAR, 2048, 14336, 4096) == 2048 * 4096 + 2 * 8192
    assert ws(_lib.Q8_OP_FP8, 4096, 4096, 14336) == 4096 * 14336 + 16384
    # decomposition: codes, scale, row sum, column flags, outlier list, count,
    # and the fp16 panels of the first 16 outlier columns of X and W
    d = ws(_lib.Q8_OP_DECOMP, 512, 4096, 4096)
    assert d == 512 * 4096 + 2048 + 2048 + 4096 + 4096 * 4 + 256 + 512 * 32 + 4096 * 32
    # static path: codes, per-row scale copy and code sums at every M
    assert ws(_lib.Q8_OP_STATIC, 1, 4096, 4096) == 4096 + 2 * 256
    assert ws(_lib.Q8_OP_STATIC, 2048, 14336, 4096) == 2048 * 4096 + 2 * 8192
    # per-group path: codes, scales and group code sums sized for groups of 64
    assert ws(_lib.Q8_OP_GROUPED, 10, 4096, 4096) == 0        # fused decode
    assert ws(_lib.Q8_OP_GROUPED, 11, 4096, 4096) == 11 * 4096 + 256 + 11 * 64 * 4
    assert ws(_lib.Q8_OP_GROUPED, 2048, 14336, 4096) == 2048 * 4096 + 8192 + 2048 * 64 * 4
    # an empty batch needs no workspace on any path
    for op in (_lib.Q8_OP_LINEAR, _lib.Q8_OP_DECOMP, _lib.Q8_OP_FP8, _lib.Q8_OP_STATIC, _lib.Q8_OP_GROUPED):
        assert ws(op, 0, 4096, 4096) == 0
    # invalid shapes give 0
    assert ws(_lib.Q8_OP_LINEAR, -1, 16, 16) == 0
    assert ws(_lib.Q8_OP_LINEAR, 16, 16, 24) == 0
    assert ws(_lib.Q8_OP_DECOMP, 16, 0, 16) == 0


def test_quantize_weight_validation():
    L = _lib.lib()
    f = L.q8_quantize_weight
    E = _lib
    assert f(E.Q8_INT8_SYM, P, E.Q8_F32, 4, 16, P, P, P, None) == 4        # BAD_FORMAT
    assert f(E.Q8_INT8_ASYM, P, 7, 4, 16, P, P, P, None) == 3              # BAD_DTYPE
    assert f(E.Q8_INT8_ASYM, P, E.Q8_F32, 0, 16, P, P, P, None) == 2       # BAD_SHAPE
    assert f(E.Q8_INT8_ASYM, P, E.Q8_F32, 4, 24, P, P, P, None) == 2       # K % 16
    assert f(E.Q8_INT8_ASYM, P, E.Q8_F32, 4, 65536 + 16, P, P, P, None) == 2
    assert f(E.Q8_INT8_ASYM, None, E.Q8_F32, 4, 16, P, P, P, None) == 1    # NULL
    assert f(E.Q8_INT8_ASYM, P, E.Q8_F32, 4, 16, P, P, None, None) == 1    # zero-point required
    assert f(E.Q8_FP8_E4M3, P, E.Q8_F32, 4, 16, P, P, P, None) == 5        # zp must be NULL
    assert f(E.Q8_INT8_ASYM, MIS, E.Q8_F32, 4, 16, P, P, P, None) == 6     # ALIGN


def test_quantize_act_validation():
    f = _lib.lib().q8_quantize_act
    E = _lib
    assert f(E.Q8_INT8_ASYM, P, E.Q8_BF16, 4, 16, INF, P, P, P, None) == 4
    assert f(E.Q8_INT8_SYM, P, 9, 4, 16, INF, P, P, P, None) == 3
    assert f(E.Q8_INT8_SYM, P, E.Q8_BF16, -1, 16, INF, P, P, P, None) == 2
    assert f(E.Q8_INT8_SYM, P, E.Q8_BF16, 4, 16, INF, None, P, P, None) == 1
    assert f(E.Q8_FP8_E4M3, P, E.Q8_BF16, 4, 16, NAN, P, P, None, None) == 5
    assert f(E.Q8_FP8_E4M3, P, E.Q8_BF16, 4, 16, 0.0, P, P, None, None) == 5
    assert f(E.Q8_FP8_E4M3, P, E.Q8_BF16, 4, 16, -3.0, P, P, None, None) == 5
    assert f(E.Q8_FP8_E4M3, P, E.Q8_BF16, 4, 16, 1200.0, P, P, P, None) == 5   # no row sum for fp8
    assert f(E.Q8_INT8_SYM, P, E.Q8_BF16, 4, 16, INF, P, P, MIS, None) == 6


def test_linear_validation():
    f = _lib.lib().q8_linear
    E = _lib
    ok = dict(x=P, xd=E.Q8_BF16, M=64, K=64, wq=P, ws=P, wz=P, N=64, b=None, y=P, yd=E.Q8_BF16,
              w=P2, wb=1 << 20, acc=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["xd"], a["M"], a["K"], a["wq"], a["ws"], a["wz"], a["N"], a["b"], a["y"],
                 a["yd"], a["w"], a["wb"], a["acc"], None)

    assert call(xd=5) == 3
    assert call(yd=-1) == 3
    assert call(N=0) == 2
    assert call(K=100) == 2
    assert call(wz=None) == 1
    assert call(y=None) == 1
    assert call(w=None) == 7                   # workspace needed for M > 10
    assert call(wb=100) == 7
    assert call(b=MIS) == 6
    assert call(acc=MIS) == 6
    assert call(M=11, w=None, wb=0) == 7
    # decode up to 10 tokens needs no workspace: with none given, the next
    # check (alignment) decides
    assert call(M=10, w=None, wb=0, y=MIS) == 6


def test_decomp_and_fp8_validation():
    E = _lib
    f = _lib.lib().q8_linear_int8_decomp
    assert f(P, 64, 64, P, P, P, 64, NAN, None, P, P2, 1 << 24, None, None, None, None) == 5
    assert f(P, 64, 64, P, P, P, 64, 6.0, None, P, None, 0, None, None, None, None) == 7
    assert f(P, 64, 64, P, P, P, 64, 6.0, None, P, P2, 1 << 24, MIS, None, None, None) == 6
    assert f(P, 64, 40, P, P, P, 64, 6.0, None, P, P2, 1 << 24, None, None, None, None) == 2
    g = _lib.lib().q8_linear_fp8
    assert g(P, 64, 64, P, P, 64, NAN, None, P, P2, 1 << 24, None) == 5
    assert g(P, 64, 64, P, P, 64, 1200.0, None, P, P2, 10, None) == 7
    assert g(None, 64, 64, P, P, 64, 1200.0, None, P, P2, 1 << 24, None) == 1


def test_empty_batch_validation():
    """M = 0 (an empty batch) is a valid shape: the pointers to M-sized
    arrays may be NULL, and every other argument is still checked (each call
    here fails before the device check, so no GPU work can start)."""
    L = _lib.lib()
    E = _lib
    lin = L.q8_linear
    # wq still required / K % 16 / N >= 1 / dtype / M < 0
    assert lin(None, E.Q8_BF16, 0, 64, None, P, P, 64, None, None, E.Q8_BF16, None, 0, None, None) == 1
    assert lin(None, E.Q8_BF16, 0, 40, P, P, P, 64, None, None, E.Q8_BF16, None, 0, None, None) == 2
    assert lin(None, E.Q8_BF16, 0, 64, P, P, P, 0, None, None, E.Q8_BF16, None, 0, None, None) == 2
    assert lin(None, 9, 0, 64, P, P, P, 64, None, None, E.Q8_BF16, None, 0, None, None) == 3
    assert lin(None, E.Q8_BF16, -1, 64, P, P, P, 64, None, None, E.Q8_BF16, None, 0, None, None) == 2
    # NaN threshold, misaligned bias, NaN scale bound: still rejected at M = 0
    assert L.q8_linear_int8_decomp(None, 0, 64, P, P, P, 64, NAN, None, None, None, 0, None, None, None,
                                   None) == 5
    assert L.q8_linear_int8_decomp(None, 0, 64, P, P, P, 64, 6.0, MIS, None, None, 0, None, None, None,
                                   None) == 6
    assert L.q8_linear_fp8(None, 0, 64, P, P, 64, NAN, None, None, None, 0, None) == 5
    assert L.q8_gemm_int8(None, None, None, 0, 64, None, P, P, 64, None, None, E.Q8_BF16, None, None) == 1
    assert L.q8_gemm_fp8(None, None, 0, 40, P, P, 64, None, None, None) == 2
    assert L.q8_quantize_act(E.Q8_FP8_E4M3, None, E.Q8_BF16, 0, 64, 0.0, None, None, None, None) == 5
    assert L.q8_quantize_act_static(None, E.Q8_BF16, 0, 64, 0.0, None, None, None) == 5
    assert L.q8_linear_static(None, E.Q8_BF16, 0, 64, 0.5, P, P, P, 64, None, NAN, None, None, 0, None) == 5
    assert L.q8_linear_w8a16(None, E.Q8_F32, 0, 64, P, P, P, 64, None, None, E.Q8_BF16, None) == 3
    assert L.q8_linear_grouped(None, E.Q8_BF16, 0, 64, P, P, P, 96, 64, None, None, E.Q8_BF16, None, 0,
                               None) == 2
    assert L.q8_linear_fp8_grouped(None, 0, 64, P, 0, P, P, 64, 1200.0, None, None, 0, None) == 2
    # weights have no empty case: N = 0 stays a shape error
    assert L.q8_quantize_weight(E.Q8_INT8_ASYM, P, E.Q8_F32, 0, 16, P, P, P, None) == 2


def test_valid_arguments_without_a_device_report_device_error():
    """With every argument valid, the call reaches the device check, which
    fails cleanly when there is no GPU (the CPU test host).  Never run where a
    GPU is visible: the fake pointers would then reach a kernel."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; the no-device path is checked on CPU hosts only")
    E = _lib
    st = _lib.lib().q8_quantize_weight(E.Q8_INT8_ASYM, P, E.Q8_F32, 4, 16, P, P, P, None)
    assert st == 8
    # an empty batch with NULL activations and outputs passes every argument check
    st = _lib.lib().q8_linear(None, E.Q8_BF16, 0, 64, P, P, P, 64, None, None, E.Q8_BF16, None, 0, None, None)
    assert st == 8


def test_w8a16_validation():
    f = _lib.lib().q8_linear_w8a16
    E = _lib
    ok = dict(x=P, xd=E.Q8_BF16, M=4, K=64, wq=P, ws=P, wz=P, N=64, b=None, y=P, yd=E.Q8_BF16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["xd"], a["M"], a["K"], a["wq"], a["ws"], a["wz"], a["N"], a["b"], a["y"], a["yd"], None)

    assert call(xd=E.Q8_F32) == 3            # 16-bit activations only
    assert call(yd=9) == 3
    assert call(M=17) == 2                    # decode sizes only
    assert call(K=40) == 2
    assert call(wz=None) == 1
    assert call(y=MIS) == 6


def test_static_validation():
    E = _lib
    q = _lib.lib().q8_quantize_act_static
    assert q(P, E.Q8_BF16, 4, 64, 0.0, P, P, None) == 5
    assert q(P, E.Q8_BF16, 4, 64, -1.0, P, P, None) == 5
    assert q(P, E.Q8_BF16, 4, 64, NAN, P, P, None) == 5
    assert q(P, E.Q8_BF16, 4, 64, INF, P, P, None) == 5
    assert q(P, 7, 4, 64, 0.1, P, P, None) == 3
    assert q(P, E.Q8_BF16, 4, 40, 0.1, P, P, None) == 2
    assert q(None, E.Q8_BF16, 4, 64, 0.1, P, P, None) == 1
    assert q(P, E.Q8_BF16, 4, 64, 0.1, MIS, P, None) == 6
    f = _lib.lib().q8_linear_static
    ok = dict(x=P, xd=E.Q8_BF16, M=64, K=64, sx=0.1, wq=P, ws=P, wz=P, N=64, b=None, sy=0.5, y=P, w=P2, wb=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["xd"], a["M"], a["K"], a["sx"], a["wq"], a["ws"], a["wz"], a["N"], a["b"], a["sy"],
                 a["y"], a["w"], a["wb"], None)

    assert call(sx=0.0) == 5
    assert call(sy=NAN) == 5
    assert call(sy=-2.0) == 5
    assert call(w=None) == 7
    assert call(M=1, wb=100) == 7            # the static path always needs its workspace
    assert call(y=MIS) == 6
    assert call(wz=None) == 1


def test_fp8_grouped_validation():
    f = _lib.lib().q8_linear_fp8_grouped
    ok = dict(x=P, T=64, K=64, off=P, E=4, wq=P, ws=P, N=64, ub=1200.0, y=P, w=P2, wb=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["T"], a["K"], a["off"], a["E"], a["wq"], a["ws"], a["N"], a["ub"], a["y"], a["w"],
                 a["wb"], None)

    assert call(E=0) == 2
    assert call(E=1025) == 2              # at most 1024 experts
    assert call(E=1024, N=16) != 2
    assert call(K=40) == 2
    assert call(off=None) == 1
    assert call(ub=NAN) == 5
    assert call(ub=0.0) == 5
    assert call(w=None) == 7
    assert call(y=MIS) == 6


def test_grouped_validation():
    E = _lib
    q = _lib.lib().q8_quantize_weight_grouped
    assert q(P, E.Q8_BF16, 64, 256, 32, P, P, P, None) == 2             # group 64 or 128 only
    assert q(P, E.Q8_BF16, 64, 192, 128, P, P, P, None) == 2            # K a multiple of the group
    assert q(P, 7, 64, 256, 128, P, P, P, None) == 3
    assert q(P, E.Q8_BF16, 64, 256, 128, P, P, None, None) == 1
    assert q(P, E.Q8_BF16, 64, 256, 128, P, MIS, P, None) == 6
    f = _lib.lib().q8_linear_grouped
    ok = dict(x=P, xd=E.Q8_BF16, M=64, K=256, wq=P, ws=P, wz=P, g=128, N=64, b=None, y=P, yd=E.Q8_BF16,
              w=P2, wb=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["xd"], a["M"], a["K"], a["wq"], a["ws"], a["wz"], a["g"], a["N"], a["b"], a["y"],
                 a["yd"], a["w"], a["wb"], None)

    assert call(g=96) == 2
    assert call(K=320) == 2                  # not a multiple of 128
    assert call(K=320, g=64, w=None) == 7    # a multiple of 64 passes the shape check
    assert call(xd=9) == 3
    assert call(wz=None) == 1
    assert call(w=None) == 7
    assert call(M=11, wb=100) == 7           # above the fused decode path the workspace is needed
    assert call(y=MIS) == 6
    assert call(ws=MIS) == 6


def test_bench_mfma_loop_validation():
    f = _lib.lib().q8_bench_mfma_loop
    E = _lib
    assert f(E.Q8_INT8_ASYM, 10, 8, P, None) == 4
    assert f(E.Q8_INT8_SYM, 0, 8, P, None) == 5
    assert f(E.Q8_INT8_SYM, 10, 0, P, None) == 5
    assert f(E.Q8_FP8_E4M3, 10, 65537, P, None) == 5
    assert f(E.Q8_INT8_SYM, 10, 8, None, None) == 1
    assert f(E.Q8_INT8_SYM, 10, 8, MIS, None) == 6


def test_bench_stream_read_validation():
    f = _lib.lib().q8_bench_stream_read
    assert f(P, 0, 8, P2, None) == 5
    assert f(P, 24, 8, P2, None) == 5
    assert f(P, 1 << 31, 8, P2, None) == 5
    assert f(P, 4096, 0, P2, None) == 5
    assert f(P, 4096, 65537, P2, None) == 5
    assert f(None, 4096, 8, P2, None) == 1
    assert f(MIS, 4096, 8, P2, None) == 6


def test_probe_fp8_mfma_validation():
    f = _lib.lib().q8_probe_fp8_mfma
    assert f(P, P, P, P2, 0, None) == 5
    assert f(P, P, P, P2, 65537, None) == 5
    assert f(None, P, P, P2, 1, None) == 1
    assert f(P, P, P, None, 1, None) == 1
    assert f(P, MIS, P, P2, 1, None) == 6


def test_gemm_tile_query():
    """The tile rule on the shapes the parity tests use for each tile (host
    only: nothing is launched)."""
    from w8a8_quantized_linear_channel_amd import ops
    assert ops.q8_gemm_tile("linear", 2000, 6100, 208) == (256, 256)
    assert ops.q8_gemm_tile("linear", 2048, 14336, 4096) == (256, 256)
    assert ops.q8_gemm_tile("linear", 1000, 3000, 208) == (128, 128)
    assert ops.q8_gemm_tile("linear", 500, 3000, 208) == (64, 128)
    assert ops.q8_gemm_tile("linear", 512, 4096, 4096) == (64, 128)
    assert ops.q8_gemm_tile("linear", 100, 500, 208) == (64, 64)
    assert ops.q8_gemm_tile("linear", 16, 4096, 4096) == (0, 0)          # the decode kernels
    assert ops.q8_gemm_tile("static", 17, 4096, 4096) == (64, 64)
    assert ops.q8_gemm_tile("decomp", 2000, 6100, 208) == (128, 128)     # no 256 x 256 there
    assert ops.q8_gemm_tile("decomp", 4, 64, 64) == (64, 64)
    assert ops.q8_gemm_tile("fp8", 4096, 4096, 14336) == (256, 256)
    assert ops.q8_gemm_tile("fp8", 1024, 4096, 4096) == (128, 128)
    assert ops.q8_gemm_tile("fp8", 0, 4096, 4096) == (0, 0)
    f = _lib.lib().q8_gemm_tile
    assert f(_lib.Q8_OP_GROUPED, 100, 100, 64, P, P2) == 5
    assert f(_lib.Q8_OP_LINEAR, 100, 100, 8, P, P2) == 2
    assert f(_lib.Q8_OP_LINEAR, 100, 100, 64, None, P2) == 1


def test_linear_noalloc_validation():
    """Argument errors and the scratch limit are reported before any HIP call
    (host only)."""
    f = _lib.lib().q8_linear_noalloc
    E = _lib
    ok = dict(x=P, xd=E.Q8_BF16, M=64, K=4096, wq=P, ws=P, wz=P, N=128, b=None, y=P2, yd=E.Q8_BF16, acc=None)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["x"], a["xd"], a["M"], a["K"], a["wq"], a["ws"], a["wz"], a["N"], a["b"], a["y"], a["yd"],
                 a["acc"], None)
    assert call(K=8) == 2
    assert call(xd=9) == 3
    assert call(wz=None) == 1
    assert call(y=MIS) == 6
    # scratch: M * K + 8 M + alignment must fit 32 MiB
    assert call(M=4096, K=8192) == 7
    assert call(M=8192, K=4096) == 7
    assert _lib.lib().q8_workspace_bytes(E.Q8_OP_LINEAR, 4096, 128, 8192) > 32 << 20
    assert _lib.lib().q8_workspace_bytes(E.Q8_OP_LINEAR, 4090, 128, 8192) <= 32 << 20


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without libq8.so every call raises (there is no CPU path)."""
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libq8.so"))
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()
