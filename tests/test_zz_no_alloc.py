"""q8_linear_noalloc (the allocation-free q8_linear) against q8_linear, through
the C ABI: same outputs and INT32 accumulators bit for bit, on calls in a row
whose sizes go down (the library's scratch array keeps the previous call's
contents), across the three dispatch regimes, and at the largest shape its
32 MiB scratch accepts."""
import sys

import pytest
import torch

from w8a8_quantized_linear_channel_amd import inputs
from w8a8_quantized_linear_channel_amd import ops as q8

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(M, N, K, seed, dt=torch.bfloat16, od=torch.bfloat16, bias=False):
    dev = torch.device("cuda:0")
    x = inputs.random_matrix(seed, (M, K), 1.0, dt).to(dev)
    w = inputs.random_matrix(seed + 1, (N, K), 0.02, torch.float32).to(dev)
    b = inputs.random_matrix(seed + 2, (N,), 0.3, torch.float32).to(dev) if bias else None
    wq, ws, wz = q8.q8_quantize_weight(w, "int8_asym")
    return x, wq, ws, wz, b, od


def _same(args, what):
    x, wq, ws, wz, b, od = args
    y0, a0 = q8.q8_linear(x, wq, ws, wz, bias=b, out_dtype=od, acc_out=True)
    y1, a1 = q8.q8_linear_noalloc(x, wq, ws, wz, bias=b, out_dtype=od, acc_out=True)
    torch.cuda.synchronize()
    assert torch.equal(a0, a1), f"{what}: INT32 accumulator differs"
    assert torch.equal(y0.view(torch.uint8), y1.view(torch.uint8)), f"{what}: output differs"
    log(f"  {what}: {tuple(y1.shape)} bit-identical to q8_linear")


def test_noalloc_calls_in_a_row_with_shrinking_sizes():
    log("[noalloc] 2048x1024x4096, then 300x520x1040, then 13 and 5 tokens")
    _same(_case(2048, 1024, 4096, 300), "GEMM 2048x1024x4096")
    _same(_case(300, 520, 1040, 310, bias=True, od=torch.float32), "GEMM 300x520x1040 (smaller, after)")
    _same(_case(13, 100, 4112, 320, dt=torch.float16), "decode on codes, 13 tokens")
    _same(_case(5, 100, 4112, 330), "fused decode, 5 tokens (no scratch)")


def test_noalloc_largest_scratch():
    log("[noalloc] 4090x256x8192: the scratch nearly full")
    _same(_case(4090, 256, 8192, 340), "GEMM 4090x256x8192")
    _same(_case(17, 64, 128, 350), "GEMM 17x64x128 (after)")
