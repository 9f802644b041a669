"""Seeded synthetic inputs for the W8A8 linear layer workloads.

This module only draws random numbers and casts them to the storage dtype
(torch's round-to-nearest-even cast).  It holds none of the method's
arithmetic: no scale, no code, no product.  Both the CPU oracle and the HIP
path consume exactly the tensors returned here, so they see the same bits.

All generation uses ``numpy.random.default_rng(seed)`` (PCG64).  Values are
drawn in float32 and cast at the end.  The workloads stand in for the
Llama-3-8B layer shapes the pages quantize (q_proj 4096x4096, FFN up
14336x4096); no model weights or datasets are used.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


def _cast(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype) if dtype != torch.float32 else t


def normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


@dataclass
class Workload:
    name: str
    x: torch.Tensor            # activations [M, K] in their input dtype (CPU)
    w: torch.Tensor            # float32 weights [N, K] (CPU), quantized by the path
    out_dtype: torch.dtype
    extra: dict


def tiny_linear(seed: int = 0, M: int = 16, K: int = 256, N: int = 256) -> Workload:
    """X fp32 [16,256] ~ N(0,1); W fp32 [256,256] ~ N(0,0.02); fp32 out."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (M, K))
    w = normal(rng, (N, K), 0.02)
    return Workload("tiny_w8a8_16x256x256", _cast(x, torch.float32),
                    _cast(w, torch.float32), torch.float32, {})


def decode_qproj(seed: int = 1, M: int = 16, K: int = 4096, N: int = 4096) -> Workload:
    """X bf16 [M,4096] ~ N(0,1) for decode M in 1..16; W [4096,4096] ~ N(0,0.02)."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (M, K))
    w = normal(rng, (N, K), 0.02)
    return Workload(f"decode_qproj_M{M}_N{N}_K{K}", _cast(x, torch.bfloat16),
                    _cast(w, torch.float32), torch.bfloat16, {})


def decode_weight_copy(copy: int, N: int = 4096, K: int = 4096) -> torch.Tensor:
    """Extra weight sets for cache-rotating decode timing (copy >= 1 -> seed 1000+copy)."""
    rng = np.random.default_rng(1000 + copy)
    return _cast(normal(rng, (N, K), 0.02), torch.float32)


def prefill_ffn_up(seed: int = 2, M: int = 2048, K: int = 4096, N: int = 14336) -> Workload:
    """X bf16 [2048,4096] ~ N(0,1); W [14336,4096] ~ N(0,0.02); bf16 out."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (M, K))
    w = normal(rng, (N, K), 0.02)
    return Workload(f"prefill_ffn_up_M{M}_N{N}_K{K}", _cast(x, torch.bfloat16),
                    _cast(w, torch.float32), torch.bfloat16, {})


def llm_int8_outliers(seed: int = 3, M: int = 512, K: int = 4096, N: int = 4096,
                      n_outlier_cols: int = 6) -> Workload:
    """X fp16 [512,4096]: a few fixed feature columns hold |x| ~ U[6,60] with a
    random sign, every other entry is N(0,1) clipped to [-3.5, 3.5];
    W [4096,4096] ~ N(0,0.02); fp16 out.

    Draw order: outlier column ids, base X, outlier magnitudes, outlier signs, W.
    """
    rng = np.random.default_rng(seed)
    cols = np.sort(rng.choice(K, n_outlier_cols, replace=False)) if n_outlier_cols else \
        np.zeros(0, dtype=np.int64)
    x = np.clip(normal(rng, (M, K)), np.float32(-3.5), np.float32(3.5))
    mag = rng.uniform(6.0, 60.0, (M, len(cols))).astype(np.float32)
    sign = np.where(rng.random((M, len(cols))) < 0.5, np.float32(-1), np.float32(1))
    x[:, cols] = mag * sign
    w = normal(rng, (N, K), 0.02)
    return Workload(f"llm_int8_decomp_M{M}_N{N}_K{K}", _cast(x, torch.float16),
                    _cast(w, torch.float32), torch.float16,
                    {"outlier_cols": cols.astype(np.int64)})


def fp8_rowwise(seed: int = 4, M: int = 4096, K: int = 14336, N: int = 4096,
                spike_frac: float = 0.001, spike: float = 20.0) -> Workload:
    """X bf16 [4096,14336] ~ N(0,1) with 0.1% of entries (chosen without
    replacement) multiplied by 20; W [4096,14336] ~ N(0,0.02); bf16 out.

    Draw order: X, W, spike positions.
    """
    rng = np.random.default_rng(seed)
    x = normal(rng, (M, K))
    w = normal(rng, (N, K), 0.02)
    n_spike = int(round(spike_frac * M * K))
    if n_spike:
        pos = rng.choice(M * K, n_spike, replace=False)
        x.reshape(-1)[pos] *= np.float32(spike)
    return Workload(f"fp8_rowwise_M{M}_N{N}_K{K}", _cast(x, torch.bfloat16),
                    _cast(w, torch.float32), torch.bfloat16, {"scale_ub": 1200.0})


def moe_fp8(seed: int = 5, T: int = 4096, E: int = 8, K: int = 4096, N: int = 4096,
            alpha: float = 1.0) -> Workload:
    """One FP8 expert projection of a mixture-of-experts layer on routed tokens:
    X bf16 [T,K] ~ N(0,1), already grouped by expert; W [E,N,K] ~ N(0,0.02),
    one matrix per expert; the token count of each expert is drawn from a
    multinomial over Dirichlet(alpha) expert probabilities (a top-1 routing
    stand-in), and extra["offsets"] are the cumulative counts [E+1].

    Draw order: expert probabilities, counts, X, W.
    """
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(E, alpha))
    counts = rng.multinomial(T, p)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = normal(rng, (T, K))
    w = normal(rng, (E, N, K), 0.02)
    return Workload(f"moe_fp8_T{T}_E{E}_N{N}_K{K}", _cast(x, torch.bfloat16), _cast(w, torch.float32),
                    torch.bfloat16, {"offsets": torch.from_numpy(offsets), "scale_ub": 1200.0})


def random_matrix(seed: int, shape, std: float = 1.0,
                  dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Generic N(0, std) matrix for ragged-shape parity cases."""
    rng = np.random.default_rng(seed)
    return _cast(normal(rng, shape, std), dtype)


def extreme_codes(seed: int = 11, M: int = 33, N: int = 64, K: int = 65536) -> Workload:
    """Largest accumulator magnitudes at the largest K: every activation row is
    a positive constant (all its int8 codes are +127); weight rows n % 3 == 0
    are a negative constant (codes -128, zero point 127), rows n % 3 == 1 a
    positive constant (codes 127, zero point -128), the rest N(0, 0.02).  The
    constants are multiples of 1/64 and 1/1024, exact in bf16 and fp32."""
    rng = np.random.default_rng(seed)
    x = np.repeat((0.5 + np.arange(M, dtype=np.float32) / 64)[:, None], K, axis=1)
    w = normal(rng, (N, K), 0.02)
    n = np.arange(N)
    mag = (0.25 + n.astype(np.float32) / 1024).astype(np.float32)
    w[n % 3 == 0] = -mag[n % 3 == 0][:, None]
    w[n % 3 == 1] = mag[n % 3 == 1][:, None]
    return Workload(f"extreme_codes_M{M}_N{N}_K{K}", _cast(x, torch.bfloat16), _cast(w, torch.float32),
                    torch.bfloat16, {})


def tiled_rows(seed: int = 12, B: int = 257, K: int = 65536):
    """A weight matrix of any height from a small seeded base: row n is
    base[n % B] * mult[n] with mult[n] = 1 + (n % 7) / 8 (exact), one float32
    product per element.  Returns (base float32 [B, K], a function giving the
    rows `rows` (an index tensor) on the device of `base`)."""
    base = random_matrix(seed, (B, K), 0.02, torch.float32)

    def rows_of(base_t: torch.Tensor, rows: torch.Tensor) -> torch.Tensor:
        mult = 1.0 + (rows % 7).to(torch.float32) / 8.0
        return base_t[rows % B] * mult[:, None]

    return base, rows_of
