"""The FP8 matrix instruction's own summation, measured on the GPU.

The page's rowwise FP8 GEMM runs with fast accumulation ("Transformers FP8
(W8A8) 量化实战…" §5.3, use_fast_accum=True): the products of one instruction
are not summed exactly in fp32.  These tests run the FP8 GEMM's instruction
(v_mfma_f32_32x32x64_f8f6f4, through q8_probe_fp8_mfma) on crafted e4m3
operands whose exact sums are known, and pin the model of tests/fp8_accum.py
that the FP8 parity tolerance is derived from: groups of eight consecutive
products, each product cut toward zero 13 bits below its group's largest
exponent sum, the group sums and the accumulator input added with a few
binary32 roundings.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import q8_oracle as O
from w8a8_quantized_linear_channel_amd import ops as q8

import fp8_accum as F

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def enc(v):
    return int(O.e4m3_encode(np.array([v], np.float64))[0])


def run_probe(A, B, C):
    dev = torch.device("cuda:0")
    d = q8.q8_probe_fp8_mfma(torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                             torch.from_numpy(C).to(dev))
    return d.cpu().numpy().astype(np.float64)


def diagonal_cases(cases):
    """Each case (c, [(a, b), ...]) becomes the diagonal output (i, i) of
    problem p: row i of A and of B hold the case's factors, C[i, i] its
    accumulator input.  Returns A, B, C and the (p, i) of every case."""
    P = (len(cases) + 31) // 32
    A = np.zeros((P, 32, 64), np.uint8)
    B = np.zeros((P, 32, 64), np.uint8)
    C = np.zeros((P, 32, 32), np.float32)
    where = []
    for t, (c, prods) in enumerate(cases):
        p, i = divmod(t, 32)
        for k, (a, b) in (prods.items() if isinstance(prods, dict) else enumerate(prods)):
            A[p, i, k], B[p, i, k] = enc(a), enc(b)
            assert O.e4m3_decode(A[p, i, k]) == a and O.e4m3_decode(B[p, i, k]) == b
        C[p, i, i] = c
        where.append((p, i))
    return A, B, C, where


def test_fp8_mfma_groups_of_eight_consecutive_products():
    """A product of 2^16 at k_b and one of 60 at k_s: the 60 is cut to 56 (a
    multiple of 2^(16-13) = 8) exactly when k_b and k_s are in the same group
    of eight, for all 64 x 63 pairs."""
    pairs = [(kb, ks) for kb in range(64) for ks in range(64) if kb != ks]
    cases = [(0.0, {kb: (256.0, 256.0), ks: (60.0, 1.0)}) for kb, ks in pairs]
    A, B, C, where = diagonal_cases(cases)
    d = run_probe(A, B, C)
    for (kb, ks), (p, i) in zip(pairs, where):
        want = 65536.0 + (56.0 if kb // 8 == ks // 8 else 60.0)
        assert d[p, i, i] == want, (kb, ks, d[p, i, i])


def _pow2_split(t):
    """(x, y) with 1.875 2^x and 2^y both e4m3 values and x + y = t."""
    x = max(-6, min(7, t + 9))
    y = t - x
    if y > 8:
        x, y = t - 8, 8
    return x, y


def test_fp8_mfma_cut_toward_zero_below_the_largest_exponent_sum():
    """One group, C = 0: the largest factor pair sets E = e(a) + e(b) (the
    factors' exponents, not the product's: 240 x 448 = 1.64 2^16 has E = 15),
    a subnormal factor counts as e = -6, a zero product does not count, and a
    second product 1.875 2^t of either sign keeps its multiple of 2^(E - 13)
    toward zero."""
    bigs = [((256.0, 256.0), 16), ((240.0, 448.0), 15), ((2.0 ** -9, 448.0), 2), ((0.375, 2.0 ** -8), -10)]
    cases, meta = [], []
    for (big, E) in bigs:
        for t in range(max(E - 20, -15), min(E, 15) + 1):
            x, y = _pow2_split(t)
            for sign in (1.0, -1.0):
                prods = {0: big, 1: (sign * 1.875 * 2.0 ** x, 2.0 ** y)}
                cases.append((0.0, prods))
                meta.append(E)
                # a zero factor beside a large partner leaves the grid alone
                cases.append((0.0, {**prods, 5: (0.0, 448.0)}))
                meta.append(E)
    A, B, C, where = diagonal_cases(cases)
    d = run_probe(A, B, C)
    for (c, prods), E, (p, i) in zip(cases, meta, where):
        big = prods[0][0] * prods[0][1]
        small = prods[1][0] * prods[1][1]
        grid = 2.0 ** (E - 13)
        want = big + np.trunc(small / grid) * grid
        assert d[p, i, i] == want, (prods, d[p, i, i], want)


def test_fp8_mfma_accumulator_input_added_then_rounded_once():
    """C = 2^16 and a single product 1.875 2^(16-s): the sum is exact until it
    needs more than 24 bits, then rounded to nearest even (s = 21 is a tie)."""
    cases = []
    for s in range(1, 32):
        t = 16 - s
        x = max(-6, min(7, t + 9))
        y = t - x
        if y > 8:
            x, y = t - 8, 8
        for sign in (1.0, -1.0):
            cases.append((65536.0, [(sign * 1.875 * 2.0 ** x, 2.0 ** y)]))
    A, B, C, where = diagonal_cases(cases)
    d = run_probe(A, B, C)
    for (c, prods), (p, i) in zip(cases, where):
        from fractions import Fraction
        want = F.round_f32(Fraction(c) + Fraction(prods[0][0]) * Fraction(prods[0][1]))
        assert d[p, i, i] == want, (prods, d[p, i, i], want)


def _finite_codes(rng, shape, lo_e=0, hi_e=15):
    e = rng.integers(lo_e, hi_e + 1, shape)
    m = rng.integers(0, 8, shape)
    m = np.where(e == 15, np.minimum(m, 6), m)       # S.1111.111 is NaN
    s = rng.integers(0, 2, shape)
    return ((s << 7) | (e << 3) | m).astype(np.uint8)


def _operand_sets():
    rng = np.random.default_rng(2024)
    P = 4
    z = np.zeros((P, 32, 32), np.float32)
    sets = []
    sets.append(("random codes, C = 0", _finite_codes(rng, (P, 32, 64)), _finite_codes(rng, (P, 32, 64)), z))
    sets.append(("random codes, C ~ 1e3", _finite_codes(rng, (P, 32, 64), 3, 12),
                 _finite_codes(rng, (P, 32, 64), 3, 12), (rng.standard_normal((P, 32, 32)) * 1e3).astype(np.float32)))
    x = np.clip(rng.standard_normal((P, 32, 64)) * 100, -448, 448)
    w = np.clip(rng.standard_normal((P, 32, 64)) * 100, -448, 448)
    sets.append(("gaussian, C ~ 3e5", O.e4m3_encode(x), O.e4m3_encode(w),
                 (rng.standard_normal((P, 32, 32)) * 3e5).astype(np.float32)))
    # one 448 x 448 product per group, the rest small and of one sign
    A = _finite_codes(rng, (P, 32, 64)) & 0x7F
    B = _finite_codes(rng, (P, 32, 64)) & 0x7F
    A[:, :, ::8] = 0x7E
    B[:, :, ::8] = 0x7E
    sets.append(("one large product per group", A, B, z))
    # large products cancelling inside a group, small ones beside them
    A = _finite_codes(rng, (P, 32, 64), 0, 8)
    B = _finite_codes(rng, (P, 32, 64), 0, 8)
    A[:, :, 0::8], A[:, :, 1::8] = 0x7E, 0xFE
    B[:, :, 0::8], B[:, :, 1::8] = 0x7E, 0x7E
    sets.append(("cancelling large products", A, B, z))
    return sets


@pytest.mark.parametrize("k", range(5))
def test_fp8_mfma_error_within_the_model_bound(k):
    """Random and adversarial operands with random accumulator inputs: every
    output of the instruction is within the model's bound of the exact sum
    (the cuts, plus 2^-20 (|C| + sum |a b|) for the combination of the group
    sums).  Logged: the largest error as a fraction of |C| + sum |a b|, and as
    a fraction of the bound."""
    name, A, B, C = _operand_sets()[k]
    d = run_probe(A, B, C)
    av, bv = O.e4m3_decode(A), O.e4m3_decode(B)
    prod = np.einsum("pik,pjk->pijk", av, bv)
    exact = C.astype(np.float64) + prod.sum(-1)        # exact: <= 53 significant bits here
    err = np.abs(d - exact)
    mag = np.abs(C).astype(np.float64) + np.abs(prod).sum(-1)
    bound = F.instruction_bound(av, bv, C)
    assert np.all(err <= bound), (name, float(np.max(err / np.maximum(bound, 1e-300))))
    log(f"  {name}: max error / (|C| + sum|ab|) = {np.max(err / np.maximum(mag, 1e-300)):.3e}, "
        f"max error / bound = {np.max(np.where(bound > 0, err / np.maximum(bound, 1e-300), 0)):.3f}")
