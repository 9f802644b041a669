"""The static-scale quantizer decides most codes from one product.

For a calibrated scale S the kernel takes t = RN(x * RN(1/S)) and, where t is
more than 2^-14 from every half-integer, codes x as clamp(rne(t), +-127); the
values next to a half-integer (and all values when RN(1/S) is not a normal
number) go through the binary32 division.  This checks that claim on the CPU,
where numpy's binary32 product and quotient round as the GPU's do: for
hundreds of scales and every finite bf16 and f16 value up to 256 in
magnitude, the product path's code equals the division's wherever the product
path is taken.
"""
import numpy as np


def _values():
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    bf = (bits << 16).astype(np.uint32).view(np.float32)
    f16 = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    v = np.concatenate([bf, f16])
    return v[np.isfinite(v) & (np.abs(v) <= 256.0)]


def _decide(x, s):
    s = np.float32(s)
    r = np.float32(1.0) / s
    with np.errstate(over="ignore", invalid="ignore"):
        t = x * r
        d = np.abs(t - np.rint(t)) - np.float32(0.5)
        near = np.abs(d) <= np.float32(2.0 ** -14)
        fast = np.clip(np.rint(np.clip(t, -127, 127)), -127, 127)
        exact = np.clip(np.rint(x / s), -127, 127)
    return fast, exact, near, np.isfinite(r) and r >= np.finfo(np.float32).tiny


def test_product_path_matches_division():
    x = _values()
    rng = np.random.default_rng(41)
    scales = list(np.exp(rng.uniform(np.log(1e-4), np.log(1e2), 600)).astype(np.float32))
    scales += [0.25, 0.5, 1.0, 2.0, 0.1, 1.0 / 3.0, 0.0371, 7.0, 1e-3, 1.5e-38, 3e-38]
    taken = 0
    for s in scales:
        fast, exact, near, r_normal = _decide(x, s)
        assert r_normal
        ok = ~near
        taken += int(ok.sum())
        bad = np.flatnonzero(fast[ok] != exact[ok])
        assert bad.size == 0, (s, x[ok][bad[:5]], fast[ok][bad[:5]], exact[ok][bad[:5]])
    # the division handles only a small share
    assert taken > 0.995 * len(scales) * x.size


def test_reciprocal_below_normal_range_takes_the_division():
    # S = 1e38: RN(1/S) is subnormal, so the kernel divides every value
    _, _, _, r_normal = _decide(_values(), np.float32(1e38))
    assert not r_normal
