"""The cache write multiplies by 1/s instead of dividing by s when the scale s is a power of
two: a host check, over every bf16 input and every normal power-of-two scale, that the two
give the same binary32 value (overflow to infinity and subnormal results included), which is
why the write's bytes do not depend on the path.  IEEE binary32 arithmetic via numpy."""
import numpy as np


def test_multiply_by_exact_reciprocal_equals_division():
    x = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)   # every bf16 value as f32
    finite = np.isfinite(x)
    with np.errstate(over="ignore", under="ignore", invalid="ignore", divide="ignore"):
        for k in range(-126, 128):
            s = np.float32(2.0) ** np.float32(k)
            assert np.isfinite(s) and s > 0
            r = np.float32(1.0) / s
            assert r * s == np.float32(1.0), f"1/2^{k} is not exact"      # 2^-127 is subnormal
            q = x / s
            m = x * r
            same = (q.view(np.uint32) == m.view(np.uint32)) | (np.isnan(q) & np.isnan(m))
            assert same.all(), f"scale 2^{k}: {np.count_nonzero(~same)} inputs differ"
            assert np.array_equal(np.isnan(q), ~finite & np.isnan(x))


def test_non_power_of_two_scales_need_the_division():
    """For a scale that is not a power of two the reciprocal is rounded, and the product
    differs from the quotient on some bf16 inputs: the multiply is only taken for powers of
    two."""
    x = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    x = x[np.isfinite(x)]
    for s in (np.float32(3.0), np.float32(7.0), np.float32(0.0371), np.float32(36.5 / 448.0)):
        with np.errstate(over="ignore", under="ignore"):
            assert np.count_nonzero((x / s) != (x * (np.float32(1.0) / s))) > 0
