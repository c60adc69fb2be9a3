"""The fp16 prefill's operand splits (CPU): exact where they must be, and each
one needed under the 2e-3 x RMS bar of the attention parity tests."""
import numpy as np
import pytest

from gpu_cases import ATT_TOL
from prefill_split_budget import rtz_fp16, scale_split, single_rounding_errors


def _exact_in_fp16(x):
    x = np.asarray(x, dtype=np.float64)
    return np.array_equal(x.astype(np.float16).astype(np.float64), x)


def test_scale_split_exact_for_every_scale_of_fp16_range_values():
    """Every fp16 scale the writer produces for values within fp16's range
    (s <= 8188, the scale of a block whose largest |x| is 65504) and every
    code n - 8 in [-8, 7]: s_lo is an fp16 value of at most 3 significant
    bits, (n - 8) s_hi and (n - 8) s_lo are both fp16 values (the dequantised
    pieces the matrix products take), and they add up to (n - 8) s exactly."""
    bits = np.arange(0, 0x7000, dtype=np.uint16)  # 0 .. 8188 (0x6FFF), subnormals included
    s = bits.view(np.float16)
    sv = s.astype(np.float64)
    assert sv.max() == 8188.0
    hi, lo = scale_split(s)
    assert _exact_in_fp16(hi) and _exact_in_fp16(lo)
    assert np.all(lo >= 0) and np.all(lo < hi + (hi == 0))
    # at most 3 significant bits: lo is a multiple of its own leading power of two / 4
    nz = lo > 0
    lead = 2.0 ** np.floor(np.log2(lo[nz]))
    assert np.all(np.mod(lo[nz], lead / 4) == 0)
    codes = np.arange(-8, 8, dtype=np.float64)[:, None]
    assert _exact_in_fp16(codes * hi) and _exact_in_fp16(codes * lo)
    assert np.array_equal(codes * hi + codes * lo, codes * sv)


def test_weight_split_residual():
    """A weight e (fp32, P * 2^11 up to 2^15) as hi = rtz_fp16(e) and
    lo = rtz_fp16(e - hi): e - hi is exact in fp32, and hi + lo misses e by
    less than 2^-20 of e, or by less than fp16's subnormal step 2^-24 where lo
    is subnormal (e below ~2^-3: weights under 2^-14 of the row's running
    maximum, whose sum the row's total dwarfs)."""
    g = np.random.default_rng(7)
    e = (2.0 ** g.uniform(-14, 15, 200_000)).astype(np.float32).astype(np.float64)
    hi = rtz_fp16(e)
    d = e - hi
    assert np.array_equal(d.astype(np.float32).astype(np.float64), d)
    lo = rtz_fp16(d)
    assert np.all(np.abs(e - hi - lo) < np.maximum(2.0 ** -20 * e, 2.0 ** -24))
    assert np.all(np.abs(e - hi - lo)[e >= 0.25] < 2.0 ** -20 * e[e >= 0.25])
    # rounding toward zero: neither part overshoots
    assert np.all(hi <= e) and np.all(hi + lo <= e)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_one_fp16_rounding_breaks_the_bar(seed):
    """With the synthetic outlier columns (1% of channels x 8), a single
    fp16 rounding of the dequantised keys, of the dequantised values or of
    the weights (nearest even, the most favourable rounding) moves the
    output by more than the 2e-3 x RMS that the parity tests allow; none of
    the three splits can be dropped."""
    err = single_rounding_errors(seed=seed)
    print(f"seed {seed}: " + ", ".join(f"{k} {v:.2e}" for k, v in err.items()))
    for k, v in err.items():
        assert v > ATT_TOL, f"one fp16 rounding of {k}: {v:.2e} <= {ATT_TOL}"
