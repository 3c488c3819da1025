"""Pins of the oracle's numerics against mathematics and independent libraries.

* exp_spec against libm's fp64 exp (via numpy): error bound of the method.
* fixed-point softmax weights against an fp64 softmax.
* Philox4x64-10 against numpy.random.Philox (an independent implementation).
"""
import numpy as np
import pytest


def _ulp_err(y32, ref64):
    """|y - ref| in units of the fp32 spacing at ref."""
    ref32 = ref64.astype(np.float32)
    spacing = np.spacing(np.abs(ref32)).astype(np.float64)
    return np.abs(y32.astype(np.float64) - ref64) / spacing


def test_exp_spec_within_two_ulp_dense(orc):
    # every 97th fp32 value in [-32, 0]: ~1.1e7 points, all binades of the range
    lo = np.float32(-32.0).view(np.uint32)
    hi = np.float32(-0.0).view(np.uint32)
    bits = np.arange(hi, lo + 1, 97, dtype=np.uint32)
    x = bits.view(np.float32)
    y = orc.exp_spec(x)
    err = _ulp_err(y, np.exp(x.astype(np.float64)))
    assert err.max() <= 2.0, f"max ulp error {err.max()} at x={x[err.argmax()]}"


def test_exp_spec_boundaries(orc):
    assert orc.exp_spec(np.array([0.0], np.float32))[0] == 1.0
    assert orc.exp_spec(np.array([-0.0], np.float32))[0] == 1.0
    below = np.array([-32.000004, -40.0, -np.inf, np.nan], np.float32)
    assert np.all(orc.exp_spec(below) == 0.0)
    x = np.float32(-32.0)
    assert abs(orc.exp_spec(np.array([x]))[0] - np.exp(-32.0)) < 1e-20


def test_exp_spec_ln2_split(orc):
    hi, lo, log2e, c7 = orc.constants()
    # the high part of ln2 has its low 12 significand bits clear, so n * hi
    # is exact for every |n| < 2^12
    assert int(np.float32(hi).view(np.uint32)) & 0xFFF == 0
    assert abs((float(hi) + float(lo)) - np.log(2.0)) < 4e-12  # lo carries fp32 rounding
    assert float(log2e) == float(np.float32(1.0 / np.log(2.0)))
    assert float(c7) == float(np.float32(1.0 / 5040.0))


@pytest.mark.parametrize("temperature", [1.0, 0.5, 2.0])
def test_weights_are_softmax(orc, temperature):
    r = np.random.default_rng(1)
    row = (r.standard_normal(5000) * 3).astype(np.float32)
    W, Z = orc.row_weights(row, temperature)
    assert W.max() == 2 ** 44                     # the maximum maps to e^0 = 1
    assert int(W.sum(dtype=np.uint64)) == Z
    p = W.astype(np.float64) / Z
    x = row.astype(np.float64) / temperature
    ref = np.exp(x - x.max())
    ref /= ref.sum()
    # error budget of the fp32 path: l - m and * (1/T) each round once in fp32
    # (plus 1/T itself), exp_spec is within 2 ulp, W rounds to an integer.
    xs = np.abs(x - x.max())
    with np.errstate(divide="ignore"):
        per = 3 * 2.0 ** -24 * xs + 2.0 ** -22 + 0.5 / np.maximum(W.astype(np.float64), 1e-300)
    per_z = float((ref * per).sum())
    big = W > 0
    rel = np.abs(p[big] - ref[big]) / ref[big]
    assert np.all(rel <= per[big] + per_z + 1e-15), rel.max()
    # tokens whose weight rounds to zero have e^x * 2^44 < 1/2 (+ the error budget)
    assert np.all(ref[~big] * Z < 0.5 * (1 + 1e-5) * (1 + per_z) + 1e-9)


def test_weights_order_independent(orc):
    r = np.random.default_rng(2)
    row = (r.standard_normal(4096) * 3).astype(np.float32)
    W, Z = orc.row_weights(row)
    for _ in range(5):
        perm = r.permutation(row.shape[0])
        W2, Z2 = orc.row_weights(row[perm])
        assert Z2 == Z
        assert np.array_equal(W2, W[perm])
    # any chunking of the exact integer sum gives the same total
    for cs in (1, 7, 64, 1000):
        parts = [int(W[i:i + cs].sum(dtype=np.uint64)) for i in range(0, W.size, cs)]
        assert sum(parts) == Z


def test_weight_bounds(orc):
    assert orc.weight(5.0, 5.0) == 2 ** 44
    assert orc.weight(-100.0, 5.0) == 0
    # e^-31 * 2^44 = 0.6 -> 1 ; e^-31.5 * 2^44 = 0.37 -> 0
    assert orc.weight(-31.0, 0.0) == 1
    assert orc.weight(-31.5, 0.0) == 0


def _numpy_block(counter, key):
    """Philox4x64-10 block for `counter` from numpy, which advances its
    256-bit counter before producing each block of 4 outputs."""
    c = int(counter[0]) | (int(counter[1]) << 64) | (int(counter[2]) << 128) | (int(counter[3]) << 192)
    c = (c - 1) % (1 << 256)
    prev = np.array([(c >> (64 * i)) & ((1 << 64) - 1) for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=prev, key=np.asarray(key, dtype=np.uint64))
    return bg.random_raw(4)


@pytest.mark.parametrize("seed", range(6))
def test_philox_matches_numpy(orc, seed):
    r = np.random.default_rng(100 + seed)
    ctr = r.integers(0, 2 ** 63, size=4, dtype=np.uint64)
    if seed == 0:
        ctr[:] = 0
    if seed == 1:
        ctr = np.array([3, 1, 7, 0xFFFFFFFF], np.uint64)
    key = np.array([r.integers(0, 2 ** 63, dtype=np.uint64), 0], np.uint64)
    ours = orc.philox(ctr, key)
    assert np.array_equal(ours, _numpy_block(ctr, key))
