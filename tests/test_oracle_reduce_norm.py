"""Oracle pins for the reduce side, the overflow check and the exact norm."""
import math
import random

import numpy as np
import pytest

import oracle

F16 = np.float16


def _rand_fp16(rng, shape, scale):
    x = (rng.standard_normal(shape) * scale).astype(F16)
    return x


def test_single_rank_is_plain_unscale():
    # N = 1: the reduced gradient is the contribution itself, divided by the
    # loss scale (power of two, so exact).
    rng = np.random.default_rng(1)
    c = _rand_fp16(rng, (1, 5000), 30.0)
    sc = oracle.step_scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 1, 1024.0)
    g = oracle.unscale(oracle.reduce_contributions(c), sc.inv32)
    assert np.array_equal(g.astype(np.float64), c[0].astype(np.float64) / 1024.0)


@pytest.mark.parametrize("n", [2, 4, 8, 64])
def test_identical_contributions_average_to_themselves(n):
    # All N ranks hold the same gradient: the average is that gradient
    # (power-of-two N; 11 + log2 N significant bits fit in fp32).
    rng = np.random.default_rng(n)
    c0 = _rand_fp16(rng, (3000,), 50.0)
    c = np.broadcast_to(c0, (n, c0.size)).copy()
    sc = oracle.step_scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, n, 512.0)
    g = oracle.unscale(oracle.reduce_contributions(c), sc.inv32)
    assert np.array_equal(g.astype(np.float64), c0.astype(np.float64) / 512.0)


def test_fixed_rank_order_is_observable():
    # 2048 + 2^-13 ties to 2048 in fp32; so order 0,1,2 gives 0 and order 0,2,1 gives 2^-13.
    c = np.array([[2048.0], [2.0**-13], [-2048.0]], dtype=F16)
    assert oracle.reduce_contributions(c)[0] == 0.0
    assert oracle.reduce_contributions(c[[0, 2, 1]])[0] == np.float32(2.0**-13)


def test_sum_matches_fp64_when_exact():
    # Small integers: every partial sum is exact in fp32, so the result is the true sum.
    rng = np.random.default_rng(3)
    c = rng.integers(-1000, 1000, size=(16, 4000)).astype(F16)
    acc = oracle.reduce_contributions(c)
    assert np.array_equal(acc.astype(np.float64), c.astype(np.float64).sum(axis=0))


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_nonfinite_detected(bad):
    rng = np.random.default_rng(4)
    c = _rand_fp16(rng, (4, 100), 1.0)
    assert not oracle.nonfinite(oracle.reduce_contributions(c))
    c[2, 57] = bad
    assert oracle.nonfinite(oracle.reduce_contributions(c))


def test_plus_and_minus_inf_cancel_to_nan():
    c = np.zeros((2, 3), dtype=F16)
    c[0, 1], c[1, 1] = np.inf, -np.inf
    acc = oracle.reduce_contributions(c)
    assert np.isnan(acc[1]) and oracle.nonfinite(acc)


def test_exact_sq_units_against_fsum_and_bigint():
    # fsum returns the correctly rounded sum of its (exact) fp64 squares, so
    # float(Q) * 2^-48 must equal it bit for bit; Python big integers give Q itself.
    rng = np.random.default_rng(5)
    for trial in range(20):
        n = int(rng.integers(1, 65))
        scale = float(10.0 ** rng.uniform(-6, 3))
        c = _rand_fp16(rng, (n, 3001), scale)
        acc = oracle.reduce_contributions(c)
        q = oracle.exact_sq_units(acc)
        a64 = acc.astype(np.float64)
        assert float(q) * 2.0**-48 == math.fsum(a64 * a64)
        if trial < 4:
            assert q == sum(int(x) ** 2 for x in (np.abs(a64) * 2.0**24).tolist())


def test_exact_sq_units_subnormals_and_extremes():
    c = np.array([[2.0**-24, -2.0**-24, 65504.0, -65504.0, 0.0]], dtype=F16)
    acc = oracle.reduce_contributions(np.repeat(c, 64, axis=0))
    q = oracle.exact_sq_units(acc)
    expect = 2 * (64 * 1) ** 2 + 2 * (64 * 65504 * 2**24) ** 2
    assert q == expect


def test_finalize_clip_and_skip_rules():
    inv = 1.0 / (8 * 65536.0)
    # no clipping: coef is exactly 1
    r = oracle.finalize(10**30, False, inv, 0.0)
    assert r.coef == np.float32(1.0) and not r.skip
    # clipping: coef = max / (norm + 1e-6) in fp64, then one fp32 rounding
    q = 123456789 * 2**60
    r = oracle.finalize(q, False, inv, 1.0, other_sq=900.0)
    total = ((float(q) * 2.0**-48) * inv) * inv + 900.0
    assert r.total_sq == total and r.norm == math.sqrt(total)
    assert r.coef == np.float32(1.0 / (math.sqrt(total) + 1e-6)) and r.coef < 1
    # own, other and accumulator overflow each force a skip
    assert oracle.finalize(0, True, inv, 1.0).skip
    assert oracle.finalize(0, False, inv, 1.0, other_overflow=True).skip
    assert oracle.finalize(2**127, False, inv, 1.0, other_q=2**127).skip
    assert not oracle.finalize(2**127, False, inv, 1.0, other_q=2**127 - 1).skip


def test_exact_other_q_matches_unsharded_norm():
    # Exact all-reduce of Q: every split of the elements gives the same total.
    rng = np.random.default_rng(6)
    c = _rand_fp16(rng, (4, 10000), 20.0)
    acc = oracle.reduce_contributions(c)
    inv = 1.0 / (4 * 1024.0)
    whole = oracle.finalize(oracle.exact_sq_units(acc), False, inv, 1.0)
    cuts = sorted(random.Random(1).sample(range(1, 10000), 3))
    parts = np.split(acc, cuts)
    qs = [oracle.exact_sq_units(p) for p in parts]
    for i in range(len(parts)):
        r = oracle.finalize(qs[i], False, inv, 1.0, other_q=sum(qs) - qs[i])
        assert r.total_sq == whole.total_sq and r.coef == whole.coef
