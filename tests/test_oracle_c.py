"""Pin: the C form of the oracle's reduce statistics and bf16 norm tree
equals the numpy definition (and Python big integers) bit for bit."""
import numpy as np
import pytest

import oracle
from oracle import fast


@pytest.mark.parametrize("n", [1, 3, 8, 64])
def test_c_stats_equal_numpy(n):
    rng = np.random.default_rng(100 + n)
    for scale in (1e-4, 1.0, 300.0):
        c = (rng.standard_normal((n, 40_001)) * scale).astype(np.float16).view(np.uint16)
        q, bad = fast.reduce_stats(c)
        acc = oracle.reduce_contributions(c)
        assert q == oracle.exact_sq_units(acc) and bad == oracle.nonfinite(acc)


def test_c_stats_nonfinite_and_extremes():
    c = np.zeros((64, 9), dtype=np.float16)
    c[:, 0] = 65504.0
    c[:, 1] = -65504.0
    c[:, 2] = 2.0**-24
    c[3, 3] = -0.0
    q, bad = fast.reduce_stats(c.view(np.uint16))
    assert not bad and q == 2 * (64 * 65504 * 2**24) ** 2 + 64**2
    for v in (np.inf, -np.inf, np.nan):
        d = c.copy()
        d[5, 7] = v
        q2, bad2 = fast.reduce_stats(d.view(np.uint16))
        assert bad2 and q2 == q  # the non-finite element adds nothing to Q


def test_c_stats_subnormal_conversion():
    # every fp16 bit pattern converts exactly (compare single-rank sums to numpy)
    allbits = np.arange(65536, dtype=np.uint16)
    finite = np.isfinite(allbits.view(np.float16))
    rows = allbits[finite][None, :].copy()
    q, bad = fast.reduce_stats(rows)
    acc = oracle.reduce_contributions(rows)
    assert not bad and q == oracle.exact_sq_units(acc)


@pytest.mark.parametrize("n", [1, 8, 64])
def test_c_bf16_tree_equals_numpy(n):
    rng = np.random.default_rng(200 + n)
    for cols in (1, 5, 4096, 40_001):
        x = (rng.standard_normal((n, cols)) * 10.0 ** rng.uniform(-20, 20, (n, cols)))
        c = oracle.f32_to_bf16(x.astype(np.float32))
        tree, bad = fast.reduce_tree_bf16(c)
        acc = oracle.reduce_contributions_bf16(c)
        assert tree == oracle.sq_tree(acc) and bad == oracle.nonfinite(acc)
        # padding further with zeros leaves the tree unchanged
        width = 1
        while width < cols:
            width *= 2
        assert fast.reduce_tree_bf16(c, width=4 * width)[0] == tree


def test_c_bf16_tree_chunks_compose():
    # the tree of aligned power-of-two chunks, then the tree of their roots,
    # is the tree of the whole (how the full-size tests use it)
    rng = np.random.default_rng(9)
    c = oracle.f32_to_bf16(rng.standard_normal((8, 10_000)).astype(np.float32))
    whole, _ = fast.reduce_tree_bf16(c)
    roots = [fast.reduce_tree_bf16(np.ascontiguousarray(c[:, i:i + 1024]))[0]
             for i in range(0, 10_000, 1024)]
    assert oracle.pairwise_sum_f64(np.array(roots)) == whole
    c[3, 777] = 0x7F80  # +inf
    assert fast.reduce_tree_bf16(c)[1]


# ---------------------------------------------------------------------------
# The element-wise rest of the step in C (unscale, Adam, 16-bit casts), used
# for whole-shard comparisons at full sizes: pinned bit for bit to the numpy
# definitions, and the casts to numpy's and torch's conversions.

def _fp16_boundaries() -> np.ndarray:
    """Every finite fp16 value, every midpoint between neighbours (exact in
    fp32) and the fp32 values one ulp either side of each midpoint, both signs,
    plus the overflow threshold and the underflow region."""
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2.0
    top = np.array([65504.0, 65519.0, 65520.0, 65521.0, 65536.0, 1e6, 2.0**-25, 2.0**-26,
                    3 * 2.0**-26, 2.0**-24, 1e-30, 1.2e-38])
    base = np.concatenate([h, mids, top]).astype(np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    down = np.nextafter(base, np.float32(0))
    x = np.concatenate([base, up, down])
    return np.concatenate([x, -x])


def test_c_cast_fp16_equals_numpy():
    x = _fp16_boundaries()
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2**32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    r = bits.view(np.float32)
    x = np.concatenate([x, r[np.isfinite(r)], np.array([np.inf, -np.inf], np.float32)])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(fast.cast16(x), want)
    nan = fast.cast16(np.array([np.nan, -np.nan], np.float32)).view(np.float16)
    assert np.isnan(nan).all() and np.signbit(nan[1]) and not np.signbit(nan[0])


def test_c_cast_bf16_equals_numpy_and_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    bits = rng.integers(0, 2**32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    # every tie (lower half exactly 0x8000) and its neighbours, for both parities
    ties = (rng.integers(0, 2**16, size=200_000, dtype=np.uint64).astype(np.uint32) << 16)
    bits = np.concatenate([bits, ties | 0x8000, ties | 0x7FFF, ties | 0x8001])
    x = bits.view(np.float32)
    got = fast.cast16(x, bf16=True)
    assert np.array_equal(got, oracle.f32_to_bf16(x))  # NaN included
    fin = np.isfinite(x)
    t = torch.from_numpy(x[fin]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[fin], t)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("n", [1, 8, 64])
def test_c_reduce_unscale_equals_numpy(n, bf16):
    rng = np.random.default_rng(300 + n + 7 * bf16)
    for scale, inv in ((1e-3 * 65536, 1.0 / (n * 65536.0)), (1.0, 1.0 / n), (300.0, 0.37)):
        x = (rng.standard_normal((n, 20_003)) * scale).astype(np.float32)
        x[0, :5] = [np.inf, -np.inf, np.nan, 65504.0, 2.0**-24]
        if bf16:
            c = oracle.f32_to_bf16(x)
            acc = oracle.reduce_contributions_bf16(c)
        else:
            with np.errstate(over="ignore"):
                c = x.astype(np.float16).view(np.uint16)
            acc = oracle.reduce_contributions(c)
        inv32 = np.float32(inv)
        want = oracle.unscale(acc, inv32)
        got = fast.reduce_unscale(c, inv32, bf16=bf16)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        # a prefix of the columns
        got = fast.reduce_unscale(c, inv32, count=777, bf16=bf16)
        assert np.array_equal(got.view(np.uint32), want[:777].view(np.uint32))


def _adam_inputs(rng, k):
    g = (rng.standard_normal(k) * 10.0 ** rng.uniform(-12, 2, k)).astype(np.float32)
    p = (rng.standard_normal(k) * 0.02).astype(np.float32)
    m = (rng.standard_normal(k) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(k) * 1e-7).astype(np.float32)
    # extremes: subnormal g, zeros, fp16-range parameters, large moments
    g[:8] = [0.0, -0.0, 1e-45, -3e-42, 2.0**-126, 65504.0, -1e-20, 1e10]
    p[8:16] = [0.0, -0.0, 65504.0, -65504.0, 65519.0, 65520.0, 6e-8, -3e-8]
    m[16:20] = [0.0, 1e30, -1e-30, 1e-40]
    v[20:24] = [0.0, 1e30, 1e-40, 3e-45]
    return g, p, m, v


@pytest.mark.parametrize("bf16", [False, True])
def test_c_adam_update_equals_numpy(bf16):
    rng = np.random.default_rng(41 + bf16)
    cfgs = [(1e-3, 0.9, 0.999, 1e-8, 0.0, 1), (3e-4, 0.9, 0.999, 1e-8, 0.1, 3),
            (1.5e-4, 0.9, 0.95, 1e-6, 0.01, 5), (1e-2, 0.5, 0.9, 1e-3, 0.3, 1000),
            (0.0, 0.0, 0.0, 0.0, 0.0, 1)]
    for lr, b1, b2, eps, wd, t in cfgs:
        sc = oracle.step_scalars(lr, b1, b2, eps, wd, t, 8, 65536.0)
        for coef in (np.float32(1.0), np.float32(0.0337), np.float32(1e-6)):
            g, p, m, v = _adam_inputs(rng, 50_001)
            with np.errstate(all="ignore"):
                wp, wm, wv, wh = oracle.adam_apply(g, p, m, v, sc, coef)
            wh = oracle.f32_to_bf16(wp) if bf16 else wh.view(np.uint16)
            cp, cm, cv = p.copy(), m.copy(), v.copy()
            slot = np.zeros(g.size, dtype=np.uint16)
            fast.adam_update(g, cp, cm, cv, slot, sc, coef, bf16=bf16)
            for got, want in ((cp, wp), (cm, wm), (cv, wv)):
                assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (lr, t, coef)
            fin = np.isfinite(wp)
            assert np.array_equal(slot[fin], wh[fin]), (lr, t, coef)


def test_c_count_unequal():
    rng = np.random.default_rng(8)
    a = rng.integers(0, 2**32, size=100_003, dtype=np.uint64).astype(np.uint32)
    b = a.copy()
    b[[0, 17, 100_002]] ^= 1
    assert fast.count_unequal(a, b) == 3 and fast.count_unequal(a, a) == 0
    h, k = a.astype(np.uint16), b.astype(np.uint16)
    assert fast.count_unequal(h, k) == 3
