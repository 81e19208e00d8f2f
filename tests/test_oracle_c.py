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
