"""Oracle pins for the bf16 path: conversions against torch's bfloat16 (a
library routine), the pairwise tree against its recursive definition and
Higham's error bound for pairwise summation, and sharded == unsharded."""
import math
import random

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")


def test_bf16_to_f32_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = oracle.bf16_to_f32(bits)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(31)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 10.0 ** rng.uniform(-40, 38, 200_000),
        # exact ties (low 16 bits 0x8000) with even and odd kept parts
        (rng.integers(0, 2**31, 10_000, dtype=np.uint64).astype(np.uint32) & 0xFFFF0000 | 0x8000
         ).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895e38, 3.4e38, 1e-45, -1e-45], np.float32),
    ]).astype(np.float32)
    x = x[np.isfinite(x) | np.isinf(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(x), want)
    nan = oracle.f32_to_bf16(np.array([np.nan, -np.nan], np.float32))
    assert np.isnan(oracle.bf16_to_f32(nan)).all()


def _tree_recursive(x):
    n = 1
    while n < len(x):
        n *= 2
    x = list(x) + [0.0] * (n - len(x))

    def t(lo, hi):
        if hi - lo == 1:
            return x[lo]
        mid = (lo + hi) // 2
        return t(lo, mid) + t(mid, hi)
    return t(0, n)


def test_pairwise_tree_structure_and_bound():
    rnd = random.Random(5)
    rng = np.random.default_rng(6)
    for n in list(range(1, 40)) + [255, 256, 257, 1000]:
        x = np.abs(rng.standard_normal(n)) * 10.0 ** rng.uniform(-30, 30, n)
        t = oracle.pairwise_sum_f64(x)
        assert t == _tree_recursive(x.tolist())
        # Higham (2002) 4.2: |T - S| <= gamma_{ceil(log2 n)} sum |x_i|
        k = max(1, math.ceil(math.log2(n)))
        u = 2.0**-53
        assert abs(t - math.fsum(x)) <= (k * u / (1 - k * u)) * math.fsum(np.abs(x))
    # exact whenever every partial sum is an exactly representable integer
    ints = rng.integers(0, 2**40, 5000).astype(np.float64)
    assert oracle.pairwise_sum_f64(ints) == float(sum(int(v) for v in ints))
    assert oracle.pairwise_sum_f64(np.zeros(0)) == 0.0


def _bits(a):
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint16)


@pytest.mark.parametrize("max_norm", [0.0, 1.0])
def test_bf16_sharded_equals_unsharded(max_norm):
    from oracle import run as orun
    w = synth.TINY_BF16
    n, psi = w.world_size, w.psi
    p = orun.workload_plan(w)
    states = [list(orun.initial_state(w, p, r)) for r in range(n)]
    for st in states:
        st[3] = oracle.f32_to_bf16(st[0])
    up = synth.masters(w, 0, psi)
    um, uv = np.zeros(psi, np.float32), np.zeros(psi, np.float32)
    uh = oracle.f32_to_bf16(up)
    for step in range(1, 4):
        sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, step, n, 1.0)
        accs = [oracle.reduce_contributions_bf16(orun.shard_contrib(w, p, r, step, 1.0))
                for r in range(n)]
        trees = [oracle.sq_tree(a) for a in accs]
        owns = [(t * sc.inv64) * sc.inv64 for t in trees]
        coefs = []
        for r in range(n):
            other = 0.0
            for x in range(n):
                if x != r:
                    other += owns[x]
            fin = oracle.finalize_bf16(trees[r], False, sc.inv64, max_norm, other_sq=other)
            coefs.append(fin.coef)
            g = oracle.unscale(accs[r], sc.inv32)
            pp, mm, vv, _ = oracle.adam_apply(g, states[r][0], states[r][1], states[r][2], sc,
                                              fin.coef)
            states[r] = [pp, mm, vv, oracle.f32_to_bf16(pp)]
        full = np.stack([synth.contributions(w, step, q, 0, psi, 1.0) for q in range(n)])
        out = oracle.shard_step_bf16(full, up, um, uv, uh, sc, max_norm)
        up, um, uv, uh = out.p, out.m, out.v, out.h
        if max_norm == 0.0:
            for k, whole in enumerate((up, um, uv, uh)):
                cat = np.concatenate([states[r][k] for r in range(n)])[:psi]
                assert np.array_equal(_bits(cat), _bits(whole)), (step, k)
        else:
            # the tree over the whole vector and the per-rank trees round
            # differently; the coefficients agree to within a few fp32 ulp
            assert all(abs(float(c) - float(out.fin.coef)) <= 4 * 2.0**-24 * float(c)
                       for c in coefs)
            assert out.fin.coef < 1


def test_bf16_reduce_rank_order():
    # 2^24 + 1 rounds back to 2^24 in fp32, so the rank order decides the sum
    c = oracle.f32_to_bf16(np.array([[2.0**24], [1.0], [-(2.0**24)]], np.float32))
    assert oracle.reduce_contributions_bf16(c)[0] == 0.0
    assert oracle.reduce_contributions_bf16(c[::-1].copy())[0] == 1.0
    # against torch's fp32 adds, in rank order, on random data
    rng = np.random.default_rng(12)
    x = oracle.f32_to_bf16((rng.standard_normal((7, 5000)) * 1e3).astype(np.float32))
    t = torch.zeros(5000, dtype=torch.float32)
    for r in range(7):
        t = t + torch.from_numpy(x[r].view(np.int16)).view(torch.bfloat16).float()
    assert np.array_equal(oracle.reduce_contributions_bf16(x).view(np.uint32),
                          t.numpy().view(np.uint32))


def test_sq_tree_exact_and_nonfinite():
    # integer-valued sums with small squares: the tree is the exact integer
    rng = np.random.default_rng(4)
    acc = rng.integers(-3000, 3000, 10_000).astype(np.float32)
    assert oracle.sq_tree(acc) == float(sum(int(a) ** 2 for a in acc))
    acc2 = acc.copy()
    acc2[17] = np.inf
    acc2[99] = np.nan
    want = float(sum(int(a) ** 2 for i, a in enumerate(acc) if i not in (17, 99)))
    assert oracle.sq_tree(acc2) == want
    assert oracle.nonfinite(acc2) and not oracle.nonfinite(acc)


def test_finalize_bf16_exact_case():
    from fractions import Fraction
    # N * scale a power of two: both multiplications by inv are exact
    acc = np.array([3.0, -4.0, 12.0], np.float32)  # sum of squares 169
    tree = oracle.sq_tree(acc)
    sc = oracle.step_scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 4, 2.0)
    fin = oracle.finalize_bf16(tree, False, sc.inv64, 0.5, other_sq=0.25)
    own = Fraction(169, 64)
    assert fin.own_sq == float(own) and fin.total_sq == float(own + Fraction(1, 4))
    assert fin.norm == math.sqrt(float(own + Fraction(1, 4)))
    assert fin.coef == np.float32(0.5 / (fin.norm + 1e-6)) and not fin.skip
    assert fin.own_q == 0
    # no clipping below the threshold, and max_norm 0 disables it
    assert oracle.finalize_bf16(tree, False, sc.inv64, 100.0).coef == 1.0
    assert oracle.finalize_bf16(tree, False, sc.inv64, 0.0).coef == 1.0
    # either overflow flag skips; only the own one is reported as overflow
    a = oracle.finalize_bf16(tree, True, sc.inv64, 0.5)
    b = oracle.finalize_bf16(tree, False, sc.inv64, 0.5, other_overflow=True)
    assert a.skip and a.overflow and b.skip and not b.overflow


def test_finalize_bf16_norm_against_fsum():
    # the norm of the averaged, unscaled gradient, within the pairwise bound
    rng = np.random.default_rng(8)
    c = oracle.f32_to_bf16((rng.standard_normal((8, 30_000)) * 0.37).astype(np.float32))
    acc = oracle.reduce_contributions_bf16(c)
    sc = oracle.step_scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 8, 3.0)  # inv not a power of two
    fin = oracle.finalize_bf16(oracle.sq_tree(acc), False, sc.inv64, 1.0)
    exact = math.fsum((float(a) / 24.0) ** 2 for a in acc)
    k = math.ceil(math.log2(acc.size))
    assert abs(fin.own_sq - exact) <= (k + 3) * 2.0**-53 * exact


def test_shard_step_bf16_slot_and_skip():
    rng = np.random.default_rng(2)
    s = 4099
    c = oracle.f32_to_bf16((rng.standard_normal((4, s)) * 1e-2).astype(np.float32))
    p = (rng.standard_normal(s) * 0.02).astype(np.float32)
    z = np.zeros(s, np.float32)
    h = oracle.f32_to_bf16(p)
    sc = oracle.step_scalars(1e-3, 0.9, 0.999, 1e-8, 0.1, 1, 4, 1.0)
    out = oracle.shard_step_bf16(c, p, z, z.copy(), h, sc, 0.01)
    want = torch.from_numpy(out.p).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out.h, want) and not out.fin.skip and out.fin.coef < 1
    g = oracle.unscale(oracle.reduce_contributions_bf16(c), sc.inv32)
    pp, mm, vv, _ = oracle.adam_apply(g, p, z, z.copy(), sc, out.fin.coef)
    assert np.array_equal(out.p.view(np.uint32), pp.view(np.uint32))
    c2 = c.copy()
    c2[2, 100] = 0x7F80
    out2 = oracle.shard_step_bf16(c2, p, z, z.copy(), h, sc, 1.0)
    assert out2.fin.skip and out2.p is p and np.array_equal(out2.h, h)
