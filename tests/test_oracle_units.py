"""Oracle pins for the FSDP / ZeRO-3 unit layout: planner brute force, and
per-unit sharded updates concatenated back into model order equal unsharded
Adam on the all-reduced gradient bit for bit ("10.6 ZeRO 与 FSDP", §10.6.1:
all-reduce = reduce-scatter + all-gather; §10.6.4 and §10.6.7: the unit is
the sharding grain)."""
import random

import numpy as np

import oracle
import synth
from oracle import run as orun


def test_unit_planner_brute_force():
    rnd = random.Random(11)
    for _ in range(300):
        t = rnd.randint(0, 7)
        numels = [rnd.randint(0, 30) for _ in range(t)]
        units, u = [], 0
        for i in range(t):
            if i > 0 and rnd.random() < 0.4:
                u += 1
            units.append(u)
        n = rnd.randint(1, 9)
        align = rnd.choice([1, 2, 8])
        up = oracle.plan_units(numels, units, n, align)
        psi = sum(numels)
        assert up.psi == psi and up.rank_shard == sum(up.unit_shard)
        owner = {}
        for r in range(n):
            idx = oracle.unit_shard_index(up, r)
            assert idx.size == up.rank_shard
            for k, e in enumerate(idx.tolist()):
                if e >= 0:
                    assert e not in owner
                    owner[e] = (r, k)
        assert sorted(owner) == list(range(psi))  # every element owned exactly once
        for s, p in zip(up.unit_shard, up.unit_psi):
            assert s % align == 0 and s * n >= p and (s - align) * n < p or s == 0


def test_unit_layout_is_flat_layout_for_one_unit():
    w = synth.TINY
    up = oracle.plan_units(w.numels, (0, 0, 0), 4)
    p = oracle.plan(w.numels, 4)
    for r in range(4):
        idx = oracle.unit_shard_index(up, r)
        flat = np.arange(r * p.shard, (r + 1) * p.shard)
        assert np.array_equal(idx, np.where(flat < p.psi, flat, -1))


def _bits(a):
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint16)


def test_unit_sharded_equals_unsharded():
    w = synth.TINY_FSDP
    n, psi = w.world_size, w.psi
    up = orun.workload_unit_plan(w)
    assert up.unit_shard == (250000, 250, 1)
    maps = [oracle.unit_shard_index(up, r) for r in range(n)]
    # sharded: every rank, exact all-reduce of Q, clip active
    states = [list(orun.unit_rank_initial_state(w, up, r)) for r in range(n)]
    p = synth.masters(w, 0, psi)
    m, v, h = np.zeros(psi, np.float32), np.zeros(psi, np.float32), p.astype(np.float16)
    scale = w.loss_scale0
    for step in range(1, 4):
        sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, step, n, scale)
        accs = [oracle.reduce_contributions(orun.unit_rank_contrib(w, up, r, step, scale))
                for r in range(n)]
        qs = [oracle.exact_sq_units(a) for a in accs]
        for r in range(n):
            fin = oracle.finalize(qs[r], False, sc.inv64, 1.0, other_q=sum(qs) - qs[r])
            g = oracle.unscale(accs[r], sc.inv32)
            st = states[r]
            st[0], st[1], st[2], st[3] = oracle.adam_apply(g, st[0], st[1], st[2], sc, fin.coef)
        full = np.stack([synth.contributions(w, step, q, 0, psi, scale) for q in range(n)])
        out = oracle.shard_step(full, p, m, v, h, sc, 1.0)
        p, m, v, h = out.p, out.m, out.v, out.h
        assert out.fin.coef < 1
        for k, whole in enumerate((p, m, v, h)):
            got = np.zeros_like(whole)
            for r in range(n):
                real = maps[r] >= 0
                got[maps[r][real]] = states[r][k][real]
                assert not np.any(_bits(states[r][k][~real]))  # padding stays +0
            assert np.array_equal(_bits(got), _bits(whole)), (step, k)


def test_unit_model_index_pointwise():
    w = synth.GPT2_FSDP
    up = orun.workload_unit_plan(w)
    rng = np.random.default_rng(3)
    small = oracle.plan_units([10, 3, 7, 1], [0, 0, 1, 2], 4)
    for r in range(4):
        full = oracle.unit_shard_index(small, r)
        assert np.array_equal(oracle.unit_model_index(small, r, np.arange(full.size)), full)
    pos = rng.integers(0, up.rank_shard, 1000)
    e = oracle.unit_model_index(up, 5, pos)
    assert (e >= 0).all() and (e < w.psi).all()


def test_unit_planner_rejects_bad_unit_numbering():
    import pytest as _pytest
    for units in ((0, 2), (1, 1), (0, 1, 0), (0, 0, 2)):
        with _pytest.raises(ValueError):
            oracle.plan_units([3] * len(units), units, 4)
    with _pytest.raises(ValueError):
        oracle.plan_units([3, -1], (0, 0), 4)
    with _pytest.raises(ValueError):
        oracle.plan_units([3, 4], (0,), 4)
    # the C planner refuses the same tables
    abi = _pytest.importorskip("zero_sharded_optimizer_rank_amd.abi")
    try:
        abi.lib()
    except Exception as e:
        _pytest.skip(f"libzero_shard.so not loadable: {e}")
    for units in ((0, 2), (1, 1), (0, 1, 0)):
        with _pytest.raises(abi.ZeroError) as err:
            abi.zero_plan_units([3] * len(units), units, 4)
        assert err.value.code == abi.ZERO_EINVAL
