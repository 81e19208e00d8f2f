"""Oracle pin: concatenating the N shard updates reproduces unsharded Adam on
the all-reduced gradient, bit for bit.

The pages state the identity all-reduce = reduce-scatter + all-gather ("10.6
ZeRO 与 FSDP", §10.6.1) and that ZeRO leaves the optimizer's mathematics
unchanged ("第13篇 · ZeRO", §3.1 and §3.6).  The unsharded side below is plain
data parallelism: reduce the whole flat gradient, one norm, one update.
"""
import dataclasses
import math
import struct

import numpy as np
import pytest

import oracle
import synth
from oracle import run

F32 = np.float32


def _unsharded(w, steps, max_norm):
    n, psi = w.world_size, w.psi
    p = synth.masters(w, 0, psi)
    m, v = np.zeros(psi, F32), np.zeros(psi, F32)
    h = p.astype(np.float16)
    scale, good, t = w.loss_scale0, 0, 0
    out = []
    for step in range(1, steps + 1):
        c = np.stack([synth.contributions(w, step, q, 0, psi, scale) for q in range(n)])
        sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, t + 1, n, scale)
        res = oracle.shard_step(c, p, m, v, h, sc, max_norm)
        p, m, v, h = res.p, res.m, res.v, res.h
        if not res.fin.skip:
            t += 1
        out.append((res.g, res.fin, p, m, v, h, scale))
        scale, good = oracle.scaler_update(scale, good, res.fin.skip)
    return out


def _bits(a):
    return a.view(np.uint32 if a.dtype == F32 else np.uint16)


@pytest.mark.parametrize("variant", ["config", "clipped", "skip"])
def test_sharded_equals_unsharded(variant):
    w = synth.TINY
    max_norm = w.max_grad_norm
    if variant == "clipped":
        max_norm = 1.0  # the global norm is about 5 here, so the clip is active
    if variant == "skip":
        w = dataclasses.replace(w, inject_step=2)
    sharded = run.run_all_ranks(w, max_norm=max_norm)
    flat = _unsharded(w, w.steps, max_norm)
    p = run.workload_plan(w)
    assert p.psi_padded - p.psi == 1
    for rec, (g, fin, pp, mm, vv, hh, scale) in zip(sharded, flat):
        assert rec.loss_scale == scale
        for r in range(w.world_size):
            f = rec.fin[r]
            assert f.skip == fin.skip and f.coef == fin.coef and f.total_sq == fin.total_sq
        if variant == "clipped":
            assert fin.coef < 1
        for name, whole in (("g", g), ("p", pp), ("m", mm), ("v", vv), ("h", hh)):
            if name == "g":
                parts = [rec.g[r] for r in range(w.world_size)]
            else:
                parts = [getattr(rec.after[r], name) for r in range(w.world_size)]
            cat = np.concatenate(parts)
            assert np.array_equal(_bits(cat[:p.psi]), _bits(whole)), (rec.step, name)
            # the padding element stays exactly +0
            assert not np.any(_bits(cat[p.psi:])), (rec.step, name)
    if variant == "skip":
        assert [r.fin[0].skip for r in sharded] == [False, True, False]
        assert [r.loss_scale for r in sharded] == [1024.0, 1024.0, 512.0]
        assert [r.t for r in sharded] == [1, 1, 2]


def _f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


def test_brute_force_scalar_reimplementation():
    # Element by element with Python scalars rounded to fp32 after every
    # operation (struct round trips), against the vectorised oracle.
    rng = np.random.default_rng(21)
    for n, s in ((1, 5), (3, 17), (5, 64)):
        c = (rng.standard_normal((n, s)) * 40).astype(np.float16)
        p0 = (rng.standard_normal(s) * 0.02).astype(F32)
        m0 = (rng.standard_normal(s) * 1e-3).astype(F32)
        v0 = np.abs(rng.standard_normal(s) * 1e-6).astype(F32)
        sc = oracle.step_scalars(2e-3, 0.9, 0.999, 1e-8, 0.05, 4, n, 256.0)
        res = oracle.shard_step(c, p0, m0, v0, p0.astype(np.float16), sc, 0.01)
        accs = []
        for j in range(s):
            a = 0.0
            for r in range(n):
                a = _f32(a + float(c[r, j]))
            accs.append(a)
        q = sum(int(abs(a) * 2**24) ** 2 for a in accs)
        total = ((float(q) * 2.0**-48) * sc.inv64) * sc.inv64
        coef = _f32(min(1.0, 0.01 / (math.sqrt(total) + 1e-6)))
        assert coef == float(res.fin.coef)
        for j in range(s):
            g = _f32(accs[j] * float(sc.inv32))
            gc = _f32(g * coef)
            m = _f32(_f32(float(sc.b1) * float(m0[j])) + _f32(float(sc.omb1) * gc))
            v = _f32(_f32(float(sc.b2) * float(v0[j])) + _f32(float(sc.omb2) * _f32(gc * gc)))
            den = _f32(_f32(_f32(math.sqrt(v)) / float(sc.sqrt_bc2)) + float(sc.eps))
            u = _f32(_f32(m / den) * float(sc.step_size))
            p = _f32(_f32(float(p0[j]) * float(sc.decay)) - u)
            assert (g, m, v, p) == (float(res.g[j]), float(res.m[j]), float(res.v[j]),
                                    float(res.p[j])), (n, s, j)
            assert np.float16(p) == res.h[j]
