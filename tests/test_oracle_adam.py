"""Oracle pins for the Adam/AdamW update, the clip and the fp16 cast.

Closed forms (Adam's first step; a constant gradient, where bias correction
makes every step the same), Kingma & Ba's step-size bound, and the library
routine torch.optim.AdamW (CPU, fp32) as an independent implementation.
"""
import math

import numpy as np
import pytest

import oracle

F32 = np.float32
ULP = 2.0**-24  # half an fp32 ulp relative, per rounding


def _state(rng, n, g_scale):
    g = (rng.standard_normal(n) * g_scale).astype(F32)
    p = (rng.standard_normal(n) * 0.02).astype(F32)
    return g, p, np.zeros(n, F32), np.zeros(n, F32)


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_first_step_closed_form(wd):
    # t = 1 from m = v = 0: m_hat = g, sqrt(v_hat) = |g|, so
    # p1 = p0 (1 - lr wd) - lr g / (|g| + eps).
    rng = np.random.default_rng(11)
    lr, eps = 1e-3, 1e-8
    g, p, m, v = _state(rng, 20000, 1e-3)
    g[:50] *= 1e-6  # |g| near eps as well
    sc = oracle.step_scalars(lr, 0.9, 0.999, eps, wd, 1, 1, 1.0)
    p1, m1, v1, h = oracle.adam_apply(g, p, m, v, sc, F32(1.0))
    g64, p64 = g.astype(np.float64), p.astype(np.float64)
    u = lr * g64 / (np.abs(g64) + eps)
    expect = p64 * (1 - lr * wd) - u
    tol = 16 * ULP * (np.abs(p64) + np.abs(u))
    assert (np.abs(p1 - expect) <= tol).all()
    assert np.allclose(m1, 0.1 * g64, rtol=4 * ULP, atol=0)
    assert np.allclose(v1, 0.001 * g64 * g64, rtol=8 * ULP, atol=0)
    assert np.array_equal(h, p1.astype(np.float16))


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_constant_gradient_closed_form(wd):
    # Constant g: m_t = (1 - b1^t) g and v_t = (1 - b2^t) g^2, so the
    # bias-corrected step is lr g / (|g| + eps) at every t, and
    # p_T = p0 d^T - u (1 - d^T) / (1 - d) with d = 1 - lr wd.
    rng = np.random.default_rng(12)
    lr, b1, b2, eps, T = 1e-2, 0.9, 0.999, 1e-8, 12
    g, p, m, v = _state(rng, 5000, 1e-2)
    p0 = p.astype(np.float64)
    for t in range(1, T + 1):
        sc = oracle.step_scalars(lr, b1, b2, eps, wd, t, 1, 1.0)
        p, m, v, _ = oracle.adam_apply(g, p, m, v, sc, F32(1.0))
        g64 = g.astype(np.float64)
        assert np.allclose(m, (1 - b1**t) * g64, rtol=8 * t * ULP, atol=0)
        assert np.allclose(v, (1 - b2**t) * g64 * g64, rtol=8 * t * ULP, atol=0)
    g64 = g.astype(np.float64)
    u = lr * g64 / (np.abs(g64) + eps)
    d = 1 - lr * wd
    expect = p0 * d**T - (u * T if wd == 0 else u * (1 - d**T) / (1 - d))
    tol = 64 * T * ULP * (np.abs(p0) + np.abs(u) * T)
    assert (np.abs(p - expect) <= tol).all()


def test_step_bound():
    # Kingma & Ba (2015) section 2.1: |step| <= lr (1 - b1) / sqrt(1 - b2)
    # when 1 - b1 > sqrt(1 - b2).  Gradients change sign and scale wildly.
    rng = np.random.default_rng(13)
    lr, b1, b2 = 1e-3, 0.9, 0.999
    n = 4000
    p = np.zeros(n, F32)
    m, v = np.zeros(n, F32), np.zeros(n, F32)
    bound = lr * (1 - b1) / math.sqrt(1 - b2) * (1 + 1e-5)
    for t in range(1, 40):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 2, n)).astype(F32)
        sc = oracle.step_scalars(lr, b1, b2, 1e-8, 0.0, t, 1, 1.0)
        p2, m, v, _ = oracle.adam_apply(g, p, m, v, sc, F32(1.0))
        assert (np.abs(p2.astype(np.float64) - p) <= bound).all()
        assert (v >= 0).all()
        p = p2


def test_matches_torch_adamw():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(14)
    n, lr, wd, betas, eps = 30000, 3e-4, 0.1, (0.9, 0.999), 1e-8
    p0 = (rng.standard_normal(n) * 0.02).astype(F32)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=lr, betas=betas, eps=eps, weight_decay=wd,
                            foreach=False, fused=False)
    p, m, v = p0.copy(), np.zeros(n, F32), np.zeros(n, F32)
    for t in range(1, 7):
        g = (rng.standard_normal(n) * 1e-3).astype(F32)
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        sc = oracle.step_scalars(lr, betas[0], betas[1], eps, wd, t, 1, 1.0)
        p, m, v, _ = oracle.adam_apply(g, p, m, v, sc, F32(1.0))
        st = opt.state[tp]
        tm, tv, tpp = st["exp_avg"].numpy(), st["exp_avg_sq"].numpy(), tp.detach().numpy()
        # torch rounds lerp / addcdiv differently; agree to a few ulps of each term's scale
        assert np.allclose(m, tm, rtol=0, atol=16 * ULP * 1e-3)
        assert np.allclose(v, tv, rtol=32 * ULP, atol=1e-30)
        assert np.allclose(p, tpp, rtol=0, atol=32 * ULP * (0.1 + lr * 4))


def test_clip_coefficient_bounds_the_global_norm():
    # With c < 1, || c g || over all ranks <= max_norm.
    rng = np.random.default_rng(15)
    n_ranks, s = 4, 5000
    c = (rng.standard_normal((n_ranks, n_ranks * s)) * 20).astype(np.float16)
    sc = oracle.step_scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, n_ranks, 64.0)
    qs, gs = [], []
    for r in range(n_ranks):
        acc = oracle.reduce_contributions(c[:, r * s:(r + 1) * s])
        qs.append(oracle.exact_sq_units(acc))
        gs.append(oracle.unscale(acc, sc.inv32))
    g = np.concatenate(gs).astype(np.float64)
    norm = math.sqrt(math.fsum(g * g))
    max_norm = norm / 3
    r = oracle.finalize(qs[0], False, sc.inv64, max_norm, other_q=sum(qs[1:]))
    assert abs(r.norm - norm) <= 1e-15 * norm
    gc = (np.concatenate(gs) * r.coef).astype(np.float64)
    clipped = math.sqrt(math.fsum(gc * gc))
    assert clipped <= max_norm * (1 + 1e-6) and clipped >= max_norm * (1 - 1e-5)


def test_padding_stays_zero():
    sc = oracle.step_scalars(1e-3, 0.9, 0.999, 1e-8, 0.1, 3, 4, 1024.0)
    z = np.zeros(8, F32)
    p, m, v, h = oracle.adam_apply(z, z, z, z, sc, F32(0.5))
    for a in (p, m, v, h):
        assert not np.any(a) and not np.signbit(a).any()


def test_skip_leaves_state_and_slot():
    rng = np.random.default_rng(16)
    c = (rng.standard_normal((4, 100)) * 10).astype(np.float16)
    c[1, 7] = np.inf
    p = (rng.standard_normal(100) * 0.02).astype(F32)
    m, v = (p * 0.1).astype(F32), (p * p).astype(F32)
    h = p.astype(np.float16)
    sc = oracle.step_scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 4, 1024.0)
    out = oracle.shard_step(c, p, m, v, h, sc, 1.0)
    assert out.fin.skip
    assert out.p is p and out.m is m and out.v is v and out.h is h
    # the scaler halves on a skip and never drops below its floor
    assert oracle.scaler_update(65536.0, 5, True) == (32768.0, 0)
    assert oracle.scaler_update(1.0, 5, True) == (1.0, 0)
    assert oracle.scaler_update(65536.0, 998, False) == (65536.0, 999)
    assert oracle.scaler_update(65536.0, 999, False) == (131072.0, 0)
