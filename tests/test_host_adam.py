"""The offload form's host update (zero_host_adam_apply, plain host code, no
GPU): against the oracle's Adam bit for bit, at every vector width and
thread count, and its fp16 rounding against numpy's conversion."""
import numpy as np
import pytest

import oracle

abi = pytest.importorskip("zero_sharded_optimizer_rank_amd.abi")


def _lib_or_skip():
    try:
        abi.lib()
    except Exception as e:  # library not built
        pytest.skip(f"libzero_shard.so not loadable: {e}")


def _widths():
    import zero_sharded_optimizer_rank_amd.abi as a
    out = [0, 1]
    for wd in (8, 16):
        try:
            x = np.zeros(1, np.float32)
            h = np.zeros(1, np.uint16)
            a.zero_host_adam_apply(x, x.copy(), x.copy(), x.copy(), h, 1, _args(), 1.0, 1, wd)
            out.append(wd)
        except a.ZeroError:
            pass
    return out


def _args(lr=1e-3, wd=0.1, step=3, beta1=0.9, beta2=0.999, eps=1e-8):
    return abi.step_args(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=wd,
                         max_grad_norm=1.0, loss_scale=1.0, step=step)


def _oracle(g, p, m, v, lr, wd, step, coef, beta1=0.9, beta2=0.999, eps=1e-8):
    sc = oracle.step_scalars(lr, beta1, beta2, eps, wd, step, 1, 1.0)
    return oracle.adam_apply(g, p, m, v, sc, np.float32(coef))


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


@pytest.mark.parametrize("count", [1, 15, 16, 17, 63, 1000, 100_003])
@pytest.mark.parametrize("threads", [1, 3, 8])
def test_host_adam_matches_oracle(count, threads):
    _lib_or_skip()
    rng = np.random.default_rng(count * 7 + threads)
    g = (rng.standard_normal(count) * 10.0 ** rng.uniform(-12, 2, count)).astype(np.float32)
    g[::11] = 0.0
    p = (rng.standard_normal(count) * 0.02).astype(np.float32)
    m = (rng.standard_normal(count) * 1e-3).astype(np.float32)
    v = (rng.random(count) * 1e-6).astype(np.float32)
    v[::7] = 0.0
    for coef in (1.0, 0.0317):
        want = _oracle(g, p, m, v, 3e-4, 0.1, 5, coef)
        for width in _widths():
            pp, mm, vv = p.copy(), m.copy(), v.copy()
            h = np.zeros(count, np.uint16)
            abi.zero_host_adam_apply(g, pp, mm, vv, h, count, _args(lr=3e-4, step=5), coef,
                                     threads, width)
            for got, exp in zip((pp, mm, vv, h), want):
                assert np.array_equal(_bits(got), _bits(exp.view(got.dtype))), (width, coef)


@pytest.mark.parametrize("step", [38_000, 1_000_000])
def test_host_adam_late_step_bias_corrections(step):
    """At late steps both beta powers fall below 2^-54, where 1 - beta^t is
    exactly 1 in fp64: the host stops the power loop there, the oracle runs
    all t products, and the updates must still agree bit for bit."""
    _lib_or_skip()
    rng = np.random.default_rng(step)
    n = 257
    g = rng.standard_normal(n).astype(np.float32)
    p = rng.standard_normal(n).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    v = (rng.random(n) * 1e-3).astype(np.float32)
    want = _oracle(g, p, m, v, 3e-4, 0.1, step, 1.0)
    pp, mm, vv = p.copy(), m.copy(), v.copy()
    h = np.zeros(n, np.uint16)
    abi.zero_host_adam_apply(g, pp, mm, vv, h, n, _args(lr=3e-4, step=step), 1.0, 1, 1)
    for got, exp in zip((pp, mm, vv, h), want):
        assert np.array_equal(_bits(got), _bits(exp.view(got.dtype)))


def test_host_adam_subnormals_and_extremes():
    _lib_or_skip()
    g = np.array([1e-45, -1e-45, 1e-40, 3e38, -3e38, 0.0, -0.0, 2.0**-126, 1e-20, 65504.0],
                 np.float32)
    p = np.array([1e-45, 0.0, -0.0, 1.0, -1.0, 6e-8, -6e-8, 65519.0, 65520.0, 1e-5], np.float32)
    m = np.zeros_like(g)
    v = np.zeros_like(g)
    want = _oracle(g, p, m, v, 1e-3, 0.0, 1, 1.0)
    for width in _widths():
        pp, mm, vv = p.copy(), m.copy(), v.copy()
        h = np.zeros(g.size, np.uint16)
        abi.zero_host_adam_apply(g, pp, mm, vv, h, g.size, _args(wd=0.0, step=1), 1.0, 2, width)
        for got, exp in zip((pp, mm, vv, h), want):
            assert np.array_equal(_bits(got), _bits(exp.view(got.dtype))), width


def _fp32_sample():
    """fp32 patterns covering fp16's whole range densely: every pattern near
    the subnormal/normal boundary, near the overflow threshold and around 1,
    plus a stride over all finite values, both signs."""
    parts = [np.arange(0, 0x7F800000, 7919, dtype=np.uint64),
             np.arange(0x33000000 - 4096, 0x38800000 + 65536, 3, dtype=np.uint64),
             np.arange(0x477FE000 - 8192, 0x47800000 + 8192, dtype=np.uint64),
             np.arange(0x3F7FF000, 0x3F801000, dtype=np.uint64)]
    pos = np.concatenate(parts).astype(np.uint32)
    bits = np.concatenate([pos, pos | np.uint32(0x80000000)])
    return bits.view(np.float32)


def test_fp16_rounding_every_width_matches_numpy():
    """lr = 0 and wd = 0 leave the master unchanged (u = 0, decay = 1), so
    the slot holds fp16(master): checked against numpy's conversion on a
    dense sample of fp32 values, ties and subnormals included."""
    _lib_or_skip()
    x = _fp32_sample()
    want = x.astype(np.float16).view(np.uint16)
    z = np.zeros(x.size, np.float32)
    for width in _widths():
        p = x.copy()
        h = np.zeros(x.size, np.uint16)
        abi.zero_host_adam_apply(z, p, z.copy(), z.copy(), h, x.size, _args(lr=0.0, wd=0.0), 1.0,
                                 4, width)
        assert np.array_equal(p.view(np.uint32), x.view(np.uint32)), width
        bad = np.flatnonzero(h != want)
        assert bad.size == 0, (width, hex(int(x.view(np.uint32)[bad[0]])), hex(int(h[bad[0]])),
                               hex(int(want[bad[0]])))


def test_host_adam_argument_errors():
    _lib_or_skip()
    x = np.zeros(4, np.float32)
    h = np.zeros(4, np.uint16)
    for kw, code in ((dict(threads=0), abi.ZERO_EINVAL), (dict(threads=100000), abi.ZERO_EINVAL),
                     (dict(clip=0.0), abi.ZERO_EINVAL), (dict(clip=1.5), abi.ZERO_EINVAL),
                     (dict(width=3), abi.ZERO_EINVAL), (dict(count=-1), abi.ZERO_EINVAL)):
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_host_adam_apply(x, x.copy(), x.copy(), x.copy(), h, kw.get("count", 4),
                                     _args(), kw.get("clip", 1.0), kw.get("threads", 1),
                                     kw.get("width", 0))
        assert e.value.code == code
    with pytest.raises(abi.ZeroError):
        abi.zero_host_adam_apply(None, x, x, x, h, 4, _args(), 1.0, 1, 0)
    assert abi.zero_offload_staging_bytes(64) == 64 * 2 * 6
    assert abi.zero_offload_staging_bytes(65) == 0
