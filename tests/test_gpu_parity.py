"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the
same seeded inputs.  Bar and reporting as described in parity_util."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from oracle import run as orun

from parity_util import check_result, compare_state, run_window, StepReport

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _abi():
    import zero_sharded_optimizer_rank_amd.abi as abi
    return abi


@pytest.mark.parametrize("variant", ["config", "clipped", "skip"])
def test_tiny_all_shards(variant):
    """All four shards of the tiny workload, three steps; the squared-norm
    integers and overflow flags of the other ranks are exchanged exactly on
    the host (the all-reduce) between zero_reduce_check and zero_adam_apply."""
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    abi = _abi()
    w = synth.TINY
    max_norm = 1.0 if variant == "clipped" else w.max_grad_norm
    if variant == "skip":
        w = dataclasses.replace(w, inject_step=2)
    print(f"[tiny_all_shards {variant}]", flush=True)
    records = orun.run_all_ranks(w, max_norm=max_norm)
    n = w.world_size
    devs = [DeviceShard(w, r) for r in range(n)]
    for d in devs:
        d.load_initial_state()
    scaler = abi.new_scaler(w.loss_scale0)
    for rec in records:
        assert rec.loss_scale == scaler.scale
        for d in devs:
            d.load_contributions(rec.step, scaler.scale)
        base = devs[0].args(scaler.t + 1, scaler.scale, max_norm=max_norm)
        for d in devs:
            d.reduce_check(base)
        rs = [d.result() for d in devs]
        for r, d in enumerate(devs):
            other_q = sum(rs[x].own_q for x in range(n) if x != r)
            other_ovf = any(rs[x].overflow for x in range(n) if x != r)
            a = d.args(scaler.t + 1, scaler.scale, max_norm=max_norm, other_q=other_q,
                       other_overflow=other_ovf)
            d.finalize(a)
            d.adam_apply(a)
        skipped = None
        for r, d in enumerate(devs):
            res = d.result()
            check_result(res, rec.fin[r], rec.step)
            skipped = bool(res.skip)
            g = d.fetch("grad")
            assert np.array_equal(g.view(np.uint32), rec.g[r].view(np.uint32))
            rep = StepReport(rec.step, skipped, float(res.clip_coef))
            st = rec.after[r]
            for name, want in (("master", st.p), ("m", st.m), ("v", st.v),
                               ("slot", st.h.view(np.uint16))):
                compare_state(rep, name, d.fetch(name), want)
            assert all(v == 0 for v in rep.mismatches.values()), (rec.step, r, rep.mismatches)
            assert d.guards_intact()
        if variant == "clipped":
            assert rec.fin[0].coef < 1
        abi.zero_scaler_update(scaler, skipped)
        assert scaler.t == rec.t
    # the padding element of the last shard stays exactly zero
    last = devs[-1]
    for name in ("master", "m", "v", "slot"):
        assert last.fetch(name)[-1] == 0


def _windows():
    cases = []
    count = (1 << 20) + 3  # several workgroups' worth, ragged tail
    for w in (synth.GPT2, synth.FLAT75, synth.LLAMA3_8B, synth.LLAMA2_70B):
        p = orun.workload_plan(w)
        for r in w.parity_ranks:
            if w.inject_step is not None and r == 0:
                e = synth.inject_site(w, w.inject_step)[1]
                begin = max(0, e - count // 2)
            elif r == w.parity_ranks[-1]:
                begin = p.shard - count  # end of the shard
            else:
                begin = 12345
            cases.append(pytest.param(w, r, begin, count, id=f"{w.name}-r{r}"))
    return cases


@pytest.mark.parametrize("w,rank,begin,count", _windows())
def test_window_parity(w, rank, begin, count):
    """Every step of each large workload on a ~1M-element window of the parity
    ranks' shards (same N, distributions, loss-scale schedule, clip stand-in)."""
    print(f"[window {w.name} rank {rank} begin {begin} count {count}]", flush=True)
    reps = run_window(w, rank, begin, count)
    if w.inject_step is not None:
        assert reps[w.inject_step - 1].skip
    if w.max_grad_norm > 0:
        assert any(r.coef < 1 for r in reps)


def test_phase_split_equals_fused():
    print("[phase split vs fused]", flush=True)
    w = synth.LLAMA3_8B
    a = run_window(w, 1, 777, 300_001, steps=3, fused=False)
    b = run_window(w, 1, 777, 300_001, steps=3, fused=True)
    assert [r.coef for r in a] == [r.coef for r in b]


def test_run_twice_bitwise():
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    print("[determinism]", flush=True)
    w = synth.GPT2
    outs = []
    for _ in range(2):
        d = DeviceShard(w, 1, 0, 2_000_003)
        d.load_initial_state()
        d.load_contributions(1, w.loss_scale0)
        d.step(d.args(1, w.loss_scale0))
        res = d.result()
        outs.append((res.own_q, res.norm, [d.fetch(x).tobytes() for x in
                                           ("grad", "master", "m", "v", "slot")]))
    assert outs[0] == outs[1]


def _inject_case(w, rank, begin, count, where, value):
    """One step with a non-finite contribution planted on the device and in
    the oracle's copy of the inputs."""
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    d = DeviceShard(w, rank, begin, count)
    d.load_initial_state()
    d.load_contributions(1, w.loss_scale0)
    q, j = where
    bits = np.array([value], dtype=np.float16).view(np.int16)[0]
    d.contrib[q, j] = int(bits)
    before = {x: d.fetch(x).copy() for x in ("master", "m", "v", "slot")}
    d.step(d.args(1, w.loss_scale0))
    res = d.result()
    p = orun.workload_plan(w)
    c = orun.shard_contrib(w, p, rank, 1, w.loss_scale0, begin, count)
    c[q, j] = np.array([value], dtype=np.float16).view(np.uint16)[0]
    acc = oracle.reduce_contributions(c)
    sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, 1, w.world_size,
                             w.loss_scale0)
    fin = oracle.finalize(oracle.exact_sq_units(acc), oracle.nonfinite(acc), sc.inv64,
                          w.max_grad_norm)
    check_result(res, fin, 1)
    g = d.fetch("grad")
    want = oracle.unscale(acc, sc.inv32)
    assert np.array_equal(g.view(np.uint32), want.view(np.uint32))
    assert res.skip
    for x, arr in before.items():
        assert np.array_equal(d.fetch(x), arr), x  # state and slot untouched
    assert d.guards_intact()


@pytest.mark.parametrize("value", [np.inf, -np.inf, np.nan])
@pytest.mark.parametrize("pos", ["first", "last", "tail"])
def test_nonfinite_skips(value, pos):
    print(f"[nonfinite {value} at {pos}]", flush=True)
    w = synth.TINY
    p = orun.workload_plan(w)
    rank = 3  # holds the padding element
    count = p.shard
    j = {"first": 0, "last": p.real(rank) - 1, "tail": count - 5}[pos]
    _inject_case(w, rank, 0, count, (2, j), value)


def test_other_overflow_forces_skip():
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    w = synth.TINY
    d = DeviceShard(w, 0, 0, 100_000)
    d.load_initial_state()
    d.load_contributions(1, w.loss_scale0)
    before = d.fetch("master").copy()
    d.step(d.args(1, w.loss_scale0, other_overflow=True))
    res = d.result()
    assert res.skip and not res.overflow
    assert np.array_equal(d.fetch("master"), before)


@pytest.mark.parametrize("n", [1, 3, 64])
def test_world_sizes(n):
    """N = 1, a non-power-of-two N and the maximum N, with extreme values."""
    print(f"[world size {n}]", flush=True)
    w = dataclasses.replace(synth.TINY, world_size=n, max_grad_norm=0.5, weight_decay=0.01)
    p = orun.workload_plan(w)
    count = min(p.shard, 200_003)
    run_window(w, n - 1, 0, count, steps=2)


def test_extreme_magnitudes():
    """Every contribution at +-65504 with N = 64: the largest sums the kernel sees."""
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    print("[extreme magnitudes]", flush=True)
    w = dataclasses.replace(synth.TINY, world_size=64)
    count = orun.workload_plan(w).shard
    d = DeviceShard(w, 0, 0, count)
    d.load_initial_state()
    c = np.full((64, d.ld), 65504.0, dtype=np.float16)
    c[:, ::2] = -65504.0
    c[5, 7] = 2.0**-24  # and one subnormal
    d.contrib.copy_(torch.from_numpy(c.view(np.int16)))
    d.step(d.args(1, 1.0))
    res = d.result()
    acc = oracle.reduce_contributions(c[:, :count])
    sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, 1, 64, 1.0)
    fin = oracle.finalize(oracle.exact_sq_units(acc), False, sc.inv64, w.max_grad_norm)
    check_result(res, fin, 1)
    g = d.fetch("grad")
    assert np.array_equal(g.view(np.uint32), oracle.unscale(acc, sc.inv32).view(np.uint32))


def test_empty_shard():
    abi = _abi()
    n = 4
    plan = abi.zero_plan_t(0, n, 1, 0, 0)
    ws = torch.zeros(abi.zero_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    res = torch.zeros(abi.RESULT_BYTES, dtype=torch.uint8, device="cuda")
    dummy = torch.zeros(16, dtype=torch.float32, device="cuda")
    args = abi.step_args(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                         max_grad_norm=1.0, loss_scale=1.0, step=1)
    abi.zero_reduce_adam_step(plan, 0, [dummy] * n, dummy, dummy, dummy, dummy, dummy, ws,
                              ws.numel(), args, res)
    torch.cuda.synchronize()
    r = abi.zero_step_result_t.from_buffer_copy(res.cpu().numpy().tobytes())
    assert r.own_q == 0 and r.norm == 0.0 and r.clip_coef == 1.0 and not r.skip


def test_argument_errors():
    abi = _abi()
    plan, _ = abi.zero_plan([1000], 4)
    ws = torch.zeros(abi.zero_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    res = torch.zeros(abi.RESULT_BYTES, dtype=torch.uint8, device="cuda")
    buf = torch.zeros(4096, dtype=torch.float32, device="cuda")
    good = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_grad_norm=1.0,
                loss_scale=1.0, step=1)
    args = abi.step_args(**good)
    contrib = [buf.data_ptr()] * 4
    cases = [
        (abi.ZERO_EALIGN, dict(contrib=[buf.data_ptr() + 2] + contrib[1:])),
        (abi.ZERO_EALIGN, dict(grad=buf.data_ptr() + 4)),
        (abi.ZERO_ENOSPC, dict(ws_bytes=100)),
        (abi.ZERO_EINVAL, dict(rank=4)),
        (abi.ZERO_EINVAL, dict(args=abi.step_args(**{**good, "loss_scale": 0.0}))),
        (abi.ZERO_EINVAL, dict(args=abi.step_args(**{**good, "step": 0}))),
        (abi.ZERO_EINVAL, dict(args=abi.step_args(**{**good, "beta1": 1.0}))),
        (abi.ZERO_EALIGN, dict(slot=buf.data_ptr() + 1)),
    ]
    for code, over in cases:
        kw = dict(contrib=contrib, grad=buf.data_ptr(), ws_bytes=ws.numel(), rank=0, args=args,
                  slot=buf.data_ptr())
        kw.update(over)
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_reduce_adam_step(plan, kw["rank"], kw["contrib"], buf, buf, buf, kw["slot"],
                                      kw["grad"], ws, kw["ws_bytes"], kw["args"], res)
        assert e.value.code == code, (over, e.value)


@pytest.mark.parametrize("begin", range(8))
@pytest.mark.parametrize("count", [1, 3, 4, 5, 63, 255, 256, 257, 259, 1027, 70_001])
def test_slot_offsets(begin, count):
    """Every slot alignment (flat offset mod 8) with lengths that end inside a
    quad, a wave or several waves: state and slot bit-exact, guards intact."""
    run_window(synth.TINY, 0, begin, count, steps=2)


@pytest.mark.parametrize("fill", [0xAB, 0xFF])
def test_workspace_content_does_not_matter(fill):
    print(f"[workspace fill {fill:#x}]", flush=True)
    run_window(synth.LLAMA3_8B, 0, 0, 3_000_001, steps=2, ws_fill=fill)
    run_window(synth.LLAMA3_8B, 0, 0, 3_000_001, steps=2, fused=False, ws_fill=fill)


@pytest.mark.parametrize("rank", [0, 2, 3])
def test_tiny_psi_whole_padding_shard(rank):
    """psi = 5 over N = 4: S = 2, rank 2 holds one real element and one
    padding element, rank 3 holds padding only; padding stays exactly zero."""
    w = dataclasses.replace(synth.TINY, name="psi5", cfg_id=41, tensors=(("a", (5,)),),
                            world_size=4, max_grad_norm=1.0, weight_decay=0.1)
    reps = run_window(w, rank, 0, 2, steps=3)
    assert len(reps) == 3
    if rank == 3:
        from zero_sharded_optimizer_rank_amd.shard import DeviceShard
        d = DeviceShard(w, 3, 0, 2)
        d.load_initial_state()
        d.load_contributions(1, w.loss_scale0)
        d.step(d.args(1, w.loss_scale0))
        res = d.result()
        assert res.own_q == 0 and not res.skip
        for name in ("grad", "master", "m", "v"):
            assert not np.any(d.fetch(name)), name
        assert not np.any(d.fetch("slot"))
