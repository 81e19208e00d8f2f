"""GPU parity of the bf16 variant (bf16 contributions and slot, fp32 master,
m, v; the shard's squared norm as the fixed pairwise fp64 tree) through the
C ABI against the CPU oracle, on the same seeded inputs.  Bar as in
parity_util: g, the tree value, norm, clip coefficient and decisions
bit-exact; master, m, v and the slot bit-exact as well."""
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


def _oracle_all_ranks(w, max_norm, steps):
    """Host simulation of every rank: per-rank trees, the other ranks' share
    summed in rank order, global skip from the overflow flags."""
    p = orun.workload_plan(w)
    n = w.world_size
    states = [list(orun.initial_state(w, p, r)) for r in range(n)]
    scale, good, t = w.loss_scale0, 0, 0
    out = []
    for step in range(1, steps + 1):
        sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, t + 1, n, scale)
        accs = [oracle.reduce_contributions_bf16(orun.shard_contrib(w, p, r, step, scale))
                for r in range(n)]
        trees = [oracle.sq_tree(a) for a in accs]
        bads = [oracle.nonfinite(a) for a in accs]
        owns = [(x * sc.inv64) * sc.inv64 for x in trees]
        fins, gs = [], []
        for r in range(n):
            other = 0.0
            for x in range(n):
                if x != r:
                    other += owns[x]
            fins.append(oracle.finalize_bf16(trees[r], bads[r], sc.inv64, max_norm,
                                             other_sq=other,
                                             other_overflow=any(bads[x] for x in range(n)
                                                                if x != r)))
            gs.append(oracle.unscale(accs[r], sc.inv32))
        skipped = fins[0].skip
        if not skipped:
            for r in range(n):
                pp, mm, vv, _ = oracle.adam_apply(gs[r], *states[r][:3], sc, fins[r].coef)
                states[r] = [pp, mm, vv, oracle.f32_to_bf16(pp)]
            t += 1
        out.append((step, scale, fins, gs, [list(s) for s in states], t))
        scale, good = oracle.scaler_update(scale, good, skipped)
    return out


@pytest.mark.parametrize("variant", ["config", "clipped", "skip"])
def test_tiny_bf16_all_shards(variant):
    """All four shards, three steps; each rank's own_sq is exchanged on the
    host (summed in rank order) between the reduce and the update."""
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    abi = _abi()
    w = synth.TINY_BF16
    max_norm = 1e-2 if variant == "clipped" else w.max_grad_norm
    if variant == "skip":
        w = dataclasses.replace(w, inject_step=2)
    print(f"[tiny_bf16_all_shards {variant}]", flush=True)
    records = _oracle_all_ranks(w, max_norm, w.steps)
    n = w.world_size
    devs = [DeviceShard(w, r) for r in range(n)]
    for d in devs:
        d.load_initial_state()
    scaler = abi.new_scaler(w.loss_scale0)
    for step, scale, fins, gs, states, t in records:
        assert scale == scaler.scale
        for d in devs:
            d.load_contributions(step, scaler.scale)
        base = devs[0].args(scaler.t + 1, scaler.scale, max_norm=max_norm)
        for d in devs:
            d.reduce_check(base)
        rs = [d.result() for d in devs]
        for r, d in enumerate(devs):
            other = 0.0
            for x in range(n):
                if x != r:
                    other += rs[x].own_sq
            a = d.args(scaler.t + 1, scaler.scale, max_norm=max_norm, other_sq=other,
                       other_overflow=any(rs[x].overflow for x in range(n) if x != r))
            d.finalize(a)
            d.adam_apply(a)
        for r, d in enumerate(devs):
            res = d.result()
            check_result(res, fins[r], step)
            assert np.array_equal(d.fetch("grad").view(np.uint32), gs[r].view(np.uint32))
            rep = StepReport(step, bool(res.skip), float(res.clip_coef))
            for name, want in zip(("master", "m", "v", "slot"), states[r]):
                compare_state(rep, name, d.fetch(name), want)
            assert all(v == 0 for v in rep.mismatches.values()), (step, r, rep.mismatches)
            assert d.guards_intact()
        if variant == "clipped":
            assert fins[0].coef < 1
        if variant == "skip":
            assert fins[0].skip == (step == 2)
        abi.zero_scaler_update(scaler, bool(devs[0].result().skip))
        assert scaler.t == t


def _windows():
    cases = []
    w = synth.LLAMA3_8B_BF16
    p = orun.workload_plan(w)
    for r, count in ((0, (1 << 20) + 3), (1, (1 << 22) + 5), (7, (1 << 20) + 1)):
        if r == 0:
            e = synth.inject_site(w, w.inject_step)[1]
            begin = max(0, e - count // 2)
        elif r == 7:
            begin = p.shard - count
        else:
            begin = 4321
        cases.append(pytest.param(w, r, begin, count, id=f"{w.name}-r{r}"))
    return cases


@pytest.mark.parametrize("w,rank,begin,count", _windows())
def test_bf16_window_parity(w, rank, begin, count):
    print(f"[bf16 window {w.name} rank {rank} begin {begin} count {count}]", flush=True)
    reps = run_window(w, rank, begin, count)
    if rank == 0:
        assert reps[w.inject_step - 1].skip
    assert any(r.coef < 1 for r in reps)


def test_bf16_phase_split_equals_fused():
    print("[bf16 phase split vs fused]", flush=True)
    w = synth.LLAMA3_8B_BF16
    a = run_window(w, 1, 999, 500_001, steps=3, fused=False)
    b = run_window(w, 1, 999, 500_001, steps=3, fused=True)
    assert [r.coef for r in a] == [r.coef for r in b]


@pytest.mark.parametrize("begin", [0, 1, 3, 5, 7])
@pytest.mark.parametrize("count", [1, 4, 5, 257, 2049, 70_001])
def test_bf16_slot_offsets(begin, count):
    run_window(synth.TINY_BF16, 0, begin, count, steps=2)


@pytest.mark.parametrize("n", [1, 3, 64])
def test_bf16_world_sizes(n):
    print(f"[bf16 world size {n}]", flush=True)
    w = dataclasses.replace(synth.TINY_BF16, world_size=n, max_grad_norm=0.05,
                            weight_decay=0.01)
    p = orun.workload_plan(w)
    run_window(w, n - 1, 0, min(p.shard, 200_003), steps=2)


@pytest.mark.parametrize("value", [0x7F80, 0xFF80, 0x7FC0])
@pytest.mark.parametrize("pos", ["first", "tail"])
def test_bf16_nonfinite_skips(value, pos):
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    print(f"[bf16 nonfinite {value:#x} at {pos}]", flush=True)
    w = synth.TINY_BF16
    p = orun.workload_plan(w)
    rank, count = 3, p.shard
    j = {"first": 0, "tail": count - 2}[pos]
    d = DeviceShard(w, rank, 0, count)
    d.load_initial_state()
    d.load_contributions(1, 1.0)
    d.contrib[1, j] = int(np.array([value], np.uint16).view(np.int16)[0])
    before = {x: d.fetch(x).copy() for x in ("master", "m", "v", "slot")}
    d.step(d.args(1, 1.0))
    res = d.result()
    c = orun.shard_contrib(w, p, rank, 1, 1.0, 0, count)
    c[1, j] = value
    acc = oracle.reduce_contributions_bf16(c)
    sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, 1, w.world_size, 1.0)
    fin = oracle.finalize_bf16(oracle.sq_tree(acc), oracle.nonfinite(acc), sc.inv64,
                               w.max_grad_norm)
    check_result(res, fin, 1)
    assert res.skip
    assert np.array_equal(d.fetch("grad").view(np.uint32),
                          oracle.unscale(acc, sc.inv32).view(np.uint32))
    for x, arr in before.items():
        assert np.array_equal(d.fetch(x), arr), x


def test_bf16_extreme_magnitudes():
    """bf16's range: sums near fp32's largest finite value, and one that
    overflows to inf (a skip); squares stay exact in fp64."""
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    w = dataclasses.replace(synth.TINY_BF16, world_size=4)
    count = 5000
    for big, overflow in ((0x7E00, False), (0x7F7F, True)):  # 4 x 2^125 fits; 2 x max does not
        d = DeviceShard(w, 0, 0, count)
        d.load_initial_state()
        c = np.full((4, d.ld), big, dtype=np.uint16)
        c[:, 1::2] |= 0x8000
        c[0, 10] = 0x0001  # a subnormal
        d.contrib.copy_(torch.from_numpy(c.view(np.int16)))
        d.step(d.args(1, 1.0))
        res = d.result()
        acc = oracle.reduce_contributions_bf16(c[:, :count])
        sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, 1, 4, 1.0)
        fin = oracle.finalize_bf16(oracle.sq_tree(acc), oracle.nonfinite(acc), sc.inv64,
                                   w.max_grad_norm)
        check_result(res, fin, 1)
        assert bool(res.overflow) == overflow
        assert np.array_equal(d.fetch("grad").view(np.uint32),
                              oracle.unscale(acc, sc.inv32).view(np.uint32))


def test_bf16_empty_shard_and_errors():
    abi = _abi()
    n = 4
    plan = abi.zero_plan_t(0, n, 1, 0, 0)
    ws = torch.zeros(abi.zero_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    res = torch.zeros(abi.RESULT_BYTES, dtype=torch.uint8, device="cuda")
    dummy = torch.zeros(16, dtype=torch.float32, device="cuda")
    args = abi.step_args(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                         max_grad_norm=1.0, loss_scale=1.0, step=1)
    abi.zero_reduce_adam_step_bf16(plan, 0, [dummy] * n, dummy, dummy, dummy, dummy, dummy, ws,
                                   ws.numel(), args, res)
    torch.cuda.synchronize()
    r = abi.zero_step_result_t.from_buffer_copy(res.cpu().numpy().tobytes())
    assert r.own_q == 0 and r.norm == 0.0 and r.clip_coef == 1.0 and not r.skip
    plan, _ = abi.zero_plan([1000], 4)
    bad = abi.step_args(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                        max_grad_norm=1.0, loss_scale=1.0, step=1, other_q=5)
    buf = torch.zeros(4096, dtype=torch.float32, device="cuda")
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_reduce_adam_step_bf16(plan, 0, [buf] * 4, buf, buf, buf, buf, buf, ws,
                                       ws.numel(), bad, res)
    assert e.value.code == abi.ZERO_EINVAL
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_finalize_bf16(plan, bad, res)
    assert e.value.code == abi.ZERO_EINVAL


@pytest.mark.parametrize("count", [512 * 256 - 1, 512 * 256 + 1, 512 * 512 + 3, 512 * 256 * 3 + 7])
def test_bf16_tree_chunk_boundaries(count):
    """Window sizes around the tree kernel's chunk transitions (one partial
    per 512-element workgroup, at most 256 tree workgroups, power-of-two
    chunks): the value is the one fixed tree whatever the split."""
    print(f"[bf16 tree chunks count {count}]", flush=True)
    run_window(synth.LLAMA3_8B_BF16, 1, 4097, count, steps=2)
