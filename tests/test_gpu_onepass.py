"""GPU parity of the single-pass step (zero_reduce_adam_step_1pass) for steps
without clipping, through the C ABI against the CPU oracle.

The single pass reduces, adds the exact squares and applies the update from
the current master/m/v into a second set; the caller adopts that set only if
the step was not skipped.  The bar is the two-pass step's: result word and
every state element bit for bit; on a skipped step the current set must be
exactly the state before the step.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import run as orun

from parity_util import check_result, compare_state, run_window, StepReport

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _unclipped(w: synth.Workload) -> synth.Workload:
    return dataclasses.replace(w, max_grad_norm=0.0)


@pytest.mark.parametrize("variant", ["config", "skip"])
def test_onepass_tiny_all_shards(variant):
    """All four shards of the tiny workload.  Every rank runs its single pass
    first; the exact all-reduce of the squared-norm integers and overflow flags
    follows (zero_finalize with the other ranks' values), and each rank adopts
    its new set only if no rank overflowed."""
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard

    w = synth.TINY
    if variant == "skip":
        w = dataclasses.replace(w, inject_step=2)
    print(f"[onepass tiny_all_shards {variant}]", flush=True)
    records = orun.run_all_ranks(w)
    n = w.world_size
    devs = [DeviceShard(w, r, one_pass=True) for r in range(n)]
    for d in devs:
        d.load_initial_state()
    scaler = abi.new_scaler(w.loss_scale0)
    skips = []
    for rec in records:
        assert rec.loss_scale == scaler.scale
        for d in devs:
            d.load_contributions(rec.step, scaler.scale)
        base = devs[0].args(scaler.t + 1, scaler.scale)
        for d in devs:
            d.step_1pass(base)
        rs = [d.result() for d in devs]
        for r, d in enumerate(devs):
            a = d.args(scaler.t + 1, scaler.scale,
                       other_q=sum(rs[x].own_q for x in range(n) if x != r),
                       other_overflow=any(rs[x].overflow for x in range(n) if x != r))
            d.finalize(a)
        skipped = None
        for r, d in enumerate(devs):
            res = d.result()
            check_result(res, rec.fin[r], rec.step)
            skipped = bool(res.skip)
            if not skipped:
                d.adopt()
            rep = StepReport(rec.step, skipped, float(res.clip_coef))
            st = rec.after[r]
            for name, want in (("master", st.p), ("m", st.m), ("v", st.v),
                               ("slot", st.h.view(np.uint16))):
                compare_state(rep, name, d.fetch(name), want)
            assert all(v == 0 for v in rep.mismatches.values()), (rec.step, r, rep.mismatches)
            assert d.guards_intact()
        skips.append(skipped)
        abi.zero_scaler_update(scaler, skipped)
        assert scaler.t == rec.t
    assert skips == [s == w.inject_step for s in range(1, w.steps + 1)]
    last = devs[-1]
    for name in ("master", "m", "v", "slot"):
        assert last.fetch(name)[-1] == 0  # the padding element stays exactly zero


def _windows():
    count = (1 << 20) + 3
    cases = []
    for w in (synth.GPT2, _unclipped(synth.FLAT75), _unclipped(synth.LLAMA3_8B),
              _unclipped(synth.LLAMA3_8B_BF16)):
        p = orun.workload_plan(w)
        for r in w.parity_ranks:
            if w.inject_step is not None and r == 0:
                e = synth.inject_site(w, w.inject_step)[1]
                begin = max(0, e - count // 2)
            elif r == w.parity_ranks[-1]:
                begin = p.shard - count
            else:
                begin = 12345
            cases.append(pytest.param(w, r, begin, count, id=f"{w.name}-r{r}"))
    return cases


@pytest.mark.parametrize("w,rank,begin,count", _windows())
def test_onepass_window_parity(w, rank, begin, count):
    """Every step on a ~1M-element window of the parity ranks' shards: GPT-2
    as configured (unclipped, dynamic loss scale), and the flat 7.5B and
    Llama-3-8B workloads with clipping off (the latter skips its step 2, on
    rank 0 from its own overflow and on the others from another rank's)."""
    print(f"[onepass window {w.name} rank {rank} begin {begin} count {count}]", flush=True)
    reps = run_window(w, rank, begin, count, one_pass=True)
    if w.inject_step is not None:
        assert reps[w.inject_step - 1].skip
        assert not any(r.skip for i, r in enumerate(reps) if i != w.inject_step - 1)
    assert all(r.coef == 1.0 for r in reps)


@pytest.mark.parametrize("count", [1, 3, 4, 5, 255, 256, 257, 511, 4099])
@pytest.mark.parametrize("begin", [0, 1, 2, 3, 5])
def test_onepass_small_lengths_and_slot_offsets(begin, count):
    """Shard lengths inside a quad, a wave and a workgroup, at every slot
    alignment (flat offset mod 8), GPT-2 rank 1's geometry."""
    w = synth.GPT2
    print(f"[onepass small begin {begin} count {count}]", flush=True)
    run_window(w, 1, begin, count, steps=2, one_pass=True)


@pytest.mark.parametrize("count", [1, 5, 511, 513, 512 * 256 + 1, 512 * 512 + 3])
@pytest.mark.parametrize("begin", [0, 3])
def test_onepass_bf16_lengths_and_tree_chunks(begin, count):
    """bf16: lengths inside a quad and a workgroup, and around the tree
    kernel's chunk transitions, at two slot alignments."""
    w = _unclipped(synth.LLAMA3_8B_BF16)
    print(f"[onepass bf16 begin {begin} count {count}]", flush=True)
    run_window(w, 1, 4096 + begin, count, steps=2, one_pass=True)


@pytest.mark.parametrize("variant", ["config", "skip"])
def test_onepass_bf16_tiny_all_shards(variant):
    """bf16, all four tiny shards: each rank's pass first, then the other
    ranks' squared norms (summed in rank order) and overflow flags through
    zero_finalize_bf16, and the adoption only if no rank overflowed."""
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    from test_gpu_bf16 import _oracle_all_ranks

    w = synth.TINY_BF16
    if variant == "skip":
        w = dataclasses.replace(w, inject_step=2)
    print(f"[onepass bf16 tiny_all_shards {variant}]", flush=True)
    records = _oracle_all_ranks(w, w.max_grad_norm, w.steps)
    n = w.world_size
    devs = [DeviceShard(w, r, one_pass=True) for r in range(n)]
    for d in devs:
        d.load_initial_state()
    scaler = abi.new_scaler(w.loss_scale0)
    for step, scale, fins, _gs, states, t in records:
        assert scale == scaler.scale
        for d in devs:
            d.load_contributions(step, scaler.scale)
        base = devs[0].args(scaler.t + 1, scaler.scale)
        for d in devs:
            d.step_1pass(base)
        rs = [d.result() for d in devs]
        for r, d in enumerate(devs):
            other = 0.0
            for x in range(n):
                if x != r:
                    other += rs[x].own_sq
            d.finalize(d.args(scaler.t + 1, scaler.scale, other_sq=other,
                              other_overflow=any(rs[x].overflow for x in range(n) if x != r)))
        skipped = None
        for r, d in enumerate(devs):
            res = d.result()
            check_result(res, fins[r], step)
            skipped = bool(res.skip)
            if not skipped:
                d.adopt()
            rep = StepReport(step, skipped, float(res.clip_coef))
            for name, want in zip(("master", "m", "v", "slot"), states[r]):
                compare_state(rep, name, d.fetch(name), want)
            assert all(v == 0 for v in rep.mismatches.values()), (step, r, rep.mismatches)
            assert d.guards_intact()
        if variant == "skip":
            assert skipped == (step == 2)
        abi.zero_scaler_update(scaler, skipped)
        assert scaler.t == t


@pytest.mark.parametrize("fmt", ["fp16", "bf16"])
def test_onepass_empty_shard(fmt):
    """S = 0: nothing to update; the result word is still written."""
    import zero_sharded_optimizer_rank_amd.abi as abi
    step = (abi.zero_reduce_adam_step_1pass_bf16 if fmt == "bf16"
            else abi.zero_reduce_adam_step_1pass)
    n = 4
    plan = abi.zero_plan_t(0, n, 1, 0, 0)
    ws = torch.zeros(abi.zero_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    res = torch.full((abi.RESULT_BYTES,), 0xFF, dtype=torch.uint8, device="cuda")
    d = [torch.zeros(16, dtype=torch.float32, device="cuda") for _ in range(8)]
    args = abi.step_args(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                         max_grad_norm=0.0, loss_scale=1.0, step=1)
    step(plan, 0, [d[0]] * n, *d[1:8], ws, ws.numel(), args, res)
    torch.cuda.synchronize()
    r = abi.zero_step_result_t.from_buffer_copy(res.cpu().numpy().tobytes())
    assert r.own_q == 0 and r.norm == 0.0 and r.clip_coef == 1.0 and not r.skip
    assert all(int(x.abs().sum().item()) == 0 for x in d)


@pytest.mark.parametrize("wname", ["gpt2_1p5b", "llama3_8b_bf16"])
def test_onepass_matches_two_pass_bitwise(wname):
    """The single pass and the two-pass step leave the same bits (state, slot
    and result word) on the same inputs."""
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    w = _unclipped(synth.BY_NAME[wname])
    print(f"[onepass vs two-pass {wname}]", flush=True)
    rank = w.world_size - 1
    a = DeviceShard(w, rank, 1000, 200_003, one_pass=True)
    b = DeviceShard(w, rank, 1000, 200_003)
    for d in (a, b):
        d.load_initial_state()
    for step in (1, 2, 3):
        for d in (a, b):
            d.load_contributions(step, w.loss_scale0)
        args = a.args(step, w.loss_scale0, max_norm=0.0, other_sq=0.5)
        a.step_1pass(args)
        b.step(args)
        ra, rb = a.result(), b.result()
        assert bytes(ra) == bytes(rb), step
        assert not ra.skip
        a.adopt()
        for name in ("master", "m", "v", "slot"):
            assert np.array_equal(a.fetch(name), b.fetch(name)), (step, name)


def test_onepass_rejects_clipping_and_overlap():
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    w = synth.GPT2
    d = DeviceShard(w, 0, 0, 4096, one_pass=True)
    d.load_initial_state()
    d.load_contributions(1, w.loss_scale0)
    before = [d.fetch(x).copy() for x in ("master", "m", "v", "slot")]
    with pytest.raises(abi.ZeroError) as e:
        d.step_1pass(d.args(1, w.loss_scale0, max_norm=1.0))
    assert e.value.code == abi.ZERO_EINVAL
    ptrs = [d.contrib_ptrs(), d.master, d.m, d.v, d.master2, d.m2, d.v2,
            d.slot_buf2.data_ptr() + 2 * d.slot_off]
    for bad in ([d.master, d.m, d.v, d.master, d.m2, d.v2],      # out aliases in
                [d.master, d.m, d.v, d.master2, d.master2, d.v2],  # outs alias
                [d.master, d.m, d.v, d.master2, d.m2, d.m]):       # out aliases another in
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_reduce_adam_step_1pass(d.plan, 0, ptrs[0], *bad, ptrs[7], d.ws,
                                            d.ws.numel(), d.args(1, w.loss_scale0), d.res,
                                            d.stream)
        assert e.value.code == abi.ZERO_EINVAL
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_reduce_adam_step_1pass(d.plan, 0, ptrs[0], *ptrs[1:7], ptrs[7], d.ws, 16,
                                        d.args(1, w.loss_scale0), d.res, d.stream)
    assert e.value.code == abi.ZERO_ENOSPC
    after = [d.fetch(x) for x in ("master", "m", "v", "slot")]
    assert all(np.array_equal(x, y) for x, y in zip(before, after))


@pytest.mark.parametrize("value", [np.inf, -np.inf, np.nan])
@pytest.mark.parametrize("pos", ["first", "last", "tail"])
def test_onepass_nonfinite_skips(value, pos):
    """A non-finite contribution at the first, the last real and a tail
    element: the result word matches the oracle's, the step is skipped, and
    the current set (not adopted) is bitwise the state before the step."""
    import oracle
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    print(f"[onepass nonfinite {value} at {pos}]", flush=True)
    w = synth.TINY
    p = orun.workload_plan(w)
    rank, count = 3, p.shard  # rank 3 holds the padding element
    j = {"first": 0, "last": p.real(rank) - 1, "tail": count - 5}[pos]
    q = 2
    d = DeviceShard(w, rank, 0, count, one_pass=True)
    d.load_initial_state()
    d.load_contributions(1, w.loss_scale0)
    d.contrib[q, j] = int(np.array([value], dtype=np.float16).view(np.int16)[0])
    before = {x: d.fetch(x).copy() for x in ("master", "m", "v", "slot")}
    d.step_1pass(d.args(1, w.loss_scale0))
    res = d.result()
    c = orun.shard_contrib(w, p, rank, 1, w.loss_scale0, 0, count)
    c[q, j] = np.array([value], dtype=np.float16).view(np.uint16)[0]
    acc = oracle.reduce_contributions(c)
    sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, 1, w.world_size,
                             w.loss_scale0)
    fin = oracle.finalize(oracle.exact_sq_units(acc), oracle.nonfinite(acc), sc.inv64, 0.0)
    check_result(res, fin, 1)
    assert res.skip and res.overflow
    for x, arr in before.items():
        assert np.array_equal(d.fetch(x), arr), x
    assert d.guards_intact()


def test_onepass_extreme_magnitudes():
    """N = 64 with every contribution at +-65504 (and one subnormal): the
    largest sums the pass sees; result word and state against the oracle."""
    import oracle
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    print("[onepass extreme magnitudes]", flush=True)
    w = dataclasses.replace(synth.TINY, world_size=64)
    p = orun.workload_plan(w)
    count = p.shard
    d = DeviceShard(w, 0, 0, count, one_pass=True)
    d.load_initial_state()
    c = np.full((64, d.ld), 65504.0, dtype=np.float16)
    c[:, ::2] = -65504.0
    c[5, 7] = 2.0**-24
    d.contrib.copy_(torch.from_numpy(c.view(np.int16)))
    d.step_1pass(d.args(1, 1.0))
    res = d.result()
    pm, m, v, h = orun.initial_state(w, p, 0, 0, count)
    sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, 1, 64, 1.0)
    out = oracle.shard_step(c[:, :count].view(np.uint16), pm, m, v, h, sc, 0.0)
    check_result(res, out.fin, 1)
    assert not res.skip
    d.adopt()
    for name, want in (("master", out.p), ("m", out.m), ("v", out.v),
                       ("slot", out.h.view(np.uint16))):
        got = d.fetch(name)
        assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(want).view(np.uint8)), name



def _in_place_cases():
    count = 300_001
    cases = []
    for w, rank in ((synth.GPT2, 63), (_unclipped(synth.LLAMA3_8B), 0),
                    (_unclipped(synth.LLAMA3_8B), 1), (_unclipped(synth.LLAMA3_8B_BF16), 0),
                    (_unclipped(synth.LLAMA3_8B_BF16), 7)):
        p = orun.workload_plan(w)
        if w.inject_step is not None and rank == 0:
            begin = max(0, synth.inject_site(w, w.inject_step)[1] - count // 2)
        else:
            begin = p.shard - count - 3
        cases.append(pytest.param(w, rank, begin, count, id=f"{w.name}-r{rank}"))
    return cases


@pytest.mark.parametrize("w,rank,begin,count", _in_place_cases())
def test_onepass_in_place_slot(w, rank, begin, count):
    """The single pass writing the live slot, followed every step by
    zero_slot_restore: on applied steps the slot is the new cast, on the
    skipped step (the rank's own inf, or another rank's) it is restored to
    its content before the step; every step bit-exact against the oracle."""
    print(f"[onepass in-place slot {w.name} rank {rank} begin {begin}]", flush=True)
    reps = run_window(w, rank, begin, count, one_pass=True, in_place_slot=True)
    if w.inject_step is not None:
        assert reps[w.inject_step - 1].skip


def test_slot_restore_errors_and_no_op():
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard
    w = synth.GPT2
    d = DeviceShard(w, 1, 5, 1000, one_pass=True)
    d.load_initial_state()
    d.load_contributions(1, w.loss_scale0)
    d.step_1pass(d.args(1, w.loss_scale0))
    before = d.fetch("slot").copy()
    d.slot.fill_(0x1234)  # not the cast of the master: a no-op restore must keep it
    d.restore_slot()
    assert not d.result().skip
    assert (d.fetch("slot") == 0x1234).all()
    d.slot.copy_(torch.from_numpy(before.view(np.int16)))
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_slot_restore(d.plan, 1, d.master, d.master, d.res, d.stream)
    assert e.value.code == abi.ZERO_EINVAL
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_slot_restore(d.plan, 1, d.master.data_ptr() + 2, d.slot_ptr(), d.res, d.stream)
    assert e.value.code == abi.ZERO_EALIGN
