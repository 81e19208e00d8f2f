"""GPU parity of the offload form (reduce on the GPU, Adam on the host from
host-resident fp32 state, fp16 parameters back over PCIe) through the C ABI
against the CPU oracle, on the same seeded inputs.  Bar as in parity_util:
g, the exact norm and decisions, master, m, v and the slot all bit-exact."""
import numpy as np
import pytest

import oracle
import synth
from oracle import run as orun

from parity_util import check_result, compare_state, other_overflow_at, run_window, StepReport

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _windows():
    cases = []
    for w, count in ((synth.LLAMA3_8B, (1 << 20) + 3), (synth.GPT2, 300_001)):
        p = orun.workload_plan(w)
        for r in w.parity_ranks:
            if w.inject_step is not None and r == 0:
                e = synth.inject_site(w, w.inject_step)[1]
                begin = max(0, e - count // 2)
            elif r == w.parity_ranks[-1]:
                begin = p.shard - count
            else:
                begin = 777
            cases.append(pytest.param(w, r, begin, count, id=f"{w.name}-r{r}"))
    return cases


@pytest.mark.parametrize("w,rank,begin,count", _windows())
def test_offload_window_parity(w, rank, begin, count):
    print(f"[offload window {w.name} rank {rank} begin {begin} count {count}]", flush=True)
    reps = run_window(w, rank, begin, count, offload=dict(chunk=1 << 18, threads=8))
    if w.inject_step is not None and rank == 0:
        assert reps[w.inject_step - 1].skip


@pytest.mark.parametrize("chunk,threads", [(64, 1), (4096, 3), (1 << 16, 16)])
def test_offload_chunking(chunk, threads):
    """Pipeline chunk sizes from one vector to many chunks, ragged tails,
    1..16 threads, a misaligned slot (flat offset mod 8 = 5)."""
    print(f"[offload chunk {chunk} threads {threads}]", flush=True)
    run_window(synth.TINY, 1, 2, 100_003, steps=3, offload=dict(chunk=chunk, threads=threads))
    run_window(synth.TINY, 0, 0, 1, steps=2, offload=dict(chunk=chunk, threads=threads))


def test_offload_phase_split_equals_fused():
    w = synth.LLAMA3_8B
    a = run_window(w, 1, 12345, 200_001, steps=3, fused=False, offload=dict(chunk=1 << 16))
    b = run_window(w, 1, 12345, 200_001, steps=3, fused=True, offload=dict(chunk=1 << 16))
    assert [r.coef for r in a] == [r.coef for r in b]


def test_offload_errors():
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.shard import OffloadShard
    w = synth.TINY
    d = OffloadShard(w, 0, 0, 1000, chunk=64, threads=2)
    d.load_initial_state()
    d.load_contributions(1, w.loss_scale0)
    args = d.args(1, w.loss_scale0)
    d.reduce_check(args)
    bad = abi.offload_staging(d._g_pin, d._h_pin, 100)
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_offload_adam_apply(d.plan, 0, d.grad, d.h_master, d.h_m, d.h_v, d.slot_ptr(),
                                    args, d.res, bad, 2, d.stream)
    assert e.value.code == abi.ZERO_EINVAL
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_offload_adam_apply(d.plan, 0, d.grad, d.h_master, d.h_m, d.h_v, d.slot_ptr(),
                                    args, d.res, d.staging, 0, d.stream)
    assert e.value.code == abi.ZERO_EINVAL
    # nothing was changed by the failed calls; a good call then applies the step
    assert not np.any(d.h_m)
    res = d.adam_apply(args)
    assert not res.skip and np.any(d.h_m)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w,rank", [pytest.param(synth.LLAMA3_8B, 0, id="llama3_8b-r0"),
                                    pytest.param(synth.GPT2, 1, id="gpt2_1p5b-r1")])
def test_offload_full_size(w, rank):
    """Whole shards in the configuration bench.py --offload times: the exact
    norm and decisions, and every element of g and the device slot and of
    the host master, m and v, against the C form of the oracle's update."""
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.shard import OffloadShard
    from oracle import fast
    from test_gpu_fullsize import _Fetcher, _feed_and_reduce, _initial_host_state

    print(f"[offload full size {w.name} rank {rank}]", flush=True)
    dev = OffloadShard(w, rank)
    dev.load_initial_state()
    p = orun.workload_plan(w)
    op, om, ov, oh = _initial_host_state(w, dev.flat_begin, dev.count)
    hg = np.empty(dev.count, dtype=np.float32)
    fetch = _Fetcher(dev)
    other_sq = w.other_sq(p.real(rank)) if w.other_ranks_from_config else 0.0
    scaler = abi.new_scaler(w.loss_scale0)
    o_scale, o_good, o_t = w.loss_scale0, 0, 0
    for step in range(1, w.steps + 1):
        ovf_other = other_overflow_at(w, step, dev.flat_begin, dev.count)
        sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, o_t + 1, w.world_size,
                                 o_scale)
        q_all, bad_all, _ = _feed_and_reduce(dev, step, scaler.scale, sc.inv32, g_out=hg)
        res = dev.step(dev.args(scaler.t + 1, scaler.scale, other_sq=other_sq,
                                other_overflow=ovf_other))
        fin = oracle.finalize(q_all, bad_all, sc.inv64, w.max_grad_norm, other_sq=other_sq,
                              other_overflow=ovf_other)
        check_result(res, fin, step)
        rep = StepReport(step, fin.skip, float(fin.coef))
        assert fetch.compare(rep, "grad", hg) == 0, step
        if not fin.skip:
            fast.adam_update(hg, op, om, ov, oh, sc, fin.coef)
        fetch.compare(rep, "slot", oh)
        for name, want in (("master", op), ("m", om), ("v", ov)):
            rep.mismatches[name] = fast.count_unequal(dev.fetch(name), want)
        assert all(x == 0 for x in rep.mismatches.values()), (step, rep.mismatches)
        assert dev.guards_intact()
        print(f"  step {step}: skip={fin.skip} coef={float(fin.coef):.6g}, "
              f"{dev.count} elements compared", flush=True)
        abi.zero_scaler_update(scaler, bool(res.skip))
        o_scale, o_good = oracle.scaler_update(o_scale, o_good, fin.skip)
        o_t += 0 if fin.skip else 1
    del dev
    torch.cuda.empty_cache()
