"""GPU parity of the FSDP / ZeRO-3 unit path (zero_units_*): every unit a rank
holds is updated by one launch of each kernel, against the oracle on the same
seeded inputs."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from oracle import fast

from parity_util import check_result, run_units_all_ranks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(a):
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint16)


@pytest.mark.parametrize("variant", ["config", "clipped", "skip"])
def test_tiny_fsdp_all_ranks(variant):
    """All four ranks of the tiny unit layout (units of 1e6, 1000 and 3
    elements, the last padded), three steps, with the exact all-reduce of the
    squared-norm integers and overflow flags between the ranks."""
    print(f"[tiny_fsdp {variant}]", flush=True)
    w = synth.TINY_FSDP
    max_norm = 1.0 if variant == "clipped" else w.max_grad_norm
    if variant == "skip":
        w = dataclasses.replace(w, inject_step=2)
    reports = run_units_all_ranks(w, max_norm)
    if variant == "clipped":
        assert all(r.coef < 1 for r in reports)
    if variant == "skip":
        assert [r.skip for r in reports] == [s == 2 for s in range(1, w.steps + 1)]


@pytest.mark.parametrize("variant", ["config", "clipped", "skip"])
def test_units_deferred_reduce_all_ranks(variant):
    """Above N = 8 the unit reduce sums eight one-chunk workgroups' worth of
    quads per workgroup, and a workgroup's chunks may belong to different
    units.  Sixteen ranks of a layout that mixes units of one element per rank
    with units of 20 and 5 chunks, so that workgroups start and end inside
    units and span several small ones; three steps, every rank bit for bit."""
    print(f"[units deferred reduce N=16 {variant}]", flush=True)
    w = dataclasses.replace(
        synth.TINY_FSDP, name="units_n16", cfg_id=16, world_size=16,
        tensors=(("a", (1000, 37)), ("b", (5,)), ("c", (4,)), ("f", (4096, 40)),
                 ("d", (300, 7)), ("e", (2,))),
        units=(0, 1, 2, 3, 4, 5), parity_ranks=tuple(range(16)))
    max_norm = 0.05 if variant == "clipped" else w.max_grad_norm
    if variant == "skip":
        w = dataclasses.replace(w, inject_step=2)
    reports = run_units_all_ranks(w, max_norm)
    if variant == "clipped":
        assert all(r.coef < 1 for r in reports)
    if variant == "skip":
        assert [r.skip for r in reports] == [s == 2 for s in range(1, w.steps + 1)]


@pytest.mark.parametrize("variant", ["config", "skip"])
def test_tiny_fsdp_all_ranks_one_pass(variant):
    """The unit single pass on all four tiny ranks: every rank's pass, then
    the exact all-reduce and the adoption unless a rank overflowed."""
    print(f"[tiny_fsdp one pass {variant}]", flush=True)
    w = synth.TINY_FSDP
    if variant == "skip":
        w = dataclasses.replace(w, inject_step=2)
    reports = run_units_all_ranks(w, 0.0, one_pass=True)
    assert all(r.coef == 1.0 for r in reports)
    if variant == "skip":
        assert [r.skip for r in reports] == [s == 2 for s in range(1, w.steps + 1)]


@pytest.mark.parametrize("variant", ["config", "skip"])
def test_tiny_fsdp_all_ranks_one_pass_in_place_slot(variant):
    """The unit single pass writing the live unit slots, with
    zero_units_slot_restore after the all-reduce's finalize on every rank."""
    print(f"[tiny_fsdp one pass in place {variant}]", flush=True)
    w = synth.TINY_FSDP
    if variant == "skip":
        w = dataclasses.replace(w, inject_step=2)
    reports = run_units_all_ranks(w, 0.0, one_pass=True, in_place_slot=True)
    if variant == "skip":
        assert [r.skip for r in reports] == [s == 2 for s in range(1, w.steps + 1)]


def test_units_one_pass_rejects_clipping_and_overlap():
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.units import DeviceUnits
    w = synth.TINY_FSDP
    d = DeviceUnits(w, 0, one_pass=True)
    with pytest.raises(abi.ZeroError) as e:
        d.step_1pass(d.args(1, w.loss_scale0, max_norm=1.0))
    assert e.value.code == abi.ZERO_EINVAL
    # an out table whose unit 0 writes over its own input state
    bad = abi.unit_table(d.n_units)
    for u in range(d.n_units):
        bad[u] = d.table2[u]
    bad[0].m = d.table[0].m
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_units_step_1pass(w.world_size, d.table, d.table_dev, bad, d.table2_dev,
                                  d.n_units, d.args(1, w.loss_scale0, max_norm=0.0), d.ws,
                                  d.ws.numel(), d.res, d.stream)
    assert e.value.code == abi.ZERO_EINVAL


def _units_host_state(dev):
    """Per unit: the oracle's master (seeded real elements, +0 padding), m, v
    and the fp16 slot, as the device starts."""
    w, st = dev.w, []
    for u, b in enumerate(dev.bufs):
        s, real = b["shard"], dev.unit_real(u)
        p = np.zeros(s, dtype=np.float32)
        if real:
            p[:real] = synth.masters(w, dev.unit_model_start(u), real)
        st.append([p, np.zeros(s, np.float32), np.zeros(s, np.float32),
                   fast.cast16(p)])
    return st


def _feed_units_every_element(dev, step, scale, inv32):
    """Each unit's contributions, generated chunk by chunk, copied to its rows
    and reduced by the C oracle: returns (Q, overflow, g of every element of
    every unit, +0 in padding columns as on the device)."""
    w, n = dev.w, dev.w.world_size
    chunk = (1 << 27) // n
    host = torch.empty((n, chunk), dtype=torch.int16, pin_memory=True)
    hnp = host.numpy().view(np.uint16)
    q_total, bad, gs = 0, False, []
    for u, b in enumerate(dev.bufs):
        real, start = dev.unit_real(u), dev.unit_model_start(u)
        g = np.zeros(b["shard"], dtype=np.float32)
        for c0 in range(0, real, chunk):
            k = min(chunk, real - c0)
            for q in range(n):
                synth.contributions(w, step, q, start + c0, k, scale, out=hnp[q, :k])
            with torch.cuda.stream(dev.stream):
                for q in range(n):
                    b["contrib"][q, c0:c0 + k].copy_(host[q, :k], non_blocking=True)
            qc, bc = fast.reduce_stats(hnp, k)
            q_total += qc
            bad |= bc
            fast.reduce_unscale(hnp, inv32, count=k, out=g[c0:c0 + k])
            dev.stream.synchronize()
        gs.append(g)
    return q_total, bad, gs


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w,rank,one_pass", [
    pytest.param(synth.GPT2_FSDP, 1, False, id="gpt2_1p5b_fsdp-r1"),
    pytest.param(synth.GPT2_FSDP, 63, False, id="gpt2_1p5b_fsdp-r63"),
    pytest.param(synth.LLAMA3_8B_FSDP, 0, False, id="llama3_8b_fsdp-r0"),
    pytest.param(synth.GPT2_FSDP, 1, True, id="gpt2_1p5b_fsdp-r1-1pass"),
    pytest.param(dataclasses.replace(synth.LLAMA3_8B_FSDP, max_grad_norm=0.0), 0, True,
                 id="llama3_8b_fsdp-noclip-r0-1pass")])
def test_units_full_rank_every_element(w, rank, one_pass):
    """A whole rank of a many-unit layout, every step, every element of every
    unit: g (two-pass step), master, m, v and the slot bit for bit against
    the C form of the oracle's unscale and update (pinned to the numpy
    definitions), and the whole-rank Q, norm, coef and skip from the C
    oracle's reduce statistics on the same host chunks.  GPT-2 in 50 units at
    N = 64 runs the deferred unit reduce (ranks 1 and 63, the last);
    Llama-3-8B in 34 units at N = 8 the one-chunk reduce, with clipping and
    the other ranks' share of the norm; the single pass over all units on
    both, its new set adopted after each step.  Every unit of both divides by
    N, so these shards hold no padding; the padded unit layouts are the tiny
    and sixteen-rank tests above."""
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.units import DeviceUnits

    print(f"[units every element {w.name} rank {rank} one_pass={one_pass}]", flush=True)
    dev = DeviceUnits(w, rank, one_pass=one_pass)
    dev.load_initial_state()
    st = _units_host_state(dev)
    other_sq = w.other_sq(dev.real_count()) if w.other_ranks_from_config else 0.0
    scaler = abi.new_scaler(w.loss_scale0)
    o_scale, o_good, o_t = w.loss_scale0, 0, 0
    for step in range(1, w.steps + 1):
        sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, o_t + 1, w.world_size,
                                 o_scale)
        q_all, bad_all, gs = _feed_units_every_element(dev, step, scaler.scale, sc.inv32)
        args = dev.args(scaler.t + 1, scaler.scale, other_sq=other_sq)
        if one_pass:
            dev.step_1pass(args)
        else:
            dev.step(args)
        res = dev.result()
        if one_pass and not res.skip:
            dev.adopt()
        fin = oracle.finalize(q_all, bad_all, sc.inv64, w.max_grad_norm, other_sq=other_sq)
        check_result(res, fin, step)
        if not fin.skip:
            for u in range(dev.n_units):
                fast.adam_update(gs[u], *st[u], sc, fin.coef)
        for u, b in enumerate(dev.bufs):
            s = b["shard"]
            got = {"grad": b["grad"][:s], "master": b["master"][:s], "m": b["m"][:s],
                   "v": b["v"][:s]}
            want = {"grad": gs[u], "master": st[u][0], "m": st[u][1], "v": st[u][2]}
            for name in got:
                if one_pass and name == "grad":
                    continue  # the single pass writes no g
                d = got[name].cpu().numpy()
                assert fast.count_unequal(d, want[name]) == 0, (step, u, name)
            slot = dev.slot(u).cpu().numpy().view(np.uint16)
            assert fast.count_unequal(slot, st[u][3]) == 0, (step, u, "slot")
        assert dev.guards_intact()
        print(f"  step {step}: coef={float(fin.coef):.6g} norm={fin.norm:.6g}, "
              f"{sum(b['shard'] for b in dev.bufs)} elements equal", flush=True)
        abi.zero_scaler_update(scaler, bool(res.skip))
        o_scale, o_good = oracle.scaler_update(o_scale, o_good, fin.skip)
        o_t += 0 if fin.skip else 1
    del dev
    torch.cuda.empty_cache()


def test_units_workspace_content_does_not_matter():
    """Garbage in the workspace before each step changes nothing, and a rank
    with no units at all still produces a result (Q = 0, no skip)."""
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.units import DeviceUnits

    w = synth.TINY_FSDP
    a = DeviceUnits(w, 2)
    b = DeviceUnits(w, 2)
    for d in (a, b):
        d.load_initial_state()
    for step in (1, 2):
        for d, fill in ((a, None), (b, 0xCD)):
            if fill is not None:
                d.ws.fill_(fill)
            d.load_contributions(step, w.loss_scale0)
            d.step(d.args(step, w.loss_scale0, max_norm=0.5))
        ra, rb = a.result(), b.result()
        assert bytes(ra) == bytes(rb)
        for name in ("grad", "master", "m", "v", "slot"):
            assert np.array_equal(a.fetch(name), b.fetch(name)), name
    tab = abi.unit_table(0)
    res = torch.zeros(abi.RESULT_BYTES, dtype=torch.uint8, device="cuda")
    ws = torch.full((abi.zero_units_workspace_bytes(tab, 0),), 0xEE, dtype=torch.uint8,
                    device="cuda")
    args = a.args(1, 1.0)
    abi.zero_units_step(4, tab, 0, 0, args, ws, ws.numel(), res)
    torch.cuda.synchronize()
    r = abi.zero_step_result_t.from_buffer_copy(res.cpu().numpy().tobytes())
    assert r.own_q == 0 and r.norm == 0.0 and not r.skip and r.clip_coef == 1.0


@pytest.mark.parametrize("one_pass", [False, True])
def test_units_device_table_is_the_checked_one(one_pass):
    """Every zero_units_* call writes the host table it checked into the
    device table buffer before its kernels read it: a stale table left in that
    buffer (here a well-formed table of another rank's buffers) changes
    nothing, and the other buffers are never touched."""
    print(f"[units device table, one_pass={one_pass}]", flush=True)
    from zero_sharded_optimizer_rank_amd.units import DeviceUnits

    w = synth.TINY_FSDP
    kw = dict(one_pass=one_pass)
    a, ref, other = DeviceUnits(w, 1, **kw), DeviceUnits(w, 1, **kw), DeviceUnits(w, 1, **kw)
    for d in (a, ref, other):
        d.load_initial_state()
    before = {n: other.fetch(n).copy() for n in ("master", "m", "v", "slot")}

    def stale(dst, table):
        raw = bytes(table)[:dst.numel()]
        dst.copy_(torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(dst.device))
        torch.cuda.synchronize()

    for step in (1, 2):
        for d in (a, ref):
            d.load_contributions(step, w.loss_scale0)
        args = a.args(step, w.loss_scale0)
        stale(a.table_dev, other.table)
        if one_pass:
            stale(a.table2_dev, other.table2)
            a.step_1pass(args)
            ref.step_1pass(args)
        else:
            a.step(args)
            ref.step(args)
        ra, rr = a.result(), ref.result()
        assert bytes(ra) == bytes(rr), step
        if one_pass and not ra.skip:
            a.adopt()
            ref.adopt()
        for name in ("master", "m", "v", "slot") + (() if one_pass else ("grad",)):
            assert np.array_equal(_bits(a.fetch(name)), _bits(ref.fetch(name))), (step, name)
        for name, want in before.items():
            assert np.array_equal(_bits(other.fetch(name)), _bits(want)), (step, name)


def test_units_step_other_overflow_launches_no_update():
    """zero_units_step with another rank's overflow: the skip is certain, the
    update is not launched, the result word says skip and the state, slots
    and g of every unit match a phase-split step that ran the update kernel."""
    print("[units step with other_overflow]", flush=True)
    from zero_sharded_optimizer_rank_amd.units import DeviceUnits

    w = synth.TINY_FSDP
    a, b = DeviceUnits(w, 3), DeviceUnits(w, 3)
    for d in (a, b):
        d.load_initial_state()
        d.load_contributions(1, w.loss_scale0)
    before = {n: a.fetch(n).copy() for n in ("master", "m", "v", "slot")}
    args = a.args(1, w.loss_scale0, other_overflow=True)
    a.step(args)
    b.reduce_check(args)
    b.adam_apply(args)
    ra, rb = a.result(), b.result()
    assert ra.skip and bytes(ra) == bytes(rb)
    for name, want in before.items():
        assert np.array_equal(_bits(a.fetch(name)), _bits(want)), name
        assert np.array_equal(_bits(b.fetch(name)), _bits(want)), name
    assert np.array_equal(_bits(a.fetch("grad")), _bits(b.fetch("grad")))


@pytest.mark.parametrize("n", [4, 16])
def test_units_with_empty_units_all_ranks(n):
    """Units holding no elements (a tensor of size 0 as its own unit) between
    real ones, at N = 4 (one-chunk reduce) and N = 16 (deferred reduce): each
    empty unit still takes one reduce chunk that must write and count
    nothing; every rank bit for bit, with a skipped step."""
    print(f"[units with empty units N={n}]", flush=True)
    w = dataclasses.replace(
        synth.TINY_FSDP, name=f"units_empty_{n}", cfg_id=60 + n, world_size=n,
        tensors=(("z0", (0,)), ("a", (3000,)), ("z1", (0,)), ("b", (70_000,)), ("z2", (0,)),
                 ("c", (5,)), ("z3", (0,))),
        units=(0, 1, 2, 3, 4, 5, 6), parity_ranks=tuple(range(n)), inject_step=2)
    reports = run_units_all_ranks(w, 1.0)
    assert [r.skip for r in reports] == [s == 2 for s in range(1, w.steps + 1)]


def test_units_no_units():
    """n_units = 0: the step checks its arguments, launches only the finalize
    (Q = 0, nothing overflowed) and writes the result word."""
    import zero_sharded_optimizer_rank_amd.abi as abi

    print("[units: no units]", flush=True)
    dev = torch.device("cuda:0")
    table = abi.unit_table(0)
    table_dev = torch.empty(8, dtype=torch.uint8, device=dev)
    ws = torch.empty(max(abi.zero_units_workspace_bytes(table, 0), 16), dtype=torch.uint8,
                     device=dev)
    res = torch.full((abi.RESULT_BYTES,), 0xAB, dtype=torch.uint8, device=dev)
    args = abi.step_args(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                         max_grad_norm=1.0, loss_scale=1024.0, step=1, other_sq=0.25)
    abi.zero_units_step(4, table, table_dev, 0, args, ws, ws.numel(), res)
    torch.cuda.synchronize()
    r = abi.zero_step_result_t.from_buffer_copy(res.cpu().numpy().tobytes())
    fin = oracle.finalize(0, False, 1.0 / (4 * 1024.0), 1.0, other_sq=0.25)
    check_result(r, fin, 1)
    assert not r.skip
