"""The C ABI library on the CPU: it loads, exports every symbol the header
declares, and its host-only entry points (planner, state bytes, loss scaler,
argument checks) agree with the oracle.  No device work runs here."""
import os
import random
import re

import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _abi():
    from zero_sharded_optimizer_rank_amd import abi
    return abi


def _declared():
    names = []
    for f in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w \*]*?\b(zero_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    abi = _abi()
    names = _declared()
    assert sorted(names) == sorted(abi._SIGNATURES)
    so = abi.lib()
    for n in names:
        assert hasattr(so, n), n
        assert n in abi._SIGNATURES, n


def test_plan_matches_oracle_brute_force():
    abi = _abi()
    rnd = random.Random(3)
    for _ in range(400):
        numels = [rnd.randint(0, 50) for _ in range(rnd.randint(0, 7))]
        n = rnd.randint(1, 17)
        align = rnd.choice([1, 2, 8])
        plan, offs = abi.zero_plan(numels, n, align)
        want = oracle.plan(numels, n, align)
        assert (plan.psi, plan.world_size, plan.align, plan.shard, plan.psi_padded) == \
            (want.psi, want.world_size, want.align, want.shard, want.psi_padded)
        assert offs == want.offsets
        for r in range(n):
            assert abi.zero_plan_real(plan, r) == want.real(r)
            got = abi.zero_plan_segments(plan, numels, offs, r)
            assert got == [tuple(s) for s in oracle.segments(want, numels, r)]


def test_plan_workloads():
    abi = _abi()
    for w in synth.ALL:
        plan, offs = abi.zero_plan(w.numels, w.world_size)
        want = oracle.plan(w.numels, w.world_size)
        assert plan.shard == want.shard and offs == want.offsets


def test_state_bytes_matches_oracle():
    abi = _abi()
    for stage in range(4):
        for psi in (0.0, 1.5e9, 7.5e9, 1e12):
            for n in (1.0, 8.0, 64.0, 1024.0):
                for k in (12.0, 8.0):
                    assert abi.zero_state_bytes(stage, psi, n, k) == \
                        oracle.state_bytes(stage, psi, n, k)
    assert abi.zero_state_bytes(4, 1.0, 1.0, 12.0) == -1.0
    assert abi.zero_state_bytes(1, 1.0, 0.5, 12.0) == -1.0


def test_scaler_matches_oracle():
    abi = _abi()
    rnd = random.Random(5)
    s = abi.new_scaler(65536.0, growth_interval=7)
    scale, good, t = 65536.0, 0, 0
    for _ in range(300):
        skipped = rnd.random() < 0.2
        abi.zero_scaler_update(s, skipped)
        scale, good = oracle.scaler_update(scale, good, skipped, growth_interval=7)
        t += 0 if skipped else 1
        assert (s.scale, s.good_steps, s.t) == (scale, good, t)


def test_host_argument_errors():
    abi = _abi()
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_plan([3, -1], 2)
    assert e.value.code == abi.ZERO_EINVAL
    with pytest.raises(abi.ZeroError):
        abi.zero_plan([3], 2, 0)
    plan, offs = abi.zero_plan([10, 10, 10], 3)
    with pytest.raises(abi.ZeroError):
        abi.zero_plan_segments(plan, [10, 10, 10], offs, 3)
    assert abi.zero_plan_real(plan, 5) == -1
    for shard in (0, 1, 8, 2048, 2049, 10**9):
        p = abi.zero_plan_t(shard, 1, 1, shard, shard)
        quads = -(-shard // 4)  # one single-pass workgroup per 64 quads (the most partials)
        assert abi.zero_workspace_bytes(p) == 256 + 16 * (256 + max(1, -(-quads // 64)))
    assert abi.zero_workspace_bytes(abi.zero_plan_t(0, 1, 1, -1, -1)) == 0
    assert abi.RESULT_BYTES == 56


def test_plan_units_matches_oracle():
    abi = _abi()
    rnd = random.Random(9)
    for _ in range(300):
        t = rnd.randint(1, 8)
        numels = [rnd.randint(0, 40) for _ in range(t)]
        units, u = [], 0
        for i in range(t):
            if i > 0 and rnd.random() < 0.5:
                u += 1
            units.append(u)
        n = rnd.randint(1, 17)
        align = rnd.choice([1, 2, 8])
        plan, infos = abi.zero_plan_units(numels, units, n, align)
        want = oracle.plan_units(numels, units, n, align)
        assert (plan.n_units, plan.psi, plan.rank_shard) == (len(want.unit_psi), want.psi,
                                                               want.rank_shard)
        got = [(i.psi, i.shard, i.flat_offset, i.rank_offset) for i in infos]
        assert got == list(zip(want.unit_psi, want.unit_shard, want.unit_flat,
                               want.unit_rank_offset))
    for w in synth.UNIT_WORKLOADS:
        plan, infos = abi.zero_plan_units(w.numels, w.units, w.world_size)
        want = oracle.plan_units(w.numels, w.units, w.world_size)
        assert plan.rank_shard == want.rank_shard and len(infos) == len(want.unit_psi)
    with pytest.raises(abi.ZeroError):
        abi.zero_plan_units([1, 2], [0, 2], 2)  # units must be runs 0, 1, 2, ...
    with pytest.raises(abi.ZeroError):
        abi.zero_plan_units([1, 2], [1, 1], 2)


def test_units_prepare_layout_and_errors():
    abi = _abi()
    shards = [0, 5, 2048, 4096 * 3 + 1, 7]
    tab = abi.unit_table(len(shards))
    base = 1 << 40  # fake, aligned device addresses: nothing is launched here
    for i, s in enumerate(shards):
        t = tab[i]
        t.contrib = t.grad = t.master = t.m = t.v = base + i * (1 << 32)
        t.param16 = base + i * (1 << 32) + 6  # any 2-byte alignment is allowed
        t.ld = -(-max(s, 1) // 8) * 8
        t.shard = s
    b1, b2 = abi.zero_units_prepare(tab, len(shards))
    k1 = [max(1, -(-(-(-s // 4)) // 128)) for s in shards]  # 128 quads per reduce workgroup
    k2 = [-(-(-(-s // 4)) // 64) if s else 0 for s in shards]
    assert b1 == sum(k1) and b2 == sum(k2)
    assert [tab[i].reduce_block for i in range(len(shards))] == [sum(k1[:i]) for i in range(5)]
    assert [tab[i].adam_block for i in range(len(shards))] == [sum(k2[:i]) for i in range(5)]
    assert abi.zero_units_workspace_bytes(tab, len(shards)) == 256 + 16 * (256 + b1)
    tab[2].grad += 4
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_units_prepare(tab, len(shards))
    assert e.value.code == abi.ZERO_EALIGN
    tab[2].grad -= 4
    tab[3].ld = tab[3].shard - 1
    with pytest.raises(abi.ZeroError) as e:
        abi.zero_units_prepare(tab, len(shards))
    assert e.value.code == abi.ZERO_EINVAL
    tab[3].ld = -(-tab[3].shard // 8) * 8
    abi.zero_units_prepare(tab, len(shards))
    tab[4].adam_block += 1  # a stale table is refused
    assert abi.zero_units_workspace_bytes(tab, len(shards)) == 0


def test_one_pass_argument_checks_without_launching():
    """zero_reduce_adam_step_1pass rejects clipping and overlapping in / out
    state before anything reaches the GPU (the pointers here are never used)."""
    abi = _abi()
    S = 1000
    plan = abi.zero_plan_t(S, 2, 1, S, 2 * S)
    base = 1 << 32
    rows = [base, base + (1 << 20)]
    ins = [base + (2 << 20), base + (3 << 20), base + (4 << 20)]
    outs = [base + (5 << 20), base + (6 << 20), base + (7 << 20)]
    slot = base + (8 << 20)
    ws_bytes = abi.zero_workspace_bytes(plan)
    ws, res = base + (9 << 20), base + (10 << 20)

    def call(i, o, sl, clip=0.0, wsb=ws_bytes):
        args = abi.step_args(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                             max_grad_norm=clip, loss_scale=1.0, step=1)
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_reduce_adam_step_1pass(plan, 0, rows, *i, *o, sl, ws, wsb, args, res, 0)
        return e.value.code

    assert call(ins, outs, slot, clip=1.0) == abi.ZERO_EINVAL
    assert call(ins, [ins[0], outs[1], outs[2]], slot) == abi.ZERO_EINVAL       # out = in
    assert call(ins, [outs[0], ins[2] + 4 * S - 16, outs[2]], slot) == abi.ZERO_EINVAL  # tail
    assert call(ins, [outs[0], outs[0] + 16, outs[2]], slot) == abi.ZERO_EINVAL  # outs overlap
    assert call(ins, outs, outs[2] + 4 * S - 2) == abi.ZERO_EINVAL              # slot overlaps v
    assert call(ins, outs, ins[1] + 2) == abi.ZERO_EINVAL                       # slot in m_in
    assert call(ins, [outs[0] + 4, outs[1], outs[2]], slot) == abi.ZERO_EALIGN
    assert call(ins, outs, slot, wsb=16) == abi.ZERO_ENOSPC


def test_units_one_pass_argument_checks_without_launching():
    """zero_units_step_1pass rejects clipping, a shard that differs between
    the two tables and out buffers that overlap the unit's input state,
    before anything reaches the GPU (the pointers are never used)."""
    abi = _abi()
    base = 1 << 32
    shards = [1000, 24, 0]

    def table(state_at):
        t = abi.unit_table(len(shards))
        for u, s in enumerate(shards):
            x = t[u]
            o = base + (u << 24)
            x.contrib, x.ld, x.grad = o, 1024, o + (1 << 20)
            x.master = state_at + (u << 24)
            x.m, x.v = x.master + (1 << 16), x.master + (2 << 16)
            x.param16 = x.master + (3 << 16)
            x.shard = s
        abi.zero_units_prepare(t, len(shards))
        return t

    ins, outs = table(base + (1 << 30)), table(base + (2 << 30))
    ws_bytes = abi.zero_units_workspace_bytes(ins, len(shards))
    ws, res, dev_in, dev_out = base + (3 << 30), base + (3 << 30) + (1 << 24), base, base + 64

    def call(o, clip=0.0, n_units=len(shards)):
        args = abi.step_args(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                             max_grad_norm=clip, loss_scale=1.0, step=1)
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_units_step_1pass(2, ins, dev_in, o, dev_out, n_units, args, ws, ws_bytes,
                                      res, 0)
        return e.value.code

    assert call(outs, clip=1.0) == abi.ZERO_EINVAL
    other = table(base + (2 << 30))
    other[1].shard = 32
    abi.zero_units_prepare(other, len(shards))
    assert call(other) == abi.ZERO_EINVAL                      # shard differs
    alias = table(base + (2 << 30))
    alias[0].v = ins[0].m                                      # out v over in m
    assert call(alias) == abi.ZERO_EINVAL
    alias = table(base + (2 << 30))
    alias[1].param16 = alias[1].master + 4                      # slot over out master
    assert call(alias) == abi.ZERO_EINVAL
    unprepared = table(base + (2 << 30))
    unprepared[2].reduce_block += 1
    assert call(unprepared) == abi.ZERO_EINVAL


def test_slot_restore_argument_checks_without_launching():
    """zero_slot_restore rejects a bad rank, a NULL or misaligned buffer and a
    slot that overlaps the master before anything reaches the GPU."""
    abi = _abi()
    S = 1000
    plan = abi.zero_plan_t(S, 2, 1, S, 2 * S)
    base = 1 << 32
    master, slot, res = base, base + (1 << 20), base + (2 << 20)
    for f in (abi.zero_slot_restore, abi.zero_slot_restore_bf16):
        for args, code in (((plan, 2, master, slot, res), abi.ZERO_EINVAL),
                           ((plan, 0, 0, slot, res), abi.ZERO_EINVAL),
                           ((plan, 0, master, slot, 0), abi.ZERO_EINVAL),
                           ((plan, 0, master + 2, slot, res), abi.ZERO_EALIGN),
                           ((plan, 0, master, slot + 1, res), abi.ZERO_EALIGN),
                           ((plan, 0, master, master + 4 * S - 2, res), abi.ZERO_EINVAL)):
            with pytest.raises(abi.ZeroError) as e:
                f(*args)
            assert e.value.code == code, (f.__name__, args)


def test_noalloc_step_argument_checks_without_launching():
    """zero_reduce_adam_step_noalloc rejects a shard above its scratch limit,
    a bad rank and NULL or misaligned buffers before it touches the GPU (the
    pointers are never used, and no device exists here)."""
    abi = _abi()
    base = 1 << 32
    rows = [base, base + (1 << 20)]
    master, m, v, slot, grad, res = (base + (k << 20) for k in range(2, 8))
    args = abi.step_args(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                         max_grad_norm=1.0, loss_scale=1.0, step=1)

    def call(plan, rank=0, r=rows, g=grad, sl=slot, rs=res):
        with pytest.raises(abi.ZeroError) as e:
            abi.zero_reduce_adam_step_noalloc(plan, rank, r, master, m, v, sl, g, args, rs, 0)
        return e.value.code, str(e.value)

    big = abi.ZERO_NOALLOC_MAX_SHARD + 8
    code, msg = call(abi.zero_plan_t(2 * big, 2, 1, big, 2 * big))
    assert code == abi.ZERO_ENOSPC and "scratch" in msg
    S = 1000
    plan = abi.zero_plan_t(S, 2, 1, S, 2 * S)
    assert call(plan, rank=2)[0] == abi.ZERO_EINVAL
    assert call(plan, r=[base, 0])[0] == abi.ZERO_EINVAL
    assert call(plan, r=[base, base + 8])[0] == abi.ZERO_EALIGN
    assert call(plan, g=0)[0] == abi.ZERO_EINVAL
    assert call(plan, g=grad + 4)[0] == abi.ZERO_EALIGN
    assert call(plan, sl=slot + 1)[0] == abi.ZERO_EALIGN
    assert call(plan, rs=0)[0] == abi.ZERO_EINVAL
