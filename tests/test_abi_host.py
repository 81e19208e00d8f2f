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
        groups = -(-shard // 8)
        assert abi.zero_workspace_bytes(p) == 256 + 16 * (256 + max(1, -(-groups // 256)))
    assert abi.zero_workspace_bytes(abi.zero_plan_t(0, 1, 1, -1, -1)) == 0
    assert abi.RESULT_BYTES == 56
