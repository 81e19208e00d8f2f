"""Checkpoint and resume: the step's whole state is plain buffers (fp32
master, m, v, the 16-bit slot) and host scalars (Adam step t, loss scale,
clean-step count).  Four steps in one go must equal two steps, a save to
files, a fresh shard restored from them, and two more steps, bit for bit,
through a skipped step and a loss-scale change."""
import dataclasses
import json

import numpy as np
import pytest

import synth
from oracle import run as orun
from parity_util import other_overflow_at

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


STATE = ("master", "m", "v", "slot")


def _step(dev, scaler, step, other_sq, one_pass):
    import zero_sharded_optimizer_rank_amd.abi as abi
    w = dev.w
    dev.load_contributions(step, scaler.scale)
    args = dev.args(scaler.t + 1, scaler.scale, other_sq=other_sq,
                    other_overflow=other_overflow_at(w, step, dev.flat_begin, dev.count))
    if one_pass:
        dev.step_1pass(args)
    else:
        dev.step(args)
    res = dev.result()
    if one_pass and not res.skip:
        dev.adopt()
    abi.zero_scaler_update(scaler, bool(res.skip))
    return bool(res.skip)


@pytest.mark.parametrize("wname,one_pass", [("llama3_8b", False), ("gpt2_1p5b", True)])
def test_checkpoint_resume_bitwise(tmp_path, wname, one_pass):
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard

    w = synth.BY_NAME[wname]
    if w.inject_step is None:  # a skip inside the run for the unclipped workload too
        w = dataclasses.replace(w, inject_step=2)
    p = orun.workload_plan(w)
    rank = 0
    e = synth.inject_site(w, w.inject_step)[1]
    count = 300_001
    begin = min(max(0, e - 150_000), p.shard - count)
    other_sq = w.other_sq(p.real(rank)) if w.other_ranks_from_config else 0.0
    print(f"[checkpoint {wname} one_pass={one_pass}]", flush=True)

    # four steps in one go
    a = DeviceShard(w, rank, begin, count, one_pass=one_pass)
    a.load_initial_state()
    sa = abi.new_scaler(w.loss_scale0)
    skips = [_step(a, sa, s, other_sq, one_pass) for s in (1, 2, 3, 4)]
    assert skips == [False, True, False, False]
    want = {x: a.fetch(x).copy() for x in STATE}
    del a

    # two steps, save, restore into a fresh shard, two more steps
    b = DeviceShard(w, rank, begin, count, one_pass=one_pass)
    b.load_initial_state()
    sb = abi.new_scaler(w.loss_scale0)
    for s in (1, 2):
        _step(b, sb, s, other_sq, one_pass)
    np.savez(tmp_path / "state.npz", **{x: b.fetch(x) for x in STATE})
    (tmp_path / "scalars.json").write_text(json.dumps(
        {"scale": sb.scale, "good_steps": sb.good_steps, "t": sb.t}))
    del b

    c = DeviceShard(w, rank, begin, count, one_pass=one_pass)
    saved = np.load(tmp_path / "state.npz")
    for x in ("master", "m", "v"):
        getattr(c, x)[:count].copy_(torch.from_numpy(saved[x]))
    c.slot.copy_(torch.from_numpy(saved["slot"].view(np.int16)))
    sc = json.loads((tmp_path / "scalars.json").read_text())
    sr = abi.new_scaler(sc["scale"])
    sr.good_steps, sr.t = sc["good_steps"], sc["t"]
    for s in (3, 4):
        _step(c, sr, s, other_sq, one_pass)
    for x in STATE:
        assert np.array_equal(c.fetch(x).view(np.uint8), want[x].view(np.uint8)), x
    assert (sr.scale, sr.good_steps, sr.t) == (sa.scale, sa.good_steps, sa.t)
    assert c.guards_intact()
