"""The device step captured in a HIP graph: replays give the same bits as the
same calls made eagerly (the step launches kernels only: no memset, no host
synchronisation, and the workspace needs no initialisation between calls)."""
import numpy as np
import pytest

import synth
from oracle import run as orun

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _snapshot(d):
    d.stream.synchronize()
    out = {x: d.fetch(x).copy() for x in ("grad", "master", "m", "v", "slot")}
    out["res"] = d.res.cpu().numpy().copy()
    return out


@pytest.mark.parametrize("wname", ["llama3_8b", "llama3_8b_bf16"])
def test_step_graph_replays_match_eager(wname):
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard

    w = synth.BY_NAME[wname]
    p = orun.workload_plan(w)
    rank, begin, count = 1, 333, 200_003
    other_sq = w.other_sq(p.real(rank))
    print(f"[graph {wname}]", flush=True)
    s_eager, s_graph = torch.cuda.Stream(), torch.cuda.Stream()
    de = DeviceShard(w, rank, begin, count, stream=s_eager)
    dg = DeviceShard(w, rank, begin, count, stream=s_graph)
    for d in (de, dg):
        d.load_initial_state()
        d.load_contributions(1, w.loss_scale0)
    args = de.args(1, w.loss_scale0, other_sq=other_sq)
    eager = []
    for _ in range(3):
        de.step(args)
        eager.append(_snapshot(de))
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s_graph):
        dg.step(args)
    torch.cuda.synchronize()
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(dg)
        # unrelated eager work between replays
        junk = torch.randn(1 << 20, device="cuda").sum().item()
        assert np.isfinite(junk)
        for k in got:
            a, b = got[k], eager[i][k]
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (i, k)
        assert dg.guards_intact()


def test_onepass_graph_replays_match_eager():
    """Two single-pass steps captured as one graph (set 0 -> set 1 -> set 0)
    replay to the same bits as the same calls made eagerly."""
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard

    w = synth.GPT2
    rank, begin, count = 1, 777, 200_003
    print("[graph one pass]", flush=True)
    s_eager, s_graph = torch.cuda.Stream(), torch.cuda.Stream()
    de = DeviceShard(w, rank, begin, count, stream=s_eager, one_pass=True)
    dg = DeviceShard(w, rank, begin, count, stream=s_graph, one_pass=True)
    for d in (de, dg):
        d.load_initial_state()
        d.load_contributions(1, w.loss_scale0)
    args = de.args(1, w.loss_scale0)

    def two_steps(d):
        for _ in range(2):
            d.step_1pass(args)
            d.adopt()

    def snap(d):
        d.stream.synchronize()
        out = {x: d.fetch(x).copy() for x in ("master", "m", "v", "slot")}
        out["res"] = d.res.cpu().numpy().copy()
        return out

    eager = []
    for _ in range(3):
        two_steps(de)
        eager.append(snap(de))
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s_graph):
        two_steps(dg)
    torch.cuda.synchronize()
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        got = snap(dg)
        junk = torch.randn(1 << 20, device="cuda").sum().item()
        assert np.isfinite(junk)
        for k in got:
            assert np.array_equal(got[k].view(np.uint8), eager[i][k].view(np.uint8)), (i, k)
        assert dg.guards_intact()


def test_onepass_in_place_slot_graph_replays_match_eager():
    """A single pass writing the live slot plus zero_slot_restore, captured
    twice as one graph (set 0 -> set 1 -> set 0), replays to the same bits as
    eager calls; the restore reads the skip flag on the device."""
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard

    w = synth.GPT2
    rank, begin, count = 1, 777, 200_003
    print("[graph one pass in place]", flush=True)
    s_eager, s_graph = torch.cuda.Stream(), torch.cuda.Stream()
    de = DeviceShard(w, rank, begin, count, stream=s_eager, one_pass=True)
    dg = DeviceShard(w, rank, begin, count, stream=s_graph, one_pass=True)
    for d in (de, dg):
        d.load_initial_state()
        d.load_contributions(1, w.loss_scale0)
    args = de.args(1, w.loss_scale0)

    def two_steps(d):
        for _ in range(2):
            d.step_1pass(args, in_place_slot=True)
            d.restore_slot()
            d.adopt(swap_slot=False)

    def snap(d):
        d.stream.synchronize()
        out = {x: d.fetch(x).copy() for x in ("master", "m", "v", "slot")}
        out["res"] = d.res.cpu().numpy().copy()
        return out

    eager = []
    for _ in range(3):
        two_steps(de)
        eager.append(snap(de))
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s_graph):
        two_steps(dg)
    torch.cuda.synchronize()
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        got = snap(dg)
        junk = torch.randn(1 << 20, device="cuda").sum().item()
        assert np.isfinite(junk)
        for k in got:
            assert np.array_equal(got[k].view(np.uint8), eager[i][k].view(np.uint8)), (i, k)
        assert dg.guards_intact()


def test_onepass_in_place_slot_skipped_step_graph():
    """A skipped single pass that wrote the live slot, captured with its
    zero_slot_restore: every replay leaves the state untouched and the slot
    recast from the unchanged master, the same bits as the eager calls (the
    restore's rewrite branch runs from the graph)."""
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard

    w = synth.GPT2
    rank, begin, count = 1, 777, 200_003
    print("[graph one pass in place, skipped step]", flush=True)
    s_eager, s_graph = torch.cuda.Stream(), torch.cuda.Stream()
    de = DeviceShard(w, rank, begin, count, stream=s_eager, one_pass=True)
    dg = DeviceShard(w, rank, begin, count, stream=s_graph, one_pass=True)
    for d in (de, dg):
        d.load_initial_state()
        d.load_contributions(1, w.loss_scale0)
    args = de.args(1, w.loss_scale0, other_overflow=True)  # another rank overflowed

    def skipped_step(d):  # never adopted: the step is skipped
        d.step_1pass(args, in_place_slot=True)
        d.restore_slot()

    def snap(d):
        d.stream.synchronize()
        out = {x: d.fetch(x).copy() for x in ("master", "m", "v", "slot")}
        out["res"] = d.res.cpu().numpy().copy()
        return out

    start = snap(de)
    eager = []
    for _ in range(3):
        skipped_step(de)
        eager.append(snap(de))
        assert de.result().skip
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s_graph):
        skipped_step(dg)
    torch.cuda.synchronize()
    for i in range(3):
        dg.slot.fill_(0x1234)  # the restore must rewrite every element
        graph.replay()
        torch.cuda.synchronize()
        got = snap(dg)
        junk = torch.randn(1 << 20, device="cuda").sum().item()
        assert np.isfinite(junk)
        for k in got:
            assert np.array_equal(got[k].view(np.uint8), eager[i][k].view(np.uint8)), (i, k)
        for k in ("master", "m", "v", "slot"):
            assert np.array_equal(got[k].view(np.uint8), start[k].view(np.uint8)), (i, k)
        assert np.array_equal(got["slot"], got["master"].astype(np.float16).view(np.uint16))
        assert dg.result().skip and dg.guards_intact()


def test_noalloc_step_graph_replays_match_step_with_workspace():
    """zero_reduce_adam_step_noalloc captured in a HIP graph (its scratch
    address resolved by one earlier call on the device): three replays give
    the bits of three eager zero_reduce_adam_step calls with a workspace."""
    from zero_sharded_optimizer_rank_amd import abi
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard

    w = synth.LLAMA3_8B
    p = orun.workload_plan(w)
    rank, begin, count = 1, 333, 200_003
    other_sq = w.other_sq(p.real(rank))
    print("[graph noalloc]", flush=True)
    warm = DeviceShard(synth.TINY, 0, 0, 1000)  # first call on the device: resolves the scratch
    warm.load_initial_state()
    warm.load_contributions(1, synth.TINY.loss_scale0)

    def noalloc(d, args):
        abi.zero_reduce_adam_step_noalloc(d.plan, d.rank, d.contrib_ptrs(), d.master, d.m, d.v,
                                          d.slot_ptr(), d.grad, args, d.res, d.stream)

    noalloc(warm, warm.args(1, synth.TINY.loss_scale0))
    torch.cuda.synchronize()
    s_eager, s_graph = torch.cuda.Stream(), torch.cuda.Stream()
    de = DeviceShard(w, rank, begin, count, stream=s_eager)
    dg = DeviceShard(w, rank, begin, count, stream=s_graph)
    for d in (de, dg):
        d.load_initial_state()
        d.load_contributions(1, w.loss_scale0)
    args = de.args(1, w.loss_scale0, other_sq=other_sq)
    eager = []
    for _ in range(3):
        de.step(args)
        eager.append(_snapshot(de))
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s_graph):
        noalloc(dg, args)
    torch.cuda.synchronize()
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(dg)
        junk = torch.randn(1 << 20, device="cuda").sum().item()
        assert np.isfinite(junk)
        for k in got:
            assert np.array_equal(got[k].view(np.uint8), eager[i][k].view(np.uint8)), (i, k)
        assert dg.guards_intact()
