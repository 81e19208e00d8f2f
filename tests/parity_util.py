"""Helpers for the GPU parity tests: run a workload window on the GPU through
the C ABI and on the CPU through the oracle, on the same seeded inputs, and
compare.

Acceptance bar: the reduced gradient, the exact squared-norm integer, the
fp64 norm values, the clip coefficient and the overflow / skip decisions are
bit-exact; fp32 master, m and v are within 1e-6 relative error with zeros
matching exactly; the fp16 slot is within 1 ulp.  Bitwise mismatch counts are
reported and also required to be zero, since both sides run the same rounded
fp32 sequence.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

import oracle
import synth
from oracle import run as orun

F32 = np.float32


def f16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """ulp distance between fp16 bit patterns (ordered-integer mapping)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def max_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    g = got.astype(np.float64)
    w = want.astype(np.float64)
    zero = w == 0
    if np.any(g[zero] != 0):
        return float("inf")
    nz = ~zero
    if not nz.any():
        return 0.0
    return float(np.max(np.abs(g[nz] - w[nz]) / np.abs(w[nz])))


@dataclass
class StepReport:
    step: int
    skip: bool
    coef: float
    mismatches: dict = field(default_factory=dict)
    max_rel: dict = field(default_factory=dict)


def compare_state(rep: StepReport, name: str, got: np.ndarray, want: np.ndarray):
    if name == "slot":
        d = f16_ulp_diff(got, want.view(np.uint16) if want.dtype != np.uint16 else want)
        rep.max_rel[name] = float(d.max()) if d.size else 0.0
        rep.mismatches[name] = int(np.count_nonzero(d))
        assert rep.max_rel[name] <= 1, (rep.step, name, rep.max_rel[name])
    else:
        rep.max_rel[name] = max_rel_err(got, want)
        rep.mismatches[name] = int(np.count_nonzero(got.view(np.uint32) != want.view(np.uint32)))
        assert rep.max_rel[name] <= 1e-6, (rep.step, name, rep.max_rel[name])


def check_result(res, fin: oracle.FinalizeResult, step: int):
    assert res.own_q == fin.own_q, (step, res.own_q, fin.own_q)
    assert res.own_sq == fin.own_sq, (step, res.own_sq, fin.own_sq)
    assert res.total_sq == fin.total_sq, (step, res.total_sq, fin.total_sq)
    assert res.norm == fin.norm, (step, res.norm, fin.norm)
    assert np.float32(res.clip_coef) == fin.coef, (step, res.clip_coef, fin.coef)
    assert bool(res.overflow) == fin.overflow and bool(res.skip) == fin.skip, step


def other_overflow_at(w: synth.Workload, step: int, flat_begin: int, count: int) -> bool:
    """True if the workload's injected inf at `step` lies outside this window
    (so another rank, not this one, reports the overflow)."""
    site = synth.inject_site(w, step)
    if site is None:
        return False
    return not (flat_begin <= site[1] < flat_begin + count)


def run_window(w: synth.Workload, rank: int, begin: int, count: int, steps: Optional[int] = None,
               fused: bool = True, strict: bool = True,
               ws_fill: Optional[int] = None, offload: Optional[dict] = None,
               one_pass: bool = False, in_place_slot: bool = False,
               stream=None) -> List[StepReport]:
    """Run `steps` steps of the workload on one window of rank's shard on the
    GPU and in the oracle; compare every step.  With `offload` (OffloadShard
    keyword arguments) the update runs in the offload form: host state, PCIe
    pipeline.  With `one_pass` (unclipped workloads) each step is
    zero_reduce_adam_step_1pass into the second state set, adopted only when
    the step was not skipped; no gradient is written, so none is compared.
    With `in_place_slot` as well, the pass writes the live slot and
    zero_slot_restore follows every step.  `stream`: the torch stream every
    call of the window runs on (default: the thread's current stream)."""
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard, OffloadShard

    steps = w.steps if steps is None else steps
    if offload is not None:
        dev = OffloadShard(w, rank, begin, count, **offload)
    else:
        dev = DeviceShard(w, rank, begin, count, one_pass=one_pass, stream=stream)
    dev.load_initial_state()
    p = orun.workload_plan(w)
    flat_begin = rank * p.shard + begin
    assert flat_begin == dev.flat_begin
    op, om, ov, oh = orun.initial_state(w, p, rank, begin, count)
    oh = oh.view(np.uint16)
    other_sq = w.other_sq(p.real(rank)) if w.other_ranks_from_config else 0.0
    scaler = abi.new_scaler(w.loss_scale0)
    o_scale, o_good, o_t = w.loss_scale0, 0, 0
    reports = []
    for step in range(1, steps + 1):
        assert scaler.scale == o_scale
        ovf_other = other_overflow_at(w, step, flat_begin, count)
        # GPU
        if ws_fill is not None:
            dev.ws.fill_(ws_fill)  # the workspace needs no initialisation
        dev.load_contributions(step, scaler.scale)
        args = dev.args(scaler.t + 1, scaler.scale, other_sq=other_sq, other_overflow=ovf_other)
        if one_pass:
            dev.step_1pass(args, in_place_slot=in_place_slot)
            if in_place_slot:
                dev.restore_slot()
        elif fused:
            dev.step(args)
        else:
            dev.reduce_check(args)
            dev.adam_apply(args)
        res = dev.result()
        if one_pass and not res.skip:
            dev.adopt(swap_slot=not in_place_slot)
        # oracle
        c = orun.shard_contrib(w, p, rank, step, o_scale, begin, count)
        sc = oracle.step_scalars(w.lr, w.betas[0], w.betas[1], w.eps, w.weight_decay, o_t + 1,
                                 w.world_size, o_scale)
        step_fn = oracle.shard_step_bf16 if w.dtype == "bf16" else oracle.shard_step
        out = step_fn(c, op, om, ov, oh, sc, w.max_grad_norm, other_sq=other_sq,
                      other_overflow=ovf_other)
        check_result(res, out.fin, step)
        rep = StepReport(step, out.fin.skip, float(out.fin.coef))
        if not one_pass:
            g = dev.fetch("grad")
            rep.mismatches["grad"] = int(np.count_nonzero(g.view(np.uint32) !=
                                                          out.g.view(np.uint32)))
            assert rep.mismatches["grad"] == 0, (step, "grad")
        op, om, ov = out.p, out.m, out.v
        oh = out.h.view(np.uint16)
        for name, want in (("master", op), ("m", om), ("v", ov), ("slot", oh)):
            compare_state(rep, name, dev.fetch(name), want)
        if strict:
            assert all(v == 0 for v in rep.mismatches.values()), (step, rep.mismatches)
        assert dev.guards_intact(), step
        reports.append(rep)
        abi.zero_scaler_update(scaler, bool(res.skip))
        o_scale, o_good = oracle.scaler_update(o_scale, o_good, out.fin.skip)
        if not out.fin.skip:
            o_t += 1
        assert scaler.t == o_t
    return reports


def run_units_all_ranks(w: synth.Workload, max_norm: Optional[float] = None,
                        one_pass: bool = False, in_place_slot: bool = False,
                        stream=None) -> List[StepReport]:
    """Every rank of a unit layout on the GPU (zero_units_* through DeviceUnits)
    and in the oracle, all steps, with the exact all-reduce of the squared-norm
    integers and overflow flags between the ranks; every rank's g, result and
    state compared bit for bit.  With `one_pass` (no clipping) every rank runs
    zero_units_step_1pass first, the all-reduce and zero_finalize follow, and
    each rank adopts its new set unless the step was skipped; no g is written
    or compared.  With `in_place_slot` the pass writes the live unit slots and
    zero_units_slot_restore follows the finalize.  Returns rank 0's reports."""
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.units import DeviceUnits

    max_norm = w.max_grad_norm if max_norm is None else max_norm
    n = w.world_size
    up = orun.workload_unit_plan(w)
    devs = [DeviceUnits(w, r, one_pass=one_pass, in_place_slot=in_place_slot, stream=stream)
            for r in range(n)]
    for d in devs:
        d.load_initial_state()
    ost = [list(orun.unit_rank_initial_state(w, up, r)) for r in range(n)]
    ost = [[s[0], s[1], s[2], s[3].view(np.uint16)] for s in ost]
    scaler = abi.new_scaler(w.loss_scale0)
    o_scale, o_good, o_t = w.loss_scale0, 0, 0
    flat_plan = abi.zero_plan_t(0, n, 1, 0, 0)
    reports = []
    for step in range(1, w.steps + 1):
        for d in devs:
            d.load_contributions(step, scaler.scale)
        base = devs[0].args(scaler.t + 1, scaler.scale, max_norm=max_norm)
        for d in devs:
            if one_pass:
                d.step_1pass(base)
            else:
                d.reduce_check(base)
        rs = [d.result() for d in devs]
        for r, d in enumerate(devs):
            a = d.args(scaler.t + 1, scaler.scale, max_norm=max_norm,
                       other_q=sum(rs[x].own_q for x in range(n) if x != r),
                       other_overflow=any(rs[x].overflow for x in range(n) if x != r))
            abi.zero_finalize(flat_plan, a, d.res, d.stream)
            if not one_pass:
                d.adam_apply(a)
                continue
            if in_place_slot:
                d.restore_slot()
            if not d.result().skip:
                d.adopt()
        # oracle
        sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, o_t + 1, n, o_scale)
        accs = [oracle.reduce_contributions(orun.unit_rank_contrib(w, up, r, step, o_scale))
                for r in range(n)]
        qs = [oracle.exact_sq_units(x) for x in accs]
        bads = [oracle.nonfinite(x) for x in accs]
        skipped = None
        for r, d in enumerate(devs):
            fin = oracle.finalize(qs[r], bads[r], sc.inv64, max_norm,
                                  other_q=sum(qs) - qs[r],
                                  other_overflow=any(bads[x] for x in range(n) if x != r))
            check_result(d.result(), fin, step)
            skipped = fin.skip
            g = oracle.unscale(accs[r], sc.inv32)
            if not one_pass:
                assert np.array_equal(d.fetch("grad").view(np.uint32), g.view(np.uint32)), \
                    (step, r)
            if not fin.skip:
                p, m, v, h = oracle.adam_apply(g, ost[r][0], ost[r][1], ost[r][2], sc, fin.coef)
                ost[r] = [p, m, v, h.view(np.uint16)]
            rep = StepReport(step, fin.skip, float(fin.coef))
            for name, k in (("master", 0), ("m", 1), ("v", 2), ("slot", 3)):
                compare_state(rep, name, d.fetch(name), ost[r][k])
            assert all(x == 0 for x in rep.mismatches.values()), (step, r, rep.mismatches)
            assert d.guards_intact(), (step, r)
            if r == 0:
                reports.append(rep)
        abi.zero_scaler_update(scaler, skipped)
        o_scale, o_good = oracle.scaler_update(o_scale, o_good, skipped)
        o_t += 0 if skipped else 1
    return reports
