"""Oracle drivers over the synthetic workloads (test infrastructure only).

These helpers feed the oracle's step functions with the seeded inputs of
``synth`` and simulate the other data-parallel ranks on one host.  They add no
arithmetic of their own beyond exact integer sums.
"""
from __future__ import annotations

from typing import Dict, List, NamedTuple, Sequence

import numpy as np

import synth

from .zero_oracle import (
    FinalizeResult, Plan, exact_sq_units, f32_to_bf16, finalize, nonfinite, plan, reduce_contributions,
    adam_apply, scaler_update, step_scalars, unscale,
)


def workload_plan(w: synth.Workload, align: int = 1) -> Plan:
    return plan(w.numels, w.world_size, align)


def shard_contrib(w: synth.Workload, p: Plan, rank: int, step: int, loss_scale: float,
                  begin: int = 0, count: int | None = None) -> np.ndarray:
    """The owner ``rank``'s slice [begin, begin+count) of every rank's flat
    fp16 gradient at ``step``: [N, count] uint16 bit patterns."""
    if count is None:
        count = p.shard - begin
    out = np.empty((w.world_size, count), dtype=np.uint16)
    for q in range(w.world_size):
        synth.contributions(w, step, q, rank * p.shard + begin, count, loss_scale, out=out[q])
    return out


def initial_state(w: synth.Workload, p: Plan, rank: int, begin: int = 0, count: int | None = None):
    """fp32 master, m = 0, v = 0 and the fp16 (or bf16, by the workload's
    format) copy of the master for a shard range."""
    if count is None:
        count = p.shard - begin
    master = synth.masters(w, rank * p.shard + begin, count)
    z = np.zeros(count, np.float32)
    return master, z, z.copy(), half_copy(w, master)


def half_copy(w: synth.Workload, master: np.ndarray) -> np.ndarray:
    """The slot's initial 16-bit copy of fp32 masters, as bit patterns."""
    if w.dtype == "bf16":
        return f32_to_bf16(master)
    return master.astype(np.float16).view(np.uint16)


class RankState(NamedTuple):
    p: np.ndarray
    m: np.ndarray
    v: np.ndarray
    h: np.ndarray


class StepRecord(NamedTuple):
    step: int
    t: int  # Adam step index used (1-based) if applied
    loss_scale: float
    fin: Dict[int, FinalizeResult]
    g: Dict[int, np.ndarray]
    after: Dict[int, RankState]


def run_all_ranks(w: synth.Workload, ranks: Sequence[int] | None = None, steps: int | None = None,
                  max_norm: float | None = None, p: Plan | None = None) -> List[StepRecord]:
    """Run the workload's steps for every rank on the host, with an exact
    all-reduce of the squared-norm integers and of the overflow flags between
    the reduce and the update (the global clip and skip).  Small workloads only."""
    p = p or workload_plan(w)
    n = w.world_size
    ranks = list(range(n)) if ranks is None else list(ranks)
    steps = w.steps if steps is None else steps
    max_norm = w.max_grad_norm if max_norm is None else max_norm
    state = {r: RankState(*initial_state(w, p, r)) for r in range(n)}
    scale, good, t = w.loss_scale0, 0, 0
    records = []
    for step in range(1, steps + 1):
        sc = step_scalars(w.lr, w.betas[0], w.betas[1], w.eps, w.weight_decay, t + 1, n, scale)
        accs = {r: reduce_contributions(shard_contrib(w, p, r, step, scale)) for r in range(n)}
        qs = {r: exact_sq_units(a) for r, a in accs.items()}
        ovf = {r: nonfinite(a) for r, a in accs.items()}
        fins, gs = {}, {}
        for r in range(n):
            fins[r] = finalize(qs[r], ovf[r], sc.inv64, max_norm,
                               other_q=sum(qs[x] for x in range(n) if x != r),
                               other_overflow=any(ovf[x] for x in range(n) if x != r))
            gs[r] = unscale(accs[r], sc.inv32)
        skipped = fins[0].skip
        assert all(f.skip == skipped and f.coef == fins[0].coef for f in fins.values())
        if not skipped:
            for r in range(n):
                s = state[r]
                state[r] = RankState(*adam_apply(gs[r], s.p, s.m, s.v, sc, fins[r].coef))
            t += 1
        records.append(StepRecord(step, t, scale, {r: fins[r] for r in ranks},
                                  {r: gs[r] for r in ranks}, {r: state[r] for r in ranks}))
        scale, good = scaler_update(scale, good, skipped)
    return records


# --------------------------------------------------------------------------
# FSDP / ZeRO-3 unit layouts.
def workload_unit_plan(w: synth.Workload, align: int = 1):
    from .zero_oracle import plan_units
    return plan_units(w.numels, w.units, w.world_size, align)


def _runs(idx: np.ndarray):
    """Split model indexes (-1 = padding) into runs (pos, start, length) of
    consecutive real indexes."""
    real = idx >= 0
    if not real.any():
        return []
    # a run starts at a real index whose predecessor is not the index minus one
    prev = np.concatenate(([-2], idx[:-1]))
    starts = np.flatnonzero(real & (idx != prev + 1))
    ends = np.flatnonzero(real & np.concatenate((idx[1:] != idx[:-1] + 1, [True])))
    return [(int(a), int(idx[a]), int(b - a + 1)) for a, b in zip(starts, ends)]


def gather_contrib(w: synth.Workload, step: int, q: int, idx: np.ndarray, loss_scale: float,
                   out: np.ndarray | None = None) -> np.ndarray:
    """Rank q's scaled fp16 gradient at model indexes idx (-1: padding, +0)."""
    out = np.zeros(idx.size, dtype=np.uint16) if out is None else out
    out[:] = 0
    for pos, start, length in _runs(idx):
        synth.contributions(w, step, q, start, length, loss_scale, out=out[pos:pos + length])
    return out


def unit_rank_contrib(w: synth.Workload, up, rank: int, step: int, loss_scale: float,
                      begin: int = 0, count: int | None = None) -> np.ndarray:
    """[N, count] contributions for elements [begin, begin+count) of rank's
    concatenated unit shards."""
    from .zero_oracle import unit_shard_index
    idx = unit_shard_index(up, rank)
    count = idx.size - begin if count is None else count
    idx = idx[begin:begin + count]
    out = np.empty((w.world_size, count), dtype=np.uint16)
    for q in range(w.world_size):
        gather_contrib(w, step, q, idx, loss_scale, out=out[q])
    return out


def unit_rank_initial_state(w: synth.Workload, up, rank: int):
    """Initial master (+0 on padding), m, v and fp16 copy of rank's
    concatenated unit shards."""
    from .zero_oracle import unit_shard_index
    idx = unit_shard_index(up, rank)
    master = np.zeros(idx.size, dtype=np.float32)
    for pos, start, length in _runs(idx):
        synth.masters(w, start, length, out=master[pos:pos + length])
    z = np.zeros_like(master)
    return master, z, z.copy(), master.astype(np.float16)
