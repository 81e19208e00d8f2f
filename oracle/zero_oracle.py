"""The oracle's definitions, one function per step of the shard step.

Test infrastructure only (see the package docstring).  Floating point follows
the precisions the method fixes: fp16 gradient contributions and parameters,
fp32 accumulation, fp32 master weights and Adam moments, fp64 for host
scalars and the norm.  numpy float32 ufuncs round each operation to nearest
even and never fuse a multiply with an add, so every fp32 line below is one
rounded IEEE operation, in the written order.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, NamedTuple, Sequence, Tuple

import numpy as np

F32 = np.float32


# --------------------------------------------------------------------------
# Model-state bytes per rank.
#
# Pages: "ZeRO-1/2/3 分别优化了什么" (section 训练状态的显存构成: 2Ψ fp16 params,
# 2Ψ fp16 grads, 12Ψ Adam states); "第13篇 · ZeRO" §2.2 (M = 2Ψ + 2Ψ + KΨ,
# K = 12) and §3.2 (P_os: 4Ψ + KΨ/Nd, P_os+g: 2Ψ + 14Ψ/Nd, P_os+g+p: 16Ψ/Nd);
# "10.6 ZeRO 与 FSDP" table 10-2.  With general K the stage-2 term is
# (2 + K)Ψ/N and the stage-3 term (4 + K)Ψ/N; both reduce to the printed
# forms at K = 12.
def state_bytes(stage: int, psi: float, n: float, k: float = 12.0) -> float:
    if stage not in (0, 1, 2, 3) or psi < 0 or n < 1 or k < 0:
        raise ValueError("bad arguments")
    if stage == 0:
        return (2.0 + 2.0 + k) * psi
    if stage == 1:
        return 4.0 * psi + k * psi / n
    if stage == 2:
        return 2.0 * psi + (2.0 + k) * psi / n
    return (4.0 + k) * psi / n


# --------------------------------------------------------------------------
# Shard planner.
#
# Pages: "第13篇 · ZeRO" §2.1 (gradients are concatenated into one flat buffer)
# and §3.2 (process i stores and updates partition i); "10.6 ZeRO 与 FSDP"
# §10.6.2 (each GPU owns 1/N of the optimizer state and updates that 1/N of
# the parameters).  Reading: flatten in list order with no per-tensor
# alignment; shard = ceil(psi / N) rounded up to a multiple of ``align``;
# rank r owns flat [r*shard, (r+1)*shard); flat indexes >= psi are padding.
class Plan(NamedTuple):
    psi: int
    world_size: int
    align: int
    shard: int
    psi_padded: int
    offsets: Tuple[int, ...]

    def real(self, rank: int) -> int:
        """Number of non-padding elements in rank's shard."""
        return max(0, min(self.shard, self.psi - rank * self.shard))


def plan(numels: Sequence[int], world_size: int, align: int = 1) -> Plan:
    if world_size < 1 or align < 1 or any(n < 0 for n in numels):
        raise ValueError("bad arguments")
    offsets = []
    acc = 0
    for n in numels:
        offsets.append(acc)
        acc += int(n)
    psi = acc
    per_rank = -(-psi // world_size)
    shard = -(-per_rank // align) * align
    return Plan(psi, world_size, align, shard, shard * world_size, tuple(offsets))


class Segment(NamedTuple):
    tensor: int
    tensor_begin: int  # first element of the tensor inside this shard
    shard_begin: int  # where it lands in the shard
    length: int


def segments(p: Plan, numels: Sequence[int], rank: int) -> List[Segment]:
    """The pieces of each tensor that fall in rank's shard, in flat order."""
    a, b = rank * p.shard, (rank + 1) * p.shard
    out = []
    for t, (off, n) in enumerate(zip(p.offsets, numels)):
        lo, hi = max(a, off), min(b, off + n)
        if lo < hi:
            out.append(Segment(t, lo - off, lo - a, hi - lo))
    return out


# --------------------------------------------------------------------------
# Host scalars for one update.
#
# The pages fix the optimizer (Adam/AdamW with fp32 master, m and v:
# "10.6 ZeRO 与 FSDP" bytes table and the torch.optim.AdamW call in §10.6.7)
# but print no equations.  Reading: Kingma & Ba Adam with bias correction, eps
# outside the square root, decoupled weight decay (Loshchilov & Hutter) on the
# old parameter.  Each coefficient is computed in fp64 from the decimal
# hyperparameter and rounded to fp32 once (so 1 - beta1 is f32(0.1), not
# 1f - 0.9f).  beta^t is a product of t fp64 factors, taken left to right.
# The gradient average over N ranks and the loss-scale unscale are one
# multiply by inv = 1 / (N * loss_scale) ("ZeRO-1/2/3 分别优化了什么",
# section ZeRO-2: each card receives the average; the tutorial's §4.3 names
# loss scaling).
@dataclass(frozen=True)
class Scalars:
    inv64: float
    inv32: np.float32
    b1: np.float32
    omb1: np.float32
    b2: np.float32
    omb2: np.float32
    eps: np.float32
    step_size: np.float32
    sqrt_bc2: np.float32
    decay: np.float32


def step_scalars(lr: float, beta1: float, beta2: float, eps: float, weight_decay: float, t: int,
                 world_size: int, loss_scale: float) -> Scalars:
    if t < 1 or world_size < 1 or not loss_scale > 0:
        raise ValueError("bad arguments")
    p1, p2 = beta1, beta2
    for _ in range(t - 1):
        p1 *= beta1
        p2 *= beta2
    inv64 = 1.0 / (world_size * loss_scale)
    return Scalars(
        inv64=inv64, inv32=F32(inv64), b1=F32(beta1), omb1=F32(1.0 - beta1), b2=F32(beta2),
        omb2=F32(1.0 - beta2), eps=F32(eps), step_size=F32(lr / (1.0 - p1)),
        sqrt_bc2=F32(math.sqrt(1.0 - p2)), decay=F32(1.0 - lr * weight_decay),
    )


# --------------------------------------------------------------------------
# Reduce side of the reduce-scatter, done locally.
#
# Pages: "10.6 ZeRO 与 FSDP" §10.6.1 (reduce-scatter = reduce, then each GPU
# keeps its 1/N slice; all-reduce = reduce-scatter + all-gather) and §10.6.2
# step 2.  Reading: the owner's slice of every rank's fp16 gradient is
# converted to fp32 exactly and summed in rank order 0..N-1 into an fp32
# accumulator that starts at +0.
def reduce_contributions(contrib: np.ndarray) -> np.ndarray:
    """contrib: [N, S] fp16 (or its uint16 bit patterns).  Returns acc, fp32 [S]."""
    c = contrib.view(np.float16) if contrib.dtype == np.uint16 else contrib
    assert c.dtype == np.float16 and c.ndim == 2
    acc = np.zeros(c.shape[1], dtype=F32)
    for r in range(c.shape[0]):
        acc = acc + c[r].astype(F32)
    return acc


def unscale(acc: np.ndarray, inv32: np.float32) -> np.ndarray:
    """g = f32(acc * inv): the average over ranks, unscaled by the loss scale."""
    return acc * F32(inv32)


def nonfinite(acc: np.ndarray) -> bool:
    """Overflow check: any +inf, -inf or NaN in the fp32 sums (+inf + -inf
    gives NaN, so a non-finite contribution always shows here)."""
    return bool(acc.size) and not bool(np.isfinite(acc).all())


def exact_sq_units(acc: np.ndarray) -> int:
    """Exact sum of acc_j^2 over the finite elements, as an integer count of
    2^-48.  Every fp16 value is a multiple of 2^-24 and fp32 sums of such
    values stay multiples of 2^-24, so acc_j * 2^24 is an integer K_j and the
    sum is sum K_j^2 exactly (Python integers; K_j is split into 24-bit
    halves only so that numpy's int64 partial sums cannot overflow)."""
    a = acc[np.isfinite(acc)].astype(np.float64)
    k = np.abs(a) * 2.0**24
    ki = k.astype(np.int64)
    if not np.array_equal(ki.astype(np.float64), k) or (ki >= 2**48).any():
        raise ValueError("accumulator is not a multiple of 2^-24 below 2^24")
    hi, lo = ki >> 24, ki & (2**24 - 1)
    total = 0
    step = 1 << 12
    for s in range(0, ki.size, step):
        h, l = hi[s:s + step], lo[s:s + step]
        total += (int((h * h).sum()) << 48) + (int((2 * h * l).sum()) << 24) + int((l * l).sum())
    return total


# --------------------------------------------------------------------------
# Global norm, clip coefficient and skip decision.
#
# Pages: the tutorial's §4.2 sets "gradient_clipping": 1.0 and its §4.3 says
# fp16 training may need loss scaling; nothing more.  Reading (global L2
# clipping, dynamic loss scaling):
#   total_sq = ((f64(Q_own + Q_other) * 2^-48) * inv64) * inv64 + other_sq
#   norm     = sqrt(total_sq)
#   coef     = min(1, max_norm / (norm + 1e-6)) if max_norm > 0 else 1
#   skip     = own overflow or another rank's overflow or Q_own + Q_other >= 2^128
# Q_other is the other ranks' exact sum (an exact all-reduce keeps every rank
# bitwise equal to the unsharded run); other_sq is a plain fp64 stand-in for
# it.  f64 of an integer rounds once, to nearest even; the 2^-48 and the
# power-of-two inv scalings are exact.
class FinalizeResult(NamedTuple):
    own_q: int
    own_sq: float
    total_sq: float
    norm: float
    coef: np.float32
    overflow: bool
    skip: bool


def finalize(own_q: int, own_overflow: bool, inv64: float, max_norm: float, other_q: int = 0,
             other_sq: float = 0.0, other_overflow: bool = False) -> FinalizeResult:
    q_tot = own_q + other_q
    too_big = q_tot >= 2**128
    own_sq = ((float(own_q) * 2.0**-48) * inv64) * inv64
    total_sq = ((float(q_tot) * 2.0**-48) * inv64) * inv64 + other_sq
    norm = math.sqrt(total_sq)
    coef = min(1.0, max_norm / (norm + 1e-6)) if max_norm > 0 else 1.0
    skip = bool(own_overflow or other_overflow or too_big)
    return FinalizeResult(own_q, own_sq, total_sq, norm, F32(coef), bool(own_overflow), skip)


# --------------------------------------------------------------------------
# Local optimizer update on the shard and the cast into the all-gather slot.
#
# Pages: "10.6 ZeRO 与 FSDP" §10.6.2 step 3 (local 1/N optimizer state + 1/N
# gradient -> local 1/N parameters) and step 4 (all-gather of the updated fp16
# parameters); "第13篇 · ZeRO" §2.2 (fp32 master, momentum and variance).
# fp32 sequence (each line one rounding):
#   gc  = g * c
#   m   = b1*m + omb1*gc
#   v   = b2*v + omb2*(gc*gc)
#   den = sqrt(v) / sqrt_bc2 + eps
#   u   = (m / den) * step_size
#   p   = p*decay - u
#   h   = fp16(p), round to nearest even
def adam_apply(g: np.ndarray, p: np.ndarray, m: np.ndarray, v: np.ndarray, sc: Scalars,
               coef: np.float32):
    assert g.dtype == p.dtype == m.dtype == v.dtype == F32
    gc = g * F32(coef)
    m = sc.b1 * m + sc.omb1 * gc
    v = sc.b2 * v + sc.omb2 * (gc * gc)
    den = np.sqrt(v) / sc.sqrt_bc2 + sc.eps
    u = (m / den) * sc.step_size
    p = p * sc.decay - u
    return p, m, v, p.astype(np.float16)


# --------------------------------------------------------------------------
# Loss-scale update after a step (host side).  Reading of "FP16 训练可能需要
# 调 loss scaling" (tutorial §4.3): halve on an overflowed (skipped) step, not
# below min_scale; double after growth_interval clean steps in a row.
def scaler_update(scale: float, good_steps: int, skipped: bool, growth_interval: int = 1000,
                  growth: float = 2.0, backoff: float = 0.5, min_scale: float = 1.0):
    if skipped:
        return max(scale * backoff, min_scale), 0
    good_steps += 1
    if good_steps >= growth_interval:
        return scale * growth, 0
    return scale, good_steps


# --------------------------------------------------------------------------
class StepOut(NamedTuple):
    g: np.ndarray
    fin: FinalizeResult
    p: np.ndarray
    m: np.ndarray
    v: np.ndarray
    h: np.ndarray  # fp16 slot after the step (unchanged input on a skip)


def shard_step(contrib: np.ndarray, p: np.ndarray, m: np.ndarray, v: np.ndarray, h: np.ndarray,
               sc: Scalars, max_norm: float, other_q: int = 0, other_sq: float = 0.0,
               other_overflow: bool = False) -> StepOut:
    """One rank's whole step on its shard: reduce, unscale, check, norm,
    finalize, then Adam and the fp16 cast unless the step is skipped.  On a
    skip the state and the slot come back unchanged."""
    acc = reduce_contributions(contrib)
    g = unscale(acc, sc.inv32)
    fin = finalize(exact_sq_units(acc), nonfinite(acc), sc.inv64, max_norm, other_q, other_sq,
                   other_overflow)
    if fin.skip:
        return StepOut(g, fin, p, m, v, h)
    p2, m2, v2, h2 = adam_apply(g, p, m, v, sc, fin.coef)
    return StepOut(g, fin, p2, m2, v2, h2)


# --------------------------------------------------------------------------
# FSDP / ZeRO-3 units.
#
# Pages: "10.6 ZeRO 与 FSDP" §10.6.4 (stage 3: each GPU updates its 1/N of
# the parameters with its 1/N of the optimizer state and of the gradient) and
# §10.6.7 (FSDP units: the parameters of one unit, e.g. one transformer block,
# are flattened, sharded and gathered together).  Reading: each unit is a run
# of consecutive tensors; it is flattened in list order and padded on its own
# to N * S_u with S_u = ceil(psi_u / N) rounded up to `align`; rank r owns
# [r*S_u, (r+1)*S_u) of every unit; a rank's state is its unit shards
# concatenated in unit order.
class UnitPlan(NamedTuple):
    world_size: int
    align: int
    psi: int
    unit_psi: Tuple[int, ...]
    unit_shard: Tuple[int, ...]
    unit_flat: Tuple[int, ...]  # first model element of each unit
    unit_rank_offset: Tuple[int, ...]  # offset of each unit's shard in a rank's concatenation
    rank_shard: int  # elements each rank holds over all units


def plan_units(numels: Sequence[int], unit_of_tensor: Sequence[int], world_size: int,
               align: int = 1) -> UnitPlan:
    if len(numels) != len(unit_of_tensor) or world_size < 1 or align < 1:
        raise ValueError("bad arguments")
    if any(b < a for a, b in zip(unit_of_tensor, unit_of_tensor[1:])) or \
            (unit_of_tensor and unit_of_tensor[0] != 0) or \
            any(b - a > 1 for a, b in zip(unit_of_tensor, unit_of_tensor[1:])):
        raise ValueError("units must be consecutive runs numbered 0, 1, 2, ...")
    n_units = (unit_of_tensor[-1] + 1) if unit_of_tensor else 0
    psi_u = [0] * n_units
    for n, u in zip(numels, unit_of_tensor):
        if n < 0:
            raise ValueError("negative numel")
        psi_u[u] += int(n)
    shard_u, flat_u, roff_u = [], [], []
    flat = roff = 0
    for p in psi_u:
        s = -(-(-(-p // world_size)) // align) * align
        shard_u.append(s)
        flat_u.append(flat)
        roff_u.append(roff)
        flat += p
        roff += s
    return UnitPlan(world_size, align, flat, tuple(psi_u), tuple(shard_u), tuple(flat_u),
                    tuple(roff_u), roff)


def unit_shard_index(up: UnitPlan, rank: int) -> np.ndarray:
    """For each element of rank's concatenated unit shards, the model flat
    index it holds, or -1 for padding."""
    out = np.full(up.rank_shard, -1, dtype=np.int64)
    for u in range(len(up.unit_psi)):
        s, a = up.unit_shard[u], up.unit_rank_offset[u]
        local = np.arange(s, dtype=np.int64) + rank * s  # index inside the unit's flat buffer
        ok = local < up.unit_psi[u]
        out[a:a + s][ok] = up.unit_flat[u] + local[ok]
    return out


def unit_model_index(up: UnitPlan, rank: int, pos: np.ndarray) -> np.ndarray:
    """Model flat index held at positions `pos` of rank's concatenated unit
    shards (-1 for padding); the same map as unit_shard_index, pointwise."""
    pos = np.asarray(pos, dtype=np.int64)
    offs = np.asarray(up.unit_rank_offset, dtype=np.int64)
    u = np.searchsorted(offs, pos, side="right") - 1
    shard = np.asarray(up.unit_shard, dtype=np.int64)[u]
    local = pos - offs[u] + rank * shard
    real = local < np.asarray(up.unit_psi, dtype=np.int64)[u]
    return np.where(real, np.asarray(up.unit_flat, dtype=np.int64)[u] + local, -1)


# --------------------------------------------------------------------------
# bf16 variant.
#
# Pages: the tutorial's §4.3 advises bf16 where the hardware supports it, as
# the alternative to tuning fp16 loss scaling.  Reading: gradient
# contributions and the parameter slot are bfloat16, there is no loss scaling
# (loss scale 1), master / m / v stay fp32 and the Adam sequence is unchanged.
# bf16 keeps fp32's exponent range, so the fp16 path's exact integer norm
# (which needs sums that are multiples of 2^-24 below 2^22) does not apply.
# Reading for the norm: each acc_j^2 is exact in fp64 (a 24-bit significand
# squared has at most 48 bits, and the exponent stays in range); the shard's
# sum is the balanced pairwise tree over element indices, zero-padded to a
# power of two, in fp64 -- one fixed order, independent of how the work is
# split.  Across ranks the other ranks' share arrives as a plain fp64 value.
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns to fp32 (exact: bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(F32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 to bfloat16 bit patterns, round to nearest even; NaN stays a quiet
    NaN with its sign."""
    u = np.asarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(np.asarray(x, dtype=F32))
    out = np.where(nan, (u >> 16) | 0x40, rounded)
    return out.astype(np.uint16)


def reduce_contributions_bf16(contrib: np.ndarray) -> np.ndarray:
    """contrib: [N, S] bf16 bit patterns.  acc = fp32 sum in rank order from +0."""
    assert contrib.dtype == np.uint16 and contrib.ndim == 2
    acc = np.zeros(contrib.shape[1], dtype=F32)
    for r in range(contrib.shape[0]):
        acc = acc + bf16_to_f32(contrib[r])
    return acc


def pairwise_sum_f64(x: np.ndarray) -> float:
    """Balanced pairwise sum in fp64: pad with +0 to a power of two, then add
    neighbours level by level (node = left + right)."""
    x = np.asarray(x, dtype=np.float64)
    n = 1
    while n < x.size:
        n *= 2
    y = np.zeros(n, dtype=np.float64)
    y[:x.size] = x
    while y.size > 1:
        y = y[0::2] + y[1::2]
    return float(y[0])


def sq_tree(acc: np.ndarray) -> float:
    """The shard's squared norm of acc for the bf16 path: exact fp64 squares
    (non-finite elements count +0), summed by pairwise_sum_f64."""
    a = acc.astype(np.float64)
    sq = np.where(np.isfinite(a), a * a, 0.0)
    return pairwise_sum_f64(sq)


def finalize_bf16(tree_sq: float, own_overflow: bool, inv64: float, max_norm: float,
                  other_sq: float = 0.0, other_overflow: bool = False) -> FinalizeResult:
    own_sq = (tree_sq * inv64) * inv64
    total_sq = own_sq + other_sq
    norm = math.sqrt(total_sq)
    coef = min(1.0, max_norm / (norm + 1e-6)) if max_norm > 0 else 1.0
    skip = bool(own_overflow or other_overflow)
    return FinalizeResult(0, own_sq, total_sq, norm, F32(coef), bool(own_overflow), skip)


def shard_step_bf16(contrib: np.ndarray, p: np.ndarray, m: np.ndarray, v: np.ndarray,
                    h: np.ndarray, sc: Scalars, max_norm: float, other_sq: float = 0.0,
                    other_overflow: bool = False) -> StepOut:
    """One rank's bf16-path step; h and the returned slot are bf16 bit patterns."""
    acc = reduce_contributions_bf16(contrib)
    g = unscale(acc, sc.inv32)
    fin = finalize_bf16(sq_tree(acc), nonfinite(acc), sc.inv64, max_norm, other_sq,
                        other_overflow)
    if fin.skip:
        return StepOut(g, fin, p, m, v, h)
    p2, m2, v2, _ = adam_apply(g, p, m, v, sc, fin.coef)
    return StepOut(g, fin, p2, m2, v2, f32_to_bf16(p2))
