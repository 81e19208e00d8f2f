"""The five synthetic shard-step workloads: tensor lists, seeds and hyperparameters.

This module describes inputs only.  It holds no step of the method; the shard
planner, the reduction, the norm and Adam live in the oracle and in the HIP
library, each on its own.

Shapes are the published architectures' parameter lists (weights of every
linear layer, embeddings, normalisation weights and, for GPT-2, biases).  The
flat order is list order, layer by layer.  Values are synthetic and seeded.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from math import prod
from typing import Optional, Tuple

BASE_SEED = 0x5EED2019

# purposes of a Philox stream (the high byte of counter word 3)
PURPOSE_CONTRIB = 1
PURPOSE_MASTER = 2
PURPOSE_INJECT = 3


def _tiny():
    return (("w", (1000, 1000)), ("b", (1000,)), ("c", (3,)))


def _gpt2_1p5b():
    h, f, vocab, pos, layers = 1600, 6400, 50257, 1024, 48
    t = [("wte", (vocab, h)), ("wpe", (pos, h))]
    for i in range(layers):
        t += [
            (f"h{i}.ln_1.w", (h,)),
            (f"h{i}.ln_1.b", (h,)),
            (f"h{i}.attn.c_attn.w", (h, 3 * h)),
            (f"h{i}.attn.c_attn.b", (3 * h,)),
            (f"h{i}.attn.c_proj.w", (h, h)),
            (f"h{i}.attn.c_proj.b", (h,)),
            (f"h{i}.ln_2.w", (h,)),
            (f"h{i}.ln_2.b", (h,)),
            (f"h{i}.mlp.c_fc.w", (h, f)),
            (f"h{i}.mlp.c_fc.b", (f,)),
            (f"h{i}.mlp.c_proj.w", (f, h)),
            (f"h{i}.mlp.c_proj.b", (h,)),
        ]
    t += [("ln_f.w", (h,)), ("ln_f.b", (h,))]
    return tuple(t)


def _flat_7p5b():
    n_full = 447
    rem = 7_500_000_000 - n_full * 4096 * 4096
    return tuple([(f"block{i}", (4096, 4096)) for i in range(n_full)] + [("remainder", (rem,))])


def _llama(h, kv, ffn, vocab, layers):
    t = [("embed", (vocab, h))]
    for i in range(layers):
        t += [
            (f"l{i}.q", (h, h)),
            (f"l{i}.k", (kv, h)),
            (f"l{i}.v", (kv, h)),
            (f"l{i}.o", (h, h)),
            (f"l{i}.gate", (ffn, h)),
            (f"l{i}.up", (ffn, h)),
            (f"l{i}.down", (h, ffn)),
            (f"l{i}.attn_norm", (h,)),
            (f"l{i}.mlp_norm", (h,)),
        ]
    t += [("final_norm", (h,)), ("lm_head", (vocab, h))]
    return tuple(t)


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    tensors: Tuple[Tuple[str, Tuple[int, ...]], ...]
    world_size: int
    sigma: float  # std of one rank's unscaled fp16 gradient contribution
    loss_scale0: float  # loss scale at the first step
    lr: float
    weight_decay: float
    max_grad_norm: float  # <= 0: no clipping
    steps: int
    inject_step: Optional[int] = None  # 1-based step whose contributions hold one +inf
    betas: Tuple[float, float] = (0.9, 0.999)
    eps: float = 1e-8
    master_sigma: float = 0.02
    other_ranks_from_config: bool = False  # stand in the other ranks' squared norm by a constant
    parity_ranks: Tuple[int, ...] = field(default=(0,))
    units: Optional[Tuple[int, ...]] = None  # FSDP unit of each tensor (None: one flat buffer)
    dtype: str = "fp16"  # gradient contributions and parameter slot: "fp16" or "bf16"

    @property
    def numels(self) -> Tuple[int, ...]:
        return tuple(prod(s) for _, s in self.tensors)

    @property
    def psi(self) -> int:
        return sum(self.numels)

    @property
    def key(self) -> Tuple[int, int]:
        return (BASE_SEED, self.cfg_id)

    def other_sq(self, shard_real: int) -> float:
        """Stand-in for the other N-1 ranks' partial squared norms of the averaged
        unscaled gradient: (N-1) * shard * sigma^2 / N, since each element of the
        average of N contributions of std sigma has variance sigma^2 / N."""
        n = self.world_size
        return (n - 1) * shard_real * self.sigma * self.sigma / n


TINY = Workload(
    name="tiny", cfg_id=1, tensors=_tiny(), world_size=4, sigma=1e-2, loss_scale0=1024.0,
    lr=1e-3, weight_decay=0.0, max_grad_norm=0.0, steps=3, parity_ranks=(0, 1, 2, 3),
)
GPT2 = Workload(
    name="gpt2_1p5b", cfg_id=2, tensors=_gpt2_1p5b(), world_size=64, sigma=1e-3,
    loss_scale0=65536.0, lr=1.5e-4, weight_decay=0.01, max_grad_norm=0.0, steps=5,
    parity_ranks=(0, 1, 63),
)
FLAT75 = Workload(
    name="flat_7p5b", cfg_id=3, tensors=_flat_7p5b(), world_size=64, sigma=1e-3,
    loss_scale0=1024.0, lr=1e-4, weight_decay=0.0, max_grad_norm=1.0, steps=3,
    other_ranks_from_config=True, parity_ranks=(0, 1, 63),
)
LLAMA3_8B = Workload(
    name="llama3_8b", cfg_id=4, tensors=_llama(4096, 1024, 14336, 128256, 32), world_size=8,
    sigma=1e-3, loss_scale0=65536.0, lr=3e-4, weight_decay=0.1, max_grad_norm=1.0, steps=4,
    inject_step=2, other_ranks_from_config=True, parity_ranks=(0, 1, 7),
)
LLAMA2_70B = Workload(
    name="llama2_70b", cfg_id=5, tensors=_llama(8192, 1024, 28672, 32000, 80), world_size=64,
    sigma=1e-3, loss_scale0=32768.0, lr=1.5e-4, weight_decay=0.1, max_grad_norm=1.0, steps=2,
    other_ranks_from_config=True, parity_ranks=(0, 1, 63),
)

ALL = (TINY, GPT2, FLAT75, LLAMA3_8B, LLAMA2_70B)


# ZeRO-3 / FSDP layouts: the same tensor lists wrapped into units, one per
# transformer block, with the embeddings and the final norm / head as units of
# their own.  Each unit is flattened and sharded over N separately.
def _units_by_prefix(tensors, first_prefixes, last_prefixes):
    units, u = [], 0
    block = None
    for name, _ in tensors:
        if any(name.startswith(p) for p in first_prefixes):
            units.append(0)
            continue
        if any(name.startswith(p) for p in last_prefixes):
            units.append(u + 1)
            continue
        b = name.split(".")[0]
        if b != block:
            block = b
            u += 1
        units.append(u)
    return tuple(units)


TINY_FSDP = Workload(
    name="tiny_fsdp", cfg_id=11, tensors=_tiny(), world_size=4, sigma=1e-2, loss_scale0=1024.0,
    lr=1e-3, weight_decay=0.0, max_grad_norm=0.0, steps=3, parity_ranks=(0, 1, 2, 3),
    units=(0, 1, 2),
)
GPT2_FSDP = Workload(
    name="gpt2_1p5b_fsdp", cfg_id=12, tensors=_gpt2_1p5b(), world_size=64, sigma=1e-3,
    loss_scale0=65536.0, lr=1.5e-4, weight_decay=0.01, max_grad_norm=0.0, steps=5,
    parity_ranks=(0, 1, 63), units=_units_by_prefix(_gpt2_1p5b(), ("wte", "wpe"), ("ln_f",)),
)
LLAMA3_8B_FSDP = Workload(
    name="llama3_8b_fsdp", cfg_id=14, tensors=_llama(4096, 1024, 14336, 128256, 32), world_size=8,
    sigma=1e-3, loss_scale0=65536.0, lr=3e-4, weight_decay=0.1, max_grad_norm=1.0, steps=4,
    other_ranks_from_config=True, parity_ranks=(0, 1, 7),
    units=_units_by_prefix(_llama(4096, 1024, 14336, 128256, 32), ("embed",),
                           ("final_norm", "lm_head")),
)
UNIT_WORKLOADS = (TINY_FSDP, GPT2_FSDP, LLAMA3_8B_FSDP)

# bf16 variants: bf16 gradient contributions and parameter slot, no loss
# scaling (loss scale 1 throughout), fp32 master / m / v as before.
TINY_BF16 = Workload(
    name="tiny_bf16", cfg_id=21, tensors=_tiny(), world_size=4, sigma=1e-2, loss_scale0=1.0,
    lr=1e-3, weight_decay=0.0, max_grad_norm=0.0, steps=3, parity_ranks=(0, 1, 2, 3),
    dtype="bf16",
)
LLAMA3_8B_BF16 = Workload(
    name="llama3_8b_bf16", cfg_id=24, tensors=_llama(4096, 1024, 14336, 128256, 32), world_size=8,
    sigma=1e-3, loss_scale0=1.0, lr=3e-4, weight_decay=0.1, max_grad_norm=1.0, steps=4,
    inject_step=2, other_ranks_from_config=True, parity_ranks=(0, 1, 7), dtype="bf16",
)
BF16_WORKLOADS = (TINY_BF16, LLAMA3_8B_BF16)
BY_NAME = {w.name: w for w in ALL + UNIT_WORKLOADS + BF16_WORKLOADS}
