"""Seeded random configurations through the C ABI against the oracle.

Each case draws, from its own seed: the world size, the tensor list (so the
shard length, the ragged tail and the padding), whole shard or a window, the
gradient format, the loss scale, the gradient magnitude (up to where most
contributions sit at the format's largest finite value), the clipping
threshold, learning rate, betas, eps and weight
decay, an injected +inf, and whether the other ranks' share of the norm is
present.  Every step of every case must match the oracle bit for bit, as in
the hand-picked parity cases.
"""
import dataclasses
import os

import numpy as np
import pytest

import synth
from oracle import run as orun
from parity_util import run_units_all_ranks, run_window

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# ZERO_RANDOM_SCALE=k sets the multiplier of every case count below (default 4;
# larger values run an extended campaign)
SCALE = max(1, int(os.environ.get("ZERO_RANDOM_SCALE", "4")))
N_CASES = 48 * SCALE
N_UNIT_CASES = 16 * SCALE


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pick(rng, xs):
    return xs[int(rng.integers(len(xs)))]


def random_workload(seed: int) -> synth.Workload:
    rng = np.random.default_rng([0x7A3D, seed])
    n = int(_pick(rng, [1, 2, 3, 4, 5, 7, 8, 13, 16, 64]))
    tensors = []
    for i in range(int(rng.integers(1, 6))):
        if rng.random() < 0.5:
            shape = (int(rng.integers(1, 400)), int(rng.integers(1, 400)))
        else:
            shape = (int(rng.integers(1, 60_000)),)
        tensors.append((f"t{i}", shape))
    bf16 = rng.random() < 0.35
    scales = [1.0, 0.5, 1024.0] if bf16 else [1.0, 3.0, 1024.0, 65536.0, 2.0 ** 20]
    w = dataclasses.replace(
        synth.BY_NAME["tiny"], name=f"random{seed}", cfg_id=1000 + seed,
        tensors=tuple(tensors), world_size=n,
        sigma=float(_pick(rng, [1e-6, 1e-3, 1e-1, 4.0])),
        loss_scale0=float(_pick(rng, scales)),
        lr=float(_pick(rng, [0.0, 1e-4, 3e-3])),
        weight_decay=float(_pick(rng, [0.0, 0.01, 0.1])),
        max_grad_norm=float(_pick(rng, [0.0, 1e-3, 1.0, 1e4])),
        steps=3,
        inject_step=None,
        betas=_pick(rng, [(0.9, 0.999), (0.5, 0.9), (0.0, 0.99), (0.95, 0.9999)]),
        eps=float(_pick(rng, [1e-8, 1e-6, 1e-3])),
        other_ranks_from_config=bool(rng.random() < 0.5),
        parity_ranks=tuple(sorted({0, n - 1, int(rng.integers(n))})),
        dtype="bf16" if bf16 else "fp16",
    )
    inject = _pick(rng, [None, None, 1, 2, 3])
    if inject is not None and w.psi >= n:  # the injected element lies below psi // N
        w = dataclasses.replace(w, inject_step=inject)
    return w


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration_matches_oracle(seed):
    w = random_workload(seed)
    p = orun.workload_plan(w)
    rng = np.random.default_rng([0x7A3E, seed])
    for rank in w.parity_ranks:
        if rng.random() < 0.3 and p.shard > 2:
            begin = int(rng.integers(0, p.shard - 1))
            count = int(rng.integers(1, p.shard - begin + 1))
        else:
            begin, count = 0, p.shard
        print(f"[random {seed}] {w.dtype} N={w.world_size} psi={w.psi} S={p.shard} rank={rank} "
              f"window=({begin},{count}) scale={w.loss_scale0} sigma={w.sigma} "
              f"clip={w.max_grad_norm} inject={w.inject_step}", flush=True)
        run_window(w, rank, begin, count)


def random_unit_workload(seed: int) -> synth.Workload:
    """A unit layout (ZeRO-3 / FSDP): 1-8 tensors in 1-8 contiguous units,
    each unit flattened and sharded on its own; fp16 only.  Above N = 8 the
    reduce's workgroups take eight chunks that may span several units."""
    rng = np.random.default_rng([0x7A3F, seed])
    n = int(_pick(rng, [1, 2, 3, 4, 8, 13, 16, 32]))
    n_t = int(rng.integers(1, 9))
    tensors = tuple((f"t{i}", (int(rng.integers(1, 20_000 if rng.random() < 0.7 else 150_000)),))
                    for i in range(n_t))
    n_u = int(rng.integers(1, n_t + 1))
    cuts = set(int(c) for c in rng.choice(np.arange(1, n_t), n_u - 1, replace=False)) \
        if n_u > 1 else set()
    units, u = [], 0
    for i in range(n_t):
        u += i in cuts
        units.append(u)
    w = dataclasses.replace(
        synth.BY_NAME["tiny_fsdp"], name=f"random_units{seed}", cfg_id=2000 + seed,
        tensors=tensors, units=tuple(units), world_size=n,
        sigma=float(_pick(rng, [1e-6, 1e-3, 1e-1, 4.0])),
        loss_scale0=float(_pick(rng, [1.0, 3.0, 1024.0, 65536.0])),
        lr=float(_pick(rng, [1e-4, 3e-3])),
        weight_decay=float(_pick(rng, [0.0, 0.1])),
        max_grad_norm=float(_pick(rng, [0.0, 1e-3, 1.0])),
        steps=3,
        betas=_pick(rng, [(0.9, 0.999), (0.5, 0.9)]),
        eps=float(_pick(rng, [1e-8, 1e-3])),
    )
    inject = _pick(rng, [None, 1, 2])
    if inject is not None and w.psi >= n:
        w = dataclasses.replace(w, inject_step=inject)
    return w


@pytest.mark.parametrize("seed", range(N_UNIT_CASES))
def test_random_unit_layout_matches_oracle(seed):
    w = random_unit_workload(seed)
    print(f"[random units {seed}] N={w.world_size} numels={w.numels} units={w.units} "
          f"scale={w.loss_scale0} sigma={w.sigma} clip={w.max_grad_norm} "
          f"inject={w.inject_step}", flush=True)
    run_units_all_ranks(w)


@pytest.mark.parametrize("seed", range(12 * SCALE))
def test_random_configuration_offload_matches_oracle(seed):
    """The offload form (reduce on the GPU, Adam on the host, fp16 back over
    PCIe) on random fp16 configurations, with a random pipeline chunk and
    thread count."""
    w = random_workload(100 + seed)
    if w.dtype != "fp16":
        w = dataclasses.replace(w, dtype="fp16", loss_scale0=1024.0)
    p = orun.workload_plan(w)
    rng = np.random.default_rng([0x7A40, seed])
    chunk = int(_pick(rng, [64, 192, 4096, 1 << 16]))
    threads = int(_pick(rng, [1, 2, 5, 8]))
    for rank in w.parity_ranks:
        print(f"[random offload {seed}] N={w.world_size} S={p.shard} rank={rank} chunk={chunk} "
              f"threads={threads} scale={w.loss_scale0} clip={w.max_grad_norm} "
              f"inject={w.inject_step}", flush=True)
        run_window(w, rank, 0, p.shard, offload=dict(chunk=chunk, threads=threads))


@pytest.mark.parametrize("seed", range(16 * SCALE))
def test_random_configuration_onepass_matches_oracle(seed):
    """The single-pass step on random fp16 and bf16 configurations with
    clipping off, whole shards or windows, injected overflow included."""
    w = random_workload(200 + seed)
    w = dataclasses.replace(w, max_grad_norm=0.0)
    p = orun.workload_plan(w)
    rng = np.random.default_rng([0x7A41, seed])
    for rank in w.parity_ranks:
        if rng.random() < 0.3 and p.shard > 2:
            begin = int(rng.integers(0, p.shard - 1))
            count = int(rng.integers(1, p.shard - begin + 1))
        else:
            begin, count = 0, p.shard
        print(f"[random onepass {seed}] {w.dtype} N={w.world_size} psi={w.psi} S={p.shard} rank={rank} "
              f"window=({begin},{count}) scale={w.loss_scale0} sigma={w.sigma} "
              f"inject={w.inject_step}", flush=True)
        run_window(w, rank, begin, count, one_pass=True)


@pytest.mark.parametrize("seed", range(8 * SCALE))
def test_random_unit_layout_one_pass_matches_oracle(seed):
    """The unit single pass on random unit layouts with clipping off."""
    w = dataclasses.replace(random_unit_workload(100 + seed), max_grad_norm=0.0)
    in_place = seed % 2 == 1  # half of them write the live slots and restore them
    print(f"[random units one pass {seed}] N={w.world_size} numels={w.numels} units={w.units} "
          f"scale={w.loss_scale0} sigma={w.sigma} inject={w.inject_step} in_place={in_place}",
          flush=True)
    run_units_all_ranks(w, one_pass=True, in_place_slot=in_place)
