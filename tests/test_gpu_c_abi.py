"""The step driven from a plain C program (tests/c_abi_step.c) through
include/zero_shard.h, with hipMalloc buffers and no Python or torch on the
device side: its g, master, m, v, slot and result word at every step equal
the oracle's bit for bit on the same seeded inputs, and the program itself
checks that zero_reduce_adam_step and zero_reduce_adam_step_noalloc agree.
Three steps: applied, skipped (another rank overflowed), applied; a clip
threshold low enough to clip; a ragged shard whose slot is not 8-byte
aligned; N = 3 (one-chunk reduce) and N = 16 (the deferred reduce)."""
import dataclasses
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import synth
from oracle import run as orun
from parity_util import check_result

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _driver() -> str:
    from zero_sharded_optimizer_rank_amd import build
    return build.C_EXAMPLE if os.path.exists(build.C_EXAMPLE) else build.build_c_example()


@pytest.mark.parametrize("n,rank", [(3, 1), (16, 5)])
def test_c_program_step_matches_oracle(n, rank):
    from zero_sharded_optimizer_rank_amd import abi

    print(f"[c abi step N={n} rank {rank}]", flush=True)
    w = dataclasses.replace(synth.TINY, name=f"c_abi_{n}", cfg_id=40 + n,
                            tensors=(("a", (1000, 37)), ("b", (5,)), ("c", (4,))), world_size=n,
                            max_grad_norm=0.05, weight_decay=0.01, steps=3)
    p = orun.workload_plan(w)
    S = p.shard
    other_sq = 1e-4
    ovf = {1: False, 2: True, 3: False}
    master = synth.masters(w, rank * S, S)
    with tempfile.TemporaryDirectory() as td:
        fin, fout = os.path.join(td, "in.bin"), os.path.join(td, "out.bin")
        # the oracle's scale schedule decides the contributions' scale per step
        scale, good = w.loss_scale0, 0
        contribs = []
        for step in (1, 2, 3):
            contribs.append((scale, orun.shard_contrib(w, p, rank, step, scale)))
            scale, good = oracle.scaler_update(scale, good, ovf[step])
        with open(fin, "wb") as f:
            f.write(np.array([len(w.numels), n, rank, 3], dtype=np.int64).tobytes())
            f.write(np.array(w.numels, dtype=np.int64).tobytes())
            f.write(np.array([w.lr, *w.betas, w.eps, w.weight_decay, w.max_grad_norm,
                              w.loss_scale0, other_sq], dtype=np.float64).tobytes())
            f.write(master.astype(np.float32).tobytes())
            for step, (_, c) in zip((1, 2, 3), contribs):
                f.write(np.array([1 if ovf[step] else 0], dtype=np.int32).tobytes())
                f.write(np.ascontiguousarray(c, dtype=np.uint16).tobytes())
        r = subprocess.run([_driver(), fin, fout], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        raw = open(fout, "rb").read()
    rb = abi.RESULT_BYTES
    per = rb + 4 * 4 * S + 2 * S
    assert len(raw) == 3 * per
    op, om, ov = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    oh = np.zeros(S, np.uint16)
    t = 0
    for i, step in enumerate((1, 2, 3)):
        blob = raw[i * per:(i + 1) * per]
        res = abi.zero_step_result_t.from_buffer_copy(blob[:rb])
        arrs = np.frombuffer(blob[rb:rb + 16 * S], dtype=np.float32).reshape(4, S)
        slot = np.frombuffer(blob[rb + 16 * S:], dtype=np.uint16)
        scale, c = contribs[i]
        sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, t + 1, n, scale)
        out = oracle.shard_step(c, op, om, ov, oh, sc, w.max_grad_norm, other_sq=other_sq,
                                other_overflow=ovf[step])
        check_result(res, out.fin, step)
        assert bool(res.skip) == ovf[step] and (ovf[step] or float(res.clip_coef) < 1.0)
        op, om, ov, oh = out.p, out.m, out.v, out.h.view(np.uint16)
        for k, want in enumerate((out.g, op, om, ov)):
            assert np.array_equal(arrs[k].view(np.uint32), want.view(np.uint32)), (step, k)
        assert np.array_equal(slot, oh), step
        t += 0 if out.fin.skip else 1
