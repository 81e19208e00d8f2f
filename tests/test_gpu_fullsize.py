"""GPU parity at the workloads' full shard sizes, in the launch configuration
bench.py times (the whole shard of the rank).

Every step of each workload runs on the GPU, and the oracle checks it over
the whole shard, every element:
  * the exact squared-norm integer (fp16) or the pairwise fp64 tree (bf16),
    overflow flag, norm, clip coefficient and skip decision, computed by the
    C form of the oracle's reduce statistics from the same host-generated
    input chunks that are copied to the device (for bf16 each chunk is an
    aligned power-of-two subtree, and the roots are summed by the oracle's
    pairwise tree);
  * g (two-pass form), master, m, v and the 16-bit slot, bit for bit: the C
    form of the oracle's unscale and Adam update (pinned bit for bit to the
    numpy definitions on the CPU) runs on the host over the whole shard, with
    the state carried across steps, and every device array is fetched chunk
    by chunk and compared with it.

With ZERO_FULLSIZE_SAMPLED=1 in the environment the state is compared only at
~4k sampled elements per step (first, last, random, around 2^30 and 2^31 and
an injected inf), computed by the numpy oracle: a faster mode for iterating.
"""
import dataclasses
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import fast
from oracle import run as orun

from parity_util import check_result, compare_state, other_overflow_at, StepReport

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SAMPLED = os.environ.get("ZERO_FULLSIZE_SAMPLED", "") not in ("", "0")
FETCH = 1 << 26  # elements per device-to-host comparison chunk


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _sample_indices(w, rank, shard, k=4096):
    rng = np.random.default_rng(7 + rank)
    idx = set(rng.integers(0, shard, size=k).tolist())
    idx.update(range(0, 32))
    idx.update(range(max(0, shard - 32), shard))
    for mark in (1 << 30, (1 << 31) - 16):
        if mark < shard:
            idx.update(range(mark - 8, min(shard, mark + 9)))
    site = synth.inject_site(w, w.inject_step) if w.inject_step else None
    if site is not None:
        p = orun.workload_plan(w)
        j = site[1] - rank * p.shard
        if 0 <= j < shard:
            idx.update(range(max(0, j - 8), min(shard, j + 9)))
    return np.array(sorted(idx), dtype=np.int64)


def _feed_and_reduce(dev, step, scale, inv32, idx=None, g_out=None):
    """Generate the step's contributions chunk by chunk on the host, copy each
    chunk to the device, and reduce the same chunk with the C oracle.  Returns
    (Q or, for bf16, the tree value; overflow; contributions at idx or None).
    With g_out, the oracle's g = f32(acc * inv32) of every element goes there."""
    w, n, count = dev.w, dev.w.world_size, dev.count
    chunk = (1 << 28) // (2 * n)  # 256 MiB of host staging
    bf16 = w.dtype == "bf16"
    assert not bf16 or chunk & (chunk - 1) == 0
    roots = []
    host = torch.empty((n, chunk), dtype=torch.int16, pin_memory=True)
    hnp = host.numpy().view(np.uint16)
    q_total, bad = 0, False
    cols = None if idx is None else np.zeros((n, idx.size), dtype=np.uint16)
    for c0 in range(0, count, chunk):
        k = min(chunk, count - c0)
        for q in range(n):
            synth.contributions(w, step, q, dev.flat_begin + c0, k, scale, out=hnp[q, :k])
        with torch.cuda.stream(dev.stream):
            for q in range(n):
                dev.contrib[q, c0:c0 + k].copy_(host[q, :k], non_blocking=True)
        if bf16:
            qc, bc = fast.reduce_tree_bf16(hnp, k, width=chunk)
            roots.append(qc)
        else:
            qc, bc = fast.reduce_stats(hnp, k)
            q_total += qc
        bad |= bc
        if g_out is not None:
            fast.reduce_unscale(hnp, inv32, count=k, bf16=bf16, out=g_out[c0:c0 + k])
        if cols is not None:
            sel = (idx >= c0) & (idx < c0 + k)
            cols[:, sel] = hnp[:, idx[sel] - c0]
        dev.stream.synchronize()
    if bf16:
        return oracle.pairwise_sum_f64(np.array(roots)), bad, cols
    return q_total, bad, cols


class _Fetcher:
    """Device array -> host chunks through one pinned buffer."""

    def __init__(self, dev):
        self.dev = dev
        self.buf32 = torch.empty(min(FETCH, max(dev.count, 1)), dtype=torch.float32,
                                 pin_memory=True)
        self.buf16 = self.buf32.view(torch.int16)

    def compare(self, rep, name, want):
        """Bitwise mismatches of the whole device array `name` against `want`;
        on a mismatch, also the 1e-6 / 1-ulp bar over the offending chunk."""
        d = self.dev
        t = {"grad": d.grad, "master": d.master, "m": d.m, "v": d.v}.get(name)
        t = d.slot if name == "slot" else t[:d.count]
        mism, worst = 0, 0.0
        for s in range(0, d.count, FETCH):
            k = min(FETCH, d.count - s)
            buf = self.buf16[:k] if name == "slot" else self.buf32[:k]
            with torch.cuda.stream(d.stream):
                buf.copy_(t[s:s + k], non_blocking=True)
            d.stream.synchronize()
            got = buf.numpy().view(np.uint16 if name == "slot" else np.float32)
            ref = want[s:s + k]
            bad = fast.count_unequal(got, ref)
            if bad:
                mism += bad
                sub = StepReport(rep.step, rep.skip, rep.coef)
                try:
                    compare_state(sub, name, got.copy(), ref.copy())
                finally:
                    worst = max(worst, sub.max_rel.get(name, float("inf")))
        rep.mismatches[name] = mism
        rep.max_rel[name] = worst
        return mism


# The largest shard the ABI accepts (2^31 - 8 elements) at N = 2: element
# offsets pass 2^31 in the flat buffer and approach it inside the shard; rank
# 1's shard ends with one padding element.
_MAX = 0x7FFFFFF8
MAX_SHARD = dataclasses.replace(
    synth.TINY, name="max_shard", cfg_id=31, tensors=(("w", (2 * _MAX - 1,)),), world_size=2,
    sigma=1e-2, loss_scale0=1024.0, weight_decay=0.01, max_grad_norm=1.0, steps=2,
    other_ranks_from_config=True, parity_ranks=(1,))
MAX_SHARD_BF16 = dataclasses.replace(MAX_SHARD, name="max_shard_bf16", cfg_id=32, dtype="bf16",
                                     loss_scale0=1.0, steps=1)


def _cases():
    cases = [pytest.param(w, r, False, id=f"{w.name}-r{r}") for w, r in (
        (synth.GPT2, 0), (synth.GPT2, 1), (synth.GPT2, 63),
        (synth.FLAT75, 0), (synth.FLAT75, 1),
        (synth.LLAMA3_8B, 0),
        (synth.LLAMA2_70B, 0),
        (synth.LLAMA3_8B_BF16, 0), (synth.LLAMA3_8B_BF16, 7),
        (MAX_SHARD, 1), (MAX_SHARD_BF16, 1),
    )]
    # the single-pass step (unclipped workloads) as bench.py --one-pass times it, and at
    # the largest shard the ABI accepts (clipping off), fp16 and bf16
    cases += [pytest.param(synth.GPT2, r, True, id=f"gpt2_1p5b-r{r}-1pass") for r in (0, 1)]
    cases += [pytest.param(dataclasses.replace(w, max_grad_norm=0.0), 1, True,
                           id=f"{w.name}-r1-1pass") for w in (MAX_SHARD, MAX_SHARD_BF16)]
    return cases


def _initial_host_state(w, flat_begin, count):
    """Oracle state of the whole shard: seeded fp32 masters, m = v = 0, and
    the 16-bit cast of the masters."""
    p = np.empty(count, dtype=np.float32)
    for s in range(0, count, 1 << 26):
        k = min(1 << 26, count - s)
        synth.masters(w, flat_begin + s, k, out=p[s:s + k])
    return p, np.zeros(count, np.float32), np.zeros(count, np.float32), \
        fast.cast16(p, bf16=w.dtype == "bf16")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w,rank,one_pass", _cases())
def test_full_size_shard(w, rank, one_pass):
    import zero_sharded_optimizer_rank_amd.abi as abi
    from zero_sharded_optimizer_rank_amd.shard import DeviceShard

    mode = "sampled" if SAMPLED else "every element"
    print(f"[full size {w.name} rank {rank}{' one pass' if one_pass else ''}, {mode}]",
          flush=True)
    dev = DeviceShard(w, rank, one_pass=one_pass)
    dev.load_initial_state()
    p = orun.workload_plan(w)
    assert dev.count == p.shard and dev.flat_begin == rank * p.shard
    bf16 = w.dtype == "bf16"
    if SAMPLED:
        idx = _sample_indices(w, rank, p.shard)
        flat = rank * p.shard + idx
        op = np.array([synth.masters(w, int(e), 1)[0] for e in flat], dtype=np.float32)
        om, ov = np.zeros_like(op), np.zeros_like(op)
        oh = orun.half_copy(w, op)
        hg = None
    else:
        idx = None
        op, om, ov, oh = _initial_host_state(w, dev.flat_begin, dev.count)
        hg = np.empty(dev.count, dtype=np.float32)
        fetch = _Fetcher(dev)
    other_sq = w.other_sq(p.real(rank)) if w.other_ranks_from_config else 0.0
    scaler = abi.new_scaler(w.loss_scale0)
    o_scale, o_good, o_t = w.loss_scale0, 0, 0
    skips = []
    for step in range(1, w.steps + 1):
        assert scaler.scale == o_scale
        sc = oracle.step_scalars(w.lr, *w.betas, w.eps, w.weight_decay, o_t + 1, w.world_size,
                                 o_scale)
        ovf_other = other_overflow_at(w, step, dev.flat_begin, dev.count)
        q_all, bad_all, cols = _feed_and_reduce(dev, step, scaler.scale, sc.inv32, idx, hg)
        args = dev.args(scaler.t + 1, scaler.scale, other_sq=other_sq, other_overflow=ovf_other)
        if one_pass:
            dev.step_1pass(args)
        else:
            dev.step(args)
        res = dev.result()
        if one_pass and not res.skip:
            dev.adopt()
        fin_fn = oracle.finalize_bf16 if bf16 else oracle.finalize
        fin = fin_fn(q_all, bad_all, sc.inv64, w.max_grad_norm, other_sq=other_sq,
                     other_overflow=ovf_other)
        check_result(res, fin, step)
        rep = StepReport(step, fin.skip, float(fin.coef))
        if SAMPLED:
            acc = (oracle.reduce_contributions_bf16 if bf16 else oracle.reduce_contributions)(cols)
            g = oracle.unscale(acc, sc.inv32)
            if not one_pass:  # the single pass writes no gradient
                assert np.array_equal(dev.fetch("grad", idx).view(np.uint32),
                                      g.view(np.uint32)), step
            if not fin.skip:
                op, om, ov, h = oracle.adam_apply(g, op, om, ov, sc, fin.coef)
                oh = oracle.f32_to_bf16(op) if bf16 else h.view(np.uint16)
            for name, want in (("master", op), ("m", om), ("v", ov), ("slot", oh)):
                compare_state(rep, name, dev.fetch(name, idx), want)
        else:
            if not one_pass:  # the single pass writes no gradient
                assert fetch.compare(rep, "grad", hg) == 0, (step, rep.max_rel)
            if not fin.skip:
                fast.adam_update(hg, op, om, ov, oh, sc, fin.coef, bf16=bf16)
            for name, want in (("master", op), ("m", om), ("v", ov), ("slot", oh)):
                fetch.compare(rep, name, want)
        assert all(x == 0 for x in rep.mismatches.values()), (step, rep.mismatches, rep.max_rel)
        assert dev.guards_intact()
        print(f"  step {step}: skip={fin.skip} coef={float(fin.coef):.6g} norm={fin.norm:.6g} "
              f"stat={q_all if bf16 else q_all.bit_length()} compared="
              f"{idx.size if SAMPLED else dev.count} x {sorted(rep.mismatches)}", flush=True)
        skips.append(fin.skip)
        abi.zero_scaler_update(scaler, bool(res.skip))
        o_scale, o_good = oracle.scaler_update(o_scale, o_good, fin.skip)
        o_t += 0 if fin.skip else 1
        assert scaler.t == o_t and scaler.scale == o_scale
    if w.inject_step is not None and rank == 0:
        assert skips[w.inject_step - 1] and not any(s for i, s in enumerate(skips)
                                                    if i != w.inject_step - 1)
    del dev
    torch.cuda.empty_cache()

