"""Independent steps in flight at once: several host threads, each with its
own torch stream and its own buffers, workspace and unit tables, call the
library at the same time, so calls interleave on the host and their kernels
overlap on the GPU.  Every step of every thread must still equal the oracle
bit for bit: the library keeps no state shared between calls other than the
no-allocation entry point's scratch array (not used here), and its error
message buffer is per thread."""
import dataclasses
from concurrent.futures import ThreadPoolExecutor

import pytest

import synth
from oracle import run as orun
from parity_util import run_units_all_ranks, run_window

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _jobs():
    tiny, bf16, gpt2 = synth.TINY, synth.BY_NAME["tiny_bf16"], synth.GPT2
    tiny_skip = dataclasses.replace(tiny, inject_step=2)
    shard = orun.workload_plan(gpt2).shard
    st, sb = orun.workload_plan(tiny).shard, orun.workload_plan(bf16).shard
    return [
        ("tiny rank 0, fused step", lambda s: run_window(tiny, 0, 0, st, stream=s)),
        ("tiny rank 3, split step, inf at step 2",
         lambda s: run_window(tiny_skip, 3, 0, st, fused=False, stream=s)),
        ("tiny bf16 rank 1", lambda s: run_window(bf16, 1, 0, sb, stream=s)),
        ("GPT-2 rank 1 window, single pass",
         lambda s: run_window(gpt2, 1, shard - (1 << 20) - 5, (1 << 20) + 5, steps=3,
                              one_pass=True, stream=s)),
        ("tiny FSDP units, all ranks", lambda s: run_units_all_ranks(synth.TINY_FSDP, stream=s)),
    ]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("rounds", [2])
def test_concurrent_streams_and_threads_match_oracle(rounds):
    jobs = _jobs()
    print(f"[concurrent: {len(jobs)} threads x {rounds} rounds]", flush=True)
    streams = [torch.cuda.Stream() for _ in jobs]

    def run(i):
        name, fn = jobs[i]
        with torch.cuda.stream(streams[i]):
            fn(streams[i])
        return name

    for r in range(rounds):
        with ThreadPoolExecutor(len(jobs)) as ex:
            futs = [ex.submit(run, i) for i in range(len(jobs))]
            for f in futs:
                print(f"  round {r}: {f.result()} ok", flush=True)
    torch.cuda.synchronize()
