"""The 16-bit casts of the slot, for every fp32 bit pattern.

The update kernels and the slot restore share one fp32 -> fp16 / bf16
conversion per format (hardware conversion instructions of gfx950).  Here the
slot restore, forced to rewrite the slot (the result word says skip), casts
all 2^32 fp32 bit patterns in chunks of 2^28, and every result is compared
with the oracle's cast (its C form, pinned bitwise to the numpy definitions
on the CPU): bitwise for bf16, NaN included (round to nearest even, a NaN
keeps its top half with the quiet bit set); bitwise for fp16 on every non-NaN
input (round to nearest even, overflow to inf, subnormal results), and a NaN
of the same sign for a NaN input (the oracle leaves the NaN payload open).
"""
import numpy as np
import pytest

from oracle import fast

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CHUNK = 1 << 28


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", ["fp16", "bf16"])
def test_slot_cast_every_fp32_pattern(fmt):
    import zero_sharded_optimizer_rank_amd.abi as abi

    print(f"[slot cast, every fp32 pattern, {fmt}]", flush=True)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    plan = abi.zero_plan_t(CHUNK, 1, 1, CHUNK, CHUNK)
    master = torch.empty(CHUNK, dtype=torch.float32, device=dev)
    slot = torch.empty(CHUNK, dtype=torch.int16, device=dev)
    res = torch.zeros(abi.RESULT_BYTES, dtype=torch.uint8, device=dev)
    args = abi.step_args(lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                         max_grad_norm=0.0, loss_scale=1.0, step=1, other_overflow=True)
    abi.zero_finalize(plan, args, res, stream)  # skip = 1: the restore rewrites the slot
    restore = abi.zero_slot_restore_bf16 if fmt == "bf16" else abi.zero_slot_restore
    host = torch.empty(CHUNK, dtype=torch.int32, pin_memory=True)
    back = torch.empty(CHUNK, dtype=torch.int16, pin_memory=True)
    hu = host.numpy().view(np.uint32)
    base = np.arange(CHUNK, dtype=np.uint32)
    for c0 in range(0, 1 << 32, CHUNK):
        np.add(base, np.uint32(c0), out=hu)
        master.view(torch.int32).copy_(host, non_blocking=True)
        restore(plan, 0, master, slot, res, stream)
        back.copy_(slot, non_blocking=True)
        stream.synchronize()
        x = hu.view(np.float32)
        got = back.numpy().view(np.uint16)
        want = fast.cast16(x, bf16=(fmt == "bf16"))
        if fmt == "bf16":
            bad = fast.count_unequal(got, want)
        else:
            nan = np.isnan(x)
            bad = fast.count_unequal(np.where(nan, 0, got).astype(np.uint16),
                                     np.where(nan, 0, want).astype(np.uint16))
            if nan.any():
                g16 = got[nan].view(np.float16)
                bad += int((~np.isnan(g16)).sum())
                bad += int((np.signbit(g16) != np.signbit(x[nan])).sum())
        assert bad == 0, (fmt, hex(c0), bad)
    r = abi.zero_step_result_t.from_buffer_copy(res.cpu().numpy().tobytes())
    assert r.skip
