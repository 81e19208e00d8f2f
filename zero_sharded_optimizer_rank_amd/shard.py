"""One rank's shard on one GPU: device buffers, seeded input feeding, step calls.

PyTorch supplies device memory, pinned host memory and the stream; the work of
the step runs in libzero_shard.so through ``abi``.  Inputs come from the
seeded generator in ``synth`` (host, pinned staging, async copies).

A ``DeviceShard`` can hold a window [begin, begin+count) of the rank's shard
instead of the whole shard: the kernels then treat the window as the shard,
which is how parity runs at sizes the oracle finishes quickly.  The fp16 slot
keeps the misalignment it has in the real flat buffer (flat16 + rank*S +
begin), and guard words on either side catch stray writes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

import synth

from . import abi

GUARD = 64  # fp16 guard elements on each side of the slot
GUARD_WORD = 0x5A5A
CHUNK = 1 << 25  # elements per host staging chunk
ROW_ALIGN = 128  # contribution rows start on 256-byte boundaries (whole cache lines)
STAGGER = 4096  # consecutive buffers of the arena are offset by 4 KiB ...
STAGGER_PERIOD = 1 << 16  # ... modulo 64 KiB


def round_up(x: int, a: int) -> int:
    return (x + a - 1) // a * a


class DeviceShard:
    def __init__(self, w: synth.Workload, rank: int, begin: int = 0, count: Optional[int] = None,
                 device: str = "cuda:0", stream: Optional[torch.cuda.Stream] = None,
                 row_align: int = ROW_ALIGN, device_state: bool = True, one_pass: bool = False):
        self.w = w
        self.rank = rank
        self.device = torch.device(device)
        full_plan, self.offsets = abi.zero_plan(w.numels, w.world_size)
        self.full_plan = full_plan
        s_full = full_plan.shard
        if count is None:
            count = s_full - begin
        if not (0 <= begin and begin + count <= s_full):
            raise ValueError("window outside the shard")
        self.begin, self.count = begin, count
        if w.dtype not in ("fp16", "bf16"):
            raise ValueError(f"unknown gradient format {w.dtype!r}")
        self.bf16 = w.dtype == "bf16"
        self.flat_begin = rank * s_full + begin  # flat index of the window's first element
        real = max(0, min(count, w.psi - self.flat_begin))
        n = w.world_size
        self.plan = abi.zero_plan_t(real, n, 1, count, count * n)
        self.stream = stream or torch.cuda.current_stream(self.device)
        ld = round_up(max(count, 1), row_align)
        self.ld = ld
        # One arena holds every stream of the step.  Consecutive buffers start
        # 4 KiB apart modulo 64 KiB: with power-of-two-aligned starts the same
        # element of every stream falls on the same HBM channel interleave and
        # the multi-stream kernels lose a few percent.
        e = max(count, 1)
        self.row_pitch = round_up(2 * ld, STAGGER_PERIOD) + STAGGER
        st_pitch = round_up(4 * e, STAGGER_PERIOD) + STAGGER
        # one_pass: a second master/m/v set and slot for zero_reduce_adam_step_1pass,
        # which writes the other set and leaves the current one as it was
        self.one_pass = one_pass and device_state
        n_state = (7 if self.one_pass else 4) if device_state else 1
        rows_end = round_up(n * self.row_pitch, STAGGER_PERIOD)
        slot_elems = GUARD + 8 + count + GUARD
        slot_at = round_up(rows_end + n_state * st_pitch, STAGGER_PERIOD) + STAGGER
        slot2_at = slot_at + round_up(2 * slot_elems, STAGGER_PERIOD) + STAGGER
        end = (slot2_at if self.one_pass else slot_at) + 2 * slot_elems
        self.arena = torch.empty(end, dtype=torch.uint8, device=self.device)
        a16 = self.arena.view(torch.int16)
        self.contrib = a16.as_strided((n, ld), (self.row_pitch // 2, 1), 0)

        def state(k):
            o = rows_end + k * st_pitch
            return self.arena[o:o + 4 * e].view(torch.float32)
        self.grad = state(0)
        if device_state:
            self.master, self.m, self.v = state(1), state(2), state(3)
            self.m.zero_()
            self.v.zero_()
        else:
            self.master = self.m = self.v = None
        if self.one_pass:
            self.master2, self.m2, self.v2 = state(4), state(5), state(6)
        # slot with the real buffer's alignment (flat_begin mod 8) plus guards
        self.mis = self.flat_begin % 8
        self.slot_buf = self.arena[slot_at:slot_at + 2 * slot_elems].view(torch.int16)
        self.slot_buf.fill_(GUARD_WORD)
        self.slot_off = GUARD + self.mis
        self.slot_buf2 = None
        if self.one_pass:
            # same alignment as the first slot: both buffers start on 4 KiB boundaries
            self.slot_buf2 = self.arena[slot2_at:slot2_at + 2 * slot_elems].view(torch.int16)
            self.slot_buf2.fill_(GUARD_WORD)
        self.ws = torch.zeros(abi.zero_workspace_bytes(self.plan), dtype=torch.uint8,
                              device=self.device)
        self.res = torch.zeros(abi.RESULT_BYTES, dtype=torch.uint8, device=self.device)
        chunk = min(CHUNK, max(count, 1))
        self._pin16 = [torch.empty(chunk, dtype=torch.int16, pin_memory=True) for _ in range(2)]
        self._pin32 = torch.empty(chunk, dtype=torch.float32, pin_memory=True)
        self._chunk = chunk
        self._ev = [torch.cuda.Event() for _ in range(2)]

    # ------------------------------------------------------------------ views
    @property
    def slot(self) -> torch.Tensor:
        return self.slot_buf[self.slot_off:self.slot_off + self.count]

    def slot_ptr(self) -> int:
        return self.slot_buf.data_ptr() + 2 * self.slot_off

    def contrib_ptrs(self):
        base = self.arena.data_ptr()
        return [base + self.row_pitch * r for r in range(self.w.world_size)]

    def guards_intact(self) -> bool:
        for b in (self.slot_buf, self.slot_buf2):
            if b is None:
                continue
            lo = b[:self.slot_off]
            hi = b[self.slot_off + self.count:]
            if not ((lo == GUARD_WORD).all().item() and (hi == GUARD_WORD).all().item()):
                return False
        return True

    # ---------------------------------------------------------------- feeding
    def _feed16(self, row: torch.Tensor, fill):
        """Fill a device int16 row of self.count elements chunk by chunk."""
        with torch.cuda.stream(self.stream):
            for i, s in enumerate(range(0, self.count, self._chunk)):
                k = min(self._chunk, self.count - s)
                buf = self._pin16[i % 2]
                self._ev[i % 2].synchronize()
                fill(s, k, buf.numpy()[:k].view(np.uint16))
                row[s:s + k].copy_(buf[:k], non_blocking=True)
                self._ev[i % 2].record(self.stream)
        self.stream.synchronize()

    def load_contributions(self, step: int, loss_scale: float):
        """Rank q's row: the window of rank q's scaled fp16 gradient at `step`."""
        for q in range(self.w.world_size):
            def fill(s, k, out, q=q):
                synth.contributions(self.w, step, q, self.flat_begin + s, k, loss_scale, out=out)
            self._feed16(self.contrib[q], fill)

    def load_initial_state(self):
        """Seeded fp32 masters, m = v = 0, and the slot = fp16 (or bf16) of the
        master, rounded to nearest even."""
        with torch.cuda.stream(self.stream):
            for s in range(0, self.count, self._chunk):
                k = min(self._chunk, self.count - s)
                synth.masters(self.w, self.flat_begin + s, k, out=self._pin32.numpy()[:k])
                self.master[s:s + k].copy_(self._pin32[:k], non_blocking=True)
                self.stream.synchronize()
            self.m.zero_()
            self.v.zero_()
            half = torch.bfloat16 if self.bf16 else torch.float16
            self.slot.copy_(self.master[:self.count].to(half).view(torch.int16))
        self.stream.synchronize()

    # ------------------------------------------------------------------ steps
    def args(self, step_t: int, loss_scale: float, max_norm: Optional[float] = None,
             other_sq: float = 0.0, other_q: int = 0, other_overflow: bool = False):
        w = self.w
        return abi.step_args(lr=w.lr, beta1=w.betas[0], beta2=w.betas[1], eps=w.eps,
                             weight_decay=w.weight_decay,
                             max_grad_norm=w.max_grad_norm if max_norm is None else max_norm,
                             loss_scale=loss_scale, step=step_t, other_sq=other_sq,
                             other_q=other_q, other_overflow=other_overflow)

    def reduce_check(self, args):
        f = abi.zero_reduce_check_bf16 if self.bf16 else abi.zero_reduce_check
        f(self.plan, self.rank_in_plan, self.contrib_ptrs(), args, self.grad,
                              self.ws, self.ws.numel(), self.res, self.stream)

    def finalize(self, args):
        f = abi.zero_finalize_bf16 if self.bf16 else abi.zero_finalize
        f(self.plan, args, self.res, self.stream)

    def adam_apply(self, args):
        f = abi.zero_adam_apply_bf16 if self.bf16 else abi.zero_adam_apply
        f(self.plan, self.rank_in_plan, self.grad, self.master, self.m, self.v,
                            self.slot_ptr(), args, self.res, self.stream)

    def step(self, args):
        f = abi.zero_reduce_adam_step_bf16 if self.bf16 else abi.zero_reduce_adam_step
        f(self.plan, self.rank_in_plan, self.contrib_ptrs(), self.master,
                                  self.m, self.v, self.slot_ptr(), self.grad, self.ws,
                                  self.ws.numel(), args, self.res, self.stream)

    def step_1pass(self, args, res: Optional[torch.Tensor] = None, in_place_slot: bool = False):
        """zero_reduce_adam_step_1pass from the current master/m/v into the
        other set; adopt() makes that set current once the step is known not to
        have been skipped.  The new slot goes to the second slot buffer, or with
        `in_place_slot` into the live slot, which restore_slot() then repairs
        if the step was skipped."""
        if not self.one_pass:
            raise RuntimeError("this shard was built without the second state set")
        f = abi.zero_reduce_adam_step_1pass_bf16 if self.bf16 else abi.zero_reduce_adam_step_1pass
        slot_out = self.slot_ptr() if in_place_slot else \
            self.slot_buf2.data_ptr() + 2 * self.slot_off
        f(self.plan, self.rank_in_plan, self.contrib_ptrs(), self.master, self.m, self.v,
          self.master2, self.m2, self.v2, slot_out, self.ws, self.ws.numel(), args,
          self.res if res is None else res, self.stream)

    def restore_slot(self, res: Optional[torch.Tensor] = None):
        """zero_slot_restore on the live slot from the current master: a no-op
        unless the step in the result word was skipped."""
        f = abi.zero_slot_restore_bf16 if self.bf16 else abi.zero_slot_restore
        f(self.plan, self.rank_in_plan, self.master, self.slot_ptr(),
          self.res if res is None else res, self.stream)

    def adopt(self, swap_slot: bool = True):
        """Make the set the last step_1pass wrote the current one (with
        swap_slot=False after an in-place slot step)."""
        if not self.one_pass:
            raise RuntimeError("this shard was built without the second state set")
        self.master, self.master2 = self.master2, self.master
        self.m, self.m2 = self.m2, self.m
        self.v, self.v2 = self.v2, self.v
        if swap_slot:
            self.slot_buf, self.slot_buf2 = self.slot_buf2, self.slot_buf

    @property
    def rank_in_plan(self) -> int:
        return self.rank

    def result(self) -> abi.zero_step_result_t:
        self.stream.synchronize()
        raw = self.res.cpu().numpy().tobytes()
        return abi.zero_step_result_t.from_buffer_copy(raw)

    def fetch(self, name: str, idx=None) -> np.ndarray:
        """Copy a state array (or selected indexes of it) back to the host."""
        self.stream.synchronize()
        t = {"grad": self.grad, "master": self.master, "m": self.m, "v": self.v}.get(name)
        if name == "slot":
            t = self.slot
        else:
            t = t[:self.count]
        if idx is not None:
            t = t[torch.as_tensor(idx, device=self.device)]
        a = t.cpu().numpy()
        return a.view(np.uint16) if name == "slot" else a


def result_from_bytes(b: bytes) -> abi.zero_step_result_t:
    return abi.zero_step_result_t.from_buffer_copy(b)


__all__ = ["DeviceShard", "OffloadShard", "round_up", "result_from_bytes", "ctypes"]


class OffloadShard(DeviceShard):
    """The offload form of a rank's shard: contributions, g and the fp16 slot
    on the device; fp32 master, m and v in host memory (numpy arrays); pinned
    staging for the PCIe pipeline of zero_offload_adam_apply."""

    def __init__(self, w: synth.Workload, rank: int, begin: int = 0, count: Optional[int] = None,
                 chunk: int = 1 << 22, threads: Optional[int] = None, two_streams: bool = True,
                 **kw):
        super().__init__(w, rank, begin, count, device_state=False, **kw)
        if self.bf16:
            raise ValueError("the offload form takes fp16 contributions and slots")
        n = max(self.count, 1)
        self.h_master = np.zeros(n, dtype=np.float32)
        self.h_m = np.zeros(n, dtype=np.float32)
        self.h_v = np.zeros(n, dtype=np.float32)
        chunk = round_up(min(chunk, round_up(n, 64)), 64)
        self.chunk = chunk
        self._g_pin = torch.empty(2 * chunk, dtype=torch.float32, pin_memory=True)
        self._h_pin = torch.empty(2 * chunk, dtype=torch.int16, pin_memory=True)
        # a second stream (default priority) carries the fp16 chunks to the device
        self.upload_stream = torch.cuda.Stream(self.device) if two_streams else None
        self.staging = abi.offload_staging(self._g_pin, self._h_pin, chunk, self.upload_stream)
        # host memory saturates well before every core is busy; more threads
        # than 8 only add contention with the copies (measured 117 ms per
        # Llama-3-8B step with 8 threads against 116-162 ms with 16)
        self.threads = threads or max(1, min(8, len(os.sched_getaffinity(0))))

    def load_initial_state(self):
        synth.masters(self.w, self.flat_begin, self.count, out=self.h_master[:self.count])
        self.h_m[:] = 0
        self.h_v[:] = 0
        h16 = torch.from_numpy(self.h_master[:self.count].astype(np.float16).view(np.int16))
        with torch.cuda.stream(self.stream):
            self.slot.copy_(h16.to(self.device, non_blocking=False))
        self.stream.synchronize()

    def adam_apply(self, args):
        return abi.zero_offload_adam_apply(self.plan, self.rank, self.grad, self.h_master, self.h_m,
                                           self.h_v, self.slot_ptr(), args, self.res,
                                           self.staging, self.threads, self.stream)

    def step(self, args):
        return abi.zero_offload_step(self.plan, self.rank, self.contrib_ptrs(), self.grad, self.ws,
                                     self.ws.numel(), self.h_master, self.h_m, self.h_v,
                                     self.slot_ptr(), args, self.res, self.staging, self.threads,
                                     self.stream)

    def fetch(self, name: str, idx=None) -> np.ndarray:
        host = {"master": self.h_master, "m": self.h_m, "v": self.h_v}.get(name)
        if host is None:
            return super().fetch(name, idx)
        a = host[:self.count]
        return (a if idx is None else a[np.asarray(idx)]).copy()
