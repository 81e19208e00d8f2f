"""One rank's FSDP / ZeRO-3 units on one GPU: per-unit device buffers, the
unit table in device memory, seeded input feeding, and the one-launch step
through the C ABI (zero_units_*).

Each unit has buffers of its own (rows, g, master, m, v, slot), all carved
from one device arena at staggered starts.  The unit's fp16 slot keeps the
alignment it has in the unit's flat fp16 buffer (rank * S_u mod 8 elements),
with guard words around it.  Inputs come from ``synth`` by model element; the element each position
holds follows the library's own unit plan (zero_plan_units).
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

import synth

from . import abi
from .shard import GUARD, GUARD_WORD, ROW_ALIGN, STAGGER, STAGGER_PERIOD, round_up

CHUNK = 1 << 24



class DeviceUnits:
    def __init__(self, w: synth.Workload, rank: int, device: str = "cuda:0",
                 stream: Optional[torch.cuda.Stream] = None, one_pass: bool = False,
                 in_place_slot: bool = False):
        assert w.units is not None
        if w.dtype != "fp16":
            raise ValueError("the unit path takes fp16 contributions and slots")
        self.w, self.rank = w, rank
        self.device = torch.device(device)
        self.stream = stream or torch.cuda.current_stream(self.device)
        self.plan, self.infos = abi.zero_plan_units(w.numels, w.units, w.world_size)
        n = w.world_size
        self.n_units = len(self.infos)
        self.table = abi.unit_table(self.n_units)
        self.bufs: List[dict] = []
        # One arena, laid out by stream: the contribution rows of all units
        # side by side (row r of unit u at row r of one wide matrix), then one
        # region each for g, master, m and v holding every unit's piece, then
        # the slots.  Each stream of a unit thus sits as far from the unit's
        # other streams as in the flat layout (a whole rank's worth), and the
        # regions start 4 KiB apart modulo 64 KiB.  Unit pieces start on
        # 128-element boundaries.
        pads = [round_up(max(info.shard, 1), ROW_ALIGN) for info in self.infos]
        offs = [0]
        for pd in pads[:-1]:
            offs.append(offs[-1] + pd)
        total = max(sum(pads), ROW_ALIGN)
        row_pitch = round_up(2 * total, STAGGER_PERIOD) + STAGGER
        ld = row_pitch // 2
        st_pitch = round_up(4 * total, STAGGER_PERIOD) + STAGGER
        rows_end = round_up(n * row_pitch, STAGGER_PERIOD)
        # one_pass: master, m, v and the slots once more, for the set that
        # zero_units_step_1pass writes
        self.one_pass = one_pass
        # with in_place_slot both tables point param16 at the live slots, and
        # restore_slot() repairs them after a skipped single pass
        self.in_place_slot = one_pass and in_place_slot
        n_st = 7 if one_pass else 4
        st_at = [rows_end + k * st_pitch for k in range(n_st)]
        slots_at = round_up(rows_end + n_st * st_pitch, STAGGER_PERIOD) + STAGGER
        slot_elems = [GUARD + 8 + info.shard + GUARD for info in self.infos]
        # each unit's slot buffer starts on a 256-byte boundary, so a slot
        # with no misalignment (rank * S_u % 8 == 0) covers whole cache lines
        slot_offs = [0]
        for se in slot_elems[:-1]:
            slot_offs.append(slot_offs[-1] + round_up(se, ROW_ALIGN))
        slots_bytes = 2 * (slot_offs[-1] + round_up(slot_elems[-1], ROW_ALIGN)
                           if slot_elems else 0)
        slots2_at = slots_at + round_up(slots_bytes, STAGGER_PERIOD) + STAGGER
        nbytes = (slots2_at if one_pass else slots_at) + slots_bytes
        self.arena = torch.zeros(max(nbytes, 2), dtype=torch.uint8, device=self.device)
        a16 = self.arena.view(torch.int16)
        self.ld = ld
        self.row_pitch = row_pitch
        for u, info in enumerate(self.infos):
            s = info.shard
            e = max(s, 1)
            mis = (rank * s) % 8

            def f32(k):
                at = st_at[k] + 4 * offs[u]
                return self.arena[at:at + 4 * e].view(torch.float32)
            sa = slots_at + 2 * slot_offs[u]
            b = {
                # padding columns must read +0 (the arena starts zeroed); real
                # columns are rewritten every step
                "contrib": a16.as_strided((n, pads[u]), (ld, 1), offs[u]),
                "grad": f32(0), "master": f32(1), "m": f32(2), "v": f32(3),
                "slot_buf": self.arena[sa:sa + 2 * slot_elems[u]].view(torch.int16),
                "slot_off": GUARD + mis, "shard": s, "ld": ld,
            }
            b["slot_buf"].fill_(GUARD_WORD)
            if one_pass:
                sa2 = slots2_at + 2 * slot_offs[u]
                b.update(master2=f32(4), m2=f32(5), v2=f32(6),
                         slot_buf2=self.arena[sa2:sa2 + 2 * slot_elems[u]].view(torch.int16))
                b["slot_buf2"].fill_(GUARD_WORD)
            self.bufs.append(b)
            t = self.table[u]
            t.contrib = self.arena.data_ptr() + 2 * offs[u]
            t.ld = ld
            t.grad, t.master = b["grad"].data_ptr(), b["master"].data_ptr()
            t.m, t.v = b["m"].data_ptr(), b["v"].data_ptr()
            t.param16 = b["slot_buf"].data_ptr() + 2 * b["slot_off"]
            t.shard = s
        self.reduce_blocks, self.adam_blocks = abi.zero_units_prepare(self.table, self.n_units)
        self.table_dev = self._to_device(self.table)
        self.table2 = self.table2_dev = None
        if one_pass:
            # the second table: the same units with the second state set
            self.table2 = abi.unit_table(self.n_units)
            for u, b in enumerate(self.bufs):
                t, t2 = self.table[u], self.table2[u]
                t2.contrib, t2.ld, t2.grad, t2.shard = t.contrib, t.ld, t.grad, t.shard
                t2.master, t2.m = b["master2"].data_ptr(), b["m2"].data_ptr()
                t2.v = b["v2"].data_ptr()
                t2.param16 = t.param16 if self.in_place_slot else \
                    b["slot_buf2"].data_ptr() + 2 * b["slot_off"]
            abi.zero_units_prepare(self.table2, self.n_units)
            self.table2_dev = self._to_device(self.table2)
        self.ws = torch.zeros(max(abi.zero_units_workspace_bytes(self.table, self.n_units), 16),
                              dtype=torch.uint8, device=self.device)
        self.res = torch.zeros(abi.RESULT_BYTES, dtype=torch.uint8, device=self.device)
        self._pin16 = torch.empty(CHUNK, dtype=torch.int16, pin_memory=True)
        self._pin32 = torch.empty(CHUNK, dtype=torch.float32, pin_memory=True)

    def _to_device(self, table) -> torch.Tensor:
        """Device memory for a unit table: every zero_units_* call writes the
        host table it checks there itself, so nothing is copied here."""
        return torch.empty(max(abi.UNIT_BUFFERS_BYTES * self.n_units, 8), dtype=torch.uint8,
                           device=self.device)

    # ---------------------------------------------------------------- layout
    def unit_real(self, u: int) -> int:
        info = self.infos[u]
        return max(0, min(info.shard, info.psi - self.rank * info.shard))

    def unit_model_start(self, u: int) -> int:
        info = self.infos[u]
        return info.flat_offset + self.rank * info.shard

    def real_count(self) -> int:
        return sum(self.unit_real(u) for u in range(self.n_units))

    def slot(self, u: int) -> torch.Tensor:
        b = self.bufs[u]
        return b["slot_buf"][b["slot_off"]:b["slot_off"] + b["shard"]]

    def guards_intact(self) -> bool:
        for u, b in enumerate(self.bufs):
            for key in ("slot_buf", "slot_buf2"):
                if key not in b:
                    continue
                lo = b[key][:b["slot_off"]]
                hi = b[key][b["slot_off"] + b["shard"]:]
                if not (bool((lo == GUARD_WORD).all().item()) and
                        bool((hi == GUARD_WORD).all().item())):
                    return False
        return True

    # --------------------------------------------------------------- feeding
    def load_initial_state(self):
        with torch.cuda.stream(self.stream):
            for u, b in enumerate(self.bufs):
                real, start = self.unit_real(u), self.unit_model_start(u)
                b["master"].zero_()
                for s0 in range(0, real, CHUNK):
                    k = min(CHUNK, real - s0)
                    synth.masters(self.w, start + s0, k, out=self._pin32.numpy()[:k])
                    b["master"][s0:s0 + k].copy_(self._pin32[:k], non_blocking=True)
                    self.stream.synchronize()
                b["m"].zero_()
                b["v"].zero_()
                s = b["shard"]
                self.slot(u).copy_(b["master"][:s].to(torch.float16).view(torch.int16))
        self.stream.synchronize()

    def load_contributions(self, step: int, loss_scale: float):
        with torch.cuda.stream(self.stream):
            for u, b in enumerate(self.bufs):
                real, start = self.unit_real(u), self.unit_model_start(u)
                for q in range(self.w.world_size):
                    for s0 in range(0, real, CHUNK):
                        k = min(CHUNK, real - s0)
                        synth.contributions(self.w, step, q, start + s0, k, loss_scale,
                                            out=self._pin16.numpy()[:k].view(np.uint16))
                        b["contrib"][q, s0:s0 + k].copy_(self._pin16[:k], non_blocking=True)
                        self.stream.synchronize()
        self.stream.synchronize()

    # ----------------------------------------------------------------- steps
    def args(self, step_t: int, loss_scale: float, max_norm: Optional[float] = None,
             other_sq: float = 0.0, other_q: int = 0, other_overflow: bool = False):
        w = self.w
        return abi.step_args(lr=w.lr, beta1=w.betas[0], beta2=w.betas[1], eps=w.eps,
                             weight_decay=w.weight_decay,
                             max_grad_norm=w.max_grad_norm if max_norm is None else max_norm,
                             loss_scale=loss_scale, step=step_t, other_sq=other_sq,
                             other_q=other_q, other_overflow=other_overflow)

    def reduce_check(self, args):
        abi.zero_units_reduce_check(self.w.world_size, self.table, self.table_dev, self.n_units,
                                    args, self.ws, self.ws.numel(), self.res, self.stream)

    def adam_apply(self, args):
        abi.zero_units_adam_apply(self.table, self.table_dev, self.n_units, args, self.res,
                                  self.stream)

    def step(self, args):
        abi.zero_units_step(self.w.world_size, self.table, self.table_dev, self.n_units, args,
                            self.ws, self.ws.numel(), self.res, self.stream)

    def step_1pass(self, args, res: Optional[torch.Tensor] = None):
        """zero_units_step_1pass from the current set into the other one;
        adopt() makes it current once the step is known not to have been
        skipped."""
        if not self.one_pass:
            raise RuntimeError("these units were built without the second state set")
        abi.zero_units_step_1pass(self.w.world_size, self.table, self.table_dev, self.table2,
                                  self.table2_dev, self.n_units, args, self.ws, self.ws.numel(),
                                  self.res if res is None else res, self.stream)

    def restore_slot(self, res: Optional[torch.Tensor] = None):
        """zero_units_slot_restore on the live slots from the current masters:
        a no-op unless the step in the result word was skipped."""
        abi.zero_units_slot_restore(self.table, self.table_dev, self.n_units,
                                    self.res if res is None else res, self.stream)

    def adopt(self):
        """Make the set the last step_1pass wrote the current one."""
        if not self.one_pass:
            raise RuntimeError("these units were built without the second state set")
        self.table, self.table2 = self.table2, self.table
        self.table_dev, self.table2_dev = self.table2_dev, self.table_dev
        swapped = ("master", "m", "v") if self.in_place_slot else ("master", "m", "v", "slot_buf")
        for b in self.bufs:
            for x in swapped:
                b[x], b[x + "2"] = b[x + "2"], b[x]

    def result(self) -> abi.zero_step_result_t:
        self.stream.synchronize()
        return abi.zero_step_result_t.from_buffer_copy(self.res.cpu().numpy().tobytes())

    def locate(self, pos: np.ndarray):
        """(unit, offset inside the unit) of positions in the rank's concatenation."""
        offs = np.array([i.rank_offset for i in self.infos], dtype=np.int64)
        u = np.searchsorted(offs, pos, side="right") - 1
        return u, pos - offs[u]

    def fetch_at(self, name: str, pos: np.ndarray) -> np.ndarray:
        """Values of a state array at positions of the rank's concatenation."""
        self.stream.synchronize()
        u, j = self.locate(np.asarray(pos, dtype=np.int64))
        out = np.zeros(len(pos), dtype=np.uint16 if name == "slot" else np.float32)
        for uu in np.unique(u):
            sel = np.flatnonzero(u == uu)
            t = self.slot(int(uu)) if name == "slot" else self.bufs[int(uu)][name]
            vals = t[torch.as_tensor(j[sel], device=self.device)].cpu().numpy()
            out[sel] = vals.view(np.uint16) if name == "slot" else vals
        return out

    def fetch(self, name: str) -> np.ndarray:
        """The rank's concatenation over units (unit order) of a state array."""
        self.stream.synchronize()
        parts = []
        for u, b in enumerate(self.bufs):
            s = b["shard"]
            t = self.slot(u) if name == "slot" else b[name][:s]
            parts.append(t.cpu().numpy())
        a = np.concatenate(parts) if parts else np.zeros(0)
        return a.view(np.uint16) if name == "slot" else a
