"""ctypes binding of libzero_shard.so: the C ABI's entry points under the same
names, with argument marshalling only.  Every step of the shard step runs in
the library's HIP kernels; this module never computes any of it.

Device buffers are passed as integer addresses or as objects with a
``data_ptr()`` method (torch tensors); streams as integer handles or objects
with a ``cuda_stream`` attribute (torch streams).
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Sequence, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("ZERO_SHARD_LIB") or os.path.join(HERE, "libzero_shard.so")

ZERO_OK, ZERO_EINVAL, ZERO_EALIGN, ZERO_ENOSPC, ZERO_EHIP = 0, -1, -2, -3, -4
ZERO_MAX_RANKS = 64
ZERO_MAX_SHARD = 0x7FFFFFF8
ZERO_NOALLOC_MAX_SHARD = 9 << 27


class ZeroError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"zero_shard error {code}: {msg}")
        self.code = code


class zero_plan_t(ctypes.Structure):
    _fields_ = [("psi", ctypes.c_int64), ("world_size", ctypes.c_int64),
                ("align", ctypes.c_int64), ("shard", ctypes.c_int64),
                ("psi_padded", ctypes.c_int64)]


class zero_segment_t(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("tensor_begin", ctypes.c_int64), ("shard_begin", ctypes.c_int64),
                ("length", ctypes.c_int64)]


class zero_step_args_t(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("max_grad_norm", ctypes.c_double), ("loss_scale", ctypes.c_double),
                ("step", ctypes.c_int64), ("other_sq", ctypes.c_double),
                ("other_q_lo", ctypes.c_uint64), ("other_q_hi", ctypes.c_uint64),
                ("other_overflow", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class zero_step_result_t(ctypes.Structure):
    _fields_ = [("own_q_lo", ctypes.c_uint64), ("own_q_hi", ctypes.c_uint64),
                ("own_sq", ctypes.c_double), ("total_sq", ctypes.c_double),
                ("norm", ctypes.c_double), ("clip_coef", ctypes.c_float),
                ("overflow", ctypes.c_int32), ("skip", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]

    @property
    def own_q(self) -> int:
        return (int(self.own_q_hi) << 64) | int(self.own_q_lo)


class zero_scaler_t(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_double), ("growth", ctypes.c_double),
                ("backoff", ctypes.c_double), ("min_scale", ctypes.c_double),
                ("growth_interval", ctypes.c_int64), ("good_steps", ctypes.c_int64),
                ("t", ctypes.c_int64)]


class zero_unit_plan_t(ctypes.Structure):
    _fields_ = [("n_units", ctypes.c_int64), ("world_size", ctypes.c_int64),
                ("align", ctypes.c_int64), ("psi", ctypes.c_int64),
                ("rank_shard", ctypes.c_int64)]


class zero_unit_info_t(ctypes.Structure):
    _fields_ = [("psi", ctypes.c_int64), ("shard", ctypes.c_int64),
                ("flat_offset", ctypes.c_int64), ("rank_offset", ctypes.c_int64)]


class zero_unit_buffers_t(ctypes.Structure):
    _fields_ = [("contrib", ctypes.c_void_p), ("ld", ctypes.c_int64), ("grad", ctypes.c_void_p),
                ("master", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("param16", ctypes.c_void_p), ("shard", ctypes.c_int64),
                ("reduce_block", ctypes.c_int64), ("adam_block", ctypes.c_int64)]


class zero_offload_staging_t(ctypes.Structure):
    _fields_ = [("grad_pinned", ctypes.c_void_p), ("param16_pinned", ctypes.c_void_p),
                ("chunk", ctypes.c_int64), ("upload_stream", ctypes.c_void_p)]


RESULT_BYTES = ctypes.sizeof(zero_step_result_t)
UNIT_BUFFERS_BYTES = ctypes.sizeof(zero_unit_buffers_t)

# (name, restype, argtypes) for every symbol the header declares
_P = ctypes.POINTER
_vp = ctypes.c_void_p
_SIGNATURES = {
    "zero_plan": (ctypes.c_int, [_P(ctypes.c_int64), ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_int32, _P(zero_plan_t), _P(ctypes.c_int64)]),
    "zero_plan_real": (ctypes.c_int64, [_P(zero_plan_t), ctypes.c_int32]),
    "zero_plan_segments": (ctypes.c_int, [_P(zero_plan_t), _P(ctypes.c_int64), _P(ctypes.c_int64),
                                          ctypes.c_int32, ctypes.c_int32, _P(zero_segment_t),
                                          ctypes.c_int32, _P(ctypes.c_int32)]),
    "zero_state_bytes": (ctypes.c_double, [ctypes.c_int32, ctypes.c_double, ctypes.c_double,
                                           ctypes.c_double]),
    "zero_workspace_bytes": (ctypes.c_size_t, [_P(zero_plan_t)]),
    "zero_reduce_check": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32, _P(_vp),
                                         _P(zero_step_args_t), _vp, _vp, ctypes.c_size_t, _vp,
                                         _vp]),
    "zero_finalize": (ctypes.c_int, [_P(zero_plan_t), _P(zero_step_args_t), _vp, _vp]),
    "zero_adam_apply": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32, _vp, _vp, _vp, _vp, _vp,
                                       _P(zero_step_args_t), _vp, _vp]),
    "zero_reduce_adam_step": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32, _P(_vp), _vp, _vp,
                                             _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                             _P(zero_step_args_t), _vp, _vp]),
    "zero_reduce_adam_step_noalloc": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32, _P(_vp),
                                                     _vp, _vp, _vp, _vp, _vp,
                                                     _P(zero_step_args_t), _vp, _vp]),
    "zero_reduce_adam_step_1pass": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32, _P(_vp),
                                                   _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                   ctypes.c_size_t, _P(zero_step_args_t), _vp,
                                                   _vp]),
    "zero_reduce_adam_step_1pass_bf16": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32,
                                                        _P(_vp), _vp, _vp, _vp, _vp, _vp, _vp,
                                                        _vp, _vp, ctypes.c_size_t,
                                                        _P(zero_step_args_t), _vp, _vp]),
    "zero_slot_restore": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32, _vp, _vp, _vp, _vp]),
    "zero_slot_restore_bf16": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32, _vp, _vp, _vp,
                                              _vp]),
    "zero_reduce_check_bf16": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32, _P(_vp),
                                              _P(zero_step_args_t), _vp, _vp, ctypes.c_size_t,
                                              _vp, _vp]),
    "zero_finalize_bf16": (ctypes.c_int, [_P(zero_plan_t), _P(zero_step_args_t), _vp, _vp]),
    "zero_adam_apply_bf16": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32, _vp, _vp, _vp, _vp,
                                            _vp, _P(zero_step_args_t), _vp, _vp]),
    "zero_reduce_adam_step_bf16": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32, _P(_vp),
                                                  _vp, _vp, _vp, _vp, _vp, _vp,
                                                  ctypes.c_size_t, _P(zero_step_args_t), _vp,
                                                  _vp]),
    "zero_offload_staging_bytes": (ctypes.c_size_t, [ctypes.c_int64]),
    "zero_host_adam_apply": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int64,
                                            _P(zero_step_args_t), ctypes.c_float, ctypes.c_int32,
                                            ctypes.c_int32]),
    "zero_offload_adam_apply": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32, _vp, _vp, _vp,
                                               _vp, _vp, _P(zero_step_args_t), _vp,
                                               _P(zero_offload_staging_t), ctypes.c_int32,
                                               _P(zero_step_result_t), _vp]),
    "zero_offload_step": (ctypes.c_int, [_P(zero_plan_t), ctypes.c_int32, _P(_vp), _vp, _vp,
                                         ctypes.c_size_t, _vp, _vp, _vp, _vp,
                                         _P(zero_step_args_t), _vp, _P(zero_offload_staging_t),
                                         ctypes.c_int32, _P(zero_step_result_t), _vp]),
    "zero_plan_units": (ctypes.c_int, [_P(ctypes.c_int64), ctypes.c_int32, _P(ctypes.c_int32),
                                       ctypes.c_int32, ctypes.c_int32, _P(zero_unit_plan_t),
                                       _P(zero_unit_info_t), ctypes.c_int32]),
    "zero_units_prepare": (ctypes.c_int, [_P(zero_unit_buffers_t), ctypes.c_int32,
                                          _P(ctypes.c_int64), _P(ctypes.c_int64)]),
    "zero_units_workspace_bytes": (ctypes.c_size_t, [_P(zero_unit_buffers_t), ctypes.c_int32]),
    "zero_units_reduce_check": (ctypes.c_int, [ctypes.c_int32, _P(zero_unit_buffers_t), _vp,
                                               ctypes.c_int32, _P(zero_step_args_t), _vp,
                                               ctypes.c_size_t, _vp, _vp]),
    "zero_units_adam_apply": (ctypes.c_int, [_P(zero_unit_buffers_t), _vp, ctypes.c_int32,
                                             _P(zero_step_args_t), _vp, _vp]),
    "zero_units_step": (ctypes.c_int, [ctypes.c_int32, _P(zero_unit_buffers_t), _vp,
                                       ctypes.c_int32, _P(zero_step_args_t), _vp, ctypes.c_size_t,
                                       _vp, _vp]),
    "zero_units_step_1pass": (ctypes.c_int, [ctypes.c_int32, _P(zero_unit_buffers_t), _vp,
                                             _P(zero_unit_buffers_t), _vp, ctypes.c_int32,
                                             _P(zero_step_args_t), _vp, ctypes.c_size_t, _vp,
                                             _vp]),
    "zero_units_slot_restore": (ctypes.c_int, [_P(zero_unit_buffers_t), _vp, ctypes.c_int32,
                                               _vp, _vp]),
    "zero_scaler_update": (ctypes.c_int, [_P(zero_scaler_t), ctypes.c_int32]),
    "zero_last_error": (ctypes.c_char_p, []),
}


@functools.lru_cache(maxsize=None)
def lib() -> ctypes.CDLL:
    """Load the HIP library.  Fails loudly if it has not been built: there is
    no fallback path."""
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m zero_sharded_optimizer_rank_amd.build` "
                           "(or __graft_entry__.build())")
    so = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(so, name)
        fn.restype = res
        fn.argtypes = args
    return so


def _addr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "__array_interface__"):  # numpy array in host memory
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("host arrays passed to the library must be C-contiguous")
        return int(x.__array_interface__["data"][0])
    return int(x.data_ptr())


def _stream(s) -> int:
    if s is None:
        return 0
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _check(rc: int):
    if rc != ZERO_OK:
        raise ZeroError(rc, lib().zero_last_error().decode())


def zero_last_error() -> str:
    return lib().zero_last_error().decode()


def zero_plan(numels: Sequence[int], world_size: int, align: int = 1
              ) -> Tuple[zero_plan_t, Tuple[int, ...]]:
    n = len(numels)
    arr = (ctypes.c_int64 * max(n, 1))(*numels)
    offs = (ctypes.c_int64 * max(n, 1))()
    plan = zero_plan_t()
    _check(lib().zero_plan(arr, n, world_size, align, ctypes.byref(plan), offs))
    return plan, tuple(offs[i] for i in range(n))


def zero_plan_real(plan: zero_plan_t, rank: int) -> int:
    return int(lib().zero_plan_real(ctypes.byref(plan), rank))


def zero_plan_segments(plan: zero_plan_t, numels: Sequence[int], offsets: Sequence[int],
                       rank: int):
    n = len(numels)
    arr = (ctypes.c_int64 * max(n, 1))(*numels)
    offs = (ctypes.c_int64 * max(n, 1))(*offsets)
    count = ctypes.c_int32()
    cap = max(n, 1)
    out = (zero_segment_t * cap)()
    _check(lib().zero_plan_segments(ctypes.byref(plan), arr, offs, n, rank, out, cap,
                                    ctypes.byref(count)))
    return [(s.tensor, s.tensor_begin, s.shard_begin, s.length) for s in out[:count.value]]


def zero_state_bytes(stage: int, psi: float, n: float, k: float = 12.0) -> float:
    return float(lib().zero_state_bytes(stage, psi, n, k))


def zero_workspace_bytes(plan: zero_plan_t) -> int:
    return int(lib().zero_workspace_bytes(ctypes.byref(plan)))


def step_args(*, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
              max_grad_norm: float, loss_scale: float, step: int, other_sq: float = 0.0,
              other_q: int = 0, other_overflow: bool = False) -> zero_step_args_t:
    if not 0 <= other_q < 2**128:
        raise ValueError("other_q must fit in 128 bits")
    return zero_step_args_t(lr, beta1, beta2, eps, weight_decay, max_grad_norm, loss_scale, step,
                            other_sq, other_q & (2**64 - 1), other_q >> 64,
                            1 if other_overflow else 0, 0)


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(len(ptrs), 1))()
    for i, p in enumerate(ptrs):
        arr[i] = _addr(p)
    return arr


def zero_reduce_check(plan, rank, contrib, args, grad_out, workspace, ws_bytes, dev_result,
                      stream=None):
    _check(lib().zero_reduce_check(ctypes.byref(plan), rank, _ptr_array(contrib),
                                   ctypes.byref(args), _addr(grad_out), _addr(workspace), ws_bytes,
                                   _addr(dev_result), _stream(stream)))


def zero_finalize(plan, args, dev_result, stream=None):
    _check(lib().zero_finalize(ctypes.byref(plan), ctypes.byref(args), _addr(dev_result),
                               _stream(stream)))


def zero_adam_apply(plan, rank, grad, master, m, v, param16_slot, args, dev_result, stream=None):
    _check(lib().zero_adam_apply(ctypes.byref(plan), rank, _addr(grad), _addr(master), _addr(m),
                                 _addr(v), _addr(param16_slot), ctypes.byref(args),
                                 _addr(dev_result), _stream(stream)))


def zero_reduce_adam_step(plan, rank, contrib, master, m, v, param16_slot, grad_out, workspace,
                          ws_bytes, args, dev_result, stream=None):
    _check(lib().zero_reduce_adam_step(ctypes.byref(plan), rank, _ptr_array(contrib),
                                       _addr(master), _addr(m), _addr(v), _addr(param16_slot),
                                       _addr(grad_out), _addr(workspace), ws_bytes,
                                       ctypes.byref(args), _addr(dev_result), _stream(stream)))


def zero_reduce_adam_step_noalloc(plan, rank, contrib, master, m, v, param16_slot, grad_out, args,
                                  dev_result, stream=None):
    _check(lib().zero_reduce_adam_step_noalloc(ctypes.byref(plan), rank, _ptr_array(contrib),
                                               _addr(master), _addr(m), _addr(v),
                                               _addr(param16_slot), _addr(grad_out),
                                               ctypes.byref(args), _addr(dev_result),
                                               _stream(stream)))


def zero_reduce_adam_step_1pass(plan, rank, contrib, master_in, m_in, v_in, master_out, m_out,
                                v_out, param16_slot_out, workspace, ws_bytes, args, dev_result,
                                stream=None):
    _check(lib().zero_reduce_adam_step_1pass(ctypes.byref(plan), rank, _ptr_array(contrib),
                                             _addr(master_in), _addr(m_in), _addr(v_in),
                                             _addr(master_out), _addr(m_out), _addr(v_out),
                                             _addr(param16_slot_out), _addr(workspace), ws_bytes,
                                             ctypes.byref(args), _addr(dev_result),
                                             _stream(stream)))


def zero_reduce_adam_step_1pass_bf16(plan, rank, contrib, master_in, m_in, v_in, master_out,
                                     m_out, v_out, param_bf16_slot_out, workspace, ws_bytes, args,
                                     dev_result, stream=None):
    _check(lib().zero_reduce_adam_step_1pass_bf16(ctypes.byref(plan), rank, _ptr_array(contrib),
                                                  _addr(master_in), _addr(m_in), _addr(v_in),
                                                  _addr(master_out), _addr(m_out),
                                                  _addr(v_out), _addr(param_bf16_slot_out),
                                                  _addr(workspace), ws_bytes,
                                                  ctypes.byref(args), _addr(dev_result),
                                                  _stream(stream)))


def zero_slot_restore(plan, rank, master, param16_slot, dev_result, stream=None):
    _check(lib().zero_slot_restore(ctypes.byref(plan), rank, _addr(master), _addr(param16_slot),
                                   _addr(dev_result), _stream(stream)))


def zero_slot_restore_bf16(plan, rank, master, param_bf16_slot, dev_result, stream=None):
    _check(lib().zero_slot_restore_bf16(ctypes.byref(plan), rank, _addr(master),
                                        _addr(param_bf16_slot), _addr(dev_result),
                                        _stream(stream)))


def zero_reduce_check_bf16(plan, rank, contrib, args, grad_out, workspace, ws_bytes, dev_result,
                           stream=None):
    _check(lib().zero_reduce_check_bf16(ctypes.byref(plan), rank, _ptr_array(contrib),
                                        ctypes.byref(args), _addr(grad_out), _addr(workspace),
                                        ws_bytes, _addr(dev_result), _stream(stream)))


def zero_finalize_bf16(plan, args, dev_result, stream=None):
    _check(lib().zero_finalize_bf16(ctypes.byref(plan), ctypes.byref(args), _addr(dev_result),
                                    _stream(stream)))


def zero_adam_apply_bf16(plan, rank, grad, master, m, v, param_bf16_slot, args, dev_result,
                         stream=None):
    _check(lib().zero_adam_apply_bf16(ctypes.byref(plan), rank, _addr(grad), _addr(master),
                                      _addr(m), _addr(v), _addr(param_bf16_slot),
                                      ctypes.byref(args), _addr(dev_result), _stream(stream)))


def zero_reduce_adam_step_bf16(plan, rank, contrib, master, m, v, param_bf16_slot, grad_out,
                               workspace, ws_bytes, args, dev_result, stream=None):
    _check(lib().zero_reduce_adam_step_bf16(ctypes.byref(plan), rank, _ptr_array(contrib),
                                            _addr(master), _addr(m), _addr(v),
                                            _addr(param_bf16_slot), _addr(grad_out),
                                            _addr(workspace), ws_bytes, ctypes.byref(args),
                                            _addr(dev_result), _stream(stream)))


def zero_offload_staging_bytes(chunk):
    return int(lib().zero_offload_staging_bytes(chunk))


def offload_staging(grad_pinned, param16_pinned, chunk, upload_stream=None):
    return zero_offload_staging_t(_addr(grad_pinned), _addr(param16_pinned), chunk,
                                  _stream(upload_stream))


def zero_host_adam_apply(grad, master, m, v, param16, count, args, clip_coef, threads=1,
                         vector_width=0):
    _check(lib().zero_host_adam_apply(_addr(grad), _addr(master), _addr(m), _addr(v),
                                      _addr(param16), count, ctypes.byref(args), clip_coef,
                                      threads, vector_width))


def zero_offload_adam_apply(plan, rank, grad_dev, master_host, m_host, v_host, param16_slot_dev,
                            args, dev_result, staging, threads=1, stream=None):
    out = zero_step_result_t()
    _check(lib().zero_offload_adam_apply(ctypes.byref(plan), rank, _addr(grad_dev),
                                         _addr(master_host), _addr(m_host), _addr(v_host),
                                         _addr(param16_slot_dev), ctypes.byref(args),
                                         _addr(dev_result), ctypes.byref(staging), threads,
                                         ctypes.byref(out), _stream(stream)))
    return out


def zero_offload_step(plan, rank, contrib, grad_dev, workspace, ws_bytes, master_host, m_host,
                      v_host, param16_slot_dev, args, dev_result, staging, threads=1,
                      stream=None):
    out = zero_step_result_t()
    _check(lib().zero_offload_step(ctypes.byref(plan), rank, _ptr_array(contrib), _addr(grad_dev),
                                   _addr(workspace), ws_bytes, _addr(master_host), _addr(m_host),
                                   _addr(v_host), _addr(param16_slot_dev), ctypes.byref(args),
                                   _addr(dev_result), ctypes.byref(staging), threads,
                                   ctypes.byref(out), _stream(stream)))
    return out


def zero_plan_units(numels: Sequence[int], unit_of_tensor: Sequence[int], world_size: int,
                    align: int = 1):
    n = len(numels)
    arr = (ctypes.c_int64 * max(n, 1))(*numels)
    uot = (ctypes.c_int32 * max(n, 1))(*unit_of_tensor)
    plan = zero_unit_plan_t()
    cap = max(n, 1)
    infos = (zero_unit_info_t * cap)()
    _check(lib().zero_plan_units(arr, n, uot, world_size, align, ctypes.byref(plan), infos, cap))
    return plan, [infos[i] for i in range(plan.n_units)]


def unit_table(n_units: int):
    return (zero_unit_buffers_t * max(n_units, 1))()


def zero_units_prepare(table, n_units: int) -> Tuple[int, int]:
    b1, b2 = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().zero_units_prepare(table, n_units, ctypes.byref(b1), ctypes.byref(b2)))
    return b1.value, b2.value


def zero_units_workspace_bytes(table, n_units: int) -> int:
    return int(lib().zero_units_workspace_bytes(table, n_units))


def zero_units_reduce_check(world_size, table_host, table_dev, n_units, args, workspace, ws_bytes,
                            dev_result, stream=None):
    _check(lib().zero_units_reduce_check(world_size, table_host, _addr(table_dev), n_units,
                                         ctypes.byref(args), _addr(workspace), ws_bytes,
                                         _addr(dev_result), _stream(stream)))


def zero_units_adam_apply(table_host, table_dev, n_units, args, dev_result, stream=None):
    _check(lib().zero_units_adam_apply(table_host, _addr(table_dev), n_units, ctypes.byref(args),
                                       _addr(dev_result), _stream(stream)))


def zero_units_step(world_size, table_host, table_dev, n_units, args, workspace, ws_bytes,
                    dev_result, stream=None):
    _check(lib().zero_units_step(world_size, table_host, _addr(table_dev), n_units,
                                 ctypes.byref(args), _addr(workspace), ws_bytes,
                                 _addr(dev_result), _stream(stream)))


def zero_units_step_1pass(world_size, table_host, table_dev, out_host, out_dev, n_units, args,
                          workspace, ws_bytes, dev_result, stream=None):
    _check(lib().zero_units_step_1pass(world_size, table_host, _addr(table_dev), out_host,
                                       _addr(out_dev), n_units, ctypes.byref(args),
                                       _addr(workspace), ws_bytes, _addr(dev_result),
                                       _stream(stream)))


def zero_units_slot_restore(table_host, table_dev, n_units, dev_result, stream=None):
    _check(lib().zero_units_slot_restore(table_host, _addr(table_dev), n_units,
                                         _addr(dev_result), _stream(stream)))


def new_scaler(scale: float, growth: float = 2.0, backoff: float = 0.5, min_scale: float = 1.0,
               growth_interval: int = 1000) -> zero_scaler_t:
    return zero_scaler_t(scale, growth, backoff, min_scale, growth_interval, 0, 0)


def zero_scaler_update(s: zero_scaler_t, skipped: bool) -> zero_scaler_t:
    _check(lib().zero_scaler_update(ctypes.byref(s), 1 if skipped else 0))
    return s
