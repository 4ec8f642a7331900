"""ctypes binding of libfsdp_shard.so: the C ABI's functions under the same names.

Argument marshalling only: Python lists become int64 arrays, tensors become
their device addresses, torch streams become hipStream_t handles, and a
negative status becomes an ``FsdpError``.  Every step of the sharded path runs
in the HIP library; nothing here computes any part of it.  The library must be
built (``python -m sharded_shard_amd.build``); importing this module without it
raises ImportError.  FSDP_SHARD_LIB in the environment selects another build
of the same library (e.g. one compiled with different tile sizes).
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.environ.get("FSDP_SHARD_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "lib", "libfsdp_shard.so")

FSDP_OK = 0
FSDP_E_INVAL = -1
FSDP_E_UNSUPPORTED = -2
FSDP_E_ALIGN = -3
FSDP_E_STATE = -4
FSDP_E_HIP = -5
FSDP_E_NOMEM = -6

FSDP_ROLE_MASTER = 1
FSDP_ROLE_GRAD = 2
FSDP_ROLE_EXP_AVG = 4
FSDP_ROLE_EXP_AVG_SQ = 8
FSDP_ROLE_FULL = 16
FSDP_ROLE_FULL_GRAD = 32
FSDP_ROLE_GRAD_ACC = 64
FSDP_ROLE_FULL_FP8 = 128

FSDP_DTYPE_BF16 = 0
FSDP_DTYPE_F32 = 1

FSDP_STEP_WRITE_GRAD = 1
FSDP_STEP_UNFUSED = 2

FSDP_KERNEL_STEP = 0
FSDP_KERNEL_REDUCE = 1
FSDP_KERNEL_ADAMW = 2
FSDP_KERNEL_PACK = 3
FSDP_KERNEL_UNPACK = 4
FSDP_KERNEL_ADAMW_PACK = 5

FSDP_SET_ADAMW_COPY_IN = 1

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class ShardEntry(ctypes.Structure):
    _fields_ = [(n, _i64) for n in (
        "rows", "cols", "chunk_rows", "row_begin", "local_rows", "shard_offset",
        "shard_numel", "valid_numel", "pad_numel", "seg_numel")]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_params", _i32), ("world", _i32), ("rank", _i32), ("align_elems", _i32),
                ("S", _i64), ("V", _i64), ("F", _i64), ("pad_total", _i64),
                ("n_empty", _i32), ("bound", _i32), ("n_tiles", _i64 * 4)]


class ReshardRun(ctypes.Structure):
    _fields_ = [("param", _i32), ("src_rank", _i32), ("src_offset", _i64), ("dst_offset", _i64),
                ("numel", _i64)]


class AdamwHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


class FsdpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [{status}]")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run: python -m sharded_shard_amd.build")

# The library must use the same HIP runtime as torch, which allocates the
# tensors and owns the streams: torch ships its own libamdhip64 with the same
# soname, and loading torch first makes the dynamic linker reuse it instead
# of loading a second runtime from the system ROCm.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)

_SIGS = {
    "fsdp_abi_version": (_i32, []),
    "fsdp_status_string": (ctypes.c_char_p, [_i32]),
    "fsdp_last_error": (ctypes.c_char_p, []),
    "fsdp_plan_create": (_i32, [ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i32, _i32, _i32,
                                _i32, ctypes.POINTER(_P)]),
    "fsdp_plan_info": (_i32, [_P, ctypes.POINTER(PlanInfo)]),
    "fsdp_plan_entry": (_i32, [_P, _i32, ctypes.POINTER(ShardEntry)]),
    "fsdp_plan_rows_of_rank": (_i32, [_P, _i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "fsdp_state_bytes": (_i32, [ctypes.c_double, _i32, _i32, ctypes.POINTER(ctypes.c_double)]),
    "fsdp_plan_destroy": (None, [_P]),
    "fsdp_bind": (_i32, [_P, _PP, _PP, _PP, _PP, _PP, _P]),
    "fsdp_pack_allgather": (_i32, [_P, _P, _P]),
    "fsdp_unpack_allgather": (_i32, [_P, _P, _P]),
    "fsdp_reduce_shard": (_i32, [_P, _P, _P]),
    "fsdp_adamw_shard": (_i32, [_P, ctypes.POINTER(AdamwHparams), _i64, _P]),
    "fsdp_step_shard": (_i32, [_P, _P, _P, ctypes.POINTER(AdamwHparams), _i64, ctypes.c_uint32, _P]),
    "fsdp_bind_full_grad": (_i32, [_P, _PP, _P]),
    "fsdp_pack_reduce_scatter": (_i32, [_P, _P, _i32, _P]),
    "fsdp_bind_grad_acc": (_i32, [_P, _PP, _P]),
    "fsdp_bind_full_fp8": (_i32, [_P, _PP, _P]),
    "fsdp_pack_allgather_fp8": (_i32, [_P, _P, _P, _P]),
    "fsdp_unpack_allgather_fp8": (_i32, [_P, _P, _P]),
    "fsdp_amax_shard": (_i32, [_P, _P, _P]),
    "fsdp_accumulate_grad": (_i32, [_P, _i32, _P]),
    "fsdp_pack_reduce_scatter_acc": (_i32, [_P, _P, _P]),
    "fsdp_reduce_shard_f32": (_i32, [_P, _P, _P]),
    "fsdp_reshard_plan_create": (_i32, [ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i32, _i32,
                                        _i32, _i32, ctypes.POINTER(_P)]),
    "fsdp_reshard_plan_runs": (_i32, [_P, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "fsdp_reshard_plan_run": (_i32, [_P, _i64, ctypes.POINTER(ReshardRun)]),
    "fsdp_reshard_bind": (_i32, [_P, _PP, _PP, _i32, _P]),
    "fsdp_reshard_execute": (_i32, [_P, _P]),
    "fsdp_reshard_plan_destroy": (None, [_P]),
    "fsdp_adamw_host": (_i32, [_P, _P, _P, _P, _i64, ctypes.POINTER(AdamwHparams), _i64, _i32]),
    "fsdp_step_groups": (_i32, [_PP, _i32, _PP, _PP, _PP, ctypes.POINTER(AdamwHparams), _i64,
                                ctypes.c_uint32, _i32, _PP, _P]),
    "fsdp_group_set_create": (_i32, [_PP, _i32, _P, ctypes.POINTER(_P)]),
    "fsdp_group_set_destroy": (None, [_P]),
    "fsdp_group_set_info": (_i32, [_P, ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                                   ctypes.POINTER(_i64)]),
    "fsdp_amax_groups": (_i32, [_P, _P, _P]),
    "fsdp_pack_allgather_fp8_groups": (_i32, [_P, _P, _P, _P]),
    "fsdp_group_set_segment": (_i32, [_P, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "fsdp_adamw_groups": (_i32, [_P, ctypes.POINTER(AdamwHparams), _i64, _P]),
    "fsdp_pack_allgather_groups": (_i32, [_P, _P, _P]),
    "fsdp_adamw_pack_groups": (_i32, [_P, ctypes.POINTER(AdamwHparams), _i64, _P, _P]),
    "fsdp_step_group_set": (_i32, [_P, _PP, _P, _PP, ctypes.POINTER(AdamwHparams), _i64,
                                   ctypes.c_uint32, _i32, _PP, _P]),
    "fsdp_check_stream": (_i32, [_P]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def _check(status: int, call: str) -> None:
    if status != FSDP_OK:
        raise FsdpError(status, f"{call}: {fsdp_last_error()}")


def addr(x) -> int:
    """Device address of a tensor (or an int passed through); 0 for None."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x.ctypes.data)          # a NumPy array


def stream_handle(stream=None) -> int:
    """hipStream_t of a torch stream, an int handle, or torch's current stream."""
    if isinstance(stream, int):
        return stream
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    return int(stream.cuda_stream)


def _dims(plan):
    """(N, S, n_params) of a plan, or None for a null handle (the C call then
    reports it)."""
    if plan is None or getattr(plan, "value", 1) is None:
        return None
    info = fsdp_plan_info(plan)
    return info.world, info.S, info.n_params


def _dev(x, nbytes: int, what: str) -> int:
    """Device address of a buffer argument of at least ``nbytes`` bytes.

    The C ABI receives bare addresses and cannot see how large a buffer is, so
    a torch tensor is checked here before any launch: it must hold nbytes, be
    contiguous and live on the current GPU; otherwise ValueError.  An int is
    taken as an address whose size the caller vouches for; None is 0.
    """
    if x is None or isinstance(x, int):
        return addr(x)
    if not hasattr(x, "data_ptr"):
        raise TypeError(f"{what}: expected a torch tensor or an address")
    have = x.numel() * x.element_size()
    if have < nbytes:
        raise ValueError(f"{what} holds {have} bytes; this call reads or writes {nbytes}")
    if not x.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor (got device {x.device})")
    if not x.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    import torch
    if x.device.index != torch.cuda.current_device():
        raise ValueError(f"{what} is on {x.device}, not on the current device "
                         f"cuda:{torch.cuda.current_device()}")
    return int(x.data_ptr())


def _ptr_array(items):
    if items is None:
        return None
    arr = (ctypes.c_void_p * max(1, len(items)))()
    for i, t in enumerate(items):
        arr[i] = addr(t) or None
    return ctypes.cast(arr, _PP)


# ---- library ---------------------------------------------------------------

def fsdp_abi_version() -> int:
    return int(lib.fsdp_abi_version())


def fsdp_status_string(status: int) -> str:
    return lib.fsdp_status_string(status).decode()


def fsdp_last_error() -> str:
    return lib.fsdp_last_error().decode()


# ---- planner -------------------------------------------------------------------

def fsdp_plan_create(rows, cols, world: int, rank: int, align_elems: int = 1):
    """Returns an opaque plan handle (ctypes.c_void_p)."""
    n = len(rows)
    if len(cols) != n:
        raise ValueError("rows and cols differ in length")
    r = (_i64 * max(1, n))(*rows)
    c = (_i64 * max(1, n))(*cols)
    out = _P()
    _check(lib.fsdp_plan_create(r, c, n, world, rank, align_elems, ctypes.byref(out)),
           "fsdp_plan_create")
    return out


def fsdp_plan_info(plan) -> PlanInfo:
    info = PlanInfo()
    _check(lib.fsdp_plan_info(plan, ctypes.byref(info)), "fsdp_plan_info")
    return info


def fsdp_plan_entry(plan, i: int) -> ShardEntry:
    e = ShardEntry()
    _check(lib.fsdp_plan_entry(plan, i, ctypes.byref(e)), "fsdp_plan_entry")
    return e


def fsdp_plan_rows_of_rank(plan, i: int, j: int):
    b, lr = _i64(), _i64()
    _check(lib.fsdp_plan_rows_of_rank(plan, i, j, ctypes.byref(b), ctypes.byref(lr)),
           "fsdp_plan_rows_of_rank")
    return b.value, lr.value


def fsdp_state_bytes(n_params: float, world: int, zero_stage: int) -> float:
    out = ctypes.c_double()
    _check(lib.fsdp_state_bytes(float(n_params), world, zero_stage, ctypes.byref(out)),
           "fsdp_state_bytes")
    return out.value


def fsdp_plan_destroy(plan) -> None:
    lib.fsdp_plan_destroy(plan)


# ---- bind and hot path -----------------------------------------------------------

def fsdp_bind(plan, master=None, grad=None, exp_avg=None, exp_avg_sq=None, full=None,
              stream=None) -> None:
    """Each role is a list of tensors/addresses (one per parameter) or None."""
    _check(lib.fsdp_bind(plan, _ptr_array(master), _ptr_array(grad), _ptr_array(exp_avg),
                         _ptr_array(exp_avg_sq), _ptr_array(full), stream_handle(stream)),
           "fsdp_bind")


def fsdp_bind_full_grad(plan, full_grad, stream=None) -> None:
    _check(lib.fsdp_bind_full_grad(plan, _ptr_array(full_grad), stream_handle(stream)),
           "fsdp_bind_full_grad")


def fsdp_pack_reduce_scatter(plan, rs_out, dtype: int = FSDP_DTYPE_BF16, stream=None) -> None:
    d = _dims(plan)
    esize = 4 if dtype == FSDP_DTYPE_F32 else 2
    buf = _dev(rs_out, esize * d[0] * d[1], "rs_out") if d else addr(rs_out)
    _check(lib.fsdp_pack_reduce_scatter(plan, buf, dtype, stream_handle(stream)),
           "fsdp_pack_reduce_scatter")


def fsdp_bind_full_fp8(plan, full_fp8, stream=None) -> None:
    _check(lib.fsdp_bind_full_fp8(plan, _ptr_array(full_fp8), stream_handle(stream)),
           "fsdp_bind_full_fp8")


def fsdp_pack_allgather_fp8(plan, ag_in, scales, stream=None) -> None:
    d = _dims(plan)
    a = _dev(ag_in, d[1], "ag_in") if d else addr(ag_in)
    sc = _dev(scales, 4 * d[2], "scales") if d else addr(scales)
    _check(lib.fsdp_pack_allgather_fp8(plan, a, sc, stream_handle(stream)),
           "fsdp_pack_allgather_fp8")


def fsdp_unpack_allgather_fp8(plan, ag_out, stream=None) -> None:
    d = _dims(plan)
    a = _dev(ag_out, d[0] * d[1], "ag_out") if d else addr(ag_out)
    _check(lib.fsdp_unpack_allgather_fp8(plan, a, stream_handle(stream)),
           "fsdp_unpack_allgather_fp8")


def fsdp_amax_shard(plan, amax, stream=None) -> None:
    d = _dims(plan)
    a = _dev(amax, 4 * d[2], "amax") if d else addr(amax)
    _check(lib.fsdp_amax_shard(plan, a, stream_handle(stream)), "fsdp_amax_shard")


def fsdp_bind_grad_acc(plan, grad_acc, stream=None) -> None:
    _check(lib.fsdp_bind_grad_acc(plan, _ptr_array(grad_acc), stream_handle(stream)),
           "fsdp_bind_grad_acc")


def fsdp_accumulate_grad(plan, reset: bool, stream=None) -> None:
    _check(lib.fsdp_accumulate_grad(plan, 1 if reset else 0, stream_handle(stream)),
           "fsdp_accumulate_grad")


def fsdp_pack_reduce_scatter_acc(plan, rs_out, stream=None) -> None:
    d = _dims(plan)
    a = _dev(rs_out, 4 * d[0] * d[1], "rs_out") if d else addr(rs_out)
    _check(lib.fsdp_pack_reduce_scatter_acc(plan, a, stream_handle(stream)),
           "fsdp_pack_reduce_scatter_acc")


def fsdp_reduce_shard_f32(plan, rs_in, stream=None) -> None:
    d = _dims(plan)
    a = _dev(rs_in, 4 * d[0] * d[1], "rs_in") if d else addr(rs_in)
    _check(lib.fsdp_reduce_shard_f32(plan, a, stream_handle(stream)),
           "fsdp_reduce_shard_f32")


def fsdp_pack_allgather(plan, ag_in, stream=None) -> None:
    d = _dims(plan)
    a = _dev(ag_in, 2 * d[1], "ag_in") if d else addr(ag_in)
    _check(lib.fsdp_pack_allgather(plan, a, stream_handle(stream)), "fsdp_pack_allgather")


def fsdp_unpack_allgather(plan, ag_out, stream=None) -> None:
    d = _dims(plan)
    a = _dev(ag_out, 2 * d[0] * d[1], "ag_out") if d else addr(ag_out)
    _check(lib.fsdp_unpack_allgather(plan, a, stream_handle(stream)), "fsdp_unpack_allgather")


def fsdp_reduce_shard(plan, rs_in, stream=None) -> None:
    d = _dims(plan)
    a = _dev(rs_in, 2 * d[0] * d[1], "rs_in") if d else addr(rs_in)
    _check(lib.fsdp_reduce_shard(plan, a, stream_handle(stream)), "fsdp_reduce_shard")


def fsdp_adamw_shard(plan, lr: float, beta1: float, beta2: float, eps: float,
                     weight_decay: float, step: int, stream=None) -> None:
    hp = AdamwHparams(lr, beta1, beta2, eps, weight_decay)
    _check(lib.fsdp_adamw_shard(plan, ctypes.byref(hp), step, stream_handle(stream)),
           "fsdp_adamw_shard")


def fsdp_step_shard(plan, rs_in, ag_in, lr: float, beta1: float, beta2: float, eps: float,
                    weight_decay: float, step: int, flags: int = 0, stream=None) -> None:
    hp = AdamwHparams(lr, beta1, beta2, eps, weight_decay)
    d = _dims(plan)
    r = _dev(rs_in, 2 * d[0] * d[1], "rs_in") if d else addr(rs_in)
    a = _dev(ag_in, 2 * d[1], "ag_in") if d else addr(ag_in)
    _check(lib.fsdp_step_shard(plan, r, a, ctypes.byref(hp), step, flags,
                               stream_handle(stream)), "fsdp_step_shard")


def fsdp_adamw_host(p, g, m, v, lr: float, beta1: float, beta2: float, eps: float,
                    weight_decay: float, step: int, n_threads: int = 0) -> None:
    """p, g, m, v: contiguous fp32 host arrays (NumPy or CPU tensors) of equal size."""
    n = int(p.numel() if hasattr(p, "numel") and callable(p.numel) else p.size)
    for a in (g, m, v):
        k = int(a.numel() if hasattr(a, "numel") and callable(a.numel) else a.size)
        if k != n:
            raise ValueError("p, g, m and v must have the same size")
    hp = AdamwHparams(lr, beta1, beta2, eps, weight_decay)
    _check(lib.fsdp_adamw_host(addr(p), addr(g), addr(m), addr(v), n, ctypes.byref(hp), step,
                               n_threads), "fsdp_adamw_host")


def fsdp_reshard_plan_create(rows, cols, world_src: int, world_dst: int, rank_dst: int):
    n = len(rows)
    r = (_i64 * max(1, n))(*rows)
    c = (_i64 * max(1, n))(*cols)
    out = _P()
    _check(lib.fsdp_reshard_plan_create(r, c, n, world_src, world_dst, rank_dst, ctypes.byref(out)),
           "fsdp_reshard_plan_create")
    return out


def fsdp_reshard_plan_runs(plan):
    n, d = _i64(), _i64()
    _check(lib.fsdp_reshard_plan_runs(plan, ctypes.byref(n), ctypes.byref(d)), "fsdp_reshard_plan_runs")
    return n.value, d.value


def fsdp_reshard_plan_run(plan, i: int) -> ReshardRun:
    r = ReshardRun()
    _check(lib.fsdp_reshard_plan_run(plan, i, ctypes.byref(r)), "fsdp_reshard_plan_run")
    return r


def fsdp_reshard_bind(plan, src, dst, elem_bytes: int, stream=None) -> None:
    """src: flat list, parameter-major (param p, source rank s at p*world_src+s)."""
    _check(lib.fsdp_reshard_bind(plan, _ptr_array(src), _ptr_array(dst), elem_bytes,
                                 stream_handle(stream)), "fsdp_reshard_bind")


def fsdp_reshard_execute(plan, stream=None) -> None:
    _check(lib.fsdp_reshard_execute(plan, stream_handle(stream)), "fsdp_reshard_execute")


def fsdp_reshard_plan_destroy(plan) -> None:
    lib.fsdp_reshard_plan_destroy(plan)


class StepGroupsCall:
    """fsdp_step_groups with its pointer arrays marshalled once.

    plans: plan handles; rs_in, ag_in, ag_out: tensors/addresses per group
    (ag_out may be None to skip the copy-out).  Each call() passes only the
    step index, so the per-step host cost is one ctypes call.
    """

    def __init__(self, plans, rs_in, ag_in, ag_out, lr, beta1, beta2, eps, weight_decay,
                 flags=0, stream=None):
        n = len(plans)
        if len(rs_in) != n or len(ag_in) != n or (ag_out is not None and len(ag_out) != n):
            raise ValueError("plans, rs_in, ag_in and ag_out must have one entry per group")
        self.n = n
        self._plans = (ctypes.c_void_p * max(1, n))(*[p.value for p in plans])
        rs_p, in_p, out_p = [], [], []
        for g, p in enumerate(plans):      # tensors are size-checked once, here
            d = _dims(p)
            if d is None:
                rs_p.append(addr(rs_in[g]))
                in_p.append(addr(ag_in[g]))
                out_p.append(addr(ag_out[g]) if ag_out is not None else 0)
                continue
            rs_p.append(_dev(rs_in[g], 2 * d[0] * d[1], f"rs_in[{g}]"))
            in_p.append(_dev(ag_in[g], 2 * d[1], f"ag_in[{g}]"))
            if ag_out is not None:
                out_p.append(_dev(ag_out[g], 2 * d[0] * d[1], f"ag_out[{g}]"))
        self._rs = _ptr_array(rs_p)
        self._ag_in = _ptr_array(in_p)
        self._ag_out = _ptr_array(out_p) if ag_out is not None else None
        self._keep = (rs_in, ag_in, ag_out)
        self._hp = AdamwHparams(lr, beta1, beta2, eps, weight_decay)
        self.flags = flags
        self._stream = stream_handle(stream)

    def __call__(self, step: int, timed_kernel: int = 0, events=None) -> None:
        ev = None
        if events is not None:     # None entries leave that group untimed
            if len(events) != 2 * self.n:
                raise ValueError(f"events: need 2 per group ({2 * self.n}), got {len(events)}")
            ev = (ctypes.c_void_p * len(events))(
                *[int(e.cuda_event) if e is not None else None for e in events])
            ev = ctypes.cast(ev, _PP)
        _check(lib.fsdp_step_groups(ctypes.cast(self._plans, _PP), self.n, self._rs, self._ag_in,
                                    self._ag_out, ctypes.byref(self._hp), step, self.flags,
                                    timed_kernel, ev, self._stream), "fsdp_step_groups")


def fsdp_step_groups(plans, rs_in, ag_in, ag_out, lr: float, beta1: float, beta2: float,
                     eps: float, weight_decay: float, step: int, flags: int = 0,
                     timed_kernel: int = 0, timing_events=None, stream=None) -> None:
    StepGroupsCall(plans, rs_in, ag_in, ag_out, lr, beta1, beta2, eps, weight_decay, flags,
                   stream)(step, timed_kernel, timing_events)


# ---- group sets -------------------------------------------------------------------

def fsdp_group_set_create(plans, stream=None):
    """Returns an opaque group-set handle over the (bound) plans."""
    arr = (ctypes.c_void_p * max(1, len(plans)))(*[p.value if p is not None else None
                                                   for p in plans])
    out = _P()
    _check(lib.fsdp_group_set_create(ctypes.cast(arr, _PP), len(plans), stream_handle(stream),
                                     ctypes.byref(out)), "fsdp_group_set_create")
    return out


def fsdp_group_set_destroy(gset) -> None:
    lib.fsdp_group_set_destroy(gset)


def fsdp_group_set_info(gset):
    """(n_groups, arena_elems) of a group set."""
    n, tot = fsdp_group_set_sizes(gset)[::2]
    return n, tot


def fsdp_group_set_sizes(gset):
    """(n_groups, n_params, arena_elems) of a group set."""
    n, np_, tot = _i32(), _i32(), _i64()
    _check(lib.fsdp_group_set_info(gset, ctypes.byref(n), ctypes.byref(np_), ctypes.byref(tot)),
           "fsdp_group_set_info")
    return n.value, np_.value, tot.value


def fsdp_group_set_segment(gset, g: int):
    """(offset, arena_elems): group g's copy-in segment starts at element offset
    of an arena of arena_elems bf16 elements."""
    off, tot = _i64(), _i64()
    _check(lib.fsdp_group_set_segment(gset, g, ctypes.byref(off), ctypes.byref(tot)),
           "fsdp_group_set_segment")
    return off.value, tot.value


def _arena_elems(gset):
    if gset is None or getattr(gset, "value", 1) is None:
        return None
    return fsdp_group_set_info(gset)[1]


def fsdp_adamw_groups(gset, lr: float, beta1: float, beta2: float, eps: float,
                      weight_decay: float, step: int, stream=None) -> None:
    hp = AdamwHparams(lr, beta1, beta2, eps, weight_decay)
    _check(lib.fsdp_adamw_groups(gset, ctypes.byref(hp), step, stream_handle(stream)),
           "fsdp_adamw_groups")


def fsdp_pack_allgather_groups(gset, arena, stream=None) -> None:
    n = _arena_elems(gset)
    a = _dev(arena, 2 * n, "arena") if n is not None else addr(arena)
    _check(lib.fsdp_pack_allgather_groups(gset, a, stream_handle(stream)),
           "fsdp_pack_allgather_groups")


def fsdp_adamw_pack_groups(gset, arena, lr: float, beta1: float, beta2: float, eps: float,
                           weight_decay: float, step: int, stream=None) -> None:
    n = _arena_elems(gset)
    a = _dev(arena, 2 * n, "arena") if n is not None else addr(arena)
    hp = AdamwHparams(lr, beta1, beta2, eps, weight_decay)
    _check(lib.fsdp_adamw_pack_groups(gset, ctypes.byref(hp), step, a, stream_handle(stream)),
           "fsdp_adamw_pack_groups")


def fsdp_amax_groups(gset, amax, stream=None) -> None:
    """amax: n_params fp32 (the set's parameters in group order)."""
    if gset is None or getattr(gset, "value", 1) is None:
        a = addr(amax)
    else:
        a = _dev(amax, 4 * fsdp_group_set_sizes(gset)[1], "amax")
    _check(lib.fsdp_amax_groups(gset, a, stream_handle(stream)), "fsdp_amax_groups")


def fsdp_pack_allgather_fp8_groups(gset, arena, scales, stream=None) -> None:
    """arena: one byte per element of the set's arena; scales: n_params fp32."""
    if gset is None or getattr(gset, "value", 1) is None:
        a, sc = addr(arena), addr(scales)
    else:
        _, np_, tot = fsdp_group_set_sizes(gset)
        a = _dev(arena, tot, "arena")
        sc = _dev(scales, 4 * np_, "scales")
    _check(lib.fsdp_pack_allgather_fp8_groups(gset, a, sc, stream_handle(stream)),
           "fsdp_pack_allgather_fp8_groups")


class StepGroupSetCall:
    """fsdp_step_group_set with its pointer arrays marshalled once.

    plans: the set's plans, in its order (for the buffer size checks);
    rs_in, ag_out: tensors/addresses per group (ag_out may be None);
    arena: the copy-in arena of the set.
    """

    def __init__(self, gset, plans, rs_in, arena, ag_out, lr, beta1, beta2, eps,
                 weight_decay, flags=0, stream=None):
        n = len(plans)
        if n != fsdp_group_set_info(gset)[0]:
            raise ValueError(f"plans: {n} given, the set has {fsdp_group_set_info(gset)[0]} groups")
        if len(rs_in) != n or (ag_out is not None and len(ag_out) != n):
            raise ValueError("rs_in and ag_out must have one entry per group")
        self.n = n
        self._set = gset
        rs_p, out_p = [], []
        for g, p in enumerate(plans):
            d = _dims(p)
            rs_p.append(_dev(rs_in[g], 2 * d[0] * d[1], f"rs_in[{g}]"))
            if ag_out is not None:
                out_p.append(_dev(ag_out[g], 2 * d[0] * d[1], f"ag_out[{g}]"))
        self._arena = _dev(arena, 2 * _arena_elems(gset), "arena")
        self._rs = _ptr_array(rs_p)
        self._ag_out = _ptr_array(out_p) if ag_out is not None else None
        self._keep = (rs_in, arena, ag_out)
        self._hp = AdamwHparams(lr, beta1, beta2, eps, weight_decay)
        self.flags = flags
        self._stream = stream_handle(stream)

    def __call__(self, step: int, timed_kernel: int = 0, events=None) -> None:
        ev = None
        if events is not None:
            if len(events) != 2 * self.n:
                raise ValueError(f"events: need 2 per group ({2 * self.n}), got {len(events)}")
            ev = (ctypes.c_void_p * len(events))(
                *[int(e.cuda_event) if e is not None else None for e in events])
            ev = ctypes.cast(ev, _PP)
        _check(lib.fsdp_step_group_set(self._set, self._rs, self._arena, self._ag_out,
                                       ctypes.byref(self._hp), step, self.flags, timed_kernel,
                                       ev, self._stream), "fsdp_step_group_set")


def fsdp_check_stream(stream=None) -> None:
    _check(lib.fsdp_check_stream(stream_handle(stream)), "fsdp_check_stream")


EXPORTS = tuple(_SIGS)
