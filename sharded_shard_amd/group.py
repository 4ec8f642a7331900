"""One parameter group's persistent device state on this rank.

A ``ShardedGroup`` plans the group's segment (C ABI planner), holds this
rank's fp32 shards (master, reduced grad, AdamW m and v) and the bf16 full
parameters in HBM, binds them once, and enqueues the four hot calls.  torch is
used only to allocate device memory; every byte of the step moves in the HIP
kernels behind the C ABI.

HBM layout: one flat buffer per role, each parameter's shard at an offset
rounded up to 64 elements (256 bytes), so every shard starts 16-byte aligned
and the kernels take their vector paths.  Full parameters live in one bf16
arena per group (or a caller's shared arena, e.g. one double-buffered arena for
all groups, as FSDP2 reuses its all-gather buffers), each at a 256-byte
aligned offset.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import capi

ALIGN_F32 = 64    # elements: 256 bytes
ALIGN_BF16 = 128  # elements: 256 bytes


def _round(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def split_shape(shape) -> tuple:
    if len(shape) == 0:
        raise ValueError("0-dim parameters cannot be sharded on dim 0")
    cols = 1
    for d in shape[1:]:
        cols *= int(d)
    return int(shape[0]), cols


class ShardedGroup:
    def __init__(self, shapes: Sequence[Sequence[int]], world: int, rank: int,
                 align_elems: int = 1, device: str = "cuda",
                 full_arena: Optional[torch.Tensor] = None, bind: bool = True,
                 stream=None):
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        rc = [split_shape(s) for s in self.shapes]
        self.rows = [r for r, _ in rc]
        self.cols = [c for _, c in rc]
        self.world, self.rank = world, rank
        self.plan = capi.fsdp_plan_create(self.rows, self.cols, world, rank, align_elems)
        try:
            self.info = capi.fsdp_plan_info(self.plan)
            self.entries = [capi.fsdp_plan_entry(self.plan, i) for i in range(len(self.shapes))]
        except Exception:
            capi.fsdp_plan_destroy(self.plan)
            raise
        self.S, self.V, self.F = self.info.S, self.info.V, self.info.F
        self.device = torch.device(device)
        offs, o = [], 0
        for e in self.entries:
            offs.append(o)
            o += _round(e.valid_numel, ALIGN_F32)
        self.shard_offsets = offs
        self.shard_space = max(o, 1)
        foffs, o = [], 0
        for r, c in rc:
            foffs.append(o)
            o += _round(r * c, ALIGN_BF16)
        self.full_offsets = foffs
        self.full_space = max(o, 1)
        self.master_flat = self.grad_flat = self.m_flat = self.v_flat = None
        self.full_flat = full_arena
        if bind:
            try:
                self.allocate()
                self.bind(stream)
            except Exception:
                self.close()
                raise

    # ---- memory ---------------------------------------------------------------

    def allocate(self, full: bool = True) -> None:
        mk = lambda: torch.zeros(self.shard_space, dtype=torch.float32, device=self.device)
        self.master_flat, self.grad_flat, self.m_flat, self.v_flat = mk(), mk(), mk(), mk()
        if full and self.full_flat is None:
            self.full_flat = torch.zeros(self.full_space, dtype=torch.int16, device=self.device)
        if self.full_flat is not None and self.full_flat.numel() < self.full_space:
            raise ValueError("full-parameter arena is too small for this group")

    def shard_view(self, flat: torch.Tensor, i: int) -> torch.Tensor:
        o = self.shard_offsets[i]
        return flat[o:o + self.entries[i].valid_numel]

    def full_view(self, i: int) -> torch.Tensor:
        o = self.full_offsets[i]
        return self.full_flat[o:o + self.rows[i] * self.cols[i]].view(self.rows[i], self.cols[i])

    def _ptrs(self, flat):
        return [self.shard_view(flat, i).data_ptr() if self.entries[i].valid_numel else 0
                for i in range(len(self.entries))]

    def bind(self, stream=None) -> None:
        full = None
        if self.full_flat is not None:
            full = [self.full_view(i).data_ptr() if self.rows[i] * self.cols[i] else 0
                    for i in range(len(self.entries))]
        capi.fsdp_bind(self.plan, self._ptrs(self.master_flat), self._ptrs(self.grad_flat),
                       self._ptrs(self.m_flat), self._ptrs(self.v_flat), full, stream)

    def bind_full_grad(self, arena: Optional[torch.Tensor] = None, stream=None) -> None:
        """Bind unsharded bf16 gradients, laid out like the full parameters
        (views of ``arena``, allocated here when not given)."""
        if arena is None:
            arena = torch.zeros(self.full_space, dtype=torch.int16, device=self.device)
        if arena.numel() < self.full_space:
            raise ValueError("full-gradient arena is too small for this group")
        self.full_grad_flat = arena
        ptrs = [arena[o:o + r * c].data_ptr() if r * c else 0
                for o, r, c in zip(self.full_offsets, self.rows, self.cols)]
        capi.fsdp_bind_full_grad(self.plan, ptrs, stream)

    def bind_grad_acc(self, arena: Optional[torch.Tensor] = None, stream=None) -> None:
        """Bind fp32 unsharded gradient accumulators, laid out like the full
        parameters (views of ``arena``, allocated here when not given)."""
        if arena is None:
            arena = torch.zeros(self.full_space, dtype=torch.float32, device=self.device)
        if arena.numel() < self.full_space:
            raise ValueError("accumulator arena is too small for this group")
        self.grad_acc_flat = arena
        ptrs = [arena[o:o + r * c].data_ptr() if r * c else 0
                for o, r, c in zip(self.full_offsets, self.rows, self.cols)]
        capi.fsdp_bind_grad_acc(self.plan, ptrs, stream)

    def bind_full_fp8(self, arena: Optional[torch.Tensor] = None, stream=None) -> None:
        """Bind unsharded FP8 parameters (uint8 views of ``arena``, laid out
        like the full parameters; allocated here when not given)."""
        if arena is None:
            arena = torch.zeros(self.full_space, dtype=torch.uint8, device=self.device)
        if arena.numel() < self.full_space:
            raise ValueError("FP8 arena is too small for this group")
        self.full_fp8_flat = arena
        ptrs = [arena[o:o + r * c].data_ptr() if r * c else 0
                for o, r, c in zip(self.full_offsets, self.rows, self.cols)]
        capi.fsdp_bind_full_fp8(self.plan, ptrs, stream)

    def full_fp8_view(self, i: int) -> torch.Tensor:
        o = self.full_offsets[i]
        return self.full_fp8_flat[o:o + self.rows[i] * self.cols[i]].view(self.rows[i], self.cols[i])

    def grad_acc_view(self, i: int) -> torch.Tensor:
        o = self.full_offsets[i]
        return self.grad_acc_flat[o:o + self.rows[i] * self.cols[i]].view(self.rows[i], self.cols[i])

    def full_grad_view(self, i: int) -> torch.Tensor:
        o = self.full_offsets[i]
        return self.full_grad_flat[o:o + self.rows[i] * self.cols[i]].view(self.rows[i], self.cols[i])

    # ---- hot path -----------------------------------------------------------------

    def pack_reduce_scatter(self, rs_out, dtype: int = capi.FSDP_DTYPE_BF16, stream=None) -> None:
        capi.fsdp_pack_reduce_scatter(self.plan, rs_out, dtype, stream)

    def pack_fp8(self, ag_in, scales, stream=None) -> None:
        capi.fsdp_pack_allgather_fp8(self.plan, ag_in, scales, stream)

    def unpack_fp8(self, ag_out, stream=None) -> None:
        capi.fsdp_unpack_allgather_fp8(self.plan, ag_out, stream)

    def amax(self, out, stream=None) -> None:
        capi.fsdp_amax_shard(self.plan, out, stream)

    def accumulate_grad(self, reset: bool, stream=None) -> None:
        capi.fsdp_accumulate_grad(self.plan, reset, stream)

    def pack_reduce_scatter_acc(self, rs_out, stream=None) -> None:
        capi.fsdp_pack_reduce_scatter_acc(self.plan, rs_out, stream)

    def reduce_f32(self, rs_in, stream=None) -> None:
        capi.fsdp_reduce_shard_f32(self.plan, rs_in, stream)

    def pack(self, ag_in, stream=None) -> None:
        capi.fsdp_pack_allgather(self.plan, ag_in, stream)

    def unpack(self, ag_out, stream=None) -> None:
        capi.fsdp_unpack_allgather(self.plan, ag_out, stream)

    def reduce(self, rs_in, stream=None) -> None:
        capi.fsdp_reduce_shard(self.plan, rs_in, stream)

    def adamw(self, step: int, lr: float, beta1: float, beta2: float, eps: float,
              weight_decay: float, stream=None) -> None:
        capi.fsdp_adamw_shard(self.plan, lr, beta1, beta2, eps, weight_decay, step, stream)

    def step(self, rs_in, ag_in, step: int, lr: float, beta1: float, beta2: float, eps: float,
             weight_decay: float, write_grad: bool = False, stream=None) -> None:
        """Fused reduce -> AdamW -> pack (bit-identical to the three calls)."""
        capi.fsdp_step_shard(self.plan, rs_in, ag_in, lr, beta1, beta2, eps, weight_decay, step,
                             capi.FSDP_STEP_WRITE_GRAD if write_grad else 0, stream)

    def close(self) -> None:
        if self.plan is not None:
            capi.fsdp_plan_destroy(self.plan)
            self.plan = None

    def __enter__(self) -> "ShardedGroup":
        return self

    def __exit__(self, *exc) -> None:
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
