"""Plain, slow CPU oracle of one rank's FSDP2 sharded step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline leg may import this module.  It shares no code with the HIP library
and imports nothing from it; it uses only Python and NumPy.

Pages cited (by title and section):

[ST]  "Sharded Training: FSDP2, DTensor, Tensor and Pipeline Parallelism"
      (course module 27): the opening 16-bytes-per-parameter paragraph, the
      ZeRO paragraph, the fully_shard paragraph, "Mixed precision",
      "Other controls", Fence 1, Fence 4 and "The bug Adam hid".
[MS]  "Introduction to PyTorch FSDP2 Backend Features": "Working Principle",
      "DTensor", "Mixed Precision".
[AF]  "PyTorch FSDP2 Guide: Distributed LLM Training with DTensor": "The
      Problem: The Hidden Memory Tax of Legacy FSDP1".

Precision.  The pages fix the dtypes of this path: sharded parameters and the
optimizer stay fp32, all-gathered copies are bf16 (param_dtype), gradients are
reduced in fp32 (reduce_dtype) ([ST] "Mixed precision"; [MS] "Mixed
Precision").  The oracle therefore computes in fp32, one IEEE round-to-nearest
operation at a time in a fixed order, with NumPy float32 scalars and arrays
(NumPy never fuses a multiply and an add).  Host scalars derived from the
hyperparameters are computed in fp64 and rounded once to fp32.

Readings where the pages are silent (each also listed with the design notes):

* chunking is torch.chunk's ceil rule, so trailing ranks can be empty;
* each rank's piece of a parameter is padded to the chunk size c*cols and the
  pieces sit back to back in registration order; padding holds zeros;
* parameters are packed with no gap (align_elems = 1) unless a caller asks for
  an element alignment (8 elements = 16 bytes is the only other option);
* rows of the [N, S] buffers are in rank order;
* the reduction adds contributions in rank order starting from rank 0's value,
  then makes one fp32 division by N;
* bf16 conversion rounds to nearest even; a NaN keeps its sign and leading
  payload bits and is made quiet;
* AdamW follows the decoupled-weight-decay algorithm with the per-element
  operation order given in ``adamw``.

Parity pins for every function here live in tests/test_oracle_pins.py; none is
unpinned.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence

import numpy as np

F32 = np.float32


# ---------------------------------------------------------------------------
# Shard layout
# ---------------------------------------------------------------------------

def chunk_rows(rows: int, world: int) -> int:
    """Rows per chunk of torch.chunk(param, world, dim=0): ceil(rows / world).

    [ST] fully_shard paragraph: rank r keeps chunk r of
    torch.chunk(param, world, dim=0).
    """
    if rows <= 0:
        return 0
    return -(-rows // world)


def rows_of_rank(rows: int, world: int, j: int):
    """(row_begin, local_rows) of rank j's chunk; empty past the last chunk.

    torch.chunk makes ceil(rows/c) chunks of c rows, the last one short, so
    ranks past the last chunk own nothing ([ST] lab: a (1, 32) head leaves
    rank 1 with an empty (0, 32) shard).
    """
    c = chunk_rows(rows, world)
    begin = min(j * c, rows)
    end = min((j + 1) * c, rows)
    return begin, end - begin


@dataclass
class Entry:
    rows: int
    cols: int
    chunk_rows: int        # c: every rank's piece is padded to c rows
    row_begin: int         # first row this rank owns
    local_rows: int        # rows this rank owns (0 for an empty chunk)
    shard_offset: int      # element offset of this param's piece in a row of [N, S]
    shard_numel: int       # c * cols: the padded piece
    valid_numel: int       # local_rows * cols
    pad_numel: int         # shard_numel - valid_numel
    seg_numel: int         # shard_numel rounded up to align_elems


@dataclass
class Plan:
    world: int
    rank: int
    align: int
    entries: List[Entry]
    S: int                 # padded per-rank segment length (elements)

    @property
    def V(self) -> int:
        return sum(e.valid_numel for e in self.entries)

    @property
    def F(self) -> int:
        return sum(e.rows * e.cols for e in self.entries)


def plan(shapes: Sequence[Sequence[int]], world: int, rank: int, align: int = 1) -> Plan:
    """Layout of one parameter group's communication buffer for rank ``rank``.

    Every parameter is sharded on its own along dim 0 (per-parameter Shard(0),
    [ST] fully_shard paragraph; [MS] "FSDP2 vs. FSDP1").  One fully_shard call
    makes one group and one communication unit, so the group's pieces are
    concatenated, in registration order, into one segment of S elements per
    rank.  Each piece is padded to c*cols elements ("padded internally").
    """
    if world < 1 or not (0 <= rank < world):
        raise ValueError("need world >= 1 and 0 <= rank < world")
    if align not in (1, 8):
        raise ValueError("align must be 1 or 8")
    entries = []
    off = 0
    for shp in shapes:
        if len(shp) == 0:
            raise ValueError("0-dim parameters cannot be sharded on dim 0")
        rows = int(shp[0])
        cols = 1
        for d in shp[1:]:
            cols *= int(d)
        c = chunk_rows(rows, world)
        b, lr = rows_of_rank(rows, world, rank)
        shard = c * cols
        seg = -(-shard // align) * align
        entries.append(Entry(rows, cols, c, b, lr, off, shard, lr * cols,
                             shard - lr * cols, seg))
        off += seg
    return Plan(world, rank, align, entries, off)


# ---------------------------------------------------------------------------
# bf16 <-> fp32
# ---------------------------------------------------------------------------

def bf16_rne(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    bf16 keeps the top 16 bits of an fp32.  Adding 0x7FFF plus the lowest kept
    bit and truncating rounds the dropped 16 bits to nearest with ties going to
    an even kept mantissa; an overflowing carry turns the largest finite values
    into infinity, as IEEE rounding does.  A NaN is kept as a NaN: its sign and
    leading payload bits survive and the quiet bit is set.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=F32))
    b = a.view(np.uint32).astype(np.uint64)
    rounded = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    quiet = ((b >> 16) | 0x0040).astype(np.uint16)
    return np.where(nan, quiet, rounded)


def bf16_to_f32(u16) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact: the low 16 bits become zero)."""
    u = np.asarray(u16, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(F32)


# ---------------------------------------------------------------------------
# FP8 E4M3 (OCP e4m3fn: bias 7, 3 mantissa bits, no infinities)
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_to_f32(u8) -> np.ndarray:
    """Exact value of e4m3fn codes: S.EEEE.MMM, bias 7; exponent 0 holds
    subnormals m/8 * 2^-6; S.1111.111 is NaN (there is no infinity)."""
    b = np.asarray(u8, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return (sign * val).astype(F32)


def e4m3_sat(x) -> np.ndarray:
    """fp32 -> e4m3fn code, round to nearest even, saturating.

    Magnitudes at or beyond 448 (the largest finite code), infinities
    included, become +-448, as FP8 training casts clamp before converting; a
    NaN becomes the NaN code with its sign.  Below 2^-6 the code is a
    subnormal m/8 * 2^-6 rounded to nearest even (m = 8 is the smallest
    normal code).  Written on the fp32 bit pattern.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=F32))
    u = a.view(np.uint32).astype(np.int64)
    sign = (u >> 24) & 0x80
    mag = u & 0x7FFFFFFF
    # normal range: keep 3 of the 23 mantissa bits, ties to even, rebias 127 -> 7
    r = (mag + 0x7FFFF + ((mag >> 20) & 1)) >> 20
    normal = np.minimum(r - (120 << 3), 0x7E)
    # subnormal range: m = round_half_even(|x| * 2^9) from the 24-bit significand
    E = mag >> 23
    M = (mag & 0x7FFFFF) | 0x800000
    shift = 141 - E
    sh = np.clip(shift, 1, 40)
    sub = np.where(shift >= 40, 0, (M + (1 << (sh - 1)) - 1 + ((M >> sh) & 1)) >> sh)
    code = np.where(mag >= 0x3C800000, normal, sub)
    code = np.where(mag >= 0x43E00000, 0x7E, code)          # |x| >= 448, inf too
    code = np.where(mag > 0x7F800000, 0x7F, code)           # NaN
    return (sign | code).astype(np.uint8)


def pack_fp8(p: Plan, master_shards: Sequence[np.ndarray], scales: Sequence[float]) -> np.ndarray:
    """FP8 all-gather copy-in: bytes e4m3(fp32(master * scale_p)) at each
    shard offset of a [S] byte segment, zeros in padding.  Parameters stored
    and all-gathered as raw FP8 bytes ([AF] "Native FP8 Training with
    Float8Tensor"); the per-parameter scale comes from the caller (tensor-wise
    scaling, e.g. 448 / amax)."""
    out = np.zeros(p.S, dtype=np.uint8)
    for e, m, sc in zip(p.entries, master_shards, scales):
        flat = np.asarray(m, dtype=F32).reshape(-1)
        out[e.shard_offset:e.shard_offset + e.valid_numel] = e4m3_sat(flat * F32(sc))
    return out


def unpack_fp8(p: Plan, ag_out: np.ndarray) -> List[np.ndarray]:
    """FP8 copy-out: [N, S] bytes -> full [rows, cols] FP8 parameters (the
    bytes stay FP8 for FP8 GEMMs); same row mapping as ``unpack``."""
    ag = np.asarray(ag_out, dtype=np.uint8).reshape(p.world, p.S)
    fulls = []
    for e in p.entries:
        full = np.empty(e.rows * e.cols, dtype=np.uint8)
        for j in range(p.world):
            b, lr = rows_of_rank(e.rows, p.world, j)
            n = lr * e.cols
            full[b * e.cols:b * e.cols + n] = ag[j, e.shard_offset:e.shard_offset + n]
        fulls.append(full.reshape(e.rows, e.cols))
    return fulls


def amax(master_shards: Sequence[np.ndarray]) -> np.ndarray:
    """Per parameter, the largest |x| of this rank's shard (0 when empty): the
    input of tensor-wise FP8 scaling after a max across ranks.  Taken on the
    bit patterns of |x|, so a NaN yields NaN."""
    out = np.zeros(len(master_shards), dtype=F32)
    for i, m in enumerate(master_shards):
        b = np.asarray(m, dtype=F32).reshape(-1).view(np.uint32) & np.uint32(0x7FFFFFFF)
        out[i] = np.array([b.max() if b.size else 0], dtype=np.uint32).view(F32)[0]
    return out


# ---------------------------------------------------------------------------
# The four steps
# ---------------------------------------------------------------------------

def pack(p: Plan, master_shards: Sequence[np.ndarray]) -> np.ndarray:
    """All-gather copy-in: this rank's fp32 shards -> one bf16 segment [S].

    Parameters are cast to param_dtype = bf16 before the all-gather ("half the
    bytes", [ST] "Mixed precision"; [MS] "Mixed Precision": parameters are cast
    to low precision before compute).  Each piece lands at its shard offset;
    the rest of the segment (chunk padding and any alignment gap) is zero.
    """
    out = np.zeros(p.S, dtype=np.uint16)
    for e, m in zip(p.entries, master_shards):
        flat = np.asarray(m, dtype=F32).reshape(-1)
        if flat.size != e.valid_numel:
            raise ValueError("master shard has the wrong size")
        out[e.shard_offset:e.shard_offset + e.valid_numel] = bf16_rne(flat)
    return out


def unpack(p: Plan, ag_out: np.ndarray) -> List[np.ndarray]:
    """All-gather copy-out: [N, S] bf16 -> each parameter's full [rows, cols].

    Row j of ag_out is rank j's segment.  Rank j's piece of a parameter holds
    rows [row_begin(j), row_begin(j) + local_rows(j)); padding is dropped.
    The result is torch.cat of the chunks, i.e. the unsharded parameter
    ([MS] "DTensor": the logical tensor is the full [4096, 4096]).
    """
    ag = np.asarray(ag_out, dtype=np.uint16).reshape(p.world, p.S)
    fulls = []
    for e in p.entries:
        full = np.empty(e.rows * e.cols, dtype=np.uint16)
        for j in range(p.world):
            b, lr = rows_of_rank(e.rows, p.world, j)
            n = lr * e.cols
            full[b * e.cols:b * e.cols + n] = ag[j, e.shard_offset:e.shard_offset + n]
        fulls.append(full.reshape(e.rows, e.cols))
    return fulls


def reduce(p: Plan, rs_in: np.ndarray) -> List[np.ndarray]:
    """Reduce-scatter's local reduction for this rank: fp32 SUM, then / N.

    Gradients are reduced in reduce_dtype = fp32 ([ST] "Mixed precision";
    [MS] "Mixed Precision": BF16 gradients are cast to FP32 before the
    reduction).  FSDP sums and divides by the world size itself
    (set_force_sum_reduction_for_comms, [ST] "Other controls" and "The bug
    Adam hid").  Row j of rs_in holds rank j's bf16 contribution to every
    rank's segment, so this rank reads its own pieces in each row.
    """
    rs = np.asarray(rs_in, dtype=np.uint16).reshape(p.world, p.S)
    n_div = F32(p.world)
    grads = []
    for e in p.entries:
        sl = slice(e.shard_offset, e.shard_offset + e.valid_numel)
        acc = bf16_to_f32(rs[0, sl]).copy()
        for j in range(1, p.world):
            acc = acc + bf16_to_f32(rs[j, sl])
        grads.append((acc / n_div).astype(F32))
    return grads


def pack_reduce_scatter(p: Plan, full_grads: Sequence[np.ndarray]) -> np.ndarray:
    """Reduce-scatter copy-in: this rank's full bf16 gradients -> [N, S].

    Before the reduce-scatter each rank holds the unsharded gradient of every
    parameter; the collective gives rank j the sum of everyone's chunk j
    ([MS] "Working Principle", Reduce-Scatter state; [ST] ZeRO paragraph).  Its
    input therefore has the all-gather's layout: row j holds chunk j of every
    parameter at its shard offset, each piece padded to c*cols with zeros.
    """
    out = np.zeros((p.world, p.S), dtype=np.uint16)
    for e, g in zip(p.entries, full_grads):
        flat = np.asarray(g, dtype=np.uint16).reshape(-1)
        if flat.size != e.rows * e.cols:
            raise ValueError("full gradient has the wrong size")
        for j in range(p.world):
            b, lr = rows_of_rank(e.rows, p.world, j)
            n = lr * e.cols
            out[j, e.shard_offset:e.shard_offset + n] = flat[b * e.cols:b * e.cols + n]
    return out


def pack_reduce_scatter_f32(p: Plan, full_grads: Sequence[np.ndarray]) -> np.ndarray:
    """The same copy-in with reduce_dtype = fp32: the bf16 gradients are cast
    to fp32 before the collective ([MS] "Mixed Precision": BF16 gradients are
    cast to FP32 for the reduction).  The cast is exact; padding is +0.0."""
    return bf16_to_f32(pack_reduce_scatter(p, full_grads))


def accumulate_grad(acc, full_grads, reset: bool) -> List[np.ndarray]:
    """Gradient accumulation without sync: fp32 acc <- acc + fp32(g).

    With set_requires_gradient_sync(False) the unsharded gradients of
    successive microbatches accumulate and no reduce-scatter runs ([ST] "Other
    controls").  The sum is kept in reduce_dtype = fp32; the first microbatch
    (reset) stores the exact widening of its gradient.
    """
    out = []
    for i, g in enumerate(full_grads):
        x = bf16_to_f32(np.asarray(g, dtype=np.uint16).reshape(-1))
        if reset:
            out.append(x.copy())
        else:
            out.append((np.asarray(acc[i], dtype=F32).reshape(-1) + x).astype(F32))
    return out


def pack_reduce_scatter_acc(p: Plan, acc: Sequence[np.ndarray]) -> np.ndarray:
    """Reduce-scatter copy-in from the fp32 accumulators (the synchronizing
    microbatch): the layout of ``pack_reduce_scatter`` with fp32 values and
    +0.0 padding."""
    out = np.zeros((p.world, p.S), dtype=F32)
    for e, a in zip(p.entries, acc):
        flat = np.asarray(a, dtype=F32).reshape(-1)
        if flat.size != e.rows * e.cols:
            raise ValueError("accumulator has the wrong size")
        for j in range(p.world):
            b, lr = rows_of_rank(e.rows, p.world, j)
            n = lr * e.cols
            out[j, e.shard_offset:e.shard_offset + n] = flat[b * e.cols:b * e.cols + n]
    return out


def reduce_f32(p: Plan, rs_in: np.ndarray) -> List[np.ndarray]:
    """Local reduction of fp32 contributions (reduce_dtype = fp32 on the wire):
    fp32 sum in rank order from rank 0's value, then one division by N, as
    ``reduce`` does after widening bf16 contributions."""
    rs = np.asarray(rs_in, dtype=F32).reshape(p.world, p.S)
    n_div = F32(p.world)
    grads = []
    for e in p.entries:
        sl = slice(e.shard_offset, e.shard_offset + e.valid_numel)
        acc = rs[0, sl].copy()
        for j in range(1, p.world):
            acc = acc + rs[j, sl]
        grads.append((acc / n_div).astype(F32))
    return grads


@dataclass(frozen=True)
class AdamWScalars:
    beta1: np.float32
    one_minus_beta1: np.float32
    beta2: np.float32
    one_minus_beta2: np.float32
    eps: np.float32
    decay: np.float32          # 1 - lr * wd
    step_size: np.float32      # lr / (1 - beta1^t)
    bc2_sqrt: np.float32       # sqrt(1 - beta2^t)


def adamw_scalars(lr: float, beta1: float, beta2: float, eps: float,
                  weight_decay: float, step: int) -> AdamWScalars:
    """Per-step scalars: fp64 arithmetic on the hyperparameters, rounded once."""
    if step < 1:
        raise ValueError("AdamW steps count from 1")
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    return AdamWScalars(F32(beta1), F32(1.0 - beta1), F32(beta2), F32(1.0 - beta2),
                        F32(eps), F32(1.0 - lr * weight_decay), F32(lr / bc1),
                        F32(bc2 ** 0.5))


def adamw(param: np.ndarray, grad: np.ndarray, exp_avg: np.ndarray,
          exp_avg_sq: np.ndarray, step: int, lr: float, beta1: float,
          beta2: float, eps: float, weight_decay: float) -> None:
    """One AdamW step on fp32 shards, in place.

    The optimizer is built after sharding and sees only the shards, so its
    state is sharded too ([ST] fully_shard paragraph; [MS] "Working
    Principle", Update State).  The pages name torch.optim.AdamW with
    lr = 3e-4 but give no formula; this is Adam with decoupled weight decay,
    bias-corrected, amsgrad and maximize off, step t >= 1 with m = v = 0
    before the first step.  Per element, every operation one fp32 rounding:

        p <- p * (1 - lr*wd)
        m <- beta1*m + (1 - beta1)*g
        v <- beta2*v + (1 - beta2)*(g*g)
        d <- sqrt(v) / sqrt(1 - beta2^t) + eps
        p <- p - (lr / (1 - beta1^t)) * (m / d)
    """
    s = adamw_scalars(lr, beta1, beta2, eps, weight_decay, step)
    for a in (param, grad, exp_avg, exp_avg_sq):
        if a.dtype != F32:
            raise TypeError("AdamW state is fp32")
    g = grad
    p = param * s.decay
    m = exp_avg * s.beta1 + s.one_minus_beta1 * g
    v = exp_avg_sq * s.beta2 + s.one_minus_beta2 * (g * g)
    d = np.sqrt(v) / s.bc2_sqrt + s.eps
    p = p - s.step_size * (m / d)
    param[...] = p
    exp_avg[...] = m
    exp_avg_sq[...] = v


# ---------------------------------------------------------------------------
# Resharding (distributed checkpoint load into another world size)
# ---------------------------------------------------------------------------

def reshard_runs(rows: int, cols: int, world_src: int, world_dst: int, rank_dst: int):
    """Row overlaps rank ``rank_dst`` of ``world_dst`` reads from each source rank.

    A checkpoint saved by world_src ranks holds chunk s of every parameter in
    shard s; loading into world_dst ranks, each target rank reads only the
    chunks that overlap its own rows, so resharding is planning, not
    conversion ([ST] distributed checkpoint paragraph: 2 ranks to 1, FSDP to
    FSDP+TP).  Returns (src_rank, src_offset, dst_offset, numel) in elements,
    offsets relative to the start of each shard, in row order.
    """
    b2, l2 = rows_of_rank(rows, world_dst, rank_dst)
    runs = []
    for s in range(world_src):
        b1, l1 = rows_of_rank(rows, world_src, s)
        lo, hi = max(b1, b2), min(b1 + l1, b2 + l2)
        if hi > lo:
            runs.append((s, (lo - b1) * cols, (lo - b2) * cols, (hi - lo) * cols))
    return runs


def reshard(src_shards: Sequence[np.ndarray], rows: int, cols: int, world_dst: int,
            rank_dst: int) -> np.ndarray:
    """Target rank's shard: the unsharded rows (concatenation of the source
    shards in rank order) cut by torch.chunk for the new world size."""
    full = np.concatenate([np.asarray(x).reshape(-1) for x in src_shards])
    if full.size != rows * cols:
        raise ValueError("source shards do not add up to the parameter")
    b, lr = rows_of_rank(rows, world_dst, rank_dst)
    return full[b * cols:(b + lr) * cols].copy()


# ---------------------------------------------------------------------------
# State accounting
# ---------------------------------------------------------------------------

def state_bytes(n_params: float, world: int, zero_stage: int) -> float:
    """Per-rank bytes of training state under ZeRO stage 0..3.

    Mixed-precision AdamW holds 16 bytes per parameter: 2 for bf16 weights,
    2 for bf16 gradients, 12 for the fp32 master weights and Adam's two
    moments ([ST] opening paragraph and Fence 1; [AF] "The Problem").  Stage 1
    shards the 12, stage 2 also the gradients, stage 3 (FSDP) also the weights
    ([ST] ZeRO paragraph).
    """
    if zero_stage not in (0, 1, 2, 3) or world < 1:
        raise ValueError("stage in 0..3, world >= 1")
    params, grads, optim = 2.0 * n_params, 2.0 * n_params, 12.0 * n_params
    if zero_stage >= 1:
        optim /= world
    if zero_stage >= 2:
        grads /= world
    if zero_stage >= 3:
        params /= world
    return params + grads + optim
