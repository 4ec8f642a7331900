"""Plausible mistakes planted in the CPU oracle, one at a time (CPU only).

tests/test_oracle_mutations.py runs the oracle's pin suite once per mutation,
in a child process whose conftest calls ``apply(name)`` before any test runs,
and requires the suite to fail: every mistake listed here must be caught by
at least one pin.  Nothing outside the tests imports this module, and the
product library never sees the oracle.

Each mutation replaces one oracle function by a copy with a single mistake
of the kind a reader could make when writing it from the pages: a wrong
chunk rule, a lost row, a rounding or sign error, a dropped term, swapped
operands.
"""
import numpy as np

import oracle
from oracle import fsdp as O

F32 = np.float32


def _chunk_floor_plus_one(rows, world):
    # ceil written as floor + 1: wrong whenever world divides rows
    return 0 if rows <= 0 else rows // world + 1


def _rows_even_split(rows, world, j):
    # tensor_split's rule (remainder spread over the first ranks), not chunk's
    base, rem = divmod(max(rows, 0), world)
    begin = j * base + min(j, rem)
    return begin, base + (1 if j < rem else 0)


def _rows_lose_last(rows, world, j):
    # the last row of every non-empty chunk dropped
    c = O.chunk_rows(rows, world)
    begin = min(j * c, rows)
    end = min((j + 1) * c, rows)
    n = end - begin
    return begin, n - 1 if n > 0 else 0


_orig_plan = O.plan


def _plan_align_ignored(shapes, world, rank, align=1):
    # alignment accepted but never applied between parameters
    return _orig_plan(shapes, world, rank, 1)


def _bf16_round_half_up(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=F32))
    b = a.view(np.uint32).astype(np.uint64)
    rounded = ((b + 0x8000) >> 16).astype(np.uint16)
    quiet = ((b >> 16) | 0x0040).astype(np.uint16)
    return np.where(np.isnan(a), quiet, rounded)


def _bf16_truncate(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=F32))
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _pack_pad_left_unset(p, master_shards):
    # padding not zeroed (left as whatever the buffer held: all ones here)
    out = np.full(p.S, 0xFFFF, dtype=np.uint16)
    for e, m in zip(p.entries, master_shards):
        flat = np.asarray(m, dtype=F32).reshape(-1)
        out[e.shard_offset:e.shard_offset + e.valid_numel] = O.bf16_rne(flat)
    return out


def _unpack_from_row0(p, ag_out):
    # every rank's piece read from row 0 instead of row j
    ag = np.asarray(ag_out, dtype=np.uint16).reshape(p.world, p.S)
    fulls = []
    for e in p.entries:
        full = np.empty(e.rows * e.cols, dtype=np.uint16)
        for j in range(p.world):
            b, lr = O.rows_of_rank(e.rows, p.world, j)
            n = lr * e.cols
            full[b * e.cols:b * e.cols + n] = ag[0, e.shard_offset:e.shard_offset + n]
        fulls.append(full.reshape(e.rows, e.cols))
    return fulls


def _reduce_variant(drop_last=False, divide=True, reciprocal=False):
    def reduce(p, rs_in):
        rs = np.asarray(rs_in, dtype=np.uint16).reshape(p.world, p.S)
        grads = []
        for e in p.entries:
            sl = slice(e.shard_offset, e.shard_offset + e.valid_numel)
            acc = O.bf16_to_f32(rs[0, sl]).copy()
            for j in range(1, p.world - (1 if drop_last else 0)):
                acc = acc + O.bf16_to_f32(rs[j, sl])
            if reciprocal:
                acc = acc * (F32(1.0) / F32(p.world))
            elif divide:
                acc = acc / F32(p.world)
            grads.append(acc.astype(F32))
        return grads
    return reduce


def _reduce_f32_times_reciprocal(p, rs_in):
    rs = np.asarray(rs_in, dtype=F32).reshape(p.world, p.S)
    grads = []
    for e in p.entries:
        sl = slice(e.shard_offset, e.shard_offset + e.valid_numel)
        acc = rs[0, sl].copy()
        for j in range(1, p.world):
            acc = acc + rs[j, sl]
        grads.append((acc * (F32(1.0) / F32(p.world))).astype(F32))
    return grads


_orig_scalars = O.adamw_scalars


def _scalars_variant(**change):
    def adamw_scalars(lr, beta1, beta2, eps, weight_decay, step):
        s = _orig_scalars(lr, beta1, beta2, eps, weight_decay, step)
        vals = dict(s.__dict__)
        if change.get("no_decay"):
            vals["decay"] = F32(1.0)
        if change.get("no_bc1"):
            vals["step_size"] = F32(lr)
        if change.get("no_sqrt_bc2"):
            vals["bc2_sqrt"] = F32(1.0 - beta2 ** step)
        if change.get("swap_betas"):
            vals["beta1"], vals["beta2"] = vals["beta2"], vals["beta1"]
            vals["one_minus_beta1"], vals["one_minus_beta2"] = (vals["one_minus_beta2"],
                                                                vals["one_minus_beta1"])
        return O.AdamWScalars(**vals)
    return adamw_scalars


def _adamw_variant(sign_flip=False, eps_inside=False):
    def adamw(param, grad, exp_avg, exp_avg_sq, step, lr, beta1, beta2, eps, weight_decay):
        s = O.adamw_scalars(lr, beta1, beta2, eps, weight_decay, step)
        g = grad
        p = param * s.decay
        m = exp_avg * s.beta1 + s.one_minus_beta1 * g
        v = exp_avg_sq * s.beta2 + s.one_minus_beta2 * (g * g)
        if eps_inside:
            d = np.sqrt(v + s.eps) / s.bc2_sqrt
        else:
            d = np.sqrt(v) / s.bc2_sqrt + s.eps
        p = p + s.step_size * (m / d) if sign_flip else p - s.step_size * (m / d)
        param[...] = p
        exp_avg[...] = m
        exp_avg_sq[...] = v
    return adamw


def _state_optimizer_unsharded(n_params, world, zero_stage):
    # stage 1 forgets to shard the 12 bytes of fp32 master and moments
    if zero_stage not in (0, 1, 2, 3) or world < 1:
        raise ValueError("stage in 0..3, world >= 1")
    params, grads, optim = 2.0 * n_params, 2.0 * n_params, 12.0 * n_params
    if zero_stage >= 2:
        grads /= world
    if zero_stage >= 3:
        params /= world
    return params + grads + optim


_orig_e4m3 = O.e4m3_sat


def _e4m3_overflow_to_nan(x):
    # no saturation: magnitudes past 448 become the NaN code
    a = np.asarray(x, dtype=F32)
    code = _orig_e4m3(a)
    big = np.abs(a) >= F32(448.0)
    return np.where(big & ~np.isnan(a), (code & 0x80) | 0x7F, code).astype(np.uint8)


def _reshard_runs_dst_offset_zero(rows, cols, world_src, world_dst, rank_dst):
    # target offsets taken relative to the source chunk instead of the target
    runs = []
    b2, l2 = O.rows_of_rank(rows, world_dst, rank_dst)
    for s in range(world_src):
        b1, l1 = O.rows_of_rank(rows, world_src, s)
        lo, hi = max(b1, b2), min(b1 + l1, b2 + l2)
        if hi > lo:
            runs.append((s, (lo - b1) * cols, (lo - b1) * cols, (hi - lo) * cols))
    return runs


def _bf16_no_nan_case(x):
    # rounding applied to NaNs too: a NaN with only low payload bits becomes inf
    a = np.ascontiguousarray(np.asarray(x, dtype=F32))
    b = a.view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _accumulate_reset_adds_zero(acc, full_grads, reset):
    # the first microbatch adds to +0.0 instead of storing the widening
    out = []
    for i, g in enumerate(full_grads):
        x = O.bf16_to_f32(np.asarray(g, dtype=np.uint16).reshape(-1))
        base = np.zeros_like(x) if reset else np.asarray(acc[i], dtype=F32).reshape(-1)
        out.append((base + x).astype(F32))
    return out


def _rspack_rows_reversed(p, full_grads):
    # chunk j written to row N-1-j
    out = np.zeros((p.world, p.S), dtype=np.uint16)
    for e, g in zip(p.entries, full_grads):
        flat = np.asarray(g, dtype=np.uint16).reshape(-1)
        for j in range(p.world):
            b, lr = O.rows_of_rank(e.rows, p.world, j)
            n = lr * e.cols
            out[p.world - 1 - j, e.shard_offset:e.shard_offset + n] = flat[b * e.cols:b * e.cols + n]
    return out


def _adamw_v_without_square(param, grad, exp_avg, exp_avg_sq, step, lr, beta1, beta2, eps,
                            weight_decay):
    s = O.adamw_scalars(lr, beta1, beta2, eps, weight_decay, step)
    g = grad
    p = param * s.decay
    m = exp_avg * s.beta1 + s.one_minus_beta1 * g
    v = exp_avg_sq * s.beta2 + s.one_minus_beta2 * np.abs(g)
    d = np.sqrt(v) / s.bc2_sqrt + s.eps
    param[...] = p - s.step_size * (m / d)
    exp_avg[...] = m
    exp_avg_sq[...] = v


def _amax_signed(master_shards):
    # largest signed value instead of the largest magnitude
    out = np.zeros(len(master_shards), dtype=F32)
    for i, m in enumerate(master_shards):
        b = np.asarray(m, dtype=F32).reshape(-1)
        out[i] = b.max() if b.size else 0
    return out


def _e4m3_ties_away(x):
    # ties rounded away from zero instead of to even (normal range)
    a = np.ascontiguousarray(np.asarray(x, dtype=F32))
    code = _orig_e4m3(a)
    u = a.view(np.uint32).astype(np.int64)
    mag = u & 0x7FFFFFFF
    tie = ((mag & 0xFFFFF) == 0x80000) & (mag >= 0x3C800000) & (mag < 0x43E00000)
    up = ((mag >> 20) & 1) == 0      # ties-to-even rounded these down
    return np.where(tie & up, code + 1, code).astype(np.uint8)


_orig_reshard_runs = O.reshard_runs


def _reshard_runs_skip_last_source(rows, cols, world_src, world_dst, rank_dst):
    # the last source rank's rows never read (a loop bound one short)
    return [r for r in _orig_reshard_runs(rows, cols, world_src, world_dst, rank_dst)
            if r[0] != world_src - 1 or world_src == 1]


def _state_grads_unsharded(n_params, world, zero_stage):
    # stage 2 forgets to shard the gradients
    if zero_stage not in (0, 1, 2, 3) or world < 1:
        raise ValueError("stage in 0..3, world >= 1")
    params, grads, optim = 2.0 * n_params, 2.0 * n_params, 12.0 * n_params
    if zero_stage >= 1:
        optim /= world
    if zero_stage >= 3:
        params /= world
        grads /= world
    return params + grads + optim


def _pack_fp8_divides_by_scale(p, master_shards, scales):
    # the tensor-wise scale divided instead of multiplied
    out = np.zeros(p.S, dtype=np.uint8)
    for e, m, sc in zip(p.entries, master_shards, scales):
        flat = np.asarray(m, dtype=F32).reshape(-1)
        out[e.shard_offset:e.shard_offset + e.valid_numel] = O.e4m3_sat(flat / F32(sc))
    return out


_orig_e4m3_to_f32 = O.e4m3_to_f32


def _e4m3_decode_bias8(u8):
    # exponent bias 8 instead of 7: every value halved
    return (_orig_e4m3_to_f32(u8) * F32(0.5)).astype(F32)


def _plan_reverse_order(shapes, world, rank, align=1):
    # pieces laid out in reverse registration order
    pl = _orig_plan(list(shapes)[::-1], world, rank, align)
    pl.entries = pl.entries[::-1]
    return pl


def _decay_without_lr(lr, beta1, beta2, eps, weight_decay, step):
    # decoupled decay written as 1 - wd instead of 1 - lr * wd
    s = _orig_scalars(lr, beta1, beta2, eps, weight_decay, step)
    vals = dict(s.__dict__)
    vals["decay"] = F32(1.0 - weight_decay)
    return O.AdamWScalars(**vals)


def _rows_begin_off_by_one(rows, world, j):
    # every rank after the first starts one row late
    b, lr = _orig_rows_of_rank(rows, world, j)
    return (b + 1 if lr and j > 0 else b), lr


_orig_rows_of_rank = O.rows_of_rank


MUTATIONS = {
    "chunk_floor_plus_one": ("chunk_rows", _chunk_floor_plus_one),
    "rows_even_split": ("rows_of_rank", _rows_even_split),
    "rows_lose_last": ("rows_of_rank", _rows_lose_last),
    "plan_align_ignored": ("plan", _plan_align_ignored),
    "bf16_round_half_up": ("bf16_rne", _bf16_round_half_up),
    "bf16_truncate": ("bf16_rne", _bf16_truncate),
    "pack_pad_left_unset": ("pack", _pack_pad_left_unset),
    "unpack_from_row0": ("unpack", _unpack_from_row0),
    "reduce_drop_last_rank": ("reduce", _reduce_variant(drop_last=True)),
    "reduce_no_divide": ("reduce", _reduce_variant(divide=False)),
    "reduce_times_reciprocal": ("reduce", _reduce_variant(reciprocal=True)),
    "reduce_f32_times_reciprocal": ("reduce_f32", _reduce_f32_times_reciprocal),
    "adamw_no_weight_decay": ("adamw_scalars", _scalars_variant(no_decay=True)),
    "adamw_no_bias_correction1": ("adamw_scalars", _scalars_variant(no_bc1=True)),
    "adamw_no_sqrt_bias_correction2": ("adamw_scalars", _scalars_variant(no_sqrt_bc2=True)),
    "adamw_betas_swapped": ("adamw_scalars", _scalars_variant(swap_betas=True)),
    "adamw_update_sign_flipped": ("adamw", _adamw_variant(sign_flip=True)),
    "adamw_eps_inside_sqrt": ("adamw", _adamw_variant(eps_inside=True)),
    "state_optimizer_unsharded": ("state_bytes", _state_optimizer_unsharded),
    "e4m3_overflow_to_nan": ("e4m3_sat", _e4m3_overflow_to_nan),
    "reshard_dst_offset_wrong": ("reshard_runs", _reshard_runs_dst_offset_zero),
    "bf16_no_nan_case": ("bf16_rne", _bf16_no_nan_case),
    "accumulate_reset_adds_zero": ("accumulate_grad", _accumulate_reset_adds_zero),
    "rspack_rows_reversed": ("pack_reduce_scatter", _rspack_rows_reversed),
    "adamw_v_without_square": ("adamw", _adamw_v_without_square),
    "amax_signed": ("amax", _amax_signed),
    "e4m3_ties_away": ("e4m3_sat", _e4m3_ties_away),
    "reshard_skip_last_source": ("reshard_runs", _reshard_runs_skip_last_source),
    "state_grads_unsharded": ("state_bytes", _state_grads_unsharded),
    "pack_fp8_divides_by_scale": ("pack_fp8", _pack_fp8_divides_by_scale),
    "e4m3_decode_bias8": ("e4m3_to_f32", _e4m3_decode_bias8),
    "plan_reverse_order": ("plan", _plan_reverse_order),
    "adamw_decay_without_lr": ("adamw_scalars", _decay_without_lr),
    "rows_begin_off_by_one": ("rows_of_rank", _rows_begin_off_by_one),
}


def apply(name):
    """Replace one oracle function, in the module and the package namespace."""
    attr, fn = MUTATIONS[name]
    setattr(O, attr, fn)
    if hasattr(oracle, attr):
        setattr(oracle, attr, fn)
