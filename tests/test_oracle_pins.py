"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each pin is independent of the oracle's own code: printed values from the
pages (golden fixtures), library routines that define the same thing
(torch.chunk, torch's bf16 cast, torch.optim.AdamW), closed forms, exact
rounding by brute force, and invariants.  They are chosen so that a dropped
term, a wrong index, sign or operand order in the oracle fails at least one.
"""
import math

import numpy as np
import pytest
import torch

from conftest import golden_kv, parse_shape, read_golden
import oracle
from oracle import fsdp as O
from workloads import configs, synth

F32 = np.float32


# ---------------------------------------------------------------------------
# Layout
# ---------------------------------------------------------------------------

def test_chunk_rows_match_torch_chunk_brute_force():
    for rows in range(0, 65):
        t = torch.empty(rows, 3)
        for n in range(1, 17):
            chunks = torch.chunk(t, n, 0)
            begin = 0
            for j in range(n):
                b, lr = O.rows_of_rank(rows, n, j)
                want = chunks[j].shape[0] if j < len(chunks) else 0
                assert lr == want, (rows, n, j)
                if want:
                    assert b == begin
                begin += want
            assert sum(O.rows_of_rank(rows, n, j)[1] for j in range(n)) == rows
            # every rank's piece is padded to chunk 0's rows
            c0 = chunks[0].shape[0] if len(chunks) else 0
            assert O.chunk_rows(rows, n) == c0


def test_dtensor_local_view_4096():
    world, rows, cols, lrows, lcols = map(int, read_golden("dtensor_local_view.txt")[0].split())
    for r in range(world):
        p = O.plan([(rows, cols)], world, r)
        e = p.entries[0]
        assert (e.local_rows, e.cols) == (lrows, lcols)
        assert e.pad_numel == 0 and p.S == lrows * lcols


def test_linear_probe_fsdp2_balanced_and_zero1_contrast():
    g = golden_kv("zero1_probe.txt")
    shapes = [parse_shape(t) for t in g["shapes"]]
    world = int(g["world"][0])
    want_zero1 = [int(x) for x in g["zero1_adam_state_elems"]]
    numels = [int(np.prod(s)) for s in shapes]
    assert shapes == [p.shape for p in configs.get(0).params]
    # ZeroRedundancyOptimizer assigns whole parameters, largest first, to the
    # least-loaded rank; Adam keeps two state elements per parameter element.
    load = [0] * world
    for n in sorted(numels, reverse=True):
        load[load.index(min(load))] += n
    assert [2 * x for x in load] == want_zero1
    # FSDP2 splits every parameter on dim 0: both ranks hold half.
    per_rank = []
    for r in range(world):
        p = O.plan(shapes, world, r)
        assert [(e.local_rows, e.cols) for e in p.entries] == [(16, 16), (16, 1), (2, 32), (2, 1)]
        per_rank.append(2 * p.V)
    assert per_rank == [sum(want_zero1) // 2] * 2 == [676, 676]


def test_lab_head_leaves_rank1_empty():
    lines = read_golden("lab_head_split.txt")
    world = int(lines[0].split(":")[1])
    for ln in lines[1:]:
        lhs, rhs = ln.split("->")
        shape = parse_shape(lhs.strip())
        want = [parse_shape(t) for t in rhs.split()]
        for r in range(world):
            e = O.plan([shape], world, r).entries[0]
            local = (e.local_rows,) + tuple(shape[1:])
            assert local == want[r]
        # rank 1 still carries a padded piece of c*cols elements, all padding
        e1 = O.plan([shape], world, 1).entries[0]
        assert e1.valid_numel == 0 and e1.pad_numel == e1.shard_numel > 0


@pytest.mark.parametrize("align", [1, 8])
def test_plan_invariants_random_shapes(align):
    rng = np.random.default_rng(7)
    for _ in range(60):
        n = int(rng.integers(1, 13))
        shapes = []
        for _ in range(int(rng.integers(1, 9))):
            if rng.random() < 0.3:
                shapes.append((int(rng.integers(0, 40)),))
            else:
                shapes.append((int(rng.integers(0, 40)), int(rng.integers(1, 9))))
        plans = [O.plan(shapes, n, r, align) for r in range(n)]
        S = plans[0].S
        assert all(p.S == S for p in plans)
        for i, shp in enumerate(shapes):
            rows = shp[0]
            es = [p.entries[i] for p in plans]
            assert sum(e.local_rows for e in es) == rows
            assert all(e.shard_offset == es[0].shard_offset for e in es)
            assert es[0].shard_offset % align == 0
            nxt = 0
            for e in es:
                if e.local_rows:
                    assert e.row_begin == nxt
                nxt += e.local_rows
                assert e.valid_numel + e.pad_numel == e.shard_numel == e.chunk_rows * e.cols
                assert e.seg_numel >= e.shard_numel
        offs = [e.shard_offset for e in plans[0].entries]
        segs = [e.seg_numel for e in plans[0].entries]
        assert offs == list(np.cumsum([0] + segs[:-1]))
        assert S == sum(segs)


def test_plan_config_sizes():
    """Segment sizes of the workloads (derived by hand from the shapes)."""
    c1 = configs.get(1)
    p = O.plan([q.shape for q in c1.groups[0].params], 8, 0)
    assert p.S == p.V == 30_409_728 and p.F == 243_277_824
    c3 = configs.get(3)
    moe, root = ([q.shape for q in g.params] for g in c3.groups)
    assert O.plan(moe, 6, 0).S == 92_469_293
    assert O.plan(root, 6, 5).S == 10_924_374
    r5 = O.plan(moe, 6, 5)
    empty = sum(1 for e in r5.entries if e.local_rows == 0)
    assert empty == 2  # the (1, 2048) head and its (1,) bias
    c4 = configs.get(4)
    blk = [q.shape for q in c4.groups[0].params]
    assert O.plan(blk, 64, 0).S == 13_369_600
    assert O.plan([q.shape for q in c4.groups[-1].params], 64, 0).S == 32_833_664


def test_plan_rejects_bad_arguments():
    with pytest.raises(ValueError):
        O.plan([(4,)], 0, 0)
    with pytest.raises(ValueError):
        O.plan([(4,)], 2, 2)
    with pytest.raises(ValueError):
        O.plan([()], 2, 0)
    with pytest.raises(ValueError):
        O.plan([(4,)], 2, 0, align=4)


# ---------------------------------------------------------------------------
# State accounting
# ---------------------------------------------------------------------------

def test_state_bytes_pages_numbers():
    g = golden_kv("state_bytes.txt")
    P7 = float(g["params_7b"][0])
    assert O.state_bytes(P7, 1, 0) == float(g["bytes_7b_ddp"][0])
    assert round(O.state_bytes(P7, 1, 0) / 2**30, 1) == float(g["gib_7b_ddp"][0])
    P70 = float(g["params_70b"][0])
    parts = [float(x) * 1e9 for x in g["parts_70b_gb"]]
    assert sum(parts) == float(g["bytes_70b_total"][0]) == O.state_bytes(P70, 1, 0)
    # 2 + 2 + 8 + 4 bytes per parameter, split as the page lists them
    assert parts == [2 * P70, 2 * P70, 8 * P70, 4 * P70]


def test_state_bytes_fence1_relations():
    P = 7e9
    for n in (1, 8, 64):
        row = [O.state_bytes(P, n, s) for s in range(4)]
        assert all(a >= b for a, b in zip(row, row[1:]))
        assert row[1] == 4 * P + 12 * P / n
        assert row[2] == 2 * P + 14 * P / n
        assert row[3] == 16 * P / n
    assert O.state_bytes(P, 8, 3) == 16 * P / 8
    assert O.state_bytes(P, 64, 0) == 112e9
    with pytest.raises(ValueError):
        O.state_bytes(P, 8, 4)


# ---------------------------------------------------------------------------
# bf16 conversion
# ---------------------------------------------------------------------------

def test_bf16_rne_golden_vectors():
    for ln in read_golden("bf16_rne_cases.txt"):
        f, b = ln.split()[:2]
        x = np.array([int(f, 16)], dtype=np.uint32).view(F32)
        got = int(O.bf16_rne(x)[0])
        assert got == int(b, 16), (f, hex(got), b)


def _nearest_bf16_brute(bits: np.ndarray) -> np.ndarray:
    """Nearest bf16 by comparing the two neighbours in exact fp64 arithmetic."""
    out = np.empty(bits.size, dtype=np.uint16)
    for i, b in enumerate(bits.tolist()):
        sign = b >> 31
        mag = b & 0x7FFFFFFF
        x = abs(float(np.array([mag], dtype=np.uint32).view(F32)[0]))
        lo = mag >> 16
        def val(k):
            if k >= 0x7F80:  # one past the largest finite: 2^128, i.e. overflow
                return 2.0 ** 128
            return float(np.array([k << 16], dtype=np.uint32).view(F32)[0])
        dlo, dhi = x - val(lo), val(lo + 1) - x
        if dlo < dhi or (dlo == dhi and lo % 2 == 0):
            k = lo
        else:
            k = lo + 1
        out[i] = (sign << 15) | min(k, 0x7F80)
    return out


def test_bf16_rne_is_nearest_even_brute_force():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2**32, size=4000, dtype=np.uint64).astype(np.uint32)
    # add every tie and neighbours for a spread of exponents, incl. subnormals
    base = rng.integers(0, 2**16, size=500, dtype=np.uint64).astype(np.uint32) << 16
    extra = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001, base])
    bits = np.concatenate([bits, extra]).astype(np.uint32)
    x = bits.view(F32)
    keep = ~np.isnan(x)
    want = _nearest_bf16_brute(bits[keep])
    got = O.bf16_rne(x[keep])
    assert np.array_equal(got, want)


def test_bf16_rne_matches_torch_library_cast():
    rng = np.random.default_rng(3)
    parts = [rng.standard_normal(1 << 20).astype(F32) * s for s in (1e-3, 0.02, 1.0, 1e30)]
    parts.append((rng.standard_normal(1 << 16) * 1e-39).astype(F32))  # subnormals
    parts.append(rng.integers(0, 2**32, size=1 << 18, dtype=np.uint64).astype(np.uint32).view(F32))
    x = np.concatenate(parts)
    x = x[~np.isnan(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_rne(x), want)
    # widening back is exact and equals torch's
    back = torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy()
    w = O.bf16_to_f32(want)
    assert np.array_equal(w.view(np.uint32), back.view(np.uint32))


def test_bf16_nan_stays_nan_with_sign():
    x = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFA12345], dtype=np.uint32).view(F32)
    out = O.bf16_rne(x)
    assert np.all(np.isnan(O.bf16_to_f32(out)))
    assert [int(v) >> 15 for v in out] == [0, 1, 0, 1]


# ---------------------------------------------------------------------------
# pack / unpack
# ---------------------------------------------------------------------------

SMALL_CASES = [
    ([(32, 16), (32,), (4, 32), (4,)], 2),               # the MLP probe
    ([(1408 // 16, 2048 // 64), (2048 // 16,), (64, 32), (1, 32), (1,)], 6),
    ([(5, 3), (0, 4), (7,), (1, 5), (13, 2)], 4),
    ([(6, 3), (17,)], 8),                                # more ranks than rows
    ([(9, 7)], 1),
]


def _chunks_of(W: torch.Tensor, n: int, j: int) -> torch.Tensor:
    ch = torch.chunk(W, n, 0)
    if j < len(ch):
        return ch[j]
    return W[W.shape[0]:]


@pytest.mark.parametrize("align", [1, 8])
@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_pack_matches_torch_chunk_cast_pad_cat(case, align):
    shapes, n = SMALL_CASES[case]
    Ws = [synth.normal_f32(int(np.prod(s)) if s else 1, 0.02, ("pk", case, i)).reshape(s)
          for i, s in enumerate(shapes)]
    for r in range(n):
        p = O.plan(shapes, n, r, align)
        got = O.pack(p, [_chunks_of(W, n, r).numpy() for W in Ws])
        parts = []
        for W, e in zip(Ws, p.entries):
            piece = _chunks_of(W, n, r).reshape(-1).to(torch.bfloat16).view(torch.int16)
            pad = torch.zeros(e.seg_numel - piece.numel(), dtype=torch.int16)
            parts.append(torch.cat([piece, pad]))
        want = torch.cat(parts).numpy().view(np.uint16)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("align", [1, 8])
@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_unpack_of_packs_is_cast_of_full_params(case, align):
    shapes, n = SMALL_CASES[case]
    Ws = [synth.normal_f32(int(np.prod(s)), 0.02, ("rt", case, i)).reshape(s)
          for i, s in enumerate(shapes)]
    plans = [O.plan(shapes, n, r, align) for r in range(n)]
    ag = np.stack([O.pack(plans[r], [_chunks_of(W, n, r).numpy() for W in Ws])
                   for r in range(n)])
    # padding never reaches an output: overwrite it with the sentinel NaN
    for r in range(n):
        mask = np.ones(plans[r].S, dtype=bool)
        for e in plans[r].entries:
            mask[e.shard_offset:e.shard_offset + e.valid_numel] = False
        ag[r, mask] = synth.SENTINEL_BF16
    for r in range(n):
        fulls = O.unpack(plans[r], ag)
        for W, full in zip(Ws, fulls):
            want = W.reshape(W.shape[0], full.shape[1]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(full, want)


def test_unpack_is_rank_concatenation_of_arbitrary_rows():
    """Unpack reads row j's piece for rows of chunk j; checked on random bits."""
    shapes, n = [(11, 3), (2,), (7, 5)], 4
    p = O.plan(shapes, n, 0)
    rng = np.random.default_rng(5)
    ag = rng.integers(0, 2**16, size=(n, p.S), dtype=np.uint64).astype(np.uint16)
    fulls = O.unpack(p, ag)
    for i, (shp, e) in enumerate(zip(shapes, p.entries)):
        pieces = []
        for j in range(n):
            t = torch.chunk(torch.arange(shp[0]), n)[j] if j < len(torch.chunk(torch.arange(shp[0]), n)) else torch.arange(0)
            k = t.numel() * e.cols
            pieces.append(ag[j, e.shard_offset:e.shard_offset + k])
        assert np.array_equal(fulls[i].reshape(-1), np.concatenate(pieces))


# ---------------------------------------------------------------------------
# reduce
# ---------------------------------------------------------------------------

def _rs_buffer(p, n, key, fill_pad=True):
    rs = np.empty((n, p.S), dtype=np.uint16)
    for j in range(n):
        rs[j] = synth.bf16_bits_to_u16(synth.normal_bf16_bits(p.S, 1e-3, key + (j,)))
    if fill_pad:
        mask = np.ones(p.S, dtype=bool)
        for e in p.entries:
            mask[e.shard_offset:e.shard_offset + e.valid_numel] = False
        rs[:, mask] = synth.SENTINEL_BF16
    return rs


@pytest.mark.parametrize("n", [1, 2, 3, 6, 8, 64])
def test_reduce_all_equal_contributions_is_exact(n):
    """N equal bf16 gradients average to exactly that gradient (no 2x bug)."""
    shapes = [(130, 3), (67,)]
    p = O.plan(shapes, n, 0)
    row = synth.bf16_bits_to_u16(synth.normal_bf16_bits(p.S, 1e-3, ("eq", n)))
    rs = np.tile(row, (n, 1))
    for e, g in zip(p.entries, O.reduce(p, rs)):
        want = O.bf16_to_f32(row[e.shard_offset:e.shard_offset + e.valid_numel])
        assert np.array_equal(g.view(np.uint32), want.view(np.uint32))


def test_reduce_n1_is_exact_widening_and_keeps_negative_zero():
    p = O.plan([(5, 2)], 1, 0)
    rs = np.array([[0x8000, 0x0000, 0x3F80, 0xBF80, 0x0001, 0x8001, 0x7F80, 0xFF80, 0x4049, 0xC049]],
                  dtype=np.uint16)
    g = O.reduce(p, rs)[0].reshape(-1)
    assert np.array_equal(g.view(np.uint32), rs[0].astype(np.uint32) << 16)
    # all-(-0) contributions stay -0 at any N
    p4 = O.plan([(4,)], 4, 0)
    neg0 = np.full((4, p4.S), 0x8000, dtype=np.uint16)
    assert O.reduce(p4, neg0)[0].view(np.uint32)[0] == 0x80000000


@pytest.mark.parametrize("n", [2, 6, 8, 64])
def test_reduce_within_fp32_error_bound_of_exact_sum(n):
    shapes = [(3 * n + 1, 5), (2 * n - 1,)]
    for r in (0, n - 1):
        p = O.plan(shapes, n, r)
        rs = _rs_buffer(p, n, ("eb", n, r))
        grads = O.reduce(p, rs)
        u = 2.0 ** -24
        for e, g in zip(p.entries, grads):
            cols = [O.bf16_to_f32(rs[j, e.shard_offset:e.shard_offset + e.valid_numel]).astype(np.float64)
                    for j in range(n)]
            for i in range(e.valid_numel):
                xs = [c[i] for c in cols]
                exact = math.fsum(xs) / n
                bound = (n - 1) * u * sum(abs(x) for x in xs) / n + u * abs(exact) + 1e-45
                assert abs(float(g[i]) - exact) <= bound * 1.0001


def _nearest_f32(fr):
    """The fp32 nearest to an exact rational, ties to the even bit pattern
    (normal range), by comparing exact distances of the candidates."""
    from fractions import Fraction
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    return min(cands, key=lambda y: (abs(Fraction(float(y)) - fr),
                                     int(np.array([y], dtype=F32).view(np.uint32)[0]) & 1))


@pytest.mark.parametrize("n", [3, 6, 7, 12])
def test_reduce_divides_once_correctly_rounded(n):
    """With contributions whose fp32 sums are exact (small integers times a
    power of two), the only rounding left is the division by N: the result
    must be the correctly rounded quotient of the exact sum, which a multiply
    by a rounded 1/N misses for some sums.  The same holds for fp32
    contributions."""
    from fractions import Fraction
    p = O.plan([(4096,)], n, 0)
    rng = np.random.default_rng(1000 + n)
    k = rng.integers(-256, 257, size=(n, p.S)).astype(np.float32)
    scale = np.float32(2.0 ** -7)
    vals = torch.from_numpy(k * scale)
    rs = vals.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert torch.equal(vals.to(torch.bfloat16).float(), vals)       # bf16-exact inputs
    g = O.reduce(p, rs)[0]
    g32 = O.reduce_f32(p, k * scale)[0]
    for i in range(p.S):
        exact = Fraction(int(k[:, i].sum())) * Fraction(1, 128) / n
        want = _nearest_f32(exact) if exact != 0 else np.float32(0.0)
        assert g[i] == want, (n, i, float(exact))
        assert g32[i] == want, (n, i, float(exact))


def test_reduce_matches_torch_mean_and_never_reads_padding():
    n = 6
    shapes = [(1408 // 8, 16), (2048 // 8,), (1, 16), (1,)]
    for r in range(n):
        p = O.plan(shapes, n, r)
        rs = _rs_buffer(p, n, ("tm", r), fill_pad=True)
        t = torch.from_numpy(rs.view(np.int16)).view(torch.bfloat16).float()
        for e, g in zip(p.entries, O.reduce(p, rs)):
            assert np.all(np.isfinite(g))
            want = (t[:, e.shard_offset:e.shard_offset + e.valid_numel].sum(0) / n).numpy()
            np.testing.assert_allclose(g, want, rtol=2e-6, atol=1e-12)


# ---------------------------------------------------------------------------
# AdamW
# ---------------------------------------------------------------------------

HP = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _state(n, key):
    p = synth.normal_f32(n, 0.02, key + ("p",)).numpy().copy()
    return p, np.zeros(n, F32), np.zeros(n, F32)


def test_adamw_zero_grad_only_decays():
    p, m, v = _state(1000, ("z",))
    p0 = p.astype(np.float64)
    g = np.zeros_like(p)
    for t in (1, 2, 3):
        O.adamw(p, g, m, v, t, **HP)
        assert not m.any() and not v.any()
        want = p0 * (1 - HP["lr"] * HP["weight_decay"]) ** t
        np.testing.assert_allclose(p, want, rtol=4 * 2**-24, atol=0)


def test_adamw_first_step_closed_form():
    p, m, v = _state(5000, ("s1",))
    p0 = p.astype(np.float64)
    g = synth.normal_f32(5000, 1e-3, ("s1", "g")).numpy()
    O.adamw(p, g, m, v, 1, **HP)
    g64 = g.astype(np.float64)
    lr, wd, eps = HP["lr"], HP["weight_decay"], HP["eps"]
    want = p0 * (1 - lr * wd) - lr * g64 / (np.abs(g64) + eps)
    np.testing.assert_allclose(p, want, rtol=0, atol=8 * 2**-24 * np.abs(p0).max() + 1e-11)
    np.testing.assert_allclose(m, (1 - HP["beta1"]) * g64, rtol=2**-22)
    np.testing.assert_allclose(v, (1 - HP["beta2"]) * g64 * g64, rtol=2**-21)


def test_adamw_constant_grad_three_steps_closed_form():
    p, m, v = _state(4000, ("cg",))
    p64 = p.astype(np.float64)
    g = synth.normal_f32(4000, 1e-3, ("cg", "g")).numpy()
    g64 = g.astype(np.float64)
    lr, wd, eps, b1, b2 = HP["lr"], HP["weight_decay"], HP["eps"], HP["beta1"], HP["beta2"]
    for t in (1, 2, 3):
        O.adamw(p, g, m, v, t, **HP)
        # bias-corrected moments of a constant gradient are g and g^2 exactly
        p64 = p64 * (1 - lr * wd) - lr * g64 / (np.abs(g64) + eps)
        np.testing.assert_allclose(m, (1 - b1 ** t) * g64, rtol=8 * 2**-24)
        np.testing.assert_allclose(v, (1 - b2 ** t) * g64 * g64, rtol=16 * 2**-24)
    np.testing.assert_allclose(p, p64, rtol=0, atol=32 * 2**-24 * np.abs(p64).max())


def test_adamw_commutes_with_sharding_bit_exact():
    """AdamW on each rank's chunk == chunk of AdamW on the whole tensor."""
    shape, n = (37, 6), 4
    W = synth.normal_f32(37 * 6, 0.02, ("sc", "W")).numpy().reshape(shape)
    grads = [synth.normal_f32(37 * 6, 1e-3, ("sc", t)).numpy().reshape(shape) for t in (1, 2, 3)]
    whole = [W.copy(), np.zeros(shape, F32), np.zeros(shape, F32)]
    for t, g in enumerate(grads, 1):
        O.adamw(whole[0], g, whole[1], whole[2], t, **HP)
    for r in range(n):
        b, lr_ = O.rows_of_rank(37, n, r)
        sh = [W[b:b + lr_].copy(), np.zeros((lr_, 6), F32), np.zeros((lr_, 6), F32)]
        for t, g in enumerate(grads, 1):
            O.adamw(sh[0], np.ascontiguousarray(g[b:b + lr_]), sh[1], sh[2], t, **HP)
        for a, w in zip(sh, whole):
            assert np.array_equal(a.view(np.uint32), w[b:b + lr_].view(np.uint32))


def test_adamw_matches_torch_optim_adamw_three_steps():
    cfg = configs.get(0)
    for i, prm in enumerate(cfg.params):
        n = prm.numel
        W = synth.normal_f32(n, 0.02, ("ta", i)).reshape(prm.shape)
        tp = torch.nn.Parameter(W.clone())
        opt = torch.optim.AdamW([tp], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]),
                                eps=HP["eps"], weight_decay=HP["weight_decay"], foreach=False)
        p = W.numpy().copy()
        m, v = np.zeros_like(p), np.zeros_like(p)
        for t in (1, 2, 3):
            g = synth.normal_f32(n, 1e-3, ("ta", i, t)).reshape(prm.shape)
            tp.grad = g.clone()
            opt.step()
            O.adamw(p, g.numpy(), m, v, t, **HP)
        st = opt.state[tp]
        for ours, ref in ((p, tp.detach()), (m, st["exp_avg"]), (v, st["exp_avg_sq"])):
            ref = ref.numpy()
            assert np.abs(ours - ref).max() <= 1e-6 * np.abs(ref).max()


def test_adamw_nearly_scale_invariant_in_grad():
    """Doubling every gradient barely moves AdamW (why a 2x reduce bug hid)."""
    p1, m1, v1 = _state(2000, ("si",))
    p2, m2, v2 = p1.copy(), m1.copy(), v1.copy()
    p0 = p1.copy()
    for t in (1, 2, 3):
        g = synth.normal_f32(2000, 1e-3, ("si", t)).numpy()
        O.adamw(p1, g, m1, v1, t, **HP)
        O.adamw(p2, (g * 2).astype(F32), m2, v2, t, **HP)
    moved = np.abs(p1 - p0).max()
    # only the eps term (and nothing else) sees the scale: tiny gradients move
    assert np.abs(p1 - p2).max() < 0.05 * moved
    assert np.abs(p1 - p2).mean() < 0.002 * moved
    assert not np.array_equal(m1, m2)


def test_adamw_scalars_precision():
    s = O.adamw_scalars(3e-4, 0.9, 0.999, 1e-8, 0.01, 2)
    assert s.decay == F32(1 - 3e-6)
    assert s.step_size == F32(3e-4 / (1 - 0.81))
    assert s.bc2_sqrt == F32(math.sqrt(1 - 0.999 ** 2))
    with pytest.raises(ValueError):
        O.adamw_scalars(3e-4, 0.9, 0.999, 1e-8, 0.01, 0)


# ---------------------------------------------------------------------------
# One whole step on the MLP probe, against torch library building blocks
# ---------------------------------------------------------------------------

def test_whole_step_mlp_probe_against_torch_building_blocks():
    cfg = configs.get(0)
    n = cfg.world
    shapes = [q.shape for q in cfg.params]
    Ws = [synth.normal_f32(q.numel, 0.02, ("ws", i)).reshape(q.shape) for i, q in enumerate(cfg.params)]
    plans = [O.plan(shapes, n, r) for r in range(n)]
    for r in range(n):
        p = plans[r]
        masters = [_chunks_of(W, n, r).numpy().copy() for W in Ws]
        ms = [np.zeros_like(x) for x in masters]
        vs = [np.zeros_like(x) for x in masters]
        tparams = [torch.nn.Parameter(torch.from_numpy(x.copy())) for x in masters]
        opt = torch.optim.AdamW(tparams, lr=cfg.hp.lr, betas=(cfg.hp.beta1, cfg.hp.beta2),
                                eps=cfg.hp.eps, weight_decay=cfg.hp.weight_decay, foreach=False)
        for t in (1, 2, 3):
            rs = _rs_buffer(p, n, ("ws", r, t))
            grads = O.reduce(p, rs)
            trs = torch.from_numpy(rs.view(np.int16)).view(torch.bfloat16).float()
            for e, g, tp in zip(p.entries, grads, tparams):
                tg = trs[:, e.shard_offset:e.shard_offset + e.valid_numel].sum(0) / n
                np.testing.assert_allclose(g, tg.numpy(), rtol=2e-6, atol=1e-12)
                tp.grad = tg.reshape(tp.shape).clone()
            opt.step()
            for x, g, m, v in zip(masters, grads, ms, vs):
                O.adamw(x, g.reshape(x.shape), m, v, t, **vars(cfg.hp))
        for x, tp in zip(masters, tparams):
            ref = tp.detach().numpy()
            assert np.abs(x - ref).max() <= 1e-6 * max(np.abs(ref).max(), 1e-30)
        seg = O.pack(p, masters)
        want = torch.cat([torch.cat([tp.detach().reshape(-1).to(torch.bfloat16).view(torch.int16),
                                     torch.zeros(e.seg_numel - e.valid_numel, dtype=torch.int16)])
                          for e, tp in zip(p.entries, tparams)]).numpy().view(np.uint16)
        # the two AdamW orders may differ by an fp32 ulp, which can move a bf16 tie
        diff = np.abs(seg.astype(np.int32) - want.astype(np.int32))
        assert diff.max() <= 1


# ---------------------------------------------------------------------------
# reduce-scatter copy-in and fp32 contributions
# ---------------------------------------------------------------------------

def _bf16_grads(shapes, key):
    out = []
    for i, s in enumerate(shapes):
        cols = int(np.prod(s[1:])) if len(s) > 1 else 1
        g = synth.bf16_bits_to_u16(synth.normal_bf16_bits(int(np.prod(s)), 1e-3, key + (i,)))
        out.append(g.reshape(s[0], cols))
    return out


@pytest.mark.parametrize("align", [1, 8])
@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_pack_reduce_scatter_matches_torch_chunk_pad_cat(case, align):
    shapes, n = SMALL_CASES[case]
    grads = _bf16_grads(shapes, ("rsp", case))
    p = O.plan(shapes, n, 0, align)
    got = O.pack_reduce_scatter(p, grads)
    for j in range(n):
        parts = []
        for g, e in zip(grads, p.entries):
            piece = _chunks_of(torch.from_numpy(g.view(np.int16)), n, j).reshape(-1)
            parts.append(torch.cat([piece, torch.zeros(e.seg_numel - piece.numel(), dtype=torch.int16)]))
        want = torch.cat(parts).numpy().view(np.uint16) if parts else np.zeros(0, np.uint16)
        assert np.array_equal(got[j], want), (case, j)
    # the layout is the all-gather's: copy-out of it gives the gradients back
    for g, full in zip(grads, O.unpack(p, got)):
        assert np.array_equal(full, g)
    # row j equals rank j's own piece: pack of the fp32 widening of its chunk
    for j in range(n):
        pj = O.plan(shapes, n, j, align)
        masters = [O.bf16_to_f32(_chunks_of(torch.from_numpy(g.view(np.int16)), n, j).numpy().view(np.uint16))
                   for g in grads]
        assert np.array_equal(O.pack(pj, masters), got[j])


def test_pack_reduce_scatter_f32_is_exact_widening_with_zero_padding():
    shapes, n = SMALL_CASES[1]
    grads = _bf16_grads(shapes, ("rsp32",))
    p = O.plan(shapes, n, 2)
    f = O.pack_reduce_scatter_f32(p, grads)
    b = O.pack_reduce_scatter(p, grads)
    assert f.dtype == np.float32 and f.shape == b.shape
    want = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(f.view(np.uint32), want.view(np.uint32))
    pad = np.ones(p.S, bool)
    for e in p.entries:
        pad[e.shard_offset:e.shard_offset + e.valid_numel] = False
    rank2_pad = f[2][pad]
    assert (rank2_pad.view(np.uint32) == 0).all()


@pytest.mark.parametrize("n", [1, 2, 6, 8, 64])
def test_reduce_f32_error_bound_and_torch(n):
    shapes = [(3 * n + 1, 5), (2 * n - 1 if n > 1 else 3,)]
    p = O.plan(shapes, n, n - 1)
    rng = np.random.default_rng(n)
    rs = (rng.standard_normal((n, p.S)) * 1e-3).astype(F32)
    grads = O.reduce_f32(p, rs)
    u = 2.0 ** -24
    t = torch.from_numpy(rs)
    for e, g in zip(p.entries, grads):
        sl = slice(e.shard_offset, e.shard_offset + e.valid_numel)
        for i in range(e.valid_numel):
            xs = [float(rs[j, e.shard_offset + i]) for j in range(n)]
            exact = math.fsum(xs) / n
            bound = (n - 1) * u * sum(abs(x) for x in xs) / n + u * abs(exact) + 1e-45
            assert abs(float(g[i]) - exact) <= bound * 1.0001
        # torch sums in another order: both are within the summation bound
        sumabs = t[:, sl].abs().sum(0).numpy().astype(np.float64) / n
        diff = np.abs(g.astype(np.float64) - (t[:, sl].sum(0) / n).numpy())
        assert (diff <= 2 * n * u * sumabs + 1e-30).all()


def test_reduce_f32_special_cases():
    # N = 1 is the identity; equal bf16-representable values average exactly
    p1 = O.plan([(5, 3)], 1, 0)
    x = np.random.default_rng(0).standard_normal((1, p1.S)).astype(F32)
    assert np.array_equal(O.reduce_f32(p1, x)[0].reshape(-1).view(np.uint32), x[0].view(np.uint32))
    p6 = O.plan([(12, 2)], 6, 3)
    row = O.bf16_to_f32(synth.bf16_bits_to_u16(synth.normal_bf16_bits(p6.S, 1e-3, ("r32eq",))))
    g = O.reduce_f32(p6, np.tile(row, (6, 1)))[0]
    e = p6.entries[0]
    assert np.array_equal(g.view(np.uint32), row[e.shard_offset:e.shard_offset + e.valid_numel].view(np.uint32))


# ---------------------------------------------------------------------------
# resharding a checkpoint to another world size
# ---------------------------------------------------------------------------

def _torch_shards(W, n):
    return [_chunks_of(W, n, j).contiguous() for j in range(n)]


@pytest.mark.parametrize("n1,n2", [(2, 1), (1, 2), (2, 3), (3, 2), (4, 6), (6, 4), (8, 64), (64, 8), (5, 5)])
def test_reshard_matches_torch_rechunk(n1, n2):
    for rows, cols in [(37, 3), (1, 5), (0, 4), (130, 1), (64, 2)]:
        W = torch.arange(rows * cols, dtype=torch.int32).reshape(rows, cols)
        src = [t.numpy() for t in _torch_shards(W, n1)]
        for d in range(n2):
            got = O.reshard(src, rows, cols, n2, d)
            want = _chunks_of(W, n2, d).reshape(-1).numpy()
            assert np.array_equal(got, want), (rows, n1, n2, d)
            # the runs say where every target element comes from, once
            runs = O.reshard_runs(rows, cols, n1, n2, d)
            cover = np.zeros(want.size, dtype=int)
            for s, so, do, k in runs:
                assert np.array_equal(src[s].reshape(-1)[so:so + k], want[do:do + k])
                cover[do:do + k] += 1
            assert (cover == 1).all()
            assert [r[2] for r in runs] == sorted(r[2] for r in runs)


def test_reshard_two_ranks_to_one_is_the_full_tensor_and_round_trips():
    # the checkpoint page's example: two shards reloaded into a plain model
    W = np.random.default_rng(1).standard_normal((33, 7)).astype(F32)
    src = [x.numpy() for x in _torch_shards(torch.from_numpy(W), 2)]
    assert np.array_equal(O.reshard(src, 33, 7, 1, 0).reshape(33, 7), W)
    for n1, n2 in [(2, 5), (8, 3), (6, 64)]:
        s1 = [x.numpy() for x in _torch_shards(torch.from_numpy(W), n1)]
        s2 = [O.reshard(s1, 33, 7, n2, d) for d in range(n2)]
        back = [O.reshard(s2, 33, 7, n1, d) for d in range(n1)]
        for a, b in zip(back, s1):
            assert np.array_equal(a, b.reshape(-1))


# ---------------------------------------------------------------------------
# gradient accumulation without sync
# ---------------------------------------------------------------------------

def test_accumulate_grad_sum_and_reset():
    shapes = [(37, 3), (129,)]
    micro = [_bf16_grads(shapes, ("acc", k)) for k in range(5)]
    acc = O.accumulate_grad(None, micro[0], reset=True)
    for a, g in zip(acc, micro[0]):                     # reset: exact widening
        assert np.array_equal(a.view(np.uint32), O.bf16_to_f32(g.reshape(-1)).view(np.uint32))
    for k in range(1, 5):
        acc = O.accumulate_grad(acc, micro[k], reset=False)
    u = 2.0 ** -24
    for i, a in enumerate(acc):
        xs = np.stack([O.bf16_to_f32(m[i].reshape(-1)).astype(np.float64) for m in micro])
        for e in range(a.size):
            exact = math.fsum(xs[:, e])
            assert abs(float(a[e]) - exact) <= 4 * u * np.abs(xs[:, e]).sum() + 1e-45
        # torch's sequential fp32 adds in the same order give the same bits
        t = torch.zeros(a.size)
        t += torch.from_numpy(xs[0].astype(np.float32))
        for k in range(1, 5):
            t = t + torch.from_numpy(xs[k].astype(np.float32))
        assert np.array_equal(t.numpy().view(np.uint32), a.view(np.uint32))
    # -0 survives a reset, and the sum is bit-stable when rerun
    neg0 = [np.full((2, 2), 0x8000, np.uint16)]
    assert O.accumulate_grad(None, neg0, True)[0].view(np.uint32)[0] == 0x80000000


@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_pack_reduce_scatter_acc_layout(case):
    shapes, n = SMALL_CASES[case]
    grads = _bf16_grads(shapes, ("rspa", case))
    p = O.plan(shapes, n, 0)
    acc = O.accumulate_grad(None, grads, reset=True)
    # from a single microbatch it is the fp32 copy-in of that gradient
    assert np.array_equal(O.pack_reduce_scatter_acc(p, acc).view(np.uint32),
                          O.pack_reduce_scatter_f32(p, grads).view(np.uint32))
    # and against torch.chunk / pad / cat on fp32 values
    got = O.pack_reduce_scatter_acc(p, [a * np.float32(3) for a in acc])
    for j in range(n):
        parts = []
        for a, e, s in zip(acc, p.entries, shapes):
            rows, cols = s[0], (int(np.prod(s[1:])) if len(s) > 1 else 1)
            piece = _chunks_of(torch.from_numpy(a * np.float32(3)).reshape(rows, cols), n, j).reshape(-1)
            parts.append(torch.cat([piece, torch.zeros(e.seg_numel - piece.numel())]))
        want = torch.cat(parts).numpy() if parts else np.zeros(0, np.float32)
        assert np.array_equal(got[j].view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------------------
# FP8 E4M3 all-gather
# ---------------------------------------------------------------------------

def test_e4m3_golden_vectors():
    for ln in read_golden("e4m3_cases.txt"):
        f, b = ln.split()[:2]
        x = np.array([int(f, 16)], dtype=np.uint32).view(F32)
        assert int(O.e4m3_sat(x)[0]) == int(b, 16), (f, b)


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    dec = O.e4m3_to_f32(codes)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(dec), np.isnan(t))
    assert np.array_equal(dec[~np.isnan(dec)].view(np.uint32), t[~np.isnan(t)].view(np.uint32))


def test_e4m3_encode_is_nearest_even_brute_force_and_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_to_f32(codes).astype(np.float64)
    finite = ~np.isnan(vals)
    rng = np.random.default_rng(4)
    x = np.concatenate([(rng.standard_normal(20000) * s).astype(F32) for s in (1e-3, 0.02, 1.0, 50.0, 600.0)])
    # every midpoint between neighbouring codes and its neighbours
    pos = np.sort(np.unique(vals[finite & (vals >= 0)]))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(F32)
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    got = O.e4m3_sat(x)
    # brute force: nearest finite code in exact arithmetic, ties to even mantissa
    for xi, gi in zip(x.astype(np.float64), got):
        c = np.clip(xi, -448.0, 448.0)
        d = np.abs(vals - c)
        d[~finite] = np.inf
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            best = [b for b in best if (b & 1) == 0]
        want = best[0]
        if c == 0.0:
            want = 0x80 if np.signbit(xi) else 0x00
        assert gi == want or (vals[gi] == vals[want]), (xi, gi, want)
    t = torch.from_numpy(x).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(t, got)


@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_pack_fp8_matches_torch_and_unpack_round_trips(case):
    shapes, n = SMALL_CASES[case]
    Ws = [synth.normal_f32(int(np.prod(s)), 0.02, ("fp8", case, i)).reshape(s) for i, s in enumerate(shapes)]
    scales = [float(448.0 / max(float(W.abs().max()) if W.numel() else 1.0, 1e-12)) for W in Ws]
    plans = [O.plan(shapes, n, r) for r in range(n)]
    ag = np.stack([O.pack_fp8(plans[r], [_chunks_of(W, n, r).numpy() for W in Ws], scales)
                   for r in range(n)])
    for r in range(n):
        parts = []
        for W, e, sc in zip(Ws, plans[r].entries, scales):
            piece = (_chunks_of(W, n, r).reshape(-1) * np.float32(sc)).clamp(-448, 448)
            q = piece.to(torch.float8_e4m3fn).view(torch.uint8)
            parts.append(torch.cat([q, torch.zeros(e.seg_numel - q.numel(), dtype=torch.uint8)]))
        want = torch.cat(parts).numpy() if parts else np.zeros(0, np.uint8)
        assert np.array_equal(ag[r], want)
    for W, full, sc in zip(Ws, O.unpack_fp8(plans[0], ag), scales):
        want = O.e4m3_sat(W.reshape(-1).numpy() * np.float32(sc))
        assert np.array_equal(full.reshape(-1), want)
    # the scale maps each tensor's largest magnitude onto 448
    for W, full, sc in zip(Ws, O.unpack_fp8(plans[0], ag), scales):
        if W.numel():
            assert np.nanmax(np.abs(O.e4m3_to_f32(full))) == 448.0


def test_amax_matches_torch():
    shards = [synth.normal_f32(k, 0.02, ("amax", k)).numpy() for k in (1, 17, 4097)] + [np.zeros(0, F32)]
    got = O.amax(shards)
    for g, s in zip(got, shards):
        assert g == (np.abs(s).max() if s.size else 0.0)
    assert np.isnan(O.amax([np.array([1.0, np.nan, -3.0], F32)])[0])
    # the largest magnitude can be negative; -0 has magnitude +0
    hand = [np.array([3.0, -7.5, 2.0], F32), np.array([-1e-30], F32), np.array([-0.0, 0.0], F32),
            np.array([-np.inf, 1.0], F32)]
    got = O.amax(hand)
    assert got.view(np.uint32).tolist() == np.array([7.5, 1e-30, 0.0, np.inf], F32).view(np.uint32).tolist()
    for g, s in zip(got, hand):
        assert g == torch.from_numpy(s).abs().max().item()
