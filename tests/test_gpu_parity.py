"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: layout, pack and unpack bit-exact; casts within 1 bf16 ulp (bit-exact
expected); fp32 reductions and AdamW's master, m and v after 3 steps within a
normwise relative error of 1e-6 (bit-exact expected: both sides round every
fp32 operation once in the same order; the count of differing elements is
reported and must be 0).

Inputs are seeded synthetic draws (workloads.synth) and never come from the
HIP path.  Small and medium cases are compared whole; full-size groups of the
7B- and 70B-shaped workloads run in the same launch configuration the bench
times and are checked on sampled outputs and by exact properties that hold at
any size.
"""
import numpy as np
import pytest
import torch

from oracle import fsdp as O
from workloads import configs, synth

pytestmark = pytest.mark.gpu

capi = pytest.importorskip("sharded_shard_amd.capi")
from sharded_shard_amd.group import ShardedGroup  # noqa: E402

DEV = "cuda"
HP = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
GUARD = 4096
GUARD_VAL = 0x5A5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()


def u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32(t):
    return t.detach().cpu().contiguous().numpy()


def normwise(a, b):
    den = max(float(np.abs(b).max()) if b.size else 0.0, 1e-30)
    return float(np.abs(a.astype(np.float64) - b.astype(np.float64)).max()) / den if a.size else 0.0


def guarded_i16(n, fill=GUARD_VAL):
    """int16 device buffer with GUARD elements of guard value on each side."""
    buf = torch.full((n + 2 * GUARD,), fill - 65536 if fill > 32767 else fill,
                     dtype=torch.int16, device=DEV)
    return buf, buf[GUARD:GUARD + n]


def assert_guards(buf, n, fill=GUARD_VAL):
    h = u16(buf)
    assert (h[:GUARD] == fill).all() and (h[GUARD + n:] == fill).all(), "write outside the buffer"


def shapes_cols(shapes):
    return [int(np.prod(s[1:])) if len(s) > 1 else 1 for s in shapes]


CASES = [
    ("mlp-probe", [(32, 16), (32,), (4, 32), (4,)], 2),
    ("ragged-n6", [(1000, 70), (333,), (77, 129), (1, 2048), (1,), (64, 2048)], 6),
    ("empty-rows", [(5, 3), (0, 4), (7,), (1, 5), (13, 2)], 4),
    ("more-ranks", [(6, 3), (17,)], 8),
    ("n1", [(9, 7), (4097,)], 1),
    ("tiles", [(300, 1000), (4096, 33), (70001,)], 8),
    # odd pieces over several row batches (12 = 8 + 4, 64 = 8 x 8)
    ("odd-n12", [(1000, 37), (4097,), (129, 3), (25, 8)], 12),
    ("odd-n64", [(700, 9), (129,), (64, 33)], 64),
    # every piece a multiple of 8 elements: 16-byte aligned rows, the fused
    # step's wide kernel from 16 ranks (several tiles, empty chunks)
    ("wide-n16", [(2048, 160), (4096,), (96, 40), (17, 8)], 16),
    ("wide-n64", [(5000, 24), (64, 72), (129, 8), (1, 8)], 64),
]


def _case_ids():
    return [c[0] for c in CASES]


def _fill_masters(g, key):
    for i, e in enumerate(g.entries):
        if e.valid_numel:
            g.shard_view(g.master_flat, i).copy_(synth.normal_f32(e.valid_numel, 0.02, key + (i,)))


# ---------------------------------------------------------------------------
# copy-in
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("align", [1, 8])
@pytest.mark.parametrize("case", range(len(CASES)), ids=_case_ids())
def test_pack_bit_exact(case, align):
    name, shapes, n = CASES[case]
    for r in range(n):
        g = ShardedGroup(shapes, n, r, align)
        _fill_masters(g, ("pack", name, r))
        buf, ag = guarded_i16(n * g.S)
        row = ag[r * g.S:(r + 1) * g.S]
        g.pack(row)
        torch.cuda.synchronize()
        ref = O.pack(O.plan(shapes, n, r, align),
                     [f32(g.shard_view(g.master_flat, i)) for i in range(len(shapes))])
        got = u16(ag).reshape(n, g.S) if g.S else np.zeros((n, 0), np.uint16)
        assert np.array_equal(got[r], ref)
        others = np.delete(got, r, axis=0)
        assert (others == GUARD_VAL).all(), "pack wrote outside its row"
        assert_guards(buf, n * g.S)
        g.close()


def test_pack_special_values_and_misaligned_sources():
    """NaN, infinities, ties, subnormals; shards at every 4-byte offset mod 16."""
    specials = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0x7FA00000, 0x7F800000, 0xFF800000,
                         0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F7FFF, 0x3F808000, 0x3F818000, 0xBF818000,
                         0x00000001, 0x00008000, 0x00018000, 0x007FFFFF, 0x80000000, 0x00000000],
                        dtype=np.uint32).view(np.float32)
    rng = np.random.default_rng(0)
    shapes = [(97, 13), (1031,), (5, 8)]
    n, r = 3, 1
    plan = O.plan(shapes, n, r)
    for shift in range(4):
        g = ShardedGroup(shapes, n, r, bind=False)
        g.allocate()
        masters = []
        views = []
        base = torch.zeros(sum(e.valid_numel + 8 for e in g.entries) + 64, dtype=torch.float32, device=DEV)
        o = shift
        for e in g.entries:
            vals = rng.standard_normal(e.valid_numel).astype(np.float32) * 0.02
            k = min(len(specials), e.valid_numel)
            vals[:k] = specials[:k]
            vals[-k:] = specials[:k][::-1]
            v = base[o:o + e.valid_numel]
            v.copy_(torch.from_numpy(vals))
            masters.append(vals)
            views.append(v)
            o += e.valid_numel + 1   # consecutive shards at different alignments
        capi.fsdp_bind(g.plan, master=[v.data_ptr() for v in views], stream=None)
        for off in (0, 1, 3):      # ag_in at 2-byte offsets 0, 2, 6 mod 16
            buf = torch.zeros(g.S + 16, dtype=torch.int16, device=DEV)
            g.pack(buf[off:off + g.S])
            torch.cuda.synchronize()
            assert np.array_equal(u16(buf)[off:off + g.S], O.pack(plan, masters))
        g.close()


# ---------------------------------------------------------------------------
# copy-out
# ---------------------------------------------------------------------------

def _rand_ag(n, S, key, sentinel_mask=None):
    ag = np.empty((n, S), dtype=np.uint16)
    rng = np.random.default_rng(synth.seed_for(*key) % (2**32))
    ag[:] = rng.integers(0, 2**16, size=(n, S), dtype=np.uint16)
    if sentinel_mask is not None:
        ag[:, sentinel_mask] = synth.SENTINEL_BF16
    return ag


def _pad_mask(plan):
    m = np.ones(plan.S, dtype=bool)
    for e in plan.entries:
        m[e.shard_offset:e.shard_offset + e.valid_numel] = False
    return m


@pytest.mark.parametrize("align", [1, 8])
@pytest.mark.parametrize("case", range(len(CASES)), ids=_case_ids())
def test_unpack_bit_exact_with_guards(case, align):
    name, shapes, n = CASES[case]
    for r in sorted({0, n - 1}):
        plan = O.plan(shapes, n, r, align)
        # padding of every row holds the sentinel (any rank's padding: rank 0's
        # pieces are the longest, so mark what rank j leaves unused per row)
        ag = _rand_ag(n, plan.S, ("unpack", name, r, align))
        for j in range(n):
            ag[j, _pad_mask(O.plan(shapes, n, j, align))] = synth.SENTINEL_BF16
        g = ShardedGroup(shapes, n, r, align, bind=False)
        g.allocate(full=False)
        fbuf, full = guarded_i16(g.full_space)
        full.fill_(0x1234)
        g.full_flat = full
        g.bind()
        for off in (0, 3):   # ag_out 16-byte aligned, then at a 6-byte offset
            src = torch.zeros(n * plan.S + 8, dtype=torch.int16, device=DEV)
            src[off:off + n * plan.S].copy_(torch.from_numpy(ag.reshape(-1).view(np.int16)))
            g.unpack(src[off:off + n * plan.S])
            torch.cuda.synchronize()
            ref = O.unpack(plan, ag)
            for i, want in enumerate(ref):
                assert np.array_equal(u16(g.full_view(i)), want), (name, r, i, off)
            # the gaps between full views keep their fill
            h = u16(full)
            mask = np.ones(g.full_space, dtype=bool)
            for i in range(len(shapes)):
                o = g.full_offsets[i]
                mask[o:o + g.rows[i] * g.cols[i]] = False
            assert (h[mask] == 0x1234).all()
            assert_guards(fbuf, g.full_space)
        g.close()


@pytest.mark.parametrize("align", [1, 8])
def test_unpack_misaligned_full_destinations(align):
    """Full tensors at every 2-byte offset modulo 16; with align 8 every row
    piece of the source is 16-byte aligned (the copy-out's other block shape)."""
    shapes, n = [(37, 11), (999,), (8, 64)], 5
    plan = O.plan(shapes, n, 2, align)
    ag = _rand_ag(n, plan.S, ("mis", align))
    src = torch.from_numpy(ag.reshape(-1).view(np.int16)).to(DEV)
    ref = O.unpack(plan, ag)
    for shift in range(8):
        g = ShardedGroup(shapes, n, 2, align, bind=False)
        arena = torch.zeros(sum(r * c + 9 for r, c in zip(g.rows, g.cols)) + 16,
                            dtype=torch.int16, device=DEV)
        views, o = [], shift
        for r_, c_ in zip(g.rows, g.cols):
            views.append(arena[o:o + r_ * c_])
            o += r_ * c_ + 1
        capi.fsdp_bind(g.plan, full=[v.data_ptr() for v in views], stream=None)
        g.unpack(src)
        torch.cuda.synchronize()
        for v, want in zip(views, ref):
            assert np.array_equal(u16(v), want.reshape(-1)), shift
        g.close()


# ---------------------------------------------------------------------------
# reduce
# ---------------------------------------------------------------------------

def _rs_input(plan, n, key):
    rs = np.empty((n, plan.S), dtype=np.uint16)
    for j in range(n):
        rs[j] = synth.bf16_bits_to_u16(synth.normal_bf16_bits(plan.S, 1e-3, key + (j,)))
    rs[:, _pad_mask(plan)] = synth.SENTINEL_BF16
    return rs


def _cmp_f32(got, want, what):
    assert got.shape == want.shape
    if not got.size:
        return
    assert normwise(got, want) <= 1e-6, what
    nbad = int((got.view(np.uint32) != want.view(np.uint32)).sum())
    assert nbad == 0, f"{what}: {nbad} elements differ in bits (within tolerance)"


@pytest.mark.parametrize("case", range(len(CASES)), ids=_case_ids())
def test_reduce_matches_oracle(case):
    name, shapes, n = CASES[case]
    for r in sorted({0, n - 1, n // 2}):
        plan = O.plan(shapes, n, r)
        rs = _rs_input(plan, n, ("reduce", name, r))
        g = ShardedGroup(shapes, n, r)
        for off in (0, 1):
            src = torch.zeros(n * plan.S + 8, dtype=torch.int16, device=DEV)
            src[off:off + n * plan.S].copy_(torch.from_numpy(rs.reshape(-1).view(np.int16)))
            g.grad_flat.fill_(float("nan"))
            g.reduce(src[off:off + n * plan.S])
            torch.cuda.synchronize()
            for i, want in enumerate(O.reduce(plan, rs)):
                _cmp_f32(f32(g.shard_view(g.grad_flat, i)), want, (name, r, i, off))
        g.close()


@pytest.mark.parametrize("n", [1, 2, 6, 8, 64])
def test_reduce_all_equal_is_exact_and_odd_segments(n):
    shapes = [(3 * n + 1, 5), (2 * n + 1,), (n * 40 + 3, 67)]
    plan = O.plan(shapes, n, 0)
    row = synth.bf16_bits_to_u16(synth.normal_bf16_bits(plan.S, 1e-3, ("eq", n)))
    rs = np.tile(row, (n, 1))
    g = ShardedGroup(shapes, n, 0)
    g.reduce(torch.from_numpy(rs.reshape(-1).view(np.int16)).to(DEV))
    torch.cuda.synchronize()
    for i, e in enumerate(plan.entries):
        want = O.bf16_to_f32(row[e.shard_offset:e.shard_offset + e.valid_numel])
        got = f32(g.shard_view(g.grad_flat, i))
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    g.close()


# ---------------------------------------------------------------------------
# AdamW
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", range(len(CASES)), ids=_case_ids())
def test_adamw_three_steps_matches_oracle(case):
    name, shapes, n = CASES[case]
    r = n - 1
    g = ShardedGroup(shapes, n, r)
    _fill_masters(g, ("adamw", name))
    host = [[f32(g.shard_view(fl, i)) for i in range(len(shapes))]
            for fl in (g.master_flat, g.m_flat, g.v_flat)]
    for t in (1, 2, 3):
        for i, e in enumerate(g.entries):
            if e.valid_numel:
                gr = synth.normal_f32(e.valid_numel, 1e-3, ("adamw-g", name, t, i))
                g.shard_view(g.grad_flat, i).copy_(gr)
                O.adamw(host[0][i], gr.numpy(), host[1][i], host[2][i], t, **HP)
        g.adamw(t, **HP)
    torch.cuda.synchronize()
    for k, fl in enumerate((g.master_flat, g.m_flat, g.v_flat)):
        for i in range(len(shapes)):
            _cmp_f32(f32(g.shard_view(fl, i)), host[k][i], (name, k, i))
    g.close()


def test_adamw_misaligned_and_mixed_alignment_shards():
    """Shards whose four pointers share an offset mod 16, and ones that do not."""
    n_el = [1, 3, 4, 5, 8191, 8193, 20000]
    for mixed in (False, True):
        shapes = [(k,) for k in n_el]
        g = ShardedGroup(shapes, 1, 0, bind=False)
        bufs = [torch.zeros(sum(n_el) + 4 * len(n_el) + 16, dtype=torch.float32, device=DEV)
                for _ in range(4)]
        views = [[], [], [], []]
        for role in range(4):
            o = 1 + (role if mixed else 0)
            for k in n_el:
                views[role].append(bufs[role][o:o + k])
                o += k + 3
        host = [[], [], [], []]
        for i, k in enumerate(n_el):
            p0 = synth.normal_f32(k, 0.02, ("am", i))
            views[0][i].copy_(p0)
            host[0].append(p0.numpy().copy())
            host[2].append(np.zeros(k, np.float32))
            host[3].append(np.zeros(k, np.float32))
        capi.fsdp_bind(g.plan, *[[v.data_ptr() for v in views[role]] for role in range(4)], None)
        for t in (1, 2, 3):
            for i, k in enumerate(n_el):
                gr = synth.normal_f32(k, 1e-3, ("am-g", t, i))
                views[1][i].copy_(gr)
                O.adamw(host[0][i], gr.numpy(), host[2][i], host[3][i], t, **HP)
            g.adamw(t, **HP)
            torch.cuda.synchronize()
        for role in (0, 2, 3):
            for i in range(len(n_el)):
                _cmp_f32(f32(views[role][i]), host[role][i], (mixed, role, i))
        g.close()


# ---------------------------------------------------------------------------
# whole step on the MLP probe and the ragged MoE workload, every element
# ---------------------------------------------------------------------------

def _whole_step(cfg_index, ranks, steps=3, align=1):
    cfg = configs.get(cfg_index)
    n = cfg.world
    hp = vars(cfg.hp)
    for gi, grp in enumerate(cfg.groups):
        shapes = [p.shape for p in grp.params]
        for r in ranks:
            plan = O.plan(shapes, n, r, align)
            g = ShardedGroup(shapes, n, r, align)
            _fill_masters(g, ("step", cfg_index, gi, r))
            masters = [f32(g.shard_view(g.master_flat, i)) for i in range(len(shapes))]
            ms = [np.zeros_like(x) for x in masters]
            vs = [np.zeros_like(x) for x in masters]
            ag = torch.empty(n * plan.S, dtype=torch.int16, device=DEV)
            for t in range(1, steps + 1):
                rs = _rs_input(plan, n, ("step-rs", cfg_index, gi, r, t))
                g.reduce(torch.from_numpy(rs.reshape(-1).view(np.int16)).to(DEV))
                g.adamw(t, **hp)
                # other ranks' rows are synthetic; this rank packs its own row in place
                other = _rand_ag(n, plan.S, ("step-ag", cfg_index, gi, r, t))
                ag.copy_(torch.from_numpy(other.reshape(-1).view(np.int16)))
                g.pack(ag[r * plan.S:(r + 1) * plan.S])
                g.unpack(ag)
                torch.cuda.synchronize()
                grads = O.reduce(plan, rs)
                for x, gr, m, v in zip(masters, grads, ms, vs):
                    O.adamw(x, gr, m, v, t, **hp)
                other[r] = O.pack(plan, masters)
                for i, want in enumerate(grads):
                    _cmp_f32(f32(g.shard_view(g.grad_flat, i)), want, ("grad", gi, r, t, i))
                assert np.array_equal(u16(ag).reshape(n, plan.S)[r], other[r])
                for i, want in enumerate(O.unpack(plan, other)):
                    assert np.array_equal(u16(g.full_view(i)), want), ("full", gi, r, t, i)
            for fl, host in ((g.master_flat, masters), (g.m_flat, ms), (g.v_flat, vs)):
                for i in range(len(shapes)):
                    _cmp_f32(f32(g.shard_view(fl, i)), host[i], ("state", gi, r, i))
            g.close()
            del ag
            torch.cuda.empty_cache()


def test_whole_step_mlp_probe_all_ranks():
    _whole_step(0, ranks=(0, 1))


@pytest.mark.parametrize("rank", [5, 0])
def test_whole_step_moe_ragged(rank):
    _whole_step(3, ranks=(rank,), steps=1)


def test_whole_step_llama_block_rank0():
    _whole_step(1, ranks=(0,), steps=1)


def test_determinism_two_runs_identical():
    shapes, n = [(1000, 70), (333,), (77, 129)], 6
    outs = []
    for _ in range(2):
        g = ShardedGroup(shapes, n, 4)
        _fill_masters(g, ("det",))
        plan = O.plan(shapes, n, 4)
        rs = torch.from_numpy(_rs_input(plan, n, ("det-rs",)).reshape(-1).view(np.int16)).to(DEV)
        g.reduce(rs)
        g.adamw(1, **HP)
        ag = torch.zeros(n * plan.S, dtype=torch.int16, device=DEV)
        g.pack(ag[4 * plan.S:5 * plan.S])
        g.unpack(ag)
        torch.cuda.synchronize()
        outs.append([u16(ag), f32(g.master_flat), f32(g.grad_flat), u16(g.full_flat)])
        g.close()
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_empty_group_calls_are_no_ops():
    g = ShardedGroup([(0, 4), (0,)], 4, 1)
    g.reduce(torch.zeros(1, dtype=torch.int16, device=DEV))
    g.adamw(1, **HP)
    g.pack(torch.zeros(1, dtype=torch.int16, device=DEV))
    g.unpack(torch.zeros(1, dtype=torch.int16, device=DEV))
    capi.fsdp_check_stream()
    g.close()


# ---------------------------------------------------------------------------
# fused step: reduce -> AdamW -> pack in one pass
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("align", [1, 8])
@pytest.mark.parametrize("write_grad", [False, True], ids=["nograd", "grad"])
@pytest.mark.parametrize("case", range(len(CASES)), ids=_case_ids())
def test_fused_step_equals_separate_calls_and_oracle(case, write_grad, align):
    """align 1 puts most cases on misaligned rows (the misaligned fused
    kernel); align 8 makes every row piece 16-byte aligned, so the aligned
    kernel (below 16 ranks) and the wide one run on whole multi-tile groups."""
    name, shapes, n = CASES[case]
    hp = HP
    for r in sorted({0, n - 1}):
        plan = O.plan(shapes, n, r, align)
        ga, gb = ShardedGroup(shapes, n, r, align), ShardedGroup(shapes, n, r, align)
        _fill_masters(ga, ("fused", name, r))
        gb.master_flat.copy_(ga.master_flat)
        masters = [f32(ga.shard_view(ga.master_flat, i)) for i in range(len(shapes))]
        ms = [np.zeros_like(x) for x in masters]
        vs = [np.zeros_like(x) for x in masters]
        for t in (1, 2, 3):
            rs = _rs_input(plan, n, ("fused-rs", name, r, t))
            d_rs = torch.from_numpy(rs.reshape(-1).view(np.int16)).to(DEV)
            off = t - 1            # ag_in at 0, 2 and 4 bytes past a 16-byte boundary
            aga = torch.full((plan.S + 16,), 7, dtype=torch.int16, device=DEV)
            agb = torch.full((plan.S + 16,), 7, dtype=torch.int16, device=DEV)
            ga.reduce(d_rs)
            ga.adamw(t, **hp)
            ga.pack(aga[off:off + plan.S])
            gb.grad_flat.fill_(-1.0)
            gb.step(d_rs, agb[off:off + plan.S], t, write_grad=write_grad, **hp)
            torch.cuda.synchronize()
            assert torch.equal(aga, agb), (name, r, t)
            for fl in ("master_flat", "m_flat", "v_flat"):
                assert torch.equal(getattr(ga, fl).view(torch.int32), getattr(gb, fl).view(torch.int32))
            grads = O.reduce(plan, rs)
            for x, gr, m, v in zip(masters, grads, ms, vs):
                O.adamw(x, gr, m, v, t, **hp)
            assert np.array_equal(u16(agb)[off:off + plan.S], O.pack(plan, masters))
            for i in range(len(shapes)):
                _cmp_f32(f32(gb.shard_view(gb.master_flat, i)), masters[i], ("p", name, r, t, i))
                _cmp_f32(f32(gb.shard_view(gb.m_flat, i)), ms[i], ("m", name, r, t, i))
                _cmp_f32(f32(gb.shard_view(gb.v_flat, i)), vs[i], ("v", name, r, t, i))
                got_g = f32(gb.shard_view(gb.grad_flat, i))
                if write_grad:
                    _cmp_f32(got_g, grads[i], ("g", name, r, t, i))
                else:
                    assert (got_g == -1.0).all(), "grad written without the flag"
        ga.close()
        gb.close()


# bf16 specials injected into gradient contributions: +-inf, NaN, +-max
# finite (sums overflow), smallest and largest subnormals, -0, smallest normal
_BF16_SPECIALS = [0x7F80, 0xFF80, 0x7FC0, 0x7F7F, 0xFF7F, 0x0001, 0x8001, 0x007F, 0x8000, 0x0080]
# fp32 masters: zeros, near overflow, subnormals, infinities, NaN
_F32_SPECIALS = [0.0, -0.0, 3.0e38, -3.0e38, 1e-45, -1e-40, 1e-30, float("inf"), float("-inf"),
                 float("nan")]


def _bf16_is_nan(u):
    return ((u & 0x7F80) == 0x7F80) & ((u & 0x7F) != 0)


def _same_f32_nan_ok(got, want, what):
    """Bit-exact, except that any NaN matches any NaN: IEEE 754 leaves the sign
    and payload of a NaN that an invalid operation creates to the machine."""
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), (what, int((gn != wn).sum()))
    assert np.array_equal(got[~gn].view(np.uint32), want[~wn].view(np.uint32)), what


def _same_bf16_nan_ok(got, want, what):
    gn, wn = _bf16_is_nan(got), _bf16_is_nan(want)
    assert np.array_equal(gn, wn), (what, int((gn != wn).sum()))
    assert np.array_equal(got[~gn], want[~wn]), what


@pytest.mark.parametrize("fused", ["separate", "fused", "set"])
@pytest.mark.parametrize("n,align", [(3, 1), (6, 1), (8, 8), (16, 8), (64, 8)])
def test_step_special_values_match_oracle(n, align, fused):
    """Infinities, NaNs, overflowing sums, subnormals and signed zeros through
    reduce, AdamW and the copy-in for 3 steps, on the misaligned, aligned and
    wide kernels, and with AdamW fused with the copy-in over a group set:
    every output bit-exact with the oracle, NaNs matched as NaNs."""
    shapes = [(37, 5), (64,), (130, 3), (9, 129), (1024, 16)]
    r = n // 2
    plan = O.plan(shapes, n, r, align)
    g = ShardedGroup(shapes, n, r, align)
    gset = capi.fsdp_group_set_create([g.plan]) if fused == "set" else None
    rng = np.random.default_rng(7000 + n)
    masters = []
    for i, e in enumerate(g.entries):
        x = synth.normal_f32(e.valid_numel, 0.02, ("spec-m", n, i)).numpy().copy()
        if x.size:
            pos = rng.choice(x.size, size=min(x.size, len(_F32_SPECIALS)), replace=False)
            x[pos] = np.array(_F32_SPECIALS[:pos.size], dtype=np.float32)
        g.shard_view(g.master_flat, i).copy_(torch.from_numpy(x))
        masters.append(x)
    ms = [np.zeros_like(x) for x in masters]
    vs = [np.zeros_like(x) for x in masters]
    seen = set()
    for t in (1, 2, 3):
        rs = _rs_input(plan, n, ("spec-rs", n, t))
        mask = ~_pad_mask(plan)
        hit = (rng.random(rs.shape) < 0.2) & mask[None, :]
        rs[hit] = rng.choice(np.array(_BF16_SPECIALS, dtype=np.uint16), size=int(hit.sum()))
        # a few columns of subnormals in every row: subnormal sums and means
        cols = rng.choice(np.flatnonzero(mask), size=4, replace=False)
        rs[:, cols[:2]] = 0x0001
        rs[:, cols[2:]] = 0x807F
        d_rs = torch.from_numpy(rs.reshape(-1).view(np.int16)).to(DEV)
        ag = torch.zeros((plan.S + 7) // 8 * 8, dtype=torch.int16, device=DEV)
        if fused == "fused":
            g.step(d_rs, ag[:plan.S], t, write_grad=True, **HP)
        elif fused == "set":
            g.reduce(d_rs)
            capi.fsdp_adamw_pack_groups(gset, ag, step=t, **HP)
        else:
            g.reduce(d_rs)
            g.adamw(t, **HP)
            g.pack(ag[:plan.S])
        torch.cuda.synchronize()
        ag = ag[:plan.S]
        with np.errstate(all="ignore"):
            grads = O.reduce(plan, rs)
            for x, gr, m, v in zip(masters, grads, ms, vs):
                O.adamw(x, gr, m, v, t, **HP)
            want_ag = O.pack(plan, masters)
        for gr in grads:
            a = np.abs(gr)
            seen.update(k for k, hit in (("nan", np.isnan(gr).any()), ("inf", np.isinf(gr).any()),
                                         ("sub", ((a > 0) & (a < 2.0 ** -126)).any())) if hit)
        _same_bf16_nan_ok(u16(ag), want_ag, ("ag", n, t))
        for i in range(len(shapes)):
            _same_f32_nan_ok(f32(g.shard_view(g.grad_flat, i)), grads[i], ("g", n, t, i))
            _same_f32_nan_ok(f32(g.shard_view(g.master_flat, i)), masters[i], ("p", n, t, i))
            _same_f32_nan_ok(f32(g.shard_view(g.m_flat, i)), ms[i], ("m", n, t, i))
            _same_f32_nan_ok(f32(g.shard_view(g.v_flat, i)), vs[i], ("v", n, t, i))
    if gset is not None:
        capi.fsdp_group_set_destroy(gset)
    g.close()
    assert seen == {"nan", "inf", "sub"}, seen     # the specials reached the reduction


def test_fused_step_mixed_alignment_shards():
    """Shards whose pointers differ modulo 16 take the element-wise path."""
    shapes, n, r = [(41, 9), (777,), (3, 5)], 3, 1
    plan = O.plan(shapes, n, r)
    g = ShardedGroup(shapes, n, r, bind=False)
    bufs = [torch.zeros(plan.V + 64, dtype=torch.float32, device=DEV) for _ in range(4)]
    views = [[], [], [], []]
    for role in range(4):
        o = 1 + role
        for e in g.entries:
            views[role].append(bufs[role][o:o + e.valid_numel])
            o += e.valid_numel + 5
    host = []
    for i, e in enumerate(g.entries):
        p0 = synth.normal_f32(e.valid_numel, 0.02, ("fm", i))
        views[0][i].copy_(p0)
        host.append(p0.numpy().copy())
    capi.fsdp_bind(g.plan, *[[v.data_ptr() for v in views[role]] for role in range(4)], None)
    ms = [np.zeros_like(x) for x in host]
    vs = [np.zeros_like(x) for x in host]
    for t in (1, 2):
        rs = _rs_input(plan, n, ("fm-rs", t))
        ag = torch.zeros(plan.S + 8, dtype=torch.int16, device=DEV)
        g.step(torch.from_numpy(rs.reshape(-1).view(np.int16)).to(DEV), ag[3:3 + plan.S], t,
               write_grad=True, **HP)
        torch.cuda.synchronize()
        grads = O.reduce(plan, rs)
        for x, gr, m, v in zip(host, grads, ms, vs):
            O.adamw(x, gr, m, v, t, **HP)
        assert np.array_equal(u16(ag)[3:3 + plan.S], O.pack(plan, host))
        for i in range(len(shapes)):
            _cmp_f32(f32(views[0][i]), host[i], ("p", t, i))
            _cmp_f32(f32(views[1][i]), grads[i], ("g", t, i))
            _cmp_f32(f32(views[2][i]), ms[i], ("m", t, i))
            _cmp_f32(f32(views[3][i]), vs[i], ("v", t, i))
    g.close()


@pytest.mark.parametrize("arena_off", [0, 1, 2, 3])
def test_set_adamw_copy_in_mixed_alignment_and_output_phase(arena_off):
    """AdamW fused with the copy-in over a group set: shards whose pointers
    differ modulo 16 take the element-wise path, equal ones the vector path,
    and the bf16 output lands at every 2-byte phase; both against the oracle
    and against fsdp_adamw_groups + fsdp_pack_allgather_groups."""
    shapes, n, r = [(41, 9), (777,), (3, 5), (128, 8)], 3, 1
    plan = O.plan(shapes, n, r)
    g = ShardedGroup(shapes, n, r, bind=False)
    h = ShardedGroup(shapes, n, r)                  # equal phases: the vector path
    bufs = [torch.zeros(plan.V + 64, dtype=torch.float32, device=DEV) for _ in range(4)]
    views = [[], [], [], []]
    for role in range(4):
        o = 1 + role
        for e in g.entries:
            views[role].append(bufs[role][o:o + e.valid_numel])
            o += e.valid_numel + 5
    host = []
    for i, e in enumerate(g.entries):
        p0 = synth.normal_f32(e.valid_numel, 0.02, ("sm", i))
        g0 = synth.normal_f32(e.valid_numel, 1e-3, ("sg", i))
        views[0][i].copy_(p0)
        views[1][i].copy_(g0)
        h.shard_view(h.master_flat, i).copy_(p0)
        h.shard_view(h.grad_flat, i).copy_(g0)
        host.append((p0.numpy().copy(), g0.numpy().copy()))
    capi.fsdp_bind(g.plan, *[[v.data_ptr() for v in views[role]] for role in range(4)], None)
    ref = ShardedGroup(shapes, n, r)                # h's twin through the two launches
    ref.master_flat.copy_(h.master_flat)
    ref.grad_flat.copy_(h.grad_flat)
    sets = [capi.fsdp_group_set_create([x.plan]) for x in (g, h, ref)]
    total = capi.fsdp_group_set_info(sets[0])[1]
    arenas = [torch.full((total + 8,), 0x5A5A, dtype=torch.int16, device=DEV) for _ in range(3)]
    ms = [np.zeros_like(p) for p, _ in host]
    vs = [np.zeros_like(p) for p, _ in host]
    ps = [p.copy() for p, _ in host]
    for t in (1, 2):
        a = [x[arena_off:arena_off + total] for x in arenas]
        capi.fsdp_adamw_pack_groups(sets[0], a[0], step=t, **HP)
        capi.fsdp_adamw_pack_groups(sets[1], a[1], step=t, **HP)
        capi.fsdp_adamw_groups(sets[2], step=t, **HP)
        capi.fsdp_pack_allgather_groups(sets[2], a[2])
        torch.cuda.synchronize()
        for x, (_, gr), m, v in zip(ps, host, ms, vs):
            O.adamw(x, gr, m, v, t, **HP)
        want = O.pack(plan, ps)
        for k in range(3):
            assert np.array_equal(u16(a[k])[:plan.S], want), (k, t)
            assert (u16(arenas[k])[:arena_off] == 0x5A5A).all()
            assert (u16(arenas[k])[arena_off + plan.S:] == 0x5A5A).all()
        for i in range(len(shapes)):
            _cmp_f32(f32(views[0][i]), ps[i], ("p", t, i))
            _cmp_f32(f32(views[2][i]), ms[i], ("m", t, i))
            _cmp_f32(f32(views[3][i]), vs[i], ("v", t, i))
            for x in (h, ref):
                _cmp_f32(f32(x.shard_view(x.master_flat, i)), ps[i], ("p vec", t, i))
                _cmp_f32(f32(x.shard_view(x.m_flat, i)), ms[i], ("m vec", t, i))
    for st in sets:
        capi.fsdp_group_set_destroy(st)
    for x in (g, h, ref):
        x.close()


def test_fused_step_rejects_unbound_and_bad_flags():
    g = ShardedGroup([(8, 4)], 2, 0)
    rs = torch.zeros(2 * g.S, dtype=torch.int16, device=DEV)
    ag = torch.zeros(g.S, dtype=torch.int16, device=DEV)
    with pytest.raises(capi.FsdpError) as ei:
        capi.fsdp_step_shard(g.plan, rs, ag, 3e-4, 0.9, 0.999, 1e-8, 0.01, 1, flags=2)
    assert ei.value.status == capi.FSDP_E_INVAL
    with pytest.raises(capi.FsdpError) as ei:
        capi.fsdp_step_shard(g.plan, rs, ag, 3e-4, 0.9, 0.999, 1e-8, 0.01, 0)
    assert ei.value.status == capi.FSDP_E_INVAL
    # ag_in may not share bytes with rs_in (it is written while rs_in is read)
    both = torch.zeros(3 * g.S, dtype=torch.int16, device=DEV)
    for a in (both[g.S - 1:2 * g.S - 1], both[2 * g.S - 1:3 * g.S - 1], both[:g.S]):
        with pytest.raises(capi.FsdpError) as ei:
            capi.fsdp_step_shard(g.plan, both[:2 * g.S], a, 3e-4, 0.9, 0.999, 1e-8, 0.01, 1)
        assert ei.value.status == capi.FSDP_E_INVAL
    capi.fsdp_step_shard(g.plan, both[:2 * g.S], both[2 * g.S:], 3e-4, 0.9, 0.999, 1e-8, 0.01, 1)
    torch.cuda.synchronize()
    g.close()


def test_injected_launch_fault_reaches_the_caller(monkeypatch):
    """FSDP_FAULT=launch fails every launch before it is enqueued;
    FSDP_FAULT=launch@K only the K-th.  The caller sees FSDP_E_HIP with the
    call and group named, nothing after the fault runs, and the stream stays
    usable once the variable is gone."""
    n, r = 4, 1
    shapes = [(64, 8), (17,)]
    g = ShardedGroup(shapes, n, r)
    h = ShardedGroup(shapes, n, r)
    _fill_masters(g, ("fault", 0))
    _fill_masters(h, ("fault", 1))
    ag = torch.full((n * g.S,), 7, dtype=torch.int16, device=DEV)
    agh = torch.full((n * h.S,), 7, dtype=torch.int16, device=DEV)
    rs = torch.zeros(n * g.S, dtype=torch.int16, device=DEV)
    before = [g.master_flat.clone(), h.master_flat.clone()]
    monkeypatch.setenv("FSDP_FAULT", "launch")
    for call in (lambda: g.pack(ag[r * g.S:(r + 1) * g.S]), lambda: g.unpack(ag),
                 lambda: g.step(rs, ag[r * g.S:(r + 1) * g.S], 1, **HP)):
        with pytest.raises(capi.FsdpError) as ei:
            call()
        assert ei.value.status == capi.FSDP_E_HIP and "injected" in str(ei.value)
    torch.cuda.synchronize()
    assert (ag == 7).all() and torch.equal(before[0], g.master_flat), "a faulted call launched"
    # two groups: the third launch (group 1's fused step) fails; group 0's
    # step and copy-out ran, group 1 is untouched
    monkeypatch.setenv("FSDP_FAULT", "launch@3")
    call = capi.StepGroupsCall([g.plan, h.plan], [rs, rs],
                               [ag[r * g.S:(r + 1) * g.S], agh[r * h.S:(r + 1) * h.S]],
                               [ag, agh], **HP)
    with pytest.raises(capi.FsdpError) as ei:
        call(1)
    assert ei.value.status == capi.FSDP_E_HIP and "group 1" in str(ei.value)
    torch.cuda.synchronize()
    assert not torch.equal(before[0], g.master_flat), "group 0 did not run"
    assert torch.equal(before[1], h.master_flat) and (agh == 7).all(), "group 1 ran"
    monkeypatch.delenv("FSDP_FAULT")
    capi.fsdp_check_stream()
    g.pack(ag[r * g.S:(r + 1) * g.S])
    torch.cuda.synchronize()
    plan = O.plan(shapes, n, r)
    want = O.pack(plan, [f32(g.shard_view(g.master_flat, i)) for i in range(len(shapes))])
    assert np.array_equal(u16(ag).reshape(n, g.S)[r], want)
    g.close()
    h.close()


# ---------------------------------------------------------------------------
# native multi-group executor
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
@pytest.mark.parametrize("n,r", [(6, 5), (64, 0)], ids=["n6", "n64"])
def test_step_groups_equals_per_group_calls(unfused, n, r):
    if n == 6:
        group_shapes = [CASES[1][1], CASES[2][1], [(70001,), (300, 33)]]
    else:
        # 16-byte aligned rows (the wide row kernels) beside misaligned ones
        named = {c[0]: c[1] for c in CASES}
        group_shapes = [named["wide-n64"], named["odd-n64"], [(64 * 300, 24), (8192,)]]
    A, B, rs_bufs, ag_a, ag_b = [], [], [], [], []
    for gi, shapes in enumerate(group_shapes):
        ga, gb = ShardedGroup(shapes, n, r), ShardedGroup(shapes, n, r)
        _fill_masters(ga, ("exec", gi))
        gb.master_flat.copy_(ga.master_flat)
        plan = O.plan(shapes, n, r)
        rs = _rs_input(plan, n, ("exec-rs", gi))
        rs_bufs.append(torch.from_numpy(rs.reshape(-1).view(np.int16)).to(DEV))
        other = torch.from_numpy(_rand_ag(n, plan.S, ("exec-ag", gi)).reshape(-1).view(np.int16)).to(DEV)
        ag_a.append(other.clone())
        ag_b.append(other.clone())
        A.append(ga)
        B.append(gb)
    for t in (1, 2):
        for gi, ga in enumerate(A):
            S = ga.S
            if unfused:
                ga.reduce(rs_bufs[gi])
                ga.adamw(t, **HP)
                ga.pack(ag_a[gi][r * S:(r + 1) * S])
            else:
                ga.step(rs_bufs[gi], ag_a[gi][r * S:(r + 1) * S], t, **HP)
            ga.unpack(ag_a[gi])
        call = capi.StepGroupsCall([g.plan for g in B], rs_bufs,
                                   [ag_b[gi][r * g.S:(r + 1) * g.S] for gi, g in enumerate(B)],
                                   ag_b, flags=capi.FSDP_STEP_UNFUSED if unfused else 0, **HP)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(B))]
        for e in evs:
            e.record()
        if t == 2:                # a null pair leaves the middle group untimed
            evs[2] = evs[3] = None
        call(t, capi.FSDP_KERNEL_UNPACK, evs)
        torch.cuda.synchronize()
        assert all(evs[2 * i].elapsed_time(evs[2 * i + 1]) >= 0 for i in range(len(B))
                   if evs[2 * i] is not None)
        for ga, gb, aa, ab in zip(A, B, ag_a, ag_b):
            assert torch.equal(aa, ab)
            for fl in ("master_flat", "m_flat", "v_flat", "full_flat"):
                x, y = getattr(ga, fl), getattr(gb, fl)
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), fl
            if unfused:
                assert torch.equal(ga.grad_flat, gb.grad_flat)
    for g in A + B:
        g.close()


def _set_groups(kind):
    """(group shapes, N, rank) of the group-set cases: misaligned rows at 6
    ranks, aligned beside misaligned at 64, and 40 small ragged groups."""
    named = {c[0]: c[1] for c in CASES}
    if kind == "n6":
        return [CASES[1][1], CASES[2][1], [(70001,), (300, 33)], [(0, 4)]], 6, 5
    if kind == "n64":
        return [named["wide-n64"], named["odd-n64"], [(64 * 300, 24), (8192,)]], 64, 0
    rng = np.random.default_rng(synth.seed_for("set-many") % (2**32))
    groups = []
    for _ in range(40):
        k = int(rng.integers(1, 4))
        groups.append([(int(rng.integers(0, 300)), int(rng.integers(1, 40))) for _ in range(k)])
    return groups, 8, 3


@pytest.mark.parametrize("fuse", [False, True], ids=["two-launches", "adamw-copy-in"])
@pytest.mark.parametrize("kind", ["n6", "n64", "many"])
def test_group_set_equals_per_group_unfused_step_and_oracle(kind, fuse):
    """fsdp_step_group_set (one AdamW and one copy-in launch over every group,
    or the two fused in one launch) against fsdp_step_groups with
    FSDP_STEP_UNFUSED (per-group launches) over 3 steps, every tensor bit for
    bit, and the first step against the oracle."""
    group_shapes, n, r = _set_groups(kind)
    A, B, rs_bufs, ag_a, ag_b, plans = [], [], [], [], [], []
    for gi, shapes in enumerate(group_shapes):
        ga, gb = ShardedGroup(shapes, n, r), ShardedGroup(shapes, n, r)
        _fill_masters(ga, ("set", kind, gi))
        gb.master_flat.copy_(ga.master_flat)
        plan = O.plan(shapes, n, r)
        plans.append(plan)
        rs_bufs.append(torch.from_numpy(_rs_input(plan, n, ("set-rs", kind, gi)).reshape(-1)
                                        .view(np.int16)).to(DEV))
        other = torch.from_numpy(_rand_ag(n, plan.S, ("set-ag", kind, gi)).reshape(-1)
                                 .view(np.int16)).to(DEV)
        ag_a.append(other.clone())
        ag_b.append(other.clone())
        A.append(ga)
        B.append(gb)
    masters0 = [[f32(g.shard_view(g.master_flat, i)) for i in range(len(g.shapes))] for g in A]
    gset = capi.fsdp_group_set_create([g.plan for g in B])
    seg = [capi.fsdp_group_set_segment(gset, gi) for gi in range(len(B))]
    total = seg[0][1]
    assert [o for o, _ in seg] == list(np.cumsum([0] + [(g.S + 7) // 8 * 8 for g in B])[:-1])
    arena_buf, arena = guarded_i16(total)
    # A's copy-in goes to buffers of its own, so that both copy-outs read the
    # same synthetic all-gather buffers
    in_a = [torch.zeros(g.S, dtype=torch.int16, device=DEV) for g in A]
    call_a = capi.StepGroupsCall([g.plan for g in A], rs_bufs, in_a, ag_a,
                                 flags=capi.FSDP_STEP_UNFUSED, **HP)
    call_b = capi.StepGroupSetCall(gset, [g.plan for g in B], rs_bufs, arena, ag_b,
                                   flags=capi.FSDP_SET_ADAMW_COPY_IN if fuse else 0, **HP)
    gap = torch.ones(total, dtype=torch.bool, device=DEV)
    for (o, _), g in zip(seg, B):
        gap[o:o + g.S] = False
    for t in (1, 2, 3):
        call_a(t)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(B))]
        for e in evs:
            e.record()
        kinds = ([capi.FSDP_KERNEL_REDUCE, capi.FSDP_KERNEL_ADAMW_PACK, capi.FSDP_KERNEL_UNPACK]
                 if fuse else
                 [capi.FSDP_KERNEL_REDUCE, capi.FSDP_KERNEL_ADAMW, capi.FSDP_KERNEL_PACK])
        call_b(t, kinds[t - 1], evs)
        torch.cuda.synchronize()
        assert evs[0].elapsed_time(evs[1]) >= 0
        for gi, (ga, gb) in enumerate(zip(A, B)):
            o = seg[gi][0]
            assert torch.equal(arena[o:o + gb.S], in_a[gi]), ("segment", gi, t)
            for fl in ("master_flat", "grad_flat", "m_flat", "v_flat", "full_flat"):
                x, y = getattr(ga, fl), getattr(gb, fl)
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (fl, gi, t)
        assert bool((arena[gap] == GUARD_VAL).all()), "a gap was written"
        assert_guards(arena_buf, total)
        if t == 1:               # the set's own results against the oracle
            for gi, (gb, plan) in enumerate(zip(B, plans)):
                rs = u16(rs_bufs[gi]).reshape(n, plan.S)
                grads = O.reduce(plan, rs)
                masters = [x.copy() for x in masters0[gi]]
                ms = [np.zeros_like(x) for x in masters]
                vs = [np.zeros_like(x) for x in masters]
                for x, gr, m, v in zip(masters, grads, ms, vs):
                    O.adamw(x, gr, m, v, 1, **HP)
                for i in range(len(gb.shapes)):
                    _cmp_f32(f32(gb.shard_view(gb.grad_flat, i)), grads[i], ("grad", gi, i))
                    _cmp_f32(f32(gb.shard_view(gb.master_flat, i)), masters[i], ("master", gi, i))
                o = seg[gi][0]
                assert np.array_equal(u16(arena[o:o + plan.S]), O.pack(plan, masters))
                full_in = u16(ag_b[gi]).reshape(n, plan.S)
                for i, want in enumerate(O.unpack(plan, full_in)):
                    assert np.array_equal(u16(gb.full_view(i)), want), ("full", gi, i)
    if fuse:
        capi.fsdp_adamw_pack_groups(gset, arena, step=4, **HP)
    else:
        capi.fsdp_adamw_groups(gset, step=4, **HP)
        capi.fsdp_pack_allgather_groups(gset, arena)
    for gi, ga in enumerate(A):
        ga.adamw(4, **HP)
        ga.pack(in_a[gi])
    torch.cuda.synchronize()
    for gi, (ga, gb) in enumerate(zip(A, B)):
        assert torch.equal(ga.master_flat, gb.master_flat)
        o = seg[gi][0]
        assert torch.equal(arena[o:o + gb.S], in_a[gi])
    capi.fsdp_group_set_destroy(gset)
    for g in A + B:
        g.close()


@pytest.mark.parametrize("kind", ["n6", "n64", "many"])
def test_group_set_fp8_equals_per_group_and_oracle(kind):
    """fsdp_amax_groups and fsdp_pack_allgather_fp8_groups (one launch each
    over every group) against the per-group calls, bit for bit, and against
    the oracle; special values (NaN, infinities, huge and subnormal masters)
    in the first group, an FP8 arena at an odd byte offset."""
    group_shapes, n, r = _set_groups(kind)
    groups, plans, masters = [], [], []
    rng = np.random.default_rng(synth.seed_for("set-fp8", kind) % (2**32))
    for gi, shapes in enumerate(group_shapes):
        g = ShardedGroup(shapes, n, r)
        _fill_masters(g, ("set-fp8", kind, gi))
        if gi == 0:
            for i, e in enumerate(g.entries):
                if e.valid_numel >= len(_F32_SPECIALS) and i % 2 == 0:
                    x = f32(g.shard_view(g.master_flat, i))
                    pos = rng.choice(x.size, size=len(_F32_SPECIALS), replace=False)
                    x[pos] = np.array(_F32_SPECIALS, dtype=np.float32)
                    g.shard_view(g.master_flat, i).copy_(torch.from_numpy(x))
        groups.append(g)
        plans.append(O.plan(shapes, n, r))
        masters.append([f32(g.shard_view(g.master_flat, i)) for i in range(len(shapes))])
    gset = capi.fsdp_group_set_create([g.plan for g in groups])
    n_groups, n_params, total = capi.fsdp_group_set_sizes(gset)
    assert n_groups == len(groups) and n_params == sum(len(s) for s in group_shapes)
    amax = torch.full((max(1, n_params),), -1.0, dtype=torch.float32, device=DEV)
    capi.fsdp_amax_groups(gset, amax)
    per = []
    for g in groups:
        a = torch.full((max(1, len(g.shapes)),), -1.0, dtype=torch.float32, device=DEV)
        g.amax(a)
        per.append(a[:len(g.shapes)])
    torch.cuda.synchronize()
    per_cat = torch.cat(per) if n_params else amax[:0]
    assert torch.equal(amax[:n_params].view(torch.int32), per_cat.view(torch.int32))
    want_amax = np.concatenate([O.amax(ms) for ms in masters])
    _same_f32_nan_ok(f32(amax[:n_params]), want_amax, "amax")
    a_h = want_amax.astype(np.float64)
    scales_h = np.where(np.isfinite(a_h) & (a_h > 0), 448.0 / np.where(a_h > 0, a_h, 1.0),
                        1.0).astype(np.float32)
    scales = torch.from_numpy(scales_h).to(DEV) if n_params else torch.ones(1, device=DEV)
    buf = torch.full((total + 16,), 0x5A, dtype=torch.uint8, device=DEV)
    arena = buf[3:3 + total]
    capi.fsdp_pack_allgather_fp8_groups(gset, arena, scales)
    k = 0
    for gi, (g, plan) in enumerate(zip(groups, plans)):
        seg = torch.zeros(max(1, g.S), dtype=torch.uint8, device=DEV)
        np_g = len(g.shapes)
        g.pack_fp8(seg[:g.S], scales[k:k + np_g] if np_g else scales)
        torch.cuda.synchronize()
        o = capi.fsdp_group_set_segment(gset, gi)[0]
        assert torch.equal(arena[o:o + g.S], seg[:g.S]), ("segment", gi)
        want = O.pack_fp8(plan, masters[gi], [float(x) for x in scales_h[k:k + np_g]])
        assert np.array_equal(arena[o:o + g.S].cpu().numpy(), want), ("oracle", gi)
        k += np_g
    h = buf.cpu().numpy()
    assert (h[:3] == 0x5A).all() and (h[3 + total:] == 0x5A).all()
    capi.fsdp_group_set_destroy(gset)
    for g in groups:
        g.close()


def test_group_set_refuses_rebound_groups_and_overlapping_shards():
    n, r = 4, 1
    g1 = ShardedGroup([(64, 8), (9,)], n, r)
    g2 = ShardedGroup([(33, 3)], n, r)
    gset = capi.fsdp_group_set_create([g1.plan, g2.plan])
    capi.fsdp_adamw_groups(gset, step=1, **HP)
    spare = torch.zeros_like(g2.master_flat)
    capi.fsdp_bind(g2.plan, master=g2._ptrs(spare))
    with pytest.raises(capi.FsdpError) as ei:
        capi.fsdp_adamw_groups(gset, step=2, **HP)
    assert ei.value.status == capi.FSDP_E_STATE
    capi.fsdp_bind(g2.plan, master=g2._ptrs(g2.master_flat))
    capi.fsdp_adamw_groups(gset, step=2, **HP)
    # an arena over a shard tensor of the set is refused before any launch
    before = g1.master_flat.clone()
    for call in (lambda a: capi.fsdp_pack_allgather_groups(gset, a),
                 lambda a: capi.fsdp_adamw_pack_groups(gset, a, step=3, **HP)):
        with pytest.raises(capi.FsdpError) as ei:
            call(g1.master_flat.data_ptr() + 8)
        assert ei.value.status == capi.FSDP_E_INVAL and "overlaps" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.equal(before, g1.master_flat)
    capi.fsdp_group_set_destroy(gset)
    # g3's m shards are g1's master: one launch would race on them
    g3 = ShardedGroup([(64, 8), (9,)], n, r)
    capi.fsdp_bind(g3.plan, exp_avg=g1._ptrs(g1.master_flat))
    with pytest.raises(capi.FsdpError) as ei:
        capi.fsdp_group_set_create([g1.plan, g3.plan])
    assert ei.value.status == capi.FSDP_E_INVAL and "overlap" in str(ei.value)
    for g in (g1, g2, g3):
        g.close()


@pytest.mark.parametrize("path", ["fused", "unfused", "set"])
def test_step_captured_in_a_graph_replays_like_eager_calls(path):
    """Hot calls only enqueue kernels (no allocation, no synchronization, no
    memset), so a whole multi-group step can be captured in a HIP graph.
    Three replays, with eager work and synchronizations between them, match
    three eager calls of the same step on a twin state, bit for bit, every
    replay."""
    n, r = 6, 5
    group_shapes = [CASES[1][1], [(70001,), (300, 33)], [(64, 8)]]
    A, B, rs_bufs, ag_a, ag_b = [], [], [], [], []
    for gi, shapes in enumerate(group_shapes):
        ga, gb = ShardedGroup(shapes, n, r), ShardedGroup(shapes, n, r)
        _fill_masters(ga, ("graph", gi))
        gb.master_flat.copy_(ga.master_flat)
        plan = O.plan(shapes, n, r)
        rs_bufs.append(torch.from_numpy(_rs_input(plan, n, ("graph-rs", gi)).reshape(-1)
                                        .view(np.int16)).to(DEV))
        other = torch.from_numpy(_rand_ag(n, plan.S, ("graph-ag", gi)).reshape(-1)
                                 .view(np.int16)).to(DEV)
        ag_a.append(other.clone())
        ag_b.append(other.clone())
        A.append(ga)
        B.append(gb)

    def make(groups, ags, stream):
        if path == "set":
            gset = capi.fsdp_group_set_create([g.plan for g in groups])
            arena = torch.zeros(capi.fsdp_group_set_info(gset)[1], dtype=torch.int16, device=DEV)
            call = capi.StepGroupSetCall(gset, [g.plan for g in groups], rs_bufs, arena, ags,
                                         flags=capi.FSDP_SET_ADAMW_COPY_IN, stream=stream, **HP)
            return call, (gset, arena)
        ins = [a[r * g.S:(r + 1) * g.S] for a, g in zip(ags, groups)]
        flags = capi.FSDP_STEP_UNFUSED if path == "unfused" else capi.FSDP_STEP_WRITE_GRAD
        return capi.StepGroupsCall([g.plan for g in groups], rs_bufs, ins, ags, flags=flags,
                                   stream=stream, **HP), None

    eager, keep_a = make(A, ag_a, torch.cuda.current_stream())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        captured, keep_b = make(B, ag_b, side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            captured(1)                 # the step index is baked into the graph
    torch.cuda.synchronize()
    for k in range(3):
        eager(1)
        graph.replay()
        torch.cuda.synchronize()
        for gi, (ga, gb) in enumerate(zip(A, B)):
            for fl in ("master_flat", "grad_flat", "m_flat", "v_flat", "full_flat"):
                x, y = getattr(ga, fl), getattr(gb, fl)
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (path, k, gi, fl)
            assert torch.equal(ag_a[gi], ag_b[gi]), (path, k, gi)
        if keep_a is not None:
            assert torch.equal(keep_a[1], keep_b[1]), (path, k, "arena")
        for x in (ag_a, ag_b):          # eager work between replays
            x[0].add_(0)
    for keep in (keep_a, keep_b):
        if keep is not None:
            capi.fsdp_group_set_destroy(keep[0])
    del graph
    for g in A + B:
        g.close()


def test_rejected_bind_keeps_the_previous_binding():
    """A bind that fails argument checks changes nothing: the plan stays bound
    to its previous tensors and the hot calls still produce the oracle's
    results."""
    shapes, n, r = [(33, 5), (17,)], 4, 1
    g = ShardedGroup(shapes, n, r)
    _fill_masters(g, ("rebind",))
    plan = O.plan(shapes, n, r)
    bad = [x + 2 if x else 0 for x in g._ptrs(g.master_flat)]      # not 4-byte aligned
    with pytest.raises(capi.FsdpError) as ei:
        capi.fsdp_bind(g.plan, master=bad)
    assert ei.value.status == capi.FSDP_E_ALIGN
    ag = torch.zeros(plan.S, dtype=torch.int16, device=DEV)
    g.pack(ag)
    torch.cuda.synchronize()
    want = O.pack(plan, [f32(g.shard_view(g.master_flat, i)) for i in range(len(shapes))])
    assert np.array_equal(u16(ag), want)
    # the reshard plan: a rejected rebind keeps the previous copy table
    rows, cols = [10, 7], [3, 1]
    rp = capi.fsdp_reshard_plan_create(rows, cols, 2, 1, 0)
    src = torch.arange(37, dtype=torch.int32, device=DEV)
    dst = torch.full((37,), -1, dtype=torch.int32, device=DEV)
    s_ptrs = [src.data_ptr(), src[15:].data_ptr(), src[30:].data_ptr(), src[34:].data_ptr()]
    d_ptrs = [dst.data_ptr(), dst[30:].data_ptr()]
    capi.fsdp_reshard_bind(rp, s_ptrs, d_ptrs, 4, None)
    with pytest.raises(capi.FsdpError) as ei:
        capi.fsdp_reshard_bind(rp, s_ptrs, d_ptrs, 3, None)
    assert ei.value.status == capi.FSDP_E_UNSUPPORTED
    capi.fsdp_reshard_execute(rp)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    capi.fsdp_reshard_plan_destroy(rp)
    g.close()


def test_step_groups_checks_every_group_before_launching():
    n, r = 4, 0
    g1 = ShardedGroup([(64, 8)], n, r)
    g2 = ShardedGroup([(32,)], n, r, bind=False)     # not bound
    _fill_masters(g1, ("chk",))
    before = g1.master_flat.clone()
    rs = [torch.zeros(n * g.S, dtype=torch.int16, device=DEV) for g in (g1, g2)]
    ag = [torch.zeros(n * g.S, dtype=torch.int16, device=DEV) for g in (g1, g2)]
    call = capi.StepGroupsCall([g1.plan, g2.plan], rs, [a[:g.S] for a, g in zip(ag, (g1, g2))], ag, **HP)
    with pytest.raises(capi.FsdpError) as ei:
        call(1)
    assert ei.value.status == capi.FSDP_E_STATE
    torch.cuda.synchronize()
    assert torch.equal(before, g1.master_flat), "a group ran although a later one was invalid"
    call1 = capi.StepGroupsCall([g1.plan], rs[:1], [ag[0][:g1.S]], None, **HP)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in evs:
        e.record()
    with pytest.raises(capi.FsdpError) as ei:      # copy-out not run without ag_out
        call1(1, capi.FSDP_KERNEL_UNPACK, evs)
    assert ei.value.status == capi.FSDP_E_INVAL
    with pytest.raises(capi.FsdpError) as ei:      # reduce is not a kernel of the fused path
        call1(1, capi.FSDP_KERNEL_REDUCE, evs)
    assert ei.value.status == capi.FSDP_E_INVAL
    with pytest.raises(capi.FsdpError) as ei:      # half a pair
        call1(1, capi.FSDP_KERNEL_STEP, [evs[0], None])
    assert ei.value.status == capi.FSDP_E_INVAL
    torch.cuda.synchronize()
    assert torch.equal(before, g1.master_flat), "a rejected call launched something"
    g1.close()
    g2.close()


# ---------------------------------------------------------------------------
# reduce-scatter copy-in and fp32 contributions
# ---------------------------------------------------------------------------

def _fill_full_grads(g, key):
    for i in range(len(g.shapes)):
        n = g.rows[i] * g.cols[i]
        if n:
            g.full_grad_view(i).view(-1).copy_(synth.normal_bf16_bits(n, 1e-3, key + (i,)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("align", [1, 8])
@pytest.mark.parametrize("case", range(len(CASES)), ids=_case_ids())
def test_pack_reduce_scatter_bit_exact(case, align, dtype):
    name, shapes, n = CASES[case]
    r = n - 1
    plan = O.plan(shapes, n, r, align)
    g = ShardedGroup(shapes, n, r, align)
    g.bind_full_grad()
    _fill_full_grads(g, ("rsp", name))
    grads = [u16(g.full_grad_view(i)) for i in range(len(shapes))]
    if dtype == "bf16":
        want = O.pack_reduce_scatter(plan, grads).reshape(-1)
        for off in (0, 1, 3):
            buf, out = guarded_i16(n * plan.S + off)
            out = out[off:]
            g.pack_reduce_scatter(out, capi.FSDP_DTYPE_BF16)
            torch.cuda.synchronize()
            assert np.array_equal(u16(out), want), (name, off)
            h = u16(buf)
            assert (h[:GUARD + off] == GUARD_VAL).all() and (h[GUARD + off + n * plan.S:] == GUARD_VAL).all()
    else:
        want = O.pack_reduce_scatter_f32(plan, grads).reshape(-1)
        for off in (0, 1, 2, 3):
            buf = torch.full((n * plan.S + off + 2 * GUARD,), 7.5, dtype=torch.float32, device=DEV)
            out = buf[GUARD + off:GUARD + off + n * plan.S]
            g.pack_reduce_scatter(out, capi.FSDP_DTYPE_F32)
            torch.cuda.synchronize()
            assert np.array_equal(f32(out).view(np.uint32), want.view(np.uint32)), (name, off)
            h = f32(buf)
            assert (h[:GUARD + off] == 7.5).all() and (h[GUARD + off + n * plan.S:] == 7.5).all()
    g.close()


@pytest.mark.parametrize("align", [1, 8])
def test_pack_reduce_scatter_misaligned_full_grads_and_roundtrip(align):
    shapes, n = [(37, 11), (999,), (8, 64), (1, 5)], 5
    plan = O.plan(shapes, n, 2, align)
    for shift in range(8):
        g = ShardedGroup(shapes, n, 2, align)
        arena = torch.zeros(sum(r * c + 9 for r, c in zip(g.rows, g.cols)) + 16, dtype=torch.int16, device=DEV)
        views, o = [], shift
        for i, (r_, c_) in enumerate(zip(g.rows, g.cols)):
            v = arena[o:o + r_ * c_]
            v.copy_(synth.normal_bf16_bits(r_ * c_, 1e-3, ("rspm", shift, i)))
            views.append(v)
            o += r_ * c_ + 1
        capi.fsdp_bind_full_grad(g.plan, [v.data_ptr() for v in views], None)
        out = torch.zeros(n * plan.S, dtype=torch.int16, device=DEV)
        g.pack_reduce_scatter(out)
        torch.cuda.synchronize()
        want = O.pack_reduce_scatter(plan, [u16(v) for v in views])
        assert np.array_equal(u16(out).reshape(n, plan.S), want), shift
        # the reduce-scatter input has the all-gather layout: copy-out restores it
        g.unpack(out)
        torch.cuda.synchronize()
        for i, v in enumerate(views):
            assert torch.equal(g.full_view(i).reshape(-1), v)
        g.close()


@pytest.mark.parametrize("case", range(len(CASES)), ids=_case_ids())
def test_reduce_f32_matches_oracle(case):
    name, shapes, n = CASES[case]
    for r in sorted({0, n - 1}):
        plan = O.plan(shapes, n, r)
        rng = np.random.default_rng(synth.seed_for("r32", name, r) % (2**32))
        rs = (rng.standard_normal((n, plan.S)) * 1e-3).astype(np.float32)
        rs[:, _pad_mask(plan)] = np.float32("nan")
        g = ShardedGroup(shapes, n, r)
        for off in (0, 1, 2, 3):
            buf = torch.zeros(n * plan.S + 4, dtype=torch.float32, device=DEV)
            buf[off:off + n * plan.S].copy_(torch.from_numpy(rs.reshape(-1)))
            g.grad_flat.fill_(-7.0)
            g.reduce_f32(buf[off:off + n * plan.S])
            torch.cuda.synchronize()
            for i, want in enumerate(O.reduce_f32(plan, rs)):
                _cmp_f32(f32(g.shard_view(g.grad_flat, i)), want, (name, r, i, off))
        g.close()


@pytest.mark.parametrize("n", [2, 6, 8, 64])
def test_reduce_f32_of_widened_copy_in_equals_bf16_reduce(n):
    """reduce_f32(pack_rs_f32(G)) == reduce(pack_rs_bf16(G)), every element."""
    shapes = [(n * 40 + 3, 67), (2 * n + 1,), (3 * n - 1, 9)]
    r = n // 2
    g = ShardedGroup(shapes, n, r)
    g.bind_full_grad()
    _fill_full_grads(g, ("wid", n))
    b = torch.zeros(n * g.S, dtype=torch.int16, device=DEV)
    f = torch.zeros(n * g.S, dtype=torch.float32, device=DEV)
    g.pack_reduce_scatter(b, capi.FSDP_DTYPE_BF16)
    g.pack_reduce_scatter(f, capi.FSDP_DTYPE_F32)
    g.reduce(b)
    torch.cuda.synchronize()
    ref = g.grad_flat.clone()
    g.grad_flat.zero_()
    g.reduce_f32(f)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int32), g.grad_flat.view(torch.int32))
    g.close()


# ---------------------------------------------------------------------------
# resharding to another world size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("elem", [2, 4], ids=["bf16", "fp32"])
@pytest.mark.parametrize("n1,n2", [(2, 1), (1, 3), (8, 64), (64, 8), (6, 4), (3, 5)])
def test_reshard_execute_matches_oracle(n1, n2, elem):
    shapes = [(37, 3), (1, 5), (0, 4), (1031,), (200, 67), (64, 7)]
    rows = [s[0] for s in shapes]
    cols = [int(np.prod(s[1:])) if len(s) > 1 else 1 for s in shapes]
    dt = torch.int16 if elem == 2 else torch.int32
    rng = np.random.default_rng(n1 * 100 + n2)
    fulls = [rng.integers(-2**15, 2**15 - 1 if elem == 2 else 2**15, size=r * c).astype(
        np.int16 if elem == 2 else np.int32) for r, c in zip(rows, cols)]
    for shift in (0, 1):
        # source shards, each at its own (possibly misaligned) offset in one buffer
        total = sum(f.size for f in fulls) + 64 * len(fulls) * n1
        src_buf = torch.zeros(total, dtype=dt, device=DEV)
        src_ptrs, o = [], shift
        for f, r, c in zip(fulls, rows, cols):
            for s in range(n1):
                b, lr = O.rows_of_rank(r, n1, s)
                piece = f[b * c:(b + lr) * c]
                src_buf[o:o + piece.size].copy_(torch.from_numpy(piece))
                src_ptrs.append(src_buf[o:].data_ptr() if piece.size else 0)
                o += piece.size + 3
        for d in sorted({0, n2 - 1, n2 // 2}):
            p = capi.fsdp_reshard_plan_create(rows, cols, n1, n2, d)
            dst_buf = torch.full((sum(f.size for f in fulls) + 64 * len(fulls),), -5, dtype=dt, device=DEV)
            dst_views, o = [], shift
            for r, c in zip(rows, cols):
                k = O.rows_of_rank(r, n2, d)[1] * c
                dst_views.append(dst_buf[o:o + k])
                o += k + 5
            capi.fsdp_reshard_bind(p, src_ptrs, [v.data_ptr() if v.numel() else 0 for v in dst_views],
                                   elem, None)
            capi.fsdp_reshard_execute(p)
            torch.cuda.synchronize()
            for f, r, c, v in zip(fulls, rows, cols, dst_views):
                src = [f[O.rows_of_rank(r, n1, s)[0] * c:(O.rows_of_rank(r, n1, s)[0] + O.rows_of_rank(r, n1, s)[1]) * c]
                       for s in range(n1)]
                want = O.reshard(src, r, c, n2, d)
                assert np.array_equal(v.cpu().numpy(), want), (n1, n2, d, r, shift)
            # nothing outside the target views was touched
            h = dst_buf.cpu().numpy()
            mask = np.ones(h.size, bool)
            o = shift
            for v in dst_views:
                mask[o:o + v.numel()] = False
                o += v.numel() + 5
            assert (h[mask] == -5).all()
            capi.fsdp_reshard_plan_destroy(p)


# ---------------------------------------------------------------------------
# gradient accumulation without sync
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", range(len(CASES)), ids=_case_ids())
def test_accumulate_then_copy_in_matches_oracle(case):
    name, shapes, n = CASES[case]
    r = n - 1
    plan = O.plan(shapes, n, r)
    g = ShardedGroup(shapes, n, r)
    g.bind_full_grad()
    g.bind_grad_acc()
    g.grad_acc_flat.fill_(123.0)           # reset must overwrite whatever is there
    acc = None
    for k in range(3):
        _fill_full_grads(g, ("accg", name, k))
        grads = [u16(g.full_grad_view(i)) for i in range(len(shapes))]
        g.accumulate_grad(reset=(k == 0))
        acc = O.accumulate_grad(acc, grads, reset=(k == 0))
    torch.cuda.synchronize()
    for i, want in enumerate(acc):
        got = f32(g.grad_acc_view(i)).reshape(-1)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (name, i)
    want_rs = O.pack_reduce_scatter_acc(plan, acc).reshape(-1)
    for off in (0, 1, 3):
        buf = torch.full((n * plan.S + off + 8,), 9.0, dtype=torch.float32, device=DEV)
        g.pack_reduce_scatter_acc(buf[off:off + n * plan.S])
        torch.cuda.synchronize()
        h = f32(buf)
        assert np.array_equal(h[off:off + n * plan.S].view(np.uint32), want_rs.view(np.uint32))
        assert (h[:off] == 9.0).all() and (h[off + n * plan.S:] == 9.0).all()
    # the synchronizing microbatch: fp32 reduction of the accumulated copy-in
    rs = torch.from_numpy(want_rs).to(DEV)
    g.reduce_f32(rs)
    torch.cuda.synchronize()
    for i, want in enumerate(O.reduce_f32(plan, want_rs.reshape(n, plan.S))):
        _cmp_f32(f32(g.shard_view(g.grad_flat, i)), want, (name, i))
    g.close()


@pytest.mark.parametrize("n,align", [(6, 1), (8, 8), (64, 8)])
def test_accumulate_and_reduce_f32_special_values(n, align):
    """Infinities, NaNs, overflow and subnormals through the fp32
    accumulation (3 microbatches), its copy-in and the fp32 reduction: bit
    for bit with the oracle, NaNs created by an operation matched as NaNs."""
    shapes = [(37, 5), (130, 3), (1024, 16)]
    r = n // 2
    plan = O.plan(shapes, n, r, align)
    g = ShardedGroup(shapes, n, r, align)
    g.bind_full_grad()
    g.bind_grad_acc()
    rng = np.random.default_rng(8000 + n)
    acc = None
    for k in range(3):
        grads = []
        for i in range(len(shapes)):
            v = g.full_grad_view(i).view(-1)
            x = synth.bf16_bits_to_u16(synth.normal_bf16_bits(v.numel(), 1e-3, ("accs", n, k, i)))
            hit = rng.random(x.size) < 0.1
            x[hit] = rng.choice(np.array(_BF16_SPECIALS, dtype=np.uint16), size=int(hit.sum()))
            x[:4] = [0x0001, 0x807F, 0x7F7F, 0x7F7F]     # subnormals; a sum that overflows
            v.copy_(torch.from_numpy(x.view(np.int16)))
            grads.append(x)
        g.accumulate_grad(reset=(k == 0))
        with np.errstate(all="ignore"):
            acc = O.accumulate_grad(acc, grads, reset=(k == 0))
    torch.cuda.synchronize()
    for i, want in enumerate(acc):
        _same_f32_nan_ok(f32(g.grad_acc_view(i)).reshape(-1), want, ("acc", n, i))
    want_rs = O.pack_reduce_scatter_acc(plan, acc)
    rs = torch.zeros(n * plan.S, dtype=torch.float32, device=DEV)
    g.pack_reduce_scatter_acc(rs)
    torch.cuda.synchronize()
    _same_f32_nan_ok(f32(rs), want_rs.reshape(-1), ("rs", n))
    # the fp32 reduction of contributions holding every special value
    rsf = want_rs.copy()
    valid = ~_pad_mask(plan)
    specials = np.array([np.inf, -np.inf, np.nan, 3e38, -3e38, 1e-45, -1e-40, -0.0], np.float32)
    hit = (rng.random(rsf.shape) < 0.2) & valid[None, :]
    rsf[hit] = rng.choice(specials, size=int(hit.sum()))
    rsf[:, ~valid] = np.float32("nan")                  # padding is never read
    g.reduce_f32(torch.from_numpy(rsf.reshape(-1)).to(DEV))
    torch.cuda.synchronize()
    with np.errstate(all="ignore"):
        want_g = O.reduce_f32(plan, rsf)
    for i, want in enumerate(want_g):
        _same_f32_nan_ok(f32(g.shard_view(g.grad_flat, i)), want, ("g32", n, i))
    g.close()


def test_accumulate_misaligned_pointers_take_the_scalar_path():
    shapes = [(37, 11), (999,), (8, 64)]
    g = ShardedGroup(shapes, 2, 0, bind=True)
    gbuf = torch.zeros(sum(r * c + 5 for r, c in zip(g.rows, g.cols)) + 16, dtype=torch.int16, device=DEV)
    abuf = torch.zeros(sum(r * c + 5 for r, c in zip(g.rows, g.cols)) + 16, dtype=torch.float32, device=DEV)
    gv, av, og, oa = [], [], 1, 2
    for i, (r_, c_) in enumerate(zip(g.rows, g.cols)):
        gv.append(gbuf[og:og + r_ * c_])
        av.append(abuf[oa:oa + r_ * c_])
        og += r_ * c_ + 3
        oa += r_ * c_ + 1
    capi.fsdp_bind_full_grad(g.plan, [v.data_ptr() for v in gv], None)
    capi.fsdp_bind_grad_acc(g.plan, [v.data_ptr() for v in av], None)
    acc = None
    for k in range(2):
        for i, v in enumerate(gv):
            v.copy_(synth.normal_bf16_bits(v.numel(), 1e-3, ("accm", k, i)))
        capi.fsdp_accumulate_grad(g.plan, k == 0)
        acc = O.accumulate_grad(acc, [u16(v) for v in gv], reset=(k == 0))
    torch.cuda.synchronize()
    for v, want in zip(av, acc):
        assert np.array_equal(f32(v).view(np.uint32), want.view(np.uint32))
    g.close()


# ---------------------------------------------------------------------------
# FP8 E4M3 all-gather
# ---------------------------------------------------------------------------

def u8(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint8)


@pytest.mark.parametrize("case", range(len(CASES)), ids=_case_ids())
def test_pack_fp8_bit_exact(case):
    name, shapes, n = CASES[case]
    specials = np.array([0x7FC00000, 0xFFC00000, 0x7F800000, 0xFF800000, 0x43E80000, 0x3A800000,
                         0x3AC00000, 0x3F880000, 0x3F980000, 0x80000000, 0x00000001],
                        dtype=np.uint32).view(np.float32)
    for r in sorted({0, n - 1}):
        plan = O.plan(shapes, n, r)
        g = ShardedGroup(shapes, n, r)
        _fill_masters(g, ("fp8", name, r))
        for i, e in enumerate(g.entries):
            k = min(e.valid_numel, len(specials))
            if k:
                g.shard_view(g.master_flat, i)[:k].copy_(torch.from_numpy(specials[:k] / np.float32(20.0)))
        masters = [f32(g.shard_view(g.master_flat, i)) for i in range(len(shapes))]
        scales_h = np.array([20.0 + i for i in range(len(shapes))], dtype=np.float32)
        scales = torch.from_numpy(scales_h).to(DEV)
        want = O.pack_fp8(plan, masters, scales_h)
        for off in (0, 1, 5, 13):
            buf = torch.full((plan.S + off + 64,), 0xA5, dtype=torch.uint8, device=DEV)
            g.pack_fp8(buf[off:off + plan.S], scales)
            torch.cuda.synchronize()
            h = u8(buf)
            assert np.array_equal(h[off:off + plan.S], want), (name, r, off)
            assert (h[:off] == 0xA5).all() and (h[off + plan.S:] == 0xA5).all()
        g.close()


def test_pack_bf16_every_rounding_boundary():
    """The bf16 copy-in on every fp32 upper half (every kept pattern, so every
    exponent, both parities of the last kept bit, infinities and NaN
    payloads) times low halves 0, 1, 0x7FFF, 0x8000 (the tie), 0x8001 and
    0xFFFF: equal to the oracle bit for bit."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lo = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    x = (hi[:, None] | lo[None, :]).reshape(-1).view(np.float32)
    plan = O.plan([(x.size,)], 1, 0)
    g = ShardedGroup([(x.size,)], 1, 0)
    g.shard_view(g.master_flat, 0).copy_(torch.from_numpy(x))
    out = torch.zeros(plan.S, dtype=torch.int16, device=DEV)
    g.pack(out)
    torch.cuda.synchronize()
    want = O.pack(plan, [x])
    got = u16(out)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(hex(int(x.view(np.uint32)[i])), hex(int(got[i])), hex(int(want[i])))
                           for i in bad[:8]]
    g.close()


def test_pack_fp8_every_rounding_boundary():
    """The FP8 cast on every fp32 upper half (sign, exponent and the top 7
    mantissa bits: every kept-bit and round-bit combination of the normal and
    subnormal E4M3 ranges, saturation, infinities and NaNs) times low halves
    0, 1, 0x7FFF, 0x8000, 0x8001 and 0xFFFF (sticky bits), scale 1: equal to
    the oracle byte for byte."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lo = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    x = (hi[:, None] | lo[None, :]).reshape(-1).view(np.float32)
    plan = O.plan([(x.size,)], 1, 0)
    g = ShardedGroup([(x.size,)], 1, 0)
    g.shard_view(g.master_flat, 0).copy_(torch.from_numpy(x))
    out = torch.zeros(plan.S, dtype=torch.uint8, device=DEV)
    g.pack_fp8(out, torch.ones(1, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    with np.errstate(all="ignore"):
        want = O.pack_fp8(plan, [x], np.ones(1, np.float32))
    got = u8(out)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(hex(int(x.view(np.uint32)[i])), int(got[i]), int(want[i])) for i in bad[:8]]
    g.close()


@pytest.mark.parametrize("case", range(len(CASES)), ids=_case_ids())
def test_unpack_fp8_bit_exact_misaligned(case):
    name, shapes, n = CASES[case]
    r = 0
    plan = O.plan(shapes, n, r)
    rng = np.random.default_rng(synth.seed_for("u8", name) % (2**32))
    ag = rng.integers(0, 256, size=(n, plan.S), dtype=np.uint8)
    for j in range(n):
        ag[j, _pad_mask(O.plan(shapes, n, j))] = 0x7F
    ref = O.unpack_fp8(plan, ag)
    g = ShardedGroup(shapes, n, r, bind=False)
    for shift in (0, 3, 9):
        arena = torch.full((sum(rr * cc + 7 for rr, cc in zip(g.rows, g.cols)) + 32,), 0x5A,
                           dtype=torch.uint8, device=DEV)
        views, o = [], shift
        for rr, cc in zip(g.rows, g.cols):
            views.append(arena[o:o + rr * cc])
            o += rr * cc + 7
        capi.fsdp_bind_full_fp8(g.plan, [v.data_ptr() if v.numel() else 0 for v in views], None)
        src = torch.zeros(n * plan.S + 32, dtype=torch.uint8, device=DEV)
        src[shift + 1:shift + 1 + n * plan.S].copy_(torch.from_numpy(ag.reshape(-1)))
        g.unpack_fp8(src[shift + 1:shift + 1 + n * plan.S])
        torch.cuda.synchronize()
        h = u8(arena)
        mask = np.ones(h.size, bool)
        o = shift
        for v, want in zip(views, ref):
            assert np.array_equal(u8(v), want.reshape(-1)), (name, shift)
            mask[o:o + v.numel()] = False
            o += v.numel() + 7
        assert (h[mask] == 0x5A).all()
    g.close()


def test_amax_matches_oracle_and_propagates_nan():
    shapes, n = [(1000, 70), (333,), (77, 129), (1, 2048), (1,)], 6
    for r in (0, 5):
        g = ShardedGroup(shapes, n, r)
        _fill_masters(g, ("amax", r))
        out = torch.full((len(shapes),), -1.0, device=DEV)
        g.amax(out)
        torch.cuda.synchronize()
        want = O.amax([f32(g.shard_view(g.master_flat, i)) for i in range(len(shapes))])
        assert np.array_equal(f32(out).view(np.uint32), want.view(np.uint32))
        if g.entries[0].valid_numel:
            g.shard_view(g.master_flat, 0)[5] = float("nan")
            g.amax(out)
            torch.cuda.synchronize()
            assert torch.isnan(out[0]).item()
        g.close()


@pytest.mark.parametrize("cfg_index", [2, 4])
def test_fp8_roundtrip_full_size_block(cfg_index):
    """Every rank's FP8 copy-in, then copy-out, equals torch's saturating cast."""
    cfg = configs.get(cfg_index)
    shapes = [p.shape for p in cfg.groups[0].params]
    n = cfg.world
    Ws = []
    for i, s in enumerate(shapes):
        W = torch.empty(s, dtype=torch.float32, device=DEV)
        synth.fill_normal_f32_(W, 0.02, ("fp8rt", cfg_index, i))
        Ws.append(W)
    scales = torch.stack([448.0 / W.abs().max() for W in Ws]).float()
    g0 = ShardedGroup(shapes, n, 0, bind=False)
    S = g0.S
    ag = torch.empty(n * S, dtype=torch.uint8, device=DEV)
    for j in range(n):
        gj = ShardedGroup(shapes, n, j, bind=False)
        masters = [W.view(-1)[e.row_begin * e.cols:].data_ptr() if e.valid_numel else 0
                   for W, e in zip(Ws, gj.entries)]
        capi.fsdp_bind(gj.plan, master=masters, stream=None)
        gj.pack_fp8(ag[j * S:(j + 1) * S], scales)
        torch.cuda.synchronize()
        gj.close()
    g0.bind_full_fp8()
    g0.unpack_fp8(ag)
    torch.cuda.synchronize()
    for i, W in enumerate(Ws):
        want = (W.reshape(W.shape[0], -1) * scales[i]).clamp(-448, 448).to(torch.float8_e4m3fn)
        assert torch.equal(g0.full_fp8_view(i), want.view(torch.uint8)), i
    g0.close()
