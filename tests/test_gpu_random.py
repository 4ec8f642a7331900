"""GPU parity on seeded random parameter groups: every kernel against the oracle.

Each case draws a ragged group (1-6 parameters, 0-400 rows, 1-70 columns, some
1-D), a world size of 1-13 (16-64 for every fourth case), a rank, the
alignment option and element offsets of the [N, S] buffers and of a group
set's copy-in arena, so layouts the fixed cases do not name (misaligned rows
at every offset, partial row batches, empty chunks, tiny runs) are covered.
Bit-exact bars as in the fixed-case tests.
"""
import numpy as np
import pytest
import torch

from oracle import fsdp as O
from workloads import synth

pytestmark = pytest.mark.gpu

capi = pytest.importorskip("sharded_shard_amd.capi")
from sharded_shard_amd.group import ShardedGroup  # noqa: E402

DEV = "cuda"
HP = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
SEEDS = list(range(16))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _case(seed):
    rng = np.random.default_rng(synth.seed_for("random-group", seed) % (2**32))
    shapes = []
    for _ in range(int(rng.integers(1, 7))):
        rows = int(rng.choice([0, 1, 2, int(rng.integers(3, 401))], p=[0.1, 0.1, 0.1, 0.7]))
        if rng.random() < 0.3:
            shapes.append((rows,))
        else:
            shapes.append((rows, int(rng.integers(1, 71))))
    if seed % 5 == 4:  # an empty parameter somewhere in the group
        shapes.insert(int(rng.integers(0, len(shapes) + 1)), (0, int(rng.integers(1, 71))))
    n = int(rng.integers(1, 14)) if seed % 4 else int(rng.choice([16, 17, 24, 32, 64]))
    r = int(rng.integers(0, n))
    align = int(rng.choice([1, 8]))
    offs = [int(x) for x in rng.integers(0, 8, size=4)]
    if seed % 8 == 0:  # 16-byte aligned rows: the wide row kernels from 16 ranks
        align, offs[0], offs[2] = 8, 0, 0
    return shapes, n, r, align, offs


def _u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _f32(t):
    return t.detach().cpu().contiguous().numpy()


def _bits_equal(got, want, what):
    assert got.shape == want.shape, what
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), what


@pytest.mark.parametrize("seed", SEEDS)
def test_random_group_every_kernel(seed):
    shapes, n, r, align, offs = _case(seed)
    print(f"[random] seed={seed} shapes={shapes} n={n} r={r} align={align} offs={offs}", flush=True)
    plan = O.plan(shapes, n, r, align)
    S = plan.S
    g = ShardedGroup(shapes, n, r, align)
    assert g.S == S and g.V == plan.V and g.F == plan.F
    for i, e in enumerate(g.entries):
        assert (e.shard_offset, e.valid_numel, e.seg_numel) == \
            (plan.entries[i].shard_offset, plan.entries[i].valid_numel, plan.entries[i].seg_numel)
        if e.valid_numel:
            g.shard_view(g.master_flat, i).copy_(synth.normal_f32(e.valid_numel, 0.02, ("rg-m", seed, i)))
    host_p = [_f32(g.shard_view(g.master_flat, i)) for i in range(len(shapes))]
    host_m = [np.zeros_like(x) for x in host_p]
    host_v = [np.zeros_like(x) for x in host_p]

    # fused step, two steps, gradient written: reduce, AdamW and copy-in
    o_rs, o_ag, o_rsf, o_b = offs
    rs_buf = torch.zeros(n * S + 16, dtype=torch.int16, device=DEV)
    ag_buf = torch.zeros(n * S + 16, dtype=torch.int16, device=DEV)
    rs, ag = rs_buf[o_rs:o_rs + n * S], ag_buf[o_ag:o_ag + n * S]
    pad = np.ones(S, bool)
    for e in plan.entries:
        pad[e.shard_offset:e.shard_offset + e.valid_numel] = False
    for t in (1, 2):
        x = np.stack([synth.bf16_bits_to_u16(synth.normal_bf16_bits(S, 1e-3, ("rg-rs", seed, t, j)))
                      for j in range(n)]) if S else np.zeros((n, 0), np.uint16)
        x[:, pad] = synth.SENTINEL_BF16
        rs.copy_(torch.from_numpy(x.reshape(-1).view(np.int16)))
        g.step(rs, ag[r * S:(r + 1) * S], t, write_grad=True, **HP)
        torch.cuda.synchronize()
        grads = O.reduce(plan, x)
        for i in range(len(shapes)):
            _bits_equal(_f32(g.shard_view(g.grad_flat, i)), grads[i], ("grad", seed, i, t))
            O.adamw(host_p[i], grads[i], host_m[i], host_v[i], t, **HP)
        for i in range(len(shapes)):
            _bits_equal(_f32(g.shard_view(g.master_flat, i)), host_p[i], ("master", seed, i, t))
            _bits_equal(_f32(g.shard_view(g.m_flat, i)), host_m[i], ("m", seed, i, t))
            _bits_equal(_f32(g.shard_view(g.v_flat, i)), host_v[i], ("v", seed, i, t))
        assert np.array_equal(_u16(ag[r * S:(r + 1) * S]), O.pack(plan, host_p)), ("pack", seed, t)

    # the optimizer step fused with the copy-in over a group set of this
    # group (gradient: the last step's, still bound), into an arena at an
    # element offset of its own
    gset = capi.fsdp_group_set_create([g.plan])
    total = capi.fsdp_group_set_info(gset)[1]
    arena_buf = torch.full((total + 16,), 0x5A5A, dtype=torch.int16, device=DEV)
    arena = arena_buf[o_b:o_b + total]
    capi.fsdp_adamw_pack_groups(gset, arena, step=3, **HP)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        O.adamw(host_p[i], grads[i], host_m[i], host_v[i], 3, **HP)
        _bits_equal(_f32(g.shard_view(g.master_flat, i)), host_p[i], ("set master", seed, i))
        _bits_equal(_f32(g.shard_view(g.m_flat, i)), host_m[i], ("set m", seed, i))
        _bits_equal(_f32(g.shard_view(g.v_flat, i)), host_v[i], ("set v", seed, i))
    assert np.array_equal(_u16(arena)[:S], O.pack(plan, host_p)), ("set pack", seed)
    assert (_u16(arena_buf)[:o_b] == 0x5A5A).all() and (_u16(arena)[S:] == 0x5A5A).all()
    assert (_u16(arena_buf)[o_b + total:] == 0x5A5A).all()
    capi.fsdp_group_set_destroy(gset)

    # copy-out of a random [N, S] buffer (padding holds sentinels)
    rng = np.random.default_rng(synth.seed_for("rg-ag", seed) % (2**32))
    agh = rng.integers(0, 2**16, size=(n, S), dtype=np.uint16)
    for j in range(n):
        pj = O.plan(shapes, n, j, align)
        m = np.ones(S, bool)
        for e in pj.entries:
            m[e.shard_offset:e.shard_offset + e.valid_numel] = False
        agh[j, m] = synth.SENTINEL_BF16
    ag.copy_(torch.from_numpy(agh.reshape(-1).view(np.int16)))
    g.unpack(ag)
    torch.cuda.synchronize()
    for i, want in enumerate(O.unpack(plan, agh)):
        assert np.array_equal(_u16(g.full_view(i)).reshape(want.shape), want), ("unpack", seed, i)

    # reduce-scatter copy-ins (bf16, widened fp32) and the fp32 reduction
    g.bind_full_grad()
    full = []
    for i in range(len(shapes)):
        k = g.rows[i] * g.cols[i]
        if k:
            g.full_grad_view(i).view(-1).copy_(synth.normal_bf16_bits(k, 1e-3, ("rg-g", seed, i)))
        full.append(_u16(g.full_grad_view(i)).reshape(-1))
    g.pack_reduce_scatter(rs, capi.FSDP_DTYPE_BF16)
    rsf_buf = torch.zeros(n * S + 8, dtype=torch.float32, device=DEV)
    rsf = rsf_buf[o_rsf:o_rsf + n * S]
    g.pack_reduce_scatter(rsf, capi.FSDP_DTYPE_F32)
    torch.cuda.synchronize()
    want_b = O.pack_reduce_scatter(plan, full)
    assert np.array_equal(_u16(rs).reshape(n, S), want_b), ("rs bf16", seed)
    want_f = O.pack_reduce_scatter_f32(plan, full)
    _bits_equal(_f32(rsf).reshape(n, S), want_f, ("rs f32", seed))
    g.reduce_f32(rsf)
    torch.cuda.synchronize()
    for i, want in enumerate(O.reduce_f32(plan, want_f)):
        _bits_equal(_f32(g.shard_view(g.grad_flat, i)), want, ("reduce f32", seed, i))

    # accumulation over two microbatches and its copy-in
    g.bind_grad_acc()
    acc = None
    for k in range(2):
        if k:
            for i in range(len(shapes)):
                kk = g.rows[i] * g.cols[i]
                if kk:
                    g.full_grad_view(i).view(-1).copy_(synth.normal_bf16_bits(kk, 1e-3, ("rg-g2", seed, i)))
        grads = [_u16(g.full_grad_view(i)).reshape(-1) for i in range(len(shapes))]
        g.accumulate_grad(reset=(k == 0))
        acc = O.accumulate_grad(acc, grads, reset=(k == 0))
    g.pack_reduce_scatter_acc(rsf)
    torch.cuda.synchronize()
    for i, want in enumerate(acc):
        _bits_equal(_f32(g.grad_acc_view(i)).reshape(-1), want, ("acc", seed, i))
    _bits_equal(_f32(rsf).reshape(n, S), O.pack_reduce_scatter_acc(plan, acc), ("rs acc", seed))

    # FP8 copy-in with per-parameter scales from the oracle's amax, and copy-out
    masters = [_f32(g.shard_view(g.master_flat, i)) for i in range(len(shapes))]
    amax = torch.empty(len(shapes), dtype=torch.float32, device=DEV)
    g.amax(amax)
    torch.cuda.synchronize()
    want_amax = O.amax(masters)
    _bits_equal(_f32(amax), want_amax, ("amax", seed))
    scales_h = np.array([448.0 / a if a > 0 else 1.0 for a in want_amax], dtype=np.float32)
    fp8_buf = torch.zeros(n * S + 32, dtype=torch.uint8, device=DEV)
    fp8 = fp8_buf[o_b:o_b + n * S]
    g.pack_fp8(fp8[r * S:(r + 1) * S], torch.from_numpy(scales_h).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(fp8[r * S:(r + 1) * S].cpu().numpy(), O.pack_fp8(plan, masters, scales_h)), \
        ("fp8 pack", seed)
    g.bind_full_fp8()
    g.unpack_fp8(fp8)
    torch.cuda.synchronize()
    for i, want in enumerate(O.unpack_fp8(plan, fp8.cpu().numpy().reshape(n, S))):
        got = g.full_fp8_view(i).cpu().numpy().reshape(want.shape)
        assert np.array_equal(got, want), ("fp8 unpack", seed, i)
    g.close()
