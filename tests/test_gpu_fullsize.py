"""Full-size parity on the 7B- and 70B-shaped groups, as the bench launches them.

The groups are planned and bound exactly as bench.py does (ShardedGroup, same
plans, tiles and grids).  Outputs are checked three ways:

* whole groups: the multi-group executor the bench times (fsdp_step_groups,
  fused) runs 3 steps on whole groups of the one-block, ragged MoE and 70B
  shapes, and every element of every output is compared with the oracle run
  on the same inputs read back;
* sampled: the oracle computes chosen outputs one by one from the same inputs
  read back (first and last elements, tile edges, random picks), for the
  separate kernels and the single-group fused call;
* whole workloads through a group set: the separate-kernel path (a reduce per
  group, one AdamW and one copy-in launch over all 33 or 81 groups, or the two
  fused in one launch) equals the fused executor bit for bit in every shard
  and copy-in segment;
* exact properties over every element: unpack of every rank's pack of a full
  weight W gives bf16(W) back bit for bit, with torch's library cast as the
  reference; N equal gradient contributions reduce to exactly that gradient.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _groups(cfg_index):
    cfg = configs.get(cfg_index)
    return cfg, [(0, cfg.groups[0]), (len(cfg.groups) - 1, cfg.groups[-1])]


def _sample_idx(valid, key, k=1536):
    if valid == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng(synth.seed_for(*key) % (2**32))
    edges = []
    for t in (4096, 8192, 16384, 32768):
        m = np.arange(t, valid, t)[:8]
        edges += [m - 1, m, m + 1]
    idx = np.concatenate([np.array([0, 1, 2, 7, 8, valid - 1, valid - 2, valid - 9]),
                          rng.integers(0, valid, size=k)] + edges)
    return np.unique(np.clip(idx, 0, valid - 1))


def _col_plan(world, k):
    """A one-entry oracle plan over k sampled columns (the reduce is columnwise)."""
    e = O.Entry(rows=k, cols=1, chunk_rows=k, row_begin=0, local_rows=k, shard_offset=0,
                shard_numel=k, valid_numel=k, pad_numel=0, seg_numel=k)
    return O.Plan(world=world, rank=0, align=1, entries=[e], S=k)


# 7B and 70B block and root groups (aligned rows), and the ragged MoE
# workload's two groups at rank 5 (odd segments: every row of [N, S] and
# most shard and piece offsets misaligned)
CASES = [(2, "block"), (2, "root"), (3, "block"), (3, "root"), (4, "block"), (4, "root")]


@pytest.mark.parametrize("cfg_index,which", CASES, ids=[f"c{c}-{w}" for c, w in CASES])
def test_roundtrip_pack_unpack_every_element(cfg_index, which):
    cfg, gs = _groups(cfg_index)
    gi, grp = gs[0] if which == "block" else gs[1]
    shapes = [p.shape for p in grp.params]
    n = cfg.world
    print(f"[fullsize] roundtrip cfg={cfg_index} group={gi} n={n}", flush=True)
    Ws = []
    for i, s in enumerate(shapes):
        W = torch.empty(s, dtype=torch.float32, device=DEV)
        synth.fill_normal_f32_(W, 0.02, ("rt-full", cfg_index, gi, i))
        Ws.append(W)
    g0 = ShardedGroup(shapes, n, 0)
    S = g0.S
    ag = torch.empty(n * S, dtype=torch.int16, device=DEV)
    ag.fill_(synth.SENTINEL_BF16)
    for j in range(n):
        gj = ShardedGroup(shapes, n, j, bind=False)
        masters = []
        for W, e in zip(Ws, gj.entries):
            flat = W.view(-1)
            b = e.row_begin * e.cols
            masters.append(flat[b:b + e.valid_numel].data_ptr() if e.valid_numel else 0)
        capi.fsdp_bind(gj.plan, master=masters, stream=None)
        gj.pack(ag[j * S:(j + 1) * S])
        torch.cuda.synchronize()
        gj.close()
    g0.unpack(ag)
    torch.cuda.synchronize()
    for i, W in enumerate(Ws):
        want = W.reshape(W.shape[0], -1).to(torch.bfloat16).view(torch.int16)
        assert torch.equal(g0.full_view(i), want), (cfg_index, gi, i)
        # sampled rows against the oracle's cast
        rows = _sample_idx(W.shape[0], ("rt-rows", cfg_index, gi, i), k=16)
        wr = W.reshape(W.shape[0], -1)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
        got = g0.full_view(i)[torch.from_numpy(rows).to(DEV)].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, O.bf16_rne(wr))
    g0.close()


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("cfg_index,which", CASES, ids=[f"c{c}-{w}" for c, w in CASES])
def test_step_sampled_against_oracle(cfg_index, which, fused):
    cfg, gs = _groups(cfg_index)
    gi, grp = gs[0] if which == "block" else gs[1]
    shapes = [p.shape for p in grp.params]
    n, r = cfg.world, cfg.timing_rank
    hp = vars(cfg.hp)
    print(f"[fullsize] step cfg={cfg_index} group={gi} n={n} r={r} fused={fused}", flush=True)
    g = ShardedGroup(shapes, n, r)
    S = g.S
    for i, e in enumerate(g.entries):
        synth.fill_normal_f32_(g.shard_view(g.master_flat, i), 0.02, ("fs-m", cfg_index, gi, i))
    idxs = [_sample_idx(e.valid_numel, ("fs-idx", cfg_index, gi, i)) for i, e in enumerate(g.entries)]
    tidx = [torch.from_numpy(ix).to(DEV) for ix in idxs]
    host_p = [g.shard_view(g.master_flat, i)[tidx[i]].cpu().numpy() for i in range(len(shapes))]
    host_m = [np.zeros_like(x) for x in host_p]
    host_v = [np.zeros_like(x) for x in host_p]
    rs = torch.empty(n * S, dtype=torch.int16, device=DEV)
    ag = torch.empty(n * S, dtype=torch.int16, device=DEV)
    for t in (1, 2, 3):
        synth.fill_normal_bf16_bits_(rs, 1e-3, ("fs-rs", cfg_index, gi, t))
        synth.fill_normal_bf16_bits_(ag, 0.02, ("fs-ag", cfg_index, gi, t))
        if fused:
            g.step(rs, ag[r * S:(r + 1) * S], t, write_grad=True, **hp)
        else:
            g.reduce(rs)
        torch.cuda.synchronize()
        rs2 = rs.view(n, S)
        for i, e in enumerate(g.entries):
            if not e.valid_numel:
                continue
            cols = rs2[:, e.shard_offset + tidx[i]].cpu().numpy().view(np.uint16)
            want = O.reduce(_col_plan(n, cols.shape[1]), cols)[0]
            got = g.shard_view(g.grad_flat, i)[tidx[i]].cpu().numpy()
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), ("grad", i, t)
            O.adamw(host_p[i], want, host_m[i], host_v[i], t, **hp)
        if not fused:
            g.adamw(t, **hp)
            g.pack(ag[r * S:(r + 1) * S])
        g.unpack(ag)
        torch.cuda.synchronize()
        row = ag.view(n, S)[r]
        for i, e in enumerate(g.entries):
            if e.valid_numel:
                for fl, host in ((g.master_flat, host_p), (g.m_flat, host_m), (g.v_flat, host_v)):
                    got = g.shard_view(fl, i)[tidx[i]].cpu().numpy()
                    assert np.array_equal(got.view(np.uint32), host[i].view(np.uint32)), ("state", i, t)
                got = row[e.shard_offset + tidx[i]].cpu().numpy().view(np.uint16)
                assert np.array_equal(got, O.bf16_rne(host_p[i])), ("pack", i, t)
                # every packed element against torch's library cast
                want = g.shard_view(g.master_flat, i).to(torch.bfloat16).view(torch.int16)
                assert torch.equal(row[e.shard_offset:e.shard_offset + e.valid_numel], want)
            pad = row[e.shard_offset + e.valid_numel:e.shard_offset + e.seg_numel]
            assert (pad == 0).all()
        # copy-out: sampled rows of every parameter against the oracle's row mapping
        agh = ag.view(n, S)
        for i, e in enumerate(g.entries):
            rows = _sample_idx(e.rows, ("fs-rows", cfg_index, gi, i, t), k=24)
            full = g.full_view(i)
            for row_i in rows.tolist():
                j = min(row_i // e.chunk_rows, n - 1)
                b, lr = O.rows_of_rank(e.rows, n, j)
                assert b <= row_i < b + lr
                o = e.shard_offset + (row_i - b) * e.cols
                want = agh[j, o:o + e.cols]
                assert torch.equal(full[row_i], want), ("full", i, row_i, t)
    g.close()


@pytest.mark.parametrize("cfg_index", [2, 4])
def test_reduce_all_equal_every_element(cfg_index):
    cfg, gs = _groups(cfg_index)
    gi, grp = gs[1]
    shapes = [p.shape for p in grp.params]
    n = cfg.world
    g = ShardedGroup(shapes, n, n - 1)
    S = g.S
    row = torch.empty(S, dtype=torch.int16, device=DEV)
    synth.fill_normal_bf16_bits_(row, 1e-3, ("eq-full", cfg_index))
    rs = row.repeat(n)
    g.reduce(rs)
    torch.cuda.synchronize()
    for i, e in enumerate(g.entries):
        want = row[e.shard_offset:e.shard_offset + e.valid_numel].view(torch.bfloat16).float()
        got = g.shard_view(g.grad_flat, i)
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), i
    g.close()


@pytest.mark.parametrize("cfg_index", [2, 3, 4])
def test_next_rows_full_block_group(cfg_index):
    """The reduce-scatter copy-ins (bf16 and fp32), the fp32 reduction and
    gradient accumulation on a full group (a 7B or 70B block group; the
    ragged MoE group at rank 5, whose odd segment misaligns every row of
    [N, S]), in the bench's launch configuration.  Every element against constructions from torch's own
    ops (chunk, zero padding, exact widening, fp32 add); the fp32 reduction
    against the oracle on sampled columns and, over every element, against
    the bf16 reduction of the same values."""
    cfg, gs = _groups(cfg_index)
    gi, grp = gs[0]
    shapes = [p.shape for p in grp.params]
    n, r = cfg.world, cfg.timing_rank
    print(f"[fullsize] next rows cfg={cfg_index} group={gi} n={n}", flush=True)
    g = ShardedGroup(shapes, n, r)
    S = g.S
    g.bind_full_grad()
    g.bind_grad_acc()
    micro = []
    for k in range(2):
        arena = torch.empty(g.full_space, dtype=torch.int16, device=DEV)
        synth.fill_normal_bf16_bits_(arena, 1e-3, ("nx-g", cfg_index, k))
        micro.append(arena)
    # accumulation: reset with microbatch 0, then add microbatch 1
    g.full_grad_flat.copy_(micro[0])
    g.accumulate_grad(True)
    g.full_grad_flat.copy_(micro[1])
    g.accumulate_grad(False)
    rs_b = torch.empty(n * S, dtype=torch.int16, device=DEV)
    rs_f = torch.empty(n * S, dtype=torch.float32, device=DEV)
    rs_a = torch.empty(n * S, dtype=torch.float32, device=DEV)
    g.pack_reduce_scatter(rs_b, capi.FSDP_DTYPE_BF16)
    g.pack_reduce_scatter(rs_f, capi.FSDP_DTYPE_F32)
    g.pack_reduce_scatter_acc(rs_a)
    torch.cuda.synchronize()
    rb, rf, ra = rs_b.view(n, S), rs_f.view(n, S), rs_a.view(n, S)
    for i, e in enumerate(g.entries):
        numel = e.rows * e.cols
        o = g.full_offsets[i]
        g0 = micro[0][o:o + numel].view(torch.bfloat16).float()
        g1 = micro[1][o:o + numel].view(torch.bfloat16).float()
        acc_want = g0 + g1                                  # one fp32 add per element
        acc = g.grad_acc_flat[o:o + numel]
        assert torch.equal(acc.view(torch.int32), acc_want.view(torch.int32)), ("acc", i)
        grad1 = micro[1][o:o + numel].view(e.rows, e.cols)
        acc2 = acc_want.view(e.rows, e.cols)
        for j in range(n):
            b, lr = O.rows_of_rank(e.rows, n, j)
            k = lr * e.cols
            sl = slice(e.shard_offset, e.shard_offset + e.seg_numel)
            want_b = torch.zeros(e.seg_numel, dtype=torch.int16, device=DEV)
            want_b[:k] = grad1[b:b + lr].reshape(-1)
            assert torch.equal(rb[j, sl], want_b), ("rs bf16", i, j)
            want_f = want_b.view(torch.bfloat16).float()
            want_f[k:] = 0.0
            assert torch.equal(rf[j, sl].view(torch.int32), want_f.view(torch.int32)), ("rs f32", i, j)
            want_a = torch.zeros(e.seg_numel, dtype=torch.float32, device=DEV)
            want_a[:k] = acc2[b:b + lr].reshape(-1)
            assert torch.equal(ra[j, sl].view(torch.int32), want_a.view(torch.int32)), ("rs acc", i, j)
    # fp32 reduction of the widened copy-in == bf16 reduction, every element
    g.reduce(rs_b)
    torch.cuda.synchronize()
    ref = g.grad_flat.clone()
    g.grad_flat.zero_()
    g.reduce_f32(rs_f)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int32), g.grad_flat.view(torch.int32))
    # the fp32 reduction of the accumulators, sampled against the oracle
    g.reduce_f32(rs_a)
    torch.cuda.synchronize()
    for i, e in enumerate(g.entries):
        if not e.valid_numel:
            continue
        ix = torch.from_numpy(_sample_idx(e.valid_numel, ("nx-idx", cfg_index, i))).to(DEV)
        cols = ra[:, e.shard_offset + ix].cpu().numpy()
        want = O.reduce_f32(_col_plan(n, cols.shape[1]), cols)[0]
        got = g.shard_view(g.grad_flat, i)[ix].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), ("reduce f32", i)
    g.close()


# Whole parameter groups (one group = one communication unit, [ST] fully_shard
# paragraph) through the multi-group executor the bench times, 3 AdamW steps,
# every element of every output against the oracle, bit for bit.  The groups:
# the one-block Llama group (= a block of the 7B shape, N = 8, the aligned
# fused kernel), the 7B shape's root group (embedding, final norm, head), the
# ragged MoE workload's two groups at ranks 5 and 0 (N = 6, odd segment,
# misaligned fused kernel), and the 70B shape's first and last block and its
# root group (N = 64, the wide fused kernel).
WHOLE = [("llama-block-r0", 1, (0,), 0),
         ("llama7b-root-r0", 2, (32,), 0),
         ("moe-r5", 3, (0, 1), 5),
         ("moe-r0", 3, (0, 1), 0),
         ("llama70b-r0", 4, (0, 79, 80), 0)]


@pytest.mark.parametrize("write_grad", [False, True], ids=["nograd", "grad"])
@pytest.mark.parametrize("name,cfg_index,group_ids,rank", WHOLE, ids=[w[0] for w in WHOLE])
def test_step_groups_whole_groups_every_element(name, cfg_index, group_ids, rank, write_grad):
    cfg = configs.get(cfg_index)
    n, hp = cfg.world, vars(cfg.hp)
    flags = capi.FSDP_STEP_WRITE_GRAD if write_grad else 0
    groups, plans, rs, ag = [], [], [], []
    hosts = []            # per group: oracle masters, m, v
    for gi in group_ids:
        shapes = [p.shape for p in cfg.groups[gi].params]
        g = ShardedGroup(shapes, n, rank)
        for i, e in enumerate(g.entries):
            synth.fill_normal_f32_(g.shard_view(g.master_flat, i), cfg.master_std,
                                   ("whole-m", cfg_index, gi, rank, i))
        g.grad_flat.fill_(-1.0)
        groups.append(g)
        plans.append(O.plan(shapes, n, rank))
        rs.append(torch.empty(n * g.S, dtype=torch.int16, device=DEV))
        ag.append(torch.empty(n * g.S, dtype=torch.int16, device=DEV))
        masters = [g.shard_view(g.master_flat, i).cpu().numpy() for i in range(len(shapes))]
        hosts.append((masters, [np.zeros_like(x) for x in masters],
                      [np.zeros_like(x) for x in masters]))
    execute = capi.StepGroupsCall([g.plan for g in groups], rs,
                                  [a[rank * g.S:(rank + 1) * g.S] for a, g in zip(ag, groups)],
                                  ag, flags=flags, **hp)
    for t in (1, 2, 3):
        rs_h, ag_h = [], []
        for k, (gi, g) in enumerate(zip(group_ids, groups)):
            synth.fill_normal_bf16_bits_(rs[k], cfg.grad_std, ("whole-rs", cfg_index, gi, rank, t))
            synth.fill_normal_bf16_bits_(ag[k], cfg.master_std, ("whole-ag", cfg_index, gi, rank, t))
            # inputs as the oracle sees them, read back before the step runs
            rs_h.append(rs[k].cpu().numpy().view(np.uint16).reshape(n, g.S))
            ag_h.append(ag[k].cpu().numpy().view(np.uint16).reshape(n, g.S))
        print(f"[fullsize] whole groups {name} step {t} flags={flags}", flush=True)
        execute(t)
        torch.cuda.synchronize()
        for k, (gi, g, plan) in enumerate(zip(group_ids, groups, plans)):
            masters, ms, vs = hosts[k]
            grads = O.reduce(plan, rs_h[k])
            for x, gr, m, v in zip(masters, grads, ms, vs):
                O.adamw(x, gr, m, v, t, **hp)
            want_ag = ag_h[k]
            want_ag[rank] = O.pack(plan, masters)
            got_row = ag[k].view(n, g.S)[rank].cpu().numpy().view(np.uint16)
            assert np.array_equal(got_row, want_ag[rank]), (name, gi, t, "packed row")
            for i, e in enumerate(g.entries):
                for fl, host, what in ((g.master_flat, masters, "master"), (g.m_flat, ms, "m"),
                                       (g.v_flat, vs, "v")):
                    got = g.shard_view(fl, i).cpu().numpy()
                    assert np.array_equal(got.view(np.uint32), host[i].view(np.uint32)), \
                        (name, gi, t, what, i)
                got_g = g.shard_view(g.grad_flat, i).cpu().numpy()
                if write_grad:
                    assert np.array_equal(got_g.view(np.uint32), grads[i].view(np.uint32)), \
                        (name, gi, t, "grad", i)
                else:
                    assert (got_g == -1.0).all(), (name, gi, t, "grad written without the flag")
            for i, want in enumerate(O.unpack(plan, want_ag)):
                got = g.full_view(i).cpu().numpy().view(np.uint16)
                assert np.array_equal(got, want), (name, gi, t, "full", i)
            del grads, want_ag
        del rs_h, ag_h
    for g in groups:
        g.close()


# ---------------------------------------------------------------------------
# group set at full size: the separate-kernel path the bench times with
# --unfused (a reduce per group, one AdamW and one copy-in launch over every
# group) against the fused executor on the same inputs, every group, every
# element of the grad, master, m and v shards and of every copy-in segment
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fuse", [False, True], ids=["two-launches", "adamw-copy-in"])
@pytest.mark.parametrize("cfg_index", [2, 4])
def test_group_set_every_group_equals_fused_executor(cfg_index, fuse):
    cfg = configs.get(cfg_index)
    n, hp, rank = cfg.world, vars(cfg.hp), cfg.timing_rank
    shapes = [[p.shape for p in grp.params] for grp in cfg.groups]

    def shards_only(s):            # no full-parameter tensors: no copy-out here
        g = ShardedGroup(s, n, rank, bind=False)
        g.allocate(full=False)
        g.bind()
        return g

    A = [shards_only(s) for s in shapes]
    B = [shards_only(s) for s in shapes]
    for gi, (ga, gb) in enumerate(zip(A, B)):
        synth.fill_normal_f32_(ga.master_flat, cfg.master_std, ("set-full", cfg_index, gi))
        gb.master_flat.copy_(ga.master_flat)
    max_ns = max(n * g.S for g in A)
    rs_arena = [torch.empty(max_ns, dtype=torch.int16, device=DEV) for _ in range(2)]
    rs = [rs_arena[gi & 1][:n * g.S] for gi, g in enumerate(A)]
    in_a = [torch.empty(g.S, dtype=torch.int16, device=DEV) for g in A]
    fused = capi.StepGroupsCall([g.plan for g in A], rs, in_a, None,
                                flags=capi.FSDP_STEP_WRITE_GRAD, **hp)
    gset = capi.fsdp_group_set_create([g.plan for g in B])
    offs = [capi.fsdp_group_set_segment(gset, gi)[0] for gi in range(len(B))]
    arena = torch.empty(capi.fsdp_group_set_segment(gset, 0)[1], dtype=torch.int16, device=DEV)
    separate = capi.StepGroupSetCall(gset, [g.plan for g in B], rs, arena, None,
                                     flags=capi.FSDP_SET_ADAMW_COPY_IN if fuse else 0, **hp)
    for t in (1, 2):
        for b in range(2):
            synth.fill_normal_bf16_bits_(rs_arena[b], cfg.grad_std, ("set-full-rs", cfg_index, b, t))
        print(f"[fullsize] group set c{cfg_index} fuse={fuse} step {t}", flush=True)
        fused(t)
        separate(t)
        torch.cuda.synchronize()
        for gi, (ga, gb) in enumerate(zip(A, B)):
            for fl in ("master_flat", "grad_flat", "m_flat", "v_flat"):
                assert torch.equal(getattr(ga, fl).view(torch.int32),
                                   getattr(gb, fl).view(torch.int32)), (cfg_index, gi, t, fl)
            assert torch.equal(arena[offs[gi]:offs[gi] + gb.S], in_a[gi]), (cfg_index, gi, t)
    capi.fsdp_group_set_destroy(gset)
    for g in A + B:
        g.close()
