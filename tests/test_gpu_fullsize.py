"""Full-size parity on the 7B- and 70B-shaped groups, as the bench launches them.

The groups are planned and bound exactly as bench.py does (ShardedGroup, same
plans, tiles and grids).  The oracle cannot run whole at these sizes, so each
output is checked two ways:

* sampled: the oracle computes chosen outputs one by one from the same inputs
  read back (first and last elements, tile edges, random picks);
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


CASES = [(2, "block"), (2, "root"), (4, "block"), (4, "root")]


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
