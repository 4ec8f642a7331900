"""Host-side checks of the C ABI library (no GPU needed).

* the shared library loads and exports every function include/fsdp_shard.h
  declares;
* the C++ planner agrees with the oracle's layout bit for bit on every
  workload, every rank and both alignments;
* argument errors are reported with the documented codes before any HIP call.
"""
import os
import re
import subprocess

import numpy as np
import pytest

from conftest import ROOT
from oracle import fsdp as O
from workloads import configs

capi = pytest.importorskip("sharded_shard_amd.capi")

HEADER = os.path.join(ROOT, "include", "fsdp_shard.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fsdp_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = header_functions()
    for want in ("fsdp_plan_create", "fsdp_pack_allgather", "fsdp_unpack_allgather",
                 "fsdp_reduce_shard", "fsdp_adamw_shard", "fsdp_bind", "fsdp_state_bytes"):
        assert want in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", capi.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fsdp_\w+)", out))
    missing = [n for n in header_functions() if n not in exported]
    assert not missing, missing
    for n in header_functions():
        assert hasattr(capi.lib, n)
        assert n in capi.EXPORTS


def test_abi_version_and_status_strings():
    assert capi.fsdp_abi_version() == 1
    for s in (0, -1, -2, -3, -4, -5, -6, 7):
        assert capi.fsdp_status_string(s)


def _check_plan(shapes, world, rank, align):
    rows = [s[0] for s in shapes]
    cols = [int(np.prod(s[1:])) if len(s) > 1 else 1 for s in shapes]
    ref = O.plan(shapes, world, rank, align)
    p = capi.fsdp_plan_create(rows, cols, world, rank, align)
    try:
        info = capi.fsdp_plan_info(p)
        assert (info.S, info.V, info.F) == (ref.S, ref.V, ref.F)
        assert info.n_params == len(shapes) and info.pad_total == ref.S - ref.V
        assert info.n_empty == sum(1 for e in ref.entries if e.local_rows == 0)
        for i, e in enumerate(ref.entries):
            g = capi.fsdp_plan_entry(p, i)
            for f in ("rows", "cols", "chunk_rows", "row_begin", "local_rows", "shard_offset",
                      "shard_numel", "valid_numel", "pad_numel", "seg_numel"):
                assert getattr(g, f) == getattr(e, f), (f, i, rank)
        for i, s in enumerate(shapes):
            for j in range(world):
                assert capi.fsdp_plan_rows_of_rank(p, i, j) == O.rows_of_rank(s[0], world, j)
        return info
    finally:
        capi.fsdp_plan_destroy(p)


@pytest.mark.parametrize("align", [1, 8])
@pytest.mark.parametrize("cfg", configs.ALL)
def test_planner_matches_oracle_on_every_workload(cfg, align):
    c = configs.get(cfg)
    seen = set()
    for g in c.groups:
        shapes = tuple(p.shape for p in g.params)
        if shapes in seen:      # the repeated decoder blocks share one layout
            continue
        seen.add(shapes)
        ranks = range(c.world) if c.world <= 8 else (0, 1, 31, 62, 63)
        for r in ranks:
            _check_plan(list(shapes), c.world, r, align)


@pytest.mark.parametrize("align", [1, 8])
def test_planner_matches_oracle_random_ragged(align):
    rng = np.random.default_rng(17)
    for _ in range(40):
        n = int(rng.integers(1, 70))
        shapes = []
        for _ in range(int(rng.integers(1, 12))):
            if rng.random() < 0.3:
                shapes.append((int(rng.integers(0, 200)),))
            else:
                shapes.append((int(rng.integers(0, 200)), int(rng.integers(1, 50)), 2))
        for r in {0, n - 1, int(rng.integers(0, n))}:
            _check_plan(shapes, n, r, align)


def test_tiles_cover_the_work_exactly():
    """Tile counts: every run split into pieces of at most the tile length."""
    c = configs.get(3)
    shapes = [p.shape for p in c.groups[0].params]
    info = _check_plan(shapes, 6, 5, 1)
    ref = O.plan(shapes, 6, 5)
    cdiv = lambda a, b: -(-a // b)
    want_pack = sum(cdiv(e.seg_numel, 16384) for e in ref.entries)
    want_unpack = sum(cdiv(O.rows_of_rank(e.rows, 6, j)[1] * e.cols, 32768)
                      for e in ref.entries for j in range(6))
    want_reduce = sum(cdiv(e.valid_numel, 4096) for e in ref.entries)
    want_adamw = sum(cdiv(e.valid_numel, 8192) for e in ref.entries)
    assert list(info.n_tiles) == [want_pack, want_unpack, want_reduce, want_adamw]


def test_state_bytes_matches_pages_and_oracle():
    assert capi.fsdp_state_bytes(7e9, 1, 0) == 112e9
    assert capi.fsdp_state_bytes(70e9, 1, 0) == 1120e9
    for n in (1, 8, 64):
        for s in range(4):
            assert capi.fsdp_state_bytes(7e9, n, s) == O.state_bytes(7e9, n, s)
    with pytest.raises(capi.FsdpError) as ei:
        capi.fsdp_state_bytes(7e9, 8, 4)
    assert ei.value.status == capi.FSDP_E_UNSUPPORTED
    with pytest.raises(capi.FsdpError) as ei:
        capi.fsdp_state_bytes(7e9, 0, 1)
    assert ei.value.status == capi.FSDP_E_INVAL


@pytest.mark.parametrize("args,code", [
    (([4], [1], 0, 0, 1), capi.FSDP_E_INVAL),       # world 0
    (([4], [1], 2, 2, 1), capi.FSDP_E_INVAL),       # rank out of range
    (([4], [1], 2, -1, 1), capi.FSDP_E_INVAL),
    (([-1], [1], 2, 0, 1), capi.FSDP_E_INVAL),      # negative rows
    (([4], [0], 2, 0, 1), capi.FSDP_E_INVAL),       # cols < 1
    (([4], [1], 2, 0, 4), capi.FSDP_E_UNSUPPORTED),  # align
    (([1 << 62], [1 << 10], 2, 0, 1), capi.FSDP_E_INVAL),  # overflow
])
def test_plan_create_errors(args, code):
    with pytest.raises(capi.FsdpError) as ei:
        capi.fsdp_plan_create(*args)
    assert ei.value.status == code
    assert capi.fsdp_last_error()


def test_empty_group_and_rows_zero_are_legal():
    info = _check_plan([(0, 5), (0,)], 4, 3, 1)
    assert info.S == 0 and info.V == 0
    info = _check_plan([], 2, 0, 1)
    assert info.S == 0 and info.n_params == 0


def test_hot_calls_reject_unbound_and_bad_arguments_without_gpu():
    p = capi.fsdp_plan_create([4, 3], [2, 1], 2, 0, 1)
    try:
        for call in (lambda: capi.fsdp_pack_allgather(p, 0x1000, 0),
                     lambda: capi.fsdp_unpack_allgather(p, 0x1000, 0),
                     lambda: capi.fsdp_reduce_shard(p, 0x1000, 0),
                     lambda: capi.fsdp_adamw_shard(p, 3e-4, 0.9, 0.999, 1e-8, 0.01, 1, 0)):
            with pytest.raises(capi.FsdpError) as ei:
                call()
            assert ei.value.status == capi.FSDP_E_STATE
        # bind validation happens before any device call
        with pytest.raises(capi.FsdpError) as ei:
            capi.fsdp_bind(p, master=[0, 0x1000], stream=0)
        assert ei.value.status == capi.FSDP_E_INVAL
        with pytest.raises(capi.FsdpError) as ei:
            capi.fsdp_bind(p, master=[0x1002, 0x1000], stream=0)
        assert ei.value.status == capi.FSDP_E_ALIGN
        with pytest.raises(capi.FsdpError) as ei:
            capi.fsdp_bind(p, full=[0x1001, 0x1000], stream=0)
        assert ei.value.status == capi.FSDP_E_ALIGN
        for fn in (capi.fsdp_pack_allgather, capi.fsdp_unpack_allgather, capi.fsdp_reduce_shard):
            with pytest.raises(capi.FsdpError) as ei:
                fn(None, 0x1000, 0)
            assert ei.value.status == capi.FSDP_E_INVAL
    finally:
        capi.fsdp_plan_destroy(p)
    capi.fsdp_plan_destroy(None)


def test_step_groups_rejects_bad_arguments_without_gpu():
    p = capi.fsdp_plan_create([8, 3], [4, 1], 2, 0, 1)
    try:
        call = capi.StepGroupsCall([p], [0x1000], [0x2000], [0x3000], 3e-4, 0.9, 0.999, 1e-8,
                                   0.01, stream=0)
        with pytest.raises(capi.FsdpError) as ei:      # not bound
            call(1)
        assert ei.value.status == capi.FSDP_E_STATE
        bad = capi.StepGroupsCall([p], [0x1000], [0x2000], [0x3000], 3e-4, 0.9, 0.999, 1e-8,
                                  0.01, flags=8, stream=0)
        with pytest.raises(capi.FsdpError) as ei:      # unknown flag
            bad(1)
        assert ei.value.status == capi.FSDP_E_INVAL
        with pytest.raises(capi.FsdpError) as ei:      # step counts from 1
            call(0)
        assert ei.value.status == capi.FSDP_E_INVAL
    finally:
        capi.fsdp_plan_destroy(p)


def test_group_set_rejects_bad_arguments_without_gpu():
    """fsdp_group_set_create refuses empty, null, repeated and never-bound
    plans before any HIP call; the set calls refuse a null set."""
    p = capi.fsdp_plan_create([8, 3], [4, 1], 2, 0, 1)
    q = capi.fsdp_plan_create([5], [2], 2, 1, 1)
    try:
        for plans, code in (([], capi.FSDP_E_INVAL), ([p, None], capi.FSDP_E_INVAL),
                            ([p, q, p], capi.FSDP_E_INVAL), ([p, q], capi.FSDP_E_STATE)):
            with pytest.raises(capi.FsdpError) as ei:
                capi.fsdp_group_set_create(plans, stream=0)
            assert ei.value.status == code, plans
        hp = capi.AdamwHparams(3e-4, 0.9, 0.999, 1e-8, 0.01)
        assert capi.lib.fsdp_adamw_groups(None, capi.ctypes.byref(hp), 1, None) == \
            capi.FSDP_E_INVAL
        assert capi.lib.fsdp_pack_allgather_groups(None, 0x1000, None) == capi.FSDP_E_INVAL
        assert capi.lib.fsdp_step_group_set(None, None, 0x1000, None, capi.ctypes.byref(hp), 1,
                                            0, 0, None, None) == capi.FSDP_E_INVAL
        assert capi.lib.fsdp_adamw_pack_groups(None, capi.ctypes.byref(hp), 1, 0x1000,
                                               None) == capi.FSDP_E_INVAL
        assert capi.lib.fsdp_amax_groups(None, 0x1000, None) == capi.FSDP_E_INVAL
        assert capi.lib.fsdp_pack_allgather_fp8_groups(None, 0x1000, 0x2000,
                                                       None) == capi.FSDP_E_INVAL
        for call in (lambda: capi.fsdp_group_set_segment(None, 0),
                     lambda: capi.fsdp_group_set_info(None)):
            with pytest.raises(capi.FsdpError) as ei:
                call()
            assert ei.value.status == capi.FSDP_E_INVAL
        capi.fsdp_group_set_destroy(None)
    finally:
        capi.fsdp_plan_destroy(p)
        capi.fsdp_plan_destroy(q)


def test_check_stream_reports_hip_errors_as_fsdp_e_hip():
    """fsdp_check_stream's error branch: on a machine without a GPU the HIP
    runtime fails the stream wait, and the status and HIP's message reach the
    caller (on a GPU the same branch reports an asynchronous kernel fault)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("needs a machine without a GPU")
    with pytest.raises(capi.FsdpError) as ei:
        capi.fsdp_check_stream(0)
    assert ei.value.status == capi.FSDP_E_HIP
    assert "hipStreamSynchronize" in str(ei.value) and capi.fsdp_last_error()


def test_binding_rejects_undersized_and_host_tensors_before_launching():
    """The C ABI cannot see buffer sizes; the binding checks torch tensors
    (size for this plan, then GPU residence) before the C call, so an
    undersized or host tensor never reaches a kernel."""
    import torch
    p = capi.fsdp_plan_create([8, 3], [4, 1], 2, 0, 1)
    try:
        info = capi.fsdp_plan_info(p)
        n, S, k = info.world, info.S, info.n_params
        assert S > 0
        i16 = lambda m: torch.zeros(m, dtype=torch.int16)
        f32 = lambda m: torch.zeros(m, dtype=torch.float32)
        u8 = lambda m: torch.zeros(m, dtype=torch.uint8)
        calls = [
            (lambda b: capi.fsdp_pack_allgather(p, b, 0), i16, S),
            (lambda b: capi.fsdp_unpack_allgather(p, b, 0), i16, n * S),
            (lambda b: capi.fsdp_reduce_shard(p, b, 0), i16, n * S),
            (lambda b: capi.fsdp_reduce_shard_f32(p, b, 0), f32, n * S),
            (lambda b: capi.fsdp_pack_reduce_scatter(p, b, capi.FSDP_DTYPE_BF16, 0), i16, n * S),
            (lambda b: capi.fsdp_pack_reduce_scatter(p, b, capi.FSDP_DTYPE_F32, 0), f32, n * S),
            (lambda b: capi.fsdp_pack_reduce_scatter_acc(p, b, 0), f32, n * S),
            (lambda b: capi.fsdp_unpack_allgather_fp8(p, b, 0), u8, n * S),
            (lambda b: capi.fsdp_pack_allgather_fp8(p, b, 0x1000, 0), u8, S),
            (lambda b: capi.fsdp_pack_allgather_fp8(p, 0x1000, b, 0), f32, k),
            (lambda b: capi.fsdp_amax_shard(p, b, 0), f32, k),
            (lambda b: capi.fsdp_step_shard(p, b, 0x1000, 3e-4, 0.9, 0.999, 1e-8, 0.01, 1,
                                             stream=0), i16, n * S),
            (lambda b: capi.fsdp_step_shard(p, 0x1000, b, 3e-4, 0.9, 0.999, 1e-8, 0.01, 1,
                                             stream=0), i16, S),
        ]
        for call, make, need in calls:
            with pytest.raises(ValueError, match="bytes"):
                call(make(need - 1))
            with pytest.raises(ValueError, match="GPU tensor"):
                call(make(need))
        for rs, ag_in, ag_out in ((i16(n * S - 1), 0x2000, 0x3000),
                                  (0x1000, i16(S - 1), 0x3000),
                                  (0x1000, 0x2000, i16(n * S - 1))):
            with pytest.raises(ValueError, match="bytes"):
                capi.StepGroupsCall([p], [rs], [ag_in], [ag_out], 3e-4, 0.9, 0.999, 1e-8, 0.01,
                                    stream=0)
        with pytest.raises(ValueError, match="one entry per group"):
            capi.StepGroupsCall([p], [0x1000, 0x2000], [0x2000], None, 3e-4, 0.9, 0.999, 1e-8,
                                0.01, stream=0)
        call = capi.StepGroupsCall([p], [0x1000], [0x2000], [0x3000], 3e-4, 0.9, 0.999, 1e-8,
                                   0.01, stream=0)
        with pytest.raises(ValueError, match="2 per group"):      # 2 events per group
            call(1, capi.FSDP_KERNEL_STEP, [None, None, None])
    finally:
        capi.fsdp_plan_destroy(p)


@pytest.mark.parametrize("n1,n2", [(2, 1), (1, 2), (3, 2), (8, 64), (64, 8), (6, 4), (5, 5)])
def test_reshard_planner_matches_oracle(n1, n2):
    shapes = [(37, 3), (1, 5), (0, 4), (130, 1), (128256 // 64, 2), (64, 7)]
    rows = [s[0] for s in shapes]
    cols = [s[1] for s in shapes]
    for d in range(n2):
        p = capi.fsdp_reshard_plan_create(rows, cols, n1, n2, d)
        try:
            want = [(i,) + r for i, (rr, cc) in enumerate(shapes)
                    for r in O.reshard_runs(rr, cc, n1, n2, d)]
            n_runs, dst_numel = capi.fsdp_reshard_plan_runs(p)
            assert n_runs == len(want)
            assert dst_numel == sum(O.rows_of_rank(rr, n2, d)[1] * cc for rr, cc in shapes)
            for k, w in enumerate(want):
                r = capi.fsdp_reshard_plan_run(p, k)
                assert (r.param, r.src_rank, r.src_offset, r.dst_offset, r.numel) == w
        finally:
            capi.fsdp_reshard_plan_destroy(p)


def test_reshard_plan_errors():
    for args in (([4], [1], 0, 1, 0), ([4], [1], 1, 0, 0), ([4], [1], 2, 2, 2), ([-1], [1], 2, 2, 0),
                 ([4], [0], 2, 2, 0)):
        with pytest.raises(capi.FsdpError) as ei:
            capi.fsdp_reshard_plan_create(*args)
        assert ei.value.status == capi.FSDP_E_INVAL
    p = capi.fsdp_reshard_plan_create([4], [2], 2, 1, 0)
    try:
        with pytest.raises(capi.FsdpError) as ei:
            capi.fsdp_reshard_execute(p, 0)
        assert ei.value.status == capi.FSDP_E_STATE
        with pytest.raises(capi.FsdpError) as ei:
            capi.fsdp_reshard_bind(p, [0x1000, 0x2000], [0x3000], 8, 0)
        assert ei.value.status == capi.FSDP_E_UNSUPPORTED
        with pytest.raises(capi.FsdpError) as ei:
            capi.fsdp_reshard_bind(p, [0x1000, 0x2002], [0x3000], 4, 0)
        assert ei.value.status == capi.FSDP_E_ALIGN
        with pytest.raises(capi.FsdpError) as ei:
            capi.fsdp_reshard_bind(p, [0x1000, 0], [0x3000], 4, 0)
        assert ei.value.status == capi.FSDP_E_INVAL
    finally:
        capi.fsdp_reshard_plan_destroy(p)


@pytest.mark.parametrize("n_threads", [1, 3, 0])
def test_host_adamw_bit_exact_with_oracle(n_threads):
    from workloads import synth
    HP = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    for n in (0, 1, 7, 65537, 300001):
        p = synth.normal_f32(n, 0.02, ("hostadam", n)).numpy().copy()
        m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
        ref = [p.copy(), m.copy(), v.copy()]
        for t in (1, 2, 3):
            g = synth.normal_f32(n, 1e-3, ("hostadam-g", n, t)).numpy()
            capi.fsdp_adamw_host(p, g, m, v, step=t, n_threads=n_threads, **HP)
            O.adamw(ref[0], g, ref[1], ref[2], t, **HP)
        for a, b in zip((p, m, v), ref):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (n, n_threads)


def test_host_adamw_special_values():
    """Infinities, NaNs, subnormals, zeros and near-overflow values in the
    master and the gradient: the host update equals the oracle bit for bit,
    a NaN created by an operation matching any NaN."""
    HP = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3e38, -3e38, 1e-45, -1e-40, 1e-30],
                        np.float32)
    rng = np.random.default_rng(11)
    n = 4099
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hit = rng.random(n) < 0.2
    p[hit] = rng.choice(specials, size=int(hit.sum()))
    p[:specials.size] = specials
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    ref = [p.copy(), m.copy(), v.copy()]
    for t in (1, 2, 3):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        hit = rng.random(n) < 0.2
        g[hit] = rng.choice(specials, size=int(hit.sum()))
        g[-specials.size:] = specials
        capi.fsdp_adamw_host(p, g, m, v, step=t, n_threads=3, **HP)
        with np.errstate(all="ignore"):
            O.adamw(ref[0], g, ref[1], ref[2], t, **HP)
    for a, b in zip((p, m, v), ref):
        an, bn = np.isnan(a), np.isnan(b)
        assert np.array_equal(an, bn)
        assert np.array_equal(a[~an].view(np.uint32), b[~bn].view(np.uint32))
    assert np.isnan(ref[0]).any() and np.isinf(ref[2]).any()


def test_host_adamw_errors():
    x = np.zeros(4, np.float32)
    with pytest.raises(capi.FsdpError) as ei:
        capi.fsdp_adamw_host(x, x, x, x, 3e-4, 0.9, 0.999, 1e-8, 0.01, step=0)
    assert ei.value.status == capi.FSDP_E_INVAL
    with pytest.raises(ValueError):
        capi.fsdp_adamw_host(x, x[:3], x, x, 3e-4, 0.9, 0.999, 1e-8, 0.01, step=1)
