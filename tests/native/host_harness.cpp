// Host sanitizer harness: the library's host code (planner, C ABI argument
// checks, device-table management, the multi-group executor, fault
// injection, the reshard planner and executor, host AdamW) built with
// AddressSanitizer and UndefinedBehaviorSanitizer against a host-memory HIP
// stand-in (fake_hip.cpp) and launch stand-ins that touch and record exactly
// the ranges each uploaded tile names (fake_launch.cpp).
//
// Workloads come on stdin, one per line:
//     <name> <world> <rank> <align> <n_params> <rows_0> <cols_0> ... <rows_n-1> <cols_n-1>
// Every buffer is its own exact-size allocation, so a tile reaching past its
// tensor is an ASan report.  For each workload the harness binds every role,
// runs every hot call (and the group-set calls over two groups) and checks
// that each call writes every element of its outputs exactly once; then it
// drives the error paths and the FSDP_FAULT hook.  Prints "ALL OK" and exits 0 when every check passed.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "../../include/fsdp_shard.h"
#include "harness.hpp"

namespace {

int g_failures = 0;

#define CHECK(cond, ...)                                                   \
    do {                                                                   \
        if (!(cond)) {                                                     \
            ++g_failures;                                                  \
            std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
            std::fprintf(stderr, __VA_ARGS__);                             \
            std::fprintf(stderr, "\n");                                    \
        }                                                                  \
    } while (0)

#define CHECK_STATUS(call, want)                                                        \
    do {                                                                                \
        const fsdp_status s_ = (call);                                                  \
        CHECK(s_ == (want), "%s returned %d (%s), wanted %d", #call, s_,                \
              fsdp_last_error(), (want));                                               \
    } while (0)

std::vector<void *> g_allocs;

template <typename T>
T *alloc(int64_t n) {
    if (n <= 0) return nullptr;
    void *p = std::malloc(static_cast<size_t>(n) * sizeof(T));
    g_allocs.push_back(p);
    return static_cast<T *>(p);
}

int64_t chunk(int64_t rows, int32_t world) { return rows <= 0 ? 0 : (rows + world - 1) / world; }

void rows_of(int64_t rows, int32_t world, int32_t j, int64_t *b, int64_t *lr) {
    const int64_t c = chunk(rows, world);
    *b = std::min<int64_t>(int64_t(j) * c, rows);
    *lr = std::min<int64_t>(int64_t(j + 1) * c, rows) - *b;
}

// Every element of [0, total) of `base` written exactly once by the recorded
// spans of `kind`, and no span of that kind on that base outside it.
void check_cover(const void *base, int64_t total, int kind, const char *what,
                 const std::string &wl) {
    std::vector<uint8_t> hits(static_cast<size_t>(std::max<int64_t>(total, 0)), 0);
    bool outside = false;
    for (const harness::Span &s : harness::spans) {
        if (s.base != base || s.kind != kind) continue;
        if (s.off < 0 || s.off + s.len > total) {
            outside = true;
            continue;
        }
        for (int64_t i = s.off; i < s.off + s.len; ++i)
            if (hits[i] < 2) ++hits[i];
    }
    CHECK(!outside, "%s / %s: a write range lies outside [0, %lld)", wl.c_str(), what,
          (long long)total);
    int64_t bad = 0;
    for (uint8_t h : hits) bad += h != 1;
    CHECK(bad == 0, "%s / %s: %lld of %lld elements not written exactly once", wl.c_str(), what,
          (long long)bad, (long long)total);
}

struct Workload {
    std::string name;
    int32_t world = 1, rank = 0, align = 1;
    std::vector<int64_t> rows, cols;
};

// One plan and every tensor it can bind, each an exact-size allocation.
struct Instance {
    fsdp_plan *plan = nullptr;
    fsdp_plan_info_t info{};
    std::vector<fsdp_shard_entry_t> ents;
    std::vector<float *> master, grad, m, v, acc;
    std::vector<uint16_t *> full, full_grad;
    std::vector<uint8_t *> full8;
    uint16_t *ag = nullptr, *rs = nullptr;
    float *rs32 = nullptr, *rsacc = nullptr, *scales = nullptr, *amax = nullptr;
    uint8_t *ag8 = nullptr;

    uint16_t *ag_in() const { return ag != nullptr ? ag + int64_t(info.rank) * info.S : nullptr; }
    uint8_t *ag8_in() const { return ag8 != nullptr ? ag8 + int64_t(info.rank) * info.S : nullptr; }
};

bool make(const Workload &w, Instance *in) {
    const int32_t n = static_cast<int32_t>(w.rows.size());
    if (fsdp_plan_create(w.rows.data(), w.cols.data(), n, w.world, w.rank, w.align, &in->plan) !=
        FSDP_OK) {
        std::fprintf(stderr, "FAIL plan %s: %s\n", w.name.c_str(), fsdp_last_error());
        ++g_failures;
        return false;
    }
    CHECK_STATUS(fsdp_plan_info(in->plan, &in->info), FSDP_OK);
    in->ents.resize(n);
    for (int32_t i = 0; i < n; ++i) CHECK_STATUS(fsdp_plan_entry(in->plan, i, &in->ents[i]), FSDP_OK);
    for (int32_t i = 0; i < n; ++i) {
        const int64_t vn = in->ents[i].valid_numel, f = w.rows[i] * w.cols[i];
        in->master.push_back(alloc<float>(vn));
        in->grad.push_back(alloc<float>(vn));
        in->m.push_back(alloc<float>(vn));
        in->v.push_back(alloc<float>(vn));
        in->full.push_back(alloc<uint16_t>(f));
        in->full_grad.push_back(alloc<uint16_t>(f));
        in->acc.push_back(alloc<float>(f));
        in->full8.push_back(alloc<uint8_t>(f));
    }
    const int64_t NS = int64_t(in->info.world) * in->info.S;
    in->ag = alloc<uint16_t>(NS);
    in->rs = alloc<uint16_t>(NS);
    in->rs32 = alloc<float>(NS);
    in->rsacc = alloc<float>(NS);
    in->ag8 = alloc<uint8_t>(NS);
    in->scales = alloc<float>(n);
    in->amax = alloc<float>(n);
    return true;
}

void bind_all(Instance *in) {
    CHECK_STATUS(fsdp_bind(in->plan, in->master.data(), in->grad.data(), in->m.data(),
                           in->v.data(), in->full.data(), nullptr),
                 FSDP_OK);
    CHECK_STATUS(fsdp_bind_full_grad(in->plan, in->full_grad.data(), nullptr), FSDP_OK);
    CHECK_STATUS(fsdp_bind_grad_acc(in->plan, in->acc.data(), nullptr), FSDP_OK);
    CHECK_STATUS(fsdp_bind_full_fp8(in->plan, in->full8.data(), nullptr), FSDP_OK);
}

const fsdp_adamw_hparams_t kHp{3e-4, 0.9, 0.999, 1e-8, 0.01};

void check_shards(const Instance &in, const std::vector<float *> &role, const char *what,
                  const std::string &wl) {
    for (size_t i = 0; i < in.ents.size(); ++i)
        if (in.ents[i].valid_numel > 0)
            check_cover(role[i], in.ents[i].valid_numel, harness::kShard, what, wl);
}

void check_full(const Instance &in, const Workload &w, const std::vector<const void *> &role,
                int kind, const char *what) {
    for (size_t i = 0; i < in.ents.size(); ++i)
        if (w.rows[i] * w.cols[i] > 0)
            check_cover(role[i], w.rows[i] * w.cols[i], kind, what, w.name);
}

template <typename T>
std::vector<const void *> as_void(const std::vector<T *> &v) {
    return std::vector<const void *>(v.begin(), v.end());
}

void hot_calls(const Workload &w, Instance &in) {
    const int64_t S = in.info.S, NS = int64_t(in.info.world) * S;
    const std::string &wl = w.name;
    auto fresh = [] { harness::spans.clear(); };

    fresh();
    CHECK_STATUS(fsdp_pack_allgather(in.plan, in.ag_in(), nullptr), FSDP_OK);
    if (S > 0) check_cover(in.ag_in(), S, harness::kSegment, "copy-in", wl);
    fresh();
    CHECK_STATUS(fsdp_unpack_allgather(in.plan, in.ag, nullptr), FSDP_OK);
    check_full(in, w, as_void(in.full), harness::kFull, "copy-out");
    fresh();
    CHECK_STATUS(fsdp_reduce_shard(in.plan, in.rs, nullptr), FSDP_OK);
    check_shards(in, in.grad, "reduce", wl);
    fresh();
    CHECK_STATUS(fsdp_adamw_shard(in.plan, &kHp, 1, nullptr), FSDP_OK);
    check_shards(in, in.master, "adamw", wl);
    for (uint32_t flags : {0u, uint32_t(FSDP_STEP_WRITE_GRAD)}) {
        fresh();
        CHECK_STATUS(fsdp_step_shard(in.plan, in.rs, in.ag_in(), &kHp, 2, flags, nullptr), FSDP_OK);
        check_shards(in, in.master, "fused step", wl);
        if (S > 0) check_cover(in.ag_in(), S, harness::kSegment, "fused step copy-in", wl);
    }
    for (int32_t dt : {int32_t(FSDP_DTYPE_BF16), int32_t(FSDP_DTYPE_F32)}) {
        fresh();
        void *out = dt == FSDP_DTYPE_BF16 ? static_cast<void *>(in.rs) : static_cast<void *>(in.rs32);
        CHECK_STATUS(fsdp_pack_reduce_scatter(in.plan, out, dt, nullptr), FSDP_OK);
        if (NS > 0) check_cover(out, NS, harness::kRows, "reduce-scatter copy-in", wl);
    }
    fresh();
    CHECK_STATUS(fsdp_reduce_shard_f32(in.plan, in.rs32, nullptr), FSDP_OK);
    check_shards(in, in.grad, "fp32 reduce", wl);
    for (int32_t reset : {1, 0}) {
        fresh();
        CHECK_STATUS(fsdp_accumulate_grad(in.plan, reset, nullptr), FSDP_OK);
        check_full(in, w, as_void(in.acc), harness::kFull, "accumulate");
    }
    fresh();
    CHECK_STATUS(fsdp_pack_reduce_scatter_acc(in.plan, in.rsacc, nullptr), FSDP_OK);
    if (NS > 0) check_cover(in.rsacc, NS, harness::kRows, "accumulator copy-in", wl);
    fresh();
    CHECK_STATUS(fsdp_pack_allgather_fp8(in.plan, in.ag8_in(), in.scales, nullptr), FSDP_OK);
    if (S > 0) check_cover(in.ag8_in(), S, harness::kSegment, "FP8 copy-in", wl);
    fresh();
    CHECK_STATUS(fsdp_unpack_allgather_fp8(in.plan, in.ag8, nullptr), FSDP_OK);
    check_full(in, w, as_void(in.full8), harness::kFull, "FP8 copy-out");
    fresh();
    CHECK_STATUS(fsdp_amax_shard(in.plan, in.amax, nullptr), FSDP_OK);
    if (!in.ents.empty())
        check_cover(in.amax, int64_t(in.ents.size()), harness::kSmall, "amax", wl);
}

void executor(const Workload &w, Instance &a, Instance &b) {
    fsdp_plan *plans[2] = {a.plan, b.plan};
    const uint16_t *rs[2] = {a.rs, b.rs};
    uint16_t *ag_in[2] = {a.ag_in(), b.ag_in()};
    const uint16_t *ag_out[2] = {a.ag, b.ag};
    for (uint32_t flags : {0u, uint32_t(FSDP_STEP_WRITE_GRAD), uint32_t(FSDP_STEP_UNFUSED)}) {
        harness::spans.clear();
        CHECK_STATUS(fsdp_step_groups(plans, 2, rs, ag_in, ag_out, &kHp, 3, flags, 0, nullptr,
                                      nullptr),
                     FSDP_OK);
        for (Instance *in : {&a, &b}) {
            check_shards(*in, in->master, "executor", w.name);
            if (in->info.S > 0)
                check_cover(in->ag_in(), in->info.S, harness::kSegment, "executor copy-in", w.name);
            check_full(*in, w, as_void(in->full), harness::kFull, "executor copy-out");
        }
    }
    // timing events: a recorded pair per group, and half a pair rejected
    int ev_storage[4];
    void *evs[4] = {&ev_storage[0], &ev_storage[1], &ev_storage[2], &ev_storage[3]};
    CHECK_STATUS(fsdp_step_groups(plans, 2, rs, ag_in, ag_out, &kHp, 4, 0, FSDP_KERNEL_STEP, evs,
                                  nullptr),
                 FSDP_OK);
    evs[3] = nullptr;
    CHECK_STATUS(fsdp_step_groups(plans, 2, rs, ag_in, ag_out, &kHp, 4, 0, FSDP_KERNEL_STEP, evs,
                                  nullptr),
                 FSDP_E_INVAL);
    CHECK_STATUS(fsdp_step_groups(plans, 2, rs, ag_in, nullptr, &kHp, 4, 0, FSDP_KERNEL_UNPACK,
                                  evs, nullptr),
                 FSDP_E_INVAL);
    CHECK_STATUS(fsdp_step_groups(plans, 2, rs, ag_in, ag_out, &kHp, 4, 8u, 0, nullptr, nullptr),
                 FSDP_E_INVAL);
    CHECK_STATUS(fsdp_step_groups(plans, -1, rs, ag_in, ag_out, &kHp, 4, 0, 0, nullptr, nullptr),
                 FSDP_E_INVAL);
}

// Group sets: the one-launch AdamW and copy-in over two groups write every
// shard and every segment exactly once (and nothing between segments); the
// set executor matches the per-group unfused step's coverage; shards that
// overlap where AdamW writes are refused, shared read-only grads are not;
// rebinding a group invalidates the set until the old tensors are back.
void group_sets(const Workload &w, Instance &a, Instance &b) {
    fsdp_plan *plans[2] = {a.plan, b.plan};
    fsdp_group_set *set = nullptr;
    CHECK_STATUS(fsdp_group_set_create(plans, 2, nullptr, &set), FSDP_OK);
    if (set == nullptr) return;
    int64_t off[2] = {0, 0}, total = 0, t1 = 0;
    CHECK_STATUS(fsdp_group_set_segment(set, 0, &off[0], &total), FSDP_OK);
    CHECK_STATUS(fsdp_group_set_segment(set, 1, &off[1], &t1), FSDP_OK);
    const int64_t S = a.info.S;
    const int64_t S8 = (S + 7) / 8 * 8;
    CHECK(off[0] == 0 && off[1] == S8 && total == 2 * S8 && t1 == total,
          "%s: segments at %lld, %lld of %lld", w.name.c_str(), (long long)off[0],
          (long long)off[1], (long long)total);
    CHECK_STATUS(fsdp_group_set_segment(set, 2, &off[0], &total), FSDP_E_INVAL);
    int32_t n_groups = 0, n_params = 0;
    int64_t t2 = 0;
    CHECK_STATUS(fsdp_group_set_info(set, &n_groups, &n_params, &t2), FSDP_OK);
    CHECK(n_groups == 2 && t2 == total && n_params == int32_t(a.ents.size() + b.ents.size()),
          "%s: info %d groups, %d params, %lld elements", w.name.c_str(), n_groups, n_params,
          (long long)t2);
    CHECK_STATUS(fsdp_group_set_info(set, nullptr, &n_params, &t2), FSDP_E_INVAL);
    uint16_t *arena = alloc<uint16_t>(total);

    harness::spans.clear();
    CHECK_STATUS(fsdp_adamw_groups(set, &kHp, 1, nullptr), FSDP_OK);
    for (Instance *in : {&a, &b}) check_shards(*in, in->master, "set AdamW", w.name);

    auto check_arena = [&](const char *what, const void *base = nullptr) {
        if (base == nullptr) base = arena;
        std::vector<uint8_t> hits(static_cast<size_t>(total), 0);
        int64_t outside = 0, bad = 0;
        for (const harness::Span &sp : harness::spans) {
            if (sp.base != base || sp.kind != harness::kSegment) continue;
            if (sp.off < 0 || sp.off + sp.len > total) {
                ++outside;
                continue;
            }
            for (int64_t i = sp.off; i < sp.off + sp.len; ++i)
                if (hits[i] < 2) ++hits[i];
        }
        for (int64_t i = 0; i < total; ++i) {
            const bool in_seg = (i >= off[0] && i < off[0] + S) || (i >= off[1] && i < off[1] + S);
            bad += hits[i] != (in_seg ? 1 : 0);
        }
        CHECK(outside == 0 && bad == 0, "%s / %s: %lld ranges outside, %lld elements wrong",
              w.name.c_str(), what, (long long)outside, (long long)bad);
    };
    off[1] = S8;
    harness::spans.clear();
    CHECK_STATUS(fsdp_pack_allgather_groups(set, arena, nullptr), FSDP_OK);
    check_arena("set copy-in");

    // FP8: amax of every parameter and the FP8 copy-in of every group, one
    // launch each (amax: a clear and a launch)
    uint8_t *arena8 = alloc<uint8_t>(total);
    float *amax = alloc<float>(n_params), *scales = alloc<float>(n_params);
    harness::spans.clear();
    long l8 = harness::launches;
    CHECK_STATUS(fsdp_amax_groups(set, amax, nullptr), FSDP_OK);
    if (n_params > 0) check_cover(amax, n_params, harness::kSmall, "set amax", w.name);
    CHECK_STATUS(fsdp_pack_allgather_fp8_groups(set, arena8, scales, nullptr), FSDP_OK);
    CHECK(harness::launches == l8 + 2 || n_params == 0, "%s: %ld FP8 set launches",
          w.name.c_str(), harness::launches - l8);
    check_arena("set FP8 copy-in", arena8);
    if (n_params > 0) {
        CHECK_STATUS(fsdp_amax_groups(set, nullptr, nullptr), FSDP_E_INVAL);
        CHECK_STATUS(fsdp_pack_allgather_fp8_groups(set, arena8, nullptr, nullptr), FSDP_E_INVAL);
        CHECK_STATUS(fsdp_amax_groups(set, reinterpret_cast<float *>(
                                                reinterpret_cast<char *>(amax) + 2),
                                      nullptr),
                     FSDP_E_ALIGN);
    }

    const uint16_t *rs[2] = {a.rs, b.rs};
    const uint16_t *ag_out[2] = {a.ag, b.ag};
    harness::spans.clear();
    CHECK_STATUS(fsdp_step_group_set(set, rs, arena, ag_out, &kHp, 2, 0, 0, nullptr, nullptr),
                 FSDP_OK);
    check_arena("set executor copy-in");
    for (Instance *in : {&a, &b}) {
        check_shards(*in, in->grad, "set executor reduce", w.name);
        check_shards(*in, in->master, "set executor AdamW", w.name);
        check_full(*in, w, as_void(in->full), harness::kFull, "set executor copy-out");
    }
    int ev_storage[4];
    void *evs[4] = {&ev_storage[0], &ev_storage[1], &ev_storage[2], &ev_storage[3]};
    for (int32_t k : {FSDP_KERNEL_REDUCE, FSDP_KERNEL_ADAMW, FSDP_KERNEL_PACK, FSDP_KERNEL_UNPACK})
        CHECK_STATUS(fsdp_step_group_set(set, rs, arena, ag_out, &kHp, 3, 0, k, evs, nullptr),
                     FSDP_OK);
    CHECK_STATUS(fsdp_step_group_set(set, rs, arena, ag_out, &kHp, 3, 0, FSDP_KERNEL_STEP, evs,
                                     nullptr),
                 FSDP_E_INVAL);
    CHECK_STATUS(fsdp_step_group_set(set, rs, arena, ag_out, &kHp, 3, 0, FSDP_KERNEL_ADAMW_PACK,
                                     evs, nullptr),
                 FSDP_E_INVAL);
    CHECK_STATUS(fsdp_step_group_set(set, rs, arena, nullptr, &kHp, 3, 0, FSDP_KERNEL_UNPACK,
                                     evs, nullptr),
                 FSDP_E_INVAL);
    // AdamW and copy-in fused: one launch, the same coverage
    for (int32_t k : {FSDP_KERNEL_REDUCE, FSDP_KERNEL_ADAMW_PACK, FSDP_KERNEL_UNPACK}) {
        harness::spans.clear();
        const long l0 = harness::launches;
        CHECK_STATUS(fsdp_step_group_set(set, rs, arena, ag_out, &kHp, 3, FSDP_SET_ADAMW_COPY_IN,
                                         k, evs, nullptr),
                     FSDP_OK);
        CHECK(harness::launches == l0 + 5, "%s: %ld launches, wanted 5", w.name.c_str(),
              harness::launches - l0);
        check_arena("set executor, fused AdamW and copy-in");
        for (Instance *in : {&a, &b}) {
            check_shards(*in, in->grad, "set executor reduce", w.name);
            check_shards(*in, in->master, "set executor fused AdamW", w.name);
        }
    }
    CHECK_STATUS(fsdp_step_group_set(set, rs, arena, ag_out, &kHp, 3, FSDP_SET_ADAMW_COPY_IN,
                                     FSDP_KERNEL_ADAMW, evs, nullptr),
                 FSDP_E_INVAL);
    CHECK_STATUS(fsdp_step_group_set(set, rs, arena, ag_out, &kHp, 3, 2u, 0, nullptr, nullptr),
                 FSDP_E_INVAL);
    harness::spans.clear();
    CHECK_STATUS(fsdp_adamw_pack_groups(set, &kHp, 4, arena, nullptr), FSDP_OK);
    check_arena("fused AdamW and copy-in");
    for (Instance *in : {&a, &b}) check_shards(*in, in->master, "fused AdamW", w.name);
    CHECK_STATUS(fsdp_adamw_pack_groups(set, nullptr, 4, arena, nullptr), FSDP_E_INVAL);
    evs[1] = nullptr;
    CHECK_STATUS(fsdp_step_group_set(set, rs, arena, ag_out, &kHp, 3, 0, FSDP_KERNEL_ADAMW, evs,
                                     nullptr),
                 FSDP_E_INVAL);
    CHECK_STATUS(fsdp_step_group_set(set, nullptr, arena, ag_out, &kHp, 3, 0, 0, nullptr, nullptr),
                 FSDP_E_INVAL);
    CHECK_STATUS(fsdp_step_group_set(set, rs, arena, ag_out, &kHp, 0, 0, 0, nullptr, nullptr),
                 FSDP_E_INVAL);
    if (S > 0) {
        CHECK_STATUS(fsdp_pack_allgather_groups(set, nullptr, nullptr), FSDP_E_INVAL);
        CHECK_STATUS(fsdp_pack_allgather_groups(set, reinterpret_cast<uint16_t *>(
                                                         reinterpret_cast<char *>(arena) + 1),
                                                nullptr),
                     FSDP_E_ALIGN);
        // the arena may not cover a shard tensor of the set
        uint16_t *in_master = nullptr;
        for (size_t i = 0; i < a.ents.size() && in_master == nullptr; ++i)
            if (a.ents[i].valid_numel > 0) in_master = reinterpret_cast<uint16_t *>(a.master[i]);
        if (in_master != nullptr) {
            CHECK_STATUS(fsdp_pack_allgather_groups(set, in_master - 3, nullptr), FSDP_E_INVAL);
            CHECK_STATUS(fsdp_adamw_pack_groups(set, &kHp, 1, in_master, nullptr), FSDP_E_INVAL);
        }
        // the arena may not cover a group's reduce-scatter input
        CHECK_STATUS(fsdp_step_group_set(set, rs, const_cast<uint16_t *>(b.rs), ag_out, &kHp, 3, 0,
                                         0, nullptr, nullptr),
                     FSDP_E_INVAL);
        setenv("FSDP_FAULT", "launch", 1);
        const long l0 = harness::launches;
        CHECK_STATUS(fsdp_adamw_groups(set, &kHp, 1, nullptr), FSDP_E_HIP);
        CHECK(std::strstr(fsdp_last_error(), "injected") != nullptr, "message: %s",
              fsdp_last_error());
        CHECK(harness::launches == l0, "%s: a faulted set call launched", w.name.c_str());
        unsetenv("FSDP_FAULT");
    }

    // rebinding a group's AdamW tensors invalidates the set; binding the old
    // ones again makes it valid again
    bool any_valid = false;
    for (const fsdp_shard_entry_t &e : b.ents) any_valid = any_valid || e.valid_numel > 0;
    if (any_valid) {
        std::vector<float *> other;
        for (const fsdp_shard_entry_t &e : b.ents) other.push_back(alloc<float>(e.valid_numel));
        CHECK_STATUS(fsdp_bind(b.plan, other.data(), nullptr, nullptr, nullptr, nullptr, nullptr),
                     FSDP_OK);
        CHECK_STATUS(fsdp_adamw_groups(set, &kHp, 1, nullptr), FSDP_E_STATE);
        CHECK_STATUS(fsdp_pack_allgather_groups(set, arena, nullptr), FSDP_E_STATE);
        CHECK_STATUS(fsdp_bind(b.plan, b.master.data(), nullptr, nullptr, nullptr, nullptr,
                               nullptr),
                     FSDP_OK);
        CHECK_STATUS(fsdp_adamw_groups(set, &kHp, 1, nullptr), FSDP_OK);
    }
    fsdp_group_set_destroy(set);

    // a repeated plan, an unbound plan, overlapping written shards: refused
    fsdp_plan *twice[2] = {a.plan, a.plan};
    set = nullptr;
    CHECK_STATUS(fsdp_group_set_create(twice, 2, nullptr, &set), FSDP_E_INVAL);
    CHECK_STATUS(fsdp_group_set_create(plans, 0, nullptr, &set), FSDP_E_INVAL);
    CHECK(set == nullptr, "a refused set was returned");
    if (any_valid) {
        Instance c;
        if (!make(w, &c)) return;
        fsdp_plan *ac[2] = {a.plan, c.plan};
        CHECK_STATUS(fsdp_group_set_create(ac, 2, nullptr, &set), FSDP_E_STATE);
        // c reads a's grads: reads may be shared
        CHECK_STATUS(fsdp_bind(c.plan, c.master.data(), a.grad.data(), c.m.data(), c.v.data(),
                               nullptr, nullptr),
                     FSDP_OK);
        CHECK_STATUS(fsdp_group_set_create(ac, 2, nullptr, &set), FSDP_OK);
        fsdp_group_set_destroy(set);
        set = nullptr;
        // c's exp_avg is a's master: refused
        CHECK_STATUS(fsdp_bind(c.plan, nullptr, nullptr, a.master.data(), nullptr, nullptr,
                               nullptr),
                     FSDP_OK);
        CHECK_STATUS(fsdp_group_set_create(ac, 2, nullptr, &set), FSDP_E_INVAL);
        CHECK(std::strstr(fsdp_last_error(), "overlap") != nullptr, "message: %s",
              fsdp_last_error());
        CHECK(set == nullptr, "a refused set was returned");
        fsdp_plan_destroy(c.plan);
    }
}

// FSDP_FAULT: every launch fails before anything is recorded, or only the
// K-th one; the status and message reach the caller; unset, calls work.
void faults(const Workload &w, Instance &a, Instance &b) {
    if (a.info.S == 0) return;
    setenv("FSDP_FAULT", "launch", 1);
    harness::spans.clear();
    const long before = harness::launches;
    CHECK_STATUS(fsdp_pack_allgather(a.plan, a.ag_in(), nullptr), FSDP_E_HIP);
    CHECK(std::strstr(fsdp_last_error(), "injected") != nullptr, "message: %s", fsdp_last_error());
    CHECK_STATUS(fsdp_step_shard(a.plan, a.rs, a.ag_in(), &kHp, 1, 0, nullptr), FSDP_E_HIP);
    CHECK_STATUS(fsdp_amax_shard(a.plan, a.amax, nullptr), FSDP_E_HIP);
    CHECK_STATUS(fsdp_reduce_shard_f32(a.plan, a.rs32, nullptr), FSDP_E_HIP);
    CHECK(harness::launches == before && harness::spans.empty(), "%s: a faulted call launched",
          w.name.c_str());

    // the third launch of a two-group step (group 1's fused step) fails:
    // group 0's step and copy-out ran, nothing after the fault did
    fsdp_plan *plans[2] = {a.plan, b.plan};
    const uint16_t *rs[2] = {a.rs, b.rs};
    uint16_t *ag_in[2] = {a.ag_in(), b.ag_in()};
    const uint16_t *ag_out[2] = {a.ag, b.ag};
    setenv("FSDP_FAULT", "launch@3", 1);
    const long l0 = harness::launches;
    CHECK_STATUS(fsdp_step_groups(plans, 2, rs, ag_in, ag_out, &kHp, 1, 0, 0, nullptr, nullptr),
                 FSDP_E_HIP);
    CHECK(std::strstr(fsdp_last_error(), "group 1") != nullptr &&
              std::strstr(fsdp_last_error(), "injected") != nullptr,
          "message: %s", fsdp_last_error());
    CHECK(harness::launches == l0 + 2, "%s: %ld launches before the fault, wanted 2",
          w.name.c_str(), harness::launches - l0);
    unsetenv("FSDP_FAULT");
    CHECK_STATUS(fsdp_pack_allgather(a.plan, a.ag_in(), nullptr), FSDP_OK);
    CHECK(std::strstr(fsdp_last_error(), "injected") != nullptr,
          "the last error stays until the next failure");
}

void error_paths(const Workload &w, Instance &in) {
    fsdp_plan *p = in.plan;
    const int64_t S = in.info.S;
    CHECK_STATUS(fsdp_adamw_shard(p, nullptr, 1, nullptr), FSDP_E_INVAL);
    CHECK_STATUS(fsdp_adamw_shard(p, &kHp, 0, nullptr), FSDP_E_INVAL);
    CHECK_STATUS(fsdp_step_shard(p, in.rs, in.ag_in(), &kHp, 1, 4u, nullptr), FSDP_E_INVAL);
    CHECK_STATUS(fsdp_pack_reduce_scatter(p, in.rs, 7, nullptr), FSDP_E_UNSUPPORTED);
    CHECK_STATUS(fsdp_plan_entry(p, int32_t(in.ents.size()), nullptr), FSDP_E_INVAL);
    fsdp_shard_entry_t e;
    CHECK_STATUS(fsdp_plan_entry(p, -1, &e), FSDP_E_INVAL);
    int64_t b, lr;
    CHECK_STATUS(fsdp_plan_rows_of_rank(p, 0, in.info.world, &b, &lr), FSDP_E_INVAL);
    if (S > 0) {
        CHECK_STATUS(fsdp_pack_allgather(p, nullptr, nullptr), FSDP_E_INVAL);
        CHECK_STATUS(fsdp_unpack_allgather(p, reinterpret_cast<const uint16_t *>(
                                                  reinterpret_cast<const char *>(in.ag) + 1),
                                           nullptr),
                     FSDP_E_ALIGN);
        // ag_in inside rs_in
        CHECK_STATUS(fsdp_step_shard(p, in.rs, in.rs, &kHp, 1, 0, nullptr), FSDP_E_INVAL);
        CHECK_STATUS(fsdp_reduce_shard_f32(p, reinterpret_cast<const float *>(in.rs + 1), nullptr),
                     FSDP_E_ALIGN);
    }
    // a rejected bind keeps the previous binding
    std::vector<float *> bad = in.master;
    for (size_t i = 0; i < bad.size(); ++i) {
        if (in.ents[i].valid_numel == 0) continue;
        bad[i] = reinterpret_cast<float *>(reinterpret_cast<char *>(bad[i]) + 2);
        CHECK_STATUS(fsdp_bind(p, bad.data(), nullptr, nullptr, nullptr, nullptr, nullptr),
                     FSDP_E_ALIGN);
        bad[i] = nullptr;
        CHECK_STATUS(fsdp_bind(p, bad.data(), nullptr, nullptr, nullptr, nullptr, nullptr),
                     FSDP_E_INVAL);
        break;
    }
    CHECK_STATUS(fsdp_adamw_shard(p, &kHp, 1, nullptr), FSDP_OK);
    (void)w;
}

void reshard(const Workload &w) {
    const int32_t n = static_cast<int32_t>(w.rows.size());
    const int32_t pairs[][2] = {{w.world, 1}, {1, w.world}, {w.world, w.world + 1},
                                {w.world + 2, std::max(1, w.world / 2)}};
    for (const auto &pr : pairs) {
        const int32_t n1 = pr[0], n2 = pr[1];
        for (int32_t rd : {0, n2 - 1}) {
            fsdp_reshard_plan *rp = nullptr;
            CHECK_STATUS(fsdp_reshard_plan_create(w.rows.data(), w.cols.data(), n, n1, n2, rd, &rp),
                         FSDP_OK);
            if (rp == nullptr) continue;
            int64_t runs = 0, dnum = 0;
            CHECK_STATUS(fsdp_reshard_plan_runs(rp, &runs, &dnum), FSDP_OK);
            int64_t want = 0;
            for (int32_t i = 0; i < n; ++i) {
                int64_t b, lr;
                rows_of(w.rows[i], n2, rd, &b, &lr);
                want += lr * w.cols[i];
            }
            CHECK(dnum == want, "%s reshard %d->%d: %lld target elements, wanted %lld",
                  w.name.c_str(), n1, n2, (long long)dnum, (long long)want);
            for (int elem : {2, 4}) {
                std::vector<const void *> src(static_cast<size_t>(n) * n1, nullptr);
                std::vector<void *> dst(n, nullptr);
                std::vector<int64_t> dlen(n, 0);
                for (int32_t i = 0; i < n; ++i) {
                    for (int32_t s = 0; s < n1; ++s) {
                        int64_t b, lr;
                        rows_of(w.rows[i], n1, s, &b, &lr);
                        src[size_t(i) * n1 + s] = alloc<char>(lr * w.cols[i] * elem);
                    }
                    int64_t b, lr;
                    rows_of(w.rows[i], n2, rd, &b, &lr);
                    dlen[i] = lr * w.cols[i];
                    dst[i] = alloc<char>(dlen[i] * elem);
                }
                CHECK_STATUS(fsdp_reshard_bind(rp, src.data(), dst.data(), elem, nullptr), FSDP_OK);
                harness::spans.clear();
                CHECK_STATUS(fsdp_reshard_execute(rp, nullptr), FSDP_OK);
                // Copy tiles hold absolute addresses in 2-byte units: map each
                // written span back to the target shard that contains it.
                std::vector<std::vector<uint8_t>> hits(n);
                for (int32_t i = 0; i < n; ++i) hits[i].assign(dlen[i] * elem / 2, 0);
                int64_t stray = 0;
                for (const harness::Span &sp : harness::spans) {
                    bool placed = false;
                    for (int32_t i = 0; i < n && !placed; ++i) {
                        if (dst[i] == nullptr) continue;
                        const intptr_t d = static_cast<const char *>(sp.base) -
                                           static_cast<const char *>(dst[i]);
                        const int64_t units = int64_t(hits[i].size());
                        if (d < 0 || d % 2 != 0 || d / 2 >= units) continue;
                        placed = true;
                        if (d / 2 + sp.off + sp.len > units) {
                            ++stray;
                            continue;
                        }
                        for (int64_t u = d / 2 + sp.off; u < d / 2 + sp.off + sp.len; ++u)
                            if (hits[i][u] < 2) ++hits[i][u];
                    }
                    stray += !placed;
                }
                int64_t bad = 0;
                for (const auto &h : hits)
                    for (uint8_t x : h) bad += x != 1;
                CHECK(stray == 0 && bad == 0,
                      "%s reshard %d->%d rank %d elem %d: %lld stray runs, %lld units not "
                      "written exactly once",
                      w.name.c_str(), n1, n2, rd, elem, (long long)stray, (long long)bad);
                setenv("FSDP_FAULT", "launch", 1);
                CHECK_STATUS(fsdp_reshard_execute(rp, nullptr), FSDP_E_HIP);
                unsetenv("FSDP_FAULT");
            }
            CHECK_STATUS(fsdp_reshard_bind(rp, nullptr, nullptr, 3, nullptr), FSDP_E_INVAL);
            fsdp_reshard_plan_destroy(rp);
        }
    }
}

void host_adamw() {
    const int64_t n = 4099;
    std::vector<float> p(n, 0.01f), g(n, 1e-3f), m(n, 0.f), v(n, 0.f);
    for (int32_t threads : {1, 3, 0})
        CHECK_STATUS(fsdp_adamw_host(p.data(), g.data(), m.data(), v.data(), n, &kHp, 1, threads),
                     FSDP_OK);
    CHECK_STATUS(fsdp_adamw_host(p.data(), g.data(), m.data(), v.data(), -1, &kHp, 1, 1),
                 FSDP_E_INVAL);
    CHECK_STATUS(fsdp_adamw_host(nullptr, g.data(), m.data(), v.data(), n, &kHp, 1, 1),
                 FSDP_E_INVAL);
    CHECK_STATUS(fsdp_adamw_host(p.data(), g.data(), m.data(), v.data(), n, &kHp, 0, 1),
                 FSDP_E_INVAL);
}

void planner_errors() {
    fsdp_plan *p = nullptr;
    const int64_t r[2] = {4, 3}, c[2] = {2, 1}, neg[1] = {-1}, big_r[1] = {int64_t(1) << 62},
                  big_c[1] = {int64_t(1) << 10};
    CHECK_STATUS(fsdp_plan_create(r, c, 2, 0, 0, 1, &p), FSDP_E_INVAL);
    CHECK_STATUS(fsdp_plan_create(r, c, 2, 2, 2, 1, &p), FSDP_E_INVAL);
    CHECK_STATUS(fsdp_plan_create(r, c, 2, 2, 0, 4, &p), FSDP_E_UNSUPPORTED);
    CHECK_STATUS(fsdp_plan_create(neg, c, 1, 2, 0, 1, &p), FSDP_E_INVAL);
    CHECK_STATUS(fsdp_plan_create(big_r, big_c, 1, 2, 0, 1, &p), FSDP_E_INVAL);
    CHECK_STATUS(fsdp_plan_create(nullptr, c, 2, 2, 0, 1, &p), FSDP_E_INVAL);
    CHECK_STATUS(fsdp_plan_create(r, c, 2, 2, 0, 1, nullptr), FSDP_E_INVAL);
    double bytes = 0;
    CHECK_STATUS(fsdp_state_bytes(7e9, 8, 3, &bytes), FSDP_OK);
    CHECK(bytes == 14e9, "state bytes %g", bytes);
    CHECK_STATUS(fsdp_state_bytes(7e9, 8, 4, &bytes), FSDP_E_UNSUPPORTED);
    fsdp_plan_destroy(nullptr);
}

}  // namespace

int main() {
    planner_errors();
    host_adamw();
    std::string line;
    int count = 0;
    while (std::getline(std::cin, line)) {
        std::istringstream ss(line);
        Workload w;
        int32_t n = 0;
        if (!(ss >> w.name >> w.world >> w.rank >> w.align >> n)) continue;
        for (int32_t i = 0; i < n; ++i) {
            int64_t r = 0, c = 0;
            ss >> r >> c;
            w.rows.push_back(r);
            w.cols.push_back(c);
        }
        Instance a, b;
        if (!make(w, &a) || !make(w, &b)) return 1;
        CHECK_STATUS(fsdp_pack_allgather(a.plan, a.ag_in(), nullptr), FSDP_E_STATE);
        bind_all(&a);
        bind_all(&b);
        hot_calls(w, a);
        executor(w, a, b);
        group_sets(w, a, b);
        faults(w, a, b);
        error_paths(w, a);
        reshard(w);
        fsdp_plan_destroy(a.plan);
        fsdp_plan_destroy(b.plan);
        for (void *q : g_allocs) std::free(q);
        g_allocs.clear();
        ++count;
        std::printf("workload %s ok (N=%d rank=%d align=%d, %d params)\n", w.name.c_str(), w.world,
                    w.rank, w.align, n);
    }
    if (g_failures == 0 && count > 0) std::printf("ALL OK (%d workloads)\n", count);
    return g_failures == 0 && count > 0 ? 0 : 1;
}
