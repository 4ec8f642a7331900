// C ABI of the sharded-step library: argument checks, device tables, launches.
//
// Every exported function validates its arguments on the host before any HIP
// call, so the error paths can be exercised without a GPU.  Hot calls only
// enqueue kernels on the caller's stream.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/fsdp_shard.h"
#include "launch.hpp"
#include "plan.hpp"


struct fsdp_plan {
    fsdp::Layout L;
    std::vector<fsdp::DevEntry> host_entries;
    int32_t bound = 0;
    int device = -1;
    bool tiles_uploaded = false;  // the tile tables below hold the plan's tiles
    char *dmem = nullptr;  // one device block: entries, then the tile tables
    fsdp::DevEntry *d_entries = nullptr;
    fsdp::PackTile *d_pack = nullptr;
    fsdp::PackTile *d_rspack = nullptr;
    fsdp::UnpackTile *d_unpack = nullptr;
    fsdp::ReduceTile *d_reduce = nullptr;
    fsdp::EwTile *d_adamw = nullptr;
    fsdp::EwTile *d_full = nullptr;
};

// Bound plans whose AdamW and copy-in run as one launch each: the plans'
// entry records concatenated (group g's entries from ent_off[g]) and their
// AdamW and copy-in tiles re-indexed into that table and into one copy-in
// arena (group g's segment from seg_off[g]).  Built once; it borrows the
// plans and is valid while their AdamW tensors stay bound as they were.
struct fsdp_group_set {
    std::vector<fsdp_plan *> plans;
    std::vector<int64_t> ent_off, seg_off;  // n_groups + 1 prefix offsets
    std::vector<fsdp::DevEntry> snapshot;   // concatenated entries at creation
    std::vector<std::pair<uintptr_t, uintptr_t>> shard_bytes;  // union of the shard tensors
    int device = -1;
    char *dmem = nullptr;
    fsdp::DevEntry *d_entries = nullptr;
    fsdp::PackTile *d_pack = nullptr;
    fsdp::EwTile *d_adamw = nullptr;
    int64_t n_pack = 0, n_adamw = 0;
};

namespace {

thread_local std::string g_last_error;
thread_local bool g_fault_injected = false;

fsdp_status fail(fsdp_status s, const std::string &msg) {
    g_last_error = msg;
    return s;
}

fsdp_status hip_fail(hipError_t e, const char *what) {
    std::string msg = std::string(what) + ": " + hipGetErrorString(e);
    if (g_fault_injected) msg += " (injected by FSDP_FAULT)";
    g_fault_injected = false;
    return fail(FSDP_E_HIP, msg);
}

bool misaligned(const void *p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0;
}

size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// AdamW scalars: fp64 arithmetic on the hyperparameters, each rounded once
// to fp32 (beta1, 1-beta1, beta2, 1-beta2, eps, 1-lr*wd, lr/(1-beta1^t),
// sqrt(1-beta2^t)).
void adamw_scalars(const fsdp_adamw_hparams_t *hp, int64_t step, float out[8]) {
    const double bc1 = 1.0 - std::pow(hp->beta1, static_cast<double>(step));
    const double bc2 = 1.0 - std::pow(hp->beta2, static_cast<double>(step));
    out[0] = static_cast<float>(hp->beta1);
    out[1] = static_cast<float>(1.0 - hp->beta1);
    out[2] = static_cast<float>(hp->beta2);
    out[3] = static_cast<float>(1.0 - hp->beta2);
    out[4] = static_cast<float>(hp->eps);
    out[5] = static_cast<float>(1.0 - hp->lr * hp->weight_decay);
    out[6] = static_cast<float>(hp->lr / bc1);
    out[7] = static_cast<float>(std::pow(bc2, 0.5));
}

// Hot calls run on the device the tables live on.
fsdp_status check_device(const fsdp_plan *p) {
    int d = -1;
    hipError_t e = hipGetDevice(&d);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (d != p->device)
        return fail(FSDP_E_STATE, "current device " + std::to_string(d) +
                                      " differs from the bound device " +
                                      std::to_string(p->device));
    return FSDP_OK;
}

fsdp_status need_roles(const fsdp_plan *p, int32_t roles, const char *call) {
    if (p == nullptr) return fail(FSDP_E_INVAL, std::string(call) + ": null plan");
    if ((p->bound & roles) != roles || p->dmem == nullptr)
        return fail(FSDP_E_STATE, std::string(call) + ": the tensors it needs are not bound");
    return FSDP_OK;
}

// Upload the entry table (and, until one upload has succeeded, the tile
// tables; the device block is allocated the first time) on `st`, then record
// the newly bound roles.
fsdp_status commit_entries(fsdp_plan *p, std::vector<fsdp::DevEntry> ents, int32_t roles,
                           hipStream_t st, const char *call) {
    const std::string c(call);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, (c + ": hipGetDevice").c_str());
    if (p->dmem != nullptr && dev != p->device)
        return fail(FSDP_E_STATE, c + ": plan already bound on another device");
    const size_t n = p->L.entries.size();
    struct Table {
        void **dst;
        const void *src;
        size_t bytes;
    } tabs[7] = {
        {reinterpret_cast<void **>(&p->d_entries), nullptr, n * sizeof(fsdp::DevEntry)},
        {reinterpret_cast<void **>(&p->d_pack), p->L.pack.data(),
         p->L.pack.size() * sizeof(fsdp::PackTile)},
        {reinterpret_cast<void **>(&p->d_rspack), p->L.rspack.data(),
         p->L.rspack.size() * sizeof(fsdp::PackTile)},
        {reinterpret_cast<void **>(&p->d_unpack), p->L.unpack.data(),
         p->L.unpack.size() * sizeof(fsdp::UnpackTile)},
        {reinterpret_cast<void **>(&p->d_reduce), p->L.reduce.data(),
         p->L.reduce.size() * sizeof(fsdp::ReduceTile)},
        {reinterpret_cast<void **>(&p->d_adamw), p->L.adamw.data(),
         p->L.adamw.size() * sizeof(fsdp::EwTile)},
        {reinterpret_cast<void **>(&p->d_full), p->L.full.data(),
         p->L.full.size() * sizeof(fsdp::EwTile)},
    };
    const bool first = p->dmem == nullptr;
    if (first) {
        size_t total = 256;
        for (const Table &t : tabs) total += round256(t.bytes);
        void *mem = nullptr;
        e = hipMalloc(&mem, total);
        if (e != hipSuccess) return fail(FSDP_E_NOMEM, c + ": hipMalloc of device tables failed");
        p->dmem = static_cast<char *>(mem);
        p->device = dev;
        char *cur = p->dmem;
        for (const Table &t : tabs) {
            *t.dst = cur;
            cur += round256(t.bytes);
        }
    }
    // Kernels of this plan still queued on the stream may read the tables.
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, (c + ": hipStreamSynchronize").c_str());
    // From here the device tables change: a failure leaves the plan unbound
    // (hot calls then fail with FSDP_E_STATE) rather than half-updated.
    const int32_t prev = p->bound;
    p->bound = 0;
    const int n_tabs = p->tiles_uploaded ? 1 : 7;
    for (int k = 0; k < n_tabs; ++k) {
        if (tabs[k].bytes == 0) continue;
        const void *src = k == 0 ? static_cast<const void *>(ents.data()) : tabs[k].src;
        e = hipMemcpyAsync(*tabs[k].dst, src, tabs[k].bytes, hipMemcpyHostToDevice, st);
        if (e != hipSuccess) return hip_fail(e, (c + ": hipMemcpyAsync").c_str());
    }
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, (c + ": upload").c_str());
    p->tiles_uploaded = true;
    p->host_entries = std::move(ents);
    p->bound = prev | roles;
    return FSDP_OK;
}

}  // namespace

namespace fsdp {
// Error reporting and AdamW scalars shared with the other translation units.
fsdp_status set_error(fsdp_status s, const std::string &msg) { return fail(s, msg); }
fsdp_status set_hip_error(hipError_t e, const char *what) { return hip_fail(e, what); }

// Fault injection, to test how callers see a failed launch without breaking a
// kernel.  With FSDP_FAULT=launch in the environment every library launch
// (one per hot call, one per kernel of fsdp_step_groups) fails with
// hipErrorLaunchFailure before anything is enqueued; FSDP_FAULT=launch@K
// fails only the K-th launch counted from when a launch first sees that
// value (a launch that sees the variable unset or changed restarts the
// count).  Unset, it costs one getenv per launch.
hipError_t injected_fault() {
    static std::mutex mu;
    static std::string seen;
    static long count = 0;
    static std::atomic<bool> counting{false};
    const char *f = std::getenv("FSDP_FAULT");
    const bool at = f != nullptr && std::strncmp(f, "launch@", 7) == 0;
    if (!at) {
        if (counting.load(std::memory_order_relaxed)) {
            std::lock_guard<std::mutex> lock(mu);
            seen.clear();
            count = 0;
            counting.store(false, std::memory_order_relaxed);
        }
        if (f == nullptr || std::strcmp(f, "launch") != 0) return hipSuccess;
        g_fault_injected = true;
        return hipErrorLaunchFailure;
    }
    std::lock_guard<std::mutex> lock(mu);
    counting.store(true, std::memory_order_relaxed);
    if (seen != f) {
        seen = f;
        count = 0;
    }
    if (++count != std::strtol(f + 7, nullptr, 10)) return hipSuccess;
    g_fault_injected = true;
    return hipErrorLaunchFailure;
}
void adamw_scalars_host(const fsdp_adamw_hparams_t *hp, int64_t step, float out[8]) {
    adamw_scalars(hp, step, out);
}
}  // namespace fsdp

extern "C" {

int32_t fsdp_abi_version(void) { return FSDP_ABI_VERSION; }

const char *fsdp_status_string(fsdp_status s) {
    switch (s) {
        case FSDP_OK: return "ok";
        case FSDP_E_INVAL: return "invalid argument";
        case FSDP_E_UNSUPPORTED: return "unsupported option";
        case FSDP_E_ALIGN: return "misaligned pointer";
        case FSDP_E_STATE: return "plan not bound for this call or device";
        case FSDP_E_HIP: return "HIP runtime error";
        case FSDP_E_NOMEM: return "out of memory";
        default: return "unknown status";
    }
}

const char *fsdp_last_error(void) { return g_last_error.c_str(); }

fsdp_status fsdp_plan_create(const int64_t *rows, const int64_t *cols,
                             int32_t n_params, int32_t world, int32_t rank,
                             int32_t align_elems, fsdp_plan **out) {
    if (out == nullptr) return fail(FSDP_E_INVAL, "fsdp_plan_create: null out");
    *out = nullptr;
    try {
        fsdp_plan *p = new fsdp_plan();
        std::string err;
        fsdp_status s = fsdp::build_layout(rows, cols, n_params, world, rank,
                                           align_elems, &p->L, &err);
        if (s != FSDP_OK) {
            delete p;
            return fail(s, "fsdp_plan_create: " + err);
        }
        p->host_entries.assign(static_cast<size_t>(n_params), fsdp::DevEntry{});
        *out = p;
        return FSDP_OK;
    } catch (const std::bad_alloc &) {
        return fail(FSDP_E_NOMEM, "fsdp_plan_create: host allocation failed");
    } catch (...) {
        return fail(FSDP_E_INVAL, "fsdp_plan_create: unexpected failure");
    }
}

fsdp_status fsdp_plan_info(const fsdp_plan *p, fsdp_plan_info_t *out) {
    if (p == nullptr || out == nullptr) return fail(FSDP_E_INVAL, "fsdp_plan_info: null argument");
    std::memset(out, 0, sizeof(*out));
    out->n_params = static_cast<int32_t>(p->L.entries.size());
    out->world = p->L.world;
    out->rank = p->L.rank;
    out->align_elems = p->L.align;
    out->S = p->L.S;
    out->V = p->L.V;
    out->F = p->L.F;
    out->pad_total = p->L.S - p->L.V;
    out->n_empty = p->L.n_empty;
    out->bound = p->bound;
    out->n_tiles[0] = static_cast<int64_t>(p->L.pack.size());
    out->n_tiles[1] = static_cast<int64_t>(p->L.unpack.size());
    out->n_tiles[2] = static_cast<int64_t>(p->L.reduce.size());
    out->n_tiles[3] = static_cast<int64_t>(p->L.adamw.size());
    return FSDP_OK;
}

fsdp_status fsdp_plan_entry(const fsdp_plan *p, int32_t i, fsdp_shard_entry_t *out) {
    if (p == nullptr || out == nullptr) return fail(FSDP_E_INVAL, "fsdp_plan_entry: null argument");
    if (i < 0 || static_cast<size_t>(i) >= p->L.entries.size())
        return fail(FSDP_E_INVAL, "fsdp_plan_entry: index out of range");
    *out = p->L.entries[i];
    return FSDP_OK;
}

fsdp_status fsdp_plan_rows_of_rank(const fsdp_plan *p, int32_t i, int32_t j,
                                   int64_t *row_begin, int64_t *local_rows) {
    if (p == nullptr || row_begin == nullptr || local_rows == nullptr)
        return fail(FSDP_E_INVAL, "fsdp_plan_rows_of_rank: null argument");
    if (i < 0 || static_cast<size_t>(i) >= p->L.entries.size())
        return fail(FSDP_E_INVAL, "fsdp_plan_rows_of_rank: parameter index out of range");
    if (j < 0 || j >= p->L.world)
        return fail(FSDP_E_INVAL, "fsdp_plan_rows_of_rank: rank out of range");
    fsdp::rows_of_rank(p->L.entries[i].rows, p->L.world, j, row_begin, local_rows);
    return FSDP_OK;
}

fsdp_status fsdp_state_bytes(double n_params, int32_t world, int32_t zero_stage,
                             double *per_rank_bytes) {
    if (per_rank_bytes == nullptr || world < 1 || !(n_params >= 0.0))
        return fail(FSDP_E_INVAL, "fsdp_state_bytes: need n_params >= 0, world >= 1, non-null out");
    if (zero_stage < 0 || zero_stage > 3)
        return fail(FSDP_E_UNSUPPORTED, "fsdp_state_bytes: zero_stage must be 0..3");
    double params = 2.0 * n_params, grads = 2.0 * n_params, optim = 12.0 * n_params;
    if (zero_stage >= 1) optim /= world;
    if (zero_stage >= 2) grads /= world;
    if (zero_stage >= 3) params /= world;
    *per_rank_bytes = params + grads + optim;
    return FSDP_OK;
}

void fsdp_plan_destroy(fsdp_plan *p) {
    if (p == nullptr) return;
    if (p->dmem != nullptr) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(p->device);
        (void)hipDeviceSynchronize();
        (void)hipFree(p->dmem);
        if (cur >= 0) (void)hipSetDevice(cur);
    }
    delete p;
}

fsdp_status fsdp_bind(fsdp_plan *p, float *const *master, float *const *grad,
                      float *const *exp_avg, float *const *exp_avg_sq,
                      uint16_t *const *full, void *stream) {
    if (p == nullptr) return fail(FSDP_E_INVAL, "fsdp_bind: null plan");
    const size_t n = p->L.entries.size();
    std::vector<fsdp::DevEntry> ents = p->host_entries;
    int32_t roles = 0;
    struct RoleArr {
        float *const *arr;
        int32_t bit;
        const char *name;
    } fr[4] = {{master, FSDP_ROLE_MASTER, "master"},
               {grad, FSDP_ROLE_GRAD, "grad"},
               {exp_avg, FSDP_ROLE_EXP_AVG, "exp_avg"},
               {exp_avg_sq, FSDP_ROLE_EXP_AVG_SQ, "exp_avg_sq"}};
    for (const RoleArr &r : fr) {
        if (r.arr == nullptr) continue;
        roles |= r.bit;
        for (size_t i = 0; i < n; ++i) {
            float *q = r.arr[i];
            if (q == nullptr && p->L.entries[i].valid_numel > 0)
                return fail(FSDP_E_INVAL, std::string("fsdp_bind: null ") + r.name +
                                              " pointer for parameter " + std::to_string(i));
            if (misaligned(q, 4))
                return fail(FSDP_E_ALIGN, std::string("fsdp_bind: ") + r.name +
                                              " pointer of parameter " + std::to_string(i) +
                                              " is not 4-byte aligned");
            float **slot = r.bit == FSDP_ROLE_MASTER   ? &ents[i].master
                           : r.bit == FSDP_ROLE_GRAD    ? &ents[i].grad
                           : r.bit == FSDP_ROLE_EXP_AVG ? &ents[i].exp_avg
                                                        : &ents[i].exp_avg_sq;
            *slot = q;
        }
    }
    if (full != nullptr) {
        roles |= FSDP_ROLE_FULL;
        for (size_t i = 0; i < n; ++i) {
            const fsdp_shard_entry_t &e = p->L.entries[i];
            if (full[i] == nullptr && e.rows * e.cols > 0)
                return fail(FSDP_E_INVAL, "fsdp_bind: null full pointer for parameter " +
                                              std::to_string(i));
            if (misaligned(full[i], 2))
                return fail(FSDP_E_ALIGN, "fsdp_bind: full pointer of parameter " +
                                              std::to_string(i) + " is not 2-byte aligned");
            ents[i].full = full[i];
        }
    }
    return commit_entries(p, std::move(ents), roles, static_cast<hipStream_t>(stream),
                          "fsdp_bind");
}

fsdp_status fsdp_bind_full_fp8(fsdp_plan *p, uint8_t *const *full_fp8, void *stream) {
    if (p == nullptr || full_fp8 == nullptr)
        return fail(FSDP_E_INVAL, "fsdp_bind_full_fp8: null plan or array");
    std::vector<fsdp::DevEntry> ents = p->host_entries;
    for (size_t i = 0; i < ents.size(); ++i) {
        const fsdp_shard_entry_t &e = p->L.entries[i];
        if (full_fp8[i] == nullptr && e.rows * e.cols > 0)
            return fail(FSDP_E_INVAL, "fsdp_bind_full_fp8: null pointer for parameter " +
                                          std::to_string(i));
        ents[i].full_fp8 = full_fp8[i];
    }
    return commit_entries(p, std::move(ents), FSDP_ROLE_FULL_FP8,
                          static_cast<hipStream_t>(stream), "fsdp_bind_full_fp8");
}

fsdp_status fsdp_bind_grad_acc(fsdp_plan *p, float *const *grad_acc, void *stream) {
    if (p == nullptr || grad_acc == nullptr)
        return fail(FSDP_E_INVAL, "fsdp_bind_grad_acc: null plan or array");
    std::vector<fsdp::DevEntry> ents = p->host_entries;
    for (size_t i = 0; i < ents.size(); ++i) {
        const fsdp_shard_entry_t &e = p->L.entries[i];
        if (grad_acc[i] == nullptr && e.rows * e.cols > 0)
            return fail(FSDP_E_INVAL, "fsdp_bind_grad_acc: null pointer for parameter " +
                                          std::to_string(i));
        if (misaligned(grad_acc[i], 4))
            return fail(FSDP_E_ALIGN, "fsdp_bind_grad_acc: pointer of parameter " +
                                          std::to_string(i) + " is not 4-byte aligned");
        ents[i].grad_acc = grad_acc[i];
    }
    return commit_entries(p, std::move(ents), FSDP_ROLE_GRAD_ACC,
                          static_cast<hipStream_t>(stream), "fsdp_bind_grad_acc");
}

fsdp_status fsdp_bind_full_grad(fsdp_plan *p, uint16_t *const *full_grad, void *stream) {
    if (p == nullptr || full_grad == nullptr)
        return fail(FSDP_E_INVAL, "fsdp_bind_full_grad: null plan or array");
    std::vector<fsdp::DevEntry> ents = p->host_entries;
    for (size_t i = 0; i < ents.size(); ++i) {
        const fsdp_shard_entry_t &e = p->L.entries[i];
        if (full_grad[i] == nullptr && e.rows * e.cols > 0)
            return fail(FSDP_E_INVAL, "fsdp_bind_full_grad: null pointer for parameter " +
                                          std::to_string(i));
        if (misaligned(full_grad[i], 2))
            return fail(FSDP_E_ALIGN, "fsdp_bind_full_grad: pointer of parameter " +
                                          std::to_string(i) + " is not 2-byte aligned");
        ents[i].full_grad = full_grad[i];
    }
    return commit_entries(p, std::move(ents), FSDP_ROLE_FULL_GRAD,
                          static_cast<hipStream_t>(stream), "fsdp_bind_full_grad");
}

}  // extern "C"

// ---- hot path: host-side checks (no HIP call), then launches ----------------

namespace {

constexpr int32_t kAdamwRoles =
    FSDP_ROLE_MASTER | FSDP_ROLE_GRAD | FSDP_ROLE_EXP_AVG | FSDP_ROLE_EXP_AVG_SQ;

fsdp_status check_buf(const fsdp_plan *p, const void *buf, const char *call, const char *name) {
    if (buf == nullptr && p->L.S > 0)
        return fail(FSDP_E_INVAL, std::string(call) + ": null " + name);
    if (misaligned(buf, 2))
        return fail(FSDP_E_ALIGN, std::string(call) + ": " + name + " not 2-byte aligned");
    return FSDP_OK;
}

fsdp_status check_pack(const fsdp_plan *p, const uint16_t *ag_in, const char *call) {
    fsdp_status s = need_roles(p, FSDP_ROLE_MASTER, call);
    return s != FSDP_OK ? s : check_buf(p, ag_in, call, "ag_in");
}

fsdp_status check_unpack(const fsdp_plan *p, const uint16_t *ag_out, const char *call) {
    fsdp_status s = need_roles(p, FSDP_ROLE_FULL, call);
    return s != FSDP_OK ? s : check_buf(p, ag_out, call, "ag_out");
}

fsdp_status check_reduce(const fsdp_plan *p, const uint16_t *rs_in, const char *call) {
    fsdp_status s = need_roles(p, FSDP_ROLE_GRAD, call);
    return s != FSDP_OK ? s : check_buf(p, rs_in, call, "rs_in");
}

fsdp_status check_hparams(const fsdp_adamw_hparams_t *hp, int64_t step, const char *call) {
    if (hp == nullptr) return fail(FSDP_E_INVAL, std::string(call) + ": null hyperparameters");
    if (step < 1) return fail(FSDP_E_INVAL, std::string(call) + ": step counts from 1");
    return FSDP_OK;
}

fsdp_status check_step(const fsdp_plan *p, const uint16_t *rs_in, const uint16_t *ag_in,
                       bool write_grad, const char *call) {
    const int32_t roles = FSDP_ROLE_MASTER | FSDP_ROLE_EXP_AVG | FSDP_ROLE_EXP_AVG_SQ |
                          (write_grad ? FSDP_ROLE_GRAD : 0);
    fsdp_status s = need_roles(p, roles, call);
    if (s != FSDP_OK) return s;
    if ((s = check_buf(p, rs_in, call, "rs_in")) != FSDP_OK) return s;
    if ((s = check_buf(p, ag_in, call, "ag_in")) != FSDP_OK) return s;
    // ag_in is written while rs_in is read: the two must not share bytes
    const uintptr_t r0 = reinterpret_cast<uintptr_t>(rs_in);
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(ag_in);
    const uintptr_t rb = static_cast<uintptr_t>(p->L.world) * static_cast<uintptr_t>(p->L.S) * 2;
    const uintptr_t ab = static_cast<uintptr_t>(p->L.S) * 2;
    if (p->L.S > 0 && a0 < r0 + rb && r0 < a0 + ab)
        return fail(FSDP_E_INVAL, std::string(call) + ": ag_in overlaps rs_in");
    return FSDP_OK;
}

// Runs one library launch unless a fault is injected in its place.
template <typename F>
hipError_t guarded(F &&launch) {
    const hipError_t e = fsdp::injected_fault();
    return e != hipSuccess ? e : launch();
}

hipError_t do_pack(const fsdp_plan *p, uint16_t *ag_in, hipStream_t st) {
    return guarded([&] {
        return fsdp::launch_pack(p->d_pack, static_cast<int64_t>(p->L.pack.size()), p->d_entries,
                                 ag_in, st);
    });
}

// Every row piece starts 16-byte aligned: the offsets allow it and the
// [N, S] buffer itself is 16-byte aligned.
bool chunk_aligned(const fsdp_plan *p, const void *rows) {
    return p->L.offsets8 && (reinterpret_cast<uintptr_t>(rows) & 15u) == 0;
}

hipError_t do_unpack(const fsdp_plan *p, const uint16_t *ag_out, hipStream_t st) {
    return guarded([&] {
        return fsdp::launch_unpack(p->d_unpack, static_cast<int64_t>(p->L.unpack.size()),
                                   p->d_entries, ag_out, chunk_aligned(p, ag_out), st);
    });
}

hipError_t do_reduce(const fsdp_plan *p, const uint16_t *rs_in, hipStream_t st) {
    return guarded([&] {
        return fsdp::launch_reduce(p->d_reduce, static_cast<int64_t>(p->L.reduce.size()),
                                   p->d_entries, rs_in, p->L.S, p->L.world,
                                   chunk_aligned(p, rs_in), st);
    });
}

hipError_t do_adamw(const fsdp_plan *p, const float scal[8], hipStream_t st) {
    return guarded([&] {
        return fsdp::launch_adamw(p->d_adamw, static_cast<int64_t>(p->L.adamw.size()),
                                  p->d_entries, scal, false, st);
    });
}

hipError_t do_step(const fsdp_plan *p, const uint16_t *rs_in, uint16_t *ag_in,
                   const float scal[8], bool write_grad, hipStream_t st) {
    return guarded([&] {
        return fsdp::launch_step(p->d_pack, static_cast<int64_t>(p->L.pack.size()), p->d_entries,
                                 rs_in, ag_in, p->L.S, p->L.world, scal, write_grad,
                                 chunk_aligned(p, rs_in), st);
    });
}

fsdp_status launched(hipError_t e, const char *call) {
    return e == hipSuccess ? FSDP_OK : hip_fail(e, call);
}

}  // namespace

extern "C" {

fsdp_status fsdp_pack_allgather(const fsdp_plan *p, uint16_t *ag_in, void *stream) {
    fsdp_status s = check_pack(p, ag_in, "fsdp_pack_allgather");
    if (s != FSDP_OK || (s = check_device(p)) != FSDP_OK) return s;
    return launched(do_pack(p, ag_in, static_cast<hipStream_t>(stream)),
                    "fsdp_pack_allgather: launch");
}

fsdp_status fsdp_unpack_allgather(const fsdp_plan *p, const uint16_t *ag_out, void *stream) {
    fsdp_status s = check_unpack(p, ag_out, "fsdp_unpack_allgather");
    if (s != FSDP_OK || (s = check_device(p)) != FSDP_OK) return s;
    return launched(do_unpack(p, ag_out, static_cast<hipStream_t>(stream)),
                    "fsdp_unpack_allgather: launch");
}

fsdp_status fsdp_reduce_shard(const fsdp_plan *p, const uint16_t *rs_in, void *stream) {
    fsdp_status s = check_reduce(p, rs_in, "fsdp_reduce_shard");
    if (s != FSDP_OK || (s = check_device(p)) != FSDP_OK) return s;
    return launched(do_reduce(p, rs_in, static_cast<hipStream_t>(stream)),
                    "fsdp_reduce_shard: launch");
}

fsdp_status fsdp_adamw_shard(const fsdp_plan *p, const fsdp_adamw_hparams_t *hp,
                             int64_t step, void *stream) {
    fsdp_status s = need_roles(p, kAdamwRoles, "fsdp_adamw_shard");
    if (s != FSDP_OK || (s = check_hparams(hp, step, "fsdp_adamw_shard")) != FSDP_OK ||
        (s = check_device(p)) != FSDP_OK)
        return s;
    float scal[8];
    adamw_scalars(hp, step, scal);
    return launched(do_adamw(p, scal, static_cast<hipStream_t>(stream)),
                    "fsdp_adamw_shard: launch");
}

fsdp_status fsdp_step_shard(const fsdp_plan *p, const uint16_t *rs_in, uint16_t *ag_in,
                            const fsdp_adamw_hparams_t *hp, int64_t step, uint32_t flags,
                            void *stream) {
    const char *call = "fsdp_step_shard";
    const bool write_grad = (flags & FSDP_STEP_WRITE_GRAD) != 0;
    fsdp_status s = check_step(p, rs_in, ag_in, write_grad, call);
    if (s != FSDP_OK) return s;
    if ((flags & ~static_cast<uint32_t>(FSDP_STEP_WRITE_GRAD)) != 0)
        return fail(FSDP_E_INVAL, "fsdp_step_shard: unknown flag");
    if ((s = check_hparams(hp, step, call)) != FSDP_OK || (s = check_device(p)) != FSDP_OK)
        return s;
    float scal[8];
    adamw_scalars(hp, step, scal);
    return launched(do_step(p, rs_in, ag_in, scal, write_grad, static_cast<hipStream_t>(stream)),
                    "fsdp_step_shard: launch");
}

fsdp_status fsdp_pack_allgather_fp8(const fsdp_plan *p, uint8_t *ag_in, const float *scales,
                                    void *stream) {
    fsdp_status s = need_roles(p, FSDP_ROLE_MASTER, "fsdp_pack_allgather_fp8");
    if (s != FSDP_OK) return s;
    if (ag_in == nullptr && p->L.S > 0)
        return fail(FSDP_E_INVAL, "fsdp_pack_allgather_fp8: null ag_in");
    if (scales == nullptr && !p->L.entries.empty())
        return fail(FSDP_E_INVAL, "fsdp_pack_allgather_fp8: null scales");
    if (misaligned(scales, 4)) return fail(FSDP_E_ALIGN, "fsdp_pack_allgather_fp8: scales not 4-byte aligned");
    if ((s = check_device(p)) != FSDP_OK) return s;
    return launched(guarded([&] {
                        return fsdp::launch_pack_fp8(
                            p->d_pack, static_cast<int64_t>(p->L.pack.size()), p->d_entries,
                            ag_in, scales, static_cast<hipStream_t>(stream));
                    }),
                    "fsdp_pack_allgather_fp8: launch");
}

fsdp_status fsdp_unpack_allgather_fp8(const fsdp_plan *p, const uint8_t *ag_out, void *stream) {
    fsdp_status s = need_roles(p, FSDP_ROLE_FULL_FP8, "fsdp_unpack_allgather_fp8");
    if (s != FSDP_OK) return s;
    if (ag_out == nullptr && p->L.S > 0)
        return fail(FSDP_E_INVAL, "fsdp_unpack_allgather_fp8: null ag_out");
    if ((s = check_device(p)) != FSDP_OK) return s;
    return launched(guarded([&] {
                        return fsdp::launch_unpack_fp8(
                            p->d_unpack, static_cast<int64_t>(p->L.unpack.size()), p->d_entries,
                            ag_out, chunk_aligned(p, ag_out), static_cast<hipStream_t>(stream));
                    }),
                    "fsdp_unpack_allgather_fp8: launch");
}

fsdp_status fsdp_amax_shard(const fsdp_plan *p, float *amax, void *stream) {
    fsdp_status s = need_roles(p, FSDP_ROLE_MASTER, "fsdp_amax_shard");
    if (s != FSDP_OK) return s;
    if (amax == nullptr && !p->L.entries.empty())
        return fail(FSDP_E_INVAL, "fsdp_amax_shard: null amax");
    if (misaligned(amax, 4)) return fail(FSDP_E_ALIGN, "fsdp_amax_shard: amax not 4-byte aligned");
    if ((s = check_device(p)) != FSDP_OK) return s;
    return launched(guarded([&] {
                        return fsdp::launch_amax(p->d_adamw, static_cast<int64_t>(p->L.adamw.size()),
                                                 p->d_entries, amax,
                                                 static_cast<int32_t>(p->L.entries.size()),
                                                 static_cast<hipStream_t>(stream));
                    }),
                    "fsdp_amax_shard: launch");
}

fsdp_status fsdp_accumulate_grad(const fsdp_plan *p, int32_t reset, void *stream) {
    fsdp_status s = need_roles(p, FSDP_ROLE_FULL_GRAD | FSDP_ROLE_GRAD_ACC, "fsdp_accumulate_grad");
    if (s != FSDP_OK || (s = check_device(p)) != FSDP_OK) return s;
    return launched(guarded([&] {
                        return fsdp::launch_accumulate(
                            p->d_full, static_cast<int64_t>(p->L.full.size()), p->d_entries,
                            reset != 0, static_cast<hipStream_t>(stream));
                    }),
                    "fsdp_accumulate_grad: launch");
}

fsdp_status fsdp_pack_reduce_scatter_acc(const fsdp_plan *p, float *rs_out, void *stream) {
    fsdp_status s = need_roles(p, FSDP_ROLE_GRAD_ACC, "fsdp_pack_reduce_scatter_acc");
    if (s != FSDP_OK) return s;
    if (rs_out == nullptr && p->L.S > 0)
        return fail(FSDP_E_INVAL, "fsdp_pack_reduce_scatter_acc: null rs_out");
    if (misaligned(rs_out, 4))
        return fail(FSDP_E_ALIGN, "fsdp_pack_reduce_scatter_acc: rs_out not 4-byte aligned");
    if ((s = check_device(p)) != FSDP_OK) return s;
    return launched(guarded([&] {
                        return fsdp::launch_rspack_acc(
                            p->d_rspack, static_cast<int64_t>(p->L.rspack.size()), p->d_entries,
                            rs_out, chunk_aligned(p, rs_out), static_cast<hipStream_t>(stream));
                    }),
                    "fsdp_pack_reduce_scatter_acc: launch");
}

fsdp_status fsdp_pack_reduce_scatter(const fsdp_plan *p, void *rs_out, int32_t dtype,
                                     void *stream) {
    const char *call = "fsdp_pack_reduce_scatter";
    fsdp_status s = need_roles(p, FSDP_ROLE_FULL_GRAD, call);
    if (s != FSDP_OK) return s;
    if (dtype != FSDP_DTYPE_BF16 && dtype != FSDP_DTYPE_F32)
        return fail(FSDP_E_UNSUPPORTED, "fsdp_pack_reduce_scatter: dtype must be BF16 or F32");
    if (rs_out == nullptr && p->L.S > 0)
        return fail(FSDP_E_INVAL, "fsdp_pack_reduce_scatter: null rs_out");
    if (misaligned(rs_out, dtype == FSDP_DTYPE_F32 ? 4 : 2))
        return fail(FSDP_E_ALIGN, "fsdp_pack_reduce_scatter: rs_out misaligned for its dtype");
    if ((s = check_device(p)) != FSDP_OK) return s;
    return launched(guarded([&] {
                        return fsdp::launch_rspack(
                            p->d_rspack, static_cast<int64_t>(p->L.rspack.size()), p->d_entries,
                            rs_out, dtype == FSDP_DTYPE_F32, chunk_aligned(p, rs_out),
                            static_cast<hipStream_t>(stream));
                    }),
                    "fsdp_pack_reduce_scatter: launch");
}

fsdp_status fsdp_reduce_shard_f32(const fsdp_plan *p, const float *rs_in, void *stream) {
    const char *call = "fsdp_reduce_shard_f32";
    fsdp_status s = need_roles(p, FSDP_ROLE_GRAD, call);
    if (s != FSDP_OK) return s;
    if (rs_in == nullptr && p->L.S > 0) return fail(FSDP_E_INVAL, "fsdp_reduce_shard_f32: null rs_in");
    if (misaligned(rs_in, 4))
        return fail(FSDP_E_ALIGN, "fsdp_reduce_shard_f32: rs_in not 4-byte aligned");
    if ((s = check_device(p)) != FSDP_OK) return s;
    return launched(guarded([&] {
                        return fsdp::launch_reduce_f32(
                            p->d_reduce, static_cast<int64_t>(p->L.reduce.size()), p->d_entries,
                            rs_in, p->L.S, p->L.world, chunk_aligned(p, rs_in),
                            static_cast<hipStream_t>(stream));
                    }),
                    "fsdp_reduce_shard_f32: launch");
}

fsdp_status fsdp_step_groups(fsdp_plan *const *plans, int32_t n_groups,
                             const uint16_t *const *rs_in, uint16_t *const *ag_in,
                             const uint16_t *const *ag_out, const fsdp_adamw_hparams_t *hp,
                             int64_t step, uint32_t flags, int32_t timed_kernel,
                             void *const *timing_events, void *stream) {
    const char *call = "fsdp_step_groups";
    if (n_groups < 0 || (n_groups > 0 && (plans == nullptr || rs_in == nullptr ||
                                          ag_in == nullptr)))
        return fail(FSDP_E_INVAL, "fsdp_step_groups: null array or negative n_groups");
    const uint32_t known = FSDP_STEP_WRITE_GRAD | FSDP_STEP_UNFUSED;
    if ((flags & ~known) != 0) return fail(FSDP_E_INVAL, "fsdp_step_groups: unknown flag");
    const bool write_grad = (flags & FSDP_STEP_WRITE_GRAD) != 0;
    const bool unfused = (flags & FSDP_STEP_UNFUSED) != 0;
    if (timing_events != nullptr) {
        const bool ok = timed_kernel == FSDP_KERNEL_UNPACK ||
                        (unfused ? (timed_kernel == FSDP_KERNEL_REDUCE ||
                                    timed_kernel == FSDP_KERNEL_ADAMW ||
                                    timed_kernel == FSDP_KERNEL_PACK)
                                 : timed_kernel == FSDP_KERNEL_STEP);
        if (!ok || (timed_kernel == FSDP_KERNEL_UNPACK && ag_out == nullptr))
            return fail(FSDP_E_INVAL, "fsdp_step_groups: timed_kernel is not run by this call");
        for (int32_t g = 0; g < n_groups; ++g)
            if ((timing_events[2 * g] == nullptr) != (timing_events[2 * g + 1] == nullptr))
                return fail(FSDP_E_INVAL, "fsdp_step_groups: timing events of a group must both be "
                                          "set or both be null");
    }
    fsdp_status s = check_hparams(hp, step, call);
    if (s != FSDP_OK) return s;
    for (int32_t g = 0; g < n_groups; ++g) {
        const fsdp_plan *p = plans[g];
        if (unfused) {
            if ((s = check_reduce(p, rs_in[g], call)) != FSDP_OK ||
                (s = need_roles(p, kAdamwRoles, call)) != FSDP_OK ||
                (s = check_pack(p, ag_in[g], call)) != FSDP_OK)
                return s;
        } else if ((s = check_step(p, rs_in[g], ag_in[g], write_grad, call)) != FSDP_OK) {
            return s;
        }
        if (ag_out != nullptr && (s = check_unpack(p, ag_out[g], call)) != FSDP_OK) return s;
        if ((s = check_device(p)) != FSDP_OK) return s;
    }
    float scal[8];
    adamw_scalars(hp, step, scal);
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto mark = [&](int32_t g, int32_t kernel, int which) -> hipError_t {
        if (timing_events == nullptr || kernel != timed_kernel ||
            timing_events[2 * g + which] == nullptr)
            return hipSuccess;
        return hipEventRecord(static_cast<hipEvent_t>(timing_events[2 * g + which]), st);
    };
    for (int32_t g = 0; g < n_groups; ++g) {
        const fsdp_plan *p = plans[g];
        hipError_t e = hipSuccess;
        if (unfused) {
            if ((e = mark(g, FSDP_KERNEL_REDUCE, 0)) == hipSuccess &&
                (e = do_reduce(p, rs_in[g], st)) == hipSuccess &&
                (e = mark(g, FSDP_KERNEL_REDUCE, 1)) == hipSuccess &&
                (e = mark(g, FSDP_KERNEL_ADAMW, 0)) == hipSuccess &&
                (e = do_adamw(p, scal, st)) == hipSuccess &&
                (e = mark(g, FSDP_KERNEL_ADAMW, 1)) == hipSuccess &&
                (e = mark(g, FSDP_KERNEL_PACK, 0)) == hipSuccess &&
                (e = do_pack(p, ag_in[g], st)) == hipSuccess)
                e = mark(g, FSDP_KERNEL_PACK, 1);
        } else if ((e = mark(g, FSDP_KERNEL_STEP, 0)) == hipSuccess &&
                   (e = do_step(p, rs_in[g], ag_in[g], scal, write_grad, st)) == hipSuccess) {
            e = mark(g, FSDP_KERNEL_STEP, 1);
        }
        if (e == hipSuccess && ag_out != nullptr &&
            (e = mark(g, FSDP_KERNEL_UNPACK, 0)) == hipSuccess &&
            (e = do_unpack(p, ag_out[g], st)) == hipSuccess)
            e = mark(g, FSDP_KERNEL_UNPACK, 1);
        if (e != hipSuccess)
            return hip_fail(e, ("fsdp_step_groups: group " + std::to_string(g)).c_str());
    }
    return FSDP_OK;
}

}  // extern "C"

// ---- group sets: AdamW and copy-in of many groups in one launch each --------

namespace {

// Copy-in segments of a set start 16-byte aligned in the arena.
int64_t round8(int64_t n) { return (n + 7) & ~static_cast<int64_t>(7); }

// No element of a written AdamW shard (master, exp_avg, exp_avg_sq) may
// belong to any other bound shard of the set (those three or grad), in
// this group or another: one launch updates them all at once.
fsdp_status check_disjoint(fsdp_group_set *set) {
    struct Span {
        uintptr_t lo, hi;
        bool written;
        int32_t g, i;
    };
    std::vector<Span> spans;
    for (size_t g = 0; g < set->plans.size(); ++g) {
        const fsdp_plan *p = set->plans[g];
        for (size_t i = 0; i < p->L.entries.size(); ++i) {
            const int64_t n = p->L.entries[i].valid_numel;
            if (n <= 0) continue;
            const fsdp::DevEntry &e = p->host_entries[i];
            const float *role[4] = {e.master, e.exp_avg, e.exp_avg_sq, e.grad};
            for (int r = 0; r < 4; ++r) {
                if (role[r] == nullptr) continue;
                const uintptr_t lo = reinterpret_cast<uintptr_t>(role[r]);
                spans.push_back({lo, lo + static_cast<uintptr_t>(n) * 4, r < 3,
                                 static_cast<int32_t>(g), static_cast<int32_t>(i)});
            }
        }
    }
    std::sort(spans.begin(), spans.end(),
              [](const Span &a, const Span &b) { return a.lo < b.lo; });
    for (const Span &sp : spans)      // sorted, merged: a copy-in arena is checked against it
        if (!set->shard_bytes.empty() && sp.lo <= set->shard_bytes.back().second)
            set->shard_bytes.back().second = std::max(set->shard_bytes.back().second, sp.hi);
        else
            set->shard_bytes.emplace_back(sp.lo, sp.hi);
    // Every overlapping pair is seen when its later-starting span comes up:
    // it meets an earlier written span, or it is written and meets any.
    uintptr_t end_any = 0, end_written = 0;
    const Span *last_any = nullptr, *last_written = nullptr;
    for (const Span &sp : spans) {
        const Span *hit = sp.lo < end_written ? last_written
                          : (sp.written && sp.lo < end_any) ? last_any
                                                            : nullptr;
        if (hit != nullptr)
            return fail(FSDP_E_INVAL,
                        "fsdp_group_set_create: shard tensors overlap (group " +
                            std::to_string(hit->g) + " parameter " + std::to_string(hit->i) +
                            ", group " + std::to_string(sp.g) + " parameter " +
                            std::to_string(sp.i) + ")");
        if (sp.hi > end_any) end_any = sp.hi, last_any = &sp;
        if (sp.written && sp.hi > end_written) end_written = sp.hi, last_written = &sp;
    }
    return FSDP_OK;
}

// The set's plans still hold the AdamW tensors it was built with, on the
// current device.
fsdp_status check_set(const fsdp_group_set *set, int32_t roles, const char *call) {
    if (set == nullptr) return fail(FSDP_E_INVAL, std::string(call) + ": null set");
    size_t k = 0;
    for (const fsdp_plan *p : set->plans) {
        fsdp_status s = need_roles(p, roles, call);
        if (s != FSDP_OK) return s;
        for (const fsdp::DevEntry &e : p->host_entries) {
            const fsdp::DevEntry &o = set->snapshot[k++];
            if (e.master != o.master || e.grad != o.grad || e.exp_avg != o.exp_avg ||
                e.exp_avg_sq != o.exp_avg_sq)
                return fail(FSDP_E_STATE, std::string(call) +
                                              ": a group was rebound after the set was built");
        }
    }
    if (set->plans.empty()) return FSDP_OK;
    return check_device(set->plans[0]);
}

hipError_t do_adamw_set(const fsdp_group_set *set, const float scal[8], hipStream_t st) {
    return guarded([&] {
        return fsdp::launch_adamw(set->d_adamw, set->n_adamw, set->d_entries, scal, true, st);
    });
}

hipError_t do_pack_set(const fsdp_group_set *set, uint16_t *arena, hipStream_t st) {
    return guarded(
        [&] { return fsdp::launch_pack(set->d_pack, set->n_pack, set->d_entries, arena, st); });
}

hipError_t do_adamw_pack_set(const fsdp_group_set *set, const float scal[8], uint16_t *arena,
                             hipStream_t st) {
    return guarded([&] {
        return fsdp::launch_adamw_pack(set->d_pack, set->n_pack, set->d_entries, arena, scal, st);
    });
}

// The copy-in arena is written in the same launch that reads (and, fused,
// writes) the shards: it must not share a byte with any of them.
fsdp_status check_arena(const fsdp_group_set *set, const void *arena, const char *call,
                        uintptr_t elem_bytes = 2) {
    const int64_t elems = set->seg_off.back();
    if (arena == nullptr && elems > 0)
        return fail(FSDP_E_INVAL, std::string(call) + ": null arena");
    if (misaligned(arena, elem_bytes))
        return fail(FSDP_E_ALIGN, std::string(call) + ": arena misaligned for its element type");
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(arena);
    const uintptr_t a1 = a0 + static_cast<uintptr_t>(elems) * elem_bytes;
    // the first merged span ending after a0 is the only one that can overlap
    auto it = std::upper_bound(set->shard_bytes.begin(), set->shard_bytes.end(), a0,
                               [](uintptr_t v, const std::pair<uintptr_t, uintptr_t> &sp) {
                                   return v < sp.second;
                               });
    if (elems > 0 && it != set->shard_bytes.end() && it->first < a1)
        return fail(FSDP_E_INVAL, std::string(call) + ": arena overlaps a bound shard tensor");
    return FSDP_OK;
}

}  // namespace

extern "C" {

fsdp_status fsdp_group_set_create(fsdp_plan *const *plans, int32_t n_groups, void *stream,
                                  fsdp_group_set **out) {
    if (out == nullptr) return fail(FSDP_E_INVAL, "fsdp_group_set_create: null out");
    *out = nullptr;
    if (n_groups < 1 || plans == nullptr)
        return fail(FSDP_E_INVAL, "fsdp_group_set_create: need n_groups >= 1 and a plan array");
    for (int32_t g = 0; g < n_groups; ++g) {
        if (plans[g] == nullptr) return fail(FSDP_E_INVAL, "fsdp_group_set_create: null plan");
        for (int32_t h = 0; h < g; ++h)
            if (plans[h] == plans[g])
                return fail(FSDP_E_INVAL, "fsdp_group_set_create: plan of group " +
                                              std::to_string(g) + " repeats group " +
                                              std::to_string(h));
    }
    for (int32_t g = 0; g < n_groups; ++g) {
        if (plans[g]->dmem == nullptr)
            return fail(FSDP_E_STATE, "fsdp_group_set_create: plan of group " +
                                          std::to_string(g) + " has never been bound");
        if (plans[g]->device != plans[0]->device)
            return fail(FSDP_E_STATE, "fsdp_group_set_create: groups bound on different devices");
    }
    fsdp_group_set *set = nullptr;
    try {
        set = new fsdp_group_set();
        set->plans.assign(plans, plans + n_groups);
        set->ent_off.assign(1, 0);
        set->seg_off.assign(1, 0);
        for (const fsdp_plan *p : set->plans) {
            set->ent_off.push_back(set->ent_off.back() +
                                   static_cast<int64_t>(p->L.entries.size()));
            set->seg_off.push_back(set->seg_off.back() + round8(p->L.S));
            set->snapshot.insert(set->snapshot.end(), p->host_entries.begin(),
                                 p->host_entries.end());
            set->n_pack += static_cast<int64_t>(p->L.pack.size());
            set->n_adamw += static_cast<int64_t>(p->L.adamw.size());
        }
        fsdp_status s = check_disjoint(set);
        if (s == FSDP_OK) s = check_device(set->plans[0]);
        if (s != FSDP_OK) {
            delete set;
            return s;
        }
        // host copies of the tables, re-indexed into the set
        std::vector<fsdp::PackTile> pack;
        std::vector<fsdp::EwTile> adamw;
        pack.reserve(static_cast<size_t>(set->n_pack));
        adamw.reserve(static_cast<size_t>(set->n_adamw));
        for (int32_t g = 0; g < n_groups; ++g) {
            const fsdp::Layout &L = set->plans[g]->L;
            const int32_t eo = static_cast<int32_t>(set->ent_off[g]);
            for (fsdp::PackTile t : L.pack) {
                t.dst += set->seg_off[g];
                t.entry += eo;
                pack.push_back(t);
            }
            for (fsdp::EwTile t : L.adamw) {
                t.entry += eo;
                adamw.push_back(t);
            }
        }
        const size_t eb = set->snapshot.size() * sizeof(fsdp::DevEntry);
        const size_t pb = pack.size() * sizeof(fsdp::PackTile);
        const size_t ab = adamw.size() * sizeof(fsdp::EwTile);
        void *mem = nullptr;
        hipError_t e = hipMalloc(&mem, round256(eb) + round256(pb) + round256(ab) + 256);
        if (e != hipSuccess) {
            delete set;
            return fail(FSDP_E_NOMEM, "fsdp_group_set_create: hipMalloc of device tables failed");
        }
        set->dmem = static_cast<char *>(mem);
        set->device = set->plans[0]->device;
        set->d_entries = reinterpret_cast<fsdp::DevEntry *>(set->dmem);
        set->d_pack = reinterpret_cast<fsdp::PackTile *>(set->dmem + round256(eb));
        set->d_adamw = reinterpret_cast<fsdp::EwTile *>(set->dmem + round256(eb) + round256(pb));
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const struct {
            void *dst;
            const void *src;
            size_t bytes;
        } up[3] = {{set->d_entries, set->snapshot.data(), eb},
                   {set->d_pack, pack.data(), pb},
                   {set->d_adamw, adamw.data(), ab}};
        for (const auto &u : up) {
            if (u.bytes == 0) continue;
            if ((e = hipMemcpyAsync(u.dst, u.src, u.bytes, hipMemcpyHostToDevice, st)) !=
                hipSuccess)
                break;
        }
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) {
            fsdp_group_set_destroy(set);
            return hip_fail(e, "fsdp_group_set_create: upload");
        }
        *out = set;
        return FSDP_OK;
    } catch (const std::bad_alloc &) {
        delete set;
        return fail(FSDP_E_NOMEM, "fsdp_group_set_create: host allocation failed");
    }
}

void fsdp_group_set_destroy(fsdp_group_set *set) {
    if (set == nullptr) return;
    if (set->dmem != nullptr) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(set->device);
        (void)hipDeviceSynchronize();
        (void)hipFree(set->dmem);
        if (cur >= 0) (void)hipSetDevice(cur);
    }
    delete set;
}

fsdp_status fsdp_group_set_info(const fsdp_group_set *set, int32_t *n_groups,
                                int32_t *n_params, int64_t *arena_elems) {
    if (set == nullptr || n_groups == nullptr || n_params == nullptr || arena_elems == nullptr)
        return fail(FSDP_E_INVAL, "fsdp_group_set_info: null argument");
    *n_groups = static_cast<int32_t>(set->plans.size());
    *n_params = static_cast<int32_t>(set->ent_off.back());
    *arena_elems = set->seg_off.back();
    return FSDP_OK;
}

fsdp_status fsdp_group_set_segment(const fsdp_group_set *set, int32_t g, int64_t *offset,
                                   int64_t *arena_elems) {
    if (set == nullptr || offset == nullptr || arena_elems == nullptr)
        return fail(FSDP_E_INVAL, "fsdp_group_set_segment: null argument");
    if (g < 0 || static_cast<size_t>(g) >= set->plans.size())
        return fail(FSDP_E_INVAL, "fsdp_group_set_segment: group out of range");
    *offset = set->seg_off[g];
    *arena_elems = set->seg_off.back();
    return FSDP_OK;
}

fsdp_status fsdp_adamw_groups(const fsdp_group_set *set, const fsdp_adamw_hparams_t *hp,
                              int64_t step, void *stream) {
    const char *call = "fsdp_adamw_groups";
    fsdp_status s = check_set(set, kAdamwRoles, call);
    if (s != FSDP_OK || (s = check_hparams(hp, step, call)) != FSDP_OK) return s;
    float scal[8];
    adamw_scalars(hp, step, scal);
    return launched(do_adamw_set(set, scal, static_cast<hipStream_t>(stream)),
                    "fsdp_adamw_groups: launch");
}

fsdp_status fsdp_pack_allgather_groups(const fsdp_group_set *set, uint16_t *arena,
                                       void *stream) {
    const char *call = "fsdp_pack_allgather_groups";
    fsdp_status s = check_set(set, FSDP_ROLE_MASTER, call);
    if (s != FSDP_OK || (s = check_arena(set, arena, call)) != FSDP_OK) return s;
    return launched(do_pack_set(set, arena, static_cast<hipStream_t>(stream)),
                    "fsdp_pack_allgather_groups: launch");
}

fsdp_status fsdp_adamw_pack_groups(const fsdp_group_set *set, const fsdp_adamw_hparams_t *hp,
                                   int64_t step, uint16_t *arena, void *stream) {
    const char *call = "fsdp_adamw_pack_groups";
    fsdp_status s = check_set(set, kAdamwRoles, call);
    if (s != FSDP_OK || (s = check_hparams(hp, step, call)) != FSDP_OK ||
        (s = check_arena(set, arena, call)) != FSDP_OK)
        return s;
    float scal[8];
    adamw_scalars(hp, step, scal);
    return launched(do_adamw_pack_set(set, scal, arena, static_cast<hipStream_t>(stream)),
                    "fsdp_adamw_pack_groups: launch");
}

fsdp_status fsdp_amax_groups(const fsdp_group_set *set, float *amax, void *stream) {
    const char *call = "fsdp_amax_groups";
    fsdp_status s = check_set(set, FSDP_ROLE_MASTER, call);
    if (s != FSDP_OK) return s;
    const int64_t np = set->ent_off.back();
    if (amax == nullptr && np > 0) return fail(FSDP_E_INVAL, "fsdp_amax_groups: null amax");
    if (misaligned(amax, 4)) return fail(FSDP_E_ALIGN, "fsdp_amax_groups: amax not 4-byte aligned");
    return launched(guarded([&] {
                        return fsdp::launch_amax(set->d_adamw, set->n_adamw, set->d_entries, amax,
                                                 static_cast<int32_t>(np),
                                                 static_cast<hipStream_t>(stream));
                    }),
                    "fsdp_amax_groups: launch");
}

fsdp_status fsdp_pack_allgather_fp8_groups(const fsdp_group_set *set, uint8_t *arena,
                                           const float *scales, void *stream) {
    const char *call = "fsdp_pack_allgather_fp8_groups";
    fsdp_status s = check_set(set, FSDP_ROLE_MASTER, call);
    if (s != FSDP_OK || (s = check_arena(set, arena, call, 1)) != FSDP_OK) return s;
    if (scales == nullptr && set->ent_off.back() > 0)
        return fail(FSDP_E_INVAL, "fsdp_pack_allgather_fp8_groups: null scales");
    if (misaligned(scales, 4))
        return fail(FSDP_E_ALIGN, "fsdp_pack_allgather_fp8_groups: scales not 4-byte aligned");
    return launched(guarded([&] {
                        return fsdp::launch_pack_fp8(set->d_pack, set->n_pack, set->d_entries,
                                                     arena, scales,
                                                     static_cast<hipStream_t>(stream));
                    }),
                    "fsdp_pack_allgather_fp8_groups: launch");
}

fsdp_status fsdp_step_group_set(const fsdp_group_set *set, const uint16_t *const *rs_in,
                                uint16_t *arena, const uint16_t *const *ag_out,
                                const fsdp_adamw_hparams_t *hp, int64_t step, uint32_t flags,
                                int32_t timed_kernel, void *const *timing_events,
                                void *stream) {
    const char *call = "fsdp_step_group_set";
    fsdp_status s = check_set(set, kAdamwRoles, call);
    if (s != FSDP_OK) return s;
    const int32_t n = static_cast<int32_t>(set->plans.size());
    if (rs_in == nullptr) return fail(FSDP_E_INVAL, "fsdp_step_group_set: null rs_in array");
    if ((flags & ~static_cast<uint32_t>(FSDP_SET_ADAMW_COPY_IN)) != 0)
        return fail(FSDP_E_INVAL, "fsdp_step_group_set: unknown flag");
    const bool fused = (flags & FSDP_SET_ADAMW_COPY_IN) != 0;
    if ((s = check_hparams(hp, step, call)) != FSDP_OK ||
        (s = check_arena(set, arena, call)) != FSDP_OK)
        return s;
    if (timing_events != nullptr) {
        const bool ok = timed_kernel == FSDP_KERNEL_REDUCE ||
                        (fused ? timed_kernel == FSDP_KERNEL_ADAMW_PACK
                               : (timed_kernel == FSDP_KERNEL_ADAMW ||
                                  timed_kernel == FSDP_KERNEL_PACK)) ||
                        (timed_kernel == FSDP_KERNEL_UNPACK && ag_out != nullptr);
        if (!ok) return fail(FSDP_E_INVAL, "fsdp_step_group_set: timed_kernel is not run by this call");
        for (int32_t g = 0; g < n; ++g)
            if ((timing_events[2 * g] == nullptr) != (timing_events[2 * g + 1] == nullptr))
                return fail(FSDP_E_INVAL, "fsdp_step_group_set: timing events of a group must "
                                          "both be set or both be null");
    }
    for (int32_t g = 0; g < n; ++g) {
        const fsdp_plan *p = set->plans[g];
        if ((s = check_reduce(p, rs_in[g], call)) != FSDP_OK) return s;
        if (ag_out != nullptr && (s = check_unpack(p, ag_out[g], call)) != FSDP_OK) return s;
        // the reduce reads rs_in while the copy-in writes the arena
        const uintptr_t r0 = reinterpret_cast<uintptr_t>(rs_in[g]);
        const uintptr_t rb = static_cast<uintptr_t>(p->L.world) * static_cast<uintptr_t>(p->L.S) * 2;
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(arena);
        const uintptr_t ab = static_cast<uintptr_t>(set->seg_off.back()) * 2;
        if (rb > 0 && ab > 0 && a0 < r0 + rb && r0 < a0 + ab)
            return fail(FSDP_E_INVAL, "fsdp_step_group_set: arena overlaps rs_in of group " +
                                          std::to_string(g));
    }
    float scal[8];
    adamw_scalars(hp, step, scal);
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto mark = [&](int32_t g, int32_t kernel, int which) -> hipError_t {
        if (timing_events == nullptr || kernel != timed_kernel ||
            timing_events[2 * g + which] == nullptr)
            return hipSuccess;
        return hipEventRecord(static_cast<hipEvent_t>(timing_events[2 * g + which]), st);
    };
    hipError_t e = hipSuccess;
    for (int32_t g = 0; g < n && e == hipSuccess; ++g) {
        if ((e = mark(g, FSDP_KERNEL_REDUCE, 0)) == hipSuccess &&
            (e = do_reduce(set->plans[g], rs_in[g], st)) == hipSuccess)
            e = mark(g, FSDP_KERNEL_REDUCE, 1);
        if (e != hipSuccess)
            return hip_fail(e, ("fsdp_step_group_set: reduce of group " + std::to_string(g)).c_str());
    }
    if (fused) {
        if ((e = mark(0, FSDP_KERNEL_ADAMW_PACK, 0)) == hipSuccess &&
            (e = do_adamw_pack_set(set, scal, arena, st)) == hipSuccess)
            e = mark(0, FSDP_KERNEL_ADAMW_PACK, 1);
    } else if ((e = mark(0, FSDP_KERNEL_ADAMW, 0)) == hipSuccess &&
               (e = do_adamw_set(set, scal, st)) == hipSuccess &&
               (e = mark(0, FSDP_KERNEL_ADAMW, 1)) == hipSuccess &&
               (e = mark(0, FSDP_KERNEL_PACK, 0)) == hipSuccess &&
               (e = do_pack_set(set, arena, st)) == hipSuccess) {
        e = mark(0, FSDP_KERNEL_PACK, 1);
    }
    if (e != hipSuccess) return hip_fail(e, "fsdp_step_group_set: AdamW or copy-in");
    for (int32_t g = 0; ag_out != nullptr && g < n; ++g) {
        if ((e = mark(g, FSDP_KERNEL_UNPACK, 0)) == hipSuccess &&
            (e = do_unpack(set->plans[g], ag_out[g], st)) == hipSuccess)
            e = mark(g, FSDP_KERNEL_UNPACK, 1);
        if (e != hipSuccess)
            return hip_fail(e, ("fsdp_step_group_set: copy-out of group " + std::to_string(g)).c_str());
    }
    return FSDP_OK;
}

fsdp_status fsdp_check_stream(void *stream) {
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "fsdp_check_stream: hipStreamSynchronize");
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "fsdp_check_stream");
    return FSDP_OK;
}

}  // extern "C"
