// AdamW on host-resident fp32 shards, for CPU offload.
//
// "Sharded Training: FSDP2, DTensor, Tensor and Pipeline Parallelism",
// "Offload" paragraph: with CPU offload the parameter shards, gradients and
// optimizer state live in pinned host memory and the optimizer step runs on
// the CPU.  This is the same update as the GPU kernel, element for element:
// fp32, one rounding per operation in the order of the C header, no fused
// multiply-add (built with -ffp-contract=off), correctly rounded division
// and square root (IEEE on x86), so results are bit-identical to the device
// path.  Work is split into contiguous ranges over a few threads.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>
#include <thread>
#include <vector>

#include "../../include/fsdp_shard.h"

namespace fsdp {
fsdp_status set_error(fsdp_status s, const std::string &msg);
void adamw_scalars_host(const fsdp_adamw_hparams_t *hp, int64_t step, float out[8]);
}  // namespace fsdp

namespace {

void adamw_range(float *__restrict p, const float *__restrict g, float *__restrict m,
                 float *__restrict v, int64_t begin, int64_t end, const float c[8]) {
    const float b1 = c[0], omb1 = c[1], b2 = c[2], omb2 = c[3], eps = c[4], decay = c[5],
                step_size = c[6], bc2s = c[7];
    for (int64_t i = begin; i < end; ++i) {
        const float gi = g[i];
        float pi = p[i] * decay;
        const float mi = b1 * m[i] + omb1 * gi;
        const float vi = b2 * v[i] + omb2 * (gi * gi);
        const float d = std::sqrt(vi) / bc2s + eps;
        pi = pi - step_size * (mi / d);
        p[i] = pi;
        m[i] = mi;
        v[i] = vi;
    }
}

}  // namespace

extern "C" fsdp_status fsdp_adamw_host(float *p, const float *g, float *m, float *v, int64_t n,
                                       const fsdp_adamw_hparams_t *hp, int64_t step,
                                       int32_t n_threads) {
    if (n < 0) return fsdp::set_error(FSDP_E_INVAL, "fsdp_adamw_host: negative n");
    if (n > 0 && (p == nullptr || g == nullptr || m == nullptr || v == nullptr))
        return fsdp::set_error(FSDP_E_INVAL, "fsdp_adamw_host: null array");
    if (hp == nullptr) return fsdp::set_error(FSDP_E_INVAL, "fsdp_adamw_host: null hyperparameters");
    if (step < 1) return fsdp::set_error(FSDP_E_INVAL, "fsdp_adamw_host: step counts from 1");
    float c[8];
    fsdp::adamw_scalars_host(hp, step, c);
    int64_t t = n_threads > 0 ? n_threads : static_cast<int64_t>(std::thread::hardware_concurrency());
    t = std::max<int64_t>(1, std::min<int64_t>(t, (n + 65535) / 65536));
    if (t == 1) {
        adamw_range(p, g, m, v, 0, n, c);
        return FSDP_OK;
    }
    // A range whose thread cannot be started runs on this thread instead;
    // every started thread is joined before returning.
    const int64_t per = (n + t - 1) / t;
    std::vector<std::thread> pool;
    int64_t k = 0;
    try {
        pool.reserve(static_cast<size_t>(t));
        for (; k < t; ++k) {
            const int64_t b = k * per, e = std::min(n, b + per);
            if (b >= e) break;
            pool.emplace_back(adamw_range, p, g, m, v, b, e, c);
        }
    } catch (...) {
        // fall through: ranges k.. are done below
    }
    for (; k < t; ++k) {
        const int64_t b = k * per, e = std::min(n, b + per);
        if (b >= e) break;
        adamw_range(p, g, m, v, b, e, c);
    }
    for (std::thread &th : pool) th.join();
    return FSDP_OK;
}
