// bfo_control.cpp -- step control around the optimizer step: the learning
// rate schedule (a host function of the step number) and the outlier
// detector (a device-side ring of recent grad norms whose skip flag the
// update kernel reads, so a skipped step needs no host round trip).
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <new>

#include "bfo_internal.hpp"

struct bfo_outlier_s {
    bfo::OutlierState *state = nullptr;
    uint32_t window = 0;
    float threshold = 0.0f;
    int device = 0;
};

namespace {

int controlFail(hipError_t e) { return bfo::recordHipFailure(e); }

}  // namespace

extern "C" {

// "04 · 多 GPU 与混合精度" §4 names cosine, linear, constant and wsd
// schedules; the formulas are stated with bfo_lr_schedule in the header.
int bfo_lr_at(const bfo_lr_schedule *sch, uint64_t step, float *lr) {
    if (!sch || !lr) return BFO_EINVAL;
    if (sch->kind < BFO_LR_CONSTANT || sch->kind > BFO_LR_WSD) return BFO_EINVAL;
    if (sch->total_steps < sch->warmup_steps) return BFO_EINVAL;
    const double peak = double(sch->lr_max);
    const double lowest = double(sch->final_frac) * peak;
    if (step < sch->warmup_steps) {
        *lr = float(peak * double(step + 1) / double(sch->warmup_steps));
        return BFO_OK;
    }
    switch (sch->kind) {
        case BFO_LR_CONSTANT:
            *lr = sch->lr_max;
            return BFO_OK;
        case BFO_LR_WSD: {
            const double tail = double(sch->decay_frac) * double(sch->total_steps);
            const double tailStart = double(sch->total_steps) - tail;
            if (double(step) < tailStart || tail <= 0.0) {
                *lr = sch->lr_max;
                return BFO_OK;
            }
            double f = (double(step) - tailStart) / tail;
            if (f > 1.0) f = 1.0;
            *lr = float(peak - (peak - lowest) * f);
            return BFO_OK;
        }
        default: {
            const double span = double(sch->total_steps) - double(sch->warmup_steps);
            double f = span > 0.0 ? (double(step) - double(sch->warmup_steps)) / span : 1.0;
            if (f > 1.0) f = 1.0;
            if (sch->kind == BFO_LR_LINEAR)
                *lr = float(peak - (peak - lowest) * f);
            else
                *lr = float(lowest + (peak - lowest) * (1.0 + std::cos(M_PI * f)) / 2.0);
            return BFO_OK;
        }
    }
}

int bfo_outlier_create(uint32_t window, float threshold, bfo_outlier *out) {
    if (!out) return BFO_EINVAL;
    *out = nullptr;
    if (window == 0 || window > bfo::kOutlierMaxWindow) return BFO_EINVAL;
    bfo_outlier_s *d = new (std::nothrow) bfo_outlier_s;
    if (!d) return BFO_EINVAL;
    d->window = window;
    d->threshold = threshold;
    hipError_t he = hipGetDevice(&d->device);
    if (he == hipSuccess)
        he = hipMalloc(&d->state, sizeof(bfo::OutlierState) + sizeof(float) * (window - 1));
    if (he == hipSuccess) he = bfo::launchOutlierReset(d->state, window, nullptr);
    if (he == hipSuccess) he = hipStreamSynchronize(nullptr);
    if (he != hipSuccess) {
        if (d->state) (void)hipFree(d->state);
        delete d;
        return controlFail(he);
    }
    *out = d;
    return BFO_OK;
}

int bfo_outlier_destroy(bfo_outlier d) {
    if (!d) return BFO_OK;
    hipError_t he = hipFree(d->state);
    delete d;
    return he == hipSuccess ? BFO_OK : controlFail(he);
}

int bfo_outlier_reset(bfo_outlier d, void *stream) {
    if (!d) return BFO_EINVAL;
    hipError_t he = bfo::launchOutlierReset(d->state, d->window, static_cast<hipStream_t>(stream));
    return he == hipSuccess ? BFO_OK : controlFail(he);
}

int bfo_outlier_update(bfo_outlier d, const float *value, float *z, int32_t *skip, void *stream) {
    if (!d || !value || !z || !skip) return BFO_EINVAL;
    if ((reinterpret_cast<uintptr_t>(value) | reinterpret_cast<uintptr_t>(z) |
         reinterpret_cast<uintptr_t>(skip)) & 3u)
        return BFO_EMISALIGNED;
    int dev = -1;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return controlFail(he);
    if (dev != d->device) return BFO_EDEVICE;
    he = bfo::launchOutlierUpdate(d->state, value, d->threshold, z, skip, static_cast<hipStream_t>(stream));
    return he == hipSuccess ? BFO_OK : controlFail(he);
}

}  // extern "C"
