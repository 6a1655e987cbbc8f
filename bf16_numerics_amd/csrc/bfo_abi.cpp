// bfo_abi.cpp -- host side of the C ABI declared in include/bf16opt.h:
// argument checks, ZeRO-1 shard arithmetic, the per-table shard plan (runs
// and tile words, built and uploaded once) and the kernel launches on the
// caller's stream.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <new>
#include <vector>

#include "bfo_internal.hpp"

namespace {

thread_local int gLastHipError = 0;

int hipFail(hipError_t e) { return bfo::recordHipFailure(e); }

bool alignedTo(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The byte range [lo, hi) an array argument covers; a null pointer covers
// nothing.
struct Span {
    uintptr_t lo, hi;
};

Span span(const void *p, uint64_t bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(p);
    if (!p) return {0, 0};
    return {x, bytes > UINTPTR_MAX - x ? UINTPTR_MAX : x + uintptr_t(bytes)};
}

// True when two of the arrays of one call share a byte: the kernels read and
// write them as distinct (restrict) buffers.
bool anyOverlap(std::initializer_list<Span> spans) {
    for (const Span *a = spans.begin(); a != spans.end(); ++a)
        for (const Span *b = a + 1; b != spans.end(); ++b)
            if (a->lo < a->hi && b->lo < b->hi && a->lo < b->hi && b->lo < a->hi) return true;
    return false;
}

}  // namespace

int bfo::recordHipFailure(hipError_t e) {
    gLastHipError = int(e);
    return BFO_EHIP;
}

struct bfo_table_s {
    uint64_t n = 0, S = 0, begin = 0;
    uint32_t world = 1, rank = 0;
    int layout = BFO_LAYOUT_FLAT;
    int device = 0;
    uint64_t fingerprint = 0;        // FNV-1a over the tensor table
    std::vector<bfo_run> runs;       // host copy of the plan
    void *devBlock = nullptr;        // one allocation holding everything below
    uint32_t *tile = nullptr;        // [ntiles]
    uint64_t *local = nullptr;       // [nruns + 1], last = UINT64_MAX
    uint64_t *addr = nullptr;        // [nruns]
    uint64_t *rng = nullptr;         // [nruns]
    uint8_t *flag = nullptr;         // [nruns]
    double *normPartials = nullptr;  // [normTiles(S) + normRuns(...)], at least 1
    uint64_t *normOffset = nullptr;  // [normTiles(S)], per-tensor tables only

    bfo::ShardView view() const {
        return {tile, local, addr, rng, flag, normOffset, layout == BFO_LAYOUT_FLAT ? begin : UINT64_MAX};
    }
};

// Elements of the params and grads arrays a call addresses: the shard for
// flat tables, the whole buffer for per-tensor ones.
static uint64_t pgElems(const bfo_table_s *t) { return t->layout == BFO_LAYOUT_FLAT ? t->S : t->n; }

int bfo::rebuildParams(bfo_table_s *t, const float *master, uint16_t *params, uint64_t seed, int rounding,
                       hipStream_t stream) {
    if (t->S == 0) return BFO_OK;
    const int pgVec = (reinterpret_cast<uintptr_t>(params) & 15) == 0 ? 1 : 0;
    const hipError_t he = launchMasterToBf16(master, params, t->S, t->view(), pgVec, seed, rounding, stream);
    return he == hipSuccess ? BFO_OK : recordHipFailure(he);
}

bfo::TableFacts bfo::tableFacts(const bfo_table_s *t) {
    return {t->n, t->S, t->world, t->rank, t->layout, t->fingerprint, t->runs.data(), uint32_t(t->runs.size())};
}

extern "C" {

// "04 · 多 GPU 与混合精度" §3.2 / "LLM 分布式训练实战" §3.1.
int shard_range(uint64_t n, uint32_t world, uint32_t rank, uint64_t *begin, uint64_t *end) {
    if (!begin || !end || world == 0) return BFO_EINVAL;
    if (rank >= world) return BFO_ERANGE;
    if (n % world != 0) return BFO_ENOTDIVISIBLE;
    const uint64_t per = n / world;
    *begin = uint64_t(rank) * per;
    *end = *begin + per;
    return BFO_OK;
}

}  // extern "C"

namespace {

// The shard plan, on the host only: validates the table, then lists the runs
// of the shard (see bfo_run).  Flat: each tensor's piece of [b, e), addressed
// shard-locally.  Per tensor: rank r's 1/world slice of every tensor,
// addressed in the full buffer.  Pieces that continue one another with the
// same flag merge.  begin is b for flat tables and 0 for per-tensor ones.
int buildPlan(const bfo_tensor *tensors, uint32_t count, uint32_t world, uint32_t rank, int layout,
              std::vector<bfo_run> &runs, uint64_t &n, uint64_t &S, uint64_t &begin) {
    if (count > 0 && !tensors) return BFO_EINVAL;
    if (layout != BFO_LAYOUT_FLAT && layout != BFO_LAYOUT_PER_TENSOR) return BFO_EINVAL;
    if (count >= bfo::kTileMixed) return BFO_ETABLE;  // run ids must fit in 31 bits

    // Table: contiguous from 0, known flag bits only, no overflow.
    n = 0;
    for (uint32_t k = 0; k < count; ++k) {
        if (tensors[k].offset != n || (tensors[k].flags & ~BFO_FLAG_DECAY) || tensors[k].reserved)
            return BFO_ETABLE;
        if (tensors[k].numel > UINT64_MAX - n) return BFO_ETABLE;
        n += tensors[k].numel;
    }
    uint64_t b = 0, e = 0;
    int rc = shard_range(n, world, rank, &b, &e);
    if (rc != BFO_OK) return rc;

    runs.clear();
    auto push = [&runs](uint64_t local, uint64_t addr, uint64_t global, uint64_t len, uint32_t flags) {
        if (!runs.empty()) {
            bfo_run &p = runs.back();
            if (p.flags == flags && p.addr + p.length == addr && p.global + p.length == global) {
                p.length += len;
                return;
            }
        }
        runs.push_back(bfo_run{local, addr, global, len, flags, 0u});
    };
    S = 0;
    if (layout == BFO_LAYOUT_FLAT) {
        for (uint32_t k = 0; k < count; ++k) {
            const uint64_t lo = tensors[k].offset > b ? tensors[k].offset : b;
            const uint64_t tend = tensors[k].offset + tensors[k].numel;
            const uint64_t hi = tend < e ? tend : e;
            if (lo >= hi) continue;
            push(lo - b, lo - b, lo, hi - lo, tensors[k].flags & BFO_FLAG_DECAY);
        }
        S = e - b;
    } else {
        for (uint32_t k = 0; k < count; ++k)
            if (tensors[k].numel % world != 0) return BFO_ENOTDIVISIBLE;
        for (uint32_t k = 0; k < count; ++k) {
            const uint64_t len = tensors[k].numel / world;
            if (len == 0) continue;
            const uint64_t g = tensors[k].offset + uint64_t(rank) * len;
            push(S, g, g, len, tensors[k].flags & BFO_FLAG_DECAY);
            S += len;
        }
        b = 0;
    }
    begin = b;
    return BFO_OK;
}

}  // namespace

extern "C" {

int bfo_plan_runs(const bfo_tensor *tensors, uint32_t count, uint32_t world, uint32_t rank, int layout,
                  bfo_run *out, uint32_t capacity, uint32_t *nruns, uint64_t *shard_elems) {
    if (!nruns) return BFO_EINVAL;
    std::vector<bfo_run> runs;
    uint64_t n = 0, S = 0, b = 0;
    const int rc = buildPlan(tensors, count, world, rank, layout, runs, n, S, b);
    if (rc != BFO_OK) return rc;
    *nruns = uint32_t(runs.size());
    if (shard_elems) *shard_elems = S;
    if (out) {
        if (capacity < runs.size()) return BFO_ERANGE;
        std::memcpy(out, runs.data(), runs.size() * sizeof(bfo_run));
    }
    return BFO_OK;
}

int bfo_table_create_layout(const bfo_tensor *tensors, uint32_t count, uint32_t world, uint32_t rank,
                            int layout, bfo_table *out) {
    if (!out) return BFO_EINVAL;
    *out = nullptr;
    std::vector<bfo_run> runs;
    uint64_t n = 0, S = 0, b = 0;
    const int rc = buildPlan(tensors, count, world, rank, layout, runs, n, S, b);
    if (rc != BFO_OK) return rc;
    const uint64_t nruns = runs.size();
    std::vector<uint64_t> local(nruns + 1), addr(nruns ? nruns : 1), rng(nruns ? nruns : 1);
    std::vector<uint8_t> flag(nruns ? nruns : 1, 0);
    for (uint64_t k = 0; k < nruns; ++k) {
        local[k] = runs[k].local;
        addr[k] = runs[k].addr;
        rng[k] = runs[k].global;
        flag[k] = uint8_t(runs[k].flags & BFO_FLAG_DECAY);
    }
    local[nruns] = UINT64_MAX;

    // Tile words: the run holding each tile's first element, and whether the
    // tile runs past that run's end.
    const uint64_t ntiles = (S + bfo::kTileElems - 1) / bfo::kTileElems;
    std::vector<uint32_t> tileWord(ntiles ? ntiles : 1, 0u);
    uint64_t k = 0;
    for (uint64_t t = 0; t < ntiles; ++t) {
        const uint64_t t0 = t * bfo::kTileElems;
        const uint64_t t1 = t0 + bfo::kTileElems < S ? t0 + bfo::kTileElems : S;
        while (local[k + 1] <= t0) ++k;
        tileWord[t] = uint32_t(k) | (local[k + 1] < t1 ? bfo::kTileMixed : 0u);
    }

    // Per-tensor tables: grad-norm tiles that lie inside one run are read at a
    // constant offset from the shard-local position (8-aligned, so a
    // 16-byte-aligned grads array keeps 16-byte vectors).
    std::vector<uint64_t> normOff;
    if (layout == BFO_LAYOUT_PER_TENSOR && S > 0) {
        const uint64_t tileElems = bfo::kNormTileVecs * 8;
        const uint64_t nT = bfo::normTiles(S);
        normOff.assign(nT, bfo::kNoNormOffset);
        uint64_t r = 0;
        for (uint64_t t = 0; t < nT; ++t) {
            const uint64_t t0 = t * tileElems;
            const uint64_t t1 = t0 + tileElems < S ? t0 + tileElems : S;
            while (runs[r].local + runs[r].length <= t0) ++r;
            const bfo_run &run = runs[r];
            const uint64_t off = run.addr - run.local;
            if (t1 <= run.local + run.length && off % 8 == 0) normOff[t] = off;
        }
    }

    // Fingerprint of the table, stored in checkpoints to refuse a mismatch.
    uint64_t fp = 1469598103934665603ull;
    auto mix = [&fp](uint64_t x) {
        for (int byte = 0; byte < 8; ++byte) {
            fp ^= (x >> (8 * byte)) & 0xFFu;
            fp *= 1099511628211ull;
        }
    };
    for (uint32_t t = 0; t < count; ++t) {
        mix(tensors[t].offset);
        mix(tensors[t].numel);
        mix(tensors[t].flags);
    }

    bfo_table_s *tb = new (std::nothrow) bfo_table_s;
    if (!tb) return BFO_EINVAL;
    tb->fingerprint = fp;
    tb->n = n;
    tb->S = S;
    tb->begin = b;
    tb->world = world;
    tb->rank = rank;
    tb->layout = layout;
    tb->runs = runs;
    hipError_t he = hipGetDevice(&tb->device);
    if (he != hipSuccess) {
        delete tb;
        return hipFail(he);
    }
    auto up = [](uint64_t x) { return (x + 255) & ~uint64_t(255); };
    const uint64_t nTiles = bfo::normTiles(S);
    const uint64_t nNorm = nTiles + bfo::normRuns(nTiles) > 0 ? nTiles + bfo::normRuns(nTiles) : 1;
    const uint64_t offTile = 0;
    const uint64_t offLocal = offTile + up(tileWord.size() * sizeof(uint32_t));
    const uint64_t offAddr = offLocal + up(local.size() * sizeof(uint64_t));
    const uint64_t offRng = offAddr + up(addr.size() * sizeof(uint64_t));
    const uint64_t offFlag = offRng + up(rng.size() * sizeof(uint64_t));
    const uint64_t offNorm = offFlag + up(flag.size());
    const uint64_t offNormOff = offNorm + up(nNorm * sizeof(double));
    const uint64_t bytes = offNormOff + up(normOff.size() * sizeof(uint64_t));
    he = hipMalloc(&tb->devBlock, bytes);
    if (he != hipSuccess) {
        delete tb;
        return hipFail(he);
    }
    char *base = static_cast<char *>(tb->devBlock);
    tb->tile = reinterpret_cast<uint32_t *>(base + offTile);
    tb->local = reinterpret_cast<uint64_t *>(base + offLocal);
    tb->addr = reinterpret_cast<uint64_t *>(base + offAddr);
    tb->rng = reinterpret_cast<uint64_t *>(base + offRng);
    tb->flag = reinterpret_cast<uint8_t *>(base + offFlag);
    tb->normPartials = reinterpret_cast<double *>(base + offNorm);
    tb->normOffset = normOff.empty() ? nullptr : reinterpret_cast<uint64_t *>(base + offNormOff);
    if ((he = hipMemcpy(tb->tile, tileWord.data(), tileWord.size() * sizeof(uint32_t),
                        hipMemcpyHostToDevice)) != hipSuccess ||
        (he = hipMemcpy(tb->local, local.data(), local.size() * sizeof(uint64_t), hipMemcpyHostToDevice)) !=
            hipSuccess ||
        (he = hipMemcpy(tb->addr, addr.data(), addr.size() * sizeof(uint64_t), hipMemcpyHostToDevice)) !=
            hipSuccess ||
        (he = hipMemcpy(tb->rng, rng.data(), rng.size() * sizeof(uint64_t), hipMemcpyHostToDevice)) !=
            hipSuccess ||
        (he = hipMemcpy(tb->flag, flag.data(), flag.size(), hipMemcpyHostToDevice)) != hipSuccess ||
        (!normOff.empty() && (he = hipMemcpy(tb->normOffset, normOff.data(), normOff.size() * sizeof(uint64_t),
                                             hipMemcpyHostToDevice)) != hipSuccess)) {
        (void)hipFree(tb->devBlock);
        delete tb;
        return hipFail(he);
    }
    *out = tb;
    return BFO_OK;
}

int bfo_table_create(const bfo_tensor *tensors, uint32_t count, uint32_t world, uint32_t rank,
                     bfo_table *out) {
    return bfo_table_create_layout(tensors, count, world, rank, BFO_LAYOUT_FLAT, out);
}

int bfo_table_destroy(bfo_table table) {
    if (!table) return BFO_OK;
    hipError_t he = hipFree(table->devBlock);
    delete table;
    return he == hipSuccess ? BFO_OK : hipFail(he);
}

int bfo_table_info(bfo_table table, uint64_t *n, uint64_t *begin, uint64_t *end) {
    if (!table) return BFO_EINVAL;
    if (n) *n = table->n;
    if (begin) *begin = table->begin;
    if (end) *end = table->begin + table->S;
    return BFO_OK;
}

int bfo_table_runs(bfo_table table, bfo_run *out, uint32_t capacity, uint32_t *count) {
    if (!table || !count) return BFO_EINVAL;
    *count = uint32_t(table->runs.size());
    if (out) {
        if (capacity < table->runs.size()) return BFO_ERANGE;
        std::memcpy(out, table->runs.data(), table->runs.size() * sizeof(bfo_run));
    }
    return BFO_OK;
}

}  // extern "C"

namespace {

int checkDevice(const bfo_table_s *t) {
    int dev = -1;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return hipFail(he);
    return dev == t->device ? BFO_OK : BFO_EDEVICE;
}

// "第 13 讲" §1.7: bias correction 1 - beta^t, formed in binary64 and
// rounded once to binary32; 1 when correction is off.
float biasCorrection(float beta, uint64_t t, int32_t on) {
    return on ? float(1.0 - std::pow(double(beta), double(t))) : 1.0f;
}

bfo::StepScalars stepScalars(const bfo_adamw_hparams &hp, float lr, float bc1, float bc2) {
    bfo::StepScalars s;
    s.lr = lr;
    s.beta1 = hp.beta1;
    s.beta2 = hp.beta2;
    s.eps = hp.eps;
    s.wd = hp.weight_decay;
    s.bc1 = bc1;
    s.bc2 = bc2;
    return s;
}

// Validation and launch shared by adamw_sr_step and adamw_sr_step_scheduled.
// Argument checks of an update (and, for the one-call step, of its norm:
// `out` and `workspace`, which must not overlap the arrays either).
int checkStep(bfo_table table, uint16_t *params, const uint16_t *grads, float *master, float *m, float *v,
              const float *scale, const int32_t *skip, int rounding, const bfo_norm_result *out = nullptr,
              const void *workspace = nullptr) {
    if (!table) return BFO_EINVAL;
    if (rounding != BFO_ROUND_SR && rounding != BFO_ROUND_RNE) return BFO_EINVAL;
    const uint64_t S = table->S;
    if (S && (!params || !grads || !m || !v)) return BFO_EINVAL;
    if (!alignedTo(params, 2) || !alignedTo(grads, 2) || !alignedTo(master, 16) || !alignedTo(m, 16) ||
        !alignedTo(v, 16) || !alignedTo(scale, 4) || !alignedTo(skip, 4) || !alignedTo(out, 16) ||
        !alignedTo(workspace, 8))
        return BFO_EMISALIGNED;
    const uint64_t pg = 2 * pgElems(table);
    if (anyOverlap({span(params, pg), span(grads, pg), span(master, 4 * S), span(m, 4 * S), span(v, 4 * S),
                    span(scale, 4), span(skip, 4), span(out, sizeof(bfo_norm_result)),
                    span(workspace, bfo::normWorkspaceBytes(S))}))
        return BFO_EINVAL;
    return checkDevice(table);
}

int launchStep(bfo_table table, uint16_t *params, const uint16_t *grads, float *master, float *m, float *v,
               const bfo::StepScalars &s, const float *scale, const int32_t *skip, uint64_t seed, int rounding,
               const bfo::StepSchedule *sched, void *stream) {
    int rc = checkStep(table, params, grads, master, m, v, scale, skip, rounding);
    if (rc != BFO_OK) return rc;
    const uint64_t S = table->S;
    if (S == 0) return BFO_OK;
    const int pgVec = alignedTo(params, 16) && alignedTo(grads, 16) ? 1 : 0;
    hipError_t he = bfo::launchAdamw(params, grads, master, m, v, S, table->view(), pgVec, s, scale, skip, seed,
                                     rounding, sched, static_cast<hipStream_t>(stream));
    return he == hipSuccess ? BFO_OK : hipFail(he);
}

}  // namespace

extern "C" {

int bfo_norm_workspace_bytes(bfo_table table, uint64_t *bytes) {
    if (!table || !bytes) return BFO_EINVAL;
    *bytes = bfo::normWorkspaceBytes(table->S);
    return BFO_OK;
}

int grad_global_norm(bfo_table table, const uint16_t *grads, float max_norm, void *workspace,
                     bfo_norm_result *out, void *stream) {
    if (!table || !out || (table->S && !grads)) return BFO_EINVAL;
    if (!(max_norm > 0.0f)) return BFO_EINVAL;                // also refuses NaN; +inf disables the clip
    if (!alignedTo(grads, 2) || !alignedTo(out, 16) || !alignedTo(workspace, 8)) return BFO_EMISALIGNED;
    const uint64_t wsBytes = bfo::normWorkspaceBytes(table->S);
    if (anyOverlap({span(grads, 2 * pgElems(table)), span(out, sizeof(bfo_norm_result)),
                    span(workspace, wsBytes)}))
        return BFO_EINVAL;
    int rc = checkDevice(table);
    if (rc != BFO_OK) return rc;
    double *partials = workspace ? static_cast<double *>(workspace) : table->normPartials;
    hipError_t he = bfo::launchNorm(grads, table->S, table->view(), alignedTo(grads, 16) ? 1 : 0,
                                    table->layout == BFO_LAYOUT_FLAT, max_norm, partials, out,
                                    static_cast<hipStream_t>(stream));
    return he == hipSuccess ? BFO_OK : hipFail(he);
}

}  // extern "C"

namespace {

// Per-device address of the library's fixed norm array, looked up once per
// device (with that device current) on the first allocation-free call there.
constexpr int kMaxDevices = 64;
std::mutex gScratchLock;
void *gScratch[kMaxDevices] = {};

int staticScratch(int device, void **out) {
    if (device < 0 || device >= kMaxDevices) return BFO_EDEVICE;
    std::lock_guard<std::mutex> hold(gScratchLock);
    if (!gScratch[device]) {
        void *p = nullptr;
        const hipError_t he = bfo::staticScratchAddress(&p);
        if (he != hipSuccess) return hipFail(he);
        gScratch[device] = p;
    }
    *out = gScratch[device];
    return BFO_OK;
}

}  // namespace

extern "C" {

int grad_global_norm_noalloc(bfo_table table, const uint16_t *grads, float max_norm, bfo_norm_result *out,
                             void *stream) {
    if (!table || !out || (table->S && !grads)) return BFO_EINVAL;
    if (table->S > bfo::kStaticNormMaxElems) return BFO_ERANGE;
    if (!(max_norm > 0.0f)) return BFO_EINVAL;
    if (!alignedTo(grads, 2) || !alignedTo(out, 16)) return BFO_EMISALIGNED;
    if (anyOverlap({span(grads, 2 * pgElems(table)), span(out, sizeof(bfo_norm_result))})) return BFO_EINVAL;
    int rc = checkDevice(table);
    if (rc != BFO_OK) return rc;
    void *partials = nullptr;
    rc = staticScratch(table->device, &partials);
    if (rc != BFO_OK) return rc;
    hipError_t he = bfo::launchNorm(grads, table->S, table->view(), alignedTo(grads, 16) ? 1 : 0,
                                    table->layout == BFO_LAYOUT_FLAT, max_norm, static_cast<double *>(partials),
                                    out, static_cast<hipStream_t>(stream));
    return he == hipSuccess ? BFO_OK : hipFail(he);
}

int adamw_sr_step(bfo_table table, uint16_t *params, const uint16_t *grads, float *master, float *m,
                  float *v, const bfo_adamw_hparams *hp, const float *scale, const int32_t *skip, uint64_t t,
                  uint64_t seed, int rounding, void *stream) {
    if (!hp || t == 0) return BFO_EINVAL;
    bfo::StepScalars s = stepScalars(*hp, hp->lr, biasCorrection(hp->beta1, t, hp->bias_correction),
                                     biasCorrection(hp->beta2, t, hp->bias_correction));
    return launchStep(table, params, grads, master, m, v, s, scale, skip, seed, rounding, nullptr, stream);
}

int adamw_sr_step_with_norm(bfo_table table, uint16_t *params, const uint16_t *grads, float *master, float *m,
                            float *v, const bfo_adamw_hparams *hp, float max_norm, void *workspace,
                            bfo_norm_result *out, const int32_t *skip, uint64_t t, uint64_t seed, int rounding,
                            void *stream) {
    if (!hp || t == 0 || !out || !(max_norm > 0.0f)) return BFO_EINVAL;
    int rc = checkStep(table, params, grads, master, m, v, nullptr, skip, rounding, out, workspace);
    if (rc != BFO_OK) return rc;
    const bfo::StepScalars s = stepScalars(*hp, hp->lr, biasCorrection(hp->beta1, t, hp->bias_correction),
                                           biasCorrection(hp->beta2, t, hp->bias_correction));
    const uint64_t S = table->S;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int gVec = alignedTo(grads, 16) ? 1 : 0;
    const int pgVec = gVec && alignedTo(params, 16) ? 1 : 0;
    const bool flat = table->layout == BFO_LAYOUT_FLAT;
    const uint64_t ntiles = bfo::normTiles(S);
    hipError_t he;
    if (ntiles > 0 && ntiles <= bfo::kNormSmallTiles) {
        he = bfo::launchSmallStep(params, grads, master, m, v, S, table->view(), gVec, pgVec, flat, max_norm, out, s,
                                  skip, seed, rounding, st);
    } else {
        double *partials = workspace ? static_cast<double *>(workspace) : table->normPartials;
        he = bfo::launchNorm(grads, S, table->view(), gVec, flat, max_norm, partials, out, st);
        if (he == hipSuccess && S)
            he = bfo::launchAdamw(params, grads, master, m, v, S, table->view(), pgVec, s, &out->scale, skip, seed,
                                  rounding, nullptr, st);
    }
    return he == hipSuccess ? BFO_OK : hipFail(he);
}

int bfo_step_scalars_fill(const bfo_adamw_hparams *hp, uint64_t t, float lr, uint64_t seed,
                          bfo_step_scalars *out) {
    if (!hp || !out || t == 0) return BFO_EINVAL;
    *out = bfo_step_scalars{};
    out->lr = lr;
    out->bc1 = biasCorrection(hp->beta1, t, hp->bias_correction);
    out->bc2 = biasCorrection(hp->beta2, t, hp->bias_correction);
    out->t = t;
    out->seed = seed;
    return BFO_OK;
}

int adamw_sr_step_scheduled(bfo_table table, uint16_t *params, const uint16_t *grads, float *master, float *m,
                            float *v, const bfo_adamw_hparams *hp, const bfo_step_scalars *steps,
                            uint64_t count, const uint64_t *cursor, const float *scale, const int32_t *skip,
                            int rounding, void *stream) {
    if (!hp || !steps || !cursor) return BFO_EINVAL;
    if (!alignedTo(steps, 16) || !alignedTo(cursor, 8)) return BFO_EMISALIGNED;
    const uint64_t S = table ? table->S : 0;
    const uint64_t pg = table ? 2 * pgElems(table) : 0;
    if (count > UINT64_MAX / sizeof(bfo_step_scalars) ||
        anyOverlap({span(steps, count * sizeof(bfo_step_scalars)), span(params, pg), span(master, 4 * S),
                    span(m, 4 * S), span(v, 4 * S)}) ||
        anyOverlap({span(cursor, 8), span(params, pg), span(master, 4 * S), span(m, 4 * S), span(v, 4 * S)}))
        return BFO_EINVAL;
    const bfo::StepSchedule sched{steps, count, cursor};
    return launchStep(table, params, grads, master, m, v, stepScalars(*hp, 0.0f, 1.0f, 1.0f), scale, skip, 0,
                      rounding, &sched, stream);
}

int bfo_cursor_advance(uint64_t *cursor, void *stream) {
    if (!cursor) return BFO_EINVAL;
    if (!alignedTo(cursor, 8)) return BFO_EMISALIGNED;
    hipError_t he = bfo::launchCursorAdvance(cursor, static_cast<hipStream_t>(stream));
    return he == hipSuccess ? BFO_OK : hipFail(he);
}

int master_to_bf16(bfo_table table, const float *master, uint16_t *params, uint64_t seed, int rounding,
                   void *stream) {
    if (!table) return BFO_EINVAL;
    if (rounding != BFO_ROUND_SR && rounding != BFO_ROUND_RNE) return BFO_EINVAL;
    const uint64_t S = table->S;
    if (S && (!master || !params)) return BFO_EINVAL;
    if (!alignedTo(master, 16) || !alignedTo(params, 2)) return BFO_EMISALIGNED;
    if (anyOverlap({span(master, 4 * S), span(params, 2 * pgElems(table))})) return BFO_EINVAL;
    int rc = checkDevice(table);
    if (rc != BFO_OK) return rc;
    return bfo::rebuildParams(table, master, params, seed, rounding, static_cast<hipStream_t>(stream));
}

int master_to_bf16_sr(bfo_table table, const float *master, uint16_t *params, uint64_t seed,
                      void *stream) {
    return master_to_bf16(table, master, params, seed, BFO_ROUND_SR, stream);
}

int bfo_rng_dump(uint64_t first, uint64_t count, uint64_t seed, uint16_t *out, void *stream) {
    if (count && !out) return BFO_EINVAL;
    if (!alignedTo(out, 2)) return BFO_EMISALIGNED;
    if (count > UINT64_MAX - first) return BFO_ERANGE;
    hipError_t he = bfo::launchRngDump(first, count, seed, out, static_cast<hipStream_t>(stream));
    return he == hipSuccess ? BFO_OK : hipFail(he);
}

int bfo_decay_mask_dump(bfo_table table, uint8_t *out, void *stream) {
    if (!table || (table->S && !out)) return BFO_EINVAL;
    int rc = checkDevice(table);
    if (rc != BFO_OK) return rc;
    hipError_t he = bfo::launchDecayDump(table->view(), table->S, out, static_cast<hipStream_t>(stream));
    return he == hipSuccess ? BFO_OK : hipFail(he);
}

int bfo_stream_mix(uint16_t *params, const uint16_t *grads, float *master, float *m, float *v, uint64_t count,
                   uint32_t key, int mode, void *stream) {
    if (mode != BFO_MIX_BOTH && mode != BFO_MIX_READS && mode != BFO_MIX_WRITES) return BFO_EINVAL;
    if (count == 0) return BFO_OK;
    if (!params || !grads || !m || !v) return BFO_EINVAL;
    if (!alignedTo(params, 16) || !alignedTo(grads, 16) || !alignedTo(master, 16) || !alignedTo(m, 16) ||
        !alignedTo(v, 16))
        return BFO_EMISALIGNED;
    hipError_t he =
        bfo::launchStreamMix(params, grads, master, m, v, count, key, mode, static_cast<hipStream_t>(stream));
    return he == hipSuccess ? BFO_OK : hipFail(he);
}

int bfo_spread_layout(const uint64_t *bytes, uint32_t count, uint64_t *offsets, uint64_t *total) {
    if (!total || (count && (!bytes || !offsets))) return BFO_EINVAL;
    uint64_t end = 0;
    for (uint32_t k = 0; k < count; ++k) {
        uint64_t start = 0;
        if (k) {
            if (end > UINT64_MAX - 2 * BFO_REGION_BYTES) return BFO_ERANGE;
            start = (end + BFO_REGION_BYTES - 1) / BFO_REGION_BYTES * BFO_REGION_BYTES;
            // the fourth region of every 64 GiB-aligned block starts no array
            if ((start / BFO_REGION_BYTES) % 4 == 3) start += BFO_REGION_BYTES;
        }
        if (bytes[k] > UINT64_MAX - start) return BFO_ERANGE;
        offsets[k] = start;
        end = start + bytes[k];
    }
    *total = end;
    return BFO_OK;
}

const char *bfo_status_string(int status) {
    switch (status) {
        case BFO_OK: return "ok";
        case BFO_EINVAL: return "invalid argument";
        case BFO_ENOTDIVISIBLE: return "length not divisible by the shard count";
        case BFO_ERANGE: return "rank or range out of bounds";
        case BFO_EMISALIGNED: return "pointer not aligned as required";
        case BFO_ETABLE: return "tensor table not contiguous from 0 or undefined flag bits";
        case BFO_EHIP: return "HIP runtime call failed";
        case BFO_EDEVICE: return "current device differs from the table's device";
        case BFO_EIO: return "file could not be created, written or read";
        case BFO_EFORMAT: return "checkpoint file does not match the table or is incomplete";
        case BFO_ENOTFOUND: return "no such checkpoint";
        default: return "unknown status";
    }
}

int bfo_last_hip_error(void) { return gLastHipError; }

}  // extern "C"
