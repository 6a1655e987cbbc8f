// bfo_internal.hpp -- layout constants and kernel launchers shared by the
// host ABI (bfo_abi.cpp) and the gfx950 kernels (bfo_kernels.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/bf16opt.h"

namespace bfo {

// One workgroup of the streaming kernels: 256 lanes = 4 wave64s.
constexpr int kBlock = 256;
// Both kernels that step through the shard's tiles give a workgroup one
// tile of kTileElems elements.  Each lane of the rebuild owns kVecPerLane
// 8-element vectors of it (16 bytes of bf16, 32 bytes of fp32 per vector
// and array); each lane of the update owns kQuadsPerLane 4-element quads
// (8 bytes of bf16, 16 bytes of fp32).
constexpr int kVecPerLane = 2;
constexpr uint64_t kTileVecs = uint64_t(kBlock) * kVecPerLane;  // vectors per workgroup
constexpr uint64_t kTileElems = kTileVecs * 8;                  // elements per workgroup
constexpr int kQuadsPerLane = 4;
static_assert(uint64_t(kBlock) * kQuadsPerLane * 4 == kTileElems, "the update's quads fill a tile");
// Shard lookup: one 32-bit word per tile.  Bits 0..30 give the run that
// holds the tile's first element; bit 31 is set when the tile crosses into
// another run (lanes then scan forward from that run).
constexpr uint32_t kTileMixed = 0x80000000u;

// Grad-norm partition: stage 1 gives each workgroup one tile of
// kNormTileVecs vectors (kNormVecPerLane per lane, strided by the block; the
// last vector may be partial) and writes one binary64 partial per tile.  When there are more than
// kNormFinishDirect tiles, an intermediate pass sums each run of
// kNormReduceRun partials in its own workgroup; stage 2 (one workgroup) sums
// what is left in a fixed order.  All of it depends only on the shard length.
constexpr int kNormVecPerLane = 4;
constexpr uint64_t kNormTileVecs = uint64_t(kBlock) * kNormVecPerLane;
constexpr int kNormFinishBlock = 1024;
constexpr uint64_t kNormFinishDirect = 32768;
constexpr uint64_t kNormReduceRun = 4096;
// Shards of at most this many tiles run both stages in one workgroup.
constexpr uint32_t kNormSmallTiles = 8;

inline uint64_t normTiles(uint64_t S) { return ((S + 7) / 8 + kNormTileVecs - 1) / kNormTileVecs; }
inline uint64_t normRuns(uint64_t ntiles) {
    return ntiles > kNormFinishDirect ? (ntiles + kNormReduceRun - 1) / kNormReduceRun : 0;
}
// Device bytes of binary64 partials the norm of an S-element shard writes
// and reads back (none when one workgroup does all of it).
inline uint64_t normWorkspaceBytes(uint64_t S) {
    const uint64_t t = normTiles(S);
    return t <= kNormSmallTiles ? 0 : (t + normRuns(t)) * sizeof(double);
}

// The allocation-free norm entry point keeps its partials in a fixed device
// array of the library (one per GPU): 2^20 binary64 values, enough for the
// partition of any shard up to kStaticNormMaxElems elements.
constexpr uint64_t kStaticScratchBytes = uint64_t(8) << 20;
constexpr uint64_t kStaticNormMaxElems = uint64_t(1048320) * kNormTileVecs * 8;
// Device address of that array on the current device (bfo_kernels.hip).
hipError_t staticScratchAddress(void **out);

// Device view of a table's shard plan.  A run is a stretch of shard-local
// elements [local[k], local[k+1]) that sits at consecutive positions of the
// caller's params/grads arrays (starting at addr[k]) and of the flat buffer
// (global index rng[k], which keys the rounding draws), with one decay flag.
// local has nruns + 1 entries, the last being UINT64_MAX so scans stop.
struct ShardView {
    const uint32_t *tile;
    const uint64_t *local;
    const uint64_t *addr;
    const uint64_t *rng;
    const uint8_t *flag;
    // Per-tensor tables: for each grad-norm tile, the constant (position in
    // the grads array) - (shard element) when the whole tile lies in one run
    // and that difference is a multiple of 8, else kNoNormOffset.  Null for
    // flat tables (whose grads are shard-local anyway).
    const uint64_t *normOffset;
    // Flat tables: the shard's first global index (shard element j is then
    // params/grads position j and global index flatBegin + j); UINT64_MAX for
    // per-tensor tables.
    uint64_t flatBegin;
};
constexpr uint64_t kNoNormOffset = UINT64_MAX;

struct StepScalars {
    float lr, beta1, beta2, eps, wd, bc1, bc2;
};

// Device-resident per-step scalars of a scheduled update: steps[*cursor]
// (of count) replaces lr, bc1, bc2 and the seed at run time.
struct StepSchedule {
    const bfo_step_scalars *steps = nullptr;
    uint64_t count = 0;
    const uint64_t *cursor = nullptr;
};

// Records a failed HIP call for bfo_last_hip_error() and returns BFO_EHIP.
int recordHipFailure(hipError_t e);

// What the checkpoint code needs to know about a table (bfo_abi.cpp).
struct TableFacts {
    uint64_t n, S;
    uint32_t world, rank;
    int layout;
    uint64_t fingerprint;  // FNV-1a over every tensor's offset, numel and flags
    const bfo_run *runs;
    uint32_t nruns;
};
TableFacts tableFacts(const bfo_table_s *table);
// master_to_bf16 without the host-side argument checks (the checkpoint
// loader, which has checked its own arguments).
int rebuildParams(bfo_table_s *table, const float *master, uint16_t *params, uint64_t seed, int rounding,
                  hipStream_t stream);

// Launchers (bfo_kernels.hip).  Shapes are checked by the caller: M, m, v
// hold S shard-local elements, 16-byte aligned; P and G are addressed
// through the runs and are at least 2-byte aligned; pgVec says whether P
// and G are 16-byte aligned (then 8-element vectors at 8-aligned positions
// use 16-byte accesses).
hipError_t launchNorm(const uint16_t *g, uint64_t S, ShardView sv, int pgVec, bool flat, float maxNorm,
                      double *partials, bfo_norm_result *out, hipStream_t stream);
// sched: NULL for scalars passed by value (s, seed), else read on the device.
hipError_t launchAdamw(uint16_t *P, const uint16_t *G, float *M, float *m, float *v, uint64_t S,
                       ShardView sv, int pgVec, StepScalars s, const float *scale, const int32_t *skip,
                       uint64_t seed, int rounding, const StepSchedule *sched, hipStream_t stream);
hipError_t launchCursorAdvance(uint64_t *cursor, hipStream_t stream);
// Norm, clip scale and update in one launch, for 0 < normTiles(S) <= kNormSmallTiles.
// gVec: G 16-byte aligned (the norm's fast path); pgVec as for launchAdamw.
hipError_t launchSmallStep(uint16_t *P, const uint16_t *G, float *M, float *m, float *v, uint64_t S, ShardView sv,
                           int gVec, int pgVec, bool flat, float maxNorm, bfo_norm_result *out, StepScalars s,
                           const int32_t *skip, uint64_t seed, int rounding, hipStream_t stream);
hipError_t launchMasterToBf16(const float *M, uint16_t *P, uint64_t S, ShardView sv, int pgVec,
                              uint64_t seed, int rounding, hipStream_t stream);
hipError_t launchRngDump(uint64_t first, uint64_t count, uint64_t seed, uint16_t *out,
                         hipStream_t stream);
hipError_t launchDecayDump(ShardView sv, uint64_t S, uint8_t *out, hipStream_t stream);
hipError_t launchStreamMix(uint16_t *P, const uint16_t *G, float *M, float *m, float *v, uint64_t count,
                           uint32_t key, int mode, hipStream_t stream);

// Outlier detector state in device memory: a ring of the last `window`
// finite values (oldest at `head` once full).
struct OutlierState {
    uint32_t window, count, head, pad;
    float values[1];  // [window]
};
constexpr uint32_t kOutlierMaxWindow = 4096;

hipError_t launchOutlierUpdate(OutlierState *state, const float *value, float threshold, float *z,
                               int32_t *skip, hipStream_t stream);
hipError_t launchOutlierReset(OutlierState *state, uint32_t window, hipStream_t stream);

}  // namespace bfo
