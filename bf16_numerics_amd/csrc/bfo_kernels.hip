// bfo_kernels.hip -- gfx950 kernels of the mixed-precision AdamW step.
//
// Every kernel here is bound by HBM bandwidth: each element is touched once
// per launch, so the design goal is full-width coalesced loads and stores
// (every wave instruction over one contiguous stretch where the plan allows),
// several in flight per lane, and enough workgroups (>> 256 CUs) to keep
// every channel busy.  Nothing is a contraction, so there is no MFMA.
//
// Shard plan.  The shard's S elements are shard-local positions j; runs map
// them to positions in the caller's params/grads arrays (addr) and to global
// indices of the flat buffer (rng, which keys the rounding draws).  Work is
// cut into pieces of consecutive elements -- 4-element quads in the update,
// 8-element vectors in the rebuild and the norm -- and each piece is
//   - regular: it lies in one run and P/G are 16-byte aligned: every array
//     moves as one full-width access per piece (the common case);
//   - semi-regular: one run, but P/G not 16-byte aligned (misaligned flat
//     shards): fp32 state as full-width accesses, bf16 P/G per element;
//   - per element: the piece crosses runs or the shard end.
// A piece's draws come from one Philox block (eight consecutive global
// indices) when it sits inside one and from two otherwise.
//
// Floating point.  The update is a fixed sequence of binary32 operations
// (one IEEE operation per line of the per-element function), built with
// -ffp-contract=off so the compiler fuses nothing that is not written as
// fma, and with HIP's default correctly rounded fp32 division and sqrt and
// fp32 denormal support.  The norm accumulates in binary64, where every
// square of a bf16 value is exact.
//
// Page references (title, section):
//   "04 · 多 GPU 与混合精度": §2.2 the AdamW element update and the two-FMA
//     lerp; §2.3 stochastic rounding; §3.2 sharding; §4 grad norm and clip;
//     §5.2 rebuilding bf16 weights from the master with the same draws.
//   "第 13 讲：扩大 LLM——优化与并行训练": §1.7 bias correction and
//     decoupled weight decay.
//   Philox4x32-10: Salmon, Moraes, Dror, Shaw, SC'11.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bfo_internal.hpp"

namespace bfo {
namespace {

// ---------------------------------------------------------------------------
// Counter-based draws: Philox4x32-10.  One block of four 32-bit words serves
// the aligned group of 8 global indices (index >> 3).
// ---------------------------------------------------------------------------
struct U32x4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ U32x4 philox10(uint64_t group, uint32_t k0, uint32_t k1) {
    constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
    constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
    uint32_t c0 = uint32_t(group), c1 = uint32_t(group >> 32), c2 = 0u, c3 = 0u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t pa = uint64_t(kMulA) * c0;
        const uint64_t pb = uint64_t(kMulB) * c2;
        const uint32_t n0 = uint32_t(pb >> 32) ^ c1 ^ k0;
        const uint32_t n2 = uint32_t(pa >> 32) ^ c3 ^ k1;
        c1 = uint32_t(pb);
        c3 = uint32_t(pa);
        c0 = n0;
        c2 = n2;
        k0 += kWeylA;
        k1 += kWeylB;
    }
    return {c0, c1, c2, c3};
}

// 16-bit draw for position p (0..7) of a group: word p>>1, low half for even p.
__device__ __forceinline__ uint32_t drawOf(const U32x4 &w, int p) {
    const uint32_t word = (p >> 1) == 0 ? w.x : (p >> 1) == 1 ? w.y : (p >> 1) == 2 ? w.z : w.w;
    return (p & 1) ? (word >> 16) : (word & 0xFFFFu);
}

// Draws of the 8 consecutive global indices rng0 .. rng0+7.
__device__ __forceinline__ void draws8(uint64_t rng0, uint32_t k0, uint32_t k1, uint32_t d[8]) {
    const U32x4 a = philox10(rng0 >> 3, k0, k1);
    const int s = int(rng0 & 7);
    if (s == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] = drawOf(a, e);
    } else {
        const U32x4 b = philox10((rng0 >> 3) + 1, k0, k1);
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] = (s + e) < 8 ? drawOf(a, s + e) : drawOf(b, s + e - 8);
    }
}

// ---------------------------------------------------------------------------
// binary32 -> bf16 write-back.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool isNanBits(uint32_t b) { return (b & 0x7FFFFFFFu) > 0x7F800000u; }

// Stochastic rounding: step the truncated pattern one unit (next bf16 away
// from zero) when the 16 discarded bits exceed the draw.
__device__ __forceinline__ uint32_t roundSR(float x, uint32_t r) {
    const uint32_t b = __float_as_uint(x);
    const uint32_t h = (b >> 16) + ((b & 0xFFFFu) > r ? 1u : 0u);
    return isNanBits(b) ? ((b >> 16) | 0x40u) : h;
}

// Round to nearest even: add just under half a unit, plus the kept LSB.
__device__ __forceinline__ uint32_t roundRNE(float x) {
    const uint32_t b = __float_as_uint(x);
    const uint32_t h = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
    return isNanBits(b) ? ((b >> 16) | 0x40u) : h;
}

__device__ __forceinline__ float bf16Lo(uint32_t word) { return __uint_as_float(word << 16); }
__device__ __forceinline__ float bf16Hi(uint32_t word) { return __uint_as_float(word & 0xFFFF0000u); }
__device__ __forceinline__ float bf16At(const uint16_t *p, uint64_t i) { return __uint_as_float(uint32_t(p[i]) << 16); }

template <int kRound>
__device__ __forceinline__ uint32_t writeBack(float p, uint32_t draw) {
    if constexpr (kRound == BFO_ROUND_SR) return roundSR(p, draw);
    else return roundRNE(p);
}

// Eight consecutive bf16 patterns from a 2-byte-aligned address, packed as in
// a 16-byte load.
__device__ __forceinline__ uint4 load8Narrow(const uint16_t *p) {
    return make_uint4(uint32_t(p[0]) | (uint32_t(p[1]) << 16), uint32_t(p[2]) | (uint32_t(p[3]) << 16),
                      uint32_t(p[4]) | (uint32_t(p[5]) << 16), uint32_t(p[6]) | (uint32_t(p[7]) << 16));
}

// Cache policy.  Nontemporal loads and stores (the lines are marked for
// early eviction from the caches) for data that a kernel touches once:
//   - the grads, only read, in the norm and in the update: their lines then
//     do not push out the dirty lines of what the previous kernel stored;
//     after an update, the norm's read of the next grads no longer has to
//     drain the update's write-back as it goes (in-step norm on the 1.5B
//     shard 109 -> 66 us; the whole step 2.5% faster, 3% also when fresh
//     grads are written before every step, as a backward pass would);
//   - everything else the update moves, except the params when there is no
//     master: m, v and the master loaded and stored nontemporally, and the
//     params (written, never read, when there is a master) stored so.  With
//     the update's wave-contiguous plan (below) this policy ran 2.1-2.4%
//     faster than plain m, v and master accesses (1.5B shard, 7B state), and
//     plan and policy together 1.6-3.3% faster than the plan they replaced
//     (a lane owning two 8-element vectors, so that each fp32 instruction
//     covered half of every 32-byte piece), where the same policy had been
//     3-8% slower than plain accesses.  Without a master the params are read
//     and written back; nontemporal accesses of them made that update 4%
//     slower, so they stay plain;
//   - the rebuild: nontemporal master loads (4-6% faster than plain ones on
//     its 4 B read + 2 B write pattern) and params stores (a further 4-5%).
typedef unsigned int U32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int U32x2v __attribute__((ext_vector_type(2)));
typedef float F32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 loadOnce16(const uint16_t *p, uint64_t vec) {
    const U32x4v t = __builtin_nontemporal_load(reinterpret_cast<const U32x4v *>(p) + vec);
    return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void storeOnce16(uint16_t *p, uint64_t vec, const uint4 &x) {
    __builtin_nontemporal_store(U32x4v{x.x, x.y, x.z, x.w}, reinterpret_cast<U32x4v *>(p) + vec);
}

// Loads and stores with the nontemporal hint on or off at compile time.
template <bool kNt, typename T>
__device__ __forceinline__ T loadHint(const T *p) {
    if constexpr (kNt) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool kNt, typename T>
__device__ __forceinline__ void storeHint(T *p, const T &x) {
    if constexpr (kNt) __builtin_nontemporal_store(x, p);
    else *p = x;
}

// Four consecutive bf16 patterns from a 2-byte-aligned address, packed as in
// an 8-byte load.
__device__ __forceinline__ U32x2v load4Narrow(const uint16_t *p) {
    return U32x2v{uint32_t(p[0]) | (uint32_t(p[1]) << 16), uint32_t(p[2]) | (uint32_t(p[3]) << 16)};
}

// ---------------------------------------------------------------------------
// Shard plan lookups.
// ---------------------------------------------------------------------------
// Where a piece of consecutive shard elements (an 8-element vector of the
// rebuild and the norm, a 4-element quad of the update) sits.
struct Place {
    uint32_t run;   // run holding the piece's first element
    bool inRun;     // all its elements exist and lie in that run
    uint64_t addr0; // P/G position of the first element
    uint64_t rng0;  // global index of the first element
};

__device__ __forceinline__ Place placeVector(const ShardView &sv, uint32_t tileWord, uint64_t j0, uint64_t S) {
    Place pl;
    if (sv.flatBegin != UINT64_MAX && !(tileWord & kTileMixed)) {
        // Flat table, tile inside one run: positions follow from j0 alone, so
        // no lookup stands between the lane and its params/grads access.
        pl.run = tileWord;
        pl.inRun = j0 + 8 <= S;
        pl.addr0 = j0;
        pl.rng0 = sv.flatBegin + j0;
        return pl;
    }
    uint32_t k = tileWord & ~kTileMixed;
    uint64_t runEnd = UINT64_MAX;
    if (tileWord & kTileMixed) {
        while (sv.local[k + 1] <= j0) ++k;
        runEnd = sv.local[k + 1];
    }
    pl.run = k;
    pl.inRun = j0 + 8 <= S && j0 + 8 <= runEnd;
    const uint64_t off = j0 - sv.local[k];
    pl.addr0 = sv.addr[k] + off;
    pl.rng0 = sv.rng[k] + off;
    return pl;
}

// Element j: advances k to its run, returns its P/G position and global index.
__device__ __forceinline__ void placeElement(const ShardView &sv, uint32_t &k, uint64_t j, uint64_t &addr,
                                             uint64_t &rng) {
    while (sv.local[k + 1] <= j) ++k;
    const uint64_t off = j - sv.local[k];
    addr = sv.addr[k] + off;
    rng = sv.rng[k] + off;
}

// Tile words for a workgroup of a partition shifted by `shift` vectors
// (0..7): workgroup t takes vectors [t*kTileVecs - shift, (t+1)*kTileVecs -
// shift), which lie in the plan's tiles t-1 and t.  The rebuild shifts a
// flat shard whose bf16 params start 32, 64 or 96 bytes into a 128-byte
// line so that every wave's 1 KiB of params stores starts on a line (the
// fp32 master, 32 bytes per vector, then starts on a 64-byte boundary).
// Measured on the 1.5B model's shards, one process, against the unshifted
// partition: rebuild +0.8% (rank 1), +2.2% (rank 2), +1.5% (rank 3), equal
// on rank 0; the update loses 0.5-0.8% with the same shift (its master, m
// and v are 12 of its 14 bytes written), so it keeps the plain partition.
struct TileWords {
    uint32_t before, at;  // plan words of tiles t-1 (when shifted) and t
    __device__ __forceinline__ uint32_t of(uint64_t q, uint64_t t) const { return q < t * kTileVecs ? before : at; }
};

__device__ __forceinline__ TileWords tileWords(const ShardView &sv, uint64_t t, uint32_t shift, uint64_t S) {
    const uint64_t planTiles = (S + kTileElems - 1) / kTileElems;
    TileWords w;
    w.at = t < planTiles ? sv.tile[t] : 0u;
    w.before = (shift && t) ? sv.tile[t - 1] : w.at;
    return w;
}

// ---------------------------------------------------------------------------
// One element of the AdamW step.  `w` is the element's decay (wd or 0),
// `old` the fp32 weight before the step; returns the new fp32 weight.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float adamwElem(float graw, float &m, float &v, float old, float w,
                                           const StepScalars &s, float scale) {
    const float g = scale * graw;
    const float m1 = __builtin_fmaf(s.beta1, m, __builtin_fmaf(-s.beta1, g, g));
    const float gg = g * g;
    const float v1 = __builtin_fmaf(s.beta2, v, __builtin_fmaf(-s.beta2, gg, gg));
    const float mh = m1 / s.bc1;
    const float vh = v1 / s.bc2;
    const float den = sqrtf(vh) + s.eps;
    const float u = mh / den;
    const float d = w * old;
    const float sum = u + d;
    const float q = s.lr * sum;
    m = m1;
    v = v1;
    return old - q;
}

enum : int { kNone = 0, kRegular = 1, kSemi = 2, kPerElement = 3 };

// ---------------------------------------------------------------------------
// Fused update.  Workgroup `tile` owns shard-local elements
// [tile * kTileElems, +kTileElems); wave w of it owns the 1024 elements
// from 1024 w, and lane t of the wave the kQuadsPerLane quads (4 consecutive
// elements) at 4 t + 256 k.  Every load and store instruction of a wave so
// covers one contiguous stretch: 1 KiB of an fp32 array (16 bytes a lane)
// or 512 bytes of a bf16 one (8 bytes a lane).  A quad is
//   - regular: in one run, with P and G 16-byte aligned (so the quad's 8
//     bytes of each are aligned): every array moves as one access;
//   - semi-regular: in one run, P and G not 16-byte aligned: fp32 state as
//     16-byte accesses, bf16 P/G per element;
//   - per element: it crosses runs or the shard end.
// A quad's four draws are one half of a Philox block when its global index
// is 0 or 4 mod 8, the other half belonging to the neighbouring lane, and
// come from one or two blocks otherwise.  With a master each lane computes
// the blocks of its own quads.  Without one (fewer bytes per element, so the
// same arithmetic weighs more) lanes 2i and 2i+1 split the work when the
// whole wave allows it (pairDraws): 1.4% faster on the 1.5B shard there, and
// 0.2% slower with a master, where it is not used.  All loads are
// issued before any math.  kScheduled: lr, bias corrections and seed come
// from steps[*cursor] in device memory instead of the launch arguments, so
// one recorded launch serves every step; the cursor is read before the data
// loads are issued and the scalars after, so their round trips overlap.
// ---------------------------------------------------------------------------
__device__ __forceinline__ Place placeQuad(const ShardView &sv, uint32_t tileWord, uint64_t j0, uint64_t S) {
    Place pl;
    if (sv.flatBegin != UINT64_MAX && !(tileWord & kTileMixed)) {
        pl.run = tileWord;
        pl.inRun = j0 + 4 <= S;
        pl.addr0 = j0;
        pl.rng0 = sv.flatBegin + j0;
        return pl;
    }
    uint32_t k = tileWord & ~kTileMixed;
    uint64_t runEnd = UINT64_MAX;
    if (tileWord & kTileMixed) {
        while (sv.local[k + 1] <= j0) ++k;
        runEnd = sv.local[k + 1];
    }
    pl.run = k;
    pl.inRun = j0 + 4 <= S && j0 + 4 <= runEnd;
    const uint64_t off = j0 - sv.local[k];
    pl.addr0 = sv.addr[k] + off;
    pl.rng0 = sv.rng[k] + off;
    return pl;
}

// Draws of the 4 consecutive global indices rng0 .. rng0+3.
__device__ __forceinline__ void draws4(uint64_t rng0, uint32_t k0, uint32_t k1, uint32_t d[4]) {
    const U32x4 a = philox10(rng0 >> 3, k0, k1);
    const int s = int(rng0 & 7);
    if ((s & 3) == 0) {
        const uint32_t lo = s ? a.z : a.x, hi = s ? a.w : a.y;
        d[0] = lo & 0xFFFFu;
        d[1] = lo >> 16;
        d[2] = hi & 0xFFFFu;
        d[3] = hi >> 16;
    } else {
        const U32x4 b = s > 4 ? philox10((rng0 >> 3) + 1, k0, k1) : a;
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = (s + e) < 8 ? drawOf(a, s + e) : drawOf(b, s + e - 8);
    }
}

// Per-element path of the update: elements j0 .. j0+count-1 (stopping at the
// shard end), which may cross runs.
template <bool kMaster, int kRound>
__device__ void adamwElementwise(uint16_t *P, const uint16_t *G, float *M, float *Mom, float *Var, uint64_t j0,
                                 int count, uint64_t S, const ShardView &sv, uint32_t run, const StepScalars &s,
                                 float scale, uint32_t key0, uint32_t key1) {
    uint32_t k = run;
    uint64_t cachedGroup = UINT64_MAX;
    U32x4 cached{0u, 0u, 0u, 0u};
    for (int e = 0; e < count; ++e) {
        const uint64_t j = j0 + uint64_t(e);
        if (j >= S) break;
        uint64_t addr, rng;
        placeElement(sv, k, j, addr, rng);
        const float w = sv.flag[k] ? s.wd : 0.0f;
        uint32_t draw = 0;
        if constexpr (kRound == BFO_ROUND_SR) {
            if ((rng >> 3) != cachedGroup) {
                cachedGroup = rng >> 3;
                cached = philox10(cachedGroup, key0, key1);
            }
            draw = drawOf(cached, int(rng & 7));
        }
        float mm = Mom[j], vv = Var[j];
        const float old = kMaster ? M[j] : bf16At(P, addr);
        const float p = adamwElem(bf16At(G, addr), mm, vv, old, w, s, scale);
        Mom[j] = mm;
        Var[j] = vv;
        if constexpr (kMaster) M[j] = p;
        P[addr] = uint16_t(writeBack<kRound>(p, draw));
    }
}

// Draws for the four quads of this lane when lanes 2i (quads at global
// indices 0 mod 8) and 2i+1 (4 mod 8) hold the two halves of the same four
// Philox blocks: each lane computes two of the blocks and the halves the
// other lane needs cross over by a DPP quad permutation [1,0,3,2].  Returns
// false, with lo/hi untouched, unless every lane of the wave has all four
// quads in runs, at the expected index mod 8, and sharing its partner's
// blocks.  Must be reached by all 64 lanes of the wave together.
__device__ __forceinline__ uint32_t swapPairLanes(uint32_t x) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ bool pairDraws(const Place pl[kQuadsPerLane], const int mode[kQuadsPerLane],
                                          uint32_t key0, uint32_t key1, uint32_t lo[kQuadsPerLane],
                                          uint32_t hi[kQuadsPerLane]) {
    const bool odd = (threadIdx.x & 1) != 0;
    bool ok = true;
#pragma unroll
    for (int k = 0; k < kQuadsPerLane; ++k) {
        const bool inRun = mode[k] == kRegular || mode[k] == kSemi;
        const uint64_t block = inRun ? pl[k].rng0 >> 3 : 0;
        ok = ok && inRun && (uint32_t(pl[k].rng0) & 7u) == (odd ? 4u : 0u);
        const uint64_t partner = (uint64_t(swapPairLanes(uint32_t(block >> 32))) << 32) | swapPairLanes(uint32_t(block));
        ok = ok && partner == block;
    }
    if (__builtin_amdgcn_ballot_w64(ok) != ~0ull) return false;
    // even lanes compute the blocks of quads 0 and 1, odd lanes those of 2 and 3
    const U32x4 a = philox10((odd ? pl[2].rng0 : pl[0].rng0) >> 3, key0, key1);
    const U32x4 b = philox10((odd ? pl[3].rng0 : pl[1].rng0) >> 3, key0, key1);
    // words the partner needs: the even lane's quads use x, y; the odd lane's z, w
    const uint32_t r0 = swapPairLanes(odd ? a.x : a.z), r1 = swapPairLanes(odd ? a.y : a.w);
    const uint32_t r2 = swapPairLanes(odd ? b.x : b.z), r3 = swapPairLanes(odd ? b.y : b.w);
    const uint32_t o0 = odd ? a.z : a.x, o1 = odd ? a.w : a.y, o2 = odd ? b.z : b.x, o3 = odd ? b.w : b.y;
    lo[0] = odd ? r0 : o0; hi[0] = odd ? r1 : o1;
    lo[1] = odd ? r2 : o2; hi[1] = odd ? r3 : o3;
    lo[2] = odd ? o0 : r0; hi[2] = odd ? o1 : r1;
    lo[3] = odd ? o2 : r2; hi[3] = odd ? o3 : r3;
    return true;
}

// Shard-local element of lane threadIdx.x's first quad in workgroup `tile`.
__device__ __forceinline__ uint64_t quadBase(uint64_t tile) {
    return tile * kTileElems + uint64_t(threadIdx.x >> 6) * 1024 + uint64_t(threadIdx.x & 63) * 4;
}

// Draws of quad k: the lane pair's shared blocks when the wave paired, else
// the quad's own block(s).
template <int kRound>
__device__ __forceinline__ void quadDraws(bool paired, uint32_t lo, uint32_t hi, uint64_t rng0, uint32_t key0,
                                          uint32_t key1, uint32_t d[4]) {
    if (paired) {
        d[0] = lo & 0xFFFFu;
        d[1] = lo >> 16;
        d[2] = hi & 0xFFFFu;
        d[3] = hi >> 16;
    } else if constexpr (kRound == BFO_ROUND_SR) {
        draws4(rng0, key0, key1, d);
    } else {
        d[0] = d[1] = d[2] = d[3] = 0u;
    }
}

// The four elements of a quad: m and v updated in place, the new fp32
// weights in pn and their bf16 patterns in hb.
template <int kRound>
__device__ __forceinline__ void stepQuad(const float gr[4], float mm[4], float vv[4], const float old[4], float w,
                                         const StepScalars &s, float scale, const uint32_t d[4], float pn[4],
                                         uint32_t hb[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pn[e] = adamwElem(gr[e], mm[e], vv[e], old[e], w, s, scale);
        hb[e] = writeBack<kRound>(pn[e], d[e]);
    }
}

// The update of one tile by one workgroup (the body of adamwTileKernel and
// of the one-launch small step).  cur: the schedule cursor, read by the
// caller (kScheduled only).
template <bool kMaster, int kRound, bool kScheduled>
__device__ __forceinline__ void adamwTile(uint16_t *__restrict__ P, const uint16_t *__restrict__ G,
                                          float *__restrict__ M, float *__restrict__ Mom, float *__restrict__ Var,
                                          uint64_t S, const ShardView &sv, int pgVec, StepScalars s, float scale,
                                          uint32_t key0, uint32_t key1, uint64_t tile,
                                          const bfo_step_scalars *__restrict__ steps, uint64_t nsteps,
                                          uint64_t cur) {
    constexpr bool kPairDraws = kRound == BFO_ROUND_SR && !kMaster;
    const uint32_t tileWord = sv.tile[tile];
    const uint64_t base = quadBase(tile);

    U32x2v gq[kQuadsPerLane], pq[kQuadsPerLane];
    F32x4 mq[kQuadsPerLane], vq[kQuadsPerLane], wq[kQuadsPerLane];
    Place pl[kQuadsPerLane];
    int mode[kQuadsPerLane];

#pragma unroll
    for (int k = 0; k < kQuadsPerLane; ++k) {
        const uint64_t j0 = base + uint64_t(k) * 256;
        mode[k] = kNone;
        if constexpr (kPairDraws) pl[k].rng0 = 0;   // read by pairDraws for every quad
        if (j0 >= S) continue;
        pl[k] = placeQuad(sv, tileWord, j0, S);
        if (!pl[k].inRun) {
            mode[k] = kPerElement;
            continue;
        }
        mode[k] = (pgVec && (pl[k].addr0 & 3) == 0) ? kRegular : kSemi;
        mq[k] = loadHint<true>(reinterpret_cast<const F32x4 *>(Mom + j0));
        vq[k] = loadHint<true>(reinterpret_cast<const F32x4 *>(Var + j0));
        if constexpr (kMaster) wq[k] = loadHint<true>(reinterpret_cast<const F32x4 *>(M + j0));
        if (mode[k] == kRegular) {
            gq[k] = loadHint<true>(reinterpret_cast<const U32x2v *>(G + pl[k].addr0));
            if constexpr (!kMaster) pq[k] = loadHint<false>(reinterpret_cast<const U32x2v *>(P + pl[k].addr0));
        } else {
            gq[k] = load4Narrow(G + pl[k].addr0);
            if constexpr (!kMaster) pq[k] = load4Narrow(P + pl[k].addr0);
        }
    }
    if constexpr (kScheduled) {
        if (cur >= nsteps) return;    // past the scheduled steps: no update (nothing stored yet)
        const bfo_step_scalars st = steps[cur];
        s.lr = st.lr;
        s.bc1 = st.bc1;
        s.bc2 = st.bc2;
        key0 = uint32_t(st.seed);
        key1 = uint32_t(st.seed >> 32);
    }

    uint32_t pairLo[kQuadsPerLane], pairHi[kQuadsPerLane];
    bool paired = false;
    if constexpr (kPairDraws) paired = pairDraws(pl, mode, key0, key1, pairLo, pairHi);

#pragma unroll
    for (int k = 0; k < kQuadsPerLane; ++k) {
        if (mode[k] == kNone) continue;
        const uint64_t j0 = base + uint64_t(k) * 256;
        if (mode[k] == kPerElement) {
            adamwElementwise<kMaster, kRound>(P, G, M, Mom, Var, j0, 4, S, sv, pl[k].run, s, scale, key0, key1);
            continue;
        }
        uint32_t draws[4];
        quadDraws<kRound>(kPairDraws && paired, pairLo[k], pairHi[k], pl[k].rng0, key0, key1, draws);
        const float w = sv.flag[pl[k].run] ? s.wd : 0.0f;

        const float gr[4] = {bf16Lo(gq[k].x), bf16Hi(gq[k].x), bf16Lo(gq[k].y), bf16Hi(gq[k].y)};
        float mm[4] = {mq[k].x, mq[k].y, mq[k].z, mq[k].w};
        float vv[4] = {vq[k].x, vq[k].y, vq[k].z, vq[k].w};
        float old[4];
        if constexpr (kMaster) {
            old[0] = wq[k].x; old[1] = wq[k].y; old[2] = wq[k].z; old[3] = wq[k].w;
        } else {
            old[0] = bf16Lo(pq[k].x); old[1] = bf16Hi(pq[k].x); old[2] = bf16Lo(pq[k].y); old[3] = bf16Hi(pq[k].y);
        }
        float pn[4];
        uint32_t hb[4];
        stepQuad<kRound>(gr, mm, vv, old, w, s, scale, draws, pn, hb);
        storeHint<true>(reinterpret_cast<F32x4 *>(Mom + j0), F32x4{mm[0], mm[1], mm[2], mm[3]});
        storeHint<true>(reinterpret_cast<F32x4 *>(Var + j0), F32x4{vv[0], vv[1], vv[2], vv[3]});
        if constexpr (kMaster) storeHint<true>(reinterpret_cast<F32x4 *>(M + j0), F32x4{pn[0], pn[1], pn[2], pn[3]});
        if (mode[k] == kRegular) {
            storeHint<kMaster>(reinterpret_cast<U32x2v *>(P + pl[k].addr0),
                               U32x2v{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)});
        } else {
            uint16_t *p = P + pl[k].addr0;
#pragma unroll
            for (int e = 0; e < 4; ++e) p[e] = uint16_t(hb[e]);
        }
    }
}

// ---------------------------------------------------------------------------
// The same update for a tile of a flat shard that lies in one run, with P and
// G 16-byte aligned (almost every tile of a flat shard): the five arrays are
// addressed through buffer resources based at the tile's first element, so a
// lane's addresses are 32-bit offsets from workgroup-uniform bases instead
// of 64-bit pointer arithmetic per access, and the cache policy (the
// nontemporal bit) rides on each buffer instruction.  Same quads, same
// order of operations and same draws as adamwTile, so the same bits.
// Measured against adamwTile on these tiles: 0.3-0.6% faster with a master
// (7B state, 1.5B shards at both params alignments), equal without one.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tileResource(const void *base, uint32_t bytes) {
    // raw buffer: no stride, `bytes` records, the gfx9 default format word
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

constexpr int kPolicyNt = 2;     // cache-policy operand of the buffer builtins: the nontemporal bit
constexpr int kPolicyPlain = 0;

template <bool kMaster, int kRound, bool kScheduled>
__device__ __forceinline__ void adamwTileFlat(uint16_t *__restrict__ P, const uint16_t *__restrict__ G,
                                              float *__restrict__ M, float *__restrict__ Mom,
                                              float *__restrict__ Var, uint64_t S, const ShardView &sv,
                                              StepScalars s, float scale, uint32_t key0, uint32_t key1,
                                              uint64_t tile, const bfo_step_scalars *__restrict__ steps,
                                              uint64_t nsteps, uint64_t cur) {
    constexpr bool kPairDraws = kRound == BFO_ROUND_SR && !kMaster;
    constexpr int kParamsPolicy = kMaster ? kPolicyNt : kPolicyPlain;
    const uint32_t run = sv.tile[tile];
    const uint64_t e0 = tile * kTileElems;
    const uint32_t n = uint32_t(S - e0 < kTileElems ? S - e0 : kTileElems);   // the tile's elements in the shard
    const __amdgpu_buffer_rsrc_t rm = tileResource(Mom + e0, n * 4), rv = tileResource(Var + e0, n * 4);
    const __amdgpu_buffer_rsrc_t rM = tileResource(kMaster ? M + e0 : Mom + e0, n * 4);
    const __amdgpu_buffer_rsrc_t rG = tileResource(G + e0, n * 2), rP = tileResource(P + e0, n * 2);
    const uint32_t lane = (threadIdx.x >> 6) * 1024 + (threadIdx.x & 63) * 4;   // quadBase within the tile

    U32x2v gq[kQuadsPerLane], pq[kQuadsPerLane];
    U32x4v mq[kQuadsPerLane], vq[kQuadsPerLane], wq[kQuadsPerLane];
    Place pl[kQuadsPerLane];
    int mode[kQuadsPerLane];

#pragma unroll
    for (int k = 0; k < kQuadsPerLane; ++k) {
        const uint32_t off = lane + 256u * k;
        mode[k] = off + 4 <= n ? kRegular : (off < n ? kPerElement : kNone);
        pl[k].run = run;
        pl[k].inRun = mode[k] == kRegular;
        pl[k].addr0 = e0 + off;
        pl[k].rng0 = sv.flatBegin + e0 + off;
        if (mode[k] != kRegular) continue;
        mq[k] = __builtin_amdgcn_raw_buffer_load_b128(rm, off * 4, 0, kPolicyNt);
        vq[k] = __builtin_amdgcn_raw_buffer_load_b128(rv, off * 4, 0, kPolicyNt);
        if constexpr (kMaster) wq[k] = __builtin_amdgcn_raw_buffer_load_b128(rM, off * 4, 0, kPolicyNt);
        gq[k] = __builtin_amdgcn_raw_buffer_load_b64(rG, off * 2, 0, kPolicyNt);
        if constexpr (!kMaster) pq[k] = __builtin_amdgcn_raw_buffer_load_b64(rP, off * 2, 0, kParamsPolicy);
    }
    if constexpr (kScheduled) {
        if (cur >= nsteps) return;    // past the scheduled steps: no update (nothing stored yet)
        const bfo_step_scalars st = steps[cur];
        s.lr = st.lr;
        s.bc1 = st.bc1;
        s.bc2 = st.bc2;
        key0 = uint32_t(st.seed);
        key1 = uint32_t(st.seed >> 32);
    }

    uint32_t pairLo[kQuadsPerLane], pairHi[kQuadsPerLane];
    bool paired = false;
    if constexpr (kPairDraws) paired = pairDraws(pl, mode, key0, key1, pairLo, pairHi);
    const float w = sv.flag[run] ? s.wd : 0.0f;

#pragma unroll
    for (int k = 0; k < kQuadsPerLane; ++k) {
        if (mode[k] == kNone) continue;
        const uint32_t off = lane + 256u * k;
        if (mode[k] == kPerElement) {
            adamwElementwise<kMaster, kRound>(P, G, M, Mom, Var, e0 + off, 4, S, sv, run, s, scale, key0, key1);
            continue;
        }
        uint32_t draws[4];
        quadDraws<kRound>(kPairDraws && paired, pairLo[k], pairHi[k], pl[k].rng0, key0, key1, draws);
        const float gr[4] = {bf16Lo(gq[k].x), bf16Hi(gq[k].x), bf16Lo(gq[k].y), bf16Hi(gq[k].y)};
        float mm[4] = {__uint_as_float(mq[k].x), __uint_as_float(mq[k].y), __uint_as_float(mq[k].z),
                       __uint_as_float(mq[k].w)};
        float vv[4] = {__uint_as_float(vq[k].x), __uint_as_float(vq[k].y), __uint_as_float(vq[k].z),
                       __uint_as_float(vq[k].w)};
        float old[4];
        if constexpr (kMaster) {
            old[0] = __uint_as_float(wq[k].x); old[1] = __uint_as_float(wq[k].y);
            old[2] = __uint_as_float(wq[k].z); old[3] = __uint_as_float(wq[k].w);
        } else {
            old[0] = bf16Lo(pq[k].x); old[1] = bf16Hi(pq[k].x); old[2] = bf16Lo(pq[k].y); old[3] = bf16Hi(pq[k].y);
        }
        float pn[4];
        uint32_t hb[4];
        stepQuad<kRound>(gr, mm, vv, old, w, s, scale, draws, pn, hb);
        __builtin_amdgcn_raw_buffer_store_b128(U32x4v{__float_as_uint(mm[0]), __float_as_uint(mm[1]),
                                                      __float_as_uint(mm[2]), __float_as_uint(mm[3])},
                                               rm, off * 4, 0, kPolicyNt);
        __builtin_amdgcn_raw_buffer_store_b128(U32x4v{__float_as_uint(vv[0]), __float_as_uint(vv[1]),
                                                      __float_as_uint(vv[2]), __float_as_uint(vv[3])},
                                               rv, off * 4, 0, kPolicyNt);
        if constexpr (kMaster)
            __builtin_amdgcn_raw_buffer_store_b128(U32x4v{__float_as_uint(pn[0]), __float_as_uint(pn[1]),
                                                          __float_as_uint(pn[2]), __float_as_uint(pn[3])},
                                                   rM, off * 4, 0, kPolicyNt);
        __builtin_amdgcn_raw_buffer_store_b64(U32x2v{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)}, rP, off * 2, 0,
                                              kParamsPolicy);
    }
}

template <bool kMaster, int kRound, bool kScheduled>
__global__ __launch_bounds__(kBlock) void adamwTileKernel(
    uint16_t *__restrict__ P, const uint16_t *__restrict__ G, float *__restrict__ M,
    float *__restrict__ Mom, float *__restrict__ Var, uint64_t S, ShardView sv, int pgVec, StepScalars s,
    const float *__restrict__ scalePtr, const int32_t *__restrict__ skipPtr, uint32_t key0, uint32_t key1,
    uint64_t tileBase, const bfo_step_scalars *__restrict__ steps, uint64_t nsteps,
    const uint64_t *__restrict__ cursor) {
    if (skipPtr && *skipPtr) return;  // step control decided to skip this update
    uint64_t cur = 0;
    if constexpr (kScheduled) cur = *cursor;
    const float scale = scalePtr ? *scalePtr : 1.0f;
    const uint64_t tile = tileBase + blockIdx.x;
    if (sv.flatBegin != UINT64_MAX && pgVec && !(sv.tile[tile] & kTileMixed))
        adamwTileFlat<kMaster, kRound, kScheduled>(P, G, M, Mom, Var, S, sv, s, scale, key0, key1, tile, steps,
                                                   nsteps, cur);
    else
        adamwTile<kMaster, kRound, kScheduled>(P, G, M, Mom, Var, S, sv, pgVec, s, scale, key0, key1, tile, steps,
                                               nsteps, cur);
}

// ---------------------------------------------------------------------------
// Measurement kernel: the update's memory traffic without its arithmetic.
// Same tile, lane and quad plan as the regular path of adamwTileKernel and
// the same cache policies (everything nontemporal except, without a master,
// the params).  kMode:
//   BFO_MIX_BOTH: the update's reads and writes (with a master: reads G, m,
//     v, M and writes m, v, M, P; without: reads G, P, m, v and writes P, m,
//     v), each output a bit-XOR of its inputs and the key, so nothing can be
//     elided; key 0 leaves m, v and M bitwise as they were;
//   BFO_MIX_READS: the update's reads alone; the loaded words are folded
//     into one 64-bit value per lane, which is compared with a constant: on
//     a match (odds 2^-64 per lane) the lane stores the m quad it loaded
//     back unchanged, so the loads stay and no state changes;
//   BFO_MIX_WRITES: the update's writes alone, of words made from the key
//     and the element index (m, v, M and P are overwritten).
// BOTH is the ceiling of the update's own mix; READS and WRITES time its two
// directions on their own, for the bound the mix would have if HBM served
// reads and writes one after the other.
// ---------------------------------------------------------------------------
template <bool kMaster, int kMode>
__global__ __launch_bounds__(kBlock) void streamMixKernel(uint16_t *__restrict__ P, const uint16_t *__restrict__ G,
                                                          float *__restrict__ M, float *__restrict__ Mom,
                                                          float *__restrict__ Var, uint64_t count, uint32_t key,
                                                          uint64_t tileBase) {
    constexpr bool kRead = kMode != BFO_MIX_WRITES;
    const uint64_t base = quadBase(tileBase + blockIdx.x);
    U32x2v gq[kQuadsPerLane], pq[kQuadsPerLane];
    U32x4v mq[kQuadsPerLane], vq[kQuadsPerLane], wq[kQuadsPerLane];
    int mode[kQuadsPerLane];
#pragma unroll
    for (int k = 0; k < kQuadsPerLane; ++k) {
        const uint64_t j0 = base + uint64_t(k) * 256;
        mode[k] = j0 + 4 <= count ? kRegular : (j0 < count ? kPerElement : kNone);
        if (mode[k] != kRegular || !kRead) continue;
        gq[k] = loadHint<true>(reinterpret_cast<const U32x2v *>(G + j0));
        mq[k] = loadHint<true>(reinterpret_cast<const U32x4v *>(Mom + j0));
        vq[k] = loadHint<true>(reinterpret_cast<const U32x4v *>(Var + j0));
        if constexpr (kMaster) wq[k] = loadHint<true>(reinterpret_cast<const U32x4v *>(M + j0));
        else pq[k] = loadHint<false>(reinterpret_cast<const U32x2v *>(P + j0));
    }
    if constexpr (kMode == BFO_MIX_READS) {
#pragma unroll
        for (int k = 0; k < kQuadsPerLane; ++k) {
            if (mode[k] != kRegular) continue;
            U32x4v x = mq[k] ^ vq[k];
            if constexpr (kMaster) x = x ^ wq[k];
            else x = x ^ U32x4v{pq[k].x, pq[k].y, 0u, 0u};
            const uint64_t folded = (uint64_t(x.x ^ x.z ^ gq[k].x) << 32) | uint64_t(x.y ^ x.w ^ gq[k].y);
            const uint64_t j0 = base + uint64_t(k) * 256;
            if (folded == (0x9E3779B97F4A7C15ull ^ key)) *reinterpret_cast<U32x4v *>(Mom + j0) = mq[k];
        }
        return;
    }
    const uint32_t key2 = (key & 0xFFFFu) | (key << 16);
#pragma unroll
    for (int k = 0; k < kQuadsPerLane; ++k) {
        const uint64_t j0 = base + uint64_t(k) * 256;
        if (mode[k] == kPerElement && kMode == BFO_MIX_BOTH) {
            for (uint64_t j = j0; j < count; ++j) {
                Mom[j] = __uint_as_float(__float_as_uint(Mom[j]) ^ key);
                Var[j] = __uint_as_float(__float_as_uint(Var[j]) ^ key);
                if constexpr (kMaster) {
                    M[j] = __uint_as_float(__float_as_uint(M[j]) ^ key);
                    P[j] = uint16_t(G[j] ^ key);
                } else {
                    P[j] = uint16_t(P[j] ^ G[j] ^ key);
                }
            }
            continue;
        }
        if (mode[k] == kPerElement) {
            for (uint64_t j = j0; j < count; ++j) {
                const uint32_t x = key ^ uint32_t(j);
                Mom[j] = __uint_as_float(x);
                Var[j] = __uint_as_float(x ^ 1u);
                if constexpr (kMaster) M[j] = __uint_as_float(x ^ 2u);
                P[j] = uint16_t(x);
            }
            continue;
        }
        if (mode[k] != kRegular) continue;
        if constexpr (kMode == BFO_MIX_WRITES) {
            const uint32_t x = key ^ uint32_t(j0);
            mq[k] = U32x4v{x, x + 1, x + 2, x + 3};
            vq[k] = mq[k] ^ 1u;
            wq[k] = mq[k] ^ 2u;
            gq[k] = U32x2v{x, x ^ 5u};
            pq[k] = U32x2v{0u, 0u};
        }
        storeHint<true>(reinterpret_cast<U32x4v *>(Mom + j0), mq[k] ^ key);
        storeHint<true>(reinterpret_cast<U32x4v *>(Var + j0), vq[k] ^ key);
        if constexpr (kMaster) {
            storeHint<true>(reinterpret_cast<U32x4v *>(M + j0), wq[k] ^ key);
            storeHint<true>(reinterpret_cast<U32x2v *>(P + j0), gq[k] ^ key2);
        } else {
            storeHint<false>(reinterpret_cast<U32x2v *>(P + j0), pq[k] ^ gq[k] ^ key2);
        }
    }
}

// ---------------------------------------------------------------------------
// Rebuild bf16 weights from the master: P = SR(M, draw) (or RNE(M)).  One
// workgroup per 4,096-element tile; lane t takes 8-element vectors t and
// t + 256 of it (16-byte params stores, 32 bytes of master per vector: one
// Philox block per vector; the update's quad plan, which needs a block per
// quad, measured slower here).  The master is only read and the params only
// written here: nontemporal loads (4-6% faster than plain ones on this
// 4 B read + 2 B write pattern) and nontemporal stores (a further 4-5%).
// ---------------------------------------------------------------------------
template <int kRound>
__global__ __launch_bounds__(kBlock) void masterToBf16Kernel(const float *__restrict__ M,
                                                             uint16_t *__restrict__ P, uint64_t S,
                                                             ShardView sv, int pgVec, uint32_t key0,
                                                             uint32_t key1, uint64_t tileBase, uint32_t shift) {
    const uint64_t tile = tileBase + blockIdx.x;
    const TileWords tw = tileWords(sv, tile, shift, S);
    F32x4 a[kVecPerLane], b[kVecPerLane];
    Place pl[kVecPerLane];
    int mode[kVecPerLane];
#pragma unroll
    for (int k = 0; k < kVecPerLane; ++k) {
        const uint64_t u = tile * kTileVecs + uint64_t(k) * kBlock + threadIdx.x;
        const uint64_t q = u - shift;
        mode[k] = kNone;
        if (u < shift || q * 8 >= S) continue;
        pl[k] = placeVector(sv, tw.of(q, tile), q * 8, S);
        if (!pl[k].inRun) {
            mode[k] = kPerElement;
            continue;
        }
        mode[k] = (pgVec && (pl[k].addr0 & 7) == 0) ? kRegular : kSemi;
        a[k] = __builtin_nontemporal_load(reinterpret_cast<const F32x4 *>(M) + 2 * q);
        b[k] = __builtin_nontemporal_load(reinterpret_cast<const F32x4 *>(M) + 2 * q + 1);
    }
#pragma unroll
    for (int k = 0; k < kVecPerLane; ++k) {
        if (mode[k] == kNone) continue;
        const uint64_t q = tile * kTileVecs + uint64_t(k) * kBlock + threadIdx.x - shift;
        if (mode[k] == kPerElement) {
            uint32_t run = pl[k].run;
            uint64_t cachedGroup = UINT64_MAX;
            U32x4 cached{0u, 0u, 0u, 0u};
            for (int e = 0; e < 8; ++e) {
                const uint64_t j = q * 8 + uint64_t(e);
                if (j >= S) break;
                uint64_t addr, rng;
                placeElement(sv, run, j, addr, rng);
                uint32_t draw = 0;
                if constexpr (kRound == BFO_ROUND_SR) {
                    if ((rng >> 3) != cachedGroup) {
                        cachedGroup = rng >> 3;
                        cached = philox10(cachedGroup, key0, key1);
                    }
                    draw = drawOf(cached, int(rng & 7));
                }
                P[addr] = uint16_t(writeBack<kRound>(M[j], draw));
            }
            continue;
        }
        uint32_t d[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        if constexpr (kRound == BFO_ROUND_SR) draws8(pl[k].rng0, key0, key1, d);
        const uint32_t h0 = writeBack<kRound>(a[k].x, d[0]), h1 = writeBack<kRound>(a[k].y, d[1]);
        const uint32_t h2 = writeBack<kRound>(a[k].z, d[2]), h3 = writeBack<kRound>(a[k].w, d[3]);
        const uint32_t h4 = writeBack<kRound>(b[k].x, d[4]), h5 = writeBack<kRound>(b[k].y, d[5]);
        const uint32_t h6 = writeBack<kRound>(b[k].z, d[6]), h7 = writeBack<kRound>(b[k].w, d[7]);
        if (mode[k] == kRegular) {
            storeOnce16(P, pl[k].addr0 >> 3,
                        make_uint4(h0 | (h1 << 16), h2 | (h3 << 16), h4 | (h5 << 16), h6 | (h7 << 16)));
        } else {
            uint16_t *p = P + pl[k].addr0;
            p[0] = uint16_t(h0); p[1] = uint16_t(h1); p[2] = uint16_t(h2); p[3] = uint16_t(h3);
            p[4] = uint16_t(h4); p[5] = uint16_t(h5); p[6] = uint16_t(h6); p[7] = uint16_t(h7);
        }
    }
}

// ---------------------------------------------------------------------------
// Grad norm.  Stage 1: workgroup b owns shard-local vectors
// [b*1024, (b+1)*1024); lane t takes vectors t, t+256, t+512, t+768 (four
// 16-byte loads in flight on the regular path), sums their squares in
// binary64 in element order, and the 256 lanes are reduced in a fixed tree
// (wave64 butterfly, then the 4 waves through LDS) into one partial per tile.
// Large shards (more than kNormFinishDirect tiles) add an intermediate pass:
// workgroup r sums partials [r*4096, (r+1)*4096) (lane t takes t, t+256, ...
// in order, then the fixed tree).  Stage 2: one 1024-lane workgroup adds the
// remaining partials (lane t takes t, t+1024, ... in order) in a fixed tree
// and derives norm and scale.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double sumSquares8(double acc, const uint4 &x) {
    const double d0 = double(bf16Lo(x.x)), d1 = double(bf16Hi(x.x));
    const double d2 = double(bf16Lo(x.y)), d3 = double(bf16Hi(x.y));
    const double d4 = double(bf16Lo(x.z)), d5 = double(bf16Hi(x.z));
    const double d6 = double(bf16Lo(x.w)), d7 = double(bf16Hi(x.w));
    acc = __builtin_fma(d0, d0, acc);
    acc = __builtin_fma(d1, d1, acc);
    acc = __builtin_fma(d2, d2, acc);
    acc = __builtin_fma(d3, d3, acc);
    acc = __builtin_fma(d4, d4, acc);
    acc = __builtin_fma(d5, d5, acc);
    acc = __builtin_fma(d6, d6, acc);
    acc = __builtin_fma(d7, d7, acc);
    return acc;
}

// Fixed-order sum over the workgroup; the result is valid in thread 0.
template <int kThreads>
__device__ __forceinline__ double blockSum(double x) {
    __shared__ double waveSums[kThreads / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) waveSums[wave] = x;
    __syncthreads();
    double total = 0.0;
    if (threadIdx.x == 0) {
        total = waveSums[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) total += waveSums[w];
    }
    return total;
}

// The per-lane part of stage 1 for one tile: `lane` (0..255) takes vectors
// lane, lane + 256, lane + 512, lane + 768 of the tile and adds the squares in
// that order.  Every stage-1 path below runs these functions and reduces the
// 256 lanes with tileSum, so they all give the same bits for the same tile.
//
// normTileDirect: the tile's grads sit at consecutive positions starting
// 16-byte aligned (shard element j at base[j]), so a lane's address needs no
// plan lookup (two dependent loads that would stand before every grad load
// and cost a quarter of the bandwidth).
__device__ __forceinline__ double normTileDirect(const uint16_t *__restrict__ base, uint64_t S, uint64_t tile,
                                                 uint32_t lane) {
    const uint64_t full = S / 8;  // vectors with all eight elements in the shard
    uint4 x[kNormVecPerLane];
#pragma unroll
    for (int k = 0; k < kNormVecPerLane; ++k) {
        const uint64_t q = tile * kNormTileVecs + uint64_t(k) * kBlock + lane;
        if (q < full) x[k] = loadOnce16(base, q);
    }
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kNormVecPerLane; ++k) {
        const uint64_t q = tile * kNormTileVecs + uint64_t(k) * kBlock + lane;
        if (q < full) {
            acc = sumSquares8(acc, x[k]);
        } else if (q * 8 < S) {
            for (uint64_t j = q * 8; j < S; ++j) {
                const double d = double(bf16At(base, j));
                acc = __builtin_fma(d, d, acc);
            }
        }
    }
    return acc;
}

// normTilePlanned: the general case -- each vector is placed through the
// shard plan (per-tensor tables, grads that are not 16-byte aligned), except
// that a per-tensor tile inside one run with 16-byte-aligned grads sits at a
// per-tile offset and goes direct.
__device__ __forceinline__ double normTilePlanned(const uint16_t *__restrict__ G, uint64_t S, const ShardView &sv,
                                                  int pgVec, uint64_t tile, uint32_t lane) {
    const uint64_t offset = (sv.normOffset && pgVec) ? sv.normOffset[tile] : kNoNormOffset;
    if (offset != kNoNormOffset) return normTileDirect(G + offset, S, tile, lane);
    uint4 x[kNormVecPerLane];
    Place pl[kNormVecPerLane];
    int mode[kNormVecPerLane];
#pragma unroll
    for (int k = 0; k < kNormVecPerLane; ++k) {
        const uint64_t q = tile * kNormTileVecs + uint64_t(k) * kBlock + lane;
        mode[k] = kNone;
        if (q * 8 >= S) continue;
        pl[k] = placeVector(sv, sv.tile[q / kTileVecs], q * 8, S);
        if (!pl[k].inRun) {
            mode[k] = kPerElement;
        } else if (pgVec && (pl[k].addr0 & 7) == 0) {
            mode[k] = kRegular;
            x[k] = loadOnce16(G, pl[k].addr0 >> 3);
        } else {
            mode[k] = kSemi;
            x[k] = load8Narrow(G + pl[k].addr0);
        }
    }
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kNormVecPerLane; ++k) {
        if (mode[k] == kRegular || mode[k] == kSemi) {
            acc = sumSquares8(acc, x[k]);
        } else if (mode[k] == kPerElement) {
            const uint64_t q = tile * kNormTileVecs + uint64_t(k) * kBlock + lane;
            uint32_t run = pl[k].run;
            for (int e = 0; e < 8; ++e) {
                const uint64_t j = q * 8 + uint64_t(e);
                if (j >= S) break;
                uint64_t addr, rng;
                placeElement(sv, run, j, addr, rng);
                const double d = double(bf16At(G, addr));
                acc = __builtin_fma(d, d, acc);
            }
        }
    }
    return acc;
}

// The tile's partial from its 256 lanes (four waves): butterfly within each
// wave, then the four wave sums added in wave order by the group's first
// lane.  `waveSums` holds one slot per wave of the workgroup; `group` is the
// 256-lane group of the workgroup that worked on the tile.  Every lane of the
// workgroup must call it (it synchronises the workgroup).
__device__ __forceinline__ double tileSum(double x, double *waveSums, uint32_t group) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    if ((threadIdx.x & 63) == 0) waveSums[threadIdx.x >> 6] = x;
    __syncthreads();
    double total = waveSums[group * 4];
#pragma unroll
    for (int w = 1; w < 4; ++w) total += waveSums[group * 4 + w];
    return total;
}

// Flat shards with 16-byte-aligned grads: shard element j is grads[j].
__global__ __launch_bounds__(kBlock) void normStage1FlatKernel(const uint16_t *__restrict__ G, uint64_t S,
                                                               double *__restrict__ partials, uint64_t tileBase,
                                                               uint64_t lastTile) {
    __shared__ double waveSums[kBlock / 64];
    const uint64_t tile = lastTile - (tileBase + blockIdx.x);
    const double total = tileSum(normTileDirect(G, S, tile, threadIdx.x), waveSums, 0);
    if (threadIdx.x == 0) partials[tile] = total;
}

// Workgroups take tiles from the shard's end backwards: the partial of a tile
// depends only on its index, so the order changes no bit of the result.  The
// order was chosen for plain loads, whose last lines (the shard's start) the
// update, walking forward, could still find in the memory-side cache; with
// nontemporal loads forward and backward measured the same.
__global__ __launch_bounds__(kBlock) void normStage1Kernel(const uint16_t *__restrict__ G, uint64_t S,
                                                           ShardView sv, int pgVec,
                                                           double *__restrict__ partials, uint64_t tileBase,
                                                           uint64_t lastTile) {
    __shared__ double waveSums[kBlock / 64];
    const uint64_t tile = lastTile - (tileBase + blockIdx.x);
    const double total = tileSum(normTilePlanned(G, S, sv, pgVec, tile, threadIdx.x), waveSums, 0);
    if (threadIdx.x == 0) partials[tile] = total;
}

// Shards of at most kNormSmallTiles tiles: both stages in one 1024-lane
// workgroup, so a small step pays one launch for its norm instead of two.
// Each 256-lane group computes a tile's partial exactly as stage 1 does (same
// lane map, same tileSum), the partials wait in LDS, and the final sum runs
// the stage-2 code on them (lane t adds partial t to 0, then the block sum):
// the bits equal those of the two-kernel path.
__global__ __launch_bounds__(kNormFinishBlock) void normSmallKernel(const uint16_t *__restrict__ G, uint64_t S,
                                                                    ShardView sv, int pgVec, int flat,
                                                                    uint32_t ntiles, float maxNorm,
                                                                    bfo_norm_result *__restrict__ out) {
    __shared__ double waveSums[kNormFinishBlock / 64];
    __shared__ double partial[kNormSmallTiles];
    constexpr uint32_t kGroups = kNormFinishBlock / kBlock;
    const uint32_t group = threadIdx.x / kBlock, lane = threadIdx.x % kBlock;
    for (uint32_t base = 0; base < ntiles; base += kGroups) {
        const uint32_t tile = base + group;
        double acc = 0.0;
        if (tile < ntiles)
            acc = (flat && pgVec) ? normTileDirect(G, S, tile, lane) : normTilePlanned(G, S, sv, pgVec, tile, lane);
        const double total = tileSum(acc, waveSums, group);
        if (lane == 0 && tile < ntiles) partial[tile] = total;
        __syncthreads();  // partial written; waveSums free for the next round
    }
    double acc = 0.0;
    if (threadIdx.x < ntiles) acc += partial[threadIdx.x];
    const double sumsq = blockSum<kNormFinishBlock>(acc);
    if (threadIdx.x == 0) {
        const float norm = float(sqrt(sumsq));
        const float scale = norm > maxNorm ? maxNorm / norm : 1.0f;
        out->sumsq = sumsq;
        out->norm = norm;
        out->scale = scale;
    }
}

// A whole small step in one launch (shards of at most kNormSmallTiles norm
// tiles, i.e. at most 16 update tiles).  Every workgroup forms the shard's
// sum of squares itself -- tile by tile with stage 1's lane map and tileSum,
// then partial t in lane t of a wave (+0 elsewhere) through the same
// butterfly as normSmallKernel's final sum, whose other waves only add +0
// -- so its sum, norm and scale are those of the two-launch path bit for
// bit (the grads, at most 128 KiB, come from the cache after the first
// workgroup).  Workgroup 0 writes `out`; each workgroup then updates its own
// tile with that scale, unless the skip flag is set.
template <bool kMaster, int kRound>
__global__ __launch_bounds__(kBlock) void adamwSmallStepKernel(
    uint16_t *__restrict__ P, const uint16_t *__restrict__ G, float *__restrict__ M, float *__restrict__ Mom,
    float *__restrict__ Var, uint64_t S, ShardView sv, int gVec, int pgVec, int flat, uint32_t ntiles,
    float maxNorm, bfo_norm_result *__restrict__ out, StepScalars s, const int32_t *__restrict__ skipPtr,
    uint32_t key0, uint32_t key1) {
    __shared__ double waveSums[kBlock / 64];
    __shared__ double partial[kNormSmallTiles];
    for (uint32_t tile = 0; tile < ntiles; ++tile) {
        const double acc = (flat && gVec) ? normTileDirect(G, S, tile, threadIdx.x)
                                          : normTilePlanned(G, S, sv, gVec, tile, threadIdx.x);
        const double total = tileSum(acc, waveSums, 0);
        if (threadIdx.x == 0) partial[tile] = total;
        __syncthreads();  // partial written; waveSums free for the next tile
    }
    const uint32_t lane = threadIdx.x & 63;
    double x = 0.0;
    if (lane < ntiles) x += partial[lane];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    // every lane now holds the same sum: each butterfly stage adds the same
    // two values on both lanes of a pair, and addition is commutative
    const float norm = float(sqrt(x));
    const float scale = norm > maxNorm ? maxNorm / norm : 1.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        out->sumsq = x;
        out->norm = norm;
        out->scale = scale;
    }
    if (skipPtr && *skipPtr) return;
    adamwTile<kMaster, kRound, false>(P, G, M, Mom, Var, S, sv, pgVec, s, scale, key0, key1, blockIdx.x, nullptr,
                                      0, 0);
}

__global__ __launch_bounds__(kBlock) void normReduceKernel(const double *__restrict__ in, uint64_t count,
                                                           double *__restrict__ out) {
    const uint64_t lo = uint64_t(blockIdx.x) * kNormReduceRun;
    const uint64_t hi = lo + kNormReduceRun < count ? lo + kNormReduceRun : count;
    constexpr int kPer = int(kNormReduceRun / kBlock);
    double p[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const uint64_t k = lo + uint64_t(j) * kBlock + threadIdx.x;
        p[j] = k < hi ? in[k] : 0.0;
    }
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) acc += p[j];
    const double total = blockSum<kBlock>(acc);
    if (threadIdx.x == 0) out[blockIdx.x] = total;
}

__global__ __launch_bounds__(kNormFinishBlock) void normStage2Kernel(const double *__restrict__ partials,
                                                                     uint64_t count, float maxNorm,
                                                                     bfo_norm_result *__restrict__ out) {
    // Lane t adds partials t, t+1024, t+2048, ... in that order.  Up to
    // kNormFinishDirect partials (all that launchNorm ever passes) are loaded
    // at once, 32 per lane, so the whole read is one round trip; absent ones
    // load as +0, which leaves the non-negative running sum unchanged.
    constexpr int kPer = int(kNormFinishDirect / kNormFinishBlock);
    double p[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const uint64_t k = threadIdx.x + uint64_t(j) * kNormFinishBlock;
        p[j] = k < count ? partials[k] : 0.0;
    }
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) acc += p[j];
    for (uint64_t k = threadIdx.x + kNormFinishDirect; k < count; k += kNormFinishBlock) acc += partials[k];
    const double sumsq = blockSum<kNormFinishBlock>(acc);
    if (threadIdx.x == 0) {
        const float norm = float(sqrt(sumsq));
        const float scale = norm > maxNorm ? maxNorm / norm : 1.0f;
        out->sumsq = sumsq;
        out->norm = norm;
        out->scale = scale;
    }
}

// ---------------------------------------------------------------------------
// Test exports.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void rngDumpKernel(uint64_t first, uint64_t count, uint64_t seed,
                                                        uint16_t *out, uint64_t blockBase) {
    const uint64_t k = (blockBase + blockIdx.x) * kBlock + threadIdx.x;
    if (k >= count) return;
    const uint64_t i = first + k;
    const U32x4 d = philox10(i >> 3, uint32_t(seed), uint32_t(seed >> 32));
    out[k] = uint16_t(drawOf(d, int(i & 7)));
}

__global__ __launch_bounds__(kBlock) void decayDumpKernel(ShardView sv, uint64_t S, uint8_t *out,
                                                          uint64_t blockBase) {
    const uint64_t q = (blockBase + blockIdx.x) * kBlock + threadIdx.x;
    const uint64_t j0 = q * 8;
    if (j0 >= S) return;
    uint32_t run = sv.tile[q / kTileVecs] & ~kTileMixed;
    for (int e = 0; e < 8 && j0 + e < S; ++e) {
        uint64_t addr, rng;
        placeElement(sv, run, j0 + e, addr, rng);
        out[j0 + e] = sv.flag[run];
    }
}

// Partials of grad_global_norm_noalloc: a fixed array that every GPU the
// library runs on holds until the process ends.  Host code must not pass its
// name to a kernel (in host code it is a stand-in, not a device address):
// staticScratchAddress gives the address on the current device.
static __device__ __align__(256) double scratch[kStaticScratchBytes / sizeof(double)];

// A launch's lane count must stay below 2^32: split long 1-D grids.
constexpr uint64_t kMaxBlocksPerLaunch = uint64_t(1) << 22;

// ---------------------------------------------------------------------------
// Outlier z-score ("04 · 多 GPU 与混合精度" §4): compares the new value with
// the window of previous finite values (binary64 mean and population
// variance, each summed oldest to newest), writes z (NaN until the window is
// full) and the skip flag, then appends the value if finite.  The wave copies
// the ring into LDS in age order; one lane then runs the two serial sums in
// that order, reading eight values per step.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double sumOldestFirst(const float *win, uint32_t W, double mean, bool centered) {
    double acc = 0.0;
    uint32_t k = 0;
    for (; k + 8 <= W; k += 8) {
        const float4 a = *reinterpret_cast<const float4 *>(win + k);
        const float4 b = *reinterpret_cast<const float4 *>(win + k + 4);
        const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (centered) {
                const double d = double(x[e]) - mean;
                acc += d * d;
            } else {
                acc += double(x[e]);
            }
        }
    }
    for (; k < W; ++k) {
        if (centered) {
            const double d = double(win[k]) - mean;
            acc += d * d;
        } else {
            acc += double(win[k]);
        }
    }
    return acc;
}

__global__ __launch_bounds__(64) void outlierUpdateKernel(OutlierState *st, const float *value, float threshold,
                                                          float *zOut, int32_t *skipOut) {
    __shared__ __align__(16) float win[kOutlierMaxWindow];
    const uint32_t W = st->window, count = st->count, head = st->head;
    const bool full = count == W;
    if (full) {
        for (uint32_t k = threadIdx.x; k < W; k += 64) {
            uint32_t idx = head + k;
            if (idx >= W) idx -= W;
            win[k] = st->values[idx];
        }
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    const float x = *value;
    double z = __builtin_nan("");
    if (full) {
        const double mean = sumOldestFirst(win, W, 0.0, false) / double(W);
        const double sq = sumOldestFirst(win, W, mean, true);
        z = (double(x) - mean) / sqrt(sq / double(W));
    }
    const bool finite = (__float_as_uint(x) & 0x7F800000u) != 0x7F800000u;
    *zOut = float(z);
    *skipOut = (!finite || (threshold > 0.0f && z > double(threshold))) ? 1 : 0;
    if (finite) {
        st->values[head] = x;
        st->head = head + 1 == W ? 0u : head + 1;
        if (count < W) st->count = count + 1;
    }
}

__global__ __launch_bounds__(64) void outlierResetKernel(OutlierState *st, uint32_t window) {
    if (threadIdx.x != 0) return;
    st->window = window;
    st->count = 0;
    st->head = 0;
    st->pad = 0;
}

// The rebuild's partition shift (in 8-element vectors) that puts every
// wave's params stores on a 128-byte line: flat shards with 16-byte-aligned
// params that start an even number of 16-byte units into a line (an odd
// number would leave the master 32 bytes off a 64-byte boundary: no shift).
uint32_t lineShift(const uint16_t *P, const ShardView &sv, int pgVec) {
    if (sv.flatBegin == UINT64_MAX || !pgVec) return 0;
    const uint32_t units = uint32_t(reinterpret_cast<uintptr_t>(P) >> 4) & 7u;
    return (units & 1u) ? 0u : units;
}

template <bool kMaster, int kRound, bool kScheduled>
hipError_t launchAdamwT(uint16_t *P, const uint16_t *G, float *M, float *m, float *v, uint64_t S,
                        ShardView sv, int pgVec, StepScalars s, const float *scale, const int32_t *skip,
                        uint64_t seed, const StepSchedule &sched, hipStream_t stream) {
    const uint32_t k0 = uint32_t(seed), k1 = uint32_t(seed >> 32);
    const uint64_t tiles = (S + kTileElems - 1) / kTileElems;
    for (uint64_t base = 0; base < tiles; base += kMaxBlocksPerLaunch) {
        const uint64_t nb = tiles - base < kMaxBlocksPerLaunch ? tiles - base : kMaxBlocksPerLaunch;
        hipLaunchKernelGGL((adamwTileKernel<kMaster, kRound, kScheduled>), dim3(uint32_t(nb)), dim3(kBlock), 0,
                           stream, P, G, M, m, v, S, sv, pgVec, s, scale, skip, k0, k1, base, sched.steps,
                           sched.count, sched.cursor);
    }
    return hipGetLastError();
}

template <bool kScheduled>
hipError_t launchAdamwS(uint16_t *P, const uint16_t *G, float *M, float *m, float *v, uint64_t S,
                        ShardView sv, int pgVec, StepScalars s, const float *scale, const int32_t *skip,
                        uint64_t seed, int rounding, const StepSchedule &sched, hipStream_t stream) {
    if (M) {
        return rounding == BFO_ROUND_SR
                   ? launchAdamwT<true, BFO_ROUND_SR, kScheduled>(P, G, M, m, v, S, sv, pgVec, s, scale, skip, seed,
                                                                  sched, stream)
                   : launchAdamwT<true, BFO_ROUND_RNE, kScheduled>(P, G, M, m, v, S, sv, pgVec, s, scale, skip,
                                                                   seed, sched, stream);
    }
    return rounding == BFO_ROUND_SR
               ? launchAdamwT<false, BFO_ROUND_SR, kScheduled>(P, G, M, m, v, S, sv, pgVec, s, scale, skip, seed,
                                                               sched, stream)
               : launchAdamwT<false, BFO_ROUND_RNE, kScheduled>(P, G, M, m, v, S, sv, pgVec, s, scale, skip, seed,
                                                                sched, stream);
}

__global__ __launch_bounds__(64) void cursorAdvanceKernel(uint64_t *cursor) {
    if (threadIdx.x == 0) *cursor += 1;
}

}  // namespace

hipError_t staticScratchAddress(void **out) { return hipGetSymbolAddress(out, HIP_SYMBOL(scratch)); }

hipError_t launchNorm(const uint16_t *g, uint64_t S, ShardView sv, int pgVec, bool flat, float maxNorm,
                      double *partials, bfo_norm_result *out, hipStream_t stream) {
    const uint64_t ntiles = normTiles(S);
    if (ntiles > 0 && ntiles <= kNormSmallTiles) {
        hipLaunchKernelGGL(normSmallKernel, dim3(1), dim3(kNormFinishBlock), 0, stream, g, S, sv, pgVec,
                           flat ? 1 : 0, uint32_t(ntiles), maxNorm, out);
        return hipGetLastError();
    }
    for (uint64_t base = 0; base < ntiles; base += kMaxBlocksPerLaunch) {
        const uint64_t nb = ntiles - base < kMaxBlocksPerLaunch ? ntiles - base : kMaxBlocksPerLaunch;
        if (flat && pgVec)
            hipLaunchKernelGGL(normStage1FlatKernel, dim3(uint32_t(nb)), dim3(kBlock), 0, stream, g, S, partials,
                               base, ntiles - 1);
        else
            hipLaunchKernelGGL(normStage1Kernel, dim3(uint32_t(nb)), dim3(kBlock), 0, stream, g, S, sv, pgVec,
                               partials, base, ntiles - 1);
    }
    const double *finishIn = partials;
    uint64_t finishCount = ntiles;
    const uint64_t runs = normRuns(ntiles);
    if (runs) {
        double *second = partials + ntiles;
        hipLaunchKernelGGL(normReduceKernel, dim3(uint32_t(runs)), dim3(kBlock), 0, stream, partials, ntiles,
                           second);
        finishIn = second;
        finishCount = runs;
    }
    hipLaunchKernelGGL(normStage2Kernel, dim3(1), dim3(kNormFinishBlock), 0, stream, finishIn, finishCount,
                       maxNorm, out);
    return hipGetLastError();
}

hipError_t launchAdamw(uint16_t *P, const uint16_t *G, float *M, float *m, float *v, uint64_t S,
                       ShardView sv, int pgVec, StepScalars s, const float *scale, const int32_t *skip,
                       uint64_t seed, int rounding, const StepSchedule *sched, hipStream_t stream) {
    if (sched) return launchAdamwS<true>(P, G, M, m, v, S, sv, pgVec, s, scale, skip, 0, rounding, *sched, stream);
    return launchAdamwS<false>(P, G, M, m, v, S, sv, pgVec, s, scale, skip, seed, rounding, StepSchedule{},
                               stream);
}

hipError_t launchSmallStep(uint16_t *P, const uint16_t *G, float *M, float *m, float *v, uint64_t S, ShardView sv,
                           int gVec, int pgVec, bool flat, float maxNorm, bfo_norm_result *out, StepScalars s,
                           const int32_t *skip, uint64_t seed, int rounding, hipStream_t stream) {
    const uint32_t k0 = uint32_t(seed), k1 = uint32_t(seed >> 32);
    const uint32_t ntiles = uint32_t(normTiles(S));
    const dim3 grid(uint32_t((S + kTileElems - 1) / kTileElems)), block(kBlock);
    const int fl = flat ? 1 : 0;
    if (M && rounding == BFO_ROUND_SR)
        hipLaunchKernelGGL((adamwSmallStepKernel<true, BFO_ROUND_SR>), grid, block, 0, stream, P, G, M, m, v, S, sv,
                           gVec, pgVec, fl, ntiles, maxNorm, out, s, skip, k0, k1);
    else if (M)
        hipLaunchKernelGGL((adamwSmallStepKernel<true, BFO_ROUND_RNE>), grid, block, 0, stream, P, G, M, m, v, S, sv,
                           gVec, pgVec, fl, ntiles, maxNorm, out, s, skip, k0, k1);
    else if (rounding == BFO_ROUND_SR)
        hipLaunchKernelGGL((adamwSmallStepKernel<false, BFO_ROUND_SR>), grid, block, 0, stream, P, G, M, m, v, S, sv,
                           gVec, pgVec, fl, ntiles, maxNorm, out, s, skip, k0, k1);
    else
        hipLaunchKernelGGL((adamwSmallStepKernel<false, BFO_ROUND_RNE>), grid, block, 0, stream, P, G, M, m, v, S,
                           sv, gVec, pgVec, fl, ntiles, maxNorm, out, s, skip, k0, k1);
    return hipGetLastError();
}

hipError_t launchCursorAdvance(uint64_t *cursor, hipStream_t stream) {
    hipLaunchKernelGGL(cursorAdvanceKernel, dim3(1), dim3(64), 0, stream, cursor);
    return hipGetLastError();
}

hipError_t launchOutlierUpdate(OutlierState *state, const float *value, float threshold, float *z,
                               int32_t *skip, hipStream_t stream) {
    hipLaunchKernelGGL(outlierUpdateKernel, dim3(1), dim3(64), 0, stream, state, value, threshold, z, skip);
    return hipGetLastError();
}

hipError_t launchOutlierReset(OutlierState *state, uint32_t window, hipStream_t stream) {
    hipLaunchKernelGGL(outlierResetKernel, dim3(1), dim3(64), 0, stream, state, window);
    return hipGetLastError();
}

hipError_t launchMasterToBf16(const float *M, uint16_t *P, uint64_t S, ShardView sv, int pgVec,
                              uint64_t seed, int rounding, hipStream_t stream) {
    const uint32_t k0 = uint32_t(seed), k1 = uint32_t(seed >> 32);
    const uint32_t shift = lineShift(P, sv, pgVec);
    const uint64_t tiles = ((S + 7) / 8 + shift + kTileVecs - 1) / kTileVecs;
    for (uint64_t base = 0; base < tiles; base += kMaxBlocksPerLaunch) {
        const uint64_t nb = tiles - base < kMaxBlocksPerLaunch ? tiles - base : kMaxBlocksPerLaunch;
        if (rounding == BFO_ROUND_SR)
            hipLaunchKernelGGL(masterToBf16Kernel<BFO_ROUND_SR>, dim3(uint32_t(nb)), dim3(kBlock), 0, stream, M, P,
                               S, sv, pgVec, k0, k1, base, shift);
        else
            hipLaunchKernelGGL(masterToBf16Kernel<BFO_ROUND_RNE>, dim3(uint32_t(nb)), dim3(kBlock), 0, stream, M,
                               P, S, sv, pgVec, k0, k1, base, shift);
    }
    return hipGetLastError();
}

template <bool kMaster, int kMode>
void launchStreamMixT(uint16_t *P, const uint16_t *G, float *M, float *m, float *v, uint64_t count, uint32_t key,
                      hipStream_t stream) {
    const uint64_t tiles = (count + kTileElems - 1) / kTileElems;
    for (uint64_t base = 0; base < tiles; base += kMaxBlocksPerLaunch) {
        const uint64_t nb = tiles - base < kMaxBlocksPerLaunch ? tiles - base : kMaxBlocksPerLaunch;
        hipLaunchKernelGGL((streamMixKernel<kMaster, kMode>), dim3(uint32_t(nb)), dim3(kBlock), 0, stream, P, G, M, m,
                           v, count, key, base);
    }
}

hipError_t launchStreamMix(uint16_t *P, const uint16_t *G, float *M, float *m, float *v, uint64_t count,
                           uint32_t key, int mode, hipStream_t stream) {
    if (M) {
        if (mode == BFO_MIX_READS) launchStreamMixT<true, BFO_MIX_READS>(P, G, M, m, v, count, key, stream);
        else if (mode == BFO_MIX_WRITES) launchStreamMixT<true, BFO_MIX_WRITES>(P, G, M, m, v, count, key, stream);
        else launchStreamMixT<true, BFO_MIX_BOTH>(P, G, M, m, v, count, key, stream);
    } else {
        if (mode == BFO_MIX_READS) launchStreamMixT<false, BFO_MIX_READS>(P, G, M, m, v, count, key, stream);
        else if (mode == BFO_MIX_WRITES) launchStreamMixT<false, BFO_MIX_WRITES>(P, G, M, m, v, count, key, stream);
        else launchStreamMixT<false, BFO_MIX_BOTH>(P, G, M, m, v, count, key, stream);
    }
    return hipGetLastError();
}

hipError_t launchRngDump(uint64_t first, uint64_t count, uint64_t seed, uint16_t *out,
                         hipStream_t stream) {
    if (count) {
        const uint64_t blocks = (count + kBlock - 1) / kBlock;
        for (uint64_t base = 0; base < blocks; base += kMaxBlocksPerLaunch) {
            const uint64_t nb = blocks - base < kMaxBlocksPerLaunch ? blocks - base : kMaxBlocksPerLaunch;
            hipLaunchKernelGGL(rngDumpKernel, dim3(uint32_t(nb)), dim3(kBlock), 0, stream, first, count, seed,
                               out, base);
        }
    }
    return hipGetLastError();
}

hipError_t launchDecayDump(ShardView sv, uint64_t S, uint8_t *out, hipStream_t stream) {
    const uint64_t nv = (S + 7) / 8;
    if (nv) {
        const uint64_t blocks = (nv + kBlock - 1) / kBlock;
        for (uint64_t base = 0; base < blocks; base += kMaxBlocksPerLaunch) {
            const uint64_t nb = blocks - base < kMaxBlocksPerLaunch ? blocks - base : kMaxBlocksPerLaunch;
            hipLaunchKernelGGL(decayDumpKernel, dim3(uint32_t(nb)), dim3(kBlock), 0, stream, sv, S, out, base);
        }
    }
    return hipGetLastError();
}

}  // namespace bfo
