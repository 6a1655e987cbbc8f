// bfo_checkpoint.cpp -- per-rank optimizer-state files and resume.
//
// "04 · 多 GPU 与混合精度" §5.1-5.2: each rank writes its own state (m, v,
// fp32 master, the rounding state of the last update); a DONE marker makes a
// checkpoint count; resume takes the newest step with a marker, reads the
// state back and rebuilds the bf16 weights from the master with the last
// update's draws, so they come back bit-identical.  Without a master (the
// no-master update path) the bf16 weights are the state and are stored.
//
// File state_<step:08>_<rank:05>.bin, little-endian:
//   header (kHeaderBytes): magic "BFOSTATE", version, header bytes, step,
//     seed, n, S, world, rank, layout, has_master, table fingerprint
//     (FNV-1a over every tensor's offset, numel and flags);
//   payload: master S x fp32 (or, without a master, the shard's bf16 params
//     in shard-local order), then m S x fp32, then v S x fp32.
// Written to a temporary name and renamed into place, so a file under the
// final name is complete.
#include <hip/hip_runtime_api.h>

#include <dirent.h>
#include <unistd.h>

#include <cerrno>
#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "bfo_internal.hpp"

namespace {

constexpr char kMagic[8] = {'B', 'F', 'O', 'S', 'T', 'A', 'T', 'E'};
constexpr uint32_t kVersion = 1;
constexpr uint32_t kHeaderBytes = 96;
constexpr size_t kStageBytes = size_t(64) << 20;

struct Header {
    char magic[8];
    uint32_t version;
    uint32_t headerBytes;
    uint64_t step;
    uint64_t seed;
    uint64_t n;
    uint64_t S;
    uint32_t world;
    uint32_t rank;
    uint32_t layout;
    uint32_t hasMaster;
    uint64_t fingerprint;
    uint8_t reserved[24];
};
static_assert(sizeof(Header) == kHeaderBytes, "checkpoint header layout");

std::string statePath(const char *dir, uint64_t step, uint32_t rank) {
    char name[64];
    std::snprintf(name, sizeof name, "/state_%08" PRIu64 "_%05u.bin", step, rank);
    return std::string(dir) + name;
}

std::string donePath(const char *dir, uint64_t step) {
    char name[48];
    std::snprintf(name, sizeof name, "/DONE_%08" PRIu64, step);
    return std::string(dir) + name;
}

// Moves bytes between a device array and a file through two pinned halves of
// a staging buffer, so that the copy of one chunk overlaps the file I/O of
// the other.  Every copy is queued on the caller's stream and waited for
// through an event before its half is reused.
struct Stage {
    static constexpr size_t kHalf = kStageBytes / 2;
    char *buf = nullptr;
    hipEvent_t done[2] = {nullptr, nullptr};
    hipStream_t stream = nullptr;
    hipError_t err = hipSuccess;
    ~Stage() {
        // No copy may still target the buffer when it is freed (error paths
        // can leave one queued).
        if (buf) (void)hipStreamSynchronize(stream);
        for (hipEvent_t &e : done)
            if (e) (void)hipEventDestroy(e);
        if (buf) (void)hipHostFree(buf);
    }
    bool open(hipStream_t s) {
        stream = s;
        if ((err = hipHostMalloc(reinterpret_cast<void **>(&buf), kStageBytes, hipHostMallocDefault)) != hipSuccess)
            return false;
        for (hipEvent_t &e : done)
            if ((err = hipEventCreateWithFlags(&e, hipEventDisableTiming)) != hipSuccess) return false;
        return true;
    }
    char *half(int h) { return buf + size_t(h) * kHalf; }
    // Device -> file: chunk k+1 is copied while chunk k is written.
    int write(FILE *f, const void *dev, uint64_t bytes) {
        const char *src = static_cast<const char *>(dev);
        const uint64_t chunks = (bytes + kHalf - 1) / kHalf;
        auto len = [&](uint64_t k) { return size_t(bytes - k * kHalf < kHalf ? bytes - k * kHalf : kHalf); };
        auto fetch = [&](uint64_t k) {
            const int h = int(k & 1);
            if ((err = hipMemcpyAsync(half(h), src + k * kHalf, len(k), hipMemcpyDeviceToHost, stream)) != hipSuccess)
                return false;
            return (err = hipEventRecord(done[h], stream)) == hipSuccess;
        };
        if (chunks && !fetch(0)) return BFO_EHIP;
        for (uint64_t k = 0; k < chunks; ++k) {
            const int h = int(k & 1);
            if ((err = hipEventSynchronize(done[h])) != hipSuccess) return BFO_EHIP;
            if (k + 1 < chunks && !fetch(k + 1)) return BFO_EHIP;
            if (std::fwrite(half(h), 1, len(k), f) != len(k)) return BFO_EIO;
        }
        return BFO_OK;
    }
    // File -> device: chunk k+1 is read while chunk k is copied.
    int read(FILE *f, void *dev, uint64_t bytes) {
        char *dst = static_cast<char *>(dev);
        const uint64_t chunks = (bytes + kHalf - 1) / kHalf;
        int rc = BFO_OK;
        bool pending[2] = {false, false};
        for (uint64_t k = 0; k < chunks && rc == BFO_OK; ++k) {
            const int h = int(k & 1);
            const size_t n = size_t(bytes - k * kHalf < kHalf ? bytes - k * kHalf : kHalf);
            if (pending[h] && (err = hipEventSynchronize(done[h])) != hipSuccess) {
                rc = BFO_EHIP;
                break;
            }
            pending[h] = false;
            if (std::fread(half(h), 1, n, f) != n) {
                rc = BFO_EFORMAT;
                break;
            }
            if ((err = hipMemcpyAsync(dst + k * kHalf, half(h), n, hipMemcpyHostToDevice, stream)) != hipSuccess ||
                (err = hipEventRecord(done[h], stream)) != hipSuccess) {
                rc = BFO_EHIP;
                break;
            }
            pending[h] = true;
        }
        // Both halves must be idle before the buffer can be freed or reused.
        const hipError_t e = hipStreamSynchronize(stream);
        if (rc == BFO_OK && e != hipSuccess) {
            err = e;
            rc = BFO_EHIP;
        }
        return rc;
    }
};

int fail(Stage &st, int rc) { return rc == BFO_EHIP ? bfo::recordHipFailure(st.err) : rc; }

}  // namespace

extern "C" {

int bfo_checkpoint_save(const char *dir, bfo_table table, const uint16_t *params, const float *master,
                        const float *m, const float *v, uint64_t step, uint64_t seed, void *stream) {
    if (!dir || !table || (!master && !params)) return BFO_EINVAL;
    const bfo::TableFacts tf = bfo::tableFacts(table);
    if (tf.S && (!m || !v)) return BFO_EINVAL;
    Header h;
    std::memset(&h, 0, sizeof h);
    std::memcpy(h.magic, kMagic, sizeof kMagic);
    h.version = kVersion;
    h.headerBytes = kHeaderBytes;
    h.step = step;
    h.seed = seed;
    h.n = tf.n;
    h.S = tf.S;
    h.world = tf.world;
    h.rank = tf.rank;
    h.layout = uint32_t(tf.layout);
    h.hasMaster = master ? 1u : 0u;
    h.fingerprint = tf.fingerprint;

    Stage st;
    if (!st.open(static_cast<hipStream_t>(stream))) return fail(st, BFO_EHIP);
    const std::string path = statePath(dir, step, tf.rank);
    const std::string tmp = path + ".tmp";
    FILE *f = std::fopen(tmp.c_str(), "wb");
    if (!f) return BFO_EIO;
    int rc = std::fwrite(&h, 1, sizeof h, f) == sizeof h ? BFO_OK : BFO_EIO;
    if (rc == BFO_OK && master) rc = st.write(f, master, tf.S * sizeof(float));
    if (rc == BFO_OK && !master) {
        for (uint32_t k = 0; rc == BFO_OK && k < tf.nruns; ++k)
            rc = st.write(f, params + tf.runs[k].addr, tf.runs[k].length * sizeof(uint16_t));
    }
    if (rc == BFO_OK) rc = st.write(f, m, tf.S * sizeof(float));
    if (rc == BFO_OK) rc = st.write(f, v, tf.S * sizeof(float));
    if (std::fflush(f) != 0 || fsync(fileno(f)) != 0) rc = rc == BFO_OK ? BFO_EIO : rc;
    if (std::fclose(f) != 0) rc = rc == BFO_OK ? BFO_EIO : rc;
    if (rc == BFO_OK && std::rename(tmp.c_str(), path.c_str()) != 0) rc = BFO_EIO;
    if (rc != BFO_OK) std::remove(tmp.c_str());
    return fail(st, rc);
}

int bfo_checkpoint_done(const char *dir, uint64_t step) {
    if (!dir) return BFO_EINVAL;
    FILE *f = std::fopen(donePath(dir, step).c_str(), "wb");
    if (!f) return BFO_EIO;
    return std::fclose(f) == 0 ? BFO_OK : BFO_EIO;
}

int bfo_checkpoint_latest(const char *dir, uint64_t *step) {
    if (!dir || !step) return BFO_EINVAL;
    DIR *d = opendir(dir);
    if (!d) return BFO_EIO;
    bool found = false;
    uint64_t best = 0;
    while (const dirent *e = readdir(d)) {
        const char *name = e->d_name;
        if (std::strncmp(name, "DONE_", 5) != 0) continue;
        const char *digits = name + 5;
        if (!*digits) continue;
        uint64_t val = 0;
        bool ok = true;
        for (const char *c = digits; *c; ++c) {
            if (*c < '0' || *c > '9' || val > (UINT64_MAX - 9) / 10) {
                ok = false;
                break;
            }
            val = val * 10 + uint64_t(*c - '0');
        }
        if (ok && (!found || val > best)) {
            best = val;
            found = true;
        }
    }
    closedir(d);
    if (!found) return BFO_ENOTFOUND;
    *step = best;
    return BFO_OK;
}

int bfo_checkpoint_load(const char *dir, uint64_t step, bfo_table table, uint16_t *params, float *master,
                        float *m, float *v, uint64_t *seed, void *stream) {
    if (!dir || !table || (!master && !params)) return BFO_EINVAL;
    const bfo::TableFacts tf = bfo::tableFacts(table);
    if (tf.S && (!m || !v)) return BFO_EINVAL;
    const std::string path = statePath(dir, step, tf.rank);
    FILE *f = std::fopen(path.c_str(), "rb");
    if (!f) return errno == ENOENT ? BFO_ENOTFOUND : BFO_EIO;
    Header h;
    int rc = std::fread(&h, 1, sizeof h, f) == sizeof h ? BFO_OK : BFO_EFORMAT;
    if (rc == BFO_OK &&
        (std::memcmp(h.magic, kMagic, sizeof kMagic) != 0 || h.version != kVersion || h.headerBytes != kHeaderBytes ||
         h.step != step || h.n != tf.n || h.S != tf.S || h.world != tf.world || h.rank != tf.rank ||
         h.layout != uint32_t(tf.layout) || h.fingerprint != tf.fingerprint || h.hasMaster != (master ? 1u : 0u)))
        rc = BFO_EFORMAT;
    if (rc == BFO_OK) {
        const uint64_t payload = (h.hasMaster ? 4 : 2) * tf.S + 8 * tf.S;
        if (std::fseek(f, 0, SEEK_END) != 0) rc = BFO_EIO;
        else if (uint64_t(std::ftell(f)) != kHeaderBytes + payload) rc = BFO_EFORMAT;
        else if (std::fseek(f, long(kHeaderBytes), SEEK_SET) != 0) rc = BFO_EIO;
    }
    Stage st;
    if (rc == BFO_OK && !st.open(static_cast<hipStream_t>(stream))) rc = BFO_EHIP;
    if (rc == BFO_OK && master) rc = st.read(f, master, tf.S * sizeof(float));
    if (rc == BFO_OK && !master) {
        for (uint32_t k = 0; rc == BFO_OK && k < tf.nruns; ++k)
            rc = st.read(f, params + tf.runs[k].addr, tf.runs[k].length * sizeof(uint16_t));
    }
    if (rc == BFO_OK) rc = st.read(f, m, tf.S * sizeof(float));
    if (rc == BFO_OK) rc = st.read(f, v, tf.S * sizeof(float));
    std::fclose(f);
    if (rc == BFO_OK && seed) *seed = h.seed;
    return fail(st, rc);
}

}  // extern "C"
