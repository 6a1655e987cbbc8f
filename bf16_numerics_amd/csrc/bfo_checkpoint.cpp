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

// Moves bytes between a device array and a file through a pinned buffer.
struct Stage {
    char *buf = nullptr;
    hipStream_t stream = nullptr;
    hipError_t err = hipSuccess;
    ~Stage() {
        if (buf) (void)hipHostFree(buf);
    }
    bool open(hipStream_t s) {
        stream = s;
        err = hipHostMalloc(reinterpret_cast<void **>(&buf), kStageBytes, hipHostMallocDefault);
        return err == hipSuccess;
    }
    int write(FILE *f, const void *dev, uint64_t bytes) {
        const char *src = static_cast<const char *>(dev);
        for (uint64_t off = 0; off < bytes; off += kStageBytes) {
            const size_t len = size_t(bytes - off < kStageBytes ? bytes - off : kStageBytes);
            if ((err = hipMemcpyAsync(buf, src + off, len, hipMemcpyDeviceToHost, stream)) != hipSuccess ||
                (err = hipStreamSynchronize(stream)) != hipSuccess)
                return BFO_EHIP;
            if (std::fwrite(buf, 1, len, f) != len) return BFO_EIO;
        }
        return BFO_OK;
    }
    int read(FILE *f, void *dev, uint64_t bytes) {
        char *dst = static_cast<char *>(dev);
        for (uint64_t off = 0; off < bytes; off += kStageBytes) {
            const size_t len = size_t(bytes - off < kStageBytes ? bytes - off : kStageBytes);
            if (std::fread(buf, 1, len, f) != len) return BFO_EFORMAT;
            if ((err = hipMemcpyAsync(dst + off, buf, len, hipMemcpyHostToDevice, stream)) != hipSuccess ||
                (err = hipStreamSynchronize(stream)) != hipSuccess)
                return BFO_EHIP;
        }
        return BFO_OK;
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
