// bfo_checkpoint.cpp -- per-rank optimizer-state files and resume.
//
// "04 · 多 GPU 与混合精度" §5.1-5.2: each rank writes its own state (m, v,
// fp32 master, the rounding state of the last update); a DONE marker makes a
// checkpoint count; resume takes the newest step with a marker, reads the
// state back and rebuilds the bf16 weights from the master with the last
// update's draws, so they come back bit-identical.  Because only the master
// is needed, the same state can also resume a run of another precision
// setup: loaded without a master buffer, it rebuilds the bf16 weights and
// the run goes on with no master.  Without a master (the no-master update
// path) the bf16 weights are the state and are stored.
//
// File state_<step:08>_<rank:05>.bin, little-endian:
//   header (kHeaderBytes): magic "BFOSTATE", version, header bytes, step,
//     seed, n, S, world, rank, layout, has_master, table fingerprint
//     (FNV-1a over every tensor's offset, numel and flags), rounding mode
//     of the last update, has_params, a 64-bit checksum of each payload
//     array (bfo_checksum64 of its bytes as stored) and a checksum of the
//     header bytes before it;
//   payload: master S x fp32 (if has_master), the shard's bf16 params in
//     shard-local order (if has_params), then m S x fp32, then v S x fp32.
// Written to a temporary name, synced, renamed into place and the directory
// synced, so a file under the final name is complete and durable; the DONE
// marker is synced with its directory too, so after a power loss a marker
// never outlives the files it vouches for.
#include <hip/hip_runtime_api.h>

#include <dirent.h>
#include <fcntl.h>
#include <unistd.h>

#include <cerrno>
#include <cstddef>
#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "bfo_internal.hpp"

namespace {

constexpr char kMagic[8] = {'B', 'F', 'O', 'S', 'T', 'A', 'T', 'E'};
constexpr uint32_t kVersion = 2;
constexpr uint32_t kHeaderBytes = 128;
constexpr size_t kStageBytes = size_t(64) << 20;

enum { kSumMaster = 0, kSumParams = 1, kSumM = 2, kSumV = 3 };

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
    uint32_t rounding;
    uint32_t hasParams;
    uint64_t checksum[4];     // master, params, m, v (0 when absent)
    uint64_t headerChecksum;  // of the bytes above
    uint8_t reserved[8];
};
static_assert(sizeof(Header) == kHeaderBytes, "checkpoint header layout");
constexpr size_t kHeaderSummed = offsetof(Header, headerChecksum);

// Streaming form of bfo_checksum64: four lanes, each folding every fourth
// 8-byte word of the data in by xor and a multiply by the 64-bit FNV prime
// (both invertible, so a change confined to one word always changes the
// result); the bytes are taken in 32-byte blocks, the last one padded with
// zeros, and the lanes and the byte count are folded together at the end.
class Checksum {
  public:
    void add(const void *data, size_t len) {
        const uint8_t *p = static_cast<const uint8_t *>(data);
        total_ += len;
        if (pending_) {
            const size_t take = len < 32 - pending_ ? len : 32 - pending_;
            std::memcpy(buf_ + pending_, p, take);
            pending_ += take;
            p += take;
            len -= take;
            if (pending_ < 32) return;
            block(buf_);
            pending_ = 0;
        }
        for (; len >= 32; p += 32, len -= 32) block(p);
        std::memcpy(buf_, p, len);
        pending_ = len;
    }
    uint64_t finish() {
        if (pending_) {
            std::memset(buf_ + pending_, 0, 32 - pending_);
            block(buf_);
            pending_ = 0;
        }
        uint64_t x = kBasis ^ total_;
        for (uint64_t h : lane_) {
            x = (x ^ h) * kPrime;
            x ^= x >> 29;
        }
        return x;
    }

  private:
    static constexpr uint64_t kPrime = 1099511628211ull;      // FNV-1a 64-bit prime
    static constexpr uint64_t kBasis = 14695981039346656037ull;  // FNV-1a 64-bit offset basis
    void block(const uint8_t *p) {
        for (int l = 0; l < 4; ++l) {
            uint64_t w;
            std::memcpy(&w, p + 8 * l, 8);
            lane_[l] = (lane_[l] ^ w) * kPrime;
        }
    }
    uint64_t lane_[4] = {kBasis, kBasis + 1, kBasis + 2, kBasis + 3};
    uint64_t total_ = 0;
    uint8_t buf_[32];
    size_t pending_ = 0;
};

// Adds one chunk to a checksum on a helper thread, so that the sum of a
// staged chunk overlaps the file write (or the device copy and the next
// read) of the same bytes.  Chunks are added strictly in order: a chunk's
// task is joined before the next one starts.
class SumTask {
  public:
    ~SumTask() { join(); }
    void start(Checksum &sum, const char *p, size_t n) {
        join();
        try {
            th_ = std::thread([&sum, p, n] { sum.add(p, n); });
        } catch (...) {
            sum.add(p, n);  // no thread to be had: sum on this one
        }
    }
    void join() {
        if (th_.joinable()) th_.join();
    }

  private:
    std::thread th_;
};

uint64_t headerSum(const Header &h) {
    Checksum c;
    c.add(&h, kHeaderSummed);
    return c.finish();
}

// fsync of a directory, so that a rename or a new file in it survives a crash.
int syncDir(const char *dir) {
    const int fd = open(dir, O_RDONLY | O_DIRECTORY);
    if (fd < 0) return BFO_EIO;
    const int rc = fsync(fd);
    close(fd);
    return rc == 0 ? BFO_OK : BFO_EIO;
}

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
    // Device -> file: chunk k+1 is copied while chunk k is written; every
    // byte written also goes into `sum`.
    int write(FILE *f, const void *dev, uint64_t bytes, Checksum &sum) {
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
        SumTask task;
        for (uint64_t k = 0; k < chunks; ++k) {
            const int h = int(k & 1);
            if ((err = hipEventSynchronize(done[h])) != hipSuccess) return BFO_EHIP;
            // the other half is refilled only once its sum is done
            task.join();
            if (k + 1 < chunks && !fetch(k + 1)) return BFO_EHIP;
            task.start(sum, half(h), len(k));
            if (std::fwrite(half(h), 1, len(k), f) != len(k)) return BFO_EIO;
        }
        return BFO_OK;
    }
    // File -> device: chunk k+1 is read while chunk k is copied; every byte
    // read also goes into `sum`.
    int read(FILE *f, void *dev, uint64_t bytes, Checksum &sum) {
        char *dst = static_cast<char *>(dev);
        const uint64_t chunks = (bytes + kHalf - 1) / kHalf;
        int rc = BFO_OK;
        bool pending[2] = {false, false};
        SumTask task;
        for (uint64_t k = 0; k < chunks && rc == BFO_OK; ++k) {
            const int h = int(k & 1);
            const size_t n = size_t(bytes - k * kHalf < kHalf ? bytes - k * kHalf : kHalf);
            if (pending[h] && (err = hipEventSynchronize(done[h])) != hipSuccess) {
                rc = BFO_EHIP;
                break;
            }
            pending[h] = false;
            // half h was summed as chunk k-2; chunk k-1's sum must finish
            // before chunk k's starts, and it overlaps this read
            if (std::fread(half(h), 1, n, f) != n) {
                rc = BFO_EFORMAT;
                break;
            }
            task.start(sum, half(h), n);
            if ((err = hipMemcpyAsync(dst + k * kHalf, half(h), n, hipMemcpyHostToDevice, stream)) != hipSuccess ||
                (err = hipEventRecord(done[h], stream)) != hipSuccess) {
                rc = BFO_EHIP;
                break;
            }
            pending[h] = true;
        }
        task.join();
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

// The shard's bf16 params, shard-local order, through the run plan.
int writeParams(Stage &st, FILE *f, const bfo::TableFacts &tf, const uint16_t *params, Checksum &sum) {
    int rc = BFO_OK;
    for (uint32_t k = 0; rc == BFO_OK && k < tf.nruns; ++k)
        rc = st.write(f, params + tf.runs[k].addr, tf.runs[k].length * sizeof(uint16_t), sum);
    return rc;
}

int readParams(Stage &st, FILE *f, const bfo::TableFacts &tf, uint16_t *params, Checksum &sum) {
    int rc = BFO_OK;
    for (uint32_t k = 0; rc == BFO_OK && k < tf.nruns; ++k)
        rc = st.read(f, params + tf.runs[k].addr, tf.runs[k].length * sizeof(uint16_t), sum);
    return rc;
}

// Skips `bytes` of the file, adding them to `sum` (the checksum of an array
// that this load does not need still has to hold).
int skipSummed(FILE *f, uint64_t bytes, Checksum &sum, std::vector<char> &buf) {
    buf.resize(size_t(1) << 20);
    while (bytes) {
        const size_t n = bytes < buf.size() ? size_t(bytes) : buf.size();
        if (std::fread(buf.data(), 1, n, f) != n) return BFO_EFORMAT;
        sum.add(buf.data(), n);
        bytes -= n;
    }
    return BFO_OK;
}

}  // namespace

extern "C" {

uint64_t bfo_checksum64(const void *data, uint64_t bytes) {
    Checksum c;
    if (bytes) c.add(data, size_t(bytes));
    return c.finish();
}

int bfo_checkpoint_save(const char *dir, bfo_table table, const uint16_t *params, const float *master,
                        const float *m, const float *v, uint64_t step, uint64_t seed, int rounding, void *stream) {
    if (!dir || !table || (!master && !params)) return BFO_EINVAL;
    if (rounding != BFO_ROUND_SR && rounding != BFO_ROUND_RNE) return BFO_EINVAL;
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
    h.hasParams = params ? 1u : 0u;
    h.fingerprint = tf.fingerprint;
    h.rounding = uint32_t(rounding);

    Stage st;
    if (!st.open(static_cast<hipStream_t>(stream))) return fail(st, BFO_EHIP);
    const std::string path = statePath(dir, step, tf.rank);
    const std::string tmp = path + ".tmp";
    FILE *f = std::fopen(tmp.c_str(), "wb");
    if (!f) return BFO_EIO;
    // The header goes in last, once the payload's checksums are known.
    int rc = std::fseek(f, long(kHeaderBytes), SEEK_SET) == 0 ? BFO_OK : BFO_EIO;
    Checksum sums[4];
    if (rc == BFO_OK && master) rc = st.write(f, master, tf.S * sizeof(float), sums[kSumMaster]);
    if (rc == BFO_OK && params) rc = writeParams(st, f, tf, params, sums[kSumParams]);
    if (rc == BFO_OK) rc = st.write(f, m, tf.S * sizeof(float), sums[kSumM]);
    if (rc == BFO_OK) rc = st.write(f, v, tf.S * sizeof(float), sums[kSumV]);
    if (rc == BFO_OK) {
        if (master) h.checksum[kSumMaster] = sums[kSumMaster].finish();
        if (params) h.checksum[kSumParams] = sums[kSumParams].finish();
        h.checksum[kSumM] = sums[kSumM].finish();
        h.checksum[kSumV] = sums[kSumV].finish();
        h.headerChecksum = headerSum(h);
        if (std::fseek(f, 0, SEEK_SET) != 0 || std::fwrite(&h, 1, sizeof h, f) != sizeof h) rc = BFO_EIO;
    }
    if (std::fflush(f) != 0 || fsync(fileno(f)) != 0) rc = rc == BFO_OK ? BFO_EIO : rc;
    if (std::fclose(f) != 0) rc = rc == BFO_OK ? BFO_EIO : rc;
    if (rc == BFO_OK && std::rename(tmp.c_str(), path.c_str()) != 0) rc = BFO_EIO;
    if (rc == BFO_OK) rc = syncDir(dir);
    if (rc != BFO_OK) std::remove(tmp.c_str());
    return fail(st, rc);
}

int bfo_checkpoint_done(const char *dir, uint64_t step) {
    if (!dir) return BFO_EINVAL;
    const int fd = open(donePath(dir, step).c_str(), O_WRONLY | O_CREAT | O_TRUNC, 0644);
    if (fd < 0) return BFO_EIO;
    const int synced = fsync(fd);
    if (close(fd) != 0 || synced != 0) return BFO_EIO;
    return syncDir(dir);
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
         h.headerChecksum != headerSum(h) || h.step != step || h.n != tf.n || h.S != tf.S || h.world != tf.world ||
         h.rank != tf.rank || h.layout != uint32_t(tf.layout) || h.fingerprint != tf.fingerprint ||
         h.hasMaster > 1 || h.hasParams > 1 || (!h.hasMaster && !h.hasParams) ||
         (h.rounding != BFO_ROUND_SR && h.rounding != BFO_ROUND_RNE)))
        rc = BFO_EFORMAT;
    // A master buffer needs a stored master; without one, the params are
    // read or (from a master) rebuilt.
    if (rc == BFO_OK && master && !h.hasMaster) rc = BFO_EFORMAT;
    if (rc == BFO_OK) {
        const uint64_t payload = (h.hasMaster ? 4 : 0) * tf.S + (h.hasParams ? 2 : 0) * tf.S + 8 * tf.S;
        if (std::fseek(f, 0, SEEK_END) != 0) rc = BFO_EIO;
        else if (uint64_t(std::ftell(f)) != kHeaderBytes + payload) rc = BFO_EFORMAT;
        else if (std::fseek(f, long(kHeaderBytes), SEEK_SET) != 0) rc = BFO_EIO;
    }
    Stage st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (rc == BFO_OK && !st.open(s)) rc = BFO_EHIP;
    Checksum sums[4];
    std::vector<char> skipBuf;
    // Where the stored master goes: the caller's master, or -- to rebuild the
    // params of a run without one -- v's buffer, which is read last.
    const bool rebuild = params && !h.hasParams;
    float *masterDst = master ? master : (rebuild ? v : nullptr);
    if (rc == BFO_OK && h.hasMaster) {
        rc = masterDst ? st.read(f, masterDst, tf.S * sizeof(float), sums[kSumMaster])
                       : skipSummed(f, tf.S * sizeof(float), sums[kSumMaster], skipBuf);
        if (rc == BFO_OK && sums[kSumMaster].finish() != h.checksum[kSumMaster]) rc = BFO_EFORMAT;
    }
    if (rc == BFO_OK && h.hasParams) {
        rc = params ? readParams(st, f, tf, params, sums[kSumParams])
                    : skipSummed(f, tf.S * sizeof(uint16_t), sums[kSumParams], skipBuf);
        if (rc == BFO_OK && sums[kSumParams].finish() != h.checksum[kSumParams]) rc = BFO_EFORMAT;
    }
    // Rebuild before v's buffer is overwritten (same stream, so in order).
    if (rc == BFO_OK && rebuild) rc = bfo::rebuildParams(table, masterDst, params, h.seed, int(h.rounding), s);
    if (rc == BFO_OK) rc = st.read(f, m, tf.S * sizeof(float), sums[kSumM]);
    if (rc == BFO_OK && sums[kSumM].finish() != h.checksum[kSumM]) rc = BFO_EFORMAT;
    if (rc == BFO_OK) rc = st.read(f, v, tf.S * sizeof(float), sums[kSumV]);
    if (rc == BFO_OK && sums[kSumV].finish() != h.checksum[kSumV]) rc = BFO_EFORMAT;
    std::fclose(f);
    if (rc == BFO_OK && seed) *seed = h.seed;
    return fail(st, rc);
}

}  // extern "C"
