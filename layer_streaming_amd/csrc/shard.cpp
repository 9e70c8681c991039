// Checkpoint shards: one file per unit holding the unit's whole tile (BF16
// W and G, FP32 master, m and v), so a run can resume from the state of any
// layer and a restore can load each layer only when the stream reaches it
// ([Hotdry] "Checkpoint 分片与恢复策略": per-layer shards on the host side,
// lazy loading on restart).
//
// File layout: a 256-byte header (magic, format version, unit index, the
// model shape, region length in elements, the step count, a checksum of the
// five regions), then the regions W | G | master | m | v back to back.  The
// checksum is FNV-1a (64-bit, over 8-byte words) of each 16 MiB chunk,
// mixed with the chunk's index and summed, so it does not depend on how the
// chunks are split among threads.
#include <errno.h>
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <atomic>
#include <cstring>
#include <string>

#include "host.h"

namespace mt {

namespace {

constexpr char MAGIC[8] = {'M', 'T', 'T', 'I', 'L', 'E', '0', '1'};
constexpr uint32_t VERSION = 1;
constexpr int64_t CHUNK = int64_t(16) << 20;

struct Header {
    char magic[8];
    uint32_t version;
    int32_t unit;
    mt_shape shape;
    int64_t elems;
    int64_t step;
    uint64_t checksum;
};
static_assert(sizeof(Header) <= 256, "header fits its 256-byte slot");

inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t fnv1a_words(const uint8_t* p, int64_t n) {
    uint64_t h = 0xCBF29CE484222325ull;
    int64_t i = 0;
    for (; i + 8 <= n; i += 8) {
        uint64_t w;
        memcpy(&w, p + i, 8);
        h = (h ^ w) * 0x100000001B3ull;
    }
    for (; i < n; ++i) h = (h ^ p[i]) * 0x100000001B3ull;
    return h;
}

struct Region {
    uint8_t* p;
    int64_t bytes;
};

void regions_of(const TilePtrs& t, int64_t elems, Region (&r)[5]) {
    r[0] = {reinterpret_cast<uint8_t*>(t.w), elems * 2};
    r[1] = {reinterpret_cast<uint8_t*>(t.g), elems * 2};
    r[2] = {reinterpret_cast<uint8_t*>(t.master), elems * 4};
    r[3] = {reinterpret_cast<uint8_t*>(t.m), elems * 4};
    r[4] = {reinterpret_cast<uint8_t*>(t.v), elems * 4};
}

uint64_t checksum(ThreadPool& pool, const Region (&r)[5]) {
    std::atomic<uint64_t> sum{0};
    uint64_t base = 0;  // running chunk index across regions
    for (const Region& g : r) {
        const int64_t nch = (g.bytes + CHUNK - 1) / CHUNK;
        pool.parallel_for(nch, 1, [&](int64_t b, int64_t e) {
            uint64_t s = 0;
            for (int64_t c = b; c < e; ++c) {
                const int64_t lo = c * CHUNK, n = std::min(CHUNK, g.bytes - lo);
                s += mix64(fnv1a_words(g.p + lo, n) + (base + uint64_t(c)) * 0x9E3779B97F4A7C15ull);
            }
            sum.fetch_add(s, std::memory_order_relaxed);
        });
        base += uint64_t(nch);
    }
    return sum.load();
}

bool write_all(int fd, const uint8_t* p, int64_t n) {
    while (n > 0) {
        const ssize_t w = ::write(fd, p, size_t(std::min<int64_t>(n, int64_t(1) << 30)));
        if (w < 0 && errno == EINTR) continue;
        if (w <= 0) return false;
        p += w;
        n -= w;
    }
    return true;
}

bool read_all(int fd, uint8_t* p, int64_t n) {
    while (n > 0) {
        const ssize_t r = ::read(fd, p, size_t(std::min<int64_t>(n, int64_t(1) << 30)));
        if (r < 0 && errno == EINTR) continue;
        if (r <= 0) return false;
        p += r;
        n -= r;
    }
    return true;
}

bool same_shape(const mt_shape& a, const mt_shape& b) {
    return a.n_layers == b.n_layers && a.d_model == b.d_model && a.n_heads == b.n_heads &&
           a.n_kv_heads == b.n_kv_heads && a.head_dim == b.head_dim && a.ffn_dim == b.ffn_dim &&
           a.vocab == b.vocab && a.rms_eps == b.rms_eps && a.rope_base == b.rope_base;
}

}  // namespace

std::string shard_path(const std::string& dir, int unit) {
    char name[32];
    snprintf(name, sizeof name, "/unit_%05d.mtt", unit);
    return dir + name;
}

int save_shard(ThreadPool& pool, const std::string& dir, const TilePtrs& t, const Layout& lay, int unit,
               int64_t step) {
    if (mkdir(dir.c_str(), 0755) != 0 && errno != EEXIST)
        MT_FAIL(MT_E_IO, "cannot create checkpoint directory %s: %s", dir.c_str(), strerror(errno));
    Region r[5];
    regions_of(t, lay.units[unit].elems, r);
    uint8_t hdr[256] = {};
    Header h{};
    memcpy(h.magic, MAGIC, 8);
    h.version = VERSION;
    h.unit = unit;
    h.shape = lay.sh;
    h.elems = lay.units[unit].elems;
    h.step = step;
    h.checksum = checksum(pool, r);
    memcpy(hdr, &h, sizeof h);
    const std::string path = shard_path(dir, unit), tmp = path + ".tmp";
    const int fd = ::open(tmp.c_str(), O_WRONLY | O_CREAT | O_TRUNC, 0644);
    if (fd < 0) MT_FAIL(MT_E_IO, "cannot create %s: %s", tmp.c_str(), strerror(errno));
    bool ok = write_all(fd, hdr, sizeof hdr);
    for (const Region& g : r) ok = ok && write_all(fd, g.p, g.bytes);
    ok = (::close(fd) == 0) && ok;
    if (!ok || ::rename(tmp.c_str(), path.c_str()) != 0) {
        ::unlink(tmp.c_str());
        MT_FAIL(MT_E_IO, "cannot write %s: %s", path.c_str(), strerror(errno));
    }
    return MT_OK;
}

int check_shard(const std::string& dir, const Layout& lay, int unit, int64_t* step) {
    const std::string path = shard_path(dir, unit);
    const int fd = ::open(path.c_str(), O_RDONLY);
    if (fd < 0) MT_FAIL(MT_E_IO, "cannot open %s: %s", path.c_str(), strerror(errno));
    uint8_t hdr[256];
    const bool ok = read_all(fd, hdr, sizeof hdr);
    struct stat st {};
    const bool sized = fstat(fd, &st) == 0;
    ::close(fd);
    if (!ok) MT_FAIL(MT_E_IO, "%s: short header", path.c_str());
    Header h;
    memcpy(&h, hdr, sizeof h);
    if (memcmp(h.magic, MAGIC, 8) != 0 || h.version != VERSION)
        MT_FAIL(MT_E_IO, "%s is not a checkpoint shard of this format", path.c_str());
    if (h.unit != unit || !same_shape(h.shape, lay.sh) || h.elems != lay.units[unit].elems)
        MT_FAIL(MT_E_INVAL, "%s holds unit %d of another model shape", path.c_str(), h.unit);
    if (!sized || int64_t(st.st_size) != 256 + lay.units[unit].tile_bytes())
        MT_FAIL(MT_E_IO, "%s: size %lld, expected %lld", path.c_str(), (long long)st.st_size,
                (long long)(256 + lay.units[unit].tile_bytes()));
    if (h.step < 0) MT_FAIL(MT_E_IO, "%s: bad step count", path.c_str());
    *step = h.step;
    return MT_OK;
}

int load_shard(ThreadPool& pool, const std::string& dir, const TilePtrs& t, const Layout& lay, int unit) {
    const std::string path = shard_path(dir, unit);
    const int fd = ::open(path.c_str(), O_RDONLY);
    if (fd < 0) MT_FAIL(MT_E_IO, "cannot open %s: %s", path.c_str(), strerror(errno));
    uint8_t hdr[256];
    Region r[5];
    regions_of(t, lay.units[unit].elems, r);
    bool ok = read_all(fd, hdr, sizeof hdr);
    for (const Region& g : r) ok = ok && read_all(fd, g.p, g.bytes);
    ::close(fd);
    if (!ok) MT_FAIL(MT_E_IO, "%s: short read", path.c_str());
    Header h;
    memcpy(&h, hdr, sizeof h);
    if (checksum(pool, r) != h.checksum) MT_FAIL(MT_E_IO, "%s: checksum mismatch", path.c_str());
    return MT_OK;
}

}  // namespace mt
