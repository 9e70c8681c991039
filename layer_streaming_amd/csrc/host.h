// Host-side pieces of the layer-streamed trainer: the unit/tile layout, the
// host master store, the host Adam, a small thread pool, error reporting.
#pragma once
#include <stdint.h>

#include <atomic>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/mt.h"

namespace mt {

// ------------------------------------------------------------ errors ----
void set_error(const std::string& msg);
const char* last_error();
struct Status {
    int code = MT_OK;
    bool ok() const { return code == MT_OK; }
};
#define MT_FAIL(code_, ...)                                         \
    do {                                                            \
        ::mt::set_error(::mt::strfmt(__VA_ARGS__));                 \
        return (code_);                                             \
    } while (0)
std::string strfmt(const char* fmt, ...);

// ------------------------------------------------------------ layout ----
// A unit is a decoder layer, the LM head or the input embedding.  Its tile
// in the host store is [W bf16 | G bf16 | master f32 | m f32 | v f32], each
// region `elems` long (elems a multiple of 128, so every region is 256-byte
// aligned); tensor offsets are the same in every region.
enum UnitKind { UNIT_LAYER = 0, UNIT_HEAD = 1, UNIT_EMBED = 2 };
enum LayerTensor { T_G1 = 0, T_WQ, T_WK, T_WV, T_WO, T_G2, T_WG, T_WU, T_WD };
enum HeadTensor { T_GF = 0, T_EOUT = 1 };

struct TensorDesc {
    const char* name;
    int64_t rows, cols;  // gains: rows = 1
    int64_t off;         // element offset inside the unit region
};
struct UnitLayout {
    int kind;
    int ntensors;
    TensorDesc t[9];
    int64_t elems;  // padded element count of one region
    int64_t tile_bytes() const { return elems * 16; }
};
struct Layout {
    mt_shape sh{};
    std::vector<UnitLayout> units;   // L layers, head, embedding
    std::vector<int64_t> tile_off;   // byte offset of each tile in the store
    int64_t store_bytes = 0;
    // With the weights kept apart in one page-locked block: byte offset of
    // each unit's W region in that block, and its size.
    std::vector<int64_t> w_off;
    int64_t w_bytes = 0;
    int64_t max_stream_elems = 0;    // largest streamed unit (layers, head)
    int64_t n_params = 0;            // unpadded parameter count
    int L() const { return sh.n_layers; }
    int head() const { return sh.n_layers; }
    int embed() const { return sh.n_layers + 1; }
};
int validate_shape(const mt_shape* sh);
Layout make_layout(const mt_shape& sh);

// Host pointers into a unit tile.  With `wblock` (the page-locked weight
// block) W points there instead of into the tile.
struct TilePtrs {
    uint16_t* w;
    uint16_t* g;
    float* master;
    float* m;
    float* v;
};
inline TilePtrs tile_ptrs(uint8_t* store, const Layout& lay, int unit, uint8_t* wblock = nullptr) {
    uint8_t* b = store + lay.tile_off[unit];
    const int64_t n = lay.units[unit].elems;
    TilePtrs p;
    p.w = reinterpret_cast<uint16_t*>(wblock ? wblock + lay.w_off[unit] : b);
    p.g = reinterpret_cast<uint16_t*>(b + 2 * n);
    p.master = reinterpret_cast<float*>(b + 4 * n);
    p.m = reinterpret_cast<float*>(b + 8 * n);
    p.v = reinterpret_cast<float*>(b + 12 * n);
    return p;
}

// --------------------------------------------------------- bf16 (host) ----
inline float bf16_to_f32(uint16_t b) {
    uint32_t u = uint32_t(b) << 16;
    float f;
    __builtin_memcpy(&f, &u, 4);
    return f;
}
inline uint16_t f32_to_bf16(float f) {
    uint32_t u;
    __builtin_memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return uint16_t((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// -------------------------------------------------------- thread pool ----
// parallel_for splits [0, n) into chunks of at least `grain` and runs them
// on the pool's workers and the calling thread.  Submissions from several
// threads are serialised.
class ThreadPool {
public:
    explicit ThreadPool(int nthreads);
    ~ThreadPool();
    int size() const { return int(workers_.size()) + 1; }
    void parallel_for(int64_t n, int64_t grain, const std::function<void(int64_t, int64_t)>& fn);

private:
    void worker_loop();
    void run_chunks();
    std::vector<std::thread> workers_;
    std::mutex submit_mu_, mu_;
    std::condition_variable cv_, done_cv_;
    const std::function<void(int64_t, int64_t)>* fn_ = nullptr;
    int64_t n_ = 0, chunk_ = 1, nchunks_ = 0;
    std::atomic<int64_t> next_{0};
    int active_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
};

// Copy `bytes` with the pool (pack of a unit into pinned staging).
void parallel_copy(ThreadPool& pool, void* dst, const void* src, int64_t bytes);

// ------------------------------------------------------------- store ----
// Deterministic init of one unit: matrices N(0, std^2) from a counter-based
// SplitMix64 stream per tensor and Box-Muller, rounded to bf16; gains 1.0;
// master = W; G = m = v = 0; padding 0.
void init_unit(ThreadPool& pool, uint8_t* store, const Layout& lay, int unit, uint64_t seed,
               float std_, uint8_t* wblock = nullptr);

// Adam hyper-parameters for one step (bias corrections already computed).
struct AdamStep {
    float lr, b1, omb1, b2, omb2, eps, bc1, bc2;
};
AdamStep adam_step_params(const mt_options& o, int64_t t);
// Fused gradient unpack + Adam over elements [0, n) of a tile: G <- gsrc
// (bf16), then m, v, master updated in fp32 and W refreshed as bf16(master).
// If gsrc == tile G region, the copy is skipped.
void adam_range(const TilePtrs& p, const uint16_t* gsrc, int64_t b, int64_t e, const AdamStep& a);
void adam_unit(ThreadPool& pool, const TilePtrs& p, const uint16_t* gsrc, int64_t n,
               const AdamStep& a);
// G <- bf16(G + src) elementwise (gradient accumulation across micro-batches).
void accum_range(uint16_t* G, const uint16_t* src, int64_t b, int64_t e);
void accum_unit(ThreadPool& pool, uint16_t* G, const uint16_t* src, int64_t n);

// ------------------------------------------------- checkpoint shards ----
std::string shard_path(const std::string& dir, int unit);
int save_shard(ThreadPool& pool, const std::string& dir, const TilePtrs& t, const Layout& lay, int unit,
               int64_t step);
int check_shard(const std::string& dir, const Layout& lay, int unit, int64_t* step);
int load_shard(ThreadPool& pool, const std::string& dir, const TilePtrs& t, const Layout& lay, int unit);

}  // namespace mt
