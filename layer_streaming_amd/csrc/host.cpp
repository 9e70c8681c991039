// Host side: layout, errors, thread pool, store init and host Adam.
//
// Pages cited:
//   [Review]  MegaTrain review, dimensionstp.github.io/study-concept/megatrain/
//   [Hotdry]  MegaTrain checkpoint strategy and communication overlap, blog.hotdry.top
//   [Lilting] MegaTrain article, lilting.ch
#include <immintrin.h>
#include <math.h>
#include <stdarg.h>
#include <string.h>

#include <algorithm>

#include "host.h"

namespace mt {

// ------------------------------------------------------------ errors ----
static thread_local std::string tl_error;
void set_error(const std::string& msg) { tl_error = msg; }
const char* last_error() { return tl_error.c_str(); }
std::string strfmt(const char* fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return buf;
}

// ------------------------------------------------------------ layout ----
// One contiguous tile per unit holding BF16 W, BF16 G and the FP32 master,
// m and v, so a unit's weights leave the store as one burst ([Review] 3-2
// item 4 "Layer-contiguous tiling"; [Hotdry] "主机端内存布局"; [Lilting]
// 16 bytes per parameter).  Inside the W region the fused GEMM operands
// wq|wk|wv and wg|wu are contiguous; other tensors start on 128 elements.
static int64_t al128(int64_t x) { return (x + 127) & ~int64_t(127); }

int validate_shape(const mt_shape* sh) {
    if (!sh) MT_FAIL(MT_E_INVAL, "shape is NULL");
    if (sh->n_layers < 1 || sh->d_model < 8 || sh->n_heads < 1 || sh->n_kv_heads < 1 ||
        sh->ffn_dim < 8 || sh->vocab < 8)
        MT_FAIL(MT_E_INVAL, "shape has a non-positive dimension");
    if ((sh->d_model & 7) || (sh->ffn_dim & 7) || (sh->vocab & 7))
        MT_FAIL(MT_E_INVAL, "d_model, ffn_dim and vocab must be multiples of 8");
    if (sh->head_dim != 64 && sh->head_dim != 128) MT_FAIL(MT_E_INVAL, "head_dim must be 64 or 128");
    if (sh->n_heads % sh->n_kv_heads) MT_FAIL(MT_E_INVAL, "n_heads must be a multiple of n_kv_heads");
    if (sh->d_model > 8192) MT_FAIL(MT_E_INVAL, "d_model above 8192 is not supported");
    if (!(sh->rms_eps > 0.f) || !(sh->rope_base > 1.f)) MT_FAIL(MT_E_INVAL, "bad rms_eps or rope_base");
    return MT_OK;
}

Layout make_layout(const mt_shape& sh) {
    Layout lay;
    lay.sh = sh;
    const int64_t d = sh.d_model, hq = int64_t(sh.n_heads) * sh.head_dim,
                  hkv = int64_t(sh.n_kv_heads) * sh.head_dim, f = sh.ffn_dim, V = sh.vocab;
    UnitLayout ly{};
    ly.kind = UNIT_LAYER;
    ly.ntensors = 9;
    int64_t o = 0;
    ly.t[T_G1] = {"g1", 1, d, o};           o = al128(o + d);
    ly.t[T_WQ] = {"wq", hq, d, o};          o += hq * d;
    ly.t[T_WK] = {"wk", hkv, d, o};         o += hkv * d;
    ly.t[T_WV] = {"wv", hkv, d, o};         o = al128(o + hkv * d);
    ly.t[T_WO] = {"wo", d, hq, o};          o = al128(o + d * hq);
    ly.t[T_G2] = {"g2", 1, d, o};           o = al128(o + d);
    ly.t[T_WG] = {"wg", f, d, o};           o += f * d;
    ly.t[T_WU] = {"wu", f, d, o};           o = al128(o + f * d);
    ly.t[T_WD] = {"wd", d, f, o};           o = al128(o + d * f);
    ly.elems = o;
    UnitLayout hd{};
    hd.kind = UNIT_HEAD;
    hd.ntensors = 2;
    o = 0;
    hd.t[T_GF] = {"gf", 1, d, o};           o = al128(o + d);
    hd.t[T_EOUT] = {"e_out", V, d, o};      o = al128(o + V * d);
    hd.elems = o;
    UnitLayout em{};
    em.kind = UNIT_EMBED;
    em.ntensors = 1;
    em.t[0] = {"e_in", V, d, 0};
    em.elems = al128(V * d);

    for (int i = 0; i < sh.n_layers; ++i) lay.units.push_back(ly);
    lay.units.push_back(hd);
    lay.units.push_back(em);
    int64_t off = 0;
    for (auto& u : lay.units) {
        lay.tile_off.push_back(off);
        off += (u.tile_bytes() + 4095) & ~int64_t(4095);
    }
    lay.store_bytes = off;
    int64_t woff = 0;
    for (auto& u : lay.units) {
        lay.w_off.push_back(woff);
        woff += (u.elems * 2 + 4095) & ~int64_t(4095);
    }
    lay.w_bytes = woff;
    lay.max_stream_elems = std::max(ly.elems, hd.elems);
    int64_t per_layer = 0;
    for (int i = 0; i < 9; ++i) per_layer += ly.t[i].rows * ly.t[i].cols;
    lay.n_params = per_layer * sh.n_layers + d + V * d + V * d;
    return lay;
}

// -------------------------------------------------------- thread pool ----
ThreadPool::ThreadPool(int nthreads) {
    for (int i = 1; i < std::max(1, nthreads); ++i) workers_.emplace_back([this] { worker_loop(); });
}
ThreadPool::~ThreadPool() {
    {
        std::lock_guard<std::mutex> lk(mu_);
        stop_ = true;
    }
    cv_.notify_all();
    for (auto& t : workers_) t.join();
}
void ThreadPool::run_chunks() {
    for (;;) {
        const int64_t c = next_.fetch_add(1);
        if (c >= nchunks_) break;
        const int64_t b = c * chunk_, e = std::min(n_, b + chunk_);
        (*fn_)(b, e);
    }
}
void ThreadPool::worker_loop() {
    uint64_t seen = 0;
    for (;;) {
        {
            std::unique_lock<std::mutex> lk(mu_);
            cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
            if (stop_) return;
            seen = gen_;
            // Woken after every chunk of this job was claimed: the submitter may
            // already have returned and be writing the next job's fields (and
            // resetting the chunk counter) without waiting for this thread, so
            // it must not touch them; it waits for the next generation instead.
            if (next_.load() >= nchunks_) continue;
            ++active_;
        }
        run_chunks();
        {
            std::lock_guard<std::mutex> lk(mu_);
            if (--active_ == 0) done_cv_.notify_all();
        }
    }
}
void ThreadPool::parallel_for(int64_t n, int64_t grain,
                              const std::function<void(int64_t, int64_t)>& fn) {
    if (n <= 0) return;
    std::lock_guard<std::mutex> sub(submit_mu_);
    const int64_t parts = int64_t(size()) * 4;
    int64_t chunk = std::max<int64_t>(grain, (n + parts - 1) / parts);
    if (workers_.empty() || n <= chunk) {
        fn(0, n);
        return;
    }
    {
        std::lock_guard<std::mutex> lk(mu_);
        fn_ = &fn;
        n_ = n;
        chunk_ = chunk;
        nchunks_ = (n + chunk - 1) / chunk;
        next_.store(0);
        ++gen_;
    }
    cv_.notify_all();
    run_chunks();
    std::unique_lock<std::mutex> lk(mu_);
    done_cv_.wait(lk, [&] { return active_ == 0 && next_.load() >= nchunks_; });
    fn_ = nullptr;
}

// Copy into a buffer the CPU does not read back (a pinned staging buffer the
// DMA engine drains): streaming stores skip the read-for-ownership of every
// destination line, a third of a plain copy's memory traffic.
static void nt_copy(char* dst, const char* src, int64_t n) {
    const int64_t head = std::min<int64_t>(n, int64_t((32 - (reinterpret_cast<uintptr_t>(dst) & 31)) & 31));
    memcpy(dst, src, size_t(head));
    int64_t i = head;
    for (; i + 128 <= n; i += 128) {
        const __m256i a = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(src + i));
        const __m256i b = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(src + i + 32));
        const __m256i c = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(src + i + 64));
        const __m256i d = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(src + i + 96));
        _mm256_stream_si256(reinterpret_cast<__m256i*>(dst + i), a);
        _mm256_stream_si256(reinterpret_cast<__m256i*>(dst + i + 32), b);
        _mm256_stream_si256(reinterpret_cast<__m256i*>(dst + i + 64), c);
        _mm256_stream_si256(reinterpret_cast<__m256i*>(dst + i + 96), d);
    }
    memcpy(dst + i, src + i, size_t(n - i));
    _mm_sfence();  // drain the write-combining buffers before the copy is reported done
}

void parallel_copy(ThreadPool& pool, void* dst, const void* src, int64_t bytes) {
    const int64_t unit = 1 << 20;
    const int64_t nblk = (bytes + unit - 1) / unit;
    pool.parallel_for(nblk, 1, [&](int64_t b, int64_t e) {
        const int64_t lo = b * unit, hi = std::min(bytes, e * unit);
        nt_copy(static_cast<char*>(dst) + lo, static_cast<const char*>(src) + lo, hi - lo);
    });
}

// ------------------------------------------------------------- init -----
// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", 2014): output n of a generator seeded with `key` is
// mix(key + (n + 1) * golden).  Used counter-style, one stream per tensor.
static inline uint64_t splitmix_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static constexpr uint64_t GOLDEN = 0x9E3779B97F4A7C15ull;
static inline uint64_t splitmix_at(uint64_t key, uint64_t n) { return splitmix_mix(key + (n + 1) * GOLDEN); }

void init_unit(ThreadPool& pool, uint8_t* store, const Layout& lay, int unit, uint64_t seed,
               float std_, uint8_t* wblock) {
    const UnitLayout& u = lay.units[unit];
    const TilePtrs p = tile_ptrs(store, lay, unit, wblock);
    const int64_t n = u.elems;
    // Zero everything first (padding included), in parallel: first touch.
    pool.parallel_for(n, 1 << 16, [&](int64_t b, int64_t e) {
        memset(p.w + b, 0, size_t(e - b) * 2);
        memset(p.g + b, 0, size_t(e - b) * 2);
        memset(p.m + b, 0, size_t(e - b) * 4);
        memset(p.v + b, 0, size_t(e - b) * 4);
        memset(p.master + b, 0, size_t(e - b) * 4);
    });
    for (int j = 0; j < u.ntensors; ++j) {
        const TensorDesc& td = u.t[j];
        const int64_t cnt = td.rows * td.cols;
        uint16_t* w = p.w + td.off;
        float* ms = p.master + td.off;
        if (td.rows == 1) {  // gain vector: 1.0
            for (int64_t i = 0; i < cnt; ++i) {
                w[i] = 0x3F80;
                ms[i] = 1.0f;
            }
            continue;
        }
        const uint64_t key = splitmix_mix(seed ^ (uint64_t(unit) * 16 + uint64_t(j) + 1) * GOLDEN);
        const int64_t npairs = (cnt + 1) / 2;
        pool.parallel_for(npairs, 1 << 14, [&](int64_t b, int64_t e) {
            for (int64_t pi = b; pi < e; ++pi) {
                const uint64_t x = splitmix_at(key, uint64_t(2 * pi));
                const uint64_t y = splitmix_at(key, uint64_t(2 * pi + 1));
                const double u1 = double((x >> 11) + 1) * 0x1.0p-53;  // (0, 1]
                const double u2 = double(y >> 11) * 0x1.0p-53;        // [0, 1)
                const double r = sqrt(-2.0 * log(u1));
                const double a = 6.283185307179586 * u2;
                const int64_t i0 = 2 * pi;
                const uint16_t w0 = f32_to_bf16(float(r * cos(a) * std_));
                w[i0] = w0;
                ms[i0] = bf16_to_f32(w0);
                if (i0 + 1 < cnt) {
                    const uint16_t w1 = f32_to_bf16(float(r * sin(a) * std_));
                    w[i0 + 1] = w1;
                    ms[i0 + 1] = bf16_to_f32(w1);
                }
            }
        });
    }
}

// ------------------------------------------------------------- Adam -----
// Adam on the FP32 master, m and v held in host memory, run by host threads
// as soon as a unit's BF16 gradients land, then the BF16 weight refreshed
// ([Review] 3-2 item 6 "CPU-side optimizer update"; [Hotdry] the background
// CPU thread that unpacks gradient slabs and runs Adam).  Kingma-Ba with
// bias correction, eps after the square root, no weight decay.
AdamStep adam_step_params(const mt_options& o, int64_t t) {
    AdamStep a;
    a.lr = o.lr;
    a.b1 = o.beta1;
    a.b2 = o.beta2;
    a.omb1 = float(1.0 - double(o.beta1));
    a.omb2 = float(1.0 - double(o.beta2));
    a.eps = o.adam_eps;
    a.bc1 = float(1.0 - pow(double(o.beta1), double(t)));
    a.bc2 = float(1.0 - pow(double(o.beta2), double(t)));
    return a;
}

// 8 bf16 <-> 8 fp32, the conversions of bf16_to_f32 / f32_to_bf16 (round to
// nearest even, NaN kept quiet) lane by lane.
static inline __m256 bf16x8_to_f32(__m128i h) {
    return _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(h), 16));
}
static inline __m128i f32x8_to_bf16(__m256 x) {
    const __m256i u = _mm256_castps_si256(x);
    const __m256i lsb = _mm256_and_si256(_mm256_srli_epi32(u, 16), _mm256_set1_epi32(1));
    __m256i r = _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(u, _mm256_set1_epi32(0x7FFF)), lsb), 16);
    const __m256i is_nan =
        _mm256_cmpgt_epi32(_mm256_and_si256(u, _mm256_set1_epi32(0x7FFFFFFF)), _mm256_set1_epi32(0x7F800000));
    r = _mm256_blendv_epi8(r, _mm256_or_si256(_mm256_srli_epi32(u, 16), _mm256_set1_epi32(0x40)), is_nan);
    // every lane is in [0, 0xFFFF], so the saturating pack is exact
    const __m256i p = _mm256_permute4x64_epi64(_mm256_packus_epi32(r, r), 0x08);
    return _mm256_castsi256_si128(p);
}

// One Adam element; the vector loop below performs the same fp32 operations
// in the same order (no contraction into FMA), so results are bit-identical.
static inline void adam_one(const AdamStep& a, uint16_t gb, float& M, float& V, float& th, uint16_t& W) {
    const float g = bf16_to_f32(gb);
    const float mi = a.b1 * M + a.omb1 * g;
    const float vi = a.b2 * V + a.omb2 * (g * g);
    M = mi;
    V = vi;
    const float upd = a.lr * (mi / a.bc1) / (sqrtf(vi / a.bc2) + a.eps);
    th = th - upd;
    W = f32_to_bf16(th);
}

void adam_range(const TilePtrs& p, const uint16_t* gsrc, int64_t b, int64_t e, const AdamStep& a) {
    const bool copy_g = gsrc != p.g;
    uint16_t* __restrict__ G = p.g;
    const uint16_t* __restrict__ gs = gsrc;
    float* __restrict__ M = p.m;
    float* __restrict__ Vv = p.v;
    float* __restrict__ th = p.master;
    uint16_t* __restrict__ W = p.w;
    int64_t i = b;
    // scalar head up to 16-byte alignment of W (G shares it in practice; if
    // not, the whole range stays scalar)
    while (i < e && (reinterpret_cast<uintptr_t>(W + i) & 15)) {
        if (copy_g) G[i] = gs[i];
        adam_one(a, gs[i], M[i], Vv[i], th[i], W[i]);
        ++i;
    }
    const bool vec = !copy_g || (reinterpret_cast<uintptr_t>(G + i) & 15) == 0;
    if (vec) {
        const __m256 b1 = _mm256_set1_ps(a.b1), b2 = _mm256_set1_ps(a.b2);
        const __m256 omb1 = _mm256_set1_ps(a.omb1), omb2 = _mm256_set1_ps(a.omb2);
        const __m256 lr = _mm256_set1_ps(a.lr), bc1 = _mm256_set1_ps(a.bc1), bc2 = _mm256_set1_ps(a.bc2);
        const __m256 eps = _mm256_set1_ps(a.eps);
        for (; i + 8 <= e; i += 8) {
            const __m128i gb = _mm_loadu_si128(reinterpret_cast<const __m128i*>(gs + i));
            // G and W are not read again by this pass: streaming stores
            if (copy_g) _mm_stream_si128(reinterpret_cast<__m128i*>(G + i), gb);
            const __m256 g = bf16x8_to_f32(gb);
            const __m256 mi = _mm256_add_ps(_mm256_mul_ps(b1, _mm256_loadu_ps(M + i)), _mm256_mul_ps(omb1, g));
            const __m256 vi =
                _mm256_add_ps(_mm256_mul_ps(b2, _mm256_loadu_ps(Vv + i)), _mm256_mul_ps(omb2, _mm256_mul_ps(g, g)));
            _mm256_storeu_ps(M + i, mi);
            _mm256_storeu_ps(Vv + i, vi);
            const __m256 den = _mm256_add_ps(_mm256_sqrt_ps(_mm256_div_ps(vi, bc2)), eps);
            const __m256 upd = _mm256_div_ps(_mm256_mul_ps(lr, _mm256_div_ps(mi, bc1)), den);
            const __m256 t = _mm256_sub_ps(_mm256_loadu_ps(th + i), upd);
            _mm256_storeu_ps(th + i, t);
            _mm_stream_si128(reinterpret_cast<__m128i*>(W + i), f32x8_to_bf16(t));
        }
        _mm_sfence();
    }
    for (; i < e; ++i) {
        if (copy_g) G[i] = gs[i];
        adam_one(a, gs[i], M[i], Vv[i], th[i], W[i]);
    }
}

void adam_unit(ThreadPool& pool, const TilePtrs& p, const uint16_t* gsrc, int64_t n,
               const AdamStep& a) {
    pool.parallel_for(n, 1 << 15, [&](int64_t b, int64_t e) { adam_range(p, gsrc, b, e, a); });
}

// Gradient accumulation into the host G ([Review] 3-2 item 1: the host holds
// the accumulated gradient; [Hotdry] "三层 CUDA Stream 流水线与双缓冲调度": the
// CPU thread unpacks each slab and accumulates it into the master store).
// G <- bf16_RNE(f32(G) + f32(src)): the sum of two bf16 values is exact in
// fp32 whenever it can round differently, so this is one rounding of the
// exact sum.  The vector loop does the same operations lane by lane.
void accum_range(uint16_t* G, const uint16_t* src, int64_t b, int64_t e) {
    int64_t i = b;
    while (i < e && (reinterpret_cast<uintptr_t>(G + i) & 15)) {
        G[i] = f32_to_bf16(bf16_to_f32(G[i]) + bf16_to_f32(src[i]));
        ++i;
    }
    for (; i + 8 <= e; i += 8) {
        const __m256 a = bf16x8_to_f32(_mm_load_si128(reinterpret_cast<const __m128i*>(G + i)));
        const __m256 c = bf16x8_to_f32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(src + i)));
        _mm_store_si128(reinterpret_cast<__m128i*>(G + i), f32x8_to_bf16(_mm256_add_ps(a, c)));
    }
    for (; i < e; ++i) G[i] = f32_to_bf16(bf16_to_f32(G[i]) + bf16_to_f32(src[i]));
}

void accum_unit(ThreadPool& pool, uint16_t* G, const uint16_t* src, int64_t n) {
    pool.parallel_for(n, 1 << 15, [&](int64_t b, int64_t e) { accum_range(G, src, b, e); });
}

}  // namespace mt
