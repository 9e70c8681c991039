// Causal grouped-query flash attention for gfx950: forward (O and the
// log-sum-exp), and a deterministic backward split into a dQ kernel and a
// dK/dV kernel, neither using atomics.
//
// q and k arrive in fp16, v, dO and O in bf16.  The score products Q K^T run
// on v_mfma_f32_32x32x16_f16, every other contraction on the bf16 form; the
// fp16 q/k tiles that feed a gradient product are rounded to bf16 when staged.
// Both MFMA forms share one register layout.  The MFMA writes element
// r of lane l of a 32x32 result at row 8*(r/4) + 4*(l/32) + r%4, column l%32,
// and takes its A operand as row l%32, k = 8*(l/32)..+7 and its B operand as
// column l%32, same k.  The kernels exploit that:
//  * forward and dQ compute S^T = K Q^T, so a lane owns one query (a column)
//    and holds 16 of its scores in registers: the softmax state of a query
//    lives in one lane (plus its partner lane l^32), no LDS reductions;
//  * the probabilities then feed the next MFMA directly as its B operand,
//    with the contraction index (keys) permuted the same way in the A
//    operand, which is read from a transposed LDS image of V (or K);
//  * dK/dV compute S = Q K^T instead, so a lane owns one key and the key
//    gradients accumulate per lane over every query head of the KV group in
//    a fixed order.
// K/V (or Q/dO) tiles are staged in LDS twice-buffered: global loads of the
// next tile are issued before the MFMAs on the current one.
#include "kcommon.h"
#include "kernels.h"

namespace mt {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int BKV = 64;  // keys (or queries) per staged tile
#ifndef MT_ATTN_SPLIT
#define MT_ATTN_SPLIT 0  // 1: dK and dV of the direct-load backward in two launches
#endif

#define MFMA32(a, b, c) __builtin_amdgcn_mfma_f32_32x32x16_bf16((a), (b), (c), 0, 0, 0)
// 2^x on the hardware instruction alone: results below 2^-126 (probabilities
// that add nothing at fp32 precision) flush to zero instead of being formed
// as denormals, which costs the library form four more instructions.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
// Scores from fp16 q and k (the logit path is kept in fp16: its rounding
// error enters the softmax in proportion to the logits' size).
#define MFMA32H(a, b, c) __builtin_amdgcn_mfma_f32_32x32x16_f16((a), (b), (c), 0, 0, 0)

__device__ __forceinline__ uint32_t h2b(uint32_t h) { return f2bf(h2f(uint16_t(h))); }

// Row-major tile image [rows][HD] bf16 in 16-byte chunks, chunk index
// XOR-swizzled with the row.
template <int HD>
struct RowTile {
    static constexpr int NCH = HD / 8;
    static constexpr int SW = (NCH < 16 ? NCH : 16) - 1;
    __device__ static __forceinline__ int idx(int row, int chunk) { return row * NCH + (chunk ^ (row & SW)); }
};
// Transposed tile image [HD][64 positions] bf16 in 8-byte chunks of four
// positions, chunk index XOR-swizzled with the d row.
struct ColTile {
    __device__ static __forceinline__ int idx(int d, int chunk4) { return d * 16 + (chunk4 ^ (d & 15)); }
};

__device__ __forceinline__ uint32_t h16(const uint4& v, int e) {
    uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// A 4-position x 8-d block of a [pos x d] row-major source, kept in
// registers and written out both as rows and transposed.
struct Blk48 {
    uint4 v[4];
    __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld, int pos0,
                                         int npos, int d0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = pos0 + j;
            v[j] = p < npos ? *reinterpret_cast<const uint4*>(base + int64_t(p) * ld + d0)
                            : make_uint4(0, 0, 0, 0);
        }
    }
    template <int HD>
    __device__ __forceinline__ void store_rows(uint4* __restrict__ lds, int prow0, int dchunk) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) lds[RowTile<HD>::idx(prow0 + j, dchunk)] = v[j];
    }
    // FROM_F16: the source holds fp16; the transposed image is written as bf16
    // (it feeds a bf16 product of the gradient path).
    template <bool FROM_F16 = false>
    __device__ __forceinline__ void store_cols(uint2* __restrict__ lds, int prow0, int d0) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t x0 = h16(v[0], e), x1 = h16(v[1], e), x2 = h16(v[2], e), x3 = h16(v[3], e);
            if constexpr (FROM_F16) { x0 = h2b(x0); x1 = h2b(x1); x2 = h2b(x2); x3 = h2b(x3); }
            uint2 w;
            w.x = x0 | (x1 << 16);
            w.y = x2 | (x3 << 16);
            lds[ColTile::idx(d0 + e, prow0 >> 2)] = w;
        }
    }
};

// Read an A operand (rows = d, k = 16 positions starting at 16*s2 of the
// 32-position sub-tile t) from a transposed image, with the key permutation
// that matches the accumulator layout: k-slot j of lane half hh is position
// 4*hh + j (j < 4) or 8 + 4*hh + (j - 4).
__device__ __forceinline__ bf16x8_t read_colT(const uint2* __restrict__ lds, int d, int t, int s2, int hh) {
    const int c0 = 8 * t + 4 * s2 + hh;
    const uint2 lo = lds[ColTile::idx(d, c0)];
    const uint2 hi = lds[ColTile::idx(d, c0 + 2)];
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Pack accumulator registers 8*s2..8*s2+7 into a bf16 B operand.
__device__ __forceinline__ bf16x8_t pack_b(const float* v) {
    return as_bf16x8(make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])));
}

// ----------------------------------------------------------- forward ------
// Block: 4 waves x 32 queries of one (b, h); key tiles of 64.
template <int HD>
__global__ __launch_bounds__(256) void attn_fwd_k(AttnArgs a, int n_qt) {
    constexpr int NS = HD / 16;   // k-steps over head dim
    constexpr int ND = HD / 32;   // 32-wide d tiles
    __shared__ uint4 Ks[2][BKV * HD / 8];
    __shared__ uint2 Vt[2][HD * 16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, c = lane & 31;
    const int qt = n_qt - 1 - int(blockIdx.x % n_qt);
    const int bh = int(blockIdx.x / n_qt);
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int hk = h / (a.Hq / a.Hkv);
    const int S = a.S;
    const int q0 = qt * 128;
    const int qw = q0 + wave * 32;
    const int q = qw + c;
    const uint16_t* base = a.qkv + int64_t(b) * S * a.ld;
    const int kcol = (a.Hq + hk) * HD, vcol = (a.Hq + a.Hkv + hk) * HD;

    f16x8_t qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (q < S) v = *reinterpret_cast<const uint4*>(base + int64_t(q) * a.ld + h * HD + (2 * s + hh) * 8);
        qf[s] = as_f16x8(v);
    }

    // Tile loaders: K as rows (HD/32 chunks per thread), V as 4x8 blocks.
    constexpr int KCH = BKV * HD / 8 / 256;
    uint4 kreg[KCH];
    Blk48 vreg;
    const bool vthread = tid < 2 * HD;  // (64/4) * (HD/8) blocks
    const int vdg = tid % (HD / 8), vkg = tid / (HD / 8);
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int cc = tid + i * 256;
            const int row = cc / (HD / 8), kc = cc % (HD / 8);
            kreg[i] = (k0 + row < S) ? *reinterpret_cast<const uint4*>(base + int64_t(k0 + row) * a.ld + kcol + kc * 8)
                                     : make_uint4(0, 0, 0, 0);
        }
        if (vthread) vreg.load(base + vcol, a.ld, k0 + 4 * vkg, S, 8 * vdg);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int cc = tid + i * 256;
            const int row = cc / (HD / 8), kc = cc % (HD / 8);
            Ks[buf][RowTile<HD>::idx(row, kc)] = kreg[i];
        }
        if (vthread) vreg.store_cols(Vt[buf], 4 * vkg, 8 * vdg);
    };

    f32x16_t o[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
    float m = -INFINITY, lsum = 0.f;
    const float sc = LOG2E * rsqrtf(float(HD));

    const int k_end = min(S, q0 + 128);
    const int nkb = (k_end + BKV - 1) / BKV;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        const int cur = kb & 1;
        const int k0 = kb * BKV;
        if (kb + 1 < nkb) gload(k0 + BKV);
        if (k0 <= qw + 31) {
            f32x16_t st[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int r = 0; r < 16; ++r) st[t][r] = 0.f;
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    st[t] = MFMA32H(as_f16x8(Ks[cur][RowTile<HD>::idx(32 * t + c, 2 * s + hh)]), qf[s], st[t]);
            }
            // Raw scores; the scale goes into the exponent's FMA.  A tile
            // every query of the wave sees whole (below the diagonal, inside
            // the sequence) needs no mask.
            const bool full = k0 + BKV - 1 <= qw && k0 + BKV <= S;
            float mx = -INFINITY;
            if (full) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[t][r]);
            } else {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
                        if (key > q || key >= S) st[t][r] = -INFINITY;
                        mx = fmaxf(mx, st[t][r]);
                    }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mn = fmaxf(m, mx * sc);  // running max of the scaled scores (log2 units)
            const float alpha = (m == -INFINITY) ? 0.f : ex2(m - mn);
            m = mn;
            const float nb = (mn == -INFINITY) ? 0.f : -mn;  // masked scores give exp2(-inf) = 0
            float ps = 0.f;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = ex2(fmaf(st[t][r], sc, nb));
                    st[t][r] = p;
                    ps += p;
                }
            lsum = lsum * alpha + ps;
            // Rescale the output only when some lane's maximum moved.
            if (__ballot(alpha != 1.0f)) {
#pragma unroll
                for (int i = 0; i < ND; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
            }
            bf16x8_t pb[2][2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    float tmp[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) tmp[j] = st[t][8 * s2 + j];
                    pb[t][s2] = pack_b(tmp);
                }
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        o[dt] = MFMA32(read_colT(Vt[cur], 32 * dt + c, t, s2, hh), pb[t][s2], o[dt]);
        }
        if (kb + 1 < nkb) lstore(cur ^ 1);
        __syncthreads();
    }

    const float ltot = lsum + __shfl_xor(lsum, 32, 64);
    if (q < S) {
        const float inv = 1.0f / ltot;
        uint16_t* orow = a.o + (int64_t(b) * S + q) * a.ldo + h * HD;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hh;
                *reinterpret_cast<uint2*>(orow + d) =
                    make_uint2(pack2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                               pack2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv));
            }
        if (hh == 0) a.lse[(int64_t(b) * a.Hq + h) * S + q] = (m + log2f(ltot)) * LN2;
    }
}

// ------------------------------------------- forward, direct-load form ----
// K and V tiles go from global memory straight into LDS
// (`buffer_load_dwordx4 ... lds`: no staging registers, no LDS stores), both
// row-major with 16-byte chunks XOR-swizzled by aswz(row).  K fragments are
// read as rows; the transposed V fragments of the P.V product come from
// ds_read_b64_tr_b16, which hands lane i of a 16-lane group element i of
// the four rows the group addresses.  The swizzle serves both reads without
// bank conflicts: 16 consecutive rows of one chunk (K) and 4 rows x 4
// chunks (V^T, 32 lanes per cycle) each land on distinct banks.  No staging
// registers and a small register set let two blocks share a CU, so one
// wave's softmax runs while the other's products do.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// Buffer resource (gfx9 layout): base, stride 0, extent in bytes, the
// default data-format word.  Reads at offsets >= extent return zero.
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    i32x4_t r;
    r.x = int(uint32_t(p));
    r.y = int(uint32_t(p >> 32) & 0xFFFFu);
    r.z = int(bytes);
    r.w = 0x00020000;
    return r;
}
// 16 bytes per lane from the buffer at byte offset voff into LDS at
// lds_addr + 16 * lane (inline assembly, so the compiler adds no waits for it
// before unrelated LDS reads; the kernel waits on vmcnt itself).
__device__ __forceinline__ void dma16(i32x4_t rs, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rs)
                 : "memory");
}
__device__ __forceinline__ void wait_vmem0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Block barrier after this wave's loads landed (vmcnt) and its LDS reads
// completed (lgkmcnt through the builtin, so the compiler knows).
__device__ __forceinline__ void barrier_tile() {
    wait_vmem0();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
template <int HD>
__device__ __forceinline__ int aswz(int r) {
    if constexpr (HD == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

template <int HD>
__global__ __launch_bounds__(256, 2) void attn_fwd2_k(AttnArgs a, int n_qt) {
    constexpr int NS = HD / 16, ND = HD / 32, NCH = HD / 8;
    constexpr int TILE = BKV * NCH;  // 16-byte chunks per tile
    constexpr int NI = TILE / 256;   // wave instructions per tile and operand
    constexpr int RB = NCH * 16;     // bytes per LDS row
    __shared__ uint4 Ks[2][TILE];
    __shared__ uint4 Vs[2][TILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, c = lane & 31;
    const int qt = n_qt - 1 - int(blockIdx.x % n_qt);
    const int bh = int(blockIdx.x / n_qt);
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int hk = h / (a.Hq / a.Hkv);
    const int S = a.S;
    const int q0 = qt * 128;
    const int qw = q0 + wave * 32;
    const int q = qw + c;
    const uint16_t* base = a.qkv + int64_t(b) * S * a.ld;

    f16x8_t qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (q < S) v = *reinterpret_cast<const uint4*>(base + int64_t(q) * a.ld + h * HD + (2 * s + hh) * 8);
        qf[s] = as_f16x8(v);
    }

    // Loads: instruction i of wave w fills chunks (4 i + w) * 64 + lane of the
    // tile; the lane fetches the logical chunk the swizzle places there.
    const uint32_t ext = uint32_t((int64_t(S - 1) * a.ld + HD) * 2);
    const i32x4_t rk = make_rsrc(base + (a.Hq + hk) * HD, ext);
    const i32x4_t rv = make_rsrc(base + (a.Hq + a.Hkv + hk) * HD, ext);
    uint32_t doff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int p = (4 * i + wave) * 64 + lane;
        const int row = p / NCH;
        const int lc = (p % NCH) ^ aswz<HD>(row);
        doff[i] = uint32_t((int64_t(row) * a.ld + lc * 8) * 2);
    }
    auto issue = [&](int k0, int buf) {
        const uint32_t kof = uint32_t(int64_t(k0) * a.ld * 2);
        const uint32_t kl = lds_addr(&Ks[buf][0]), vl = lds_addr(&Vs[buf][0]);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t la = uint32_t((4 * i + wave) * 1024);
            dma16(rk, __builtin_amdgcn_readfirstlane(kl + la), doff[i] + kof);
            dma16(rv, __builtin_amdgcn_readfirstlane(vl + la), doff[i] + kof);
        }
    };
    // K fragment (row 32 t + c, logical chunk 2 s + hh): byte offset in a tile.
    auto koff = [&](int t, int s) { return (32 * t + c) * RB + (((2 * s + hh) ^ aswz<HD>(32 * t + c)) * 16); };
    // V^T fragment for d-tile dt, keys 32 t + 16 s2 + 4 hh + 8 e2 .. +3: the
    // lane addresses row (j / 4) of its group's four rows, 8 bytes at column
    // dbase + 4 (j % 4); lane i then holds column dbase + i of the four rows.
    const int j = lane & 15, g16 = (lane >> 4) & 1;
    auto voff = [&](int dt, int t, int s2, int e2) {
        const int row = 32 * t + 16 * s2 + 8 * e2 + 4 * hh + (j >> 2);
        const int col = 32 * dt + 16 * g16 + 4 * (j & 3);
        return row * RB + (((col >> 3) ^ aswz<HD>(row)) * 16) + (col & 7) * 2;
    };

    f32x16_t o[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
    float m = -INFINITY, lsum = 0.f;
    const float sc = LOG2E * rsqrtf(float(HD));

    const int k_end = min(S, q0 + 128);
    const int nkb = (k_end + BKV - 1) / BKV;
    issue(0, 0);
    barrier_tile();
    for (int kb = 0; kb < nkb; ++kb) {
        const int cur = kb & 1;
        const int k0 = kb * BKV;
        if (kb + 1 < nkb) issue(k0 + BKV, cur ^ 1);
        if (k0 <= qw + 31) {
            const char* kt = reinterpret_cast<const char*>(&Ks[cur][0]);
            const char* vt = reinterpret_cast<const char*>(&Vs[cur][0]);
            f32x16_t st[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int r = 0; r < 16; ++r) st[t][r] = 0.f;
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    st[t] = MFMA32H(as_f16x8(*reinterpret_cast<const uint4*>(kt + koff(t, s))), qf[s], st[t]);
            }
            const bool full = k0 + BKV - 1 <= qw && k0 + BKV <= S;
            float mx = -INFINITY;
            if (full) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[t][r]);
            } else {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
                        if (key > q || key >= S) st[t][r] = -INFINITY;
                        mx = fmaxf(mx, st[t][r]);
                    }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mn = fmaxf(m, mx * sc);
            const float alpha = (m == -INFINITY) ? 0.f : ex2(m - mn);
            m = mn;
            const float nb = (mn == -INFINITY) ? 0.f : -mn;
            float ps = 0.f;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = ex2(fmaf(st[t][r], sc, nb));
                    st[t][r] = p;
                    ps += p;
                }
            lsum = lsum * alpha + ps;
            if (__ballot(alpha != 1.0f)) {
#pragma unroll
                for (int i = 0; i < ND; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
            }
            bf16x8_t pb[2][2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    float tmp[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) tmp[e] = st[t][8 * s2 + e];
                    pb[t][s2] = pack_b(tmp);
                }
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4_t*)(lds_ptr_t)(vt + voff(dt, t, s2, 0)));
                        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4_t*)(lds_ptr_t)(vt + voff(dt, t, s2, 1)));
                        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
                        o[dt] = MFMA32(as_bf16x8(make_uint4(l2.x, l2.y, h2.x, h2.y)), pb[t][s2], o[dt]);
                    }
        }
        barrier_tile();
    }

    const float ltot = lsum + __shfl_xor(lsum, 32, 64);
    if (q < S) {
        const float inv = 1.0f / ltot;
        uint16_t* orow = a.o + (int64_t(b) * S + q) * a.ldo + h * HD;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hh;
                *reinterpret_cast<uint2*>(orow + d) =
                    make_uint2(pack2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                               pack2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv));
            }
        if (hh == 0) a.lse[(int64_t(b) * a.Hq + h) * S + q] = (m + log2f(ltot)) * LN2;
    }
}

// ------------------------------------- backward, direct-load forms -----
// Offsets of the DMA chunks of a 64-row tile: instruction i of wave w fills
// tile chunks (4 i + w) * 64 + lane with the logical chunk the swizzle puts
// there, from rows that are ld elements apart.
template <int HD, int NI>
__device__ __forceinline__ void tile_offsets(uint32_t (&off)[NI], int wave, int lane, int64_t ld) {
    constexpr int NCH = HD / 8;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int p = (4 * i + wave) * 64 + lane;
        const int row = p / NCH;
        const int lc = (p % NCH) ^ aswz<HD>(row);
        off[i] = uint32_t((int64_t(row) * ld + lc * 8) * 2);
    }
}
template <int NI>
__device__ __forceinline__ void tile_issue(i32x4_t rs, const uint32_t (&off)[NI], uint32_t rowoff, uint32_t lds,
                                           int wave) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
        dma16(rs, __builtin_amdgcn_readfirstlane(lds + uint32_t((4 * i + wave) * 1024)), off[i] + rowoff);
}
// Row fragment (row, logical chunk) of a swizzled tile.
template <int HD>
__device__ __forceinline__ uint4 tile_row(const uint4* t, int row, int ch) {
    return t[row * (HD / 8) + (ch ^ aswz<HD>(row))];
}
// Transposed fragment: 8 elements of column (32 dt + lane % 32), rows
// 32 t + 16 s2 + 4 hh + {0..3} and + 8 + {0..3}, the key/query permutation of
// the accumulator layout (the lane addresses one 8-byte piece of its group's
// four rows; ds_read_b64_tr_b16 hands lane i column i of them).
template <int HD>
__device__ __forceinline__ bf16x8_t tile_colT(const uint4* t, int dt, int tt, int s2, int lane) {
    constexpr int RB = HD / 8 * 16;
    const int j = lane & 15, g16 = (lane >> 4) & 1, hh = lane >> 5;
    const int col = 32 * dt + 16 * g16 + 4 * (j & 3);
    const char* base = reinterpret_cast<const char*>(t);
    uint2 r[2];
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
        const int row = 32 * tt + 16 * s2 + 8 * e2 + 4 * hh + (j >> 2);
        const int off = row * RB + (((col >> 3) ^ aswz<HD>(row)) * 16) + (col & 7) * 2;
        const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(lds_ptr_t)(base + off));
        r[e2] = __builtin_bit_cast(uint2, v);
    }
    return as_bf16x8(make_uint4(r[0].x, r[0].y, r[1].x, r[1].y));
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <int I, int N, class F>
__device__ __forceinline__ void static_for_from(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_from<I + 1, N>(f);
    }
}
template <int N, class F>
__device__ __forceinline__ void static_for_n(F&& f) { static_for_from<0, N>(f); }

// dQ: block = 4 waves x 32 queries of one (b, h); key tiles of 64 staged as
// fp16 K rows (scores), bf16 K (read transposed for dQ) and bf16 V rows.
template <int HD>
__global__ __launch_bounds__(256) void attn_dq2_k(AttnBwdArgs a, int n_qt) {
    constexpr int NS = HD / 16, ND = HD / 32, NCH = HD / 8;
    constexpr int TILE = BKV * NCH, NI = TILE / 256;
    __shared__ uint4 Kh[2][TILE];
    __shared__ uint4 Kb[2][TILE];
    __shared__ uint4 Vs[2][TILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, c = lane & 31;
    const int qt = n_qt - 1 - int(blockIdx.x % n_qt);
    const int bh = int(blockIdx.x / n_qt);
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int hk = h / (a.Hq / a.Hkv);
    const int S = a.S;
    const int q0 = qt * 128, qw = q0 + wave * 32, q = qw + c;
    const uint16_t* base = a.qkv + int64_t(b) * S * a.ld;
    const uint16_t* bbase = a.qkb + int64_t(b) * S * a.ldb;
    const uint16_t* dbase = a.dout + int64_t(b) * S * a.ldo;

    f16x8_t qf[NS];
    bf16x8_t dof[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0), w = v;
        if (q < S) {
            v = *reinterpret_cast<const uint4*>(base + int64_t(q) * a.ld + h * HD + (2 * s + hh) * 8);
            w = *reinterpret_cast<const uint4*>(dbase + int64_t(q) * a.ldo + h * HD + (2 * s + hh) * 8);
        }
        qf[s] = as_f16x8(v);
        dof[s] = as_bf16x8(w);
    }
    const int64_t st_off = (int64_t(b) * a.Hq + h) * S;
    const float lse2 = q < S ? a.lse[st_off + q] * LOG2E : 0.f;
    const float dq_d = q < S ? a.dsum[st_off + q] : 0.f;

    const i32x4_t rkh = make_rsrc(base + (a.Hq + hk) * HD, uint32_t((int64_t(S - 1) * a.ld + HD) * 2));
    const i32x4_t rv = make_rsrc(base + (a.Hq + a.Hkv + hk) * HD, uint32_t((int64_t(S - 1) * a.ld + HD) * 2));
    const i32x4_t rkb = make_rsrc(bbase + (a.Hq + hk) * HD, uint32_t((int64_t(S - 1) * a.ldb + HD) * 2));
    uint32_t offa[NI], offb[NI];
    tile_offsets<HD>(offa, wave, lane, a.ld);
    tile_offsets<HD>(offb, wave, lane, a.ldb);
    auto issue = [&](int k0, int buf) {
        tile_issue(rkh, offa, uint32_t(int64_t(k0) * a.ld * 2), lds_addr(&Kh[buf][0]), wave);
        tile_issue(rv, offa, uint32_t(int64_t(k0) * a.ld * 2), lds_addr(&Vs[buf][0]), wave);
        tile_issue(rkb, offb, uint32_t(int64_t(k0) * a.ldb * 2), lds_addr(&Kb[buf][0]), wave);
    };

    f32x16_t acc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    const float sc = LOG2E * rsqrtf(float(HD));

    const int k_end = min(S, q0 + 128);
    const int nkb = (k_end + BKV - 1) / BKV;
    issue(0, 0);
    barrier_tile();
    for (int kb = 0; kb < nkb; ++kb) {
        const int cur = kb & 1;
        const int k0 = kb * BKV;
        if (kb + 1 < nkb) issue(k0 + BKV, cur ^ 1);
        if (k0 <= qw + 31) {
            f32x16_t st[2], dp[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) { st[t][r] = 0.f; dp[t][r] = 0.f; }
            // k-step s+1's fragments are read while step s multiplies
            uint4 fk[2][2], fv[2][2];
            auto rd = [&](int s, uint4(&k)[2], uint4(&v)[2]) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    k[t] = tile_row<HD>(Kh[cur], 32 * t + c, 2 * s + hh);
                    v[t] = tile_row<HD>(Vs[cur], 32 * t + c, 2 * s + hh);
                }
            };
            rd(0, fk[0], fv[0]);
            static_for_n<NS>([&](auto s_) {
                constexpr int s = decltype(s_)::value;
                if constexpr (s + 1 < NS) rd(s + 1, fk[(s + 1) & 1], fv[(s + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    st[t] = MFMA32H(as_f16x8(fk[s & 1][t]), qf[s], st[t]);
                    dp[t] = MFMA32(as_bf16x8(fv[s & 1][t]), dof[s], dp[t]);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            bf16x8_t dsb[2][2];
            const bool full = k0 + BKV - 1 <= qw && k0 + BKV <= S;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    float tmp[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int r = 8 * s2 + j;
                        float p = ex2(fmaf(st[t][r], sc, -lse2));
                        if (!full) {
                            const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
                            if (key > q || key >= S) p = 0.f;
                        }
                        tmp[j] = p * (dp[t][r] - dq_d);
                    }
                    dsb[t][s2] = pack_b(tmp);
                }
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        acc[dt] = MFMA32(tile_colT<HD>(Kb[cur], dt, t, s2, lane), dsb[t][s2], acc[dt]);
        }
        barrier_tile();
    }
    if (q < S) {
        const float scale = rsqrtf(float(HD));
        uint16_t* row = a.dqkv + (int64_t(b) * S + q) * a.ldd + h * HD;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hh;
                *reinterpret_cast<uint2*>(row + d) =
                    make_uint2(pack2(acc[dt][4 * g] * scale, acc[dt][4 * g + 1] * scale),
                               pack2(acc[dt][4 * g + 2] * scale, acc[dt][4 * g + 3] * scale));
            }
    }
}

// dK, dV: block = 4 waves x 32 keys of one (b, kv head); query tiles of 64
// over the group's heads, staged as fp16 Q rows (scores), bf16 Q (read
// transposed for dK) and bf16 dO (rows for dP, transposed for dV).  MODE 0
// computes both; MODE 1 dK only and MODE 2 dV only (P and dO, no dP), for a
// split into two launches with fewer registers each.
template <int HD, int MODE>
__global__ __launch_bounds__(256, MODE == 2 ? 2 : 1) void attn_dkdv2_k(AttnBwdArgs a, int n_kt) {
    constexpr bool WK = MODE != 2, WV = MODE != 1;  // dK, dV wanted
    constexpr int NS = HD / 16, ND = HD / 32, NCH = HD / 8;
    constexpr int TILE = BKV * NCH, NI = TILE / 256;
    __shared__ uint4 Qh[2][TILE];
    __shared__ uint4 Qb[WK ? 2 : 1][WK ? TILE : 1];
    __shared__ uint4 Ds[2][TILE];
    __shared__ __align__(16) float Ls[2][BKV];
    __shared__ __align__(16) float Dd[2][BKV];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, c = lane & 31;
    const int kt = int(blockIdx.x % n_kt);
    const int bk = int(blockIdx.x / n_kt);
    const int hk = bk % a.Hkv, b = bk / a.Hkv;
    const int G = a.Hq / a.Hkv;
    const int S = a.S;
    const int k0 = kt * 128, kw = k0 + wave * 32, key = kw + c;
    const uint16_t* base = a.qkv + int64_t(b) * S * a.ld;
    const uint16_t* bbase = a.qkb + int64_t(b) * S * a.ldb;
    const uint16_t* dbase = a.dout + int64_t(b) * S * a.ldo;
    const int kcol = (a.Hq + hk) * HD, vcol = (a.Hq + a.Hkv + hk) * HD;

    f16x8_t kf[NS];
    bf16x8_t vf[WK ? NS : 1];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (key < S) v = *reinterpret_cast<const uint4*>(base + int64_t(key) * a.ld + kcol + (2 * s + hh) * 8);
        kf[s] = as_f16x8(v);
        if constexpr (WK) {
            uint4 w = make_uint4(0, 0, 0, 0);
            if (key < S) w = *reinterpret_cast<const uint4*>(base + int64_t(key) * a.ld + vcol + (2 * s + hh) * 8);
            vf[s] = as_bf16x8(w);
        }
    }

    uint32_t offa[NI], offb[NI], offd[NI];
    tile_offsets<HD>(offa, wave, lane, a.ld);
    if constexpr (WK) tile_offsets<HD>(offb, wave, lane, a.ldb);
    tile_offsets<HD>(offd, wave, lane, a.ldo);
    const uint32_t exa = uint32_t((int64_t(S - 1) * a.ld + HD) * 2);
    const uint32_t exb = uint32_t((int64_t(S - 1) * a.ldb + HD) * 2);
    const uint32_t exd = uint32_t((int64_t(S - 1) * a.ldo + HD) * 2);
    float lreg = 0.f, dreg = 0.f;
    auto issue = [&](int hq, int q0, int buf) {
        tile_issue(make_rsrc(base + hq * HD, exa), offa, uint32_t(int64_t(q0) * a.ld * 2), lds_addr(&Qh[buf][0]),
                   wave);
        if constexpr (WK)
            tile_issue(make_rsrc(bbase + hq * HD, exb), offb, uint32_t(int64_t(q0) * a.ldb * 2),
                       lds_addr(&Qb[buf][0]), wave);
        tile_issue(make_rsrc(dbase + hq * HD, exd), offd, uint32_t(int64_t(q0) * a.ldo * 2),
                   lds_addr(&Ds[buf][0]), wave);
        if (tid < BKV) {
            const int64_t off = (int64_t(b) * a.Hq + hq) * S;
            const int qq = q0 + tid;
            lreg = qq < S ? a.lse[off + qq] * LOG2E : 0.f;
            if constexpr (WK) dreg = qq < S ? a.dsum[off + qq] : 0.f;
        }
    };

    f32x16_t dk[ND], dv[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dk[i][r] = 0.f; dv[i][r] = 0.f; }
    const float sc = LOG2E * rsqrtf(float(HD));

    const int qb0 = k0 / BKV;
    const int nqb = (S + BKV - 1) / BKV - qb0;  // per head
    const int total = nqb * G;
    if (total > 0) {
        issue(hk * G, qb0 * BKV, 0);
        if (tid < BKV) {
            Ls[0][tid] = lreg;
            Dd[0][tid] = dreg;
        }
    }
    barrier_tile();
    for (int it = 0; it < total; ++it) {
        const int cur = it & 1;
        const int q0 = (qb0 + it % nqb) * BKV;
        if (it + 1 < total) issue(hk * G + (it + 1) / nqb, (qb0 + (it + 1) % nqb) * BKV, cur ^ 1);
        {  // every wave computes; a tile wholly before its keys is masked to zero
            
            f32x16_t st[2], dp[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) { st[t][r] = 0.f; dp[t][r] = 0.f; }
            // S^T and dP^T over the head dimension in k-steps of 16: the
            // fragments of step s+1 are read while step s multiplies (left to
            // itself the compiler waits for each fragment right before its
            // MFMA), and the four accumulations of a step are independent.
            uint4 fq[2][2], fd[2][2];
            auto rd = [&](int s, uint4(&q)[2], uint4(&d)[2]) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    q[t] = tile_row<HD>(Qh[cur], 32 * t + c, 2 * s + hh);
                    if constexpr (WK) d[t] = tile_row<HD>(Ds[cur], 32 * t + c, 2 * s + hh);
                }
            };
            rd(0, fq[0], fd[0]);
            static_for_n<NS>([&](auto s_) {
                constexpr int s = decltype(s_)::value;
                if constexpr (s + 1 < NS) rd(s + 1, fq[(s + 1) & 1], fd[(s + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    st[t] = MFMA32H(as_f16x8(fq[s & 1][t]), kf[s], st[t]);
                    if constexpr (WK) dp[t] = MFMA32(as_bf16x8(fd[s & 1][t]), vf[s], dp[t]);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            bf16x8_t pb[2][2], dsb[2][2];
            const bool full = kw + 31 <= q0 && q0 + BKV <= S && kw + 32 <= S;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    float tp[8], td[8];
#pragma unroll
                    for (int g4 = 0; g4 < 2; ++g4) {
                        // four consecutive queries' statistics in one 16-byte read each
                        const int qb = 32 * t + 8 * (2 * s2 + g4) + 4 * hh;
                        float lv[4], dv4[4];
                        *reinterpret_cast<float4*>(lv) = *reinterpret_cast<const float4*>(&Ls[cur][qb]);
                        if constexpr (WK) *reinterpret_cast<float4*>(dv4) = *reinterpret_cast<const float4*>(&Dd[cur][qb]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int j = 4 * g4 + e, r = 8 * s2 + j;
                            float p = ex2(fmaf(st[t][r], sc, -lv[e]));
                            if (!full) {
                                const int qq = q0 + qb + e;
                                if (key > qq || qq >= S || key >= S) p = 0.f;
                            }
                            tp[j] = p;
                            if constexpr (WK) td[j] = p * (dp[t][r] - dv4[e]);
                        }
                    }
                    if constexpr (WV) pb[t][s2] = pack_b(tp);
                    if constexpr (WK) dsb[t][s2] = pack_b(td);
                }
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        if constexpr (WV) dv[dt] = MFMA32(tile_colT<HD>(Ds[cur], dt, t, s2, lane), pb[t][s2], dv[dt]);
                        if constexpr (WK)
                            dk[dt] = MFMA32(tile_colT<HD>(Qb[cur], dt, t, s2, lane), dsb[t][s2], dk[dt]);
                    }
        }
        if (it + 1 < total && tid < BKV) {
            Ls[cur ^ 1][tid] = lreg;
            Dd[cur ^ 1][tid] = dreg;
        }
        barrier_tile();
    }
    if (key < S) {
        const float scale = rsqrtf(float(HD));
        uint16_t* row = a.dqkv + (int64_t(b) * S + key) * a.ldd;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hh;
                if constexpr (WK)
                    *reinterpret_cast<uint2*>(row + kcol + d) =
                        make_uint2(pack2(dk[dt][4 * g] * scale, dk[dt][4 * g + 1] * scale),
                                   pack2(dk[dt][4 * g + 2] * scale, dk[dt][4 * g + 3] * scale));
                if constexpr (WV)
                    *reinterpret_cast<uint2*>(row + vcol + d) =
                    make_uint2(pack2(dv[dt][4 * g], dv[dt][4 * g + 1]), pack2(dv[dt][4 * g + 2], dv[dt][4 * g + 3]));
            }
    }
}

// ------------------------------------------------- D = rowsum(dO * O) -----
template <int HD>
__global__ void attn_dsum_k(AttnBwdArgs a) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t T = int64_t(a.B) * a.S;
    if (i >= T * a.Hq) return;
    const int h = int(i % a.Hq);
    const int64_t t = i / a.Hq;
    const uint4* o = reinterpret_cast<const uint4*>(a.o + t * a.ldo + h * HD);
    const uint4* g = reinterpret_cast<const uint4*>(a.dout + t * a.ldo + h * HD);
    float s = 0.f;
#pragma unroll 4
    for (int j = 0; j < HD / 8; ++j) {
        float x[8], y[8];
        unpack8(o[j], x);
        unpack8(g[j], y);
#pragma unroll
        for (int k = 0; k < 8; ++k) s += x[k] * y[k];
    }
    const int b = int(t / a.S), sq = int(t % a.S);
    a.dsum[(int64_t(b) * a.Hq + h) * a.S + sq] = s;
}

// --------------------------------------------------------------- dQ -------
template <int HD>
__global__ __launch_bounds__(256) void attn_dq_k(AttnBwdArgs a, int n_qt) {
    constexpr int NS = HD / 16, ND = HD / 32;
    __shared__ uint4 Ks[2][BKV * HD / 8];
    __shared__ uint4 Vs[2][BKV * HD / 8];
    __shared__ uint2 Kt[2][HD * 16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, c = lane & 31;
    const int qt = n_qt - 1 - int(blockIdx.x % n_qt);
    const int bh = int(blockIdx.x / n_qt);
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int hk = h / (a.Hq / a.Hkv);
    const int S = a.S;
    const int q0 = qt * 128, qw = q0 + wave * 32, q = qw + c;
    const uint16_t* base = a.qkv + int64_t(b) * S * a.ld;
    const uint16_t* dbase = a.dout + int64_t(b) * S * a.ldo;
    const int kcol = (a.Hq + hk) * HD, vcol = (a.Hq + a.Hkv + hk) * HD;

    f16x8_t qf[NS];
    bf16x8_t dof[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0), w = v;
        if (q < S) {
            v = *reinterpret_cast<const uint4*>(base + int64_t(q) * a.ld + h * HD + (2 * s + hh) * 8);
            w = *reinterpret_cast<const uint4*>(dbase + int64_t(q) * a.ldo + h * HD + (2 * s + hh) * 8);
        }
        qf[s] = as_f16x8(v);
        dof[s] = as_bf16x8(w);
    }
    const int64_t st_off = (int64_t(b) * a.Hq + h) * S;
    const float lse2 = q < S ? a.lse[st_off + q] * LOG2E : 0.f;
    const float dq_d = q < S ? a.dsum[st_off + q] : 0.f;

    // K blocks feed both the row image (scores) and the transposed image (dQ).
    const int dg = tid % (HD / 8), kg = tid / (HD / 8);
    const bool bthread = tid < 2 * HD;
    Blk48 kreg, vreg;
    auto gload = [&](int k0) {
        if (bthread) {
            kreg.load(base + kcol, a.ld, k0 + 4 * kg, S, 8 * dg);
            vreg.load(base + vcol, a.ld, k0 + 4 * kg, S, 8 * dg);
        }
    };
    auto lstore = [&](int buf) {
        if (bthread) {
            kreg.store_rows<HD>(Ks[buf], 4 * kg, dg);
            kreg.store_cols<true>(Kt[buf], 4 * kg, 8 * dg);
            vreg.store_rows<HD>(Vs[buf], 4 * kg, dg);
        }
    };

    f32x16_t acc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    const float sc = LOG2E * rsqrtf(float(HD));

    const int k_end = min(S, q0 + 128);
    const int nkb = (k_end + BKV - 1) / BKV;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        const int cur = kb & 1;
        const int k0 = kb * BKV;
        if (kb + 1 < nkb) gload(k0 + BKV);
        if (k0 <= qw + 31) {
            f32x16_t st[2], dp[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int r = 0; r < 16; ++r) { st[t][r] = 0.f; dp[t][r] = 0.f; }
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    st[t] = MFMA32H(as_f16x8(Ks[cur][RowTile<HD>::idx(32 * t + c, 2 * s + hh)]), qf[s], st[t]);
                    dp[t] = MFMA32(as_bf16x8(Vs[cur][RowTile<HD>::idx(32 * t + c, 2 * s + hh)]), dof[s], dp[t]);
                }
            }
            bf16x8_t dsb[2][2];
            // a tile every query of the wave sees whole needs no mask
            const bool full = k0 + BKV - 1 <= qw && k0 + BKV <= S;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    float tmp[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int r = 8 * s2 + j;
                        float p = ex2(fmaf(st[t][r], sc, -lse2));
                        if (!full) {
                            const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
                            if (key > q || key >= S) p = 0.f;
                        }
                        tmp[j] = p * (dp[t][r] - dq_d);
                    }
                    dsb[t][s2] = pack_b(tmp);
                }
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        acc[dt] = MFMA32(read_colT(Kt[cur], 32 * dt + c, t, s2, hh), dsb[t][s2], acc[dt]);
        }
        if (kb + 1 < nkb) lstore(cur ^ 1);
        __syncthreads();
    }
    if (q < S) {
        const float scale = rsqrtf(float(HD));
        uint16_t* row = a.dqkv + (int64_t(b) * S + q) * a.ldd + h * HD;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hh;
                *reinterpret_cast<uint2*>(row + d) =
                    make_uint2(pack2(acc[dt][4 * g] * scale, acc[dt][4 * g + 1] * scale),
                               pack2(acc[dt][4 * g + 2] * scale, acc[dt][4 * g + 3] * scale));
            }
    }
}

// ------------------------------------------------------------ dK, dV ------
// Block: 4 waves x 32 keys of one (b, kv head); loops over the query heads
// of the group and over 64-query tiles from the diagonal on.
template <int HD>
__global__ __launch_bounds__(256) void attn_dkdv_k(AttnBwdArgs a, int n_kt) {
    constexpr int NS = HD / 16, ND = HD / 32;
    __shared__ uint4 Qs[2][BKV * HD / 8];
    __shared__ uint4 Ds[2][BKV * HD / 8];
    __shared__ uint2 Qt[2][HD * 16];
    __shared__ uint2 Dt[2][HD * 16];
    __shared__ float Ls[2][BKV], Dd[2][BKV];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, c = lane & 31;
    const int kt = int(blockIdx.x % n_kt);
    const int bk = int(blockIdx.x / n_kt);
    const int hk = bk % a.Hkv, b = bk / a.Hkv;
    const int G = a.Hq / a.Hkv;
    const int S = a.S;
    const int k0 = kt * 128, kw = k0 + wave * 32, key = kw + c;
    const uint16_t* base = a.qkv + int64_t(b) * S * a.ld;
    const uint16_t* dbase = a.dout + int64_t(b) * S * a.ldo;
    const int kcol = (a.Hq + hk) * HD, vcol = (a.Hq + a.Hkv + hk) * HD;

    f16x8_t kf[NS];
    bf16x8_t vf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0), w = v;
        if (key < S) {
            v = *reinterpret_cast<const uint4*>(base + int64_t(key) * a.ld + kcol + (2 * s + hh) * 8);
            w = *reinterpret_cast<const uint4*>(base + int64_t(key) * a.ld + vcol + (2 * s + hh) * 8);
        }
        kf[s] = as_f16x8(v);
        vf[s] = as_bf16x8(w);
    }

    const int dg = tid % (HD / 8), qg = tid / (HD / 8);
    const bool bthread = tid < 2 * HD;
    Blk48 qreg, dreg;
    float lreg = 0.f, dreg_s = 0.f;
    auto gload = [&](int h, int q0) {
        if (bthread) {
            qreg.load(base + h * HD, a.ld, q0 + 4 * qg, S, 8 * dg);
            dreg.load(dbase + h * HD, a.ldo, q0 + 4 * qg, S, 8 * dg);
        }
        if (tid < BKV) {
            const int64_t off = (int64_t(b) * a.Hq + h) * S;
            const int qq = q0 + tid;
            lreg = qq < S ? a.lse[off + qq] * LOG2E : 0.f;
            dreg_s = qq < S ? a.dsum[off + qq] : 0.f;
        }
    };
    auto lstore = [&](int buf) {
        if (bthread) {
            qreg.store_rows<HD>(Qs[buf], 4 * qg, dg);
            qreg.store_cols<true>(Qt[buf], 4 * qg, 8 * dg);
            dreg.store_rows<HD>(Ds[buf], 4 * qg, dg);
            dreg.store_cols(Dt[buf], 4 * qg, 8 * dg);
        }
        if (tid < BKV) {
            Ls[buf][tid] = lreg;
            Dd[buf][tid] = dreg_s;
        }
    };

    f32x16_t dk[ND], dv[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dk[i][r] = 0.f; dv[i][r] = 0.f; }
    const float sc = LOG2E * rsqrtf(float(HD));

    const int qb0 = k0 / BKV;
    const int nqb = (S + BKV - 1) / BKV - qb0;  // per head
    const int total = nqb * G;
    if (total > 0) {
        gload(hk * G, qb0 * BKV);
        lstore(0);
    }
    __syncthreads();
    for (int it = 0; it < total; ++it) {
        const int cur = it & 1;
        const int q0 = (qb0 + it % nqb) * BKV;
        if (it + 1 < total) gload(hk * G + (it + 1) / nqb, (qb0 + (it + 1) % nqb) * BKV);
        if (kw <= q0 + BKV - 1) {
            f32x16_t st[2], dp[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int r = 0; r < 16; ++r) { st[t][r] = 0.f; dp[t][r] = 0.f; }
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    st[t] = MFMA32H(as_f16x8(Qs[cur][RowTile<HD>::idx(32 * t + c, 2 * s + hh)]), kf[s], st[t]);
                    dp[t] = MFMA32(as_bf16x8(Ds[cur][RowTile<HD>::idx(32 * t + c, 2 * s + hh)]), vf[s], dp[t]);
                }
            }
            bf16x8_t pb[2][2], dsb[2][2];
            // every key of the wave before every query of the tile, all inside
            // the sequence: no mask
            const bool full = kw + 31 <= q0 && q0 + BKV <= S && kw + 32 <= S;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    float tp[8], td[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int r = 8 * s2 + j;
                        const int ql = 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
                        float p = ex2(fmaf(st[t][r], sc, -Ls[cur][ql]));
                        if (!full) {
                            const int qq = q0 + ql;
                            if (key > qq || qq >= S || key >= S) p = 0.f;
                        }
                        tp[j] = p;
                        td[j] = p * (dp[t][r] - Dd[cur][ql]);
                    }
                    pb[t][s2] = pack_b(tp);
                    dsb[t][s2] = pack_b(td);
                }
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        dv[dt] = MFMA32(read_colT(Dt[cur], 32 * dt + c, t, s2, hh), pb[t][s2], dv[dt]);
                        dk[dt] = MFMA32(read_colT(Qt[cur], 32 * dt + c, t, s2, hh), dsb[t][s2], dk[dt]);
                    }
        }
        if (it + 1 < total) lstore(cur ^ 1);
        __syncthreads();
    }
    if (key < S) {
        const float scale = rsqrtf(float(HD));
        uint16_t* row = a.dqkv + (int64_t(b) * S + key) * a.ldd;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hh;
                *reinterpret_cast<uint2*>(row + kcol + d) =
                    make_uint2(pack2(dk[dt][4 * g] * scale, dk[dt][4 * g + 1] * scale),
                               pack2(dk[dt][4 * g + 2] * scale, dk[dt][4 * g + 3] * scale));
                *reinterpret_cast<uint2*>(row + vcol + d) =
                    make_uint2(pack2(dv[dt][4 * g], dv[dt][4 * g + 1]),
                               pack2(dv[dt][4 * g + 2], dv[dt][4 * g + 3]));
            }
    }
}

bool attn_shape_ok(int B, int S, int Hq, int Hkv, int hd, int64_t ld, int64_t ldo) {
    if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return false;
    if (hd != 64 && hd != 128) return false;
    if ((ld & 7) || (ldo & 7)) return false;
    if (ld < int64_t(Hq + 2 * Hkv) * hd || ldo < int64_t(Hq) * hd) return false;
    return true;
}

}  // namespace

hipError_t attn_fwd(const AttnArgs& a, hipStream_t s) {
    if (!attn_shape_ok(a.B, a.S, a.Hq, a.Hkv, a.hd, a.ld, a.ldo)) return hipErrorInvalidValue;
    const int n_qt = (a.S + 127) / 128;
    const dim3 grid(unsigned(int64_t(n_qt) * a.B * a.Hq));
    // The direct-load kernel addresses one sequence's K (or V) rows through a
    // 32-bit buffer extent.
    const bool direct = int64_t(a.S) * a.ld * 2 < (int64_t(1) << 32);
    if (direct) {
        if (a.hd == 128) attn_fwd2_k<128><<<grid, 256, 0, s>>>(a, n_qt);
        else attn_fwd2_k<64><<<grid, 256, 0, s>>>(a, n_qt);
    } else {
        if (a.hd == 128) attn_fwd_k<128><<<grid, 256, 0, s>>>(a, n_qt);
        else attn_fwd_k<64><<<grid, 256, 0, s>>>(a, n_qt);
    }
    return hipGetLastError();
}

hipError_t attn_bwd(const AttnBwdArgs& a, hipStream_t s) {
    if (!attn_shape_ok(a.B, a.S, a.Hq, a.Hkv, a.hd, a.ld, a.ldo)) return hipErrorInvalidValue;
    if (a.ldd < int64_t(a.Hq + 2 * a.Hkv) * a.hd || (a.ldd & 7)) return hipErrorInvalidValue;
    const int64_t rows = int64_t(a.B) * a.S * a.Hq;
    const unsigned nb = unsigned((rows + 255) / 256);
    const int n_qt = (a.S + 127) / 128;
    const int n_kt = (a.S + 127) / 128;
    const dim3 gq(unsigned(int64_t(n_qt) * a.B * a.Hq));
    const dim3 gk(unsigned(int64_t(n_kt) * a.B * a.Hkv));
    const int64_t lim = int64_t(1) << 32;  // 32-bit buffer extents of one sequence's rows
    const bool direct = a.qkb && a.ldb >= int64_t(a.Hq + a.Hkv) * a.hd && (a.ldb & 7) == 0 &&
                        int64_t(a.S) * a.ld * 2 < lim && int64_t(a.S) * a.ldb * 2 < lim &&
                        int64_t(a.S) * a.ldo * 2 < lim;
    if (direct) {
        if (a.hd == 128) {
            attn_dsum_k<128><<<nb, 256, 0, s>>>(a);
            attn_dq2_k<128><<<gq, 256, 0, s>>>(a, n_qt);
            if (MT_ATTN_SPLIT) {
                attn_dkdv2_k<128, 1><<<gk, 256, 0, s>>>(a, n_kt);
                attn_dkdv2_k<128, 2><<<gk, 256, 0, s>>>(a, n_kt);
            } else {
                attn_dkdv2_k<128, 0><<<gk, 256, 0, s>>>(a, n_kt);
            }
        } else {
            attn_dsum_k<64><<<nb, 256, 0, s>>>(a);
            attn_dq2_k<64><<<gq, 256, 0, s>>>(a, n_qt);
            attn_dkdv2_k<64, 0><<<gk, 256, 0, s>>>(a, n_kt);
        }
        return hipGetLastError();
    }
    if (a.hd == 128) {
        attn_dsum_k<128><<<nb, 256, 0, s>>>(a);
        attn_dq_k<128><<<gq, 256, 0, s>>>(a, n_qt);
        attn_dkdv_k<128><<<gk, 256, 0, s>>>(a, n_kt);
    } else {
        attn_dsum_k<64><<<nb, 256, 0, s>>>(a);
        attn_dq_k<64><<<gq, 256, 0, s>>>(a, n_qt);
        attn_dkdv_k<64><<<gk, 256, 0, s>>>(a, n_kt);
    }
    return hipGetLastError();
}

}  // namespace mt
