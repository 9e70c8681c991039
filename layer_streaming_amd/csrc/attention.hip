// Causal grouped-query flash attention for gfx950: forward (O and the
// log-sum-exp), and a deterministic backward split into a dQ kernel and a
// dK/dV kernel, neither using atomics.
//
// Everything runs on v_mfma_f32_32x32x16_f16.  The forward takes q, k and v
// in fp16, rounds P to fp16 for the P.V products and writes O in fp16
// (saturated to the fp16 range and counted).  The backward runs on fp16 too:
// dO (bf16, a gradient, far below fp16's normal range at this loss scale) is
// multiplied by a power of two 2^k chosen from max|dO| and max|v| so that
// every |dP|, |D| and |dS| stays below 2^15, and the results are scaled back
// by 2^-k (exact).  fp16 keeps three more mantissa bits than bf16 in every
// product, and q, k, v are used in the very form the forward used.
// The MFMA writes element r of lane l of a 32x32 result at row
// 8*(r/4) + 4*(l/32) + r%4, column l%32, and takes its A operand as row l%32,
// k = 8*(l/32)..+7 and its B operand as column l%32, same k.  The kernels
// exploit that:
//  * forward and dQ compute S^T = K Q^T, so a lane owns one query (a column)
//    and holds 16 of its scores in registers: the softmax state of a query
//    lives in one lane (plus its partner lane l^32), no LDS reductions;
//  * the probabilities then feed the next MFMA directly as its B operand,
//    with the contraction index (keys) permuted the same way in the A
//    operand, which is read transposed from the LDS image of V (or K);
//  * dK/dV compute S = Q K^T instead, so a lane owns one key and the key
//    gradients accumulate per lane over every query head of the KV group in
//    a fixed order.
// Tiles of 64 rows go from global memory straight into LDS
// (`buffer_load_dwordx4 ... lds`: no staging registers, no LDS stores),
// twice-buffered: the loads of the next tile are issued before the MFMAs on
// the current one.  Each tile has a buffer resource of its own based at its
// first row, so a sequence may span any number of bytes, and rows past the
// sequence's end read as zero.
#include "kcommon.h"
#include "kernels.h"

namespace mt {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int BKV = 64;  // keys (or queries) per staged tile

#define MFMA32H(a, b, c) __builtin_amdgcn_mfma_f32_32x32x16_f16((a), (b), (c), 0, 0, 0)
// 2^x on the hardware instruction alone: results below 2^-126 (probabilities
// that add nothing at fp32 precision) flush to zero instead of being formed
// as denormals, which costs the library form four more instructions.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Pack eight fp32 values (probabilities, or scaled dS bounded by 2^15) into an
// fp16 MFMA operand, round to nearest even: pairs through gfx950's
// v_cvt_pk_f16_f32 (one instruction per two values).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f16x8_t pack_h8(const float* v) {
    auto p = [](float a, float b) {
        const f32x2_t f = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
    };
    return as_f16x8(make_uint4(p(v[0], v[1]), p(v[2], v[3]), p(v[4], v[5]), p(v[6], v[7])));
}

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
// 4 bytes per lane into LDS at lds_addr + 4 * lane (as dma16).
__device__ __forceinline__ void dma4(i32x4_t rs, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rs)
                 : "memory");
}
__device__ __forceinline__ void wait_vmem0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's vector-memory operations are in flight
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else static_assert(N < 0, "unsupported count");
}
// Block barrier after this wave's loads landed (vmcnt) and its LDS reads
// completed (lgkmcnt through the builtin, so the compiler knows).
__device__ __forceinline__ void barrier_tile() {
    wait_vmem0();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// Row-major tile image [64][HD] in 16-byte chunks, chunk index XOR-swizzled
// by aswz(row): one function of the row that serves both read patterns
// without bank conflicts, 16 consecutive rows of one chunk (row fragments)
// and 4 rows x 4 chunks (transposed fragments, 32 lanes per cycle).
template <int HD>
__device__ __forceinline__ int aswz(int r) {
    if constexpr (HD == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

// Byte offsets of the DMA chunks of a 64-row tile: instruction i of wave w
// fills tile chunks (4 i + w) * 64 + lane with the logical chunk the swizzle
// puts there, from rows that are ld elements apart.
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
// Issue this wave's loads of the tile whose row 0 is `base` (a column block
// of HD elements); `valid` rows exist (<= 0: none; the rest read as zero).
template <int HD, int NI>
__device__ __forceinline__ void tile_issue(const uint16_t* base, int64_t ld, int valid, const uint32_t (&off)[NI],
                                           uint32_t lds, int wave) {
    const int rows = valid < BKV ? valid : BKV;
    const i32x4_t rs = make_rsrc(base, rows > 0 ? uint32_t((int64_t(rows - 1) * ld + HD) * 2) : 0u);
#pragma unroll
    for (int i = 0; i < NI; ++i)
        dma16(rs, __builtin_amdgcn_readfirstlane(lds + uint32_t((4 * i + wave) * 1024)), off[i]);
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
__device__ __forceinline__ f16x8_t tile_colT(const uint4* t, int dt, int tt, int s2, int lane) {
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
    return as_f16x8(make_uint4(r[0].x, r[0].y, r[1].x, r[1].y));
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

// ----------------------------------------------------------- forward ------
// Block: 4 waves x 32 queries of one (b, h); key tiles of 64.  A small
// register set lets two blocks share a CU, so one wave's softmax runs while
// the other's products do.
template <int HD>
__global__ __launch_bounds__(256, 2) void attn_fwd_k(AttnArgs a, int n_qt, int qt_slow) {
    constexpr int NS = HD / 16, ND = HD / 32, NCH = HD / 8;
    constexpr int TILE = BKV * NCH;  // 16-byte chunks per tile
    constexpr int NI = TILE / 256;   // wave instructions per tile and operand
    constexpr int RB = NCH * 16;     // bytes per LDS row
    __shared__ uint4 Ks[2][TILE];
    __shared__ uint4 Vs[2][TILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, c = lane & 31;
    // Query tile heaviest first: across all (b, h) when qt_slow (up to 256
    // tiles per head: the last blocks out are the lightest), else within each
    // (b, h) (longer sequences: the blocks in flight share one head's K and V
    // in L2; measured at S = 131072 the global order was 5% slower).
    const int nbh = a.B * a.Hq;
    const int qt = n_qt - 1 - (qt_slow ? int(blockIdx.x / unsigned(nbh)) : int(blockIdx.x % unsigned(n_qt)));
    const int bh = qt_slow ? int(blockIdx.x % unsigned(nbh)) : int(blockIdx.x / unsigned(n_qt));
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int hk = h / (a.Hq / a.Hkv);
    const int S = a.S;
    const int q0 = qt * 128;
    const int qw = q0 + wave * 32;
    const int q = qw + c;
    const uint16_t* base = a.qkv + int64_t(b) * S * a.ld;
    const uint16_t* kbase = base + (a.Hq + hk) * HD;
    const uint16_t* vbase = base + (a.Hq + a.Hkv + hk) * HD;

    f16x8_t qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (q < S) v = *reinterpret_cast<const uint4*>(base + int64_t(q) * a.ld + h * HD + (2 * s + hh) * 8);
        qf[s] = as_f16x8(v);
    }

    uint32_t doff[NI];
    tile_offsets<HD>(doff, wave, lane, a.ld);
    auto issue = [&](int k0, int buf) {
        tile_issue<HD>(kbase + int64_t(k0) * a.ld, a.ld, S - k0, doff, lds_addr(&Ks[buf][0]), wave);
        tile_issue<HD>(vbase + int64_t(k0) * a.ld, a.ld, S - k0, doff, lds_addr(&Vs[buf][0]), wave);
    };
    // K fragment (row 32 t + c, logical chunk 2 s + hh): byte offset in a tile.
    auto koff = [&](int t, int s) { return (32 * t + c) * RB + (((2 * s + hh) ^ aswz<HD>(32 * t + c)) * 16); };

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
            f32x16_t st[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int r = 0; r < 16; ++r) st[t][r] = 0.f;
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    st[t] = MFMA32H(as_f16x8(*reinterpret_cast<const uint4*>(kt + koff(t, s))), qf[s], st[t]);
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
            f16x8_t pb[2][2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    float tmp[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) tmp[e] = st[t][8 * s2 + e];
                    pb[t][s2] = pack_h8(tmp);
                }
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        o[dt] = MFMA32H(tile_colT<HD>(Vs[cur], dt, t, s2, lane), pb[t][s2], o[dt]);
        }
        barrier_tile();
    }

    const float ltot = lsum + __shfl_xor(lsum, 32, 64);
    if (q < S) {
        const float inv = 1.0f / ltot;
        uint16_t* orow = a.o + (int64_t(b) * S + q) * a.ldo + h * HD;
        uint32_t nov = 0;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hh;
                *reinterpret_cast<uint2*>(orow + d) =
                    make_uint2(pack2h_sat(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, nov),
                               pack2h_sat(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv, nov));
            }
        count_ovf(a.ovf, nov);
        if (hh == 0) a.lse[(int64_t(b) * a.Hq + h) * S + q] = (m + log2f(ltot)) * LN2;
    }
}

// ----------------------------------------------- backward: the scale ------
// 2^k for the fp16 backward: the largest power of two with
// max|dO| 2^k max|v| hd <= 2^14 (so |dP| = |dO . v| and |D| = |dO . o| stay
// <= 2^14, o being a convex combination of v, and |dS| = P |dP - D| <= 2^15)
// and max|dO| 2^k <= 2^14; 1 when dO is zero.  amax holds each maximum as
// AMAX_W partial maxima, one per 256-byte line (dO's in lines 0.., v's in
// lines AMAX_W..), as float bit patterns (non-negative floats order like
// their bits): the blocks of attn_amax_k spread their atomics over them, as
// atomics on one word, or on words of one line, serialise (about 11 ns each
// measured: 20 us for 1152 blocks).  The reads here are uniform, so they are
// scalar loads.
constexpr int AMAX_W = ATTN_AMAX_PARTS, AMAX_LINE = ATTN_AMAX_LINE;  // partial maxima per quantity; words per line
constexpr int AMAX_U = 8;                    // 16-byte loads in flight per lane of the maxima kernel
static_assert(2 * AMAX_W * AMAX_LINE * 4 == ATTN_AMAX_BYTES, "maxima scratch size");
__device__ __forceinline__ float grad_scale(const uint32_t* amax, int hd) {
    uint32_t ab = 0, vb = 0;
#pragma unroll
    for (int i = 0; i < AMAX_W; ++i) {
        ab = max(ab, amax[i * AMAX_LINE]);
        vb = max(vb, amax[(AMAX_W + i) * AMAX_LINE]);
    }
    const float a = __uint_as_float(ab), v = __uint_as_float(vb);
    if (!(a > 0.f)) return 1.f;
    float lim = 16384.f / a;
    if (v > 0.f) lim = fminf(lim, 16384.f / (a * v * float(hd)));
    lim = fminf(lim, 0x1p100f);
    int e;
    frexpf(lim, &e);  // lim = f 2^e, f in [0.5, 1): the largest power of two <= lim is 2^(e-1)
    return ldexpf(1.f, e - 1);
}

// max |dO| over [T x Hq*hd] (row stride ldo) and max |v| over the value
// heads of qkv into the partial maxima of amax (zeroed first): the first
// nb_do blocks stride over dO, the rest over v, AMAX_U 16-byte loads in
// flight per lane (all issued before the first is used); one atomic max per
// block, block i into partial i % AMAX_W of its maximum.  Indices are 32-bit
// (the host checks T*Hq*hd/8 < 2^31).
template <int HD>
__global__ __launch_bounds__(256) void attn_amax_k(AttnBwdArgs a, int nb_do) {
    __shared__ float red[4];
    const uint32_t T = uint32_t(int64_t(a.B) * a.S);
    const bool is_do = int(blockIdx.x) < nb_do;
    const uint32_t bi = is_do ? blockIdx.x : blockIdx.x - nb_do;
    const uint32_t nb = is_do ? uint32_t(nb_do) : gridDim.x - nb_do;
    const uint32_t per_row = uint32_t(is_do ? a.Hq : a.Hkv) * (HD / 8);  // 16-byte chunks per row
    const uint32_t n = T * per_row, stride = nb * 256;
    const uint16_t* vcol = a.qkv + int64_t(a.Hq + a.Hkv) * HD;
    auto chunk = [&](uint32_t i) {
        const uint32_t t = i / per_row, cc = i - t * per_row;
        return is_do ? reinterpret_cast<const uint4*>(a.dout + int64_t(t) * a.ldo)[cc]
                     : reinterpret_cast<const uint4*>(vcol + int64_t(t) * a.ld)[cc];
    };
    auto fold = [&](const uint4& v, float& mx) {
        float f[8];
        if (is_do) unpack8(v, f);
        else unpack8h(v, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(f[e]));
    };
    float mx = 0.f;
    for (uint32_t i0 = bi * 256 + threadIdx.x; i0 < n; i0 += AMAX_U * stride) {
        uint4 v[AMAX_U];
#pragma unroll
        for (int u = 0; u < AMAX_U; ++u) {
            const uint32_t i = i0 + u * stride;
            v[u] = i < n ? chunk(i) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < AMAX_U; ++u) fold(v[u], mx);
    }
    mx = wave_max(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0)
        atomicMax(a.amax + ((is_do ? 0 : AMAX_W) + bi % AMAX_W) * AMAX_LINE,
                  __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

// -D 2^k = -rowsum(dO * O) 2^k (O fp16) into dsum (negated: the dK/dV kernel
// starts its dP accumulation from it, so the MFMA forms dP - D), the
// log-sum-exp in base 2 (lse log2 e) into its second half, and dO 2^k in fp16 into
// do16 (range-guarded; the scale keeps it below 2^14).  One lane per 16-byte
// chunk of a (token, query head) row: the HD/8 lanes of a row are adjacent,
// so a wave instruction covers whole rows, and the row's dot product is
// reduced across them in a fixed order.  Rows go in the [B x Hq x S] order of
// dsum and lse, so a wave's sixteen rows of those are one 64-byte piece (in
// token order, their 4-byte entries lay S apart and each took a memory
// transaction of its own).
template <int HD>
__global__ __launch_bounds__(256) void attn_prep_k(AttnBwdArgs a) {
    constexpr int L = HD / 8;  // lanes per row
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    const uint32_t nrow = uint32_t(int64_t(a.B) * a.S) * uint32_t(a.Hq);
    const uint32_t r = i / L;  // (b, h, sq) with sq fastest: the index into dsum and lse
    const int j = int(i % L);
    const float s2k = grad_scale(a.amax, HD);
    float s = 0.f;
    uint32_t nov = 0;
    if (r < nrow) {
        const uint32_t bh = r / uint32_t(a.S), sq = r - bh * uint32_t(a.S);
        const uint32_t b = bh / uint32_t(a.Hq);
        const int h = int(bh - b * uint32_t(a.Hq));
        const int64_t t = int64_t(b) * a.S + sq;
        const uint4 ov = reinterpret_cast<const uint4*>(a.o + t * a.ldo + h * HD)[j];
        const uint4 gv = reinterpret_cast<const uint4*>(a.dout + t * a.ldo + h * HD)[j];
        float x[8], y[8];
        unpack8h(ov, x);
        unpack8(gv, y);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            s += x[k] * y[k];
            y[k] *= s2k;
        }
        reinterpret_cast<uint4*>(a.do16 + t * (int64_t(a.Hq) * HD) + h * HD)[j] = pack8h_sat(y, nov);
    }
#pragma unroll
    for (int o = L / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (r < nrow && j == 0) {
        a.dsum[r] = -(s * s2k);
        a.dsum[int64_t(nrow) + r] = a.lse[r] * LOG2E;
    }
    count_ovf(a.ovf, nov);
}

// Write four consecutive gradient columns of one row: fp32 into the fp32
// buffer when there is one, else bf16.
__device__ __forceinline__ void store_grad4(float* f32row, uint16_t* b16row, int d, float x0, float x1, float x2,
                                            float x3) {
    if (f32row) *reinterpret_cast<float4*>(f32row + d) = make_float4(x0, x1, x2, x3);
    else *reinterpret_cast<uint2*>(b16row + d) = make_uint2(pack2(x0, x1), pack2(x2, x3));
}

// The (cos, sin) pairs a lane's dQ columns rotate with at sequence position
// pos: pairs e = 32 dt + 8 g + 4 hh + 0..3 for dt < ND/2, two float4 (four
// pairs) per (dt, g).  Zero without a table.
template <int HD>
__device__ __forceinline__ void load_rope_row(const AttnBwdArgs& a, int pos, int hh, float4 (&cs)[HD / 8]) {
    constexpr int ND = HD / 32;
    if (!a.rope_tab) {
#pragma unroll
        for (int i = 0; i < HD / 8; ++i) cs[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    const float4* tr = reinterpret_cast<const float4*>(a.rope_tab + int64_t(pos) * (HD / 2));
#pragma unroll
    for (int dt = 0; dt < ND / 2; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int e = 32 * dt + 8 * g + 4 * hh;
            cs[2 * (4 * dt + g)] = tr[e / 2];
            cs[2 * (4 * dt + g) + 1] = tr[e / 2 + 1];
        }
}

// One row's gradient as a lane of the dQ and dK/dV kernels holds it
// (columns 32 dt + 8 g + 4 hh + 0..3, acc scaled by `scale`), rotated by
// -theta with the pairs load_rope_row gave (e and e + HD/2 sit in the same
// lane, blocks dt and dt + ND/2) and rounded to bf16 once into r16.  The
// rotation is the transpose of the forward's: lo' = lo cos + hi sin,
// hi' = hi cos - lo sin.
template <int HD>
__device__ __forceinline__ void store_rot_bf16(uint16_t* r16, const f32x16_t (&acc)[HD / 32], float scale, int hh,
                                               const float4 (&cs)[HD / 8]) {
    constexpr int ND = HD / 32;
#pragma unroll
    for (int dt = 0; dt < ND / 2; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int e = 32 * dt + 8 * g + 4 * hh;
            const float4 c0 = cs[2 * (4 * dt + g)], c1 = cs[2 * (4 * dt + g) + 1];
            const float cv[4] = {c0.x, c0.z, c1.x, c1.z}, sv[4] = {c0.y, c0.w, c1.y, c1.w};
            float ol[4], oh[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo = acc[dt][4 * g + j] * scale, hi = acc[dt + ND / 2][4 * g + j] * scale;
                ol[j] = lo * cv[j] + hi * sv[j];
                oh[j] = hi * cv[j] - lo * sv[j];
            }
            *reinterpret_cast<uint2*>(r16 + e) = make_uint2(pack2(ol[0], ol[1]), pack2(ol[2], ol[3]));
            *reinterpret_cast<uint2*>(r16 + e + HD / 2) = make_uint2(pack2(oh[0], oh[1]), pack2(oh[2], oh[3]));
        }
}

// dQ of one query row: rotated and rounded once with a.rope_tab, else
// stored as store_grad4 does (fp32 into dqk32 when set, else bf16).
template <int HD>
__device__ __forceinline__ void store_dq_row(const AttnBwdArgs& a, const f32x16_t (&acc)[HD / 32], float scale,
                                             int64_t row, int h, int hh, const float4 (&cs)[HD / 8]) {
    constexpr int ND = HD / 32;
    uint16_t* r16 = a.dqkv + row * a.ldd + h * HD;
    if (a.rope_tab) {
        store_rot_bf16<HD>(r16, acc, scale, hh, cs);
        return;
    }
    float* r32 = a.dqk32 ? a.dqk32 + row * a.ld32 + h * HD : nullptr;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            store_grad4(r32, r16, 32 * dt + 8 * g + 4 * hh, acc[dt][4 * g] * scale, acc[dt][4 * g + 1] * scale,
                        acc[dt][4 * g + 2] * scale, acc[dt][4 * g + 3] * scale);
}

// dQ: block = 4 waves x 32 queries of one (b, h); key tiles of 64 staged as
// fp16 K (rows for the scores, read transposed for dQ) and fp16 V (rows for
// dP).
template <int HD>
__global__ __launch_bounds__(256, 2) void attn_dq_k(AttnBwdArgs a, int n_qt, int qt_slow) {
    constexpr int NS = HD / 16, ND = HD / 32, NCH = HD / 8;
    constexpr int TILE = BKV * NCH, NI = TILE / 256;
    __shared__ uint4 Ks[2][TILE];
    __shared__ uint4 Vs[2][TILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, c = lane & 31;
    // Query tile heaviest first: across all (b, h) when qt_slow (up to 256
    // tiles per head: the last blocks out are the lightest), else within each
    // (b, h) (longer sequences: the blocks in flight share one head's K and V
    // in L2; measured at S = 131072 the global order was 5% slower).
    const int nbh = a.B * a.Hq;
    const int qt = n_qt - 1 - (qt_slow ? int(blockIdx.x / unsigned(nbh)) : int(blockIdx.x % unsigned(n_qt)));
    const int bh = qt_slow ? int(blockIdx.x % unsigned(nbh)) : int(blockIdx.x / unsigned(n_qt));
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int hk = h / (a.Hq / a.Hkv);
    const int S = a.S;
    const int q0 = qt * 128, qw = q0 + wave * 32, q = qw + c;
    const int64_t ldg = int64_t(a.Hq) * HD;  // do16 row stride
    const uint16_t* base = a.qkv + int64_t(b) * S * a.ld;
    const uint16_t* gbase = a.do16 + int64_t(b) * S * ldg;
    const uint16_t* kbase = base + (a.Hq + hk) * HD;
    const uint16_t* vbase = base + (a.Hq + a.Hkv + hk) * HD;
    const float s2k = grad_scale(a.amax, HD);

    f16x8_t qf[NS], dof[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0), w = v;
        if (q < S) {
            v = *reinterpret_cast<const uint4*>(base + int64_t(q) * a.ld + h * HD + (2 * s + hh) * 8);
            w = *reinterpret_cast<const uint4*>(gbase + int64_t(q) * ldg + h * HD + (2 * s + hh) * 8);
        }
        qf[s] = as_f16x8(v);
        dof[s] = as_f16x8(w);
    }
    const int64_t st_off = (int64_t(b) * a.Hq + h) * S;
    const float lse2 = q < S ? a.lse[st_off + q] * LOG2E : 0.f;
    const float dq_nd = q < S ? a.dsum[st_off + q] : 0.f;  // -D 2^k

    uint32_t off[NI];
    tile_offsets<HD>(off, wave, lane, a.ld);
    auto issue = [&](int k0, int buf) {
        tile_issue<HD>(kbase + int64_t(k0) * a.ld, a.ld, S - k0, off, lds_addr(&Ks[buf][0]), wave);
        tile_issue<HD>(vbase + int64_t(k0) * a.ld, a.ld, S - k0, off, lds_addr(&Vs[buf][0]), wave);
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
        // dS of the tile, zero where the whole tile lies above the wave's
        // queries; the dQ products then run unconditionally, which lets the
        // accumulators stay in place across iterations (a conditional update
        // made the compiler copy all 64 of them in and out every tile)
        f16x8_t dsb[2][2];
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
                    k[t] = tile_row<HD>(Ks[cur], 32 * t + c, 2 * s + hh);
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
                    dp[t] = MFMA32H(as_f16x8(fv[s & 1][t]), dof[s], dp[t]);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            const bool full = k0 + BKV - 1 <= qw && k0 + BKV <= S;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    float tmp[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) tmp[j] = ex2(fmaf(st[t][8 * s2 + j], sc, -lse2));
                    if (__builtin_expect(!full, 0)) {  // a uniform branch: only tiles crossing the diagonal or the end
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const int r = 8 * s2 + j;
                            const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
                            if (key > q || key >= S) tmp[j] = 0.f;
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) tmp[j] *= dp[t][8 * s2 + j] + dq_nd;
                    dsb[t][s2] = pack_h8(tmp);
                }
        } else {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) dsb[t][s2] = f16x8_t{};
        }
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    acc[dt] = MFMA32H(tile_colT<HD>(Ks[cur], dt, t, s2, lane), dsb[t][s2], acc[dt]);
        barrier_tile();
    }
    if (q < S) {
        float4 cs[HD / 8];   // loaded here: this kernel has no registers to spare over its loop
        load_rope_row<HD>(a, q, hh, cs);
        store_dq_row<HD>(a, acc, rsqrtf(float(HD)) / s2k, int64_t(b) * S + q, h, hh, cs);
    }
}

// dQ = dS K from the dS the dK/dV pass stored (stored-dS form, short
// sequences): block = 4 waves x 32 queries of one (b, h), key tiles of 64.
// Each tile stages K and the matching 64 keys x 128 queries of dS (eight
// stored 32 x 32 blocks) with the same swizzled row layout, and both
// operands are read transposed, dS with lane = query position, so the
// contraction runs over the same key permutation in both; lane c's output
// row is the query its position holds in the stored order.  Key blocks of
// 32 above the wave's queries were never written and are skipped; keys past
// the sequence read as zero, and query columns past it only reach rows that
// are not stored.
template <int HD>
__global__ __launch_bounds__(256, 2) void attn_dq_ds_k(AttnBwdArgs a, int n_qt, int qt_slow) {
    constexpr int ND = HD / 32, NCH = HD / 8;
    constexpr int TILE = BKV * NCH, NI = TILE / 256;
    constexpr int STILE = BKV * 16, SNI = STILE / 256;  // dS tile: 64 keys x 128 queries
    __shared__ uint4 Ks[2][TILE];
    __shared__ uint4 Ss[2][STILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, c = lane & 31;
    const int nbh = a.B * a.Hq;
    const int qt = n_qt - 1 - (qt_slow ? int(blockIdx.x / unsigned(nbh)) : int(blockIdx.x % unsigned(n_qt)));
    const int bh = qt_slow ? int(blockIdx.x % unsigned(nbh)) : int(blockIdx.x / unsigned(n_qt));
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int hk = h / (a.Hq / a.Hkv);
    const int S = a.S;
    const int q0 = qt * 128, qw = q0 + wave * 32, q = qw + c;
    const uint16_t* kbase = a.qkv + int64_t(b) * S * a.ld + (a.Hq + hk) * HD;
    const int nb = int(a.ds_ld / 32);
    const uint16_t* dsbase = a.ds + (int64_t(b) * a.Hq + h) * nb * nb * 1024 + (q0 / 32) * 1024;
    const float s2k = grad_scale(a.amax, HD);
    // the rotation's (cos, sin) pairs of the lane's output row (query of
    // position c in the stored order), loaded now so they arrive during the loop
    const int qs = qw + 8 * ((c >> 2) & 3) + 4 * (c >> 4) + (c & 3);
    float4 cs[HD / 8];
    load_rope_row<HD>(a, min(qs, S - 1), hh, cs);

    uint32_t koff[NI], soff[SNI];
    int srow[SNI];
    tile_offsets<HD>(koff, wave, lane, a.ld);
    // the dS tile's LDS slot (row r, chunk) takes logical chunk lc of row r:
    // key block r / 32, query block lc / 4, row r % 32, 16 bytes at 16 (lc % 4)
#pragma unroll
    for (int i = 0; i < SNI; ++i) {
        const int pos = (4 * i + wave) * 64 + lane;
        const int r = pos / 16;
        const int lc = (pos % 16) ^ aswz<128>(r);
        soff[i] = uint32_t((((r / 32) * nb + lc / 4) * 1024 + (r % 32) * 32 + (lc % 4) * 8) * 2);
        srow[i] = r;
    }
    auto issue = [&](int k0, int buf) {
        tile_issue<HD>(kbase + int64_t(k0) * a.ld, a.ld, S - k0, koff, lds_addr(&Ks[buf][0]), wave);
        const i32x4_t rs = make_rsrc(dsbase + int64_t(k0 / 32) * nb * 1024, uint32_t((int64_t(nb + 3) * 1024 + 1024) * 2));
        const uint32_t lds = lds_addr(&Ss[buf][0]);
#pragma unroll
        for (int i = 0; i < SNI; ++i)
            dma16(rs, __builtin_amdgcn_readfirstlane(lds + uint32_t((4 * i + wave) * 1024)),
                  k0 + srow[i] < S ? soff[i] : 0x80000000u);
    };

    f32x16_t acc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

    const int k_end = min(S, q0 + 128);
    const int nkb = (k_end + BKV - 1) / BKV;
    issue(0, 0);
    barrier_tile();
    for (int kb = 0; kb < nkb; ++kb) {
        const int cur = kb & 1;
        const int k0 = kb * BKV;
        if (kb + 1 < nkb) issue(k0 + BKV, cur ^ 1);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (k0 + 32 * t <= qw + 31) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const f16x8_t dsf = tile_colT<128>(Ss[cur], wave, t, s2, lane);
#pragma unroll
                    for (int dt = 0; dt < ND; ++dt)
                        acc[dt] = MFMA32H(tile_colT<HD>(Ks[cur], dt, t, s2, lane), dsf, acc[dt]);
                }
            }
        }
        barrier_tile();
    }
    // qs: the query of position c in the stored order, 8 (c / 4 % 4) + 4 (c / 16) + c % 4
    if (qs < S) store_dq_row<HD>(a, acc, rsqrtf(float(HD)) / s2k, int64_t(b) * S + qs, h, hh, cs);
}

// dK, dV: block = 8 waves over 128 keys of one (b, kv head), looping over
// 64-query tiles of the group's query heads (or, split ns ways, of the
// split's share of them), head by head, each from the block's diagonal to
// the end of the sequence.  The work of a key tile shrinks with its position
// (causal), so blocks go out heaviest first when kt_slow (key tile the
// slowest index), else key tiles of one (b, kv head) in a row.  With ns > 1
// each block writes its fp32 partial sums, which attn_dkdv_reduce_k adds in
// split order.
//
// Waves w and w+4 (one SIMD) share keys k0 + 32 w ..+31 and work as a
// two-stage pipeline over half tiles of 32 queries.  The front wave (w < 4)
// holds K and V of its keys, forms S = Q K^T and dP = dO V^T for half h,
// then P and dS = P (dP - D) in fp32, and hands both over through LDS in the
// fp16 form the products take.  The back wave accumulates dV += P^T dO and
// dK += dS^T Q for half h - 1 meanwhile, so one barrier per half tile
// separates the stages and each SIMD always has one wave's products beside
// the other's exponentials.  Q and dO tiles sit in three LDS buffers: a tile
// is used by the front wave in two phases and by the back wave one phase
// later, and its successor's loads are issued three phases before it is
// needed; the log-sum-exp and D rows come in with the same direct loads.
template <int HD>
__global__ __launch_bounds__(512, 1) void attn_dkdv_k(AttnBwdArgs a, int n_kt, int ns, int kt_slow) {
    constexpr int NS = HD / 16, ND = HD / 32, NCH = HD / 8;
    constexpr int TILE = BKV * NCH, NI = TILE / 256;
    __shared__ uint4 Qs[3][TILE];
    __shared__ uint4 Ds[3][TILE];
    __shared__ __align__(16) float Ls[3][BKV];
    __shared__ __align__(16) float Dd[3][BKV];
    __shared__ uint4 Xh[2][4][4][64];  // per half tile and key group: P (s2 = 0, 1) and dS (s2 = 0, 1) per lane

    // the wave index as a scalar, so that every per-wave test below is a branch
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pw = wave & 3;
    const bool front = wave < 4;
    const int hh = lane >> 5, c = lane & 31;
    int kt, bk;
    const int split = int(blockIdx.x % unsigned(ns));
    {
        const int r = int(blockIdx.x / unsigned(ns)), nbk = a.B * a.Hkv;
        kt = kt_slow ? r / nbk : r % n_kt;
        bk = kt_slow ? r % nbk : r / n_kt;
    }
    const int hk = bk % a.Hkv, b = bk / a.Hkv;
    const int G = a.Hq / a.Hkv;
    const int h_lo = hk * G + split * G / ns, ng = hk * G + (split + 1) * G / ns - h_lo;
    const int S = a.S;
    const int k0 = kt * 128, kw = k0 + pw * 32, key = kw + c;
    const int64_t ldg = int64_t(a.Hq) * HD;  // do16 row stride
    const uint16_t* base = a.qkv + int64_t(b) * S * a.ld;
    const uint16_t* gbase = a.do16 + int64_t(b) * S * ldg;
    const int kcol = (a.Hq + hk) * HD, vcol = (a.Hq + a.Hkv + hk) * HD;
    const float s2k = grad_scale(a.amax, HD);

    const int qb0 = k0 / BKV;
    const int nqb = (S + BKV - 1) / BKV - qb0;  // query tiles per head
    const int tt = nqb * ng;                     // tiles: head h_lo + j / nqb, query tile qb0 + j % nqb

    uint32_t off[NI];
    tile_offsets<HD>(off, pw, lane, front ? a.ld : ldg);
    int last_issued = -1;
    auto issue_tile = [&](int j) {  // tile j into buffer j % 3
        const int hq = h_lo + j / nqb, q0 = (qb0 + j % nqb) * BKV, buf = j % 3;
        if (front) tile_issue<HD>(base + int64_t(q0) * a.ld + hq * HD, a.ld, S - q0, off, lds_addr(&Qs[buf][0]), pw);
        else tile_issue<HD>(gbase + int64_t(q0) * ldg + hq * HD, ldg, S - q0, off, lds_addr(&Ds[buf][0]), pw);
        if (wave == 0) {
            const int64_t o = (int64_t(b) * a.Hq + hq) * S + q0;
            const uint32_t ext = uint32_t(min(BKV, S - q0)) * 4u;
            const float* lse2 = a.dsum + int64_t(a.B) * a.S * a.Hq;  // base-2 log-sum-exp, written by prep
            dma4(make_rsrc(lse2 + o, ext), __builtin_amdgcn_readfirstlane(lds_addr(&Ls[buf][0])), uint32_t(lane) * 4u);
            dma4(make_rsrc(a.dsum + o, ext), __builtin_amdgcn_readfirstlane(lds_addr(&Dd[buf][0])), uint32_t(lane) * 4u);
        }
        last_issued = j;
    };
    // End of a phase: this wave's LDS traffic done, and every tile up to
    // `need` landed (only a newer tile's loads may still be in flight).
    auto phase_end = [&](int need) {
        if (last_issued > need) {
            if (wave == 0) wait_vmem<NI + 2>();
            else wait_vmem<NI>();
        } else {
            wait_vmem<0>();
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // Phase p: the front wave works on half tile p, the back wave on p - 1;
    // the tile two ahead of the front wave's is issued on odd phases.  Both
    // loops below run the same phases and barriers.
    auto next_tile = [&](int p) {
        if ((p & 1) && (p + 3) / 2 < tt) issue_tile((p + 3) / 2);
    };

    issue_tile(0);
    if (tt > 1) issue_tile(1);
    phase_end(0);
    if (front) {
        // K and V of the wave's keys: the B operands of S and dP.
        f16x8_t kf[NS], vf[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            uint4 u = make_uint4(0, 0, 0, 0), v = u;
            if (key < S) {
                u = *reinterpret_cast<const uint4*>(base + int64_t(key) * a.ld + kcol + (2 * s + hh) * 8);
                v = *reinterpret_cast<const uint4*>(base + int64_t(key) * a.ld + vcol + (2 * s + hh) * 8);
            }
            kf[s] = as_f16x8(u);
            vf[s] = as_f16x8(v);
        }
        const float sc = LOG2E * rsqrtf(float(HD));
        // stored-dS form: the previous phase's dS goes out at the start of
        // the next one, before its tile loads, so the end-of-phase wait
        // (loads land in order) finds those stores long acknowledged.  A
        // 32-key x 32-query block is 2 KB: key row c holds the 32 queries in
        // the order 0-3, 8-11, 16-19, 24-27, 4-7, 12-15, 20-23, 28-31, which
        // puts each lane's two fp16 octets (s2 = 0, 1) side by side at byte
        // 32 hh + 16 s2: every store instruction fills whole row segments
        uint4 ds_prev[2];
        uint16_t* ds_row = nullptr;  // this lane's key row of the previous phase's block, at its first query
        for (int p = 0; p <= 2 * tt; ++p) {
            if (ds_row) {
                *reinterpret_cast<uint4*>(ds_row) = ds_prev[0];
                *reinterpret_cast<uint4*>(ds_row + 8) = ds_prev[1];
                ds_row = nullptr;
            }
            next_tile(p);
            const int h = p;
            const int j = h >> 1, t = h & 1, buf = j % 3;
            const int q0 = (qb0 + j % nqb) * BKV, qh = q0 + 32 * t;
            // some query of the half at or after one of the pair's keys
            if (h < 2 * tt && kw <= qh + 31) {
                uint4* X = &Xh[h & 1][pw][0][0];
                f32x16_t st, dp;
                constexpr int PA = 3;
                uint4 fa[PA][2];
                auto rd = [&](int s, uint4(&f)[2]) {
                    f[0] = tile_row<HD>(Qs[buf], 32 * t + c, 2 * s + hh);
                    f[1] = tile_row<HD>(Ds[buf], 32 * t + c, 2 * s + hh);
                };
                static_for_n<PA - 1>([&](auto s_) { rd(decltype(s_)::value, fa[decltype(s_)::value]); });
                // dP starts from -D of each element's query, so the products
                // leave dP - D (element r: query 8 (r/4) + 4 hh + r%4 of the half)
                f32x16_t dinit;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 nd = *reinterpret_cast<const float4*>(&Dd[buf][32 * t + 8 * g + 4 * hh]);
                    dinit[4 * g] = nd.x;
                    dinit[4 * g + 1] = nd.y;
                    dinit[4 * g + 2] = nd.z;
                    dinit[4 * g + 3] = nd.w;
                }
                static_for_n<NS>([&](auto s_) {
                    constexpr int s = decltype(s_)::value;
                    if constexpr (s + PA - 1 < NS) rd(s + PA - 1, fa[(s + PA - 1) % PA]);
                    __builtin_amdgcn_sched_barrier(0);
                    st = MFMA32H(as_f16x8(fa[s % PA][0]), kf[s], s == 0 ? f32x16_t{} : st);
                    dp = MFMA32H(as_f16x8(fa[s % PA][1]), vf[s], s == 0 ? dinit : dp);
                    __builtin_amdgcn_sched_barrier(0);
                });
                const bool full = kw + 31 <= qh && qh + 32 <= S && kw + 32 <= S;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    float tp[8], td[8];
#pragma unroll
                    for (int g4 = 0; g4 < 2; ++g4) {
                        const int qb = 32 * t + 8 * (2 * s2 + g4) + 4 * hh;  // query within the tile
                        float lv[4];
                        *reinterpret_cast<float4*>(lv) = *reinterpret_cast<const float4*>(&Ls[buf][qb]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) tp[4 * g4 + e] = ex2(fmaf(st[8 * s2 + 4 * g4 + e], sc, -lv[e]));
                    }
                    // causal and sequence-end masks only on the wave's tiles that
                    // cross the diagonal or the end (a uniform branch)
                    if (__builtin_expect(!full, 0)) {
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj) {
                            const int qq = q0 + 32 * t + 8 * (2 * s2 + (jj >> 2)) + 4 * hh + (jj & 3);
                            if (key > qq || qq >= S || key >= S) tp[jj] = 0.f;
                        }
                    }
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) td[jj] = tp[jj] * dp[8 * s2 + jj];  // dp holds dP - D
                    X[s2 * 64 + lane] = __builtin_bit_cast(uint4, pack_h8(tp));
                    const uint4 dsv = __builtin_bit_cast(uint4, pack_h8(td));
                    X[(2 + s2) * 64 + lane] = dsv;
                    ds_prev[s2] = dsv;
                }
                if (a.ds && key < S) {
                    const int hq = h_lo + j / nqb, nb = int(a.ds_ld / 32);
                    ds_row = a.ds + (((int64_t(b) * a.Hq + hq) * nb + kw / 32) * nb + qh / 32) * 1024 + c * 32 + 16 * hh;
                }
            }
            phase_end((p + 1) >> 1);
        }
        return;
    }
    f32x16_t acc_v[ND], acc_k[ND];  // dV and dK, transposed (rows = head dim, lane = key)
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc_v[i][r] = 0.f;
            acc_k[i][r] = 0.f;
        }
    for (int p = 0; p <= 2 * tt; ++p) {
        next_tile(p);
        const int h = p - 1;
        if (h >= 0) {
            const int j = h >> 1, t = h & 1, buf = j % 3;
            const int qh = (qb0 + j % nqb) * BKV + 32 * t;
            if (kw <= qh + 31) {
                const uint4* X = &Xh[h & 1][pw][0][0];
                f16x8_t op[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) op[i] = as_f16x8(X[i * 64 + lane]);
                // dV += P^T dO and dK += dS^T Q over the half's 32 queries: the
                // accumulators take turns; fragments read PB - 1 products ahead.
                constexpr int NP = 4 * ND, PB = 4;
                auto frag = [&](int i) {
                    const int dt = (i >> 1) % ND, s2 = (i >> 1) / ND, k = i & 1;
                    return tile_colT<HD>(k ? Qs[buf] : Ds[buf], dt, t, s2, lane);
                };
                f16x8_t fb[PB];
                static_for_n<PB - 1>([&](auto i_) { fb[decltype(i_)::value] = frag(decltype(i_)::value); });
                static_for_n<NP>([&](auto i_) {
                    constexpr int i = decltype(i_)::value;
                    constexpr int dt = (i >> 1) % ND, s2 = (i >> 1) / ND, k = i & 1;
                    if constexpr (i + PB - 1 < NP) fb[(i + PB - 1) % PB] = frag(i + PB - 1);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (k) acc_k[dt] = MFMA32H(fb[i % PB], op[2 + s2], acc_k[dt]);
                    else acc_v[dt] = MFMA32H(fb[i % PB], op[s2], acc_v[dt]);
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
        }
        phase_end((p + 1) >> 1);
    }
    if (key < S) {
        const float inv = 1.0f / s2k, scale = rsqrtf(float(HD)) * inv;
        const int64_t row = int64_t(b) * S + key;
        if (ns > 1) {
            const int64_t T = int64_t(a.B) * S, w = int64_t(a.Hkv) * HD;
            float* prow = a.dpart + (int64_t(split) * T + row) * (2 * w) + hk * HD;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = 32 * dt + 8 * g + 4 * hh;
                    *reinterpret_cast<float4*>(prow + d) =
                        make_float4(acc_k[dt][4 * g] * scale, acc_k[dt][4 * g + 1] * scale,
                                    acc_k[dt][4 * g + 2] * scale, acc_k[dt][4 * g + 3] * scale);
                    *reinterpret_cast<float4*>(prow + w + d) =
                        make_float4(acc_v[dt][4 * g] * inv, acc_v[dt][4 * g + 1] * inv, acc_v[dt][4 * g + 2] * inv,
                                    acc_v[dt][4 * g + 3] * inv);
                }
        } else {
            uint16_t* rk = a.dqkv + row * a.ldd + kcol;
            uint16_t* rv = a.dqkv + row * a.ldd + vcol;
            if (a.rope_tab) {
                float4 cs[HD / 8];
                load_rope_row<HD>(a, key, hh, cs);
                store_rot_bf16<HD>(rk, acc_k, scale, hh, cs);
            } else {
                float* r32 = a.dqk32 ? a.dqk32 + row * a.ld32 + (a.Hq + hk) * HD : nullptr;
#pragma unroll
                for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        store_grad4(r32, rk, 32 * dt + 8 * g + 4 * hh, acc_k[dt][4 * g] * scale,
                                    acc_k[dt][4 * g + 1] * scale, acc_k[dt][4 * g + 2] * scale,
                                    acc_k[dt][4 * g + 3] * scale);
            }
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = 32 * dt + 8 * g + 4 * hh;
                    *reinterpret_cast<uint2*>(rv + d) =
                        make_uint2(pack2(acc_v[dt][4 * g] * inv, acc_v[dt][4 * g + 1] * inv),
                                   pack2(acc_v[dt][4 * g + 2] * inv, acc_v[dt][4 * g + 3] * inv));
                }
        }
    }
}

// Sum of the ns partials of the split dK/dV pass, in split order: dK into
// the fp32 buffer (or bf16 dqkv), dV into dqkv in bf16.  One lane per four
// columns of a row's [dK | dV] partial, all of its partials loaded before the
// first is added.  Indices are 32-bit: a pass splits only with fewer than 512
// key-tile blocks, so T*Hkv < 2^16 and T*Hkv*hd/2 < 2^22 (a 64-bit division
// here had cost more than the loads).
__global__ __launch_bounds__(256) void attn_dkdv_reduce_k(AttnBwdArgs a, int ns) {
    constexpr int NP = 8;  // partials loaded at once
    const uint32_t T = uint32_t(a.B) * uint32_t(a.S);
    const uint32_t w = uint32_t(a.Hkv * a.hd), q4 = w / 2;  // columns of one half; float4s per row
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= T * q4) return;
    const uint32_t row = i / q4;
    const uint32_t j = (i - row * q4) * 4;
    const float* src = a.dpart + int64_t(row) * (2 * w) + j;
    const int64_t pstride = int64_t(T) * (2 * w);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = 0; p0 < ns; p0 += NP) {
        float4 v[NP];
#pragma unroll
        for (int u = 0; u < NP; ++u)
            if (p0 + u < ns) v[u] = *reinterpret_cast<const float4*>(src + (p0 + u) * pstride);
#pragma unroll
        for (int u = 0; u < NP; ++u)
            if (p0 + u < ns) {
                acc.x += v[u].x;
                acc.y += v[u].y;
                acc.z += v[u].z;
                acc.w += v[u].w;
            }
    }
    const int64_t orow = int64_t(row);
    if (j < w) {
        const int col = a.Hq * a.hd + int(j);
        if (a.dqk32) *reinterpret_cast<float4*>(a.dqk32 + orow * a.ld32 + col) = acc;
        else *reinterpret_cast<uint2*>(a.dqkv + orow * a.ldd + col) = make_uint2(pack2(acc.x, acc.y), pack2(acc.z, acc.w));
    } else {
        const int col = (a.Hq + a.Hkv) * a.hd + int(j - w);
        *reinterpret_cast<uint2*>(a.dqkv + orow * a.ldd + col) = make_uint2(pack2(acc.x, acc.y), pack2(acc.z, acc.w));
    }
}

// The same sum with dK rotated by -theta and rounded to bf16 once (a.rope_tab
// set): one lane per four columns e..e+3 and their partners e+hd/2.. of one
// head's dK or dV in one row, the first Hkv*hd/8 lanes of a row on dK, the
// rest on dV.  Rotation as in store_rot_bf16.
__global__ __launch_bounds__(256) void attn_dkdv_reduce_rot_k(AttnBwdArgs a, int ns) {
    const uint32_t T = uint32_t(a.B) * uint32_t(a.S);
    const uint32_t hd = uint32_t(a.hd), half = hd / 2, w = uint32_t(a.Hkv) * hd;
    const uint32_t per_row = w / 4, gph = hd / 8;  // lanes per row; 4-column groups per head half
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= T * per_row) return;
    const uint32_t row = i / per_row, t = i - row * per_row;
    const bool is_k = t < per_row / 2;
    const uint32_t u = is_k ? t : t - per_row / 2;
    const uint32_t hk = u / gph, e = (u - hk * gph) * 4;
    const uint32_t c0 = hk * hd + e;  // column of the pair's first half within dK (or dV)
    const float* src = a.dpart + int64_t(row) * (2 * w) + (is_k ? 0 : w) + c0;
    const int64_t pstride = int64_t(T) * (2 * w);
    float lo[4] = {0.f, 0.f, 0.f, 0.f}, hi[4] = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < ns; ++p) {
        const float4 x = *reinterpret_cast<const float4*>(src + p * pstride);
        const float4 y = *reinterpret_cast<const float4*>(src + p * pstride + half);
        lo[0] += x.x; lo[1] += x.y; lo[2] += x.z; lo[3] += x.w;
        hi[0] += y.x; hi[1] += y.y; hi[2] += y.z; hi[3] += y.w;
    }
    uint16_t* dst = a.dqkv + int64_t(row) * a.ldd + (is_k ? a.Hq : a.Hq + a.Hkv) * a.hd + c0;
    if (is_k) {
        const float4* tr = reinterpret_cast<const float4*>(a.rope_tab + int64_t(row % uint32_t(a.S)) * half + e);
        const float4 q0 = tr[0], q1 = tr[1];
        const float cv[4] = {q0.x, q0.z, q1.x, q1.z}, sv[4] = {q0.y, q0.w, q1.y, q1.w};
        float ol[4], oh[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ol[j] = lo[j] * cv[j] + hi[j] * sv[j];
            oh[j] = hi[j] * cv[j] - lo[j] * sv[j];
        }
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack2(ol[0], ol[1]), pack2(ol[2], ol[3]));
        *reinterpret_cast<uint2*>(dst + half) = make_uint2(pack2(oh[0], oh[1]), pack2(oh[2], oh[3]));
    } else {
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
        *reinterpret_cast<uint2*>(dst + half) = make_uint2(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
    }
}

bool attn_shape_ok(int B, int S, int Hq, int Hkv, int hd, int64_t ld, int64_t ldo) {
    if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return false;
    if (hd != 64 && hd != 128) return false;
    if ((ld & 7) || (ldo & 7)) return false;
    if (ld < int64_t(Hq + 2 * Hkv) * hd || ldo < int64_t(Hq) * hd) return false;
    // a tile's 64 rows addressed through one 32-bit buffer extent
    if (int64_t(BKV) * std::max(ld, int64_t(Hq) * hd) * 2 >= (int64_t(1) << 31)) return false;
    return true;
}

}  // namespace

hipError_t attn_fwd(const AttnArgs& a, hipStream_t s) {
    if (!attn_shape_ok(a.B, a.S, a.Hq, a.Hkv, a.hd, a.ld, a.ldo)) return hipErrorInvalidValue;
    const int n_qt = (a.S + 127) / 128;
    const dim3 grid(unsigned(int64_t(n_qt) * a.B * a.Hq));
    const int qt_slow = n_qt <= 256;
    if (a.hd == 128) attn_fwd_k<128><<<grid, 256, 0, s>>>(a, n_qt, qt_slow);
    else attn_fwd_k<64><<<grid, 256, 0, s>>>(a, n_qt, qt_slow);
    return hipGetLastError();
}

int attn_dkdv_splits(int B, int S, int Hq, int Hkv, int hd, int64_t part_elems, int req) {
    if (B <= 0 || S <= 0 || Hkv <= 0 || Hq % Hkv) return 1;
    const int G = Hq / Hkv;
    const int64_t blocks = int64_t(B) * Hkv * ((S + 127) / 128);
    int ns = req > 0 ? std::min(req, G) : blocks >= 512 ? 1 : int(std::min<int64_t>(G, (512 + blocks - 1) / blocks));
    const int64_t per = int64_t(B) * S * 2 * Hkv * hd;
    while (ns > 1 && ns * per > part_elems) --ns;
    return std::max(ns, 1);
}

int64_t attn_bwd_part_elems(int B, int S, int Hq, int Hkv, int hd) {
    const int ns = attn_dkdv_splits(B, S, Hq, Hkv, hd, INT64_MAX, 0);
    return ns > 1 ? int64_t(ns) * B * S * 2 * Hkv * hd : 0;
}

namespace {
int64_t al256(int64_t x) { return (x + 255) & ~int64_t(255); }
}  // namespace

// The stored form trades two of dQ's three products for writing and reading
// dS (4 bytes per score): measured at B8 x S1024 (28 / 4 heads) it takes the
// backward from 0.493 to 0.456 ms, at B4 x S2048 (40 / 8) from 1.092 to 1.075
// ms, where dQ already runs its products well; so only up to S = 1024.
int64_t attn_ds_bytes(int B, int S, int Hq) {
    if (B <= 0 || S <= 0 || Hq <= 0 || S > 1024) return 0;
    const int64_t sp = (int64_t(S) + 127) / 128 * 128;
    const int64_t bytes = int64_t(B) * Hq * sp * sp * 2;
    return bytes <= (int64_t(1) << 30) ? bytes : 0;
}

int64_t attn_bwd_work_bytes(int B, int S, int Hq, int Hkv, int hd) {
    const int64_t T = int64_t(B) * S;
    return al256(2 * T * Hq * 4) + al256(T * Hq * hd * 2) + ATTN_AMAX_BYTES +
           al256(attn_bwd_part_elems(B, S, Hq, Hkv, hd) * 4) +
           al256(attn_ds_bytes(B, S, Hq));
}

void attn_bwd_carve(void* work, int B, int S, int Hq, int Hkv, int hd, AttnBwdArgs& a, bool with_ds) {
    const int64_t T = int64_t(B) * S;
    uint8_t* p = static_cast<uint8_t*>(work);
    a.dsum = reinterpret_cast<float*>(p);
    p += al256(2 * T * Hq * 4);
    a.do16 = reinterpret_cast<uint16_t*>(p);
    p += al256(T * Hq * hd * 2);
    a.amax = reinterpret_cast<uint32_t*>(p);
    p += ATTN_AMAX_BYTES;
    a.dpart_elems = attn_bwd_part_elems(B, S, Hq, Hkv, hd);
    a.dpart = a.dpart_elems ? reinterpret_cast<float*>(p) : nullptr;
    p += al256(a.dpart_elems * 4);
    const int64_t dsb = with_ds ? attn_ds_bytes(B, S, Hq) : 0;
    a.ds = dsb ? reinterpret_cast<uint16_t*>(p) : nullptr;
    a.ds_ld = dsb ? (int64_t(S) + 127) / 128 * 128 : 0;
}

hipError_t attn_bwd(const AttnBwdArgs& a, hipStream_t s) {
    if (!attn_shape_ok(a.B, a.S, a.Hq, a.Hkv, a.hd, a.ld, a.ldo)) return hipErrorInvalidValue;
    if (a.ldd < int64_t(a.Hq + 2 * a.Hkv) * a.hd || (a.ldd & 7)) return hipErrorInvalidValue;
    if (!a.dsum || !a.do16 || !a.amax || !a.dqkv) return hipErrorInvalidValue;
    if (a.dqk32 && (a.ld32 < int64_t(a.Hq + a.Hkv) * a.hd || (a.ld32 & 3))) return hipErrorInvalidValue;
    const int64_t T = int64_t(a.B) * a.S;
    // the maxima and prep kernels index 16-byte chunks with 32 bits (with
    // room for a grid stride past the end)
    if (T * a.Hq * (a.hd / 8) >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    const int ns = attn_dkdv_splits(a.B, a.S, a.Hq, a.Hkv, a.hd, a.dpart ? a.dpart_elems : 0, a.splits);
    // the split reduction indexes with 32 bits (never reached: splits stop at 512 key-tile blocks)
    if (ns > 1 && T * (a.Hkv * a.hd / 2) >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    const int n_qt = (a.S + 127) / 128;
    const int n_kt = (a.S + 127) / 128;
    const int64_t nk = int64_t(n_kt) * a.B * a.Hkv * ns;
    const int kt_slow = nk <= 2048;
    const dim3 gq(unsigned(int64_t(n_qt) * a.B * a.Hq));
    const dim3 gk(static_cast<unsigned>(nk));
    const unsigned np = unsigned((T * a.Hq * (a.hd / 8) + 255) / 256);
    // maxima: one pass of AMAX_U loads per lane where 2048 blocks (eight per
    // CU) cover the tensors, else 2048 blocks striding over their parts
    const int64_t ck_do = T * a.Hq * a.hd / 8, ck_v = T * a.Hkv * a.hd / 8, per_block = 256 * AMAX_U;
    const int nb_v = int(std::min<int64_t>(256, (ck_v + per_block - 1) / per_block));
    const int nb_do = int(std::min<int64_t>(2048 - nb_v, (ck_do + per_block - 1) / per_block));
    if (!a.amax_ready) {
        const hipError_t e = fill_zero(a.amax, ATTN_AMAX_BYTES, s);
        if (e != hipSuccess) return e;
    }
    // stored-dS form: dS must cover every key row and 128-query block
    const bool use_ds = a.ds != nullptr;
    if (use_ds && (a.ds_ld < (int64_t(a.S) + 127) / 128 * 128 || (a.ds_ld & 127))) return hipErrorInvalidValue;
    auto run = [&](auto hd_) {
        constexpr int HD = decltype(hd_)::value;
        if (!a.amax_ready) attn_amax_k<HD><<<nb_do + nb_v, 256, 0, s>>>(a, nb_do);
        attn_prep_k<HD><<<np, 256, 0, s>>>(a);
        if (!use_ds) attn_dq_k<HD><<<gq, 256, 0, s>>>(a, n_qt, n_qt <= 256);
        attn_dkdv_k<HD><<<gk, 512, 0, s>>>(a, n_kt, ns, kt_slow);
        if (use_ds) attn_dq_ds_k<HD><<<gq, 256, 0, s>>>(a, n_qt, n_qt <= 256);
    };
    if (a.hd == 128) run(std::integral_constant<int, 128>{});
    else run(std::integral_constant<int, 64>{});
    if (ns > 1) {
        const int64_t n4 = T * (a.Hkv * a.hd / 2);
        if (a.rope_tab) attn_dkdv_reduce_rot_k<<<unsigned((n4 / 2 + 255) / 256), 256, 0, s>>>(a, ns);
        else attn_dkdv_reduce_k<<<unsigned((n4 + 255) / 256), 256, 0, s>>>(a, ns);
    }
    return hipGetLastError();
}

}  // namespace mt
