// Memory-bound kernels of the decoder block on gfx950: RMSNorm forward and
// backward, rotary embedding, SwiGLU forward and backward, the LM-head
// cross-entropy, and small conversions.  All read and write bf16 in 16-byte
// vectors (8 elements per lane), keep statistics in fp32 and reduce in a
// fixed order, so every result is bit-reproducible run to run.
#include <mutex>

#include "kcommon.h"
#include "kernels.h"

namespace mt {
namespace {

// ------------------------------------------------------------- RMSNorm ----
// The input of a norm is bf16 (layer inputs) or fp32 (the residual stream
// inside a layer); eight elements at a time either way.
__device__ __forceinline__ void load8(const uint16_t* __restrict__ row, int c, float* f) {
    unpack8(reinterpret_cast<const uint4*>(row)[c], f);
}
__device__ __forceinline__ void load8(const float* __restrict__ row, int c, float* f) {
    const float4 a = reinterpret_cast<const float4*>(row)[2 * c];
    const float4 b = reinterpret_cast<const float4*>(row)[2 * c + 1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// One wave per row, four rows per 256-thread block.  The row stays in
// registers (CPL 8-element chunks per lane) between the sum of squares and
// the scaling, so it is read from memory once; all of a lane's loads are
// issued before the first is used.
template <class TX, int CPL>
__global__ __launch_bounds__(256) void rmsnorm_fwd_k(const TX* __restrict__ x,
                                                     const uint4* __restrict__ gamma,
                                                     uint4* __restrict__ n, uint4* __restrict__ n16,
                                                     float* __restrict__ rstd, int T, int d, float eps,
                                                     uint32_t* __restrict__ ovf, uint4* __restrict__ clear) {
    if (clear && blockIdx.x == 0)  // words the caller needs zeroed before later kernels of the stream
        for (int i = threadIdx.x; i < int(ATTN_AMAX_BYTES / 16); i += 256) clear[i] = make_uint4(0, 0, 0, 0);
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= T) return;
    const int nv = d >> 3;
    const TX* xr = x + int64_t(row) * d;
    float f[CPL][8];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = lane + 64 * k;
        if (c < nv) load8(xr, c, f[k]);
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k)
        if (lane + 64 * k < nv) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += f[k][e] * f[k][e];
        }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / float(d) + eps);
    uint4* nr = n + int64_t(row) * nv;
    uint4* nh = n16 ? n16 + int64_t(row) * nv : nullptr;
    uint32_t nov = 0;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = lane + 64 * k;
        if (c < nv) {
            float g[8];
            unpack8(gamma[c], g);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[k][e] = (f[k][e] * r) * g[e];
            nr[c] = pack8(f[k]);
            if (nh) nh[c] = pack8h_sat(f[k], nov);
        }
    }
    count_ovf(ovf, nov);
    if (lane == 0) rstd[row] = r;
}

// Backward.  Block b (four waves) takes the rows [T b / nb, T (b+1) / nb),
// its waves interleaved (wave w: rows r0 + w, r0 + w + 4, ...).  A wave keeps
// one row's dn, x and residual chunks in registers (every load issued before
// the first use), forms the row's dot product with a wave reduction, writes
// dx and accumulates the gain gradient of its lane's columns in fp32
// registers; gamma sits in LDS.  The block's four waves then add their sums
// in LDS in wave order into one partial row per block, and dgamma_reduce sums
// the blocks' rows in block order: the order is fixed, so results are
// bit-reproducible.  At most RMS_BWD_MAX_BLOCKS blocks (several per CU, so
// that the loads of one wave overlap the arithmetic of others), and at most
// 4M partial floats.
constexpr int RMS_BWD_MAX_BLOCKS = 512;

__device__ __forceinline__ void load_raw(const uint16_t* __restrict__ row, int c, uint4 (&v)[2]) {
    v[0] = reinterpret_cast<const uint4*>(row)[c];
}
__device__ __forceinline__ void load_raw(const float* __restrict__ row, int c, uint4 (&v)[2]) {
    v[0] = reinterpret_cast<const uint4*>(row)[2 * c];
    v[1] = reinterpret_cast<const uint4*>(row)[2 * c + 1];
}
__device__ __forceinline__ void unpack_raw(const uint4 (&v)[2], float* f, uint16_t) { unpack8(v[0], f); }
__device__ __forceinline__ void unpack_raw(const uint4 (&v)[2], float* f, float) {
    const float4 a = __builtin_bit_cast(float4, v[0]), b = __builtin_bit_cast(float4, v[1]);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

template <int NCL, class TX>
__global__ __launch_bounds__(256) void rmsnorm_bwd_k(const uint4* __restrict__ dn,
                                                     const TX* __restrict__ x,
                                                     const uint4* __restrict__ gamma,
                                                     const float* __restrict__ rstd,
                                                     const uint4* __restrict__ resid,
                                                     uint4* __restrict__ dx,
                                                     float* __restrict__ partial, int T, int d) {
    __shared__ uint4 gs[64 * NCL];     // gamma
    __shared__ float red[512 * NCL];   // the block's gain-gradient row
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nv = d >> 3;
    for (int c = threadIdx.x; c < nv; c += 256) gs[c] = gamma[c];
    __syncthreads();
    const int nb = gridDim.x;
    const int r0 = int(int64_t(T) * blockIdx.x / nb), r1 = int(int64_t(T) * (blockIdx.x + 1) / nb);
    float dg[NCL][8];
#pragma unroll
    for (int j = 0; j < NCL; ++j)
#pragma unroll
        for (int k = 0; k < 8; ++k) dg[j][k] = 0.f;
    for (int row = r0 + wave; row < r1; row += 4) {
        const float r = rstd[row];
        const uint4* dnr = dn + int64_t(row) * nv;
        const TX* xr = x + int64_t(row) * d;
        const uint4* rr_ = resid ? resid + int64_t(row) * nv : nullptr;
        // the residual's loads go out with the others up to 7 chunks per lane
        // (d <= 3584: 209 / 229 VGPRs for bf16 / fp32 x, still two waves per
        // SIMD; one memory round trip per row instead of two, 52.8 -> 50.9 and
        // 65.5 -> 60.7 us at T 8192, d 3584); wider rows load it after the
        // row's reduction, keeping the registers below 256
        constexpr bool EARLY_Q = NCL <= 7;
        uint4 a[NCL], q[NCL], xv[NCL][2];
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
            const int c = lane + 64 * j;
            if (c < nv) {
                a[j] = dnr[c];
                load_raw(xr, c, xv[j]);
                if (EARLY_Q && rr_) q[j] = rr_[c];
            }
        }
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
            const int c = lane + 64 * j;
            if (c < nv) {
                float av[8], xf[8], g8[8];
                unpack8(a[j], av);
                unpack_raw(xv[j], xf, TX());
                unpack8(gs[c], g8);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float nh = xf[k] * r;
                    dot += (av[k] * g8[k]) * nh;
                    dg[j][k] += av[k] * nh;
                }
            }
        }
        dot = wave_sum(dot) / float(d);
        // Keep only the packed row in registers across the reduction: the
        // unpacked values are formed again below (a few bit operations)
        // instead of being held, which would double the registers per row.
        auto opaque = [](uint4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); };
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
            opaque(a[j]);
            opaque(xv[j][0]);
            if constexpr (sizeof(TX) == 4) opaque(xv[j][1]);
        }
        if (!EARLY_Q && rr_) {
#pragma unroll
            for (int j = 0; j < NCL; ++j) {
                const int c = lane + 64 * j;
                if (c < nv) q[j] = rr_[c];
            }
        }
        uint4* dxr = dx + int64_t(row) * nv;
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
            const int c = lane + 64 * j;
            if (c < nv) {
                float av[8], xf[8], g8[8], o[8], qv[8];
                unpack8(a[j], av);
                unpack_raw(xv[j], xf, TX());
                unpack8(gs[c], g8);
                if (rr_) unpack8(q[j], qv);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float nh = xf[k] * r;
                    o[k] = r * ((av[k] * g8[k]) - nh * dot);
                    if (rr_) o[k] += qv[k];
                }
                dxr[c] = pack8(o);
            }
        }
    }
    // the waves' gain gradients, added in wave order
#pragma unroll 1
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int j = 0; j < NCL; ++j) {
                const int c = lane + 64 * j;
                if (c < nv) {
#pragma unroll
                    for (int k = 0; k < 8; ++k) red[c * 8 + k] = (w == 0 ? 0.f : red[c * 8 + k]) + dg[j][k];
                }
            }
        }
        __syncthreads();
    }
    float* pr = partial + int64_t(blockIdx.x) * d;
    for (int i = threadIdx.x; i < d; i += 256) pr[i] = red[i];
}

// 64 columns per block, 16 waves: wave w sums partial rows w, w+16, ... of
// its lane's column (coalesced 256-byte row segments), then wave 0 adds the
// 16 sums in wave order: a fixed order, so the result is deterministic.
__global__ __launch_bounds__(1024) void dgamma_reduce_k(const float* __restrict__ partial, int nrows, int d,
                                                        uint16_t* __restrict__ dgamma) {
    __shared__ float red[16][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + lane;
    float s = 0.f;
    if (c < d)
#pragma unroll 8
        for (int r = w; r < nrows; r += 16) s += partial[int64_t(r) * d + c];
    red[w][lane] = s;
    __syncthreads();
    if (w == 0 && c < d) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) t += red[i][lane];
        dgamma[c] = f2bf(t);
    }
}

// ---------------------------------------------------------------- RoPE ----
__global__ void rope_table_k(float2* tab, int S, int half, int hd, double base) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= int64_t(S) * half) return;
    const int s = int(i / half), e = int(i % half);
    const double th = double(s) * pow(base, -2.0 * double(e) / double(hd));
    tab[i] = make_float2(float(cos(th)), float(sin(th)));
}

// One thread rotates 8 pairs (e..e+7, e+half..e+half+7) of one head.
__global__ void rope_apply_k(uint16_t* __restrict__ qkv, int64_t ld, const float2* __restrict__ tab,
                             int T, int S, int nh, int hd, int dir) {
    const int half = hd >> 1;
    const int per_head = half >> 3;
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= int64_t(T) * nh * per_head) return;
    const int e8 = int(i % per_head);
    const int64_t th = i / per_head;
    const int h = int(th % nh);
    const int t = int(th / nh);
    const int s = t % S;
    uint16_t* base = qkv + int64_t(t) * ld + int64_t(h) * hd + e8 * 8;
    uint4* plo = reinterpret_cast<uint4*>(base);
    uint4* phi = reinterpret_cast<uint4*>(base + half);
    float lo[8], hi[8], ol[8], oh[8];
    unpack8(*plo, lo);
    unpack8(*phi, hi);
    const float2* tr = tab + int64_t(s) * half + e8 * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float2 cs = tr[k];
        const float sn = dir > 0 ? cs.y : -cs.y;
        ol[k] = lo[k] * cs.x - hi[k] * sn;
        oh[k] = hi[k] * cs.x + lo[k] * sn;
    }
    *plo = pack8(ol);
    *phi = pack8(oh);
}

// Rotation of the fp32 input's first nrot heads, one thread per 8 pairs
// (e..e+7, e+half..e+half+7) of one head, written as bf16.
__global__ void rope_f32_bf16_k(const float* __restrict__ in, int64_t ldin, uint16_t* __restrict__ out,
                                int64_t ldout, const float2* __restrict__ tab, int T, int S, int nrot, int hd,
                                int dir) {
    const int half = hd >> 1, per_head = half >> 3;
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= int64_t(T) * nrot * per_head) return;
    const int e8 = int(i % per_head);
    const int64_t th = i / per_head;
    const int h = int(th % nrot);
    const int t = int(th / nrot);
    const int s = t % S;
    const float* src = in + int64_t(t) * ldin + int64_t(h) * hd + e8 * 8;
    float lo[8], hi[8], ol[8], oh[8];
    *reinterpret_cast<float4*>(lo) = reinterpret_cast<const float4*>(src)[0];
    *reinterpret_cast<float4*>(lo + 4) = reinterpret_cast<const float4*>(src)[1];
    *reinterpret_cast<float4*>(hi) = reinterpret_cast<const float4*>(src + half)[0];
    *reinterpret_cast<float4*>(hi + 4) = reinterpret_cast<const float4*>(src + half)[1];
    const float2* tr = tab + int64_t(s) * half + e8 * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float2 cs = tr[k];
        const float sn = dir > 0 ? cs.y : -cs.y;
        ol[k] = lo[k] * cs.x - hi[k] * sn;
        oh[k] = hi[k] * cs.x + lo[k] * sn;
    }
    uint16_t* dst = out + int64_t(t) * ldout + int64_t(h) * hd + e8 * 8;
    *reinterpret_cast<uint4*>(dst) = pack8(ol);
    *reinterpret_cast<uint4*>(dst + half) = pack8(oh);
}

// Eight fp16 in a uint4 rounded to eight bf16 (RNE).
__device__ __forceinline__ uint4 h8_to_bf8(const uint4& v) {
    auto c = [](uint32_t w) {
        return uint32_t(f2bf(h2f(uint16_t(w & 0xFFFFu)))) | (uint32_t(f2bf(h2f(uint16_t(w >> 16)))) << 16);
    };
    return make_uint4(c(v.x), c(v.y), c(v.z), c(v.w));
}

// Rotary embedding on the fp32 output of the QKV projection, written as the
// fp16 operands of attention (q and k rotated, v as it is), each value
// saturated and counted by the fp16 range guard.  outb (optional) receives
// the same fp16 values rounded to bf16, for the gradient products of the
// attention backward (bf16 MFMA): the operands the kernels that stage
// through registers would form themselves.
__global__ void qkv_rope_cvt_k(const float* __restrict__ in, int64_t ldin, uint16_t* __restrict__ out,
                               int64_t ldout, uint16_t* __restrict__ outb, int64_t ldb,
                               const float2* __restrict__ tab, int T, int S, int nrot, int nall, int hd,
                               uint32_t* __restrict__ ovf, uint32_t* __restrict__ vmax) {
    const int half = hd >> 1, per_head = half >> 3;
    float vm = 0.f;  // max |v| of this lane's (fp16) values
    const int64_t n_rot_items = int64_t(T) * nrot * per_head;
    const int64_t n_v_items = int64_t(T) * (nall - nrot) * (hd >> 3);
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t nov = 0;
    if (i < n_rot_items) {
        const int e8 = int(i % per_head);
        const int64_t th = i / per_head;
        const int h = int(th % nrot);
        const int t = int(th / nrot);
        const int s = t % S;
        const float* src = in + int64_t(t) * ldin + int64_t(h) * hd + e8 * 8;
        float lo[8], hi[8], ol[8], oh[8];
        const float4* s4 = reinterpret_cast<const float4*>(src);
        const float4* h4 = reinterpret_cast<const float4*>(src + half);
        *reinterpret_cast<float4*>(lo) = s4[0];
        *reinterpret_cast<float4*>(lo + 4) = s4[1];
        *reinterpret_cast<float4*>(hi) = h4[0];
        *reinterpret_cast<float4*>(hi + 4) = h4[1];
        const float2* tr = tab + int64_t(s) * half + e8 * 8;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float2 cs = tr[k];
            ol[k] = lo[k] * cs.x - hi[k] * cs.y;
            oh[k] = hi[k] * cs.x + lo[k] * cs.y;
        }
        uint16_t* dst = out + int64_t(t) * ldout + int64_t(h) * hd + e8 * 8;
        const uint4 hl = pack8h_sat(ol, nov), hh = pack8h_sat(oh, nov);
        *reinterpret_cast<uint4*>(dst) = hl;
        *reinterpret_cast<uint4*>(dst + half) = hh;
        if (outb) {
            uint16_t* db = outb + int64_t(t) * ldb + int64_t(h) * hd + e8 * 8;
            *reinterpret_cast<uint4*>(db) = h8_to_bf8(hl);
            *reinterpret_cast<uint4*>(db + half) = h8_to_bf8(hh);
        }
    } else if (i < n_rot_items + n_v_items) {
        const int64_t j = i - n_rot_items;
        const int vw = (nall - nrot) * hd;
        const int c8 = int(j % (vw >> 3));
        const int t = int(j / (vw >> 3));
        const int64_t col = int64_t(nrot) * hd + c8 * 8;
        const float* src = in + int64_t(t) * ldin + col;
        float f[8];
        *reinterpret_cast<float4*>(f) = reinterpret_cast<const float4*>(src)[0];
        *reinterpret_cast<float4*>(f + 4) = reinterpret_cast<const float4*>(src)[1];
        const uint4 h8 = pack8h_sat(f, nov);
        *reinterpret_cast<uint4*>(out + int64_t(t) * ldout + col) = h8;
        if (outb) *reinterpret_cast<uint4*>(outb + int64_t(t) * ldb + col) = h8_to_bf8(h8);
        if (vmax) {
            float g[8];
            unpack8h(h8, g);
#pragma unroll
            for (int k = 0; k < 8; ++k) vm = fmaxf(vm, fabsf(g[k]));
        }
    }
    count_ovf(ovf, nov);
    if (vmax) {  // uniform: every thread of the block takes part; one atomic max per block
        __shared__ float wm[4];
        vm = wave_max(vm);
        if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = vm;
        __syncthreads();
        if (threadIdx.x == 0) {
            const float m = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
            if (m > 0.f)
                atomicMax(vmax + ATTN_AMAX_V_OFFSET + (blockIdx.x % ATTN_AMAX_PARTS) * ATTN_AMAX_LINE,
                          __float_as_uint(m));
        }
    }
}

__global__ void bf16_to_f16_k(const uint4* __restrict__ in, uint4* __restrict__ out, int64_t n8,
                              uint32_t* __restrict__ ovf) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    float f[8];
    unpack8(in[i], f);
    uint32_t nov = 0;
    out[i] = pack8h_sat(f, nov);
    count_ovf(ovf, nov);
}

// -------------------------------------------------------------- SwiGLU ----
__device__ __forceinline__ float sigm(float z) { return 1.0f / (1.0f + expf(-z)); }

__global__ void swiglu_fwd_k(const uint4* __restrict__ gu, uint4* __restrict__ m, int T, int F) {
    const int fv = F >> 3;
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= int64_t(T) * fv) return;
    const int64_t t = i / fv;
    const int c = int(i % fv);
    float a[8], b[8], o[8];
    unpack8(gu[t * 2 * fv + c], a);
    unpack8(gu[t * 2 * fv + fv + c], b);
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = (a[k] * sigm(a[k])) * b[k];
    m[t * fv + c] = pack8(o);
}

__global__ void swiglu_bwd_k(const uint4* __restrict__ dm, const uint4* __restrict__ gu,
                             uint4* __restrict__ dgu, int T, int F) {
    const int fv = F >> 3;
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= int64_t(T) * fv) return;
    const int64_t t = i / fv;
    const int c = int(i % fv);
    float a[8], b[8], g[8], da[8], db[8];
    unpack8(gu[t * 2 * fv + c], a);
    unpack8(gu[t * 2 * fv + fv + c], b);
    unpack8(dm[t * fv + c], g);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float s = sigm(a[k]);
        db[k] = g[k] * (a[k] * s);
        da[k] = g[k] * b[k] * (s * (1.0f + a[k] * (1.0f - s)));
    }
    dgu[t * 2 * fv + c] = pack8(da);
    dgu[t * 2 * fv + fv + c] = pack8(db);
}

// ------------------------------------------------------- Cross-entropy ----
// One 256-thread block per token row.
__global__ __launch_bounds__(256) void ce_k(const float* __restrict__ logits,
                                            const int32_t* __restrict__ labels,
                                            float* __restrict__ loss_rows,
                                            uint16_t* __restrict__ dlogits, int V, float inv_T) {
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const float* x = logits + int64_t(row) * V;
    const float4* x4 = reinterpret_cast<const float4*>(x);
    const int nv4 = V >> 2;
    // Pass 1: running (max, sum of exp) per thread, then a fixed-order merge.
    float mx = -INFINITY, sm = 0.f;
    for (int c = tid; c < nv4; c += 256) {
        const float4 v = x4[c];
        const float vm = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
        if (vm > mx) { sm *= expf(mx - vm); mx = vm; }
        sm += expf(v.x - mx) + expf(v.y - mx) + expf(v.z - mx) + expf(v.w - mx);
    }
    __shared__ float smx[256], ssm[256];
    smx[tid] = mx;
    ssm[tid] = sm;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) {
            const float m1 = smx[tid], m2 = smx[tid + o];
            const float m = fmaxf(m1, m2);
            const float s = (m1 == -INFINITY ? 0.f : ssm[tid] * expf(m1 - m)) +
                            (m2 == -INFINITY ? 0.f : ssm[tid + o] * expf(m2 - m));
            smx[tid] = m;
            ssm[tid] = s;
        }
        __syncthreads();
    }
    const float lse = smx[0] + logf(ssm[0]);
    const int lab = labels[row];
    const bool lab_ok = lab >= 0 && lab < V;
    if (tid == 0) loss_rows[row] = lab_ok ? lse - x[lab] : NAN;
    // Pass 2: dlogits = (softmax - onehot) / T in bf16, 4 per thread-step.
    uint2* d2 = reinterpret_cast<uint2*>(dlogits + int64_t(row) * V);
    for (int c = tid; c < nv4; c += 256) {
        const float4 v = x4[c];
        float p0 = expf(v.x - lse), p1 = expf(v.y - lse), p2 = expf(v.z - lse), p3 = expf(v.w - lse);
        const int b = c * 4;
        if (lab == b) p0 -= 1.f;
        if (lab == b + 1) p1 -= 1.f;
        if (lab == b + 2) p2 -= 1.f;
        if (lab == b + 3) p3 -= 1.f;
        d2[c] = make_uint2(pack2(p0 * inv_T, p1 * inv_T), pack2(p2 * inv_T, p3 * inv_T));
    }
}

// Cross-entropy over vocabulary chunks (the LM head streamed in row chunks
// of E_out).  Forward, per row: the chunk's (max, sum of exp) merged into the
// running (m, l) of the chunks before it, and the label's logit picked up by
// the chunk that holds it.  After the last chunk, LSE = m + log l and the
// row's loss LSE - z.  Backward: dlogits = (exp(x - LSE) - onehot) / T.
__global__ __launch_bounds__(256) void ce_chunk_fwd_k(const float* __restrict__ logits,
                                                      const int32_t* __restrict__ labels, int Vc, int v0,
                                                      int first, float* __restrict__ m, float* __restrict__ l,
                                                      float* __restrict__ z) {
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const float* x = logits + int64_t(row) * Vc;
    const float4* x4 = reinterpret_cast<const float4*>(x);
    const int nv4 = Vc >> 2;
    float mx = -INFINITY, sm = 0.f;
    for (int c = tid; c < nv4; c += 256) {
        const float4 v = x4[c];
        const float vm = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
        if (vm > mx) { sm *= expf(mx - vm); mx = vm; }
        sm += expf(v.x - mx) + expf(v.y - mx) + expf(v.z - mx) + expf(v.w - mx);
    }
    __shared__ float smx[256], ssm[256];
    smx[tid] = mx;
    ssm[tid] = sm;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) {
            const float m1 = smx[tid], m2 = smx[tid + o];
            const float mm = fmaxf(m1, m2);
            const float s = (m1 == -INFINITY ? 0.f : ssm[tid] * expf(m1 - mm)) +
                            (m2 == -INFINITY ? 0.f : ssm[tid + o] * expf(m2 - mm));
            smx[tid] = mm;
            ssm[tid] = s;
        }
        __syncthreads();
    }
    if (tid == 0) {
        float M = first ? -INFINITY : m[row], L = first ? 0.f : l[row];
        const float cm = smx[0], cs = ssm[0];
        const float nm = fmaxf(M, cm);
        L = (M == -INFINITY ? 0.f : L * expf(M - nm)) + (cm == -INFINITY ? 0.f : cs * expf(cm - nm));
        m[row] = nm;
        l[row] = L;
        const int lab = labels[row] - v0;
        if (lab >= 0 && lab < Vc) z[row] = x[lab];
    }
}

__global__ void ce_chunk_final_k(const float* __restrict__ m, const float* __restrict__ l,
                                 const float* __restrict__ z, float* __restrict__ lse,
                                 float* __restrict__ loss_rows, int T) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const float s = m[t] + logf(l[t]);
    lse[t] = s;
    loss_rows[t] = s - z[t];
}

__global__ __launch_bounds__(256) void ce_chunk_bwd_k(const float* __restrict__ logits,
                                                      const int32_t* __restrict__ labels,
                                                      const float* __restrict__ lse, int Vc, int v0,
                                                      uint16_t* __restrict__ dlogits, float inv_T) {
    const int row = blockIdx.x;
    const float4* x4 = reinterpret_cast<const float4*>(logits + int64_t(row) * Vc);
    uint2* d2 = reinterpret_cast<uint2*>(dlogits + int64_t(row) * Vc);
    const float s = lse[row];
    const int lab = labels[row] - v0;
    for (int c = threadIdx.x; c < (Vc >> 2); c += 256) {
        const float4 v = x4[c];
        float p0 = expf(v.x - s), p1 = expf(v.y - s), p2 = expf(v.z - s), p3 = expf(v.w - s);
        const int b = c * 4;
        if (lab == b) p0 -= 1.f;
        if (lab == b + 1) p1 -= 1.f;
        if (lab == b + 2) p2 -= 1.f;
        if (lab == b + 3) p3 -= 1.f;
        d2[c] = make_uint2(pack2(p0 * inv_T, p1 * inv_T), pack2(p2 * inv_T, p3 * inv_T));
    }
}

__global__ __launch_bounds__(256) void mean_reduce_k(const float* __restrict__ x, float* out, int n) {
    __shared__ float sh[256];
    float s = 0.f;
    for (int i = threadIdx.x; i < n; i += 256) s += x[i];
    sh[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = sh[0] / float(n);
}

__global__ void f32_to_bf16_k(const float4* __restrict__ x, uint2* __restrict__ y, int64_t n4) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const float4 v = x[i];
    y[i] = make_uint2(pack2(v.x, v.y), pack2(v.z, v.w));
}

// 16-bit element e (0..7, compile-time after unrolling) of a uint4.
__device__ __forceinline__ uint32_t h16of(const uint4& v, int e) {
    const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// dst[c][r] = src[r][c] for bf16 (any 16-bit) matrices; with F16_TO_BF16 the
// source holds fp16 and every element is rounded to bf16 on the way (RNE).  One wave per
// 64 x 64 tile; lane (tx, ty) = (lane % 8, lane / 8) moves the 8 x 8 block at
// rows 8 ty.., columns 8 tx..: eight 16-byte row loads, a transpose in
// registers, eight 16-byte row stores.  Eight lanes cover 128 contiguous
// bytes of a source row on load and of a destination row on store.  VEC: rows
// of both matrices start 16-byte aligned; blocks that cross the matrix edge,
// and every block when !VEC, go element by element.
__device__ __forceinline__ uint32_t h2bf(uint32_t h) { return f2bf(h2f(uint16_t(h))); }

template <bool VEC, bool F16_TO_BF16>
__global__ __launch_bounds__(256) void transpose16_k(const uint16_t* __restrict__ src, int64_t lds,
                                                     uint16_t* __restrict__ dst, int64_t ldd, int R, int C,
                                                     int tiles_c, int64_t n_tiles) {
    const int lane = threadIdx.x & 63;
    const int64_t tile = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (tile >= n_tiles) return;
    const int r = int(tile / tiles_c) * 64 + 8 * (lane >> 3);
    const int c = int(tile % tiles_c) * 64 + 8 * (lane & 7);
    if (r >= R || c >= C) return;
    if (VEC && r + 8 <= R && c + 8 <= C) {
        uint4 in[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) in[i] = *reinterpret_cast<const uint4*>(src + int64_t(r + i) * lds + c);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                uint32_t a = h16of(in[i], j), b = h16of(in[i + 1], j);
                if constexpr (F16_TO_BF16) { a = h2bf(a); b = h2bf(b); }
                w[i >> 1] = a | (b << 16);
            }
            *reinterpret_cast<uint4*>(dst + int64_t(c + j) * ldd + r) = make_uint4(w[0], w[1], w[2], w[3]);
        }
        return;
    }
    const int nr = min(8, R - r), nc = min(8, C - c);
    for (int i = 0; i < nr; ++i)
        for (int j = 0; j < nc; ++j) {
            const uint16_t v = src[int64_t(r + i) * lds + c + j];
            dst[int64_t(c + j) * ldd + r + i] = F16_TO_BF16 ? uint16_t(h2bf(v)) : v;
        }
}

__global__ void fill_zero_k(uint4* __restrict__ p, int64_t n16) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n16) p[i] = make_uint4(0, 0, 0, 0);
}

__global__ void fill_u32_k(uint4* __restrict__ p, int64_t n16, uint32_t v) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += int64_t(gridDim.x) * blockDim.x)
        p[i] = make_uint4(v, v, v, v);
}

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline unsigned blocks(int64_t n, int b) { return unsigned((n + b - 1) / b); }

}  // namespace

hipError_t rmsnorm_fwd(const void* x, bool x_f32, const uint16_t* gamma, uint16_t* n, uint16_t* n_f16,
                       float* rstd, int T, int d, float eps, hipStream_t s, uint32_t* ovf, uint32_t* clear_amax) {
    if (T < 0 || d <= 0 || (d & 7) || !al16(x) || !al16(gamma) || !al16(n) || (n_f16 && !al16(n_f16)))
        return hipErrorInvalidValue;
    if (clear_amax && !al16(clear_amax)) return hipErrorInvalidValue;
    if (T == 0) return clear_amax ? fill_zero(clear_amax, ATTN_AMAX_BYTES, s) : hipSuccess;
    uint4* clr = reinterpret_cast<uint4*>(clear_amax);
    const uint4* g = reinterpret_cast<const uint4*>(gamma);
    uint4* nv = reinterpret_cast<uint4*>(n);
    uint4* nh = reinterpret_cast<uint4*>(n_f16);
    // chunks of 8 per lane: d / 512 rounded up to a power of two (d <= 8192)
    const int need = (d / 8 + 63) / 64;
    auto run = [&](auto cpl_) {
        constexpr int CPL = decltype(cpl_)::value;
        if (x_f32)
            rmsnorm_fwd_k<float, CPL><<<blocks(T, 4), 256, 0, s>>>(static_cast<const float*>(x), g, nv, nh, rstd, T, d,
                                                                   eps, ovf, clr);
        else
            rmsnorm_fwd_k<uint16_t, CPL><<<blocks(T, 4), 256, 0, s>>>(static_cast<const uint16_t*>(x), g, nv, nh, rstd,
                                                                      T, d, eps, ovf, clr);
    };
    if (need <= 1) run(std::integral_constant<int, 1>{});
    else if (need <= 2) run(std::integral_constant<int, 2>{});
    else if (need <= 4) run(std::integral_constant<int, 4>{});
    else if (need <= 8) run(std::integral_constant<int, 8>{});
    else if (need <= 16) run(std::integral_constant<int, 16>{});
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t rope_f32_to_bf16(const float* in, int64_t ldin, uint16_t* out, int64_t ldout, const float2* tab, int T,
                            int S, int n_rot_heads, int hd, int dir, hipStream_t s) {
    if (T < 0 || S <= 0 || n_rot_heads < 0 || (hd & 15) || (ldin & 3) || (ldout & 7) ||
        ldin < int64_t(n_rot_heads) * hd || ldout < int64_t(n_rot_heads) * hd || !al16(in) || !al16(out) || !tab)
        return hipErrorInvalidValue;
    const int64_t n = int64_t(T) * n_rot_heads * (hd / 16);
    if (n == 0) return hipSuccess;
    rope_f32_bf16_k<<<blocks(n, 256), 256, 0, s>>>(in, ldin, out, ldout, tab, T, S, n_rot_heads, hd, dir);
    return hipGetLastError();
}

hipError_t qkv_rope_cvt(const float* in, int64_t ldin, uint16_t* out, int64_t ldout, uint16_t* outb, int64_t ldb,
                        const float2* tab, int T, int S, int n_rot_heads, int n_heads, int hd, hipStream_t s,
                        uint32_t* ovf, uint32_t* vmax) {
    if (T < 0 || S <= 0 || n_rot_heads < 0 || n_heads < n_rot_heads || (hd & 15) || (ldin & 3) || (ldout & 7) ||
        ldin < int64_t(n_heads) * hd || ldout < int64_t(n_heads) * hd || !al16(in) || !al16(out))
        return hipErrorInvalidValue;
    if (outb && ((ldb & 7) || ldb < int64_t(n_heads) * hd || !al16(outb))) return hipErrorInvalidValue;
    if (T == 0) return hipSuccess;
    const int64_t n = int64_t(T) * n_rot_heads * (hd / 16) + int64_t(T) * (n_heads - n_rot_heads) * (hd / 8);
    qkv_rope_cvt_k<<<blocks(n, 256), 256, 0, s>>>(in, ldin, out, ldout, outb, ldb, tab, T, S, n_rot_heads, n_heads,
                                                   hd, ovf, vmax);
    return hipGetLastError();
}

hipError_t bf16_to_f16(const uint16_t* in, uint16_t* out, int64_t n, hipStream_t s, uint32_t* ovf) {
    if (n < 0 || (n & 7) || !al16(in) || !al16(out)) return hipErrorInvalidValue;
    if (n == 0) return hipSuccess;
    bf16_to_f16_k<<<blocks(n / 8, 256), 256, 0, s>>>(reinterpret_cast<const uint4*>(in),
                                                     reinterpret_cast<uint4*>(out), n / 8, ovf);
    return hipGetLastError();
}

static int rmsnorm_bwd_blocks(int T) { return std::max(1, std::min(T / 4 + (T % 4 != 0), RMS_BWD_MAX_BLOCKS)); }

int64_t rmsnorm_bwd_partial_elems(int T, int d) { return T <= 0 ? 0 : int64_t(rmsnorm_bwd_blocks(T)) * d; }

template <class TX>
static void rmsnorm_bwd_launch(int ncl, unsigned nb, const uint4* dn, const TX* x, const uint4* g,
                               const float* rstd, const uint4* resid, uint4* dx, float* partial, int T, int d,
                               hipStream_t s) {
    // chunks of 8 columns per lane: the exact count up to 8 (d <= 4096), else 16
    auto go = [&](auto n_) {
        rmsnorm_bwd_k<decltype(n_)::value, TX><<<nb, 256, 0, s>>>(dn, x, g, rstd, resid, dx, partial, T, d);
    };
    switch (ncl) {
        case 1: go(std::integral_constant<int, 1>{}); break;
        case 2: go(std::integral_constant<int, 2>{}); break;
        case 3: go(std::integral_constant<int, 3>{}); break;
        case 4: go(std::integral_constant<int, 4>{}); break;
        case 5: go(std::integral_constant<int, 5>{}); break;
        case 6: go(std::integral_constant<int, 6>{}); break;
        case 7: go(std::integral_constant<int, 7>{}); break;
        case 8: go(std::integral_constant<int, 8>{}); break;
        default: go(std::integral_constant<int, 16>{});
    }
}

hipError_t rmsnorm_bwd(const uint16_t* dn, const void* x, bool x_f32, const uint16_t* gamma,
                       const float* rstd, const uint16_t* resid, uint16_t* dx, uint16_t* dgamma,
                       float* partial, int T, int d, hipStream_t s) {
    if (T <= 0 || d <= 0 || (d & 7) || d > 8192) return hipErrorInvalidValue;
    if (!al16(dn) || !al16(x) || !al16(gamma) || !al16(dx) || (resid && !al16(resid)))
        return hipErrorInvalidValue;
    const unsigned nb = unsigned(rmsnorm_bwd_blocks(T));
    const int ncl = ((d >> 3) + 63) / 64;
    auto U = [](const uint16_t* p) { return reinterpret_cast<const uint4*>(p); };
    uint4* dxv = reinterpret_cast<uint4*>(dx);
    const uint4* rv = resid ? U(resid) : nullptr;
    if (x_f32)
        rmsnorm_bwd_launch<float>(ncl, nb, U(dn), static_cast<const float*>(x), U(gamma), rstd, rv, dxv, partial,
                                  T, d, s);
    else
        rmsnorm_bwd_launch<uint16_t>(ncl, nb, U(dn), static_cast<const uint16_t*>(x), U(gamma), rstd, rv, dxv,
                                     partial, T, d, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dgamma_reduce_k<<<(d + 63) / 64, 1024, 0, s>>>(partial, int(nb), d, dgamma);
    return hipGetLastError();
}

// ------------------------------------------ allocation-free entry ----
// The gain-gradient partials of rmsnorm_bwd in a file-scope device array:
// one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, looked up once
// per device with that device current.
static __device__ __align__(256) float scratch[RMSNORM_NOALLOC_FLOATS];

namespace {
std::mutex noalloc_mu;
float* noalloc_ptr[64] = {};
}  // namespace

hipError_t rmsnorm_bwd_noalloc(const uint16_t* dn, const void* x, bool x_f32, const uint16_t* gamma,
                               const float* rstd, const uint16_t* resid, uint16_t* dx, uint16_t* dgamma, int T, int d,
                               hipStream_t s) {
    if (T <= 0 || d <= 0 || (d & 7) || d > 8192) return hipErrorInvalidValue;
    if (rmsnorm_bwd_partial_elems(T, d) > RMSNORM_NOALLOC_FLOATS) return hipErrorInvalidValue;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    float* ptr;
    {
        std::lock_guard<std::mutex> lk(noalloc_mu);
        if (!noalloc_ptr[dev]) {
            void* p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            noalloc_ptr[dev] = static_cast<float*>(p);
        }
        ptr = noalloc_ptr[dev];
    }
    // Every partial row is written by rmsnorm_bwd_k before dgamma_reduce_k
    // reads it, so the buffer needs no clearing between calls.
    return rmsnorm_bwd(dn, x, x_f32, gamma, rstd, resid, dx, dgamma, ptr, T, d, s);
}

hipError_t rope_table(float2* tab, int S, int hd, float base, hipStream_t s) {
    if (S <= 0 || hd <= 0 || (hd & 15)) return hipErrorInvalidValue;
    const int half = hd / 2;
    rope_table_k<<<blocks(int64_t(S) * half, 256), 256, 0, s>>>(tab, S, half, hd, double(base));
    return hipGetLastError();
}

hipError_t rope_apply(uint16_t* qkv, int64_t ld, const float2* tab, int T, int S, int nh, int hd,
                      int dir, hipStream_t s) {
    if (T < 0 || S <= 0 || nh <= 0 || (hd & 15) || (ld & 7) || !al16(qkv)) return hipErrorInvalidValue;
    if (T == 0) return hipSuccess;
    const int64_t n = int64_t(T) * nh * (hd / 16);
    rope_apply_k<<<blocks(n, 256), 256, 0, s>>>(qkv, ld, tab, T, S, nh, hd, dir);
    return hipGetLastError();
}

hipError_t swiglu_fwd(const uint16_t* gu, uint16_t* m, int T, int F, hipStream_t s) {
    if (T < 0 || F <= 0 || (F & 7) || !al16(gu) || !al16(m)) return hipErrorInvalidValue;
    if (T == 0) return hipSuccess;
    swiglu_fwd_k<<<blocks(int64_t(T) * (F / 8), 256), 256, 0, s>>>(
        reinterpret_cast<const uint4*>(gu), reinterpret_cast<uint4*>(m), T, F);
    return hipGetLastError();
}

hipError_t swiglu_bwd(const uint16_t* dm, const uint16_t* gu, uint16_t* dgu, int T, int F,
                      hipStream_t s) {
    if (T < 0 || F <= 0 || (F & 7) || !al16(gu) || !al16(dm) || !al16(dgu)) return hipErrorInvalidValue;
    if (T == 0) return hipSuccess;
    swiglu_bwd_k<<<blocks(int64_t(T) * (F / 8), 256), 256, 0, s>>>(
        reinterpret_cast<const uint4*>(dm), reinterpret_cast<const uint4*>(gu),
        reinterpret_cast<uint4*>(dgu), T, F);
    return hipGetLastError();
}

hipError_t ce_fwd_bwd(const float* logits, const int32_t* labels, float* loss_rows,
                      uint16_t* dlogits, int Tc, int V, float inv_T, hipStream_t s) {
    if (Tc < 0 || V <= 0 || (V & 7) || !al16(logits) || !al16(dlogits)) return hipErrorInvalidValue;
    if (Tc == 0) return hipSuccess;
    ce_k<<<Tc, 256, 0, s>>>(logits, labels, loss_rows, dlogits, V, inv_T);
    return hipGetLastError();
}

hipError_t mean_reduce(const float* x, float* out, int n, hipStream_t s) {
    if (n <= 0) return hipErrorInvalidValue;
    mean_reduce_k<<<1, 256, 0, s>>>(x, out, n);
    return hipGetLastError();
}

hipError_t f32_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t s) {
    if (n < 0 || (n & 3) || !al16(x)) return hipErrorInvalidValue;
    if (n == 0) return hipSuccess;
    f32_to_bf16_k<<<blocks(n / 4, 256), 256, 0, s>>>(reinterpret_cast<const float4*>(x),
                                                     reinterpret_cast<uint2*>(y), n / 4);
    return hipGetLastError();
}

hipError_t ce_chunk_fwd(const float* logits, const int32_t* labels, int rows, int Vc, int v0, bool first, float* m,
                        float* l, float* z, hipStream_t s) {
    if (rows < 0 || Vc <= 0 || (Vc & 7) || !al16(logits)) return hipErrorInvalidValue;
    if (rows == 0) return hipSuccess;
    ce_chunk_fwd_k<<<rows, 256, 0, s>>>(logits, labels, Vc, v0, first ? 1 : 0, m, l, z);
    return hipGetLastError();
}

hipError_t ce_chunk_final(const float* m, const float* l, const float* z, float* lse, float* loss_rows, int T,
                          hipStream_t s) {
    if (T < 0) return hipErrorInvalidValue;
    if (T == 0) return hipSuccess;
    ce_chunk_final_k<<<blocks(T, 256), 256, 0, s>>>(m, l, z, lse, loss_rows, T);
    return hipGetLastError();
}

hipError_t ce_chunk_bwd(const float* logits, const int32_t* labels, const float* lse, int rows, int Vc, int v0,
                        uint16_t* dlogits, float inv_T, hipStream_t s) {
    if (rows < 0 || Vc <= 0 || (Vc & 7) || !al16(logits) || !al16(dlogits)) return hipErrorInvalidValue;
    if (rows == 0) return hipSuccess;
    ce_chunk_bwd_k<<<rows, 256, 0, s>>>(logits, labels, lse, Vc, v0, dlogits, inv_T);
    return hipGetLastError();
}

hipError_t transpose16(const uint16_t* src, int64_t lds, uint16_t* dst, int64_t ldd, int R, int C, hipStream_t s,
                       bool f16_to_bf16) {
    if (R < 0 || C < 0 || !src || !dst || lds < C || ldd < R) return hipErrorInvalidValue;
    if (R == 0 || C == 0) return hipSuccess;
    const int tiles_c = (C + 63) / 64;
    const int64_t n_tiles = int64_t((R + 63) / 64) * tiles_c;
    const int64_t nb = (n_tiles + 3) / 4;
    if (nb > INT32_MAX) return hipErrorInvalidValue;
    const bool vec = (lds % 8) == 0 && (ldd % 8) == 0 && al16(src) && al16(dst);
    auto go = [&](auto vec_, auto cvt_) {
        transpose16_k<decltype(vec_)::value, decltype(cvt_)::value>
            <<<unsigned(nb), 256, 0, s>>>(src, lds, dst, ldd, R, C, tiles_c, n_tiles);
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    if (vec) f16_to_bf16 ? go(T_{}, T_{}) : go(T_{}, F_{});
    else f16_to_bf16 ? go(F_{}, T_{}) : go(F_{}, F_{});
    return hipGetLastError();
}

hipError_t fill_u32(void* p, int64_t bytes, uint32_t pattern, hipStream_t s) {
    if (bytes < 0 || (bytes & 15) || !al16(p)) return hipErrorInvalidValue;
    if (bytes == 0) return hipSuccess;
    const int64_t n16 = bytes / 16;
    fill_u32_k<<<unsigned(std::min<int64_t>(4096, (n16 + 255) / 256)), 256, 0, s>>>(reinterpret_cast<uint4*>(p), n16,
                                                                                   pattern);
    return hipGetLastError();
}

hipError_t fill_zero(void* p, int64_t bytes, hipStream_t s) {
    if (bytes < 0 || (bytes & 15) || !al16(p)) return hipErrorInvalidValue;
    if (bytes == 0) return hipSuccess;
    fill_zero_k<<<blocks(bytes / 16, 256), 256, 0, s>>>(reinterpret_cast<uint4*>(p), bytes / 16);
    return hipGetLastError();
}

}  // namespace mt
