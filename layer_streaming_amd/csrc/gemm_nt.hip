// NT GEMM (C = A B^T, both operands k-contiguous) for gfx950 with the tile
// loads going straight from global memory into LDS.
//
// This is the layout of every forward projection of the decoder (fused QKV,
// O, fused gate|up, down, LM head).  Design:
//  * buffer_load_dwordx4 ... lds moves each 16-byte chunk from global memory
//    into LDS without passing through registers: no staging VGPRs and no LDS
//    store instructions.  One wave instruction fills 1 KB of LDS (64 lanes x
//    16 bytes, in lane order), i.e. 16 tile rows of 32 k; each lane fetches
//    the global chunk that the XOR swizzle places at its LDS slot;
//  * k-tiles of 32 in four LDS stages, loads issued three tiles ahead, so a
//    load has three tiles of MFMA work to arrive in; one barrier per tile,
//    whose wait counts only the loads of the tile about to be read;
//  * per block, buffer resources based at the block's first row bound the
//    reads: chunks past the last valid row, and k-chunks past K (given an
//    offset beyond the resource), read as zero, so edge tiles need no clamped
//    addresses or masks;
//  * fragments are double-buffered in registers: the LDS reads of the next
//    16-deep k-step are issued before the MFMAs of the current one, and the
//    last step of a tile runs its MFMAs after the barrier, behind the first
//    reads of the next tile;
//  * the MFMA takes the B fragment as its first operand, so a lane's
//    accumulator holds 4 consecutive output columns of one row;
//  * the epilogue passes the accumulators through LDS so that every store
//    instruction writes whole row segments (8 or 16 bytes per lane);
//  * large problems (from about half a 256 x 256 tile per CU) take a second form
//    of the main loop with 64-deep k-tiles in two stages (gemm_nt64_k below):
//    whole 128-byte rows per load request and half the barriers.  Measured
//    on MI355X at the 7B gate|up shape (8192 x 37888 x 3584, random bf16):
//    1215 TFLOP/s against 1111 for the 32-deep form with the LDS epilogue
//    and 1076 with stores straight from the accumulators.
#include <type_traits>

#include "kcommon.h"
#include "kernels.h"

namespace mt {
namespace {

// Build-time variants; the defaults are the faster ones as measured on
// MI355X with random bf16 operands (gate|up 8192 x 37888 x 3584): raised
// priority over the MFMA groups 1215 TFLOP/s vs 1143 without (1090 vs 1028
// in the 32-deep form); non-temporal C stores 741 (32-deep, direct stores);
// 4 x 2 waves instead of 2 x 4, all loads of a tile with one k-step, tile
// groups 4 or 16 deep: within 1-2% of the default.  Four waves of 128 x 128
// (one per SIMD) lose 4-6%.
#ifndef MT_NT_PRIO
#define MT_NT_PRIO 1      // 1: raise the wave's issue priority over its MFMA groups
#endif
#ifndef MT_NT_NTSTORE
#define MT_NT_NTSTORE 0   // 1: non-temporal epilogue stores (C does not stay in L2)
#endif
#ifndef MT_NT_STAGED
#define MT_NT_STAGED 1    // 1: the epilogue goes through LDS so that stores cover whole row segments
#endif
#ifndef MT_NT_K64
#define MT_NT_K64 1       // 1: 64-deep k-tiles in two stages for the large-tile shape
#endif
#ifndef MT_NT_BIG_MIN
// Fewest 256 x 256 tiles for the large-tile form.  Measured (K = 8192, bf16,
// TFLOP/s, 64-deep 256 x 256 against 32-deep 128 x 128): 64 tiles 467/748,
// 100 698/685 (540/658 at K = 2048), 121 828/648, 144 988/637, 196 1177/723,
// 252 1320/754: a grid that leaves some CUs idle still wins from about half
// the CUs up.
#define MT_NT_BIG_MIN 120
#endif
#ifndef MT_NT_ST8
#define MT_NT_ST8 1       // 1: bf16 epilogues store 8 columns (16 bytes) per lane
#endif
#ifndef MT_NT_L1
#define MT_NT_L1 -1       // 64-deep form: loads of a tile issued one k-step later (-1: half)
#endif
#ifndef MT_NT_GROUP
#define MT_NT_GROUP 8     // 64-deep form: tiles grouped this deep along M
#endif
#ifndef MT_NT_NW
#define MT_NT_NW 8        // waves of the 256 x 256 block
#endif
#ifndef MT_NT_WM
#define MT_NT_WM 2        // of which along M
#endif
#ifndef MT_GEMM_KMAJOR
#define MT_GEMM_KMAJOR 1  // 1: NN and TN products read k-major operands straight (256 x 256 grids)
#endif

typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int BK = 32;                 // k per tile; an LDS row is 64 bytes
constexpr uint32_t OOB = 0x80000000u;  // beyond every resource's extent

// Physical chunk (of four 16-byte chunks) of logical chunk c in LDS row r.
// The LDS serves a 128-bit read 16 lanes (256 bytes, all 64 banks) per
// cycle; 16 consecutive rows span four 256-byte lines, and mixing row bits
// 2..3 into the chunk gives them 16 distinct bank positions (measured: the
// bits-1..2 variant doubles the LDS cycles through conflicts).
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

// Buffer resource (gfx9 layout): base, stride 0, extent in bytes, and the
// default data-format word.  Reads at offsets >= extent return zero.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4_t r;
    r.x = int(uint32_t(a));
    r.y = int(uint32_t(a >> 32) & 0xFFFFu);
    r.z = int(bytes);
    r.w = 0x00020000;
    return r;
}

// 16 bytes per lane from the buffer at byte offset voff into LDS at
// lds_addr + 16 * lane.  Issued as inline assembly: the compiler then does
// not treat every later LDS read as a possible reader of this load (it cannot
// tell the stages apart) and does not insert waits for it; the kernel waits
// on vmcnt itself.
__device__ __forceinline__ void dma16(i32x4_t rs, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rs)
                 : "memory");
}

template <int V> struct IntC { static constexpr int value = V; };
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(IntC<B>{});
        static_for<B + 1, E>(f);
    }
}

template <int N>
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// Block barrier without the full memory fence of __syncthreads (which would
// also wait for the loads still in flight for later tiles); LDS reads done.
// The lgkmcnt(0) wait goes through the builtin (gfx9 encoding: vmcnt 63,
// expcnt 7, lgkmcnt 0) so that the compiler knows the earlier fragment reads
// have completed and adds no waits of its own after the barrier.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Loads of one operand's ROWS x 32 tile by NW waves: NI wave instructions
// each, instruction i of wave w covering tile rows 16*(i*NW + w) .. +15.
template <int ROWS, int NW>
struct DirectLoader {
    static constexpr int NI = ROWS / (16 * NW);
    static_assert(NI >= 1 && ROWS % (16 * NW) == 0, "tile rows must cover the waves");
    uint32_t off[NI];  // byte offset of the lane's chunk at k = 0
    int kk[NI];        // its first k within the tile

    __device__ __forceinline__ void init(int lane, int wave, int64_t ld) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = (i * NW + wave) * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz(r);
            off[i] = uint32_t((int64_t(r) * ld + c * 8) * 2);
            kk[i] = c * 8;
        }
    }
    // Instruction i of this wave for the tile at k0.
    __device__ __forceinline__ void issue_one(int i, i32x4_t rs, uint4* stage, int wave, int k0, int K) const {
        const uint32_t base = uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)stage));
        uint32_t v = off[i] + uint32_t(k0) * 2u;
        if (k0 + kk[i] >= K) v = OOB;
        dma16(rs, __builtin_amdgcn_readfirstlane(base + uint32_t(i * NW + wave) * 1024u), v);
    }
    __device__ __forceinline__ void issue(i32x4_t rs, uint4* stage, int wave, int k0, int K) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) issue_one(i, rs, stage, wave, k0, K);
    }
};

// Fragments of one 16-deep k-step: the wave's FM A row-blocks and FN B
// row-blocks of 32, lane l holding row l%32, k = 8*(l/32)..+7 of the step.
template <int FM, int FN, int TM, int TN>
__device__ __forceinline__ void read_frags(const uint4* __restrict__ a_l, const uint4* __restrict__ b_l, int ks,
                                           int wm, int wn, int lane, uint4 (&fa)[FM], uint4 (&fb)[FN]) {
    const int kc = ks * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int r = wm * TM + i * 32 + (lane & 31);
        fa[i] = a_l[r * 4 + (kc ^ swz(r))];
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int r = wn * TN + j * 32 + (lane & 31);
        fb[j] = b_l[r * 4 + (kc ^ swz(r))];
    }
}

// MFMAs number q0 .. q0+NQ-1 of a k-step, in (i, j) row-major order.
template <int FM, int FN, bool F16, int Q0, int NQ>
__device__ __forceinline__ void mma_part(const uint4 (&fa)[FM], const uint4 (&fb)[FN], f32x16_t (&acc)[FM][FN]) {
#pragma unroll
    for (int q = Q0; q < Q0 + NQ; ++q) {
        const int i = q / FN, j = q % FN;
        if constexpr (F16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(fb[j]), as_f16x8(fa[i]), acc[i][j], 0, 0, 0);
        else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fb[j]), as_bf16x8(fa[i]), acc[i][j], 0, 0, 0);
    }
}

template <int FM, int FN, bool F16>
__device__ __forceinline__ void mma_frags(const uint4 (&fa)[FM], const uint4 (&fb)[FN], f32x16_t (&acc)[FM][FN]) {
    mma_part<FM, FN, F16, 0, FM * FN>(fa, fb, acc);
}

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_f4(float* p, const float* w) {
    const f32x4v v = {w[0], w[1], w[2], w[3]};
    if (MT_NT_NTSTORE) __builtin_nontemporal_store(v, reinterpret_cast<f32x4v*>(p));
    else *reinterpret_cast<f32x4v*>(p) = v;
}
__device__ __forceinline__ void st_b4(uint16_t* p, const float* w) {
    const u32x2v v = {pack2(w[0], w[1]), pack2(w[2], w[3])};
    if (MT_NT_NTSTORE) __builtin_nontemporal_store(v, reinterpret_cast<u32x2v*>(p));
    else *reinterpret_cast<u32x2v*>(p) = v;
}

// Epilogue of 4 consecutive columns col..col+3 of one row.
template <int EPI>
__device__ __forceinline__ void store4(const GemmArgs& p, int row, int col, const float* v) {
    const int64_t ci = int64_t(row) * p.ldc + col;
    if (col + 4 <= p.N) {
        float w[4] = {v[0], v[1], v[2], v[3]};
        if constexpr (EPI == EPI_BF16_RESID || EPI == EPI_F32_RESID || EPI == EPI_F32_F16IN_RESID) {
            const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.R) + int64_t(row) * p.ldr + col);
            w[0] += bflo(r.x); w[1] += bfhi(r.x); w[2] += bflo(r.y); w[3] += bfhi(r.y);
        } else if constexpr (EPI == EPI_BF16_RESID32) {
            const float4 r = *reinterpret_cast<const float4*>(static_cast<const float*>(p.R) + int64_t(row) * p.ldr + col);
            w[0] += r.x; w[1] += r.y; w[2] += r.z; w[3] += r.w;
        } else if constexpr (EPI == EPI_BF16_ACCF32) {
            const float4 r = *reinterpret_cast<const float4*>(p.Cacc + int64_t(row) * p.ldacc + col);
            w[0] += r.x; w[1] += r.y; w[2] += r.z; w[3] += r.w;
        } else if constexpr (EPI == EPI_F32_ACC) {
            const float4 r = *reinterpret_cast<const float4*>(static_cast<const float*>(p.C) + ci);
            w[0] += r.x; w[1] += r.y; w[2] += r.z; w[3] += r.w;
        }
        if constexpr (EPI == EPI_F32 || EPI == EPI_F32_F16IN || EPI == EPI_F32_ACC || EPI == EPI_F32_RESID ||
                      EPI == EPI_F32_F16IN_RESID)
            st_f4(static_cast<float*>(p.C) + ci, w);
        else
            st_b4(static_cast<uint16_t*>(p.C) + ci, w);
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = col + e;
        if (c >= p.N) break;
        float w = v[e];
        if constexpr (EPI == EPI_BF16_RESID || EPI == EPI_F32_RESID || EPI == EPI_F32_F16IN_RESID)
            w += bf2f(static_cast<const uint16_t*>(p.R)[int64_t(row) * p.ldr + c]);
        else if constexpr (EPI == EPI_BF16_RESID32)
            w += static_cast<const float*>(p.R)[int64_t(row) * p.ldr + c];
        else if constexpr (EPI == EPI_BF16_ACCF32)
            w += p.Cacc[int64_t(row) * p.ldacc + c];
        else if constexpr (EPI == EPI_F32_ACC)
            w += static_cast<const float*>(p.C)[ci + e];
        if constexpr (EPI == EPI_F32 || EPI == EPI_F32_F16IN || EPI == EPI_F32_ACC || EPI == EPI_F32_RESID ||
                      EPI == EPI_F32_F16IN_RESID)
            static_cast<float*>(p.C)[ci + e] = w;
        else
            static_cast<uint16_t*>(p.C)[ci + e] = f2bf(w);
    }
}

// Epilogue through LDS.  Stored straight from the accumulators, one store
// instruction would cover 32 rows with 16 bytes each, i.e. 32 separate
// memory requests, and with every block finishing at about the same time the
// requests, not the bytes, bound the epilogue.  Instead each wave passes its
// accumulators through CAP bytes of LDS of its own (st), in P passes of FM/P
// row blocks, as fp32 rows of TN values (16-byte chunks XOR-swizzled with
// the row's low 4 bits, which makes both the column-wise writes and the
// row-wise reads conflict-free), and reads them back so that a store
// instruction covers whole row segments of TN values.  The caller's last
// barrier came after every wave's last LDS read and after every load into
// LDS had landed, so the region is free.  row0/col0: the wave's first output.
template <int FM, int FN, int TM, int TN, int CAP, int EPI>
__device__ __forceinline__ void staged_store(const GemmArgs& p, const f32x16_t (&acc)[FM][FN], float4* st, int lane,
                                             int row0, int col0) {
    constexpr int P = (TM * TN * 4 + CAP - 1) / CAP;   // passes
    constexpr int FMP = FM / P, RP = FMP * 32, CPR = TN / 4;
    static_assert(FM % P == 0 && RP * CPR * 16 <= CAP && CPR >= 16 && 64 % CPR == 0, "staging layout");
    static_assert(EPI != EPI_BF16_AMAX || MT_NT_ST8, "the maxima ride on the 8-column bf16 stores");
    float amx = 0.f;  // EPI_BF16_AMAX: max |stored value| of this lane
    static_for<0, P>([&](auto pass_) {
        constexpr int pass = decltype(pass_)::value;
#pragma unroll
        for (int ii = 0; ii < FMP; ++ii) {
            const int r = ii * 32 + (lane & 31);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16_t& a = acc[pass * FMP + ii][j];
                    const int c = j * 8 + 2 * q + (lane >> 5);
                    st[r * CPR + (c ^ (r & 15))] = make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
                }
        }
        if constexpr ((EPI == EPI_BF16 || EPI == EPI_BF16_AMAX) && MT_NT_ST8) {
            // bf16 out, no epilogue operand: 8 columns (16 bytes) per lane
#pragma unroll
            for (int it = 0; it < RP * CPR / 128; ++it) {
                const int e = it * 64 + lane;
                const int r = e / (CPR / 2), c = 2 * (e % (CPR / 2));
                const float4 w0 = st[r * CPR + (c ^ (r & 15))];
                const float4 w1 = st[r * CPR + ((c + 1) ^ (r & 15))];
                const int row = row0 + pass * RP + r, col = col0 + c * 4;
                if (row < p.M && col < p.N) {
                    if (col + 8 <= p.N && (p.ldc & 7) == 0) {
                        const uint4 v = make_uint4(pack2(w0.x, w0.y), pack2(w0.z, w0.w), pack2(w1.x, w1.y),
                                                   pack2(w1.z, w1.w));
                        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.C) + int64_t(row) * p.ldc + col) = v;
                        if constexpr (EPI == EPI_BF16_AMAX) {  // max |value| of the stored bf16 values
                            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                            for (int q = 0; q < 4; ++q) amx = fmaxf(amx, fmaxf(fabsf(bflo(wv[q])), fabsf(bfhi(wv[q]))));
                        }
                    } else {
                        const float v0[4] = {w0.x, w0.y, w0.z, w0.w}, v1[4] = {w1.x, w1.y, w1.z, w1.w};
                        store4<EPI_BF16>(p, row, col, v0);
                        if (col + 4 < p.N) store4<EPI_BF16>(p, row, col + 4, v1);
                        if constexpr (EPI == EPI_BF16_AMAX) {  // the columns stored, rounded as stored
#pragma unroll
                            for (int q = 0; q < 8; ++q)
                                if (col + q < p.N) amx = fmaxf(amx, fabsf(bf2f(f2bf(q < 4 ? v0[q] : v1[q - 4]))));
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int it = 0; it < RP * CPR / 64; ++it) {
                const int e = it * 64 + lane;
                const int r = e / CPR, c = e % CPR;
                const float4 w = st[r * CPR + (c ^ (r & 15))];
                const int row = row0 + pass * RP + r, col = col0 + c * 4;
                if (row < p.M && col < p.N) {
                    const float v[4] = {w.x, w.y, w.z, w.w};
                    store4<EPI>(p, row, col, v);
                }
            }
        }
    });
    if constexpr (EPI == EPI_BF16_AMAX) {  // one atomic max per block into its partial maximum
        __shared__ float wm[16];
        amx = wave_max(amx);
        if (lane == 0) wm[threadIdx.x >> 6] = amx;
        __syncthreads();
        if (threadIdx.x == 0) {
            float m = 0.f;
            for (int w = 0; w < int(blockDim.x >> 6); ++w) m = fmaxf(m, wm[w]);
            if (m > 0.f) atomicMax(p.amax + (blockIdx.x % ATTN_AMAX_PARTS) * ATTN_AMAX_LINE, __float_as_uint(m));
        }
    }
}

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void gemm_nt_k(GemmArgs p, int tiles_m, int tiles_n) {
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr bool F16 = EPI == EPI_F32_F16IN || EPI == EPI_F32_F16IN_RESID;
    // four stages, one array each, so that the compiler can tell the LDS
    // reads of one stage from the loads in flight into another
    __shared__ uint4 As0[BM * 4], As1[BM * 4], As2[BM * 4], As3[BM * 4];
    __shared__ uint4 Bs0[BN * 4], Bs1[BN * 4], Bs2[BN * 4], Bs3[BN * 4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // Blocks dispatched to one XCD (every 8th) take a contiguous range of
    // tiles, grouped 8 deep along M so neighbours share A rows and B rows.
    const int total = tiles_m * tiles_n;
    int pid = blockIdx.x;
    if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
    constexpr int GROUP = 8;
    const int per_group = GROUP * tiles_n;
    const int g = pid / per_group;
    const int first_m = g * GROUP;
    const int gsz = min(tiles_m - first_m, GROUP);
    const int tm = first_m + (pid % per_group) % gsz;
    const int tn = (pid % per_group) / gsz;
    const int m0 = tm * BM, n0 = tn * BN;

    const int rows_a = min(BM, p.M - m0), rows_b = min(BN, p.N - n0);
    const auto ra = make_rsrc(static_cast<const uint16_t*>(p.A) + int64_t(m0) * p.lda,
                              uint32_t((int64_t(rows_a - 1) * p.lda + p.K) * 2));
    const auto rb = make_rsrc(static_cast<const uint16_t*>(p.B) + int64_t(n0) * p.ldb,
                              uint32_t((int64_t(rows_b - 1) * p.ldb + p.K) * 2));
    DirectLoader<BM, NW> la;
    DirectLoader<BN, NW> lb;
    la.init(lane, wave, p.lda);
    lb.init(lane, wave, p.ldb);
    constexpr int NIT = DirectLoader<BM, NW>::NI + DirectLoader<BN, NW>::NI;  // loads per wave per tile

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (p.K + BK - 1) / BK;
    uint4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];

#define ISSUE(SA, SB, T)                         \
    la.issue(ra, SA, wave, (T) * BK, p.K);      \
    lb.issue(rb, SB, wave, (T) * BK, p.K);      \
    __builtin_amdgcn_sched_barrier(0)
#define RD(SA, SB, KS, FA, FB) read_frags<FM, FN, TM, TN>(SA, SB, KS, wm, wn, lane, FA, FB)
#define MM(FA, FB) mma_frags<FM, FN, F16>(FA, FB, acc)
// The loads of a tile are spread over the MFMAs of the tile three earlier:
// NIT/2 with each of its two k-steps, one per MG MFMAs, so the wave never
// stalls on a full address FIFO with MFMAs left to issue.
    constexpr int NIA = DirectLoader<BM, NW>::NI;
    constexpr int HALF = NIT / 2;
    constexpr int MG = FM * FN / HALF;
    static_assert(NIT % 2 == 0 && (FM * FN) % HALF == 0, "load interleave");
// Wait until tile T's loads have landed (those of tile T+1 and the first
// half of tile T+2 may still be in flight), then a block barrier.
#define WAIT_TILE(T)                                  \
    do {                                              \
        const int later = min(nk - 1 - (T), 2);       \
        if (later >= 2) wait_vmem<NIT + HALF>();      \
        else if (later == 1) wait_vmem<NIT>();        \
        else wait_vmem<0>();                          \
        barrier_lds();                                \
    } while (0)
#define LOAD_ONE(g, XA, XB, T)                                                           \
    if constexpr ((g) < NIA) la.issue_one((g), ra, XA, wave, (T) * BK, p.K);             \
    else lb.issue_one((g) - NIA, rb, XB, wave, (T) * BK, p.K)
// Half h of a k-step's MFMAs interleaved with half h of tile T3's loads.
#define MM_LOADS(FA, FB, h, XA, XB, T3, do_load)                                         \
    static_for<0, HALF>([&](auto g_) {                                                   \
        constexpr int g = decltype(g_)::value;                                           \
        if (do_load) { LOAD_ONE((h) * HALF + g, XA, XB, T3); }                           \
        mma_part<FM, FN, F16, g * MG, MG>(FA, FB, acc);                                  \
        __builtin_amdgcn_sched_barrier(0);                                               \
    })
// Tile T in stage (SA, SB): read step 1 while step 0 multiplies, barrier,
// read step 0 of tile T+1 from (NA, NB) while step 1 multiplies; the loads
// of tile T+3 into stage (XA, XB) ride along.
#define TILE(T, SA, SB, NA, NB, XA, XB)                                    \
    if ((T) < nk) {                                                        \
        const bool ld3 = (T) + 3 < nk;                                     \
        RD(SA, SB, 1, fa1, fb1);                                           \
        __builtin_amdgcn_sched_barrier(0);                                 \
        if (MT_NT_PRIO) __builtin_amdgcn_s_setprio(1);                     \
        MM_LOADS(fa0, fb0, 0, XA, XB, (T) + 3, ld3);                       \
        if (MT_NT_PRIO) __builtin_amdgcn_s_setprio(0);                     \
        WAIT_TILE((T) + 1);                                                \
        if ((T) + 1 < nk) { RD(NA, NB, 0, fa0, fb0); }                     \
        __builtin_amdgcn_sched_barrier(0);                                 \
        if (MT_NT_PRIO) __builtin_amdgcn_s_setprio(1);                     \
        MM_LOADS(fa1, fb1, 1, XA, XB, (T) + 3, ld3);                       \
        if (MT_NT_PRIO) __builtin_amdgcn_s_setprio(0);                     \
    }

    ISSUE(As0, Bs0, 0);
    if (nk > 1) { ISSUE(As1, Bs1, 1); }
    if (nk > 2) { ISSUE(As2, Bs2, 2); }
    WAIT_TILE(0);
    RD(As0, Bs0, 0, fa0, fb0);
    for (int t = 0; t < nk; t += 4) {
        TILE(t, As0, Bs0, As1, Bs1, As3, Bs3)
        TILE(t + 1, As1, Bs1, As2, Bs2, As0, Bs0)
        TILE(t + 2, As2, Bs2, As3, Bs3, As1, Bs1)
        TILE(t + 3, As3, Bs3, As0, Bs0, As2, Bs2)
    }
#undef TILE
#undef MM_LOADS
#undef LOAD_ONE
#undef WAIT_TILE
#undef MM
#undef RD
#undef ISSUE

    // acc[i][j] element r of lane l: row m0 + wm*TM + 32i + l%32, column
    // n0 + wn*TN + 32j + 8*(r/4) + 4*(l/32) + r%4.
#if MT_NT_STAGED
    {
        static_assert(BM == BN && NW <= 8, "one stage array per wave");
        uint4* const arr = wave == 0 ? As0 : wave == 1 ? As1 : wave == 2 ? As2 : wave == 3 ? As3
                         : wave == 4 ? Bs0 : wave == 5 ? Bs1 : wave == 6 ? Bs2 : Bs3;
        staged_store<FM, FN, TM, TN, BM * 64, EPI>(p, acc, reinterpret_cast<float4*>(arr), lane, m0 + wm * TM,
                                                    n0 + wn * TN);
    }
#else
    static_assert(EPI != EPI_BF16_AMAX, "the maxima ride on the staged epilogue");
    const int ml = lane & 31, nq = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = m0 + wm * TM + i * 32 + ml;
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = n0 + wn * TN + j * 32 + 8 * q + nq;
                if (col >= p.N) continue;
                const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                store4<EPI>(p, row, col, v);
            }
    }
#endif
}


// ---------------------------------------------------------------------------
// The same product with 64-deep k-tiles in two LDS stages.  A tile row is then
// 128 bytes, one whole cache line, so a load instruction makes 8 line-sized
// requests instead of 16 half-line ones, and the block synchronises once per
// 64 k instead of once per 32.  With two stages the loads of tile t+2 go into
// the stage of tile t as soon as the barrier at the end of tile t has passed
// (half with the last k-step of tile t, half with the first of tile t+1), so
// they have a whole tile of MFMA work to arrive in, as many cycles as the
// four 32-deep stages give.
constexpr int BK64 = 64;

// Tile (tm, tn) of position pid in the order of gemm_nt_k: tiles grouped
// MT_NT_GROUP deep along M, N-major within a group.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
    constexpr int GROUP = MT_NT_GROUP;
    const int per_group = GROUP * tiles_n;
    const int g = pid / per_group;
    const int first_m = g * GROUP;
    const int gsz = min(tiles_m - first_m, GROUP);
    tm = first_m + (pid % per_group) % gsz;
    tn = (pid % per_group) / gsz;
}

// Physical chunk (of eight) of logical chunk c in a 128-byte LDS row r: a
// 128-bit read of 16 consecutive rows touches each of the 16 positions of a
// 256-byte bank line once when rows of one parity take distinct chunks.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// Loads of one operand's ROWS x 64 tile: instruction i of wave w covers tile
// rows 8*(i*NW + w) .. +7 (64 lanes x 16 bytes = 8 rows of 128 bytes).
template <int ROWS, int NW>
struct DirectLoader64 {
    static constexpr int NI = ROWS / (8 * NW);
    static_assert(NI >= 1 && ROWS % (8 * NW) == 0, "tile rows must cover the waves");
    uint32_t off[NI];
    int kk[NI];

    __device__ __forceinline__ void init(int lane, int wave, int64_t ld) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = (i * NW + wave) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ swz8(r);
            off[i] = uint32_t((int64_t(r) * ld + c * 8) * 2);
            kk[i] = c * 8;
        }
    }
    __device__ __forceinline__ void issue_one(int i, i32x4_t rs, uint4* stage, int wave, int k0, int K) const {
        const uint32_t base = uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)stage));
        uint32_t v = off[i] + uint32_t(k0) * 2u;
        if (k0 + kk[i] >= K) v = OOB;
        dma16(rs, __builtin_amdgcn_readfirstlane(base + uint32_t(i * NW + wave) * 1024u), v);
    }
    __device__ __forceinline__ void issue(i32x4_t rs, uint4* stage, int wave, int k0, int K) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) issue_one(i, rs, stage, wave, k0, K);
    }
};

// An operand stored k-major ([K x rows], the layouts NN and TN take for B,
// and TN for A) is tiled the other way round: LDS row k holds the tile's
// COLS output rows at that k (COLS * 2 bytes, one whole global row segment
// per load request), and a fragment's 8 k of one output row are read
// across rows with ds_read_b64_tr_b16.  Physical chunk of logical chunk c in
// tile row k: c ^ 4 (k & 3), so the four rows one such read spans land in
// four distinct 64-byte bank groups.
__device__ __forceinline__ int swzT(int k) { return (k & 3) << 2; }

// Loads of one k-major operand's 64 x COLS tile: instruction i of wave w
// fills LDS chunks (i*NW + w)*64 + lane, RPI whole tile rows.
template <int COLS, int NW>
struct DirectLoader64T {
    static constexpr int CPR = COLS / 8;                 // 16-byte chunks per tile row
    static constexpr int RPI = 64 / CPR;                 // tile rows per wave instruction
    static constexpr int NI = 64 / (RPI * NW);
    static_assert(CPR * RPI == 64 && NI >= 1 && RPI * NW * NI == 64, "tile rows must cover the waves");
    uint32_t off[NI];
    int kr[NI];   // the lane's tile row (k within the tile)
    uint32_t ld2;

    __device__ __forceinline__ void init(int lane, int wave, int64_t ld) {
        ld2 = uint32_t(ld * 2);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int pos = (i * NW + wave) * 64 + lane;
            const int r = pos / CPR;
            const int c = (pos % CPR) ^ swzT(r);
            off[i] = uint32_t((int64_t(r) * ld + c * 8) * 2);
            kr[i] = r;
        }
    }
    __device__ __forceinline__ void issue_one(int i, i32x4_t rs, uint4* stage, int wave, int k0, int K) const {
        const uint32_t base = uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)stage));
        uint32_t v = off[i] + uint32_t(k0) * ld2;
        if (k0 + kr[i] >= K) v = OOB;
        dma16(rs, __builtin_amdgcn_readfirstlane(base + uint32_t(i * NW + wave) * 1024u), v);
    }
    __device__ __forceinline__ void issue(i32x4_t rs, uint4* stage, int wave, int k0, int K) const {
#pragma unroll
        for (int i = 0; i < NI; ++i) issue_one(i, rs, stage, wave, k0, K);
    }
};

// Fragment of k-step ks for output rows col0 .. col0+31 of a k-major tile:
// lane l gets row col0 + l%32 at k = 16 ks + 8 (l/32) + 0..7, the layout a
// 128-bit read of a k-contiguous tile gives.  Each ds_read_b64_tr_b16 reads
// four tile rows (k) x 16 columns per 16 lanes, every lane addressing one
// 8-byte piece, and hands lane i column i of them.
template <int COLS>
__device__ __forceinline__ uint4 frag_kmajor(const uint4* t, int ks, int col0, int lane) {
    const int j = lane & 15, g16 = (lane >> 4) & 1, hh = lane >> 5;
    const int col = col0 + 16 * g16 + 4 * (j & 3);
    const char* base = reinterpret_cast<const char*>(t);
    uint2 r[2];
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
        const int k = 16 * ks + 8 * hh + 4 * e2 + (j >> 2);
        const int off = k * (COLS * 2) + (((col >> 3) ^ swzT(k)) * 16) + (col & 7) * 2;
        typedef short i16x4_t __attribute__((ext_vector_type(4)));
        const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(lds_ptr_t)(base + off));
        r[e2] = __builtin_bit_cast(uint2, v);
    }
    return make_uint4(r[0].x, r[0].y, r[1].x, r[1].y);
}

// fp16 fragment rounded to bf16 (exact widening, then round to nearest even).
__device__ __forceinline__ uint4 f16_frag_to_bf16(const uint4& v) {
    typedef float f32x8_t __attribute__((ext_vector_type(8)));
    const f32x8_t f = __builtin_convertvector(as_f16x8(v), f32x8_t);
    return __builtin_bit_cast(uint4, __builtin_convertvector(f, bf16x8_t));
}

template <int FM, int FN, int TM, int TN, bool TA = false, bool TB = false, int BM = 0, int BN = 0, bool BH = false>
__device__ __forceinline__ void read_frags64(const uint4* __restrict__ a_l, const uint4* __restrict__ b_l, int ks,
                                             int wm, int wn, int lane, uint4 (&fa)[FM], uint4 (&fb)[FN]) {
    const int kc = ks * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        if constexpr (TA) {
            fa[i] = frag_kmajor<BM>(a_l, ks, wm * TM + i * 32, lane);
        } else {
            const int r = wm * TM + i * 32 + (lane & 31);
            fa[i] = a_l[r * 8 + (kc ^ swz8(r))];
        }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        if constexpr (TB) {
            fb[j] = frag_kmajor<BN>(b_l, ks, wn * TN + j * 32, lane);
            if constexpr (BH) fb[j] = f16_frag_to_bf16(fb[j]);
        } else {
            const int r = wn * TN + j * 32 + (lane & 31);
            fb[j] = b_l[r * 8 + (kc ^ swz8(r))];
        }
    }
}

// TA / TB: A / B stored k-major (A [K x M], B [K x N]); the other layouts
// of C = op(A) op(B) then run on the same main loop with no transposed copy.
// BH: B holds fp16 values, rounded to bf16 as each fragment is read.
template <int BM, int BN, int WM, int WN, int EPI, bool TA = false, bool TB = false, bool BH = false>
__global__ __launch_bounds__(WM * WN * 64) void gemm_nt64_k(GemmArgs p, int tiles_m, int tiles_n, GemmSplit sp) {
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr bool F16 = EPI == EPI_F32_F16IN || EPI == EPI_F32_F16IN_RESID;
    __shared__ uint4 As0[BM * 8], As1[BM * 8];
    __shared__ uint4 Bs0[BN * 8], Bs1[BN * 8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // Blocks below sp.n_full take whole tiles in the order of gemm_nt_k; each
    // later block takes k-steps [kb, kb + nkl) of tile n_full + slot / splits
    // and leaves its fp32 partial in scratch slot `slot`.
    const int nk = (p.K + BK64 - 1) / BK64;
    int pid = blockIdx.x, kb = 0, nkl = nk, slot = -1;
    if (pid < sp.n_full) {
        if ((sp.n_full & 7) == 0) pid = (pid & 7) * (sp.n_full >> 3) + (pid >> 3);
    } else {
        slot = pid - sp.n_full;
        pid = sp.n_full + slot / sp.splits;
        kb = (slot % sp.splits) * sp.kper;
        nkl = min(nk - kb, sp.kper);
    }
    int tm, tn;
    tile_coords(pid, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int rows_a = min(BM, p.M - m0), rows_b = min(BN, p.N - n0);
    // The resources end at the block's last element: past it (rows beyond M
    // or N of a k-contiguous operand, k beyond K of a k-major one) reads give
    // zero.  A k-major operand's columns past M or N inside the extent read
    // neighbouring elements, which reach only accumulator rows or columns
    // that are never stored.
    const auto ra = TA ? make_rsrc(static_cast<const uint16_t*>(p.A) + m0,
                                   uint32_t((int64_t(p.K - 1) * p.lda + rows_a) * 2))
                       : make_rsrc(static_cast<const uint16_t*>(p.A) + int64_t(m0) * p.lda,
                                   uint32_t((int64_t(rows_a - 1) * p.lda + p.K) * 2));
    const auto rb = TB ? make_rsrc(static_cast<const uint16_t*>(p.B) + n0,
                                   uint32_t((int64_t(p.K - 1) * p.ldb + rows_b) * 2))
                       : make_rsrc(static_cast<const uint16_t*>(p.B) + int64_t(n0) * p.ldb,
                                   uint32_t((int64_t(rows_b - 1) * p.ldb + p.K) * 2));
    using LA = std::conditional_t<TA, DirectLoader64T<BM, NW>, DirectLoader64<BM, NW>>;
    using LB = std::conditional_t<TB, DirectLoader64T<BN, NW>, DirectLoader64<BN, NW>>;
    LA la;
    LB lb;
    la.init(lane, wave, p.lda);
    lb.init(lane, wave, p.ldb);
    constexpr int NIA = LA::NI;
    constexpr int NIT = NIA + LB::NI;  // loads per wave per tile
    // loads of a tile issued with the last k-step of the tile two earlier
    // (NIT - L1) and with the first k-step of the tile before it (L1)
    constexpr int L1 = MT_NT_L1 < 0 ? NIT / 2 : MT_NT_L1;
    static_assert(L1 >= 0 && L1 < NIT && (FM * FN) % (NIT - L1) == 0 && (L1 == 0 || (FM * FN) % L1 == 0),
                  "load interleave");

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    uint4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];

#define RD(SA, SB, KS, FA, FB) read_frags64<FM, FN, TM, TN, TA, TB, BM, BN, BH>(SA, SB, KS, wm, wn, lane, FA, FB)
#define MM(FA, FB) mma_frags<FM, FN, F16>(FA, FB, acc)
#define PRIO(x) if (MT_NT_PRIO) __builtin_amdgcn_s_setprio(x)
#define LOAD_ONE(g, XA, XB, T)                                                           \
    if constexpr ((g) < NIA) la.issue_one((g), ra, XA, wave, (kb + (T)) * BK64, p.K);    \
    else lb.issue_one((g) - NIA, rb, XB, wave, (kb + (T)) * BK64, p.K)
// One k-step's MFMAs with loads G0 .. G0+NL-1 of tile T2, spread evenly.
#define MM_LOADS(FA, FB, G0, NL, XA, XB, T2, do_load)                                    \
    static_for<0, NL>([&](auto g_) {                                                     \
        constexpr int g = decltype(g_)::value;                                           \
        constexpr int mg = FM * FN / (NL);                                               \
        if (do_load) { LOAD_ONE((G0) + g, XA, XB, T2); }                                 \
        mma_part<FM, FN, F16, g * mg, mg>(FA, FB, acc);                                  \
        __builtin_amdgcn_sched_barrier(0);                                               \
    })
// Tile T in stage (SA, SB), the other stage (NA, NB) receiving tile T+1.
// Step 0 multiplies (fragments read before) while step 1 is read, and
// carries the second half of tile T+1's loads; steps 1 and 2 likewise; then
// the block waits for tile T+1 (the only loads in flight), reads its step 0
// and multiplies step 3 of tile T with the first half of tile T+2's loads,
// which go into this tile's stage, free since the barrier.
#define TILE(T, SA, SB, NA, NB)                                                          \
    if ((T) < nkl) {                                                                     \
        const bool ld1 = (T) >= 1 && (T) + 1 < nkl;                                      \
        const bool ld2 = (T) + 2 < nkl;                                                  \
        RD(SA, SB, 1, fa1, fb1);                                                         \
        __builtin_amdgcn_sched_barrier(0);                                               \
        PRIO(1);                                                                         \
        if constexpr (L1 > 0) { MM_LOADS(fa0, fb0, NIT - L1, L1, NA, NB, (T) + 1, ld1); }  \
        else { MM(fa0, fb0); }                                                           \
        PRIO(0);                                                                         \
        RD(SA, SB, 2, fa0, fb0);                                                         \
        __builtin_amdgcn_sched_barrier(0);                                               \
        PRIO(1);                                                                         \
        MM(fa1, fb1);                                                                    \
        PRIO(0);                                                                         \
        __builtin_amdgcn_sched_barrier(0);                                               \
        RD(SA, SB, 3, fa1, fb1);                                                         \
        __builtin_amdgcn_sched_barrier(0);                                               \
        PRIO(1);                                                                         \
        MM(fa0, fb0);                                                                    \
        PRIO(0);                                                                         \
        wait_vmem<0>();                                                                  \
        barrier_lds();                                                                   \
        if ((T) + 1 < nkl) { RD(NA, NB, 0, fa0, fb0); }                                  \
        __builtin_amdgcn_sched_barrier(0);                                               \
        PRIO(1);                                                                         \
        MM_LOADS(fa1, fb1, 0, NIT - L1, SA, SB, (T) + 2, ld2);                           \
        PRIO(0);                                                                         \
    }

    la.issue(ra, As0, wave, kb * BK64, p.K);
    lb.issue(rb, Bs0, wave, kb * BK64, p.K);
    if (nkl > 1) {
        la.issue(ra, As1, wave, (kb + 1) * BK64, p.K);
        lb.issue(rb, Bs1, wave, (kb + 1) * BK64, p.K);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmem<NIT>();
    } else {
        wait_vmem<0>();
    }
    barrier_lds();
    RD(As0, Bs0, 0, fa0, fb0);
    for (int t = 0; t < nkl; t += 2) {
        TILE(t, As0, Bs0, As1, Bs1)
        TILE(t + 1, As1, Bs1, As0, Bs0)
    }
#undef TILE
#undef MM_LOADS
#undef LOAD_ONE
#undef PRIO
#undef MM
#undef RD

    {
        static_assert(BM == BN && NW % 4 == 0 && NW <= 8, "stage arrays split among the waves");
        constexpr int PER = NW / 4;                  // waves per stage array
        constexpr int CAP = BM * 128 / PER;          // bytes per wave
        const int q = wave / PER;
        uint4* const arr = q == 0 ? As0 : q == 1 ? As1 : q == 2 ? Bs0 : Bs1;
        float4* const st = reinterpret_cast<float4*>(arr) + (wave % PER) * (CAP / 16);
        if (slot >= 0) {
            // partial tile: fp32 rows of BN values in scratch slot `slot`
            GemmArgs q2 = p;
            q2.C = p.ws + int64_t(slot) * (BM * BN);
            q2.ldc = BN;
            q2.M = BM;
            q2.N = BN;
            staged_store<FM, FN, TM, TN, CAP, EPI_F32>(q2, acc, st, lane, wm * TM, wn * TN);
        } else {
            staged_store<FM, FN, TM, TN, CAP, EPI>(p, acc, st, lane, m0 + wm * TM, n0 + wn * TN);
        }
    }
}

// Tail tiles of a split product: output tile n_full + blockIdx.x / 64 is the
// sum of its `splits` fp32 partials in split order (k-ranges ascending), then
// the product's epilogue.  Thread: 4 consecutive columns of one row.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_split_fixup_k(GemmArgs p, int tiles_m, int tiles_n, GemmSplit sp) {
    const int t = blockIdx.x >> 6;
    const int e = (blockIdx.x & 63) * 256 + threadIdx.x;
    const int r = e >> 6, c = (e & 63) * 4;
    int tm, tn;
    tile_coords(sp.n_full + t, tiles_m, tiles_n, tm, tn);
    const int row = tm * 256 + r, col = tn * 256 + c;
    if (row >= p.M || col >= p.N) return;
    const float* w = p.ws + int64_t(t) * sp.splits * 65536 + r * 256 + c;
    float4 a = *reinterpret_cast<const float4*>(w);
    for (int i = 1; i < sp.splits; ++i) {
        const float4 b = *reinterpret_cast<const float4*>(w + int64_t(i) * 65536);
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    const float v[4] = {a.x, a.y, a.z, a.w};
    store4<EPI>(p, row, col, v);
}

// The split a direct-form launch on 256 x 256 tiles takes (see gemm_split_plan).
hipError_t split_for(const GemmArgs& a, int tm, int tn, GemmSplit& sp) {
    const int total = tm * tn, nk = (a.K + 63) / 64;
    sp = GemmSplit{total, 1, nk};
    if (!a.ws) return hipSuccess;
    if (a.force_splits <= 0) {
        sp = gemm_split_plan(a.M, a.N, a.K, a.ws_bytes);
        return hipSuccess;
    }
    if (a.force_splits == 1) return hipSuccess;
    const int n_full = (total / 256) * 256;
    if (n_full == total) return hipSuccess;
    const int kper = (nk + a.force_splits - 1) / a.force_splits;
    const int splits = (nk + kper - 1) / kper;   // every split non-empty
    if (splits <= 1) return hipSuccess;
    if (uint64_t(total - n_full) * splits * 65536u * 4u > a.ws_bytes) return hipErrorInvalidValue;
    sp = GemmSplit{n_full, splits, kper};
    return hipSuccess;
}

template <int EPI>
void launch_fixup_e(const GemmArgs& a, int tm, int tn, const GemmSplit& sp, hipStream_t s) {
    const int tail = tm * tn - sp.n_full;
    gemm_split_fixup_k<EPI><<<dim3(tail * 64), dim3(256), 0, s>>>(a, tm, tn, sp);
}

hipError_t launch_fixup(GemmEpi epi, const GemmArgs& a, int tm, int tn, const GemmSplit& sp, hipStream_t s) {
    switch (epi) {
        case EPI_BF16: launch_fixup_e<EPI_BF16>(a, tm, tn, sp, s); break;
        case EPI_BF16_RESID: launch_fixup_e<EPI_BF16_RESID>(a, tm, tn, sp, s); break;
        case EPI_F32: launch_fixup_e<EPI_F32>(a, tm, tn, sp, s); break;
        case EPI_F32_ACC: launch_fixup_e<EPI_F32_ACC>(a, tm, tn, sp, s); break;
        case EPI_BF16_ACCF32: launch_fixup_e<EPI_BF16_ACCF32>(a, tm, tn, sp, s); break;
        case EPI_F32_RESID: launch_fixup_e<EPI_F32_RESID>(a, tm, tn, sp, s); break;
        case EPI_BF16_RESID32: launch_fixup_e<EPI_BF16_RESID32>(a, tm, tn, sp, s); break;
        case EPI_F32_F16IN: launch_fixup_e<EPI_F32_F16IN>(a, tm, tn, sp, s); break;
        case EPI_F32_F16IN_RESID: launch_fixup_e<EPI_F32_F16IN_RESID>(a, tm, tn, sp, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Grid of a split launch: whole tiles, then `splits` blocks per tail tile.
inline dim3 split_grid(int tm, int tn, const GemmSplit& sp) {
    return dim3(sp.n_full + (tm * tn - sp.n_full) * sp.splits);
}

template <int BM, int BN, int WM, int WN, bool K64>
hipError_t launch(GemmEpi epi, const GemmArgs& a, hipStream_t s) {
    const int tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
    const dim3 block(WM * WN * 64);
    GemmSplit sp{tm * tn, 1, (a.K + 63) / 64};
    if constexpr (K64 && BM == 256 && BN == 256) {
        if (epi != EPI_BF16_AMAX) {  // the maxima are taken in the whole-tile epilogue only
            const hipError_t e = split_for(a, tm, tn, sp);
            if (e != hipSuccess) return e;
        }
    }
    const dim3 grid = K64 ? split_grid(tm, tn, sp) : dim3(tm * tn);
    switch (epi) {
        case EPI_BF16:
            if constexpr (K64) gemm_nt64_k<BM, BN, WM, WN, EPI_BF16><<<grid, block, 0, s>>>(a, tm, tn, sp);
            else gemm_nt_k<BM, BN, WM, WN, EPI_BF16><<<grid, block, 0, s>>>(a, tm, tn);
            break;
        case EPI_BF16_RESID:
            if constexpr (K64) gemm_nt64_k<BM, BN, WM, WN, EPI_BF16_RESID><<<grid, block, 0, s>>>(a, tm, tn, sp);
            else gemm_nt_k<BM, BN, WM, WN, EPI_BF16_RESID><<<grid, block, 0, s>>>(a, tm, tn);
            break;
        case EPI_F32:
            if constexpr (K64) gemm_nt64_k<BM, BN, WM, WN, EPI_F32><<<grid, block, 0, s>>>(a, tm, tn, sp);
            else gemm_nt_k<BM, BN, WM, WN, EPI_F32><<<grid, block, 0, s>>>(a, tm, tn);
            break;
        case EPI_F32_ACC:
            if constexpr (K64) gemm_nt64_k<BM, BN, WM, WN, EPI_F32_ACC><<<grid, block, 0, s>>>(a, tm, tn, sp);
            else gemm_nt_k<BM, BN, WM, WN, EPI_F32_ACC><<<grid, block, 0, s>>>(a, tm, tn);
            break;
        case EPI_BF16_ACCF32:
            if constexpr (K64) gemm_nt64_k<BM, BN, WM, WN, EPI_BF16_ACCF32><<<grid, block, 0, s>>>(a, tm, tn, sp);
            else gemm_nt_k<BM, BN, WM, WN, EPI_BF16_ACCF32><<<grid, block, 0, s>>>(a, tm, tn);
            break;
        case EPI_F32_RESID:
            if constexpr (K64) gemm_nt64_k<BM, BN, WM, WN, EPI_F32_RESID><<<grid, block, 0, s>>>(a, tm, tn, sp);
            else gemm_nt_k<BM, BN, WM, WN, EPI_F32_RESID><<<grid, block, 0, s>>>(a, tm, tn);
            break;
        case EPI_BF16_RESID32:
            if constexpr (K64) gemm_nt64_k<BM, BN, WM, WN, EPI_BF16_RESID32><<<grid, block, 0, s>>>(a, tm, tn, sp);
            else gemm_nt_k<BM, BN, WM, WN, EPI_BF16_RESID32><<<grid, block, 0, s>>>(a, tm, tn);
            break;
        case EPI_F32_F16IN:
            if constexpr (K64) gemm_nt64_k<BM, BN, WM, WN, EPI_F32_F16IN><<<grid, block, 0, s>>>(a, tm, tn, sp);
            else gemm_nt_k<BM, BN, WM, WN, EPI_F32_F16IN><<<grid, block, 0, s>>>(a, tm, tn);
            break;
        case EPI_F32_F16IN_RESID:
            if constexpr (K64) gemm_nt64_k<BM, BN, WM, WN, EPI_F32_F16IN_RESID><<<grid, block, 0, s>>>(a, tm, tn, sp);
            else gemm_nt_k<BM, BN, WM, WN, EPI_F32_F16IN_RESID><<<grid, block, 0, s>>>(a, tm, tn);
            break;
        case EPI_BF16_AMAX:
            if constexpr (K64) gemm_nt64_k<BM, BN, WM, WN, EPI_BF16_AMAX><<<grid, block, 0, s>>>(a, tm, tn, sp);
            else gemm_nt_k<BM, BN, WM, WN, EPI_BF16_AMAX><<<grid, block, 0, s>>>(a, tm, tn);
            break;
        default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || sp.splits <= 1) return e;
    return launch_fixup(epi, a, tm, tn, sp, s);
}

// The k-major forms (NN: B k-major; TN: both), 256 x 256 tiles only, with
// the epilogues the backward products and the head use.
template <bool TA, bool TB>
hipError_t launch_kmajor(GemmEpi epi, const GemmArgs& a, hipStream_t s) {
    constexpr int WM = MT_NT_WM, WN = MT_NT_NW / MT_NT_WM;
    const int tm = (a.M + 255) / 256, tn = (a.N + 255) / 256;
    const dim3 block(WM * WN * 64);
    if (a.b_f16 && !(TA && TB && epi == EPI_BF16)) return hipErrorNotSupported;
    if (epi != EPI_BF16 && epi != EPI_F32 && epi != EPI_F32_ACC && epi != EPI_BF16_ACCF32 && epi != EPI_BF16_AMAX)
        return hipErrorNotSupported;
    GemmSplit sp{tm * tn, 1, (a.K + 63) / 64};
    if (epi != EPI_BF16_AMAX) {  // the maxima are taken in the whole-tile epilogue only
        const hipError_t e = split_for(a, tm, tn, sp);
        if (e != hipSuccess) return e;
    }
    const dim3 grid = split_grid(tm, tn, sp);
    if (a.b_f16) {
        if constexpr (TA && TB)
            gemm_nt64_k<256, 256, WM, WN, EPI_BF16, true, true, true><<<grid, block, 0, s>>>(a, tm, tn, sp);
    } else {
        switch (epi) {
            case EPI_BF16: gemm_nt64_k<256, 256, WM, WN, EPI_BF16, TA, TB><<<grid, block, 0, s>>>(a, tm, tn, sp); break;
            case EPI_F32: gemm_nt64_k<256, 256, WM, WN, EPI_F32, TA, TB><<<grid, block, 0, s>>>(a, tm, tn, sp); break;
            case EPI_F32_ACC:
                gemm_nt64_k<256, 256, WM, WN, EPI_F32_ACC, TA, TB><<<grid, block, 0, s>>>(a, tm, tn, sp);
                break;
            case EPI_BF16_AMAX:
                gemm_nt64_k<256, 256, WM, WN, EPI_BF16_AMAX, TA, TB><<<grid, block, 0, s>>>(a, tm, tn, sp);
                break;
            default:
                gemm_nt64_k<256, 256, WM, WN, EPI_BF16_ACCF32, TA, TB><<<grid, block, 0, s>>>(a, tm, tn, sp);
                break;
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || sp.splits <= 1) return e;
    return launch_fixup(epi, a, tm, tn, sp, s);
}

inline bool al16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; }

}  // namespace

hipError_t gemm_direct(GemmLayout lay, GemmEpi epi, const GemmArgs& a, hipStream_t s) {
    // Preconditions beyond gemm()'s checks: 4-column epilogue vectors stay
    // aligned, and a block's extent fits the 31-bit buffer offsets (a
    // k-contiguous operand: 256 rows x ld; a k-major one: K rows x ld).
    const bool resid = epi == EPI_BF16_RESID || epi == EPI_F32_RESID || epi == EPI_BF16_RESID32 ||
                       epi == EPI_F32_F16IN_RESID;
    if ((a.ldc & 3) || !al16(a.C)) return hipErrorNotSupported;
    if (resid && ((a.ldr & 3) || !al16(a.R))) return hipErrorNotSupported;
    if (epi == EPI_BF16_ACCF32 && ((a.ldacc & 3) || !al16(a.Cacc))) return hipErrorNotSupported;
    const bool ta = lay == GEMM_TN, tb = lay != GEMM_NT;
    if (a.b_f16 && !(ta && epi == EPI_BF16)) return hipErrorNotSupported;
    constexpr int64_t lim = (int64_t(1) << 30) - 256;  // elements below 2^31 bytes
    if (ta ? int64_t(a.K) * a.lda > lim : a.lda > (int64_t(1) << 21)) return hipErrorNotSupported;
    if (tb ? int64_t(a.K) * a.ldb > lim : a.ldb > (int64_t(1) << 21)) return hipErrorNotSupported;
    const int64_t big_tiles = int64_t((a.M + 255) / 256) * ((a.N + 255) / 256);
    if (lay == GEMM_NT) {
        if (big_tiles >= MT_NT_BIG_MIN)
            return launch<256, 256, MT_NT_WM, MT_NT_NW / MT_NT_WM, MT_NT_K64 != 0>(epi, a, s);
        return launch<128, 128, 2, 2, false>(epi, a, s);
    }
    if (!MT_GEMM_KMAJOR || !MT_NT_K64 || big_tiles < MT_NT_BIG_MIN) return hipErrorNotSupported;
    return ta ? launch_kmajor<true, true>(epi, a, s) : launch_kmajor<false, true>(epi, a, s);
}

// Cost model of the tail split, in units of one 64-deep k-step of a 256 x 256
// tile on a busy CU (~1.8 us at the clock the chip holds under dense MFMA
// load).  The first full rounds of tiles run whole; the last, partial round
// of r < 256 tiles leaves CUs idle for as long as one tile takes.  Cut into s
// k-ranges, its r * s blocks run in ceil(r * s / 256) rounds of ceil(nk / s)
// steps, each block also storing its 256 KB fp32 partial (~3 steps); a second
// kernel then reads the partials back and writes the output (~4 TB/s, plus
// ~6 steps of launch).  The split with the lowest predicted time is taken if
// it saves at least 5%; ties go to fewer splits (less scratch traffic).
GemmSplit gemm_split_plan(int64_t M, int64_t N, int64_t K, uint64_t ws_bytes) {
    const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256, total = tm * tn;
    const int64_t nk = (K + 63) / 64;
    GemmSplit best{int(total), 1, int(nk)};
    const int64_t r = total % 256, n_full = total - r, R = n_full / 256;
    if (r == 0 || total >= (int64_t(1) << 30)) return best;
    constexpr double TAU_S = 1.8e-6, FIX_BPS = 4.0e12, FIX_LAUNCH = 6.0, STORE = 3.0;
    const double base = double((total + 255) / 256) * double(nk);
    double best_t = 0.95 * base;
    for (int64_t s = 2; s <= 16; ++s) {
        const int64_t kper = (nk + s - 1) / s;
        const int64_t se = (nk + kper - 1) / kper;
        if (kper < 4 || se != s) continue;
        const int64_t units = r * s;
        if (uint64_t(units) * 65536u * 4u > ws_bytes) continue;
        const double fix_bytes = double(units) * 262144.0 + double(r) * 262144.0;
        const double t = double(R) * double(nk) + double((units + 255) / 256) * (double(kper) + STORE) +
                         fix_bytes / FIX_BPS / TAU_S + FIX_LAUNCH;
        if (t < best_t) {
            best_t = t;
            best = GemmSplit{int(n_full), int(s), int(kper)};
        }
    }
    return best;
}

}  // namespace mt
