// bf16 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), fp32
// accumulation, three operand layouts and five epilogues.
//
// The block linear maps of the decoder (fused QKV, O, fused gate|up, down,
// LM head) and their backward passes are dense contractions, so they run on
// MFMA.  Design:
//  * block tile BM x BN with BK = 64, one LDS image per operand holding 64
//    k-values per row (128 bytes, 8 chunks of 16 bytes); the chunk index is
//    XOR-swizzled with the row so both the MFMA fragment reads and the
//    transposing writes spread over all bank groups;
//  * operands stored k-contiguous ([rows x K]) are copied to LDS as they are;
//    operands stored row-contiguous ([K x rows], the weight-gradient case)
//    are transposed in registers, 4 k x 8 rows per thread, on the way in;
//  * two LDS stages: the global loads of stage k+1 are issued before the
//    MFMAs of stage k and written to the other LDS image after them, one
//    barrier per stage;
//  * blockIdx is remapped so that the tiles one XCD (every 8th block) runs
//    are a contiguous range, then grouped 8 tiles deep along M, so tiles
//    sharing A rows or B columns share that XCD's L2.
#include "kcommon.h"
#include "kernels.h"

namespace mt {
namespace {

constexpr int BK = 64;

// Physical 16-byte chunk of logical chunk kc in LDS row r is kc ^ swz(r).
// Mixing bits 3..5 of the row in keeps both the MFMA reads (32 consecutive
// rows, one chunk) and the transposing writes (rows 8 apart, one chunk)
// spread over all eight chunk positions.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ uint32_t half_of(const uint4& v, int e) {
    uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Tile loader for one operand: R rows of the tile (M or N side), 64 k.
template <int R, int NT, bool KMAJOR>
struct TileLoader {
    // k-contiguous: R*8 chunks of 8 k; row-contiguous: 2R blocks of 4 k x 8 rows.
    static constexpr int NCH = KMAJOR ? (R * 8) / NT : (2 * R) / NT;
    static constexpr int NREG = KMAJOR ? NCH : NCH * 4;
    static_assert(NCH >= 1, "tile too small for the thread count");
    uint4 reg[NREG];
    uint32_t ok[NREG];  // all-ones for lanes inside the matrix, else zero

    // Every lane issues its loads unconditionally from an address clamped into
    // the matrix; lanes outside it zero their registers when the data is
    // consumed.  (A conditional load would make the loads wait one by one.)
    __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld, int row0,
                                         int rows, int k0, int K, int tid) {
        if constexpr (KMAJOR) {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int c = tid + i * NT;
                const int r = c >> 3, kc = c & 7;
                const int gr = row0 + r, gk = k0 + kc * 8;
                ok[i] = (gr < rows && gk < K) ? 0xFFFFFFFFu : 0u;
                const int cr = min(gr, rows - 1), ck = min(gk, K - 8);
                reg[i] = *reinterpret_cast<const uint4*>(base + int64_t(cr) * ld + ck);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int c = tid + i * NT;
                const int mg = c % (R / 8), kg = c / (R / 8);
                const int gm = row0 + mg * 8;
                const int cm = min(gm, rows - 8);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int gk = k0 + kg * 4 + j;
                    ok[i * 4 + j] = (gk < K && gm < rows) ? 0xFFFFFFFFu : 0u;
                    const int ck = min(gk, K - 1);
                    reg[i * 4 + j] = *reinterpret_cast<const uint4*>(base + int64_t(ck) * ld + cm);
                }
            }
        }
    }

    // Write the registers into LDS image `lds` ([R][8] uint4, swizzled).
    __device__ __forceinline__ void store(uint4* __restrict__ lds, int tid) {
#pragma unroll
        for (int i = 0; i < NREG; ++i) {
            reg[i].x &= ok[i];
            reg[i].y &= ok[i];
            reg[i].z &= ok[i];
            reg[i].w &= ok[i];
        }
        if constexpr (KMAJOR) {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                int c = tid + i * NT;
                int r = c >> 3, kc = c & 7;
                lds[r * 8 + (kc ^ swz(r))] = reg[i];
            }
        } else {
            uint2* l2 = reinterpret_cast<uint2*>(lds);
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                int c = tid + i * NT;
                int mg = c % (R / 8), kg = c / (R / 8);
                int kc = kg >> 1, hf = kg & 1;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    int r = mg * 8 + e;
                    uint2 v;
                    v.x = half_of(reg[i * 4 + 0], e) | (half_of(reg[i * 4 + 1], e) << 16);
                    v.y = half_of(reg[i * 4 + 2], e) | (half_of(reg[i * 4 + 3], e) << 16);
                    l2[(r * 8 + (kc ^ swz(r))) * 2 + hf] = v;
                }
            }
        }
    }
};

template <int BM, int BN, int WM, int WN, bool AK, bool BKM, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(GemmArgs p, int tiles_m, int tiles_n) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    static_assert(FM >= 1 && FN >= 1, "wave tile below 32x32");
    __shared__ uint4 smem[2 * (BM + BN) * 8];
    uint4* As = smem;
    uint4* Bs = smem + 2 * BM * 8;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // XCD-aware remap, then group 8 tiles along M.
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

    const uint16_t* A = static_cast<const uint16_t*>(p.A);
    const uint16_t* B = static_cast<const uint16_t*>(p.B);

    TileLoader<BM, NT, AK> la;
    TileLoader<BN, NT, BKM> lb;

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (p.K + BK - 1) / BK;
    la.load(A, p.lda, m0, p.M, 0, p.K, tid);
    lb.load(B, p.ldb, n0, p.N, 0, p.K, tid);
    la.store(As, tid);
    lb.store(Bs, tid);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            la.load(A, p.lda, m0, p.M, (kt + 1) * BK, p.K, tid);
            lb.load(B, p.ldb, n0, p.N, (kt + 1) * BK, p.K, tid);
        }
        const uint4* a_l = As + cur * BM * 8;
        const uint4* b_l = Bs + cur * BN * 8;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int kc = ks * 2 + (lane >> 5);
            uint4 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                int r = wm * TM + i * 32 + (lane & 31);
                af[i] = a_l[r * 8 + (kc ^ swz(r))];
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                int r = wn * TN + j * 32 + (lane & 31);
                bfr[j] = b_l[r * 8 + (kc ^ swz(r))];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if constexpr (EPI == EPI_F32_F16IN || EPI == EPI_F32_F16IN_RESID)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(af[i]), as_f16x8(bfr[j]),
                                                                           acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[i]), as_bf16x8(bfr[j]),
                                                                            acc[i][j], 0, 0, 0);
                }
        }
        if (more) {
            la.store(As + (cur ^ 1) * BM * 8, tid);
            lb.store(Bs + (cur ^ 1) * BN * 8, tid);
        }
        __syncthreads();
    }

    // Epilogue.  Accumulator element r of lane l sits at row
    // 8*(r/4) + 4*(l/32) + r%4 and column l%32 of its 32x32 tile.
    const int col_l = lane & 31;
    const int row_l = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * TN + j * 32 + col_l;
            if (col >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * TM + i * 32 + (r >> 2) * 8 + row_l + (r & 3);
                if (row >= p.M) continue;
                float v = acc[i][j][r];
                if constexpr (EPI == EPI_BF16) {
                    static_cast<uint16_t*>(p.C)[int64_t(row) * p.ldc + col] = f2bf(v);
                } else if constexpr (EPI == EPI_BF16_RESID) {
                    v += bf2f(static_cast<const uint16_t*>(p.R)[int64_t(row) * p.ldr + col]);
                    static_cast<uint16_t*>(p.C)[int64_t(row) * p.ldc + col] = f2bf(v);
                } else if constexpr (EPI == EPI_F32 || EPI == EPI_F32_F16IN) {
                    static_cast<float*>(p.C)[int64_t(row) * p.ldc + col] = v;
                } else if constexpr (EPI == EPI_F32_ACC) {
                    float* c = static_cast<float*>(p.C) + int64_t(row) * p.ldc + col;
                    *c = *c + v;
                } else if constexpr (EPI == EPI_F32_RESID || EPI == EPI_F32_F16IN_RESID) {
                    v += bf2f(static_cast<const uint16_t*>(p.R)[int64_t(row) * p.ldr + col]);
                    static_cast<float*>(p.C)[int64_t(row) * p.ldc + col] = v;
                } else if constexpr (EPI == EPI_BF16_RESID32) {
                    v += static_cast<const float*>(p.R)[int64_t(row) * p.ldr + col];
                    static_cast<uint16_t*>(p.C)[int64_t(row) * p.ldc + col] = f2bf(v);
                } else {
                    v += p.Cacc[int64_t(row) * p.ldacc + col];
                    static_cast<uint16_t*>(p.C)[int64_t(row) * p.ldc + col] = f2bf(v);
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM>
hipError_t launch_epi(GemmEpi epi, const GemmArgs& a, hipStream_t s) {
    const int tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
    dim3 grid(tm * tn), block(WM * WN * 64);
    switch (epi) {
        case EPI_BF16:
            gemm_kernel<BM, BN, WM, WN, AK, BKM, EPI_BF16><<<grid, block, 0, s>>>(a, tm, tn); break;
        case EPI_BF16_RESID:
            gemm_kernel<BM, BN, WM, WN, AK, BKM, EPI_BF16_RESID><<<grid, block, 0, s>>>(a, tm, tn); break;
        case EPI_F32:
            gemm_kernel<BM, BN, WM, WN, AK, BKM, EPI_F32><<<grid, block, 0, s>>>(a, tm, tn); break;
        case EPI_F32_ACC:
            gemm_kernel<BM, BN, WM, WN, AK, BKM, EPI_F32_ACC><<<grid, block, 0, s>>>(a, tm, tn); break;
        case EPI_BF16_ACCF32:
            gemm_kernel<BM, BN, WM, WN, AK, BKM, EPI_BF16_ACCF32><<<grid, block, 0, s>>>(a, tm, tn); break;
        case EPI_F32_RESID:
            gemm_kernel<BM, BN, WM, WN, AK, BKM, EPI_F32_RESID><<<grid, block, 0, s>>>(a, tm, tn); break;
        case EPI_BF16_RESID32:
            gemm_kernel<BM, BN, WM, WN, AK, BKM, EPI_BF16_RESID32><<<grid, block, 0, s>>>(a, tm, tn); break;
        case EPI_F32_F16IN:
            if constexpr (AK && BKM) {
                gemm_kernel<BM, BN, WM, WN, AK, BKM, EPI_F32_F16IN><<<grid, block, 0, s>>>(a, tm, tn);
                break;
            }
            return hipErrorInvalidValue;
        case EPI_F32_F16IN_RESID:
            if constexpr (AK && BKM) {
                gemm_kernel<BM, BN, WM, WN, AK, BKM, EPI_F32_F16IN_RESID><<<grid, block, 0, s>>>(a, tm, tn);
                break;
            }
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool AK, bool BKM>
hipError_t launch_layout(GemmEpi epi, const GemmArgs& a, hipStream_t s) {
    // Large problems: 256x256 tiles, 8 waves of 128x64.  Small ones (fewer
    // than ~2 tiles per CU): 128x128 tiles, 4 waves of 64x64.
    // Measured on MI355X at the 7B shapes: 256x256 with 8 waves wins whenever
    // the grid has at least one tile per CU (a 1.75-wave grid of big tiles
    // still beats 7 waves of 128x128); 4 waves of 128x128 each lose latency
    // hiding at one wave per SIMD.
    const int64_t big_tiles = int64_t((a.M + 255) / 256) * ((a.N + 255) / 256);
    if (big_tiles >= 256) return launch_epi<256, 256, 2, 4, AK, BKM>(epi, a, s);
    return launch_epi<128, 128, 2, 2, AK, BKM>(epi, a, s);
}

}  // namespace

static hipError_t gemm_check(GemmLayout lay, GemmEpi epi, const GemmArgs& a) {
    if (a.M <= 0 || a.N <= 0 || a.K <= 0) return hipErrorInvalidValue;
    if (!a.A || !a.B || !a.C) return hipErrorInvalidValue;
    // 16-byte vector loads: the contiguous dimension and every leading
    // dimension must be multiples of 8 elements, base pointers 16-byte aligned.
    auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    if (!al16(a.A) || !al16(a.B) || (a.lda & 7) || (a.ldb & 7)) return hipErrorInvalidValue;
    const bool ak = lay != GEMM_TN, bk = lay == GEMM_NT;
    if (ak ? (a.K & 7) : (a.M & 7)) return hipErrorInvalidValue;
    if (bk ? (a.K & 7) : (a.N & 7)) return hipErrorInvalidValue;
    if (ak ? a.lda < a.K : a.lda < a.M) return hipErrorInvalidValue;
    if (bk ? a.ldb < a.K : a.ldb < a.N) return hipErrorInvalidValue;
    if (a.ldc < a.N) return hipErrorInvalidValue;
    if ((epi == EPI_BF16_RESID || epi == EPI_F32_RESID || epi == EPI_BF16_RESID32 || epi == EPI_F32_F16IN_RESID) &&
        (!a.R || a.ldr < a.N))
        return hipErrorInvalidValue;
    if (epi == EPI_BF16_ACCF32 && (!a.Cacc || a.ldacc < a.N)) return hipErrorInvalidValue;
    if ((epi == EPI_F32_F16IN || epi == EPI_F32_F16IN_RESID) && lay != GEMM_NT) return hipErrorInvalidValue;
    if (int(epi) < 0 || int(epi) > int(EPI_BF16_AMAX)) return hipErrorInvalidValue;
    if (epi == EPI_BF16_AMAX && (!a.amax || (reinterpret_cast<uintptr_t>(a.amax) & 255))) return hipErrorInvalidValue;
    if (a.b_f16 && (lay != GEMM_TN || epi != EPI_BF16)) return hipErrorInvalidValue;
    return hipSuccess;
}

hipError_t gemm_direct_checked(GemmLayout lay, GemmEpi epi, const GemmArgs& a, hipStream_t s) {
    const hipError_t c = gemm_check(lay, epi, a);
    return c != hipSuccess ? c : gemm_direct(lay, epi, a, s);
}

hipError_t gemm(GemmLayout lay, GemmEpi epi, const GemmArgs& a, hipStream_t s) {
    const hipError_t c = gemm_check(lay, epi, a);
    if (c != hipSuccess) return c;
    {
        const hipError_t e = gemm_direct(lay, epi, a, s);
        if (e != hipErrorNotSupported) return e;
    }
    if (a.b_f16) return hipErrorNotSupported;  // only the direct form converts B
    if (epi == EPI_BF16_AMAX) return hipErrorNotSupported;  // only the direct form takes the maxima
    switch (lay) {
        case GEMM_NT: return launch_layout<true, true>(epi, a, s);
        case GEMM_NN: return launch_layout<true, false>(epi, a, s);
        case GEMM_TN: return launch_layout<false, false>(epi, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mt
