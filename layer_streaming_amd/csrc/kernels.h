// Host-side launchers of the gfx950 kernels.  Every launcher checks the
// shapes it relies on, enqueues on `stream` and returns hipSuccess or the
// error of the launch; hipErrorInvalidValue means a shape the kernel does not
// support (the caller maps it to MT_E_INVAL before any device work).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mt {

// ---------------------------------------------------------------- GEMM ----
// C[M x N] = op(A) op(B) with fp32 accumulation on bf16 MFMA.
//   NT: A [M x K] row-major (lda), B [N x K] row-major (ldb)  -> X W^T
//   NN: A [M x K] row-major,       B [K x N] row-major          -> dY W
//   TN: A [K x M] row-major,       B [K x N] row-major          -> dY^T X
enum GemmLayout { GEMM_NT = 0, GEMM_NN = 1, GEMM_TN = 2 };
// Epilogues: what is written to C.
enum GemmEpi {
    EPI_BF16 = 0,        // C(bf16) = acc
    EPI_BF16_RESID = 1,  // C(bf16) = acc + R(bf16)
    EPI_F32 = 2,         // C(f32)  = acc
    EPI_F32_ACC = 3,     // C(f32) += acc
    EPI_BF16_ACCF32 = 4, // C(bf16) = acc + Cacc(f32)
    EPI_F32_RESID = 5,   // C(f32)  = acc + R(bf16)
    EPI_BF16_RESID32 = 6,// C(bf16) = acc + R(f32)
    EPI_F32_F16IN = 7,   // operands fp16 (not bf16), C(f32) = acc; NT layout only
    EPI_F32_F16IN_RESID = 8,  // operands fp16, C(f32) = acc + R(bf16); NT layout only
    EPI_BF16_AMAX = 9,   // C(bf16) = acc, and max |C| (of the stored bf16 values) into the partial maxima at
                         // amax (the attention backward's max |dO|); the direct form only, never split
};
struct GemmArgs {
    const void* A; int64_t lda;
    const void* B; int64_t ldb;
    void* C; int64_t ldc;
    const void* R; int64_t ldr;       // residual (EPI_*RESID*)
    const float* Cacc; int64_t ldacc; // fp32 partial sum, EPI_BF16_ACCF32
    int M, N, K;
    bool b_f16 = false;               // B holds fp16, rounded to bf16 as it is read (TN, EPI_BF16, direct form only)
    // Device scratch for the K-split of the last partial round of 256 x 256
    // tiles (fp32 partial tiles, 256 KB each); null: no split.  Used only by
    // the direct form; must not overlap A, B, C, R or Cacc.
    float* ws = nullptr;
    uint64_t ws_bytes = 0;
    int force_splits = 0;             // > 0: split the tail this many ways (tests); 0: gemm_split_plan decides
    uint32_t* amax = nullptr;         // EPI_BF16_AMAX: the partial maxima words (ATTN_AMAX_PARTS, one per line)
};
// How a direct-form product on 256 x 256 tiles is cut: the first n_full tiles
// run whole; each later tile runs as `splits` blocks over consecutive ranges
// of kper 64-deep k-steps, whose fp32 partials a second kernel adds in split
// order before the epilogue (deterministic for a given shape).
struct GemmSplit { int n_full; int splits; int kper; };
// The split the direct form takes for an M x N x K product given ws_bytes of
// scratch: splits = 1 unless cutting the last partial round of tiles is
// predicted to save at least 5% (cost model in gemm_nt.hip).
GemmSplit gemm_split_plan(int64_t M, int64_t N, int64_t K, uint64_t ws_bytes);
hipError_t gemm(GemmLayout lay, GemmEpi epi, const GemmArgs& a, hipStream_t s);
// The path with direct global->LDS tile loads (called by gemm() after its
// checks): every NT product, and NN / TN products on grids of at least
// 120 tiles of 256 x 256 with the epilogues EPI_BF16, EPI_F32, EPI_F32_ACC
// and EPI_BF16_ACCF32 (their k-major operands read transposed from LDS), and
// TN with an fp16 B (b_f16) and EPI_BF16.
// hipErrorNotSupported when a precondition fails; gemm() then uses the
// generic kernel, and the backward products transpose and take the NT form.
hipError_t gemm_direct(GemmLayout lay, GemmEpi epi, const GemmArgs& a, hipStream_t s);
// gemm()'s argument checks, then gemm_direct: hipErrorInvalidValue for bad
// arguments, hipErrorNotSupported when only the generic kernel could run it.
hipError_t gemm_direct_checked(GemmLayout lay, GemmEpi epi, const GemmArgs& a, hipStream_t s);

// ------------------------------------------------------------- RMSNorm ----
// n = gamma * x * rstd, rstd = 1/sqrt(mean(x^2)+eps); x bf16 or fp32 (x_f32),
// n and gamma bf16; n_f16 (may be null) receives the same values in fp16.
// ovf (may be null): counter of fp16 values out of range (saturated to
// +-65504), the range guard of every fp16 operand the kernels write.
// clear_amax (may be null, 16-byte aligned): ATTN_AMAX_BYTES zeroed by the
// kernel's first block (the recompute's first kernel clears the attention
// backward's maxima words before its producers add to them).
hipError_t rmsnorm_fwd(const void* x, bool x_f32, const uint16_t* gamma, uint16_t* n, uint16_t* n_f16,
                       float* rstd, int T, int d, float eps, hipStream_t s, uint32_t* ovf = nullptr,
                       uint32_t* clear_amax = nullptr);
// dx = resid + rstd*(g - nh*mean(g*nh)), g = dn*gamma, nh = x*rstd (resid may be null);
// dgamma = sum_t dn*nh written as bf16 (two-stage, fixed order).  `partial` is
// fp32 scratch of rmsnorm_bwd_partial_elems(T, d) elements.
hipError_t rmsnorm_bwd(const uint16_t* dn, const void* x, bool x_f32, const uint16_t* gamma,
                       const float* rstd, const uint16_t* resid, uint16_t* dx, uint16_t* dgamma,
                       float* partial, int T, int d, hipStream_t s);
int64_t rmsnorm_bwd_partial_elems(int T, int d);
// rmsnorm_bwd with its partials in a static per-GPU device array of
// RMSNORM_NOALLOC_FLOATS floats instead of a caller buffer (no allocation);
// hipErrorInvalidValue when rmsnorm_bwd_partial_elems(T, d) exceeds it.
// Calls that overlap on one GPU race on the array.
constexpr int64_t RMSNORM_NOALLOC_FLOATS = int64_t(4) << 20;  // 16 MiB
hipError_t rmsnorm_bwd_noalloc(const uint16_t* dn, const void* x, bool x_f32, const uint16_t* gamma,
                               const float* rstd, const uint16_t* resid, uint16_t* dx, uint16_t* dgamma, int T, int d,
                               hipStream_t s);

// ---------------------------------------------------------------- RoPE ----
// Table of cos/sin [S x hd/2] (float2), angle s*base^(-2e/hd) in double.
hipError_t rope_table(float2* tab, int S, int hd, float base, hipStream_t s);
// Rotate the first n_rot_heads heads of every row of qkv [T x ld] in place,
// position s = t % S; dir = +1 forward, -1 backward (rotation by -theta).
hipError_t rope_apply(uint16_t* qkv, int64_t ld, const float2* tab, int T, int S, int n_rot_heads,
                      int hd, int dir, hipStream_t s);
// The same rotation of the first n_rot_heads heads of fp32 in [T x ldin],
// written as bf16 to out [T x ldout] (one rounding), dir = -1 for a gradient
// rotated back by -theta (the attention backward folds this rotation into
// its own kernels; this one serves the kernel tests).
hipError_t rope_f32_to_bf16(const float* in, int64_t ldin, uint16_t* out, int64_t ldout, const float2* tab, int T,
                            int S, int n_rot_heads, int hd, int dir, hipStream_t s);
// From the fp32 QKV projection in [T x ldin] (n_heads heads of hd): rotate the
// first n_rot_heads (q and k), and write every head as fp16 (saturated and
// counted in ovf) into out [T x ldout] (the attention operand buffer); outb
// (may be null) [T x ldb, ldb >= n_heads*hd] gets the same heads in bf16.
// vmax (may be null): the partial maxima of |v| (the heads past n_rot_heads,
// as stored in fp16) are added to it, one atomic max per wave (see
// ATTN_AMAX_V_OFFSET; the caller zeroes the words).
hipError_t qkv_rope_cvt(const float* in, int64_t ldin, uint16_t* out, int64_t ldout, uint16_t* outb, int64_t ldb,
                        const float2* tab, int T, int S, int n_rot_heads, int n_heads, int hd, hipStream_t s,
                        uint32_t* ovf = nullptr, uint32_t* vmax = nullptr);
// Elementwise bf16 -> fp16 (n a multiple of 8), saturated and counted in ovf.
hipError_t bf16_to_f16(const uint16_t* in, uint16_t* out, int64_t n, hipStream_t s, uint32_t* ovf = nullptr);

// -------------------------------------------------------------- SwiGLU ----
// gu [T x 2F] = [gate | up] -> m [T x F] = silu(gate) * up.
hipError_t swiglu_fwd(const uint16_t* gu, uint16_t* m, int T, int F, hipStream_t s);
// dgu [T x 2F] = [dm*up*silu'(gate) | dm*silu(gate)].
hipError_t swiglu_bwd(const uint16_t* dm, const uint16_t* gu, uint16_t* dgu, int T, int F,
                      hipStream_t s);

// ----------------------------------------------------------- Attention ----
// qkv [B*S x ld]: q heads at column 0, k heads at Hq*hd, v heads at (Hq+Hkv)*hd,
// all fp16; the forward's products (scores and P.V) run on the fp16 MFMA and
// o is written as fp16.  dout and dqkv are bf16.
struct AttnArgs {
    const uint16_t* qkv; int64_t ld;
    uint16_t* o; int64_t ldo;   // [B*S x Hq*hd] fp16
    float* lse;                 // [B x Hq x S], natural-log sum-exp of scaled scores
    int B, S, Hq, Hkv, hd;
    uint32_t* ovf = nullptr;    // fp16 range guard: o values saturated to +-65504
};
hipError_t attn_fwd(const AttnArgs& a, hipStream_t s);
// Bytes of the attention backward's maxima scratch: 16 partial maxima of
// |dO| and 16 of |v|, each in its own 256-byte line.
constexpr int64_t ATTN_AMAX_BYTES = 8192;
constexpr int ATTN_AMAX_PARTS = 16, ATTN_AMAX_LINE = 64;  // partial maxima per quantity; uint32 words per line
// Where a producer adds to the partial maxima (float bit patterns, atomic
// max): block b of the producer of dO into word (b % PARTS) * LINE, of v into
// word (PARTS + b % PARTS) * LINE.
constexpr int ATTN_AMAX_V_OFFSET = ATTN_AMAX_PARTS * ATTN_AMAX_LINE;
struct AttnBwdArgs {
    const uint16_t* qkv; int64_t ld;  // fp16 q, k, v as the forward used them
    const uint16_t* o; const uint16_t* dout; int64_t ldo;  // o fp16, dout bf16
    const float* lse;
    float* dsum;           // scratch [2 x B x Hq x S]: -rowsum(dO * O) 2^k, then lse log2(e)
    uint16_t* do16;        // scratch [B*S x Hq*hd] fp16: dO 2^k
    uint32_t* amax;        // scratch, ATTN_AMAX_BYTES: partial maxima of |dO| and |v| that fix 2^k
    uint16_t* dqkv; int64_t ldd;  // output in qkv's column layout: dV bf16, and dQ, dK bf16 unless dqk32
    int B, S, Hq, Hkv, hd;
    // Optional: dQ and dK in fp32 [B*S x ld32] (the Hq query heads, then the
    // Hkv key heads), for a rotation that rounds them to bf16 once.
    float* dqk32 = nullptr; int64_t ld32 = 0;
    uint32_t* ovf = nullptr;  // fp16 range guard of the scaled dO
    // fp32 scratch for the partial sums of a dK/dV pass split over the query
    // heads of each KV group (short sequences: too few key tiles to fill the
    // chip).  splits: 0 = automatic, n = at most n; either way reduced to
    // what dpart_elems holds.
    float* dpart = nullptr; int64_t dpart_elems = 0;
    int splits = 0;
    // Optional: the stored-dS form of dQ (short sequences).  The dK/dV pass
    // writes dS 2^k in fp16 into ds: per (b, h) ds_ld/32 x ds_ld/32 blocks of
    // 32 keys x 32 queries (2 KB, key-major, queries in a fixed permuted
    // order; ds_ld = S rounded up to 128; only the blocks on or below the
    // diagonal), and dQ = dS K is formed from it afterwards instead of
    // recomputing the scores and dP.  nullptr: dQ recomputes them.
    uint16_t* ds = nullptr;
    int64_t ds_ld = 0;
    // Optional: the RoPE table (cos, sin) [S x hd/2].  Set, dQ and dK are
    // rotated by -theta where they are finished (the dQ kernel, the dK/dV
    // kernel or the split reduction) and written to dqkv in bf16, rounded
    // once; dqk32 is not used.
    const float2* rope_tab = nullptr;
    // The partial maxima of |dO| and |v| are already in amax, added where dO
    // and v were written (the O dX product, the recompute's rotation): the
    // maxima pass is skipped.
    bool amax_ready = false;
};
// Query-head splits the dK/dV pass takes for a shape: automatic (req 0:
// enough blocks for two per CU, at most Hq/Hkv) or at most req, reduced to
// fit part_elems floats (ns * B*S * 2*Hkv*hd).
int attn_dkdv_splits(int B, int S, int Hq, int Hkv, int hd, int64_t part_elems, int req);
// Floats of partials the automatic split needs (0 without a split).
int64_t attn_bwd_part_elems(int B, int S, int Hq, int Hkv, int hd);
// Bytes of the stored dS a shape takes the stored-dS form of dQ with (S up
// to 1024 and at most 1 GiB of dS), else 0.
int64_t attn_ds_bytes(int B, int S, int Hq);
// Scratch bytes of attn_bwd (dsum, do16, amax, the partials of the
// automatic split and the stored dS where the shape takes it) and their
// carving from one 256-byte-aligned block; with_ds = false leaves the dS
// region unused (dQ recomputes).
int64_t attn_bwd_work_bytes(int B, int S, int Hq, int Hkv, int hd);
void attn_bwd_carve(void* work, int B, int S, int Hq, int Hkv, int hd, AttnBwdArgs& a, bool with_ds = true);
hipError_t attn_bwd(const AttnBwdArgs& a, hipStream_t s);

// ------------------------------------------------------- Cross-entropy ----
// logits f32 [Tc x V], labels int32 [Tc] -> loss_rows[Tc] = lse - logit[label],
// dlogits bf16 [Tc x V] = (softmax - onehot) * inv_T.
hipError_t ce_fwd_bwd(const float* logits, const int32_t* labels, float* loss_rows,
                      uint16_t* dlogits, int Tc, int V, float inv_T, hipStream_t s);
// out[0] = sum(x[0..n)) / n in a fixed order (one block).
hipError_t mean_reduce(const float* x, float* out, int n, hipStream_t s);
// Cross-entropy over vocabulary chunks of Vc (a multiple of 8) columns
// starting at vocabulary row v0: merge the chunk into the running (m, l) per
// row (first: start afresh) and pick the label's logit into z; final: LSE and
// loss per row; bwd: dlogits = (exp(x - LSE) - onehot) * inv_T in bf16.
hipError_t ce_chunk_fwd(const float* logits, const int32_t* labels, int rows, int Vc, int v0, bool first, float* m,
                        float* l, float* z, hipStream_t s);
hipError_t ce_chunk_final(const float* m, const float* l, const float* z, float* lse, float* loss_rows, int T,
                          hipStream_t s);
hipError_t ce_chunk_bwd(const float* logits, const int32_t* labels, const float* lse, int rows, int Vc, int v0,
                        uint16_t* dlogits, float inv_T, hipStream_t s);

// --------------------------------------------------------------- misc -----
hipError_t f32_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t s);
hipError_t fill_zero(void* p, int64_t bytes, hipStream_t s);
// Every 32-bit word of [p, p + bytes) set to `pattern` (bytes a multiple of 16).
hipError_t fill_u32(void* p, int64_t bytes, uint32_t pattern, hipStream_t s);
// dst[c * ldd + r] = src[r * lds + c] for an R x C matrix of 16-bit elements;
// f16_to_bf16: the source is fp16 and the destination gets it rounded to bf16.
hipError_t transpose16(const uint16_t* src, int64_t lds, uint16_t* dst, int64_t ldd, int R, int C, hipStream_t s,
                       bool f16_to_bf16 = false);

}  // namespace mt
