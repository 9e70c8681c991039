/*
 * mt_kernels.h -- test entries of libmt.so: one call per gfx950 kernel of
 * the decoder block, on caller-owned device memory and a caller stream
 * (hipStream_t passed as void*; NULL is the null stream).  They launch and
 * return without synchronising.  Every call returns MT_OK, MT_E_INVAL for a
 * shape the kernel does not support (checked before launching) or MT_E_HIP.
 * bf16 tensors are uint16 bit patterns, row-major, 16-byte aligned; inner
 * dimensions and leading dimensions are multiples of 8 elements.
 *
 * The operations follow the decoder block the pages train, a pre-norm
 * Qwen2.5-style decoder ("MegaTrain ... Review", dimensionstp.github.io,
 * section 4-2 model list); the block itself is not spelled out on the pages.
 */
#ifndef MT_KERNELS_H
#define MT_KERNELS_H

#include <stdint.h>

#include "mt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* C[M x N] = op(A) op(B), bf16 inputs, fp32 accumulation.
 * layout 0 (NT): A [M x K] (lda), B [N x K] (ldb)   C = A B^T
 * layout 1 (NN): A [M x K],       B [K x N]         C = A B
 * layout 2 (TN): A [K x M],       B [K x N]         C = A^T B
 * epi 0: C bf16 = acc; 1: C bf16 = acc + R (bf16, ldr); 2: C f32 = acc;
 * 3: C f32 += acc; 4: C bf16 = acc + Cacc (f32, ldacc); 5: C f32 = acc + R
 * (bf16); 6: C bf16 = acc + R (f32); 7: A and B are fp16 (not bf16), C f32 =
 * acc, layout 0 only; 8: A and B fp16, C f32 = acc + R (bf16), layout 0 only. */
int mt_k_gemm(int32_t layout, int32_t epi, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
              int64_t ldc, const void* R, int64_t ldr, const void* Cacc, int64_t ldacc, int32_t M, int32_t N,
              int32_t K, void* stream);

/* mt_k_gemm with scratch for the K-split of the last partial round of
 * 256 x 256 tiles (the form the library's own products take): when the
 * product runs on 256 x 256 tiles and the tiles do not fill whole rounds of
 * the 256 CUs, the tiles of the last, partial round may be cut into `splits`
 * ranges of K, each a block of its own, whose fp32 partials (256 KB per block,
 * in `ws`) a second kernel adds in split order before the epilogue.
 * splits = 0: the library's choice (mt_k_gemm_split_plan); 1: no split;
 * n > 1: n ranges (tests), MT_E_INVAL if ws_bytes cannot hold them.  ws must
 * be 16-byte aligned and overlap no operand; ws = NULL is mt_k_gemm. */
int mt_k_gemm_split(int32_t layout, int32_t epi, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                    int64_t ldc, const void* R, int64_t ldr, const void* Cacc, int64_t ldacc, int32_t M, int32_t N,
                    int32_t K, void* ws, int64_t ws_bytes, int32_t splits, void* stream);
/* The split the library takes for an M x N x K product on 256 x 256 tiles
 * with ws_bytes of scratch (host only, no GPU): writes the number of tiles
 * that run whole, the number of K ranges of each later tile (1: no split)
 * and the 64-deep k-steps per range. */
int mt_k_gemm_split_plan(int64_t M, int64_t N, int64_t K, int64_t ws_bytes, int32_t* n_full, int32_t* splits,
                         int32_t* ksteps);

/* fp16 range guard.  Every entry that writes fp16 values (the attention
 * operands) saturates a value whose magnitude rounds beyond the fp16 range
 * (|x| >= 65520, or not finite) to +-65504 (a NaN stays a NaN) and, when
 * fp16_ovf is not NULL, adds the number of such values to the uint32 device
 * counter fp16_ovf points at (the caller zeroes it). */

/* RMSNorm: n = gamma * x / sqrt(mean(x^2) + eps) per row of x [T x d]
 * (x bf16, or f32 when x_f32 != 0); rstd [T] f32 = 1/sqrt(mean(x^2) + eps).
 * n_f16 (may be NULL) receives n rounded to fp16 instead of bf16. */
int mt_k_rmsnorm_fwd(const void* x, int32_t x_f32, const void* gamma, void* n, void* n_f16, void* rstd, int32_t T,
                     int32_t d, float eps, void* fp16_ovf, void* stream);
/* dx = resid + rstd * (g - nh * mean(g * nh)), g = dn*gamma, nh = x*rstd
 * (resid may be NULL); dgamma [d] bf16 = sum_t dn * nh, summed in a fixed
 * order through `scratch` (f32, mt_k_rmsnorm_bwd_scratch_elems(T, d) =
 * min(ceil(T / 4), 512) * d floats).  d <= 8192. */
int64_t mt_k_rmsnorm_bwd_scratch_elems(int32_t T, int32_t d);
int mt_k_rmsnorm_bwd(const void* dn, const void* x, int32_t x_f32, const void* gamma, const void* rstd,
                     const void* resid, void* dx, void* dgamma, void* scratch, int32_t T, int32_t d, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * mt_k_rmsnorm_bwd with its gain-gradient partials in a library-owned static
 * device buffer of MT_NOALLOC_SCRATCH_BYTES (16 MiB on every GPU the library
 * runs on, held until the process ends) instead of a caller scratch buffer.
 * Same arguments otherwise, same results bit for bit.  The call allocates
 * nothing; the buffer's device address is looked up once per device, on
 * the first call with that device current.  MT_E_INVAL, before any device
 * work, when the partials, mt_k_rmsnorm_bwd_scratch_elems(T, d) floats (at
 * most 512 * d), exceed the buffer's 4194304: every width the kernel
 * supports (d <= 8192) fits, for any T.  Every partial is written before it
 * is read, so the buffer needs no clearing.  Every call on one GPU shares the buffer: calls that overlap on
 * one GPU (concurrent streams or threads) race. */
#define MT_NOALLOC_SCRATCH_BYTES (16u << 20)
int mt_k_rmsnorm_bwd_noalloc(const void* dn, const void* x, int32_t x_f32, const void* gamma, const void* rstd,
                             const void* resid, void* dx, void* dgamma, int32_t T, int32_t d, void* stream);

/* Rotary embedding, rotate-half pairs (e, e+hd/2), angle s*base^(-2e/hd)
 * with s = t % S, in place on the first n_rot_heads heads of each row of
 * qkv [T x ld]; dir +1 forward, -1 backward.  table: device scratch of
 * S*hd/2 float2, filled by the call. */
int mt_k_rope(void* qkv, int64_t ld, void* table, int32_t T, int32_t S, int32_t n_rot_heads, int32_t hd,
              float base, int32_t dir, void* stream);
/* Forward rotary embedding on the f32 QKV projection in [T x ldin] (n_heads
 * heads of hd): the first n_rot_heads heads (q and k) are rotated in f32, and
 * every head is written as fp16 to out [T x ldout]; out_bf16 (may be NULL)
 * [T x ld_bf16, ld_bf16 >= n_heads*hd] also gets them in bf16 (the attention
 * backward's gradient products take them in that form).  Same angles and
 * table as mt_k_rope. */
int mt_k_qkv_rope_cvt(const void* in, int64_t ldin, void* out, int64_t ldout, void* out_bf16, int64_t ld_bf16,
                      void* table, int32_t T, int32_t S, int32_t n_rot_heads, int32_t n_heads, int32_t hd, float base,
                      void* fp16_ovf, void* stream);
/* The producers' side of the attention backward's scale 2^k (the form the
 * step runs, so that the backward needs no pass of its own over dO and v):
 * mt_k_gemm_amax is mt_k_gemm with epilogue 0 (bf16 out) that also adds the
 * maximum of the stored |C| values to the partial maxima of |dO| in `amax`
 * (words 64 i, i < 16, float bit patterns, atomic max); it takes only shapes
 * the direct form runs (MT_E_INVAL otherwise) and never splits.
 * mt_k_qkv_rope_cvt_vmax is mt_k_qkv_rope_cvt that adds max |v| of the fp16
 * heads past n_rot_heads to the partial maxima of |v| (words 64 (16 + i)).
 * amax: 8192 bytes, 256-byte aligned, zeroed by the caller. */
int mt_k_gemm_amax(int32_t layout, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                   int32_t M, int32_t N, int32_t K, void* amax, void* stream);
int mt_k_qkv_rope_cvt_vmax(const void* in, int64_t ldin, void* out, int64_t ldout, void* table, int32_t T, int32_t S,
                           int32_t n_rot_heads, int32_t n_heads, int32_t hd, float base, void* fp16_ovf, void* amax,
                           void* stream);
/* y[i] = fp16(x[i]) for bf16 x, n a multiple of 8. */
int mt_k_bf16_to_f16(const void* x, void* y, int64_t n, void* fp16_ovf, void* stream);

/* SwiGLU on gu [T x 2F] = [gate | up]: m [T x F] = silu(gate) * up;
 * backward dgu = [dm * up * silu'(gate) | dm * silu(gate)]. */
int mt_k_swiglu_fwd(const void* gu, void* m, int32_t T, int32_t F, void* stream);
int mt_k_swiglu_bwd(const void* dm, const void* gu, void* dgu, int32_t T, int32_t F, void* stream);

/* Causal GQA attention on qkv [B*S x ld] (q heads at column 0, k heads at
 * Hq*hd, v heads at (Hq+Hkv)*hd; query head h reads KV head h/(Hq/Hkv)),
 * scale 1/sqrt(hd): o [B*S x ldo], lse [B x Hq x S] f32 (natural log).
 * q, k, v and o are fp16 (o range-guarded); dout and dqkv bf16.
 * hd in {64, 128}. */
int mt_k_attn_fwd(const void* qkv, int64_t ld, void* o, int64_t ldo, void* lse, int32_t B, int32_t S, int32_t Hq,
                  int32_t Hkv, int32_t hd, void* fp16_ovf, void* stream);
/* Backward: dqkv [B*S x ldd] gets dV, and dQ and dK too unless dqk32 is
 * given, in the qkv column layout (the K and V gradients summed over each KV
 * group, in a fixed order), bf16.  dqk32 (may be NULL): dQ and dK in fp32
 * [B*S x ld32, ld32 >= (Hq+Hkv)*hd] instead (query heads, then key heads).
 * The products run on fp16: dO (bf16) is multiplied by the power of two 2^k
 * that keeps every |dP|, |D| and |dS| below 2^15 given max|dO| and max|v|
 * (range-guarded into fp16_ovf, may be NULL), the results are scaled back by
 * 2^-k.  With few key tiles (short sequences) the dK/dV pass splits each KV
 * group's query heads over head_splits blocks per key tile (0: automatic,
 * enough blocks for two per CU; n: at most n; never more than Hq/Hkv or than
 * the work buffer's partials hold) and adds their fp32 partial sums in split
 * order.  dQ either recomputes the scores and dP per query tile, or, for
 * sequences up to 1024 with at most 1 GiB of it, is formed as dS K from the
 * dS (2^k-scaled fp16) the dK/dV pass stores in the work buffer: dq_form 0
 * takes the stored form where the shape allows, 1 always recomputes, 2
 * requires the stored form (MT_E_INVAL where the shape does not allow it).
 * work: device scratch of mt_k_attn_bwd_work_bytes(B, S, Hq, Hkv, hd) bytes,
 * 256-byte aligned (D and the base-2 log-sum-exp, the scaled dO, the two
 * maxima as 8 KB of partial maxima, the partials of the automatic split, the
 * stored dS where the shape
 * takes it: B*Hq*Sp*Sp*2 bytes, Sp = S rounded up to 128);
 * B*S*Hq*hd/8 < 2^31.  mt_k_attn_dkdv_splits: the split count mt_k_attn_bwd
 * takes with such a buffer (0 on a bad shape). */
int64_t mt_k_attn_bwd_work_bytes(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t hd);
int32_t mt_k_attn_dkdv_splits(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t hd, int32_t head_splits);
int mt_k_attn_bwd(const void* qkv, int64_t ld, const void* o, const void* dout, int64_t ldo, const void* lse,
                  void* work, void* dqkv, int64_t ldd, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t hd,
                  void* dqk32, int64_t ld32, int32_t head_splits, int32_t dq_form, void* fp16_ovf, void* stream);
/* mt_k_attn_bwd with the RoPE backward folded in (the form the step runs):
 * dQ and dK are rotated by -theta where they are finished (the dQ kernel,
 * the dK/dV kernel or its split reduction) and go to dqkv's query and key
 * columns in bf16, rounded once after the rotation; dV as before; dqk32 is
 * not written (may be NULL).  The rotation uses mt_k_rope's angles
 * (positions restart every S tokens), its table ([S x hd/2] float2) computed
 * into `table` for base > 0, or taken as a previous call left it for
 * base = 0.  amax_ready != 0: the maxima words in `work` already hold the
 * maxima of this dO and v (left by a previous call on the same inputs), so
 * the maxima pass is skipped, as in the step, where the O dX product and the
 * recompute's rotation add them while they write dO and v. */
int mt_k_attn_bwd_rope(const void* qkv, int64_t ld, const void* o, const void* dout, int64_t ldo, const void* lse,
                       void* work, void* dqkv, int64_t ldd, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t hd,
                       void* dqk32, int64_t ld32, int32_t head_splits, int32_t dq_form, void* fp16_ovf, void* table,
                       float base, int32_t amax_ready, void* stream);
/* Rotary embedding of the first n_rot_heads heads of fp32 in [T x ldin]
 * (same angles and table as mt_k_rope; dir -1 rotates by -theta, the
 * backward), written as bf16 to out [T x ldout] with one rounding. */
int mt_k_rope_f32_bf16(const void* in, int64_t ldin, void* out, int64_t ldout, void* table, int32_t T, int32_t S,
                       int32_t n_rot_heads, int32_t hd, float base, int32_t dir, void* stream);

/* Cross-entropy of logits [Tc x V] f32 against int32 labels [Tc]:
 * loss_rows [Tc] = logsumexp - logit[label]; dlogits [Tc x V] bf16 =
 * (softmax - onehot) * inv_T.  mean: out[0] = sum(x[0..n)) / n. */
int mt_k_ce(const void* logits, const void* labels, void* loss_rows, void* dlogits, int32_t Tc, int32_t V,
            float inv_T, void* stream);
int mt_k_mean(const void* x, void* out, int32_t n, void* stream);
int mt_k_f32_to_bf16(const void* x, void* y, int64_t n, void* stream);
/* Transpose of an R x C matrix of 16-bit elements: dst[c*ldd + r] = src[r*lds + c]
 * (the backward products take both operands reduction-contiguous); with
 * f16_to_bf16 != 0 src holds fp16 and dst gets each value rounded to bf16.
 * Errors: MT_E_INVAL for negative sizes, lds < C or ldd < R. */
int mt_k_transpose16(const void* src, int64_t lds, void* dst, int64_t ldd, int32_t R, int32_t C, int32_t f16_to_bf16,
                     void* stream);

/* Host (CPU) entries, no GPU needed. */
/* The production host Adam over n elements of caller arrays: G <- gsrc,
 * m, v, master updated in fp32 with bias corrections for `step`, W =
 * bf16(master). */
int mt_host_adam(uint16_t* w, uint16_t* g, float* master, float* m, float* v, const uint16_t* gsrc, int64_t n,
                 int64_t step, float lr, float beta1, float beta2, float eps, int32_t threads);
/* The production gradient accumulation of micro-batch steps over n elements:
 * g[i] <- bf16_RNE(f32(g[i]) + f32(src[i])). */
int mt_host_accum(uint16_t* g, const uint16_t* src, int64_t n, int32_t threads);
/* Initialise one unit tile (16 * mt_unit_elems bytes) as mt_init would. */
int mt_host_init_unit(const mt_shape* shape, int32_t unit, uint64_t seed, float init_std, int32_t threads,
                      void* tile, uint64_t tile_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MT_KERNELS_H */
