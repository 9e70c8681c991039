// Stateless C entry points: error strings, tensor descriptions, site names,
// and the test-only kernel entries declared in include/mt_kernels.h.
#include <string.h>

#include "../../include/mt.h"
#include "../../include/mt_kernels.h"
#include "engine.h"
#include "host.h"

extern "C" {

const char* mt_strerror(int s) {
    switch (s) {
        case MT_OK: return "ok";
        case MT_E_INVAL: return "invalid argument";
        case MT_E_NOMEM: return "out of memory (host, pinned or device arena)";
        case MT_E_HIP: return "HIP runtime error";
        case MT_E_STATE: return "context failed earlier";
        case MT_E_INTERNAL: return "host worker failure";
        case MT_E_IO: return "checkpoint file I/O error";
        default: return "unknown status";
    }
}

const char* mt_last_error(void) { return mt::last_error(); }

int mt_unit_tensors(const mt_shape* sh, int32_t unit) {
    int r = mt::validate_shape(sh);
    if (r != MT_OK) return r;
    if (unit < 0 || unit > sh->n_layers + 1) MT_FAIL(MT_E_INVAL, "unit %d out of range", unit);
    return unit < sh->n_layers ? 9 : (unit == sh->n_layers ? 2 : 1);
}

uint64_t mt_unit_elems(const mt_shape* sh, int32_t unit) {
    if (mt::validate_shape(sh) != MT_OK) return 0;
    if (unit < 0 || unit > sh->n_layers + 1) return 0;
    const mt::Layout lay = mt::make_layout(*sh);
    return uint64_t(lay.units[unit].elems);
}

int mt_tensor_desc(const mt_shape* sh, int32_t unit, int32_t idx, mt_tensor_info* out) {
    int r = mt::validate_shape(sh);
    if (r != MT_OK) return r;
    if (!out) MT_FAIL(MT_E_INVAL, "out is NULL");
    if (unit < 0 || unit > sh->n_layers + 1) MT_FAIL(MT_E_INVAL, "unit %d out of range", unit);
    const mt::Layout lay = mt::make_layout(*sh);
    const mt::UnitLayout& u = lay.units[unit];
    if (idx < 0 || idx >= u.ntensors) MT_FAIL(MT_E_INVAL, "tensor %d out of range for unit %d", idx, unit);
    const mt::TensorDesc& t = u.t[idx];
    memset(out, 0, sizeof(*out));
    strncpy(out->name, t.name, sizeof(out->name) - 1);
    out->offset_elems = uint64_t(t.off);
    out->rows = t.rows;
    out->cols = t.cols;
    out->dtype = MT_DTYPE_BF16;
    return MT_OK;
}

const char* mt_site_name(int32_t site) { return mt::site_name(site); }

// ------------------------------------------------------ kernel entries ----
static int kst(hipError_t e, const char* what) {
    if (e == hipSuccess) return MT_OK;
    mt::set_error(mt::strfmt("%s: %s", what, hipGetErrorString(e)));
    return e == hipErrorInvalidValue ? MT_E_INVAL : MT_E_HIP;
}
#define S_(p) static_cast<hipStream_t>(p)
#define U16(p) static_cast<uint16_t*>(const_cast<void*>(p))
#define F32(p) static_cast<float*>(const_cast<void*>(p))

int mt_k_gemm(int32_t layout, int32_t epi, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
              int64_t ldc, const void* R, int64_t ldr, const void* Cacc, int64_t ldacc, int32_t M, int32_t N,
              int32_t K, void* stream) {
    if (layout < 0 || layout > 2 || epi < 0 || epi > 8) MT_FAIL(MT_E_INVAL, "bad layout or epilogue");
    mt::GemmArgs a{A, lda, B, ldb, C, ldc, R, ldr, static_cast<const float*>(Cacc), ldacc, M, N, K};
    return kst(mt::gemm(mt::GemmLayout(layout), mt::GemmEpi(epi), a, S_(stream)), "gemm");
}

int mt_k_gemm_split(int32_t layout, int32_t epi, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                    int64_t ldc, const void* R, int64_t ldr, const void* Cacc, int64_t ldacc, int32_t M, int32_t N,
                    int32_t K, void* ws, int64_t ws_bytes, int32_t splits, void* stream) {
    if (layout < 0 || layout > 2 || epi < 0 || epi > 8) MT_FAIL(MT_E_INVAL, "bad layout or epilogue");
    if (splits < 0 || splits > 64 || ws_bytes < 0) MT_FAIL(MT_E_INVAL, "bad split count or scratch size");
    if (ws && (reinterpret_cast<uintptr_t>(ws) & 15)) MT_FAIL(MT_E_INVAL, "scratch not 16-byte aligned");
    mt::GemmArgs a{A, lda, B, ldb, C, ldc, R, ldr, static_cast<const float*>(Cacc), ldacc, M, N, K};
    a.ws = static_cast<float*>(ws);
    a.ws_bytes = ws ? uint64_t(ws_bytes) : 0;
    a.force_splits = splits;
    return kst(mt::gemm(mt::GemmLayout(layout), mt::GemmEpi(epi), a, S_(stream)), "gemm_split");
}

int mt_k_gemm_split_plan(int64_t M, int64_t N, int64_t K, int64_t ws_bytes, int32_t* n_full, int32_t* splits,
                         int32_t* ksteps) {
    if (M <= 0 || N <= 0 || K <= 0 || ws_bytes < 0 || !n_full || !splits || !ksteps)
        MT_FAIL(MT_E_INVAL, "bad split plan arguments");
    const mt::GemmSplit sp = mt::gemm_split_plan(M, N, K, uint64_t(ws_bytes));
    *n_full = sp.n_full;
    *splits = sp.splits;
    *ksteps = sp.kper;
    return MT_OK;
}

int mt_k_gemm_amax(int32_t layout, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                   int32_t M, int32_t N, int32_t K, void* amax, void* stream) {
    if (layout < 0 || layout > 2) MT_FAIL(MT_E_INVAL, "bad layout");
    mt::GemmArgs a{A, lda, B, ldb, C, ldc, nullptr, 0, nullptr, 0, M, N, K};
    a.amax = static_cast<uint32_t*>(amax);
    const hipError_t e = mt::gemm(mt::GemmLayout(layout), mt::EPI_BF16_AMAX, a, S_(stream));
    if (e == hipErrorNotSupported) MT_FAIL(MT_E_INVAL, "gemm_amax: the direct form does not take this shape");
    return kst(e, "gemm_amax");
}

int mt_k_rmsnorm_fwd(const void* x, int32_t x_f32, const void* gamma, void* n, void* n_f16, void* rstd, int32_t T,
                     int32_t d, float eps, void* fp16_ovf, void* stream) {
    return kst(mt::rmsnorm_fwd(x, x_f32 != 0, U16(gamma), U16(n), n_f16 ? U16(n_f16) : nullptr, F32(rstd), T, d, eps,
                               S_(stream), static_cast<uint32_t*>(fp16_ovf)),
               "rmsnorm_fwd");
}

int64_t mt_k_rmsnorm_bwd_scratch_elems(int32_t T, int32_t d) { return mt::rmsnorm_bwd_partial_elems(T, d); }

int mt_k_rmsnorm_bwd(const void* dn, const void* x, int32_t x_f32, const void* gamma, const void* rstd,
                     const void* resid, void* dx, void* dgamma, void* scratch, int32_t T, int32_t d, void* stream) {
    return kst(mt::rmsnorm_bwd(U16(dn), x, x_f32 != 0, U16(gamma), F32(rstd), resid ? U16(resid) : nullptr, U16(dx),
                               U16(dgamma), F32(scratch), T, d, S_(stream)),
               "rmsnorm_bwd");
}

int mt_k_rmsnorm_bwd_noalloc(const void* dn, const void* x, int32_t x_f32, const void* gamma, const void* rstd,
                             const void* resid, void* dx, void* dgamma, int32_t T, int32_t d, void* stream) {
    if (T > 0 && d > 0 && mt::rmsnorm_bwd_partial_elems(T, d) > mt::RMSNORM_NOALLOC_FLOATS)
        MT_FAIL(MT_E_INVAL, "rmsnorm_bwd_noalloc: T = %d x d = %d needs %lld partial floats, more than the %lld of "
                "the static buffer", T, d, (long long)mt::rmsnorm_bwd_partial_elems(T, d),
                (long long)mt::RMSNORM_NOALLOC_FLOATS);
    return kst(mt::rmsnorm_bwd_noalloc(U16(dn), x, x_f32 != 0, U16(gamma), F32(rstd), resid ? U16(resid) : nullptr,
                                       U16(dx), U16(dgamma), T, d, S_(stream)),
               "rmsnorm_bwd_noalloc");
}

int mt_k_rope(void* qkv, int64_t ld, void* table, int32_t T, int32_t S, int32_t n_rot_heads, int32_t hd,
              float base, int32_t dir, void* stream) {
    hipError_t e = mt::rope_table(static_cast<float2*>(table), S, hd, base, S_(stream));
    if (e != hipSuccess) return kst(e, "rope_table");
    return kst(mt::rope_apply(U16(qkv), ld, static_cast<float2*>(table), T, S, n_rot_heads, hd, dir, S_(stream)),
               "rope_apply");
}

int mt_k_qkv_rope_cvt_vmax(const void* in, int64_t ldin, void* out, int64_t ldout, void* table, int32_t T, int32_t S,
                           int32_t n_rot_heads, int32_t n_heads, int32_t hd, float base, void* fp16_ovf, void* amax,
                           void* stream) {
    if (!amax || (reinterpret_cast<uintptr_t>(amax) & 255)) MT_FAIL(MT_E_INVAL, "qkv_rope_cvt_vmax: bad amax");
    if (S <= 0 || (hd & 15)) MT_FAIL(MT_E_INVAL, "qkv_rope_cvt_vmax: bad shape");
    hipError_t e = mt::rope_table(static_cast<float2*>(table), S, hd, base, S_(stream));
    if (e != hipSuccess) return kst(e, "rope_table");
    return kst(mt::qkv_rope_cvt(F32(in), ldin, U16(out), ldout, nullptr, 0, static_cast<float2*>(table), T, S,
                                n_rot_heads, n_heads, hd, S_(stream), static_cast<uint32_t*>(fp16_ovf),
                                static_cast<uint32_t*>(amax)),
               "qkv_rope_cvt_vmax");
}

int mt_k_qkv_rope_cvt(const void* in, int64_t ldin, void* out, int64_t ldout, void* out_bf16, int64_t ld_bf16,
                      void* table, int32_t T, int32_t S, int32_t n_rot_heads, int32_t n_heads, int32_t hd, float base,
                      void* fp16_ovf, void* stream) {
    hipError_t e = mt::rope_table(static_cast<float2*>(table), S, hd, base, S_(stream));
    if (e != hipSuccess) return kst(e, "rope_table");
    return kst(mt::qkv_rope_cvt(F32(in), ldin, U16(out), ldout, static_cast<uint16_t*>(out_bf16), ld_bf16,
                                static_cast<float2*>(table), T, S, n_rot_heads, n_heads, hd, S_(stream),
                                static_cast<uint32_t*>(fp16_ovf)),
               "qkv_rope_cvt");
}

int mt_k_bf16_to_f16(const void* x, void* y, int64_t n, void* fp16_ovf, void* stream) {
    return kst(mt::bf16_to_f16(U16(x), U16(y), n, S_(stream), static_cast<uint32_t*>(fp16_ovf)), "bf16_to_f16");
}

int mt_k_swiglu_fwd(const void* gu, void* m, int32_t T, int32_t F, void* stream) {
    return kst(mt::swiglu_fwd(U16(gu), U16(m), T, F, S_(stream)), "swiglu_fwd");
}

int mt_k_swiglu_bwd(const void* dm, const void* gu, void* dgu, int32_t T, int32_t F, void* stream) {
    return kst(mt::swiglu_bwd(U16(dm), U16(gu), U16(dgu), T, F, S_(stream)), "swiglu_bwd");
}

int mt_k_attn_fwd(const void* qkv, int64_t ld, void* o, int64_t ldo, void* lse, int32_t B, int32_t S, int32_t Hq,
                  int32_t Hkv, int32_t hd, void* fp16_ovf, void* stream) {
    mt::AttnArgs a{U16(qkv), ld, U16(o), ldo, F32(lse), B, S, Hq, Hkv, hd, static_cast<uint32_t*>(fp16_ovf)};
    return kst(mt::attn_fwd(a, S_(stream)), "attn_fwd");
}

int64_t mt_k_attn_bwd_work_bytes(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t hd) {
    if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || hd <= 0 || Hq % Hkv) return 0;
    return mt::attn_bwd_work_bytes(B, S, Hq, Hkv, hd);
}

int32_t mt_k_attn_dkdv_splits(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t hd, int32_t head_splits) {
    if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || hd <= 0 || Hq % Hkv || head_splits < 0) return 0;
    return mt::attn_dkdv_splits(B, S, Hq, Hkv, hd, mt::attn_bwd_part_elems(B, S, Hq, Hkv, hd), head_splits);
}

int mt_k_attn_bwd(const void* qkv, int64_t ld, const void* o, const void* dout, int64_t ldo, const void* lse,
                  void* work, void* dqkv, int64_t ldd, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t hd,
                  void* dqk32, int64_t ld32, int32_t head_splits, int32_t dq_form, void* fp16_ovf, void* stream) {
    if (!work || (reinterpret_cast<uintptr_t>(work) & 255)) MT_FAIL(MT_E_INVAL, "attn_bwd: work must be 256-byte aligned");
    if (head_splits < 0) MT_FAIL(MT_E_INVAL, "attn_bwd: head_splits must be >= 0");
    if (dq_form < 0 || dq_form > 2) MT_FAIL(MT_E_INVAL, "attn_bwd: dq_form must be 0, 1 or 2");
    if (dq_form == 2 && mt::attn_ds_bytes(B, S, Hq) == 0)
        MT_FAIL(MT_E_INVAL, "attn_bwd: this shape does not take the stored-dS form of dQ");
    mt::AttnBwdArgs a{U16(qkv), ld, U16(o), U16(dout), ldo, F32(lse), nullptr, nullptr, nullptr, U16(dqkv), ldd,
                      B, S, Hq, Hkv, hd, F32(dqk32), ld32, static_cast<uint32_t*>(fp16_ovf)};
    a.splits = head_splits;
    if (B > 0 && S > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && (hd == 64 || hd == 128))
        mt::attn_bwd_carve(work, B, S, Hq, Hkv, hd, a, dq_form != 1);
    return kst(mt::attn_bwd(a, S_(stream)), "attn_bwd");
}

int mt_k_attn_bwd_rope(const void* qkv, int64_t ld, const void* o, const void* dout, int64_t ldo, const void* lse,
                       void* work, void* dqkv, int64_t ldd, int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t hd,
                       void* dqk32, int64_t ld32, int32_t head_splits, int32_t dq_form, void* fp16_ovf, void* table,
                       float base, int32_t amax_ready, void* stream) {
    if (!table || (reinterpret_cast<uintptr_t>(table) & 15)) MT_FAIL(MT_E_INVAL, "attn_bwd_rope: bad table");
    if (!work || (reinterpret_cast<uintptr_t>(work) & 255)) MT_FAIL(MT_E_INVAL, "attn_bwd: work must be 256-byte aligned");
    if (head_splits < 0) MT_FAIL(MT_E_INVAL, "attn_bwd: head_splits must be >= 0");
    if (dq_form < 0 || dq_form > 2) MT_FAIL(MT_E_INVAL, "attn_bwd: dq_form must be 0, 1 or 2");
    if (dq_form == 2 && mt::attn_ds_bytes(B, S, Hq) == 0)
        MT_FAIL(MT_E_INVAL, "attn_bwd: this shape does not take the stored-dS form of dQ");
    if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || (hd != 64 && hd != 128))
        MT_FAIL(MT_E_INVAL, "attn_bwd_rope: bad shape");
    if (base < 0.f) MT_FAIL(MT_E_INVAL, "attn_bwd_rope: base must be > 0, or 0 for a table computed before");
    if (base > 0.f) {
        const hipError_t e = mt::rope_table(static_cast<float2*>(table), S, hd, base, S_(stream));
        if (e != hipSuccess) return kst(e, "rope_table");
    }
    mt::AttnBwdArgs a{U16(qkv), ld, U16(o), U16(dout), ldo, F32(lse), nullptr, nullptr, nullptr, U16(dqkv), ldd,
                      B, S, Hq, Hkv, hd, F32(dqk32), ld32, static_cast<uint32_t*>(fp16_ovf)};
    a.splits = head_splits;
    a.rope_tab = static_cast<const float2*>(table);
    a.amax_ready = amax_ready != 0;
    mt::attn_bwd_carve(work, B, S, Hq, Hkv, hd, a, dq_form != 1);
    return kst(mt::attn_bwd(a, S_(stream)), "attn_bwd_rope");
}

int mt_k_rope_f32_bf16(const void* in, int64_t ldin, void* out, int64_t ldout, void* table, int32_t T, int32_t S,
                       int32_t n_rot_heads, int32_t hd, float base, int32_t dir, void* stream) {
    hipError_t e = mt::rope_table(static_cast<float2*>(table), S, hd, base, S_(stream));
    if (e != hipSuccess) return kst(e, "rope_table");
    return kst(mt::rope_f32_to_bf16(F32(in), ldin, U16(out), ldout, static_cast<float2*>(table), T, S, n_rot_heads,
                                    hd, dir, S_(stream)),
               "rope_f32_to_bf16");
}

int mt_k_ce(const void* logits, const void* labels, void* loss_rows, void* dlogits, int32_t Tc, int32_t V,
            float inv_T, void* stream) {
    return kst(mt::ce_fwd_bwd(F32(logits), static_cast<const int32_t*>(labels), F32(loss_rows), U16(dlogits), Tc, V,
                              inv_T, S_(stream)),
               "ce_fwd_bwd");
}

int mt_k_mean(const void* x, void* out, int32_t n, void* stream) {
    return kst(mt::mean_reduce(F32(x), F32(out), n, S_(stream)), "mean_reduce");
}

int mt_k_transpose16(const void* src, int64_t lds, void* dst, int64_t ldd, int32_t R, int32_t C, int32_t f16_to_bf16,
                     void* stream) {
    return kst(mt::transpose16(U16(src), lds, U16(dst), ldd, R, C, S_(stream), f16_to_bf16 != 0), "transpose16");
}

int mt_k_f32_to_bf16(const void* x, void* y, int64_t n, void* stream) {
    return kst(mt::f32_to_bf16(F32(x), U16(y), n, S_(stream)), "f32_to_bf16");
}

// Host Adam on caller arrays (no GPU): the production update of the store.
int mt_host_adam(uint16_t* w, uint16_t* g, float* master, float* m, float* v, const uint16_t* gsrc, int64_t n,
                 int64_t step, float lr, float beta1, float beta2, float eps, int32_t threads) {
    if (!w || !g || !master || !m || !v || !gsrc || n < 0 || step < 1) MT_FAIL(MT_E_INVAL, "bad host Adam arguments");
    mt_options o;
    mt_default_options(&o);
    o.lr = lr;
    o.beta1 = beta1;
    o.beta2 = beta2;
    o.adam_eps = eps;
    const mt::AdamStep a = mt::adam_step_params(o, step);
    mt::TilePtrs p{w, g, master, m, v};
    mt::ThreadPool pool(threads > 0 ? threads : 1);
    mt::adam_unit(pool, p, gsrc, n, a);
    return MT_OK;
}

// Host gradient accumulation on caller arrays (no GPU).
int mt_host_accum(uint16_t* g, const uint16_t* src, int64_t n, int32_t threads) {
    if (!g || !src || n < 0) MT_FAIL(MT_E_INVAL, "bad host accumulation arguments");
    mt::ThreadPool pool(threads > 0 ? threads : 1);
    mt::accum_unit(pool, g, src, n);
    return MT_OK;
}

// Host init of one synthetic tensor stream, for tests of determinism.
int mt_host_init_unit(const mt_shape* sh, int32_t unit, uint64_t seed, float std_, int32_t threads, void* tile,
                      uint64_t tile_bytes) {
    int r = mt::validate_shape(sh);
    if (r != MT_OK) return r;
    if (unit < 0 || unit > sh->n_layers + 1 || !tile) MT_FAIL(MT_E_INVAL, "bad unit or tile");
    mt::Layout lay = mt::make_layout(*sh);
    if (tile_bytes < uint64_t(lay.units[unit].tile_bytes())) MT_FAIL(MT_E_INVAL, "tile buffer too small");
    // Treat the caller buffer as a one-tile store.
    std::vector<int64_t> off(lay.units.size(), 0);
    lay.tile_off = off;
    mt::ThreadPool pool(threads > 0 ? threads : 1);
    mt::init_unit(pool, static_cast<uint8_t*>(tile), lay, unit, seed, std_);
    return MT_OK;
}

}  // extern "C"
