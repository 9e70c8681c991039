// The streaming engine: context, device arena, streams and events, the
// visit schedule of a step, the stateless layer template and its Bind.
#pragma once
#include <hip/hip_runtime.h>

#include <deque>
#include <memory>
#include <vector>

#include "host.h"
#include "kernels.h"

namespace mt {

// Kernel timing sites (profile_kernels).
enum Site {
    S_RMS1_FWD, S_GEMM_QKV, S_ROPE_FWD, S_ATTN_FWD, S_GEMM_O, S_RMS2_FWD, S_GEMM_GATEUP,
    S_SWIGLU_FWD, S_GEMM_DOWN,
    S_GEMM_DOWN_DX, S_GEMM_DOWN_DW, S_SWIGLU_BWD, S_GEMM_GATEUP_DX, S_GEMM_GATEUP_DW,
    S_RMS2_BWD, S_GEMM_O_DX, S_GEMM_O_DW, S_ATTN_BWD, S_ROPE_BWD, S_GEMM_QKV_DX,
    S_GEMM_QKV_DW, S_RMS1_BWD,
    S_HEAD_RMS_FWD, S_HEAD_LOGITS, S_HEAD_CE, S_HEAD_DX, S_HEAD_DW, S_HEAD_RMS_BWD,
    S_HEAD_MISC,
    N_SITES
};
const char* site_name(int s);

// Views of one decoder layer's tensors inside a weight slot (or a gradient
// buffer): the Bind of a stateless template to streamed memory.
struct LayerView {
    uint16_t *g1, *wqkv, *wo, *g2, *wgu, *wd;
};
struct HeadView {
    uint16_t *gf, *eout;
};
LayerView bind_layer(const Layout& lay, void* base);
HeadView bind_head(const Layout& lay, void* base);

// Device activations of one layer at the workspace's maximum token count.
struct Workspace {
    int64_t maxT = 0;
    uint16_t *x[2] = {}, *xL = nullptr;
    // Backward inputs with checkpoints on the host: two banks of k buffers
    // (k = checkpoint interval), bank b buffer i = input of a block's layer i.
    std::vector<uint16_t*> xc;
    uint16_t* ckpt_dev = nullptr;  // [L+1][maxT x d] when checkpoints stay on the GPU
    uint16_t *n1, *qkv, *o, *n2, *gu, *m;
    // attention output and log-sum-exp buffers: [0] = o, lse; [1] a second
    // pair with checkpointed attention (alternate layers, so a layer's
    // checkpoint copy or restore overlaps the neighbouring layer's visit)
    uint16_t* oa[2] = {};
    float* lsea[2] = {};
    uint16_t* do16;  // attention backward: dO scaled by 2^k, fp16
    float* h1;  // residual stream inside a layer, kept in fp32
    // logit path: fp16 copies of n1 and Wqkv, fp32 QKV projection before RoPE
    uint16_t *n1h, *w16;
    float* qkv32;
    float *rstd1, *rstd2, *lse;
    uint16_t *dy[2], *dm, *dgu, *dn, *dh1, *dout, *dqkv;
    // reduction-contiguous copies of the backward products' operands
    uint16_t *tA, *tB;
    uint64_t tA_bytes = 0;  // also the dK/dV split partials of the attention backward (tA is idle then)
                            // and the fp32 partial tiles of split direct-form GEMMs (idle then too)
    float *dsum, *partial;
    float2* rope_tab;
    int32_t* labels;
    // head
    int64_t head_chunk = 0;
    uint16_t *nf, *dnf, *dlogits;
    float *rstdf, *logits, *deout_acc, *loss_rows, *loss;
    // head streamed in E_out row chunks: fp32 dnf accumulated over the
    // chunks, running max / sum of exp / label logit / LSE per token
    float *dnf_acc = nullptr, *ce_m = nullptr, *ce_l = nullptr, *ce_z = nullptr, *ce_lse = nullptr;
    uint32_t* ovf = nullptr;  // fp16 range guard: values saturated in this step
    uint32_t* amax = nullptr;  // attention backward: partial maxima of |dO|, |v| (ATTN_AMAX_BYTES)
    uint64_t bytes = 0;
};

struct Ctx;

}  // namespace mt
