// The layer-streamed training step.
//
// Pages cited:
//   [Review]  MegaTrain review, dimensionstp.github.io/study-concept/megatrain/
//   [Hotdry]  MegaTrain checkpoint strategy and communication overlap, blog.hotdry.top
//   [Lilting] MegaTrain article, lilting.ch
//   [Peter]   MegaTrain translated abstract and technical details, peter-blog.pages.dev
//   [Argon]   "Training 100B models on a single GPU ...", argonsys.com
//
// A step is a sequence of visits: forward of layers 0..L-1, the LM head
// (forward and backward fused), then backward of layers L-1..0, each
// backward visit first recomputing its layer's forward from the stored layer
// input ([Review] 3-2 item 2; [Argon] "Block-Wise Recomputation", here with
// a checkpoint interval of one layer).  Each visit binds a unit's weights:
//   pack   host thread copies the unit's BF16 W from the pageable store into
//          one of two pinned staging buffers ([Review] 3-2 item 4, JIT packing);
//   H2D    weight stream copies staging -> a GPU weight slot after that slot
//          is released, and records Weights-Ready ([Hotdry] "事件驱动同步协议");
//   Bind   compute stream waits Weights-Ready and binds tensor views of the
//          slot to the stateless layer template ([Lilting] "Stateless Layer
//          Templates"; [Peter] stateless template section);
//   G out  backward writes BF16 gradients into a gradient buffer and records
//          Backward-Done; the gradient stream copies them into a free pinned
//          slab and records Buffer-Free, and a host thread waits on the slab,
//          unpacks it into the store and runs Adam for that unit ([Hotdry]
//          K=12 slab pool and background CPU thread).
// With two slots the H2D of visit i+1 overlaps the compute of visit i and the
// D2H of visit i-1 ([Review] 3-2 item 3; [Peter] "管線雙緩衝執行引擎").
// Layer inputs are checkpointed to pinned host memory on the gradient stream,
// which is idle in forward, and copied back with the weights in backward.
#include "engine.h"

#include <algorithm>
#include <array>
#include <chrono>
#include <cstdlib>
#include <cstring>
#include <sys/mman.h>

namespace mt {

const char* site_name(int s) {
    static const char* names[N_SITES] = {
        "rms1_fwd", "gemm_qkv", "rope_fwd", "attn_fwd", "gemm_o", "rms2_fwd", "gemm_gateup",
        "swiglu_fwd", "gemm_down",
        "gemm_down_dx", "gemm_down_dw", "swiglu_bwd", "gemm_gateup_dx", "gemm_gateup_dw",
        "rms2_bwd", "gemm_o_dx", "gemm_o_dw", "attn_bwd", "rope_bwd", "gemm_qkv_dx",
        "gemm_qkv_dw", "rms1_bwd",
        "head_rms_fwd", "head_logits", "head_ce", "head_dx", "head_dw", "head_rms_bwd",
        "head_misc"};
    return (s >= 0 && s < N_SITES) ? names[s] : nullptr;
}

LayerView bind_layer(const Layout& lay, void* base) {
    const UnitLayout& u = lay.units[0];
    uint16_t* b = static_cast<uint16_t*>(base);
    return LayerView{b + u.t[T_G1].off, b + u.t[T_WQ].off, b + u.t[T_WO].off,
                     b + u.t[T_G2].off, b + u.t[T_WG].off, b + u.t[T_WD].off};
}
HeadView bind_head(const Layout& lay, void* base) {
    const UnitLayout& u = lay.units[lay.head()];
    uint16_t* b = static_cast<uint16_t*>(base);
    return HeadView{b + u.t[T_GF].off, b + u.t[T_EOUT].off};
}

namespace {

using Clock = std::chrono::steady_clock;
double ms_since(Clock::time_point t0) {
    return std::chrono::duration<double, std::milli>(Clock::now() - t0).count();
}
uint64_t al256(uint64_t x) { return (x + 255) & ~uint64_t(255); }
uint64_t al4k(uint64_t x) { return (x + 4095) & ~uint64_t(4095); }

struct Ev {
    hipEvent_t e = nullptr;
    bool rec = false;
};

// Device arena plan; with base == nullptr only sizes are computed.
struct ArenaPlan {
    uint64_t slot_bytes = 0, total = 0;
    int n_slots = 2, n_garea = 2;
    std::vector<uint64_t> wslot, garea, resident;  // offsets
    uint64_t ws_off = 0;
};

struct Carver {
    uint64_t off = 0;
    uint8_t* base = nullptr;
    template <class T>
    T* take(uint64_t bytes) {
        const uint64_t o = off;
        off = al256(off + bytes);
        return base ? reinterpret_cast<T*>(base + o) : nullptr;
    }
};

int64_t head_chunk_of(const mt_options& o, int64_t T) {
    int64_t c = o.head_chunk > 0 ? o.head_chunk : std::min<int64_t>(T, 8192);
    return std::max<int64_t>(1, std::min<int64_t>(c, T));
}

// The LM head's E_out in row chunks (head_vocab_chunk != 0).  Chunk c covers
// the head tile's elements [start, start + elems): chunk 0 also holds gf and
// the padding before E_out, so every element the head updates is in exactly
// one chunk.  Empty when the head streams as one unit.
struct HeadChunk {
    int64_t start, elems;  // head-tile element range
    int row0, rows;        // vocabulary rows of E_out
};
std::vector<HeadChunk> head_chunks(const Layout& lay, const mt_options& o) {
    std::vector<HeadChunk> v;
    if (o.head_vocab_chunk == 0) return v;
    const int64_t d = lay.sh.d_model, V = lay.sh.vocab;
    const int64_t e0 = lay.units[lay.head()].t[T_EOUT].off;
    int64_t rows = o.head_vocab_chunk;
    if (rows < 0) {
        int64_t lmax = 0;
        for (int l = 0; l < lay.L(); ++l) lmax = std::max(lmax, lay.units[l].elems);
        rows = std::max<int64_t>(8, ((lmax - e0) / d) & ~int64_t(7));
    }
    rows = std::min(rows, V);
    for (int64_t r = 0; r < V; r += rows) {
        const int64_t n = std::min(rows, V - r);
        const int64_t start = r == 0 ? 0 : e0 + r * d;
        v.push_back({start, e0 + (r + n) * d - start, int(r), int(n)});
    }
    return v;
}

// Elements of the largest block a weight slot receives.
int64_t stream_elems_max(const Layout& lay, const mt_options& o) {
    const auto ch = head_chunks(lay, o);
    if (ch.empty()) return lay.max_stream_elems;
    int64_t m = 0;
    for (int l = 0; l < lay.L(); ++l) m = std::max(m, lay.units[l].elems);
    for (const HeadChunk& c : ch) m = std::max(m, c.elems);
    return m;
}

// One layer's checkpointed attention: the fp16 output, then the fp32 log-sum-exp.
uint64_t attn_ckpt_o_bytes(const mt_shape& sh, uint64_t T) { return al4k(T * sh.n_heads * sh.head_dim * 2); }
uint64_t attn_ckpt_bytes(const mt_shape& sh, uint64_t T) {
    return attn_ckpt_o_bytes(sh, T) + al4k(T * sh.n_heads * 4);
}

// Checkpoint interval, capped at the depth, and the host ring entries it needs.
int ckpt_k(const mt_options& o, const mt_shape& sh) { return std::max(1, std::min(o.ckpt_interval, sh.n_layers)); }
int ckpt_slots(const mt_options& o, const mt_shape& sh) {
    const int k = ckpt_k(o, sh);
    return (sh.n_layers + k - 1) / k;
}

void plan_workspace(const Layout& lay, const mt_options& o, Carver& cv, Workspace& ws) {
    const mt_shape& sh = lay.sh;
    const int64_t T = int64_t(o.max_batch) * o.max_seq;
    const int64_t d = sh.d_model, F = sh.ffn_dim, V = sh.vocab;
    const int64_t nq = int64_t(sh.n_heads) * sh.head_dim;
    const int64_t nqkv = int64_t(sh.n_heads + 2 * sh.n_kv_heads) * sh.head_dim;
    const uint64_t td = uint64_t(T) * d * 2;
    ws.maxT = T;
    if (o.ckpt_on_host) {
        ws.x[0] = cv.take<uint16_t>(td);
        ws.x[1] = cv.take<uint16_t>(td);
        ws.xc.assign(size_t(2 * ckpt_k(o, sh)), nullptr);
        for (auto& b : ws.xc) b = cv.take<uint16_t>(td);
    } else {
        ws.ckpt_dev = cv.take<uint16_t>(td * uint64_t(sh.n_layers + 1));
    }
    ws.n1 = cv.take<uint16_t>(td);
    ws.n1h = cv.take<uint16_t>(td);
    ws.w16 = cv.take<uint16_t>(uint64_t(nqkv) * d * 2);
    ws.qkv32 = cv.take<float>(uint64_t(T) * nqkv * 4);
    ws.h1 = cv.take<float>(td * 2);
    ws.n2 = cv.take<uint16_t>(td);
    ws.qkv = cv.take<uint16_t>(uint64_t(T) * nqkv * 2);
    ws.do16 = cv.take<uint16_t>(uint64_t(T) * nq * 2);
    ws.dqkv = cv.take<uint16_t>(uint64_t(T) * nqkv * 2);
    ws.o = cv.take<uint16_t>(uint64_t(T) * nq * 2);
    ws.dout = cv.take<uint16_t>(uint64_t(T) * nq * 2);
    ws.gu = cv.take<uint16_t>(uint64_t(T) * 2 * F * 2);
    ws.dgu = cv.take<uint16_t>(uint64_t(T) * 2 * F * 2);
    ws.m = cv.take<uint16_t>(uint64_t(T) * F * 2);
    ws.dm = cv.take<uint16_t>(uint64_t(T) * F * 2);
    ws.dy[0] = cv.take<uint16_t>(td);
    ws.dy[1] = cv.take<uint16_t>(td);
    ws.dn = cv.take<uint16_t>(td);
    ws.dh1 = cv.take<uint16_t>(td);
    {
        const uint64_t T8 = uint64_t((T + 7) & ~int64_t(7));  // token rows padded for the dW products
        const uint64_t ta = uint64_t(std::max({d, 2 * F, nqkv})) * T8;
        // the chunked head's dX transposes one E_out chunk (d x its rows)
        uint64_t head_t = 0;
        for (const HeadChunk& c : head_chunks(lay, o)) head_t = std::max<uint64_t>(head_t, uint64_t(d) * c.rows);
        const uint64_t tb = std::max({uint64_t(F) * std::max<uint64_t>(T8, uint64_t(2 * d)),
                                      uint64_t(std::max(nq, nqkv)) * std::max<uint64_t>(T8, uint64_t(d)),
                                      uint64_t(d) * T8, head_t});
        // tA also holds the attention backward's dK/dV split partials and
        // its stored dS (it is idle then)
        // (at the largest batch x seq; smaller steps split more or recompute dQ
        // when their partials and dS do not fit)
        const uint64_t attn_b = uint64_t((attn_bwd_part_elems(o.max_batch, o.max_seq, sh.n_heads, sh.n_kv_heads,
                                                               sh.head_dim) * 4 + 255) & ~int64_t(255)) +
                                uint64_t(attn_ds_bytes(o.max_batch, o.max_seq, sh.n_heads));
        ws.tA_bytes = std::max<uint64_t>(ta * 2, attn_b);
        ws.tA = cv.take<uint16_t>(ws.tA_bytes);
        ws.tB = cv.take<uint16_t>(tb * 2);
    }
    ws.rstd1 = cv.take<float>(uint64_t(T) * 4);
    ws.rstd2 = cv.take<float>(uint64_t(T) * 4);
    ws.lse = cv.take<float>(uint64_t(T) * sh.n_heads * 4);
    ws.oa[0] = ws.oa[1] = ws.o;
    ws.lsea[0] = ws.lsea[1] = ws.lse;
    if (o.ckpt_attn) {
        ws.oa[1] = cv.take<uint16_t>(uint64_t(T) * nq * 2);
        ws.lsea[1] = cv.take<float>(uint64_t(T) * sh.n_heads * 4);
    }
    ws.dsum = cv.take<float>(uint64_t(T) * sh.n_heads * 4 * 2);
    ws.partial = cv.take<float>(uint64_t(rmsnorm_bwd_partial_elems(int(T), int(d))) * 4);
    ws.rope_tab = cv.take<float2>(uint64_t(o.max_seq) * (sh.head_dim / 2) * 8);
    ws.labels = cv.take<int32_t>(uint64_t(T) * 4);
    const int64_t tc = head_chunk_of(o, T);
    ws.head_chunk = tc;
    ws.nf = cv.take<uint16_t>(td);
    ws.dnf = cv.take<uint16_t>(td);
    ws.rstdf = cv.take<float>(uint64_t(T) * 4);
    // Vocabulary columns one logits block holds: all of V, or one E_out chunk.
    int64_t vc = V;
    const auto hch = head_chunks(lay, o);
    if (!hch.empty()) {
        vc = 0;
        for (const HeadChunk& c : hch) vc = std::max<int64_t>(vc, c.rows);
        ws.dnf_acc = cv.take<float>(uint64_t(T) * d * 4);
        ws.ce_m = cv.take<float>(uint64_t(T) * 4);
        ws.ce_l = cv.take<float>(uint64_t(T) * 4);
        ws.ce_z = cv.take<float>(uint64_t(T) * 4);
        ws.ce_lse = cv.take<float>(uint64_t(T) * 4);
    }
    ws.logits = cv.take<float>(uint64_t(tc) * vc * 4);
    ws.dlogits = cv.take<uint16_t>(uint64_t(tc) * vc * 2);
    ws.deout_acc = tc < T ? cv.take<float>(uint64_t(vc) * d * 4) : nullptr;
    ws.loss_rows = cv.take<float>(uint64_t(T) * 4);
    ws.loss = cv.take<float>(256);
    ws.ovf = cv.take<uint32_t>(256);
    ws.amax = cv.take<uint32_t>(ATTN_AMAX_BYTES);
}

// A direct-form product's tail-split scratch: tA, which no transpose holds
// while such a product runs (the fallbacks that transpose into tA get none).
GemmArgs split_ws(GemmArgs a, const Workspace& ws) {
    a.ws = reinterpret_cast<float*>(ws.tA);
    a.ws_bytes = ws.tA_bytes;
    return a;
}

ArenaPlan plan_arena(const Layout& lay, const mt_options& o, uint8_t* base, Workspace* ws) {
    ArenaPlan p;
    p.slot_bytes = o.slot_bytes_override ? al4k(o.slot_bytes_override)
                                         : al4k(uint64_t(stream_elems_max(lay, o)) * 2);
    p.n_slots = o.n_weight_slots;
    const bool combined = o.slot_mode == 1;
    p.n_garea = combined ? p.n_slots : 2;
    Carver cv;
    cv.base = base;
    for (int s = 0; s < p.n_slots; ++s) {
        p.wslot.push_back(cv.off);
        cv.take<uint8_t>(p.slot_bytes);
        if (combined) {
            p.garea.push_back(cv.off);
            cv.take<uint8_t>(p.slot_bytes);
        }
    }
    if (!combined)
        for (int g = 0; g < 2; ++g) {
            p.garea.push_back(cv.off);
            cv.take<uint8_t>(p.slot_bytes);
        }
    if (o.resident)
        for (int u = 0; u <= lay.head(); ++u) {
            p.resident.push_back(cv.off);
            cv.take<uint8_t>(al4k(uint64_t(lay.units[u].elems) * 2));
        }
    p.ws_off = cv.off;
    Workspace tmp;
    Workspace& w = ws ? *ws : tmp;
    if (o.workspace_bytes_override) {
        Carver probe;
        plan_workspace(lay, o, probe, tmp);
        const uint64_t need = probe.off;
        plan_workspace(lay, o, cv, w);
        cv.off = p.ws_off + std::max<uint64_t>(need, o.workspace_bytes_override);
    } else {
        plan_workspace(lay, o, cv, w);
    }
    w.bytes = cv.off - p.ws_off;
    p.total = cv.off;
    return p;
}

struct PinnedPlan {
    uint64_t staging = 0, slab = 0, ckpt = 0, io = 0, weights = 0, total = 0;
};
PinnedPlan plan_pinned(const Layout& lay, const mt_options& o, uint64_t slot_bytes) {
    PinnedPlan p;
    const uint64_t T = uint64_t(o.max_batch) * o.max_seq;
    p.staging = (o.pin_store || o.pin_weights) ? 0 : 2 * slot_bytes;
    p.weights = o.pin_weights ? uint64_t(lay.w_bytes) : 0;
    p.slab = uint64_t(o.n_grad_slabs) * slot_bytes;
    p.ckpt = o.ckpt_on_host ? al4k(T * lay.sh.d_model * 2) * ckpt_slots(o, lay.sh) : 0;
    if (o.ckpt_attn) p.ckpt += attn_ckpt_bytes(lay.sh, T) * uint64_t(lay.sh.n_layers);
    p.io = 2 * al4k(T * lay.sh.d_model * 2) + al4k(T * 4) + 4096;
    p.total = p.staging + p.slab + p.ckpt + p.io + p.weights;
    return p;
}

int validate_options(const mt_options* o) {
    if (!o) MT_FAIL(MT_E_INVAL, "options are NULL");
    if (o->max_batch < 1 || o->max_seq < 1) MT_FAIL(MT_E_INVAL, "max_batch and max_seq must be >= 1");
    if (int64_t(o->max_batch) * o->max_seq > (int64_t(1) << 30)) MT_FAIL(MT_E_INVAL, "max_batch*max_seq too large");
    if (o->n_weight_slots < 1 || o->n_weight_slots > 4) MT_FAIL(MT_E_INVAL, "n_weight_slots must be 1..4");
    if (o->n_grad_slabs < 1 || o->n_grad_slabs > 64) MT_FAIL(MT_E_INVAL, "n_grad_slabs must be 1..64");
    if (o->slot_mode != 0 && o->slot_mode != 1) MT_FAIL(MT_E_INVAL, "slot_mode must be 0 or 1");
    if (o->head_chunk < 0) MT_FAIL(MT_E_INVAL, "head_chunk must be >= 0");
    if (o->cross_step != 0 && o->cross_step != 1) MT_FAIL(MT_E_INVAL, "cross_step must be 0 or 1");
    if (o->ckpt_interval < 1) MT_FAIL(MT_E_INVAL, "ckpt_interval must be >= 1");
    if (o->ckpt_interval > 1 && !o->ckpt_on_host) MT_FAIL(MT_E_INVAL, "ckpt_interval > 1 needs ckpt_on_host = 1");
    if (o->pin_weights != 0 && o->pin_weights != 1) MT_FAIL(MT_E_INVAL, "pin_weights must be 0 or 1");
    if (o->pin_weights && o->pin_store) MT_FAIL(MT_E_INVAL, "pin_weights and pin_store exclude each other");
    if (o->head_vocab_chunk < -1 || (o->head_vocab_chunk > 0 && (o->head_vocab_chunk & 7)))
        MT_FAIL(MT_E_INVAL, "head_vocab_chunk must be -1, 0 or a positive multiple of 8");
    if (o->poison_released < 0 || o->poison_released > 1) MT_FAIL(MT_E_INVAL, "poison_released must be 0 or 1");
    if (o->poison_released && (o->slot_mode != 0 || o->resident))
        MT_FAIL(MT_E_INVAL, "poison_released needs slot_mode 0 and resident 0");
    if (o->keep_grads != 0 && o->keep_grads != 1) MT_FAIL(MT_E_INVAL, "keep_grads must be 0 or 1");
    if (o->ckpt_attn != 0 && o->ckpt_attn != 1) MT_FAIL(MT_E_INVAL, "ckpt_attn must be 0 or 1");
    if (o->ckpt_attn && (!o->ckpt_on_host || o->ckpt_interval != 1))
        MT_FAIL(MT_E_INVAL, "ckpt_attn needs ckpt_on_host = 1 and ckpt_interval = 1");
    if (!(o->lr >= 0.f) || !(o->beta1 >= 0.f && o->beta1 < 1.f) || !(o->beta2 >= 0.f && o->beta2 < 1.f) ||
        !(o->adam_eps > 0.f))
        MT_FAIL(MT_E_INVAL, "bad Adam hyper-parameters");
    return MT_OK;
}

}  // namespace

// ------------------------------------------------------------------------
struct Ctx {
    Layout lay;
    mt_options opt{};
    ArenaPlan plan;
    PinnedPlan pplan;
    Workspace ws;
    uint8_t* arena = nullptr;
    uint64_t arena_bytes = 0;
    // host
    uint8_t* store = nullptr;
    bool store_pinned = false;
    uint8_t* wblock = nullptr;  // page-locked W regions (pin_weights)
    uint8_t* staging[2] = {};
    std::vector<uint8_t*> slabs;
    uint8_t* ckpt_host = nullptr;
    uint8_t* attn_host = nullptr;  // ckpt_attn: per layer, o (fp16) then lse (fp32)
    uint16_t *x0_pin = nullptr, *dx0_pin = nullptr;
    int32_t* lab_pin = nullptr;
    float* loss_pin = nullptr;
    std::vector<uint8_t*> pinned_blocks;
    std::vector<float> ein_acc;        // fp32 scatter accumulator [V x d]
    std::vector<int32_t> ein_touched;  // rows with a non-zero gradient last step
    std::vector<char> ein_seen;        // rows touched so far in this step
    bool ein_clear_all = false;        // after a restore: the whole E_in gradient is stale
    std::vector<std::string> lazy_dir; // per unit: checkpoint directory still to load from (lazy restore)
    // streams and events
    hipStream_t st_c = nullptr, st_w = nullptr, st_g = nullptr;
    bool own[3] = {false, false, false};
    std::vector<Ev> wready, slot_free, bwd_done, buf_free, slab_done;
    Ev attn_ck_done[2], attn_buf_free[2];  // ckpt_attn: a buffer's D2H done / its last backward reader done
    Ev staging_free[2], xc_free[2], ckpt_done[2], xready, emb_ready, fwd_ckpt_all, dx0_done, loss_done,
        res_ready;
    std::vector<hipEvent_t> tev;  // timing events
    size_t tev_next = 0;
    // host threads
    std::unique_ptr<ThreadPool> pack_pool, adam_pool;
    std::thread slab_thread;
    std::mutex q_mu;
    std::condition_variable q_cv, free_cv;
    // One host job on a unit's gradient; slab < 0: the gradient is already
    // in the store's G region (the input embedding).  Carries its own step's
    // hyper-parameters: with cross_step it may run during the next step.
    // Modes: a one-micro-batch step copies the slab into G and runs Adam;
    // with micro-batches the first stores the slab into G, the middle ones
    // accumulate into G, the last accumulates and runs Adam.
    // JOB_ADAM_ROWS / JOB_ADAM_EXCEPT: the input embedding's update split
    // by rows (the rows the next batch gathers, then all the others).
    enum { JOB_ADAM, JOB_STORE, JOB_ACCUM, JOB_ACCUM_ADAM, JOB_ADAM_ROWS, JOB_ADAM_EXCEPT };
    struct Job {
        int unit, slab;
        int64_t elems;
        AdamStep a;
        int64_t step_id;  // the step (1-based) whose gradient this is
        int mode;
        int64_t off = 0;    // first tile element (a head chunk starts inside the tile)
        bool last = true;   // completes the unit's update of this step
        std::shared_ptr<const std::vector<int32_t>> rows;  // JOB_ADAM_ROWS / _EXCEPT
    };
    std::deque<Job> jobs;
    std::vector<int64_t> adam_gen;  // updates applied per unit
    double adam_wait_ms = 0.0;
    std::vector<int> free_slabs;
    std::vector<char> slab_landed;  // the slab's copy is known complete (set by the offload thread)
    bool emb_urgent = false;        // a thread waits for the input embedding's update
    bool stop = false;
    int jobs_pending = 0;
    int worker_status = MT_OK;
    std::string worker_error;
    double adam_ms_acc = 0.0, pack_ms = 0.0;
    AdamStep cur_adam{};
    // With cross_step the input embedding's update is held back until the
    // next step's tokens are known (or until anything else needs the store):
    // then the rows that step gathers are updated first, the others after.
    bool emb_deferred = false;
    AdamStep emb_adam{};
    int64_t emb_step_id = 0;
    int64_t emb_rows_issued = 0, emb_rows_done = 0;  // JOB_ADAM_ROWS jobs
    bool emb_split = false;  // this step's gathers follow a split update
    // schedule state
    std::vector<int> slot_unit;
    int slot_ptr = 0, staging_ptr = 0;
    int cached_rope_S = -1;
    int64_t step = 0;
    bool failed = false;
    // fault injection (host side): "pack:<unit>" or "slab:<unit>"
    int fault_pack = -1, fault_slab = -1;
    std::string trace_path;  // MT_TRACE: append every step's intervals as CSV
    struct HostRec {
        const char* what;
        int unit, aux;
        Clock::time_point a, b;
    };
    std::vector<HostRec> host_recs;  // host-side spans of the step (MT_TRACE)
    Clock::time_point step_clock0;
    void host_rec(const char* what, int unit, int aux, Clock::time_point a) {
        if (trace_path.empty()) return;
        std::lock_guard<std::mutex> lk(trace_mu);
        host_recs.push_back({what, unit, aux, a, Clock::now()});
    }
    std::mutex trace_mu;
    // Gradient offload thread.  It takes Backward-Done'd gradient areas in
    // visit order, acquires a slab, and issues each D2H only once the
    // previous one has completed: a D2H queued behind another one still in
    // flight was measured to run at a quarter of the link rate.  The compute
    // thread never blocks on the offload; it waits only until the request
    // that last used a gradient area (or, combined, a slot) has been issued,
    // so that the Buffer-Free event it then waits on is the right one.
    struct OffReq {
        int unit, ga, slot, mode;  // slot >= 0: combined W/G slot released after the copy
        void* gbase;
        uint64_t bytes;
        int64_t off = 0;   // first tile element of the copied range
        bool last = true;  // the unit's last range this step
    };
    std::thread off_thread;
    std::mutex off_mu;
    std::condition_variable off_cv;
    std::deque<OffReq> off_q;
    int64_t off_submitted = 0, off_issued = 0;
    bool off_stop = false;
    int off_status = MT_OK;
    std::string off_error;
    std::vector<hipEvent_t> off_tev;
    size_t off_tev_next = 0;
    std::vector<int64_t> ga_last_req, slot_last_req;
    int off_prev_slab = -1;
    void offload_worker();
    int wait_offload(int64_t seq);
    // timing records
    struct Interval {
        hipEvent_t a, b;
        int kind;  // 0 compute, 1 h2d, 2 d2h
        uint64_t bytes;
        int visit = -1, unit = -1;  // compute: the visit kind and unit
        int slot = -1;              // compute and weight copies: the weight slot
        int64_t seq = -1;           // gradient copies: the offload request; compute: the one it waited for
        int last_h2d = -1;          // compute: index of the last weight-stream copy it waited for
    };
    std::vector<Interval> intervals;
    std::vector<Interval> off_intervals;  // gradient copies, filled by the offload thread
    struct SiteRec {
        int site;
        hipEvent_t a, b;
    };
    std::vector<SiteRec> site_recs;
    hipEvent_t t_base = nullptr;
    bool timing = true;

    ~Ctx();
    int init(const mt_shape& sh, const mt_options& o, void* arena, uint64_t bytes, void* const streams[3]);
    int train_step(const int32_t* tokens, const int32_t* labels, int n_micro, int B, int S, float* loss,
                   mt_stats* stats);
    int layer_fwd(int layer, const void* x, void* y, int B, int S);
    int layer_bwd(int layer, const void* x, const void* dy, void* dx, void* gtile, int B, int S);

    // helpers
    hipError_t rec(Ev& e, hipStream_t s) {
        e.rec = true;
        return hipEventRecord(e.e, s);
    }
    hipError_t wait(hipStream_t s, const Ev& e) { return e.rec ? hipStreamWaitEvent(s, e.e, 0) : hipSuccess; }
    hipError_t hsync(const Ev& e) { return e.rec ? hipEventSynchronize(e.e) : hipSuccess; }
    hipEvent_t next_tev() {
        if (tev_next == tev.size()) {
            hipEvent_t e;
            if (hipEventCreate(&e) != hipSuccess) return nullptr;
            tev.push_back(e);
        }
        return tev[tev_next++];
    }
    hipError_t h2d(void* dst, const void* src, uint64_t bytes, hipStream_t s, int slot = -1) {
        hipEvent_t a = timing ? next_tev() : nullptr, b = timing ? next_tev() : nullptr;
        if (a) hipEventRecord(a, s);
        hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, s);
        if (b) hipEventRecord(b, s);
        if (a && b) {
            intervals.push_back({a, b, 1, bytes});
            intervals.back().slot = slot;
            last_h2d = int(intervals.size()) - 1;
        }
        return e;
    }
    int last_h2d = -1;  // index in intervals of the latest weight-stream copy
    hipError_t d2h(void* dst, const void* src, uint64_t bytes, hipStream_t s) {
        hipEvent_t a = timing ? next_tev() : nullptr, b = timing ? next_tev() : nullptr;
        if (a) hipEventRecord(a, s);
        hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, s);
        if (b) hipEventRecord(b, s);
        if (a && b) intervals.push_back({a, b, 2, bytes});
        return e;
    }
    // kernel sites
    template <class F>
    hipError_t site(int id, F&& f) {
        if (!opt.profile_kernels) return f();
        hipEvent_t a = next_tev(), b = next_tev();
        hipEventRecord(a, st_c);
        hipError_t e = f();
        hipEventRecord(b, st_c);
        site_recs.push_back({id, a, b});
        return e;
    }
    // ob: which attention output / log-sum-exp pair (ws.oa, ws.lsea) the
    // layer uses; attn_restored: that pair already holds the checkpointed
    // attention of this layer, so the recompute skips the attention forward.
    hipError_t fwd_layer(const LayerView& w, const uint16_t* x, uint16_t* y, int B, int S, bool need_y, int ob = 0,
                         bool attn_restored = false);
    hipError_t bwd_layer(const LayerView& w, const LayerView& g, const uint16_t* x, const uint16_t* dy,
                         uint16_t* dx, int B, int S, int ob = 0, bool attn_restored = false);
    hipError_t head(const HeadView& w, const HeadView& g, const uint16_t* xL, uint16_t* dy, int B, int S,
                    float inv_tokens);
    hipError_t head_chunk_fwd(const HeadChunk& ch, bool first, bool last, const void* wbase, const uint16_t* xL,
                              int B, int S);
    hipError_t head_chunk_bwd(const HeadChunk& ch, bool first, bool last, const void* wbase, void* gbase,
                              const uint16_t* xL, uint16_t* dy, int B, int S, float inv_tokens);
    hipError_t gemm_nn_t(const uint16_t* A, int64_t lda, const uint16_t* Bm, int64_t ldb, uint16_t* C, int64_t ldc,
                         int M, int N, int K);
    hipError_t gemm_tn_t(const uint16_t* A, int64_t lda, const uint16_t* Bm, int64_t ldb, uint16_t* C, int64_t ldc,
                         int M, int N, int K, bool b_f16 = false);
    hipError_t ensure_rope(int S);
    int pick_slot(int unit, bool* need_stream);
    // Stream W of `unit` (elements [e0, e0 + n), n < 0: all) into `slot`; the
    // slot then holds block `id` (id < 0: the unit).
    int stream_unit(int unit, int slot, int id = -1, int64_t e0 = 0, int64_t n = -1);
    void slab_worker();
    int acquire_slab();
    void enqueue_job(int unit, int slab, int mode, int64_t off = 0, int64_t elems = -1, bool last = true);
    int drain_jobs();
    int wait_adam(int unit);
    int ensure_loaded(int unit);
    int checkpoint_save(const std::string& dir);
    int checkpoint_restore(const std::string& dir, bool lazy);
    int hip_fail(hipError_t e, const char* what) {
        failed = true;
        set_error(strfmt("HIP error '%s' in %s", hipGetErrorString(e), what));
        return MT_E_HIP;
    }
};

#define HIPC(expr)                                              \
    do {                                                        \
        hipError_t e_ = (expr);                                 \
        if (e_ != hipSuccess) return hip_fail(e_, #expr);       \
    } while (0)
#define HIPR(expr)                                              \
    do {                                                        \
        hipError_t e_ = (expr);                                 \
        if (e_ != hipSuccess) return e_;                        \
    } while (0)

// ---------------------------------------------------------------- init ----
static uint8_t* pinned_alloc(Ctx* c, uint64_t bytes) {
    if (bytes == 0) return nullptr;
    void* p = nullptr;
    if (hipHostMalloc(&p, bytes, hipHostMallocDefault) != hipSuccess || !p) return nullptr;
    c->pinned_blocks.push_back(static_cast<uint8_t*>(p));
    return static_cast<uint8_t*>(p);
}

int Ctx::init(const mt_shape& sh, const mt_options& o, void* arena_, uint64_t bytes,
              void* const streams[3]) {
    opt = o;
    lay = make_layout(sh);
    plan = plan_arena(lay, opt, nullptr, nullptr);
    if (!arena_) MT_FAIL(MT_E_INVAL, "gpu_arena is NULL");
    if (reinterpret_cast<uintptr_t>(arena_) & 255) MT_FAIL(MT_E_INVAL, "gpu_arena must be 256-byte aligned");
    if (bytes < plan.total)
        MT_FAIL(MT_E_NOMEM, "gpu arena of %llu bytes is smaller than the %llu needed",
                (unsigned long long)bytes, (unsigned long long)plan.total);
    if (plan.slot_bytes < uint64_t(stream_elems_max(lay, opt)) * 2)
        MT_FAIL(MT_E_INVAL, "slot_bytes_override is below the largest streamed block (%lld bytes)",
                (long long)(stream_elems_max(lay, opt) * 2));
    arena = static_cast<uint8_t*>(arena_);
    arena_bytes = bytes;
    plan = plan_arena(lay, opt, arena, &ws);
    pplan = plan_pinned(lay, opt, plan.slot_bytes);

    if (const char* f = getenv("MT_TRACE")) trace_path = f;
    if (const char* f = getenv("MT_FAULT")) {
        if (!strncmp(f, "pack:", 5)) fault_pack = atoi(f + 5);
        if (!strncmp(f, "slab:", 5)) fault_slab = atoi(f + 5);
    }

    // Host threads.
    int nth = opt.host_threads > 0 ? opt.host_threads : int(std::thread::hardware_concurrency());
    nth = std::max(1, nth);
    // Adam is the host's bandwidth-bound bulk (30 B/param) and gets every
    // thread; packing runs in short bursts on a quarter of them besides.
    const int npack = std::max(1, nth / 4);
    pack_pool.reset(new ThreadPool(npack));
    adam_pool.reset(new ThreadPool(nth));

    // Host master store: pageable, huge pages where the kernel allows.
    if (opt.pin_store) {
        void* p = nullptr;
        if (hipHostMalloc(&p, lay.store_bytes, hipHostMallocDefault) != hipSuccess || !p)
            MT_FAIL(MT_E_NOMEM, "cannot allocate a pinned host store of %lld bytes", (long long)lay.store_bytes);
        store = static_cast<uint8_t*>(p);
        store_pinned = true;
    } else {
        void* p = mmap(nullptr, lay.store_bytes, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS, -1, 0);
        if (p == MAP_FAILED) MT_FAIL(MT_E_NOMEM, "cannot map a host store of %lld bytes", (long long)lay.store_bytes);
        madvise(p, lay.store_bytes, MADV_HUGEPAGE);
        store = static_cast<uint8_t*>(p);
    }
    if (opt.pin_weights) {
        void* p = nullptr;
        if (hipHostMalloc(&p, lay.w_bytes, hipHostMallocDefault) != hipSuccess || !p)
            MT_FAIL(MT_E_NOMEM, "cannot allocate a pinned weight block of %lld bytes", (long long)lay.w_bytes);
        wblock = static_cast<uint8_t*>(p);
    }
    {
        ThreadPool init_pool(nth);
        for (int u = 0; u < int(lay.units.size()); ++u)
            init_unit(init_pool, store, lay, u, opt.seed, opt.init_std, wblock);
    }
    ein_acc.assign(size_t(sh.vocab) * sh.d_model, 0.f);
    adam_gen.assign(lay.units.size(), 0);

    // Pinned staging, slabs, checkpoint ring, I/O buffers.
    if (!opt.pin_store && !opt.pin_weights) {
        staging[0] = pinned_alloc(this, plan.slot_bytes);
        staging[1] = pinned_alloc(this, plan.slot_bytes);
        if (!staging[0] || !staging[1]) MT_FAIL(MT_E_NOMEM, "cannot allocate pinned staging buffers");
    }
    for (int k = 0; k < opt.n_grad_slabs; ++k) {
        uint8_t* p = pinned_alloc(this, plan.slot_bytes);
        if (!p) MT_FAIL(MT_E_NOMEM, "cannot allocate pinned gradient slab %d", k);
        slabs.push_back(p);
        free_slabs.push_back(k);
        slab_landed.push_back(0);
    }
    const uint64_t T = uint64_t(opt.max_batch) * opt.max_seq;
    const uint64_t td = al4k(T * sh.d_model * 2);
    if (opt.ckpt_on_host) {
        ckpt_host = pinned_alloc(this, td * uint64_t(ckpt_slots(opt, sh)));
        if (!ckpt_host) MT_FAIL(MT_E_NOMEM, "cannot allocate the pinned checkpoint ring");
    }
    if (opt.ckpt_attn) {
        attn_host = pinned_alloc(this, attn_ckpt_bytes(sh, T) * uint64_t(sh.n_layers));
        if (!attn_host) MT_FAIL(MT_E_NOMEM, "cannot allocate the pinned attention checkpoint ring");
    }
    x0_pin = reinterpret_cast<uint16_t*>(pinned_alloc(this, td));
    dx0_pin = reinterpret_cast<uint16_t*>(pinned_alloc(this, td));
    lab_pin = reinterpret_cast<int32_t*>(pinned_alloc(this, al4k(T * 4)));
    loss_pin = reinterpret_cast<float*>(pinned_alloc(this, 4096));
    if (!x0_pin || !dx0_pin || !lab_pin || !loss_pin) MT_FAIL(MT_E_NOMEM, "cannot allocate pinned I/O buffers");

    // Streams: the caller's, else our own (default priority, non-blocking).
    hipStream_t* dst[3] = {&st_c, &st_w, &st_g};
    for (int i = 0; i < 3; ++i) {
        if (streams && streams[i]) {
            *dst[i] = static_cast<hipStream_t>(streams[i]);
        } else {
            HIPC(hipStreamCreateWithFlags(dst[i], hipStreamNonBlocking));
            own[i] = true;
        }
    }
    auto mk = [&](Ev& e) { return hipEventCreateWithFlags(&e.e, hipEventDisableTiming); };
    wready.resize(plan.n_slots);
    slot_free.resize(plan.n_slots);
    bwd_done.resize(plan.n_garea);
    buf_free.resize(plan.n_garea);
    slab_done.resize(opt.n_grad_slabs);
    for (auto* v : {&wready, &slot_free, &bwd_done, &buf_free, &slab_done})
        for (auto& e : *v) HIPC(mk(e));
    for (Ev* e : {&staging_free[0], &staging_free[1], &xc_free[0], &xc_free[1], &ckpt_done[0], &ckpt_done[1],
                  &xready, &emb_ready, &fwd_ckpt_all, &dx0_done, &loss_done, &res_ready, &attn_ck_done[0],
                  &attn_ck_done[1], &attn_buf_free[0], &attn_buf_free[1]})
        HIPC(mk(*e));
    HIPC(hipEventCreate(&t_base));
    for (int i = 0; i < 1024; ++i) {
        hipEvent_t e;
        HIPC(hipEventCreate(&e));
        tev.push_back(e);
    }
    slot_unit.assign(plan.n_slots, -1);

    // Gradient areas: tensors never write their padding, so zero it once.
    for (int g = 0; g < plan.n_garea; ++g) HIPC(fill_zero(arena + plan.garea[g], plan.slot_bytes, st_c));
    HIPC(hipStreamSynchronize(st_c));
    ga_last_req.assign(plan.n_garea, -1);
    slot_last_req.assign(plan.n_slots, -1);
    for (int i = 0; i < 256; ++i) {
        hipEvent_t e;
        HIPC(hipEventCreate(&e));
        off_tev.push_back(e);
    }
    slab_thread = std::thread([this] { slab_worker(); });
    off_thread = std::thread([this] { offload_worker(); });
    return MT_OK;
}

Ctx::~Ctx() {
    // The offload thread first (pending requests dropped; the one in hand may
    // still need a slab from the slab worker), then the streams, then the
    // slab worker.
    {
        std::lock_guard<std::mutex> lk(off_mu);
        off_stop = true;
        off_q.clear();
    }
    off_cv.notify_all();
    if (off_thread.joinable()) off_thread.join();
    if (st_c) hipStreamSynchronize(st_c);
    if (st_w) hipStreamSynchronize(st_w);
    if (st_g) hipStreamSynchronize(st_g);
    {
        std::lock_guard<std::mutex> lk(q_mu);
        stop = true;
    }
    q_cv.notify_all();
    if (slab_thread.joinable()) slab_thread.join();
    for (auto e : off_tev) hipEventDestroy(e);
    for (auto* v : {&wready, &slot_free, &bwd_done, &buf_free, &slab_done})
        for (auto& e : *v)
            if (e.e) hipEventDestroy(e.e);
    for (Ev* e : {&staging_free[0], &staging_free[1], &xc_free[0], &xc_free[1], &ckpt_done[0], &ckpt_done[1],
                  &xready, &emb_ready, &fwd_ckpt_all, &dx0_done, &loss_done, &res_ready, &attn_ck_done[0],
                  &attn_ck_done[1], &attn_buf_free[0], &attn_buf_free[1]})
        if (e->e) hipEventDestroy(e->e);
    for (auto e : tev) hipEventDestroy(e);
    if (t_base) hipEventDestroy(t_base);
    for (int i = 0; i < 3; ++i) {
        hipStream_t s = i == 0 ? st_c : i == 1 ? st_w : st_g;
        if (own[i] && s) hipStreamDestroy(s);
    }
    for (auto* p : pinned_blocks) hipHostFree(p);
    if (store) {
        if (store_pinned) hipHostFree(store);
        else munmap(store, lay.store_bytes);
    }
    if (wblock) hipHostFree(wblock);
}

// ------------------------------------------------------- slab worker ----
void Ctx::slab_worker() {
    for (;;) {
        Job j;
        {
            std::unique_lock<std::mutex> lk(q_mu);
            q_cv.wait(lk, [&] { return stop || !jobs.empty(); });
            if (jobs.empty()) return;
            // With cross_step the updates go lowest rank first, in the order
            // the next forward needs the units: the input embedding, the
            // layers in order, then the head.  The backward hands gradients
            // over from the head down, so while it runs the worker takes the
            // newest arrival and the backlog it cannot keep up with piles up
            // at the top of the model, which the next forward reaches last
            // (in arrival order the backlog would be the bottom layers, and
            // the next forward would wait for it from its first layer on).
            // The number of pending jobs, and so of slabs held, does not
            // depend on the order.  Equal ranks (one unit's micro-batch jobs,
            // the head's chunks) keep arrival order.  Without cross_step
            // every update completes inside the step: arrival order.
            // The part of a split embedding update that the next gather does
            // not read goes last (it fills the worker's idle time before the
            // head's gradients land), until a thread has to wait for it.
            auto rank = [&](const Job& x) {
                if (x.mode == JOB_ADAM_ROWS) return -2;
                if (x.mode == JOB_ADAM_EXCEPT) return emb_urgent ? -1 : lay.embed() + 1;
                return x.unit == lay.embed() ? -1 : x.unit;
            };
            // Only the newest job's slab can still be in flight (a slab's
            // copy is submitted after the previous one completed), so a
            // lowest-rank pick would often wait for it while an older job's
            // gradients sit ready: take the lowest rank among the jobs the
            // offload thread has seen land, and wait only when there is none.  The earliest job of
            // the chosen rank goes first, so equal ranks keep arrival order.
            auto it = jobs.begin();
            if (opt.cross_step) {
                // (no event query here: under the queue lock it was seen to
                // stall for as long as the copy the offload thread waits on)
                auto landed = [&](const Job& x) { return x.slab < 0 || slab_landed[size_t(x.slab)] != 0; };
                auto best = jobs.end();
                for (auto k = jobs.begin(); k != jobs.end(); ++k)
                    if ((best == jobs.end() || rank(*k) < rank(*best)) && landed(*k)) best = k;
                if (best == jobs.end())
                    best = std::min_element(jobs.begin(), jobs.end(),
                                            [&](const Job& x, const Job& y) { return rank(x) < rank(y); });
                it = std::find_if(jobs.begin(), jobs.end(), [&](const Job& x) { return rank(x) == rank(*best); });
                host_rec("host_pick", it->unit, int(jobs.size()) * 100 + int(landed(*it)), Clock::now());
            }
            j = *it;
            jobs.erase(it);
            if (j.mode == JOB_ADAM_EXCEPT) emb_urgent = false;
        }
        int status = MT_OK;
        std::string err;
        hipError_t e = j.slab >= 0 ? hipEventSynchronize(slab_done[j.slab].e) : hipSuccess;
        if (e != hipSuccess) {
            status = MT_E_HIP;
            err = strfmt("HIP error '%s' waiting for gradient slab %d", hipGetErrorString(e), j.slab);
        } else if (j.unit == fault_slab) {
            status = MT_E_INTERNAL;
            err = strfmt("injected slab-worker fault at unit %d", j.unit);
        } else {
            const auto t0 = Clock::now();
            TilePtrs tp = tile_ptrs(store, lay, j.unit, wblock);
            tp.w += j.off;
            tp.g += j.off;
            tp.master += j.off;
            tp.m += j.off;
            tp.v += j.off;
            const uint16_t* src = j.slab >= 0 ? reinterpret_cast<const uint16_t*>(slabs[j.slab]) : tp.g;
            const int64_t d = lay.sh.d_model;
            switch (j.mode) {
                case JOB_ADAM:
                    // keep_grads = 0: the update reads the slab and leaves G
                    // alone (the copy into G is skipped when the two coincide)
                    if (!opt.keep_grads) tp.g = const_cast<uint16_t*>(src);
                    adam_unit(*adam_pool, tp, src, j.elems, j.a);
                    break;
                case JOB_ADAM_ROWS:
                case JOB_ADAM_EXCEPT: {
                    // one row of the embedding tile at a time
                    auto row_adam = [&](int64_t r) {
                        TilePtrs q = tp;
                        q.w += r * d;
                        q.g += r * d;
                        q.master += r * d;
                        q.m += r * d;
                        q.v += r * d;
                        adam_range(q, q.g, 0, d, j.a);
                    };
                    const std::vector<int32_t>& rows = *j.rows;
                    if (j.mode == JOB_ADAM_ROWS) {
                        adam_pool->parallel_for(int64_t(rows.size()), 16, [&](int64_t b, int64_t e) {
                            for (int64_t i = b; i < e; ++i) row_adam(rows[size_t(i)]);
                        });
                    } else {
                        std::vector<char> skip(size_t(j.elems / d), 0);
                        for (int32_t r : rows) skip[size_t(r)] = 1;
                        adam_pool->parallel_for(j.elems / d, 16, [&](int64_t b, int64_t e) {
                            for (int64_t r = b; r < e; ++r)
                                if (!skip[size_t(r)]) row_adam(r);
                        });
                    }
                    break;
                }
                case JOB_STORE: parallel_copy(*adam_pool, tp.g, src, j.elems * 2); break;
                case JOB_ACCUM: accum_unit(*adam_pool, tp.g, src, j.elems); break;
                default:
                    accum_unit(*adam_pool, tp.g, src, j.elems);
                    adam_unit(*adam_pool, tp, tp.g, j.elems, j.a);
            }
            const double ms = ms_since(t0);
            host_rec("host_job", j.unit, j.mode * 100 + j.slab, t0);
            std::lock_guard<std::mutex> lk(q_mu);
            adam_ms_acc += ms;
        }
        {
            std::lock_guard<std::mutex> lk(q_mu);
            if (status != MT_OK && worker_status == MT_OK) {
                worker_status = status;
                worker_error = err;
            }
            if (j.slab >= 0) free_slabs.push_back(j.slab);
            if (j.last && (j.mode == JOB_ADAM || j.mode == JOB_ACCUM_ADAM || j.mode == JOB_ADAM_EXCEPT))
                ++adam_gen[j.unit];
            if (j.mode == JOB_ADAM_ROWS) ++emb_rows_done;
            --jobs_pending;
        }
        free_cv.notify_all();
    }
}

// ------------------------------------------------- gradient offload ----
void Ctx::offload_worker() {
    for (;;) {
        OffReq r;
        {
            std::unique_lock<std::mutex> lk(off_mu);
            off_cv.wait(lk, [&] { return off_stop || !off_q.empty(); });
            if (off_q.empty()) return;
            r = off_q.front();
            off_q.pop_front();
        }
        const int k = acquire_slab();
        hipError_t e = hipSuccess;
        // One gradient copy in flight at a time (the previous slab's copy
        // cannot have been re-recorded: only this thread acquires slabs).
        if (off_prev_slab >= 0) e = hsync(slab_done[off_prev_slab]);
        if (e == hipSuccess && off_prev_slab >= 0 && off_prev_slab != k) {
            std::lock_guard<std::mutex> lk(q_mu);
            slab_landed[size_t(off_prev_slab)] = 1;
        }
        off_prev_slab = k;
        hipEvent_t a = nullptr, b = nullptr;
        if (e == hipSuccess) e = hipStreamWaitEvent(st_g, bwd_done[r.ga].e, 0);
        if (e == hipSuccess && timing && off_tev_next + 2 <= off_tev.size()) {
            a = off_tev[off_tev_next++];
            b = off_tev[off_tev_next++];
            e = hipEventRecord(a, st_g);
        }
        if (e == hipSuccess) e = hipMemcpyAsync(slabs[k], r.gbase, r.bytes, hipMemcpyDeviceToHost, st_g);
        if (e == hipSuccess && b) e = hipEventRecord(b, st_g);
        if (e == hipSuccess) e = rec(slab_done[k], st_g);
        // poison_released: the gradient area holds NaN from here until the
        // next visit that writes it
        if (e == hipSuccess && opt.poison_released && !(r.bytes & 15))
            e = fill_u32(r.gbase, int64_t(r.bytes), 0x7FC07FC0u, st_g);
        if (e == hipSuccess) e = rec(buf_free[r.ga], st_g);
        if (e == hipSuccess && r.slot >= 0) e = rec(slot_free[r.slot], st_g);
        // The job is queued before the request counts as issued, so a
        // compute thread that saw every request issued also sees its job.
        if (e == hipSuccess) {
            enqueue_job(r.unit, k, r.mode, r.off, int64_t(r.bytes / 2), r.last);
        } else {
            std::lock_guard<std::mutex> lk(q_mu);
            free_slabs.push_back(k);
            free_cv.notify_all();
        }
        {
            std::lock_guard<std::mutex> lk(off_mu);
            if (a && b && e == hipSuccess) {
                off_intervals.push_back({a, b, 2, r.bytes, -1, k});
                off_intervals.back().seq = off_issued;
            }
            if (e != hipSuccess && off_status == MT_OK) {
                off_status = MT_E_HIP;
                off_error = strfmt("HIP error '%s' offloading the gradient of unit %d", hipGetErrorString(e), r.unit);
            }
            ++off_issued;
        }
        off_cv.notify_all();
        // The next copy waits for this one anyway: wait here, so the slab
        // worker learns that the gradients landed also when no further
        // request follows (the backward's last unit).  An error is left to
        // the worker's own wait on the slab.
        if (e == hipSuccess && hsync(slab_done[k]) == hipSuccess) {
            std::lock_guard<std::mutex> lk(q_mu);
            slab_landed[size_t(k)] = 1;
        }
    }
}

// Block until offload request `seq` (0-based; < 0: none) has been issued.
int Ctx::wait_offload(int64_t seq) {
    std::unique_lock<std::mutex> lk(off_mu);
    off_cv.wait(lk, [&] { return off_issued > seq || off_status != MT_OK; });
    if (off_status != MT_OK) {
        failed = true;
        set_error(off_error);
        return off_status;
    }
    return MT_OK;
}

int Ctx::acquire_slab() {
    const auto t0 = Clock::now();
    int k;
    {
        std::unique_lock<std::mutex> lk(q_mu);
        free_cv.wait(lk, [&] { return !free_slabs.empty(); });
        // Lowest index first keeps the slab order deterministic.
        auto it = std::min_element(free_slabs.begin(), free_slabs.end());
        k = *it;
        free_slabs.erase(it);
        slab_landed[size_t(k)] = 0;
    }
    host_rec("host_slab_wait", -1, k, t0);
    return k;
}

void Ctx::enqueue_job(int unit, int slab, int mode, int64_t off, int64_t elems, bool last) {
    {
        std::lock_guard<std::mutex> lk(q_mu);
        jobs.push_back({unit, slab, elems < 0 ? lay.units[unit].elems : elems, cur_adam, step + 1, mode, off, last});
        ++jobs_pending;
    }
    q_cv.notify_one();
}

// Block until `unit` carries every update of the steps run so far (with
// cross_step the previous step's may still be queued).  A worker error
// fails the context.
int Ctx::wait_adam(int unit) {
    std::unique_lock<std::mutex> lk(q_mu);
    const auto t0 = Clock::now();
    if (unit == lay.embed() && adam_gen[unit] < step) emb_urgent = true;
    free_cv.wait(lk, [&] { return adam_gen[unit] >= step || worker_status != MT_OK; });
    adam_wait_ms += ms_since(t0);
    if (worker_status != MT_OK) {
        failed = true;
        set_error(worker_error);
        const int s = worker_status;
        worker_status = MT_OK;
        return s;
    }
    return MT_OK;
}

int Ctx::drain_jobs() {
    std::unique_lock<std::mutex> lk(q_mu);
    if (emb_deferred) {  // the whole update of the input embedding, unsplit
        jobs.push_back({lay.embed(), -1, lay.units[lay.embed()].elems, emb_adam, emb_step_id, JOB_ADAM});
        ++jobs_pending;
        emb_deferred = false;
        q_cv.notify_one();
    }
    free_cv.wait(lk, [&] { return jobs_pending == 0; });
    if (worker_status != MT_OK) {
        failed = true;
        set_error(worker_error);
        const int s = worker_status;
        worker_status = MT_OK;
        return s;
    }
    return MT_OK;
}

// ------------------------------------------------- checkpoint shards ----
// Load a unit whose shard a lazy restore left pending.
int Ctx::ensure_loaded(int unit) {
    if (lazy_dir.empty() || lazy_dir[unit].empty()) return MT_OK;
    const std::string dir = lazy_dir[unit];
    lazy_dir[unit].clear();
    const int r = load_shard(*pack_pool, dir, tile_ptrs(store, lay, unit, wblock), lay, unit);
    if (r != MT_OK) failed = true;
    return r;
}

int Ctx::checkpoint_save(const std::string& dir) {
    if (failed) MT_FAIL(MT_E_STATE, "context failed earlier");
    const int ds = drain_jobs();
    if (ds != MT_OK) return ds;
    for (int u = 0; u < int(lay.units.size()); ++u) {
        int r = ensure_loaded(u);
        if (r == MT_OK) r = save_shard(*pack_pool, dir, tile_ptrs(store, lay, u, wblock), lay, u, step);
        if (r != MT_OK) return r;
    }
    return MT_OK;
}

int Ctx::checkpoint_restore(const std::string& dir, bool lazy) {
    if (failed) MT_FAIL(MT_E_STATE, "context failed earlier");
    const int ds = drain_jobs();
    if (ds != MT_OK) return ds;
    // Every header first: nothing is overwritten unless all shards fit.
    const int nu = int(lay.units.size());
    int64_t s0 = -1;
    for (int u = 0; u < nu; ++u) {
        int64_t su = 0;
        const int r = check_shard(dir, lay, u, &su);
        if (r != MT_OK) return r;
        if (u == 0) s0 = su;
        else if (su != s0) MT_FAIL(MT_E_IO, "shards of %s come from different steps (%lld, %lld)", dir.c_str(),
                                   (long long)s0, (long long)su);
    }
    lazy_dir.assign(size_t(nu), std::string());
    for (int u = 0; u < nu; ++u) {
        if (lazy) {
            lazy_dir[u] = dir;
            continue;
        }
        const int r = load_shard(*pack_pool, dir, tile_ptrs(store, lay, u, wblock), lay, u);
        if (r != MT_OK) {
            failed = true;
            return r;
        }
    }
    step = s0;
    {
        std::lock_guard<std::mutex> lk(q_mu);
        adam_gen.assign(size_t(nu), s0);
    }
    slot_unit.assign(plan.n_slots, -1);
    ein_touched.clear();
    ein_clear_all = true;
    return MT_OK;
}

// ------------------------------------------------------ layer template ----
hipError_t Ctx::ensure_rope(int S) {
    if (S == cached_rope_S) return hipSuccess;
    cached_rope_S = S;
    return rope_table(ws.rope_tab, S, lay.sh.head_dim, lay.sh.rope_base, st_c);
}

// Forward of one decoder layer on the compute stream.  With need_y false
// (the recompute before backward) the last GEMM is skipped: backward needs
// the intermediates, not the output.
hipError_t Ctx::fwd_layer(const LayerView& w, const uint16_t* x, uint16_t* y, int B, int S, bool need_y, int ob,
                          bool attn_restored) {
    const mt_shape& sh = lay.sh;
    const int T = B * S, d = sh.d_model, F = sh.ffn_dim;
    const int nq = sh.n_heads * sh.head_dim;
    const int nqkv = (sh.n_heads + 2 * sh.n_kv_heads) * sh.head_dim;
    hipStream_t s = st_c;
    // Attention in fp16: n1 and Wqkv go to the QKV product as fp16 (a bf16
    // value in fp16's normal range converts exactly; smaller ones keep an
    // absolute error under 2^-25), the projection comes back in fp32, RoPE
    // rotates q and k in fp32 and q, k, v are stored as fp16; the attention
    // products run on the fp16 MFMA and o is fp16, and so are the operands of
    // the O product (Wo converted like Wqkv).  Every fp16 value is range
    // guarded (saturated and counted in ws.ovf).
    // In the recompute (need_y false) this first kernel also clears the
    // attention backward's maxima words: the rotation below adds max |v| to
    // them and the backward's O dX product max |dO|.
    HIPR(site(S_RMS1_FWD, [&] {
        return rmsnorm_fwd(x, false, w.g1, ws.n1, ws.n1h, ws.rstd1, T, d, sh.rms_eps, s, ws.ovf,
                           need_y ? nullptr : ws.amax);
    }));
    HIPR(site(S_GEMM_QKV, [&] {
        HIPR(bf16_to_f16(w.wqkv, ws.w16, int64_t(nqkv) * d, s, ws.ovf));
        GemmArgs a{ws.n1h, d, ws.w16, d, ws.qkv32, nqkv, nullptr, 0, nullptr, 0, T, nqkv, d};
        return gemm(GEMM_NT, EPI_F32_F16IN, split_ws(a, ws), s);
    }));
    // In the recompute the rotation also takes max |v| for the attention
    // backward's scale.
    HIPR(site(S_ROPE_FWD, [&] {
        return qkv_rope_cvt(ws.qkv32, nqkv, ws.qkv, nqkv, nullptr, 0, ws.rope_tab, T, S, sh.n_heads + sh.n_kv_heads,
                            sh.n_heads + 2 * sh.n_kv_heads, sh.head_dim, s, ws.ovf, need_y ? nullptr : ws.amax);
    }));
    if (!attn_restored) {
        HIPR(site(S_ATTN_FWD, [&] {
            AttnArgs a{ws.qkv, nqkv, ws.oa[ob], nq, ws.lsea[ob], B, S, sh.n_heads, sh.n_kv_heads, sh.head_dim, ws.ovf};
            return attn_fwd(a, s);
        }));
    }
    HIPR(site(S_GEMM_O, [&] {
        // ws.w16 is free again: the QKV product before it on this stream read it
        HIPR(bf16_to_f16(w.wo, ws.w16, int64_t(d) * nq, s, ws.ovf));
        GemmArgs a{ws.oa[ob], nq, ws.w16, nq, ws.h1, d, x, d, nullptr, 0, T, d, nq};
        return gemm(GEMM_NT, EPI_F32_F16IN_RESID, split_ws(a, ws), s);
    }));
    HIPR(site(S_RMS2_FWD, [&] { return rmsnorm_fwd(ws.h1, true, w.g2, ws.n2, nullptr, ws.rstd2, T, d, sh.rms_eps, s); }));
    HIPR(site(S_GEMM_GATEUP, [&] {
        GemmArgs a{ws.n2, d, w.wgu, d, ws.gu, 2 * F, nullptr, 0, nullptr, 0, T, 2 * F, d};
        return gemm(GEMM_NT, EPI_BF16, split_ws(a, ws), s);
    }));
    HIPR(site(S_SWIGLU_FWD, [&] { return swiglu_fwd(ws.gu, ws.m, T, F, s); }));
    if (need_y) {
        HIPR(site(S_GEMM_DOWN, [&] {
            GemmArgs a{ws.m, F, w.wd, F, y, d, ws.h1, d, nullptr, 0, T, d, F};
            return gemm(GEMM_NT, EPI_BF16_RESID32, split_ws(a, ws), s);
        }));
    }
    return hipSuccess;
}

// Recompute, then backward of one decoder layer; writes dx and the layer's
// BF16 gradients into the views g.
hipError_t Ctx::bwd_layer(const LayerView& w, const LayerView& g, const uint16_t* x, const uint16_t* dy,
                          uint16_t* dx, int B, int S, int ob, bool attn_restored) {
    HIPR(fwd_layer(w, x, nullptr, B, S, false, ob, attn_restored));
    const mt_shape& sh = lay.sh;
    const int T = B * S, d = sh.d_model, F = sh.ffn_dim;
    const int nq = sh.n_heads * sh.head_dim;
    const int nqkv = (sh.n_heads + 2 * sh.n_kv_heads) * sh.head_dim;
    hipStream_t s = st_c;
    // Every backward product runs as an NT product on operands made
    // reduction-contiguous by a transpose (HBM-bound, a few percent of the
    // product's time); dX = dY W and dW = dY^T X.
    // MLP
    HIPR(site(S_GEMM_DOWN_DX, [&] { return gemm_nn_t(dy, d, w.wd, F, ws.dm, F, T, F, d); }));
    HIPR(site(S_GEMM_DOWN_DW, [&] { return gemm_tn_t(dy, d, ws.m, F, g.wd, F, d, F, T); }));
    HIPR(site(S_SWIGLU_BWD, [&] { return swiglu_bwd(ws.dm, ws.gu, ws.dgu, T, F, s); }));
    HIPR(site(S_GEMM_GATEUP_DX, [&] { return gemm_nn_t(ws.dgu, 2 * F, w.wgu, d, ws.dn, d, T, d, 2 * F); }));
    HIPR(site(S_GEMM_GATEUP_DW, [&] { return gemm_tn_t(ws.dgu, 2 * F, ws.n2, d, g.wgu, d, 2 * F, d, T); }));
    HIPR(site(S_RMS2_BWD, [&] {
        return rmsnorm_bwd(ws.dn, ws.h1, true, w.g2, ws.rstd2, dy, ws.dh1, g.g2, ws.partial, T, d, s);
    }));
    // attention
    // dO = dh1 Wo, with max |dO| added to the maxima words where the direct
    // form runs it; else the attention backward takes both maxima itself.
    bool amax_ready = false;
    HIPR(site(S_GEMM_O_DX, [&] {
        GemmArgs a{ws.dh1, d, w.wo, nq, ws.dout, nq, nullptr, 0, nullptr, 0, T, nq, d};
        a.amax = ws.amax;
        const hipError_t e = gemm_direct_checked(GEMM_NN, EPI_BF16_AMAX, a, st_c);
        if (e != hipErrorNotSupported) {
            amax_ready = e == hipSuccess;
            return e;
        }
        return gemm_nn_t(ws.dh1, d, w.wo, nq, ws.dout, nq, T, nq, d);
    }));
    // o is fp16: rounded to bf16 for the bf16 product
    HIPR(site(S_GEMM_O_DW, [&] { return gemm_tn_t(ws.dh1, d, ws.oa[ob], nq, g.wo, nq, d, nq, T, true); }));
    // The attention backward on the fp16 operands of the recomputed forward:
    // dV, and dQ and dK rotated back by -theta where they are finished,
    // rounded to bf16 once into dqkv.
    HIPR(site(S_ATTN_BWD, [&] {
        const int64_t part = std::min<int64_t>(attn_bwd_part_elems(B, S, sh.n_heads, sh.n_kv_heads, sh.head_dim),
                                               int64_t(ws.tA_bytes / 4));
        AttnBwdArgs a{ws.qkv, nqkv, ws.oa[ob], ws.dout, nq, ws.lsea[ob], ws.dsum, ws.do16, ws.amax, ws.dqkv, nqkv,
                      B, S, sh.n_heads, sh.n_kv_heads, sh.head_dim, nullptr, 0, ws.ovf,
                      reinterpret_cast<float*>(ws.tA), part, 0};
        a.rope_tab = ws.rope_tab;
        a.amax_ready = amax_ready;
        // the stored-dS form of dQ where the shape takes it (the region after
        // the partials; the workspace was sized for the largest batch x seq)
        const int64_t dsb = attn_ds_bytes(B, S, sh.n_heads);
        const uint64_t ds_off = uint64_t((part * 4 + 255) & ~int64_t(255));
        if (dsb > 0 && ds_off + uint64_t(dsb) <= ws.tA_bytes) {
            a.ds = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(ws.tA) + ds_off);
            a.ds_ld = (int64_t(S) + 127) / 128 * 128;
        }
        return attn_bwd(a, s);
    }));
    HIPR(site(S_GEMM_QKV_DX, [&] { return gemm_nn_t(ws.dqkv, nqkv, w.wqkv, d, ws.dn, d, T, d, nqkv); }));
    HIPR(site(S_GEMM_QKV_DW, [&] { return gemm_tn_t(ws.dqkv, nqkv, ws.n1, d, g.wqkv, d, nqkv, d, T); }));
    HIPR(site(S_RMS1_BWD, [&] {
        return rmsnorm_bwd(ws.dn, x, false, w.g1, ws.rstd1, ws.dh1, dx, g.g1, ws.partial, T, d, s);
    }));
    return hipSuccess;
}

// The head streamed in E_out row chunks ([Hotdry]: the pinned staging
// buffers match the largest layer; here the largest decoder layer, not the
// head).  Forward over the chunks in order: nf once (chunk 0 carries gf), the
// logits of every token chunk against the chunk's rows, the running
// logsumexp per token; after the last chunk the loss rows and the loss.
hipError_t Ctx::head_chunk_fwd(const HeadChunk& ch, bool first, bool last, const void* wbase, const uint16_t* xL,
                               int B, int S) {
    const mt_shape& sh = lay.sh;
    const int T = B * S, d = sh.d_model;
    hipStream_t s = st_c;
    const UnitLayout& hu = lay.units[lay.head()];
    const uint16_t* w = static_cast<const uint16_t*>(wbase);
    const uint16_t* E = w + (hu.t[T_EOUT].off + int64_t(ch.row0) * d - ch.start);
    if (first)
        HIPR(site(S_HEAD_RMS_FWD, [&] {
            return rmsnorm_fwd(xL, false, w + hu.t[T_GF].off, ws.nf, nullptr, ws.rstdf, T, d, sh.rms_eps, s);
        }));
    const int tc = int(std::min<int64_t>(ws.head_chunk, T));
    for (int r0 = 0; r0 < T; r0 += tc) {
        const int rows = std::min(tc, T - r0);
        HIPR(site(S_HEAD_LOGITS, [&] {
            GemmArgs a{ws.nf + int64_t(r0) * d, d, E, d, ws.logits, ch.rows, nullptr, 0, nullptr, 0, rows, ch.rows, d};
            return gemm(GEMM_NT, EPI_F32, split_ws(a, ws), s);
        }));
        HIPR(site(S_HEAD_CE, [&] {
            return ce_chunk_fwd(ws.logits, ws.labels + r0, rows, ch.rows, ch.row0, first, ws.ce_m + r0,
                                ws.ce_l + r0, ws.ce_z + r0, s);
        }));
    }
    if (last) {
        HIPR(site(S_HEAD_CE, [&] { return ce_chunk_final(ws.ce_m, ws.ce_l, ws.ce_z, ws.ce_lse, ws.loss_rows, T, s); }));
        HIPR(site(S_HEAD_MISC, [&] { return mean_reduce(ws.loss_rows, ws.loss, T, s); }));
    }
    return hipSuccess;
}

// Backward over the chunks in reverse order (the last forward chunk is still
// in its slot): the chunk's logits again, dlogits = (softmax - onehot) / T,
// dnf summed over the chunks in fp32, the chunk's dE_out summed over token
// chunks in fp32 and written as bf16 into the gradient area (element i of the
// area = element start + i of the head tile); after chunk 0, the last, the
// final RMSNorm backward writes dy and dgf.
hipError_t Ctx::head_chunk_bwd(const HeadChunk& ch, bool first, bool last, const void* wbase, void* gbase,
                               const uint16_t* xL, uint16_t* dy, int B, int S, float inv_tokens) {
    const mt_shape& sh = lay.sh;
    const int T = B * S, d = sh.d_model;
    hipStream_t s = st_c;
    const UnitLayout& hu = lay.units[lay.head()];
    const int64_t eoff = hu.t[T_EOUT].off + int64_t(ch.row0) * d - ch.start;
    const uint16_t* w = static_cast<const uint16_t*>(wbase);
    uint16_t* g = static_cast<uint16_t*>(gbase);
    const uint16_t* E = w + eoff;
    uint16_t* gE = g + eoff;
    const int tc = int(std::min<int64_t>(ws.head_chunk, T));
    const int nch = (T + tc - 1) / tc;
    bool tB_holds_chunk = false;  // E^T of this vocabulary chunk in the workspace
    for (int c = 0; c < nch; ++c) {
        const int r0 = c * tc, rows = std::min(tc, T - r0);
        HIPR(site(S_HEAD_LOGITS, [&] {
            GemmArgs a{ws.nf + int64_t(r0) * d, d, E, d, ws.logits, ch.rows, nullptr, 0, nullptr, 0, rows, ch.rows, d};
            return gemm(GEMM_NT, EPI_F32, split_ws(a, ws), s);
        }));
        HIPR(site(S_HEAD_CE, [&] {
            return ce_chunk_bwd(ws.logits, ws.labels + r0, ws.ce_lse + r0, rows, ch.rows, ch.row0, ws.dlogits,
                                inv_tokens, s);
        }));
        HIPR(site(S_HEAD_DX, [&] {
            // dX = dlogits E, E read k-major where the direct kernel takes
            // the grid; else the NT product on E^T, transposed once per
            // vocabulary chunk (the workspace holds d x the largest chunk)
            const GemmEpi epi = first ? EPI_F32 : EPI_F32_ACC;
            float* dx = ws.dnf_acc + int64_t(r0) * d;
            {
                GemmArgs a{ws.dlogits, ch.rows, E, d, dx, d, nullptr, 0, nullptr, 0, rows, d, ch.rows};
                const hipError_t e = gemm_direct_checked(GEMM_NN, epi, split_ws(a, ws), s);
                if (e != hipErrorNotSupported) return e;
            }
            if (!tB_holds_chunk) {
                HIPR(transpose16(E, d, ws.tB, ch.rows, ch.rows, d, s));
                tB_holds_chunk = true;
            }
            GemmArgs a{ws.dlogits, ch.rows, ws.tB, ch.rows, dx, d, nullptr, 0, nullptr, 0, rows, d, ch.rows};
            return gemm(GEMM_NT, epi, a, s);
        }));
        HIPR(site(S_HEAD_DW, [&] {
            GemmArgs a{ws.dlogits, ch.rows, ws.nf + int64_t(r0) * d, d, nullptr, d, nullptr, 0, nullptr, 0,
                       ch.rows, d, rows};
            GemmEpi epi;
            if (nch == 1) { a.C = gE; epi = EPI_BF16; }
            else if (c == 0) { a.C = ws.deout_acc; epi = EPI_F32; }
            else if (c + 1 < nch) { a.C = ws.deout_acc; epi = EPI_F32_ACC; }
            else { a.C = gE; a.Cacc = ws.deout_acc; a.ldacc = d; epi = EPI_BF16_ACCF32; }
            return gemm(GEMM_TN, epi, split_ws(a, ws), s);
        }));
    }
    if (last) {
        HIPR(site(S_HEAD_RMS_BWD, [&] {
            HIPR(f32_to_bf16(ws.dnf_acc, ws.dnf, int64_t(T) * d, s));
            return rmsnorm_bwd(ws.dnf, xL, false, w + hu.t[T_GF].off, ws.rstdf, nullptr, dy, g + hu.t[T_GF].off,
                               ws.partial, T, d, s);
        }));
    }
    return hipSuccess;
}

// C[M x N] = A[M x K] B[K x N] (B row-major): straight from the k-major B
// where the direct kernel takes the grid, else B transposed into tB, then NT.
hipError_t Ctx::gemm_nn_t(const uint16_t* A, int64_t lda, const uint16_t* Bm, int64_t ldb, uint16_t* C, int64_t ldc,
                          int M, int N, int K) {
    {
        GemmArgs a{A, lda, Bm, ldb, C, ldc, nullptr, 0, nullptr, 0, M, N, K};
        const hipError_t e = gemm_direct_checked(GEMM_NN, EPI_BF16, split_ws(a, ws), st_c);
        if (e != hipErrorNotSupported) return e;
    }
    HIPR(transpose16(Bm, ldb, ws.tB, K, K, N, st_c));
    GemmArgs a{A, lda, ws.tB, K, C, ldc, nullptr, 0, nullptr, 0, M, N, K};
    return gemm(GEMM_NT, EPI_BF16, a, st_c);
}

// C[M x N] = A^T B with A stored [K x M] and B [K x N]: straight from the
// k-major operands where the direct kernel takes the grid, else both
// transposed, then NT; K (the tokens) is then padded to a multiple of 8 with
// zero columns, which add nothing.  b_f16: B holds fp16, rounded to bf16 as
// its fragments are read, or by its transpose.
hipError_t Ctx::gemm_tn_t(const uint16_t* A, int64_t lda, const uint16_t* Bm, int64_t ldb, uint16_t* C, int64_t ldc,
                          int M, int N, int K, bool b_f16) {
    {
        GemmArgs a{A, lda, Bm, ldb, C, ldc, nullptr, 0, nullptr, 0, M, N, K};
        a.b_f16 = b_f16;
        const hipError_t e = gemm_direct_checked(GEMM_TN, EPI_BF16, split_ws(a, ws), st_c);
        if (e != hipErrorNotSupported) return e;
    }
    const int Kp = (K + 7) & ~7;
    if (Kp != K) {
        HIPR(fill_zero(ws.tA, int64_t(M) * Kp * 2, st_c));
        HIPR(fill_zero(ws.tB, int64_t(N) * Kp * 2, st_c));
    }
    HIPR(transpose16(A, lda, ws.tA, Kp, K, M, st_c));
    HIPR(transpose16(Bm, ldb, ws.tB, Kp, K, N, st_c, b_f16));
    GemmArgs a{ws.tA, Kp, ws.tB, Kp, C, ldc, nullptr, 0, nullptr, 0, M, N, Kp};
    return gemm(GEMM_NT, EPI_BF16, a, st_c);
}

// LM head, forward and backward fused over token chunks; writes dy (the
// gradient of the last layer's output) and the head gradients into g.
hipError_t Ctx::head(const HeadView& w, const HeadView& g, const uint16_t* xL, uint16_t* dy, int B, int S,
                     float inv_tokens) {
    const mt_shape& sh = lay.sh;
    const int T = B * S, d = sh.d_model, V = sh.vocab;
    hipStream_t s = st_c;
    const int tc = int(std::min<int64_t>(ws.head_chunk, T));
    const int nch = (T + tc - 1) / tc;
    HIPR(site(S_HEAD_RMS_FWD, [&] { return rmsnorm_fwd(xL, false, w.gf, ws.nf, nullptr, ws.rstdf, T, d, sh.rms_eps, s); }));
    for (int c = 0; c < nch; ++c) {
        const int r0 = c * tc, rows = std::min(tc, T - r0);
        HIPR(site(S_HEAD_LOGITS, [&] {
            GemmArgs a{ws.nf + int64_t(r0) * d, d, w.eout, d, ws.logits, V, nullptr, 0, nullptr, 0, rows, V, d};
            return gemm(GEMM_NT, EPI_F32, split_ws(a, ws), s);
        }));
        HIPR(site(S_HEAD_CE, [&] {
            return ce_fwd_bwd(ws.logits, ws.labels + r0, ws.loss_rows + r0, ws.dlogits, rows, V, inv_tokens, s);
        }));
        HIPR(site(S_HEAD_DX, [&] {
            GemmArgs a{ws.dlogits, V, w.eout, d, ws.dnf + int64_t(r0) * d, d, nullptr, 0, nullptr, 0, rows, d, V};
            return gemm(GEMM_NN, EPI_BF16, split_ws(a, ws), s);
        }));
        HIPR(site(S_HEAD_DW, [&] {
            GemmArgs a{ws.dlogits, V, ws.nf + int64_t(r0) * d, d, nullptr, d, nullptr, 0, nullptr, 0, V, d, rows};
            GemmEpi epi;
            if (nch == 1) { a.C = g.eout; epi = EPI_BF16; }
            else if (c == 0) { a.C = ws.deout_acc; epi = EPI_F32; }
            else if (c + 1 < nch) { a.C = ws.deout_acc; epi = EPI_F32_ACC; }
            else { a.C = g.eout; a.Cacc = ws.deout_acc; a.ldacc = d; epi = EPI_BF16_ACCF32; }
            return gemm(GEMM_TN, epi, split_ws(a, ws), s);
        }));
    }
    HIPR(site(S_HEAD_RMS_BWD, [&] {
        return rmsnorm_bwd(ws.dnf, xL, false, w.gf, ws.rstdf, nullptr, dy, g.gf, ws.partial, T, d, s);
    }));
    HIPR(site(S_HEAD_MISC, [&] { return mean_reduce(ws.loss_rows, ws.loss, T, s); }));
    return hipSuccess;
}

// ------------------------------------------------------------ streaming ----
int Ctx::pick_slot(int unit, bool* need_stream) {
    for (int s = 0; s < plan.n_slots; ++s)
        if (slot_unit[s] == unit) {
            *need_stream = false;
            slot_ptr = (s + 1) % plan.n_slots;
            return s;
        }
    const int s = slot_ptr;
    slot_ptr = (s + 1) % plan.n_slots;
    *need_stream = true;
    return s;
}

// Pack unit -> pinned staging (host), then H2D staging -> slot on the weight
// stream once the slot is released.
int Ctx::stream_unit(int unit, int slot, int id, int64_t e0, int64_t n) {
    const uint64_t bytes = uint64_t(n < 0 ? lay.units[unit].elems : n) * 2;
    const uint8_t* src = (wblock ? wblock + lay.w_off[unit] : store + lay.tile_off[unit]) + e0 * 2;
    if (unit == fault_pack) {
        failed = true;
        MT_FAIL(MT_E_INTERNAL, "injected pack fault at unit %d", unit);
    }
    const int el = ensure_loaded(unit);
    if (el != MT_OK) return el;
    const int wa = wait_adam(unit);
    if (wa != MT_OK) return wa;
    const int wo = wait_offload(slot_last_req[slot]);  // combined slots: released by the offload
    if (wo != MT_OK) return wo;
    HIPC(wait(st_w, slot_free[slot]));
    if (store_pinned || wblock) {
        HIPC(h2d(arena + plan.wslot[slot], src, bytes, st_w, slot));
    } else {
        const int p = staging_ptr;
        staging_ptr ^= 1;
        const auto tw = Clock::now();
        HIPC(hsync(staging_free[p]));
        host_rec("host_staging_wait", unit, p, tw);
        const auto t0 = Clock::now();
        parallel_copy(*pack_pool, staging[p], src, int64_t(bytes));
        pack_ms += ms_since(t0);
        host_rec("host_pack", unit, p, t0);
        HIPC(h2d(arena + plan.wslot[slot], staging[p], bytes, st_w, slot));
        HIPC(rec(staging_free[p], st_w));
    }
    slot_unit[slot] = id < 0 ? unit : id;
    return MT_OK;
}

// ------------------------------------------------------------ the step ----
int Ctx::train_step(const int32_t* tokens, const int32_t* labels, int n_micro, int B, int S, float* loss_out,
                    mt_stats* stats) {
    if (failed) MT_FAIL(MT_E_STATE, "context failed earlier");
    if (!tokens || !labels || !loss_out) MT_FAIL(MT_E_INVAL, "tokens, labels and loss_out must not be NULL");
    if (B < 1 || S < 1 || int64_t(B) * S > ws.maxT || S > opt.max_seq)
        MT_FAIL(MT_E_INVAL, "batch %d x seq %d exceeds the workspace (max_batch*max_seq = %lld, max_seq = %d)",
                B, S, (long long)ws.maxT, opt.max_seq);
    if (n_micro < 1 || n_micro > MT_MAX_MICRO)
        MT_FAIL(MT_E_INVAL, "n_micro = %d outside [1, %d]", n_micro, MT_MAX_MICRO);
    const mt_shape& sh = lay.sh;
    const int T = B * S, L = sh.n_layers, d = sh.d_model, V = sh.vocab;
    for (int64_t t = 0; t < int64_t(n_micro) * T; ++t)
        if (tokens[t] < 0 || tokens[t] >= V || labels[t] < 0 || labels[t] >= V)
            MT_FAIL(MT_E_INVAL, "token or label at row %lld outside [0, %d)", (long long)t, V);

    const auto t_start = Clock::now();
    step_clock0 = t_start;
    {
        std::lock_guard<std::mutex> lk(trace_mu);
        host_recs.clear();
    }
    // Adam rewrote every unit's weights after the last step: no slot holds
    // current weights any more.
    slot_unit.assign(plan.n_slots, -1);
    slot_ptr = 0;
    tev_next = 0;
    intervals.clear();
    last_h2d = -1;
    site_recs.clear();
    {
        // The offload thread is idle between steps: every request was issued.
        std::lock_guard<std::mutex> lk(off_mu);
        off_tev_next = 0;
        off_intervals.clear();
    }
    {
        std::lock_guard<std::mutex> lk(q_mu);
        adam_ms_acc = 0.0;
        adam_wait_ms = 0.0;
    }
    pack_ms = 0.0;
    cur_adam = adam_step_params(opt, step + 1);
    timing = true;
    const uint64_t td = uint64_t(T) * d * 2;
    const uint64_t td_al = al4k(uint64_t(ws.maxT) * d * 2);
    // ckpt_attn ring: per layer at the workspace's token count, o then lse
    const uint64_t ab_al = attn_ckpt_bytes(lay.sh, uint64_t(ws.maxT));
    const uint64_t ao_al = attn_ckpt_o_bytes(lay.sh, uint64_t(ws.maxT));
    const uint64_t ao_bytes = uint64_t(B) * S * lay.sh.n_heads * lay.sh.head_dim * 2;
    const uint64_t al_bytes = uint64_t(B) * S * lay.sh.n_heads * 4;
    // Each micro-batch's loss gradient is that of the mean over all n*B*S
    // tokens: 1/(n T) (a power-of-two multiple of 1/T's rounding when n is a
    // power of two).
    const float inv_tokens = 1.0f / float(int64_t(n_micro) * T);
    HIPC(hipEventRecord(t_base, st_c));
    HIPC(fill_zero(ws.ovf, 256, st_c));  // fp16 range guard counter of this step
    HIPC(ensure_rope(S));
    if (opt.resident) {
        // The comparison run: every unit's weights copied up once, no streaming.
        for (int u = 0; u <= lay.head(); ++u) {
            const int lu = ensure_loaded(u);
            if (lu != MT_OK) return lu;
            const int wa = wait_adam(u);
            if (wa != MT_OK) return wa;
            const uint64_t bytes = uint64_t(lay.units[u].elems) * 2;
            HIPC(h2d(arena + plan.resident[u], wblock ? wblock + lay.w_off[u] : store + lay.tile_off[u], bytes, st_w));
        }
    }

    // The visit schedule: forward 0..L-1 (every k-th layer input checkpointed),
    // the head, then per checkpoint block from the top: restore the block's
    // first input, re-run the forward of its first k-1 layers to rebuild the
    // other inputs, and run the block's backward from its last layer down.
    // With k = 1 this is forward 0..L-1, head, backward L-1..0.  Every
    // micro-batch of the step runs the whole schedule with the same weights.
    enum { V_FWD, V_HEAD, V_REFWD, V_BWD, V_HFWD, V_HBWD };
    struct Visit {
        int kind, unit, block, pos;  // block: backward block counter; pos: the layer's index in its block
                                     // (head chunk visits: the chunk)
    };
    const int K = opt.ckpt_on_host ? ckpt_k(opt, sh) : 1;
    const std::vector<HeadChunk> hch = head_chunks(lay, opt);
    const int NV = int(hch.size());
    std::vector<Visit> sched;
    for (int l = 0; l < L; ++l) sched.push_back({V_FWD, l, 0, 0});
    if (hch.empty()) {
        sched.push_back({V_HEAD, lay.head(), 0, 0});
    } else {
        // The head in E_out chunks: forward in order, backward in reverse.
        for (int c = 0; c < NV; ++c) sched.push_back({V_HFWD, lay.head(), 0, c});
        for (int c = NV - 1; c >= 0; --c) sched.push_back({V_HBWD, lay.head(), 0, c});
    }
    for (int j = (L + K - 1) / K - 1, bi = 0; j >= 0; --j, ++bi) {
        const int b0 = j * K, e0 = std::min(b0 + K - 1, L - 1);
        for (int i = b0; i < e0; ++i) sched.push_back({V_REFWD, i, bi, i - b0});
        for (int l = e0; l >= b0; --l) sched.push_back({V_BWD, l, bi, l - b0});
    }
    const bool combined = opt.slot_mode == 1;
    // Phase edges per micro-batch: start, end of forward, of the head, of the backward.
    struct Phases {
        hipEvent_t start, fwd, head, bwd;
    };
    std::vector<Phases> phases;
    double loss_sum = 0.0;
    double t_bwd = 0.0;
    for (int mb = 0; mb < n_micro; ++mb) {
        const int32_t* tk = tokens + int64_t(mb) * T;
        const int32_t* lb = labels + int64_t(mb) * T;
        const int mode = n_micro == 1        ? JOB_ADAM
                         : mb == 0           ? JOB_STORE
                         : mb + 1 < n_micro ? JOB_ACCUM
                                             : JOB_ACCUM_ADAM;
        Phases ph{mb == 0 ? t_base : phases.back().bwd, nullptr, nullptr, nullptr};
        // The previous micro-batch's use of the labels and input buffers is over.
        if (mb > 0) HIPC(hipStreamWaitEvent(st_w, ph.start, 0));

        // Labels and the embedding gather (host, exact) go up on the weight stream.
        memcpy(lab_pin, lb, size_t(T) * 4);
        HIPC(h2d(ws.labels, lab_pin, uint64_t(T) * 4, st_w));
        {
            const int le = ensure_loaded(lay.embed());
            if (le != MT_OK) return le;
            // The previous step's update of E_in first.  Held back with
            // cross_step: the rows this step gathers (over all its
            // micro-batches) are updated now, the others are queued behind
            // them (they are needed by the next step's gather, or by the end
            // of this step's backward, which overwrites G).
            if (mb == 0) emb_split = false;
            if (mb == 0) {
                std::unique_lock<std::mutex> lk(q_mu);
                if (emb_deferred) {
                    auto rows = std::make_shared<std::vector<int32_t>>();
                    std::vector<char> seen(size_t(V), 0);
                    for (int64_t t = 0; t < int64_t(n_micro) * T; ++t)
                        if (!seen[size_t(tokens[t])]) {
                            seen[size_t(tokens[t])] = 1;
                            rows->push_back(tokens[t]);
                        }
                    const int64_t ne = lay.units[lay.embed()].elems;
                    Job a{lay.embed(), -1, ne, emb_adam, emb_step_id, JOB_ADAM_ROWS, 0, false, rows};
                    Job b{lay.embed(), -1, ne, emb_adam, emb_step_id, JOB_ADAM_EXCEPT, 0, true, rows};
                    jobs.push_back(a);
                    jobs.push_back(b);
                    jobs_pending += 2;
                    ++emb_rows_issued;
                    emb_deferred = false;
                    emb_split = true;
                    q_cv.notify_all();
                    const auto t0 = Clock::now();
                    free_cv.wait(lk, [&] { return emb_rows_done >= emb_rows_issued || worker_status != MT_OK; });
                    adam_wait_ms += ms_since(t0);
                    if (worker_status != MT_OK) {
                        failed = true;
                        set_error(worker_error);
                        const int st = worker_status;
                        worker_status = MT_OK;
                        return st;
                    }
                }
            }
            if (!emb_split) {  // (after a split, every micro-batch's rows are updated)
                const int we = wait_adam(lay.embed());
                if (we != MT_OK) return we;
            }
            const TilePtrs e = tile_ptrs(store, lay, lay.embed(), wblock);
            pack_pool->parallel_for(T, 64, [&](int64_t b, int64_t en) {
                for (int64_t t = b; t < en; ++t)
                    memcpy(x0_pin + t * d, e.w + int64_t(tk[t]) * d, size_t(d) * 2);
            });
        }
        uint16_t* x_first = opt.ckpt_on_host ? ws.x[0] : ws.ckpt_dev;
        HIPC(h2d(x_first, x0_pin, td, st_w));
        HIPC(rec(emb_ready, st_w));

        // A compute visit is done with its weight slot: release it (with
        // poison_released, filled with NaN first and forgotten, so any later
        // reader that was not re-streamed reads NaN).
        auto release_slot = [&](int s_) -> hipError_t {
            if (opt.poison_released) {
                const hipError_t e = fill_u32(arena + plan.wslot[s_], int64_t(plan.slot_bytes), 0x7FC07FC0u, st_c);
                if (e != hipSuccess) return e;
                slot_unit[s_] = -1;
            }
            return rec(slot_free[s_], st_c);
        };
        int gnext = 0, nbwd = 0, restored = -1;
        for (const Visit& vs : sched) {
            const int kind = vs.kind, unit = vs.unit;
            const bool hchunk = kind == V_HFWD || kind == V_HBWD;
            const HeadChunk* ch = hchunk ? &hch[size_t(vs.pos)] : nullptr;
            // Bind target: a streamed slot or the resident copy.
            int slot = 0;
            void* wbase;
            if (opt.resident) {
                wbase = arena + plan.resident[unit] + (ch ? ch->start * 2 : 0);
            } else {
                bool need = false;
                const int id = ch ? lay.embed() + 1 + vs.pos : unit;  // slot contents: unit or head chunk
                slot = pick_slot(id, &need);
                if (need) {
                    const int r = ch ? stream_unit(unit, slot, id, ch->start, ch->elems) : stream_unit(unit, slot);
                    if (r != MT_OK) {
                        drain_jobs();
                        return r;
                    }
                }
                wbase = arena + plan.wslot[slot];
            }
            const int bank = vs.block & 1;
            uint16_t* const* xb = opt.ckpt_on_host ? ws.xc.data() + size_t(bank) * K : nullptr;
            if ((kind == V_REFWD || kind == V_BWD) && opt.ckpt_on_host && vs.block != restored) {
                // Restore the block's first input from the host ring.
                restored = vs.block;
                if (vs.block == 0) HIPC(wait(st_w, fwd_ckpt_all));
                HIPC(wait(st_w, xc_free[bank]));
                HIPC(h2d(xb[0], ckpt_host + uint64_t(unit / K) * td_al, td, st_w));
            }
            // ckpt_attn: the layer's attention output and log-sum-exp come
            // back into the pair the backward visit two back has finished with
            // (the weights-ready event below covers these copies too)
            const int ob_b = opt.ckpt_attn && kind == V_BWD ? (nbwd & 1) : 0;
            if (opt.ckpt_attn && kind == V_BWD) {
                const uint8_t* h = attn_host + uint64_t(unit) * ab_al;
                HIPC(wait(st_w, fwd_ckpt_all));
                HIPC(wait(st_w, attn_buf_free[ob_b]));
                HIPC(h2d(ws.oa[ob_b], h, ao_bytes, st_w));
                HIPC(h2d(ws.lsea[ob_b], h + ao_al, al_bytes, st_w));
            }
            Ev& wr = wready[slot];
            HIPC(rec(wr, st_w));
            HIPC(wait(st_c, wr));
            const int vis_h2d = last_h2d;  // the compute waits for every weight-stream copy issued so far
            // Head and backward write a gradient area: wait until its last
            // offload is done (Buffer-Free) before the visit's clock starts.
            int ga = 0;
            int64_t vis_seq = -1;
            if (kind == V_HEAD || kind == V_BWD || kind == V_HBWD) {
                ga = combined ? slot : gnext;
                if (!combined) gnext ^= 1;
                vis_seq = ga_last_req[ga];
                const int wo = wait_offload(ga_last_req[ga]);
                if (wo != MT_OK) return wo;
                HIPC(wait(st_c, buf_free[ga]));
            }
            auto visit_rec = [&](hipEvent_t a, hipEvent_t b) {
                Interval iv{a, b, 0, 0, kind, unit};
                iv.slot = opt.resident ? -1 : slot;
                iv.seq = vis_seq;
                iv.last_h2d = vis_h2d;
                intervals.push_back(iv);
            };
            hipEvent_t va = next_tev(), vz = next_tev();
            HIPC(hipEventRecord(va, st_c));
            if (kind == V_FWD) {
                const uint16_t* x = opt.ckpt_on_host ? ws.x[unit & 1] : ws.ckpt_dev + uint64_t(unit) * ws.maxT * d;
                uint16_t* y =
                    opt.ckpt_on_host ? ws.x[(unit + 1) & 1] : ws.ckpt_dev + uint64_t(unit + 1) * ws.maxT * d;
                if (opt.ckpt_on_host) HIPC(wait(st_c, ckpt_done[(unit + 1) & 1]));
                // ckpt_attn: layers alternate attention buffers; this one's
                // previous contents (two layers back) must be on the host
                const int ob = opt.ckpt_attn ? (unit & 1) : 0;
                if (opt.ckpt_attn) HIPC(wait(st_c, attn_ck_done[ob]));
                HIPC(fwd_layer(bind_layer(lay, wbase), x, y, B, S, true, ob));
                HIPC(hipEventRecord(vz, st_c));
                visit_rec(va, vz);
                HIPC(release_slot(slot));
                if (opt.ckpt_on_host) {
                    // Checkpoint the layer input on the gradient stream (idle in forward).
                    if (unit % K == 0) {
                        HIPC(wait(st_g, unit == 0 ? emb_ready : xready));
                        HIPC(d2h(ckpt_host + uint64_t(unit / K) * td_al, x, td, st_g));
                        HIPC(rec(ckpt_done[unit & 1], st_g));
                    }
                    HIPC(rec(xready, st_c));
                    if (opt.ckpt_attn) {
                        // ... and the layer's attention output and log-sum-exp
                        uint8_t* h = attn_host + uint64_t(unit) * ab_al;
                        HIPC(wait(st_g, xready));
                        HIPC(d2h(h, ws.oa[ob], ao_bytes, st_g));
                        HIPC(d2h(h + ao_al, ws.lsea[ob], al_bytes, st_g));
                        HIPC(rec(attn_ck_done[ob], st_g));
                    }
                    if (unit == L - 1) HIPC(rec(fwd_ckpt_all, st_g));
                }
                if (unit == L - 1) {
                    ph.fwd = next_tev();
                    HIPC(hipEventRecord(ph.fwd, st_c));
                }
                continue;
            }
            if (kind == V_HFWD) {
                const uint16_t* xL = opt.ckpt_on_host ? ws.x[L & 1] : ws.ckpt_dev + uint64_t(L) * ws.maxT * d;
                HIPC(head_chunk_fwd(*ch, vs.pos == 0, vs.pos == NV - 1, wbase, xL, B, S));
                if (vs.pos == NV - 1) {
                    HIPC(hipMemcpyAsync(loss_pin, ws.loss, 4, hipMemcpyDeviceToHost, st_c));
                    HIPC(rec(loss_done, st_c));
                }
                HIPC(hipEventRecord(vz, st_c));
                visit_rec(va, vz);
                HIPC(release_slot(slot));
                continue;
            }
            if (kind == V_REFWD) {
                // Rebuild the next layer's input inside the block's bank.
                HIPC(fwd_layer(bind_layer(lay, wbase), xb[vs.pos], xb[vs.pos + 1], B, S, true));
                HIPC(hipEventRecord(vz, st_c));
                visit_rec(va, vz);
                HIPC(release_slot(slot));
                continue;
            }
            // Head or backward: gradients go to a gradient area, then to a slab.
            void* gbase = arena + plan.garea[ga];
            if (kind == V_HEAD) {
                const uint16_t* xL = opt.ckpt_on_host ? ws.x[L & 1] : ws.ckpt_dev + uint64_t(L) * ws.maxT * d;
                HIPC(head(bind_head(lay, wbase), bind_head(lay, gbase), xL, ws.dy[0], B, S, inv_tokens));
                HIPC(hipMemcpyAsync(loss_pin, ws.loss, 4, hipMemcpyDeviceToHost, st_c));
                HIPC(rec(loss_done, st_c));
            } else if (kind == V_HBWD) {
                const uint16_t* xL = opt.ckpt_on_host ? ws.x[L & 1] : ws.ckpt_dev + uint64_t(L) * ws.maxT * d;
                HIPC(head_chunk_bwd(*ch, vs.pos == NV - 1, vs.pos == 0, wbase, gbase, xL, ws.dy[0], B, S,
                                    inv_tokens));
            } else {
                const uint16_t* x = opt.ckpt_on_host ? xb[vs.pos] : ws.ckpt_dev + uint64_t(unit) * ws.maxT * d;
                HIPC(bwd_layer(bind_layer(lay, wbase), bind_layer(lay, gbase), x, ws.dy[nbwd & 1],
                               ws.dy[(nbwd + 1) & 1], B, S, ob_b, opt.ckpt_attn != 0));
                if (opt.ckpt_attn) HIPC(rec(attn_buf_free[ob_b], st_c));
                ++nbwd;
                // The block's bank is free once its first layer's backward ran.
                if (opt.ckpt_on_host && vs.pos == 0) HIPC(rec(xc_free[bank], st_c));
            }
            HIPC(hipEventRecord(vz, st_c));
            visit_rec(va, vz);
            if (!combined) HIPC(release_slot(slot));
            HIPC(rec(bwd_done[ga], st_c));
            // Gradient offload: Backward-Done -> free slab -> Buffer-Free.
            {
                std::lock_guard<std::mutex> lk(off_mu);
                if (ch)  // one head chunk: its element range of the head tile
                    off_q.push_back({unit, ga, combined ? slot : -1, mode, gbase, uint64_t(ch->elems) * 2, ch->start,
                                     vs.pos == 0});
                else
                    off_q.push_back({unit, ga, combined ? slot : -1, mode, gbase, uint64_t(lay.units[unit].elems) * 2});
                ga_last_req[ga] = off_submitted;
                if (combined) slot_last_req[slot] = off_submitted;
                ++off_submitted;
            }
            off_cv.notify_all();
            if (kind == V_HEAD || (kind == V_HBWD && vs.pos == 0)) {
                ph.head = next_tev();
                HIPC(hipEventRecord(ph.head, st_c));
            }
        }
        {
            const int wo = wait_offload(off_submitted - 1);  // every gradient copy issued
            if (wo != MT_OK) return wo;
        }
        ph.bwd = next_tev();
        HIPC(hipEventRecord(ph.bwd, st_c));
        phases.push_back(ph);
        // Embedding backward on the host: dX0 down, scatter-add in token order.
        const uint16_t* dx0 = ws.dy[L & 1];
        HIPC(hipStreamWaitEvent(st_g, ph.bwd, 0));
        HIPC(d2h(dx0_pin, dx0, td, st_g));
        HIPC(rec(dx0_done, st_g));
        HIPC(hsync(dx0_done));
        HIPC(hsync(loss_done));
        loss_sum += double(*loss_pin);
        t_bwd = ms_since(t_start);
        if (mb == 0) {  // the previous step's update of E_in reads G: it must be over
            const int we = wait_adam(lay.embed());
            if (we != MT_OK) return we;
        }
        const TilePtrs e = tile_ptrs(store, lay, lay.embed(), wblock);
        if (mb == 0) {
            // Clear last step's rows; rows not listed are zero.
            if (ein_clear_all) memset(e.g, 0, size_t(V) * d * 2);
            ein_clear_all = false;
            for (int32_t r : ein_touched) memset(e.g + int64_t(r) * d, 0, size_t(d) * 2);
            ein_touched.clear();
            ein_seen.assign(size_t(V), 0);
        }
        // This micro-batch's distinct rows, summed in fp32 in token order,
        // rounded to bf16 once, then stored (first micro-batch) or added into G
        // with one more rounding (the others), as the slab jobs do.
        std::vector<int32_t> rows;
        {
            std::vector<char> seen(size_t(V), 0);
            for (int t = 0; t < T; ++t)
                if (!seen[tk[t]]) {
                    seen[tk[t]] = 1;
                    rows.push_back(tk[t]);
                    if (!ein_seen[tk[t]]) {
                        ein_seen[tk[t]] = 1;
                        ein_touched.push_back(tk[t]);
                    }
                }
        }
        float* acc = ein_acc.data();
        pack_pool->parallel_for(d, 64, [&](int64_t c0, int64_t c1) {
            for (int32_t r : rows)
                for (int64_t c = c0; c < c1; ++c) acc[int64_t(r) * d + c] = 0.f;
            for (int t = 0; t < T; ++t) {
                float* row = acc + int64_t(tk[t]) * d;
                const uint16_t* g = dx0_pin + int64_t(t) * d;
                for (int64_t c = c0; c < c1; ++c) row[c] += bf16_to_f32(g[c]);
            }
            for (int32_t r : rows)
                for (int64_t c = c0; c < c1; ++c) {
                    uint16_t& gr = e.g[int64_t(r) * d + c];
                    const uint16_t v = f32_to_bf16(acc[int64_t(r) * d + c]);
                    gr = mb == 0 ? v : f32_to_bf16(bf16_to_f32(gr) + bf16_to_f32(v));
                }
        });
    }
    if (lay.embed() == fault_slab) {
        drain_jobs();
        failed = true;
        MT_FAIL(MT_E_INTERNAL, "injected slab-worker fault at unit %d", lay.embed());
    }
    if (opt.cross_step) {
        std::lock_guard<std::mutex> lk(q_mu);
        emb_deferred = true;
        emb_adam = cur_adam;
        emb_step_id = step + 1;
    } else {
        enqueue_job(lay.embed(), -1, JOB_ADAM);
    }
    // Synchronous step: every update lands before returning.  cross_step:
    // they run on; report a worker error that has already happened.
    int jr = MT_OK;
    if (!opt.cross_step) {
        jr = drain_jobs();
    } else {
        std::lock_guard<std::mutex> lk(q_mu);
        if (worker_status != MT_OK) {
            failed = true;
            set_error(worker_error);
            jr = worker_status;
            worker_status = MT_OK;
        }
    }
    uint32_t* ovf_pin = reinterpret_cast<uint32_t*>(loss_pin) + 1;
    HIPC(hipMemcpyAsync(ovf_pin, ws.ovf, 4, hipMemcpyDeviceToHost, st_c));
    HIPC(hsync(loss_done));
    HIPC(hipStreamSynchronize(st_c));
    HIPC(hipStreamSynchronize(st_w));
    HIPC(hipStreamSynchronize(st_g));
    if (jr != MT_OK) return jr;
    {
        std::lock_guard<std::mutex> lk(off_mu);
        intervals.insert(intervals.end(), off_intervals.begin(), off_intervals.end());
    }
    *loss_out = float(loss_sum / n_micro);  // mean over every token of the step
    ++step;
    const double t_total = ms_since(t_start);
    if (!trace_path.empty()) {
        // Debugging aid: every interval of the step on the device clock,
        // relative to the step's first event.
        if (FILE* f = fopen(trace_path.c_str(), "a")) {
            for (const Interval& iv : intervals) {
                float a = 0.f, b = 0.f;
                hipEventElapsedTime(&a, t_base, iv.a);
                hipEventElapsedTime(&b, t_base, iv.b);
                static const char* names[] = {"fwd", "head", "refwd", "bwd", "hfwd", "hbwd"};
                fprintf(f, "%lld,%s,%s,%d,%.4f,%.4f,%llu\n", (long long)step,
                        iv.kind == 0 ? "compute" : iv.kind == 1 ? "h2d" : "d2h",
                        iv.kind == 0 ? names[iv.visit] : "-", iv.unit, a, b, (unsigned long long)iv.bytes);
            }
            // Host spans on the host clock from the step's start (the device
            // clock starts within microseconds of it: the GPU is idle then).
            std::lock_guard<std::mutex> lk(trace_mu);
            for (const HostRec& h : host_recs) {
                const double a = std::chrono::duration<double, std::milli>(h.a - step_clock0).count();
                const double b = std::chrono::duration<double, std::milli>(h.b - step_clock0).count();
                fprintf(f, "%lld,%s,%d,%d,%.4f,%.4f,0\n", (long long)step, h.what, h.aux, h.unit, a, b);
            }
            fclose(f);
        }
    }

    if (stats) {
        memset(stats, 0, sizeof(*stats));
        stats->step_ms = t_total;
        auto el = [&](hipEvent_t a, hipEvent_t b) {
            float ms = 0.f;
            hipEventElapsedTime(&ms, a, b);
            return double(ms);
        };
        for (const Phases& ph : phases) {
            stats->fwd_ms += el(ph.start, ph.fwd);
            stats->head_ms += el(ph.fwd, ph.head);
            stats->bwd_ms += el(ph.head, ph.bwd);
        }
        stats->adam_tail_ms = t_total - t_bwd;
        // Interval unions: compute C, copies X = H2D u D2H.
        std::vector<std::pair<double, double>> C, X, H;
        for (auto& iv : intervals) {
            const double a = el(t_base, iv.a), b = el(t_base, iv.b);
            if (iv.kind == 0) {
                C.push_back({a, b});
                stats->compute_busy_ms += b - a;
            } else {
                X.push_back({a, b});
                if (iv.kind == 1) {
                    H.push_back({a, b});
                    stats->h2d_busy_ms += b - a;
                    stats->h2d_bytes += iv.bytes;
                } else {
                    stats->d2h_busy_ms += b - a;
                    stats->d2h_bytes += iv.bytes;
                }
            }
        }
        auto merge = [](std::vector<std::pair<double, double>> v) {
            std::sort(v.begin(), v.end());
            std::vector<std::pair<double, double>> out;
            for (auto& p : v) {
                if (!out.empty() && p.first <= out.back().second) out.back().second = std::max(out.back().second, p.second);
                else out.push_back(p);
            }
            return out;
        };
        auto len = [](const std::vector<std::pair<double, double>>& v) {
            double s = 0;
            for (auto& p : v) s += p.second - p.first;
            return s;
        };
        auto Cm = merge(C), Xm = merge(X), Hm = merge(H);
        auto intersect = [](const std::vector<std::pair<double, double>>& A,
                            const std::vector<std::pair<double, double>>& Bv) {
            double r = 0;
            size_t i = 0, j = 0;
            while (i < A.size() && j < Bv.size()) {
                const double lo = std::max(A[i].first, Bv[j].first), hi = std::min(A[i].second, Bv[j].second);
                if (hi > lo) r += hi - lo;
                if (A[i].second < Bv[j].second) ++i;
                else ++j;
            }
            return r;
        };
        auto clip = [](const std::vector<std::pair<double, double>>& v, double lo, double hi) {
            std::vector<std::pair<double, double>> out;
            for (auto& p : v) {
                const double a = std::max(p.first, lo), b = std::min(p.second, hi);
                if (b > a) out.push_back({a, b});
            }
            return out;
        };
        const double inter = intersect(Cm, Xm);
        const double lc = len(Cm), lx = len(Xm);
        stats->overlap_ratio = std::min(lc, lx) > 0 ? inter / std::min(lc, lx) : 0.0;
        stats->compute_union_ms = lc;
        stats->copy_union_ms = lx;
        stats->overlap_ms = inter;
        stats->pcie_busy_frac = t_total > 0 ? len(Hm) / t_total : 0.0;
        // The same per phase (forward, head, backward), and the transfer time
        // no compute hides, |X \ C|.
        // Summed over the micro-batches' windows of each phase.
        double ip[3] = {}, lcp[3] = {}, lxp[3] = {};
        for (const Phases& ph : phases) {
            const double edges[4] = {el(t_base, ph.start), el(t_base, ph.fwd), el(t_base, ph.head),
                                     el(t_base, ph.bwd)};
            for (int p = 0; p < 3; ++p) {
                const auto Cp = clip(Cm, edges[p], edges[p + 1]), Xp = clip(Xm, edges[p], edges[p + 1]);
                ip[p] += intersect(Cp, Xp);
                lcp[p] += len(Cp);
                lxp[p] += len(Xp);
            }
        }
        for (int p = 0; p < 3; ++p) {
            stats->overlap_phase[p] = std::min(lcp[p], lxp[p]) > 0 ? ip[p] / std::min(lcp[p], lxp[p]) : 0.0;
            stats->exposed_transfer_ms[p] = lxp[p] - ip[p];
        }
        // Switch gaps (end of a compute visit to the start of the next, by
        // the phase the next visit starts in) and device idle time (neither
        // compute nor copies) per phase.
        {
            std::vector<std::pair<double, double>> cv;
            for (auto& iv : intervals)
                if (iv.kind == 0) cv.push_back({el(t_base, iv.a), el(t_base, iv.b)});
            std::sort(cv.begin(), cv.end());
            std::vector<double> gaps[3];
            double idle[3] = {};
            for (const Phases& ph : phases) {
                const double edges[4] = {el(t_base, ph.start), el(t_base, ph.fwd), el(t_base, ph.head),
                                         el(t_base, ph.bwd)};
                for (size_t i = 1; i < cv.size(); ++i) {
                    const double st = cv[i].first;
                    for (int p = 0; p < 3; ++p)
                        if (st > edges[p] && st <= edges[p + 1]) gaps[p].push_back(std::max(0.0, st - cv[i - 1].second));
                }
                for (int p = 0; p < 3; ++p) {
                    std::vector<std::pair<double, double>> both = clip(Cm, edges[p], edges[p + 1]);
                    const auto xp = clip(Xm, edges[p], edges[p + 1]);
                    both.insert(both.end(), xp.begin(), xp.end());
                    idle[p] += (edges[p + 1] - edges[p]) - len(merge(both));
                }
            }
            for (int p = 0; p < 3; ++p) {
                auto& g = gaps[p];
                if (!g.empty()) {
                    std::nth_element(g.begin(), g.begin() + g.size() / 2, g.end());
                    stats->switch_gap_ms[p] = g[g.size() / 2];
                }
                stats->device_idle_ms[p] = std::max(0.0, idle[p]);
            }
        }
        // Why the link idled before each weight-stream copy, and the switch
        // latency of the visits that had nothing to wait for.
        {
            const double eps = 0.02;  // ms: events on one stream back to back
            std::vector<std::pair<double, double>> tm(intervals.size());
            for (size_t i = 0; i < intervals.size(); ++i) tm[i] = {el(t_base, intervals[i].a), el(t_base, intervals[i].b)};
            std::vector<std::array<double, 4>> pe;
            for (const Phases& ph : phases)
                pe.push_back({el(t_base, ph.start), el(t_base, ph.fwd), el(t_base, ph.head), el(t_base, ph.bwd)});
            auto phase_of = [&](double t) {
                for (const auto& e : pe)
                    for (int p = 0; p < 3; ++p)
                        if (t >= e[p] && t <= e[p + 1]) return p;
                return -1;
            };
            bool have_prev = false;
            double prev_end = 0.0;  // end of the previous weight-stream copy
            for (size_t i = 0; i < intervals.size(); ++i) {
                const Interval& iv = intervals[i];
                if (iv.kind != 1) continue;
                const double s0 = tm[i].first, gap = s0 - prev_end;
                const bool counted = have_prev && gap > eps;
                prev_end = have_prev ? std::max(prev_end, tm[i].second) : tm[i].second;
                have_prev = true;
                const int p = phase_of(s0);
                if (!counted || p < 0) continue;
                int cause = 2;
                if (iv.slot >= 0) {
                    // the end of the last compute visit on this slot before the copy
                    double f = -1.0;
                    for (size_t j = 0; j < intervals.size(); ++j)
                        if (intervals[j].kind == 0 && intervals[j].slot == iv.slot && tm[j].second <= s0 + eps)
                            f = std::max(f, tm[j].second);
                    cause = f >= 0.0 && s0 - f <= eps ? 0 : 1;
                }
                stats->h2d_idle_ms[p][cause] += gap;
            }
            std::vector<size_t> cvis;
            for (size_t i = 0; i < intervals.size(); ++i)
                if (intervals[i].kind == 0) cvis.push_back(i);
            std::sort(cvis.begin(), cvis.end(), [&](size_t x, size_t y) { return tm[x].first < tm[y].first; });
            std::vector<double> rs;
            for (size_t k = 1; k < cvis.size(); ++k) {
                const size_t i = cvis[k], j = cvis[k - 1];
                ++stats->switches;
                const Interval& iv = intervals[i];
                double ready = iv.last_h2d >= 0 ? tm[size_t(iv.last_h2d)].second : 0.0;
                if (iv.seq >= 0) {
                    bool found = false;
                    for (size_t m = 0; m < intervals.size(); ++m)
                        if (intervals[m].kind == 2 && intervals[m].seq == iv.seq) {
                            ready = std::max(ready, tm[m].second);
                            found = true;
                        }
                    if (!found) continue;
                }
                if (ready <= tm[j].second + eps) rs.push_back(std::max(0.0, tm[i].first - tm[j].second));
            }
            stats->ready_switches = int32_t(rs.size());
            if (!rs.empty()) {
                std::sort(rs.begin(), rs.end());
                stats->ready_switch_ms[0] = rs[rs.size() / 2];
                stats->ready_switch_ms[1] = rs[std::min(rs.size() - 1, size_t(0.9 * double(rs.size())))];
            }
        }
        stats->pack_ms = pack_ms;
        {
            std::lock_guard<std::mutex> lk(q_mu);
            stats->adam_ms = adam_ms_acc;
            stats->adam_wait_ms = adam_wait_ms;
        }
        stats->fp16_saturated = *ovf_pin;
        stats->gpu_arena_bytes = plan.total;
        stats->pinned_bytes = pplan.total;
        stats->host_store_bytes = uint64_t(lay.store_bytes);
        if (opt.profile_kernels) {
            stats->n_sites = N_SITES;
            for (auto& r : site_recs) {
                stats->site_ms[r.site] += el(r.a, r.b);
                stats->site_launches[r.site] += 1;
            }
        }
    }
    return MT_OK;
}

// ------------------------------------------------------- test entries ----
int Ctx::layer_fwd(int layer, const void* x, void* y, int B, int S) {
    if (failed) MT_FAIL(MT_E_STATE, "context failed earlier");
    if (layer < 0 || layer >= lay.L()) MT_FAIL(MT_E_INVAL, "layer %d out of range", layer);
    if (!x || !y) MT_FAIL(MT_E_INVAL, "x and y must not be NULL");
    if (B < 1 || S < 1 || int64_t(B) * S > ws.maxT || S > opt.max_seq) MT_FAIL(MT_E_INVAL, "batch x seq exceeds the workspace");
    timing = false;
    tev_next = 0;
    HIPC(ensure_rope(S));
    const int slot = 0;
    slot_unit.assign(plan.n_slots, -1);
    const int r = stream_unit(layer, slot);
    if (r != MT_OK) return r;
    HIPC(rec(wready[slot], st_w));
    HIPC(wait(st_c, wready[slot]));
    HIPC(fwd_layer(bind_layer(lay, arena + plan.wslot[slot]), static_cast<const uint16_t*>(x),
                   static_cast<uint16_t*>(y), B, S, true));
    HIPC(rec(slot_free[slot], st_c));
    HIPC(hipStreamSynchronize(st_c));
    HIPC(hipStreamSynchronize(st_w));
    slot_unit.assign(plan.n_slots, -1);
    return MT_OK;
}

int Ctx::layer_bwd(int layer, const void* x, const void* dy, void* dx, void* gtile, int B, int S) {
    if (failed) MT_FAIL(MT_E_STATE, "context failed earlier");
    if (layer < 0 || layer >= lay.L()) MT_FAIL(MT_E_INVAL, "layer %d out of range", layer);
    if (!x || !dy || !dx || !gtile) MT_FAIL(MT_E_INVAL, "device pointers must not be NULL");
    if (reinterpret_cast<uintptr_t>(gtile) & 15) MT_FAIL(MT_E_INVAL, "grad_tile_dev must be 16-byte aligned");
    if (B < 1 || S < 1 || int64_t(B) * S > ws.maxT || S > opt.max_seq) MT_FAIL(MT_E_INVAL, "batch x seq exceeds the workspace");
    timing = false;
    tev_next = 0;
    HIPC(ensure_rope(S));
    const int slot = 0;
    slot_unit.assign(plan.n_slots, -1);
    const int r = stream_unit(layer, slot);
    if (r != MT_OK) return r;
    HIPC(rec(wready[slot], st_w));
    HIPC(wait(st_c, wready[slot]));
    HIPC(fill_zero(gtile, (uint64_t(lay.units[layer].elems) * 2 + 15) & ~uint64_t(15), st_c));
    HIPC(bwd_layer(bind_layer(lay, arena + plan.wslot[slot]), bind_layer(lay, gtile),
                   static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(dy), static_cast<uint16_t*>(dx), B,
                   S));
    HIPC(rec(slot_free[slot], st_c));
    HIPC(hipStreamSynchronize(st_c));
    HIPC(hipStreamSynchronize(st_w));
    slot_unit.assign(plan.n_slots, -1);
    return MT_OK;
}

}  // namespace mt

// ================================================================ C ABI ====
using mt::Ctx;

struct mt_ctx {
    Ctx impl;
};

extern "C" {

int mt_default_options(mt_options* o) {
    if (!o) return MT_E_INVAL;
    memset(o, 0, sizeof(*o));
    o->max_batch = 1;
    o->max_seq = 128;
    o->n_weight_slots = 2;
    o->n_grad_slabs = 12;
    o->slot_mode = 0;
    o->ckpt_on_host = 1;
    o->resident = 0;
    o->host_threads = 0;
    o->head_chunk = 0;
    o->profile_kernels = 0;
    o->pin_store = 0;
    o->cross_step = 0;
    o->ckpt_interval = 1;
    o->pin_weights = 0;
    o->head_vocab_chunk = 0;
    o->poison_released = 0;
    o->keep_grads = 1;
    o->ckpt_attn = 0;
    o->lr = 1e-4f;
    o->beta1 = 0.9f;
    o->beta2 = 0.999f;
    o->adam_eps = 1e-8f;
    o->init_std = 0.02f;
    o->seed = 1234;
    return MT_OK;
}

int mt_workspace_bytes(const mt_shape* sh, const mt_options* o, uint64_t* gpu_arena, uint64_t* pinned,
                       uint64_t* host_store) {
    int r = mt::validate_shape(sh);
    if (r != MT_OK) return r;
    r = mt::validate_options(o);
    if (r != MT_OK) return r;
    const mt::Layout lay = mt::make_layout(*sh);
    const mt::ArenaPlan p = mt::plan_arena(lay, *o, nullptr, nullptr);
    const mt::PinnedPlan pp = mt::plan_pinned(lay, *o, p.slot_bytes);
    if (gpu_arena) *gpu_arena = p.total;
    if (pinned) *pinned = pp.total;
    if (host_store) *host_store = uint64_t(lay.store_bytes);
    return MT_OK;
}

int mt_init(const mt_shape* sh, const mt_options* o, void* gpu_arena, uint64_t arena_bytes,
            void* const streams[3], mt_ctx** out) {
    if (!out) {
        mt::set_error("out is NULL");
        return MT_E_INVAL;
    }
    *out = nullptr;
    int r = mt::validate_shape(sh);
    if (r != MT_OK) return r;
    r = mt::validate_options(o);
    if (r != MT_OK) return r;
    mt_ctx* c = new (std::nothrow) mt_ctx;
    if (!c) {
        mt::set_error("out of host memory");
        return MT_E_NOMEM;
    }
    try {
        r = c->impl.init(*sh, *o, gpu_arena, arena_bytes, streams);
    } catch (const std::bad_alloc&) {
        mt::set_error("out of host memory during init");
        r = MT_E_NOMEM;
    } catch (...) {
        mt::set_error("unexpected exception during init");
        r = MT_E_INTERNAL;
    }
    if (r != MT_OK) {
        delete c;
        return r;
    }
    *out = c;
    return MT_OK;
}

int mt_train_step(mt_ctx* c, const int32_t* tokens, const int32_t* labels, int32_t batch, int32_t seq,
                  float* loss_out, mt_stats* stats) {
    if (!c) {
        mt::set_error("ctx is NULL");
        return MT_E_INVAL;
    }
    try {
        return c->impl.train_step(tokens, labels, 1, batch, seq, loss_out, stats);
    } catch (...) {
        c->impl.failed = true;
        mt::set_error("unexpected exception in mt_train_step");
        return MT_E_INTERNAL;
    }
}

int mt_train_step_accum(mt_ctx* c, const int32_t* tokens, const int32_t* labels, int32_t n_micro, int32_t batch,
                        int32_t seq, float* loss_out, mt_stats* stats) {
    if (!c) {
        mt::set_error("ctx is NULL");
        return MT_E_INVAL;
    }
    try {
        return c->impl.train_step(tokens, labels, n_micro, batch, seq, loss_out, stats);
    } catch (...) {
        c->impl.failed = true;
        mt::set_error("unexpected exception in mt_train_step_accum");
        return MT_E_INTERNAL;
    }
}

int mt_layer_fwd(mt_ctx* c, int32_t layer, const void* x, void* y, int32_t batch, int32_t seq) {
    if (!c) {
        mt::set_error("ctx is NULL");
        return MT_E_INVAL;
    }
    try {
        return c->impl.layer_fwd(layer, x, y, batch, seq);
    } catch (...) {
        c->impl.failed = true;
        mt::set_error("unexpected exception in mt_layer_fwd");
        return MT_E_INTERNAL;
    }
}

int mt_layer_bwd(mt_ctx* c, int32_t layer, const void* x, const void* dy, void* dx, void* gtile, int32_t batch,
                 int32_t seq) {
    if (!c) {
        mt::set_error("ctx is NULL");
        return MT_E_INVAL;
    }
    try {
        return c->impl.layer_bwd(layer, x, dy, dx, gtile, batch, seq);
    } catch (...) {
        c->impl.failed = true;
        mt::set_error("unexpected exception in mt_layer_bwd");
        return MT_E_INTERNAL;
    }
}

int mt_get_tensor(mt_ctx* c, int32_t unit, int32_t idx, int32_t which, void* dst, uint64_t bytes) {
    if (!c || !dst) {
        mt::set_error("ctx and host_dst must not be NULL");
        return MT_E_INVAL;
    }
    const mt::Layout& lay = c->impl.lay;
    if (unit < 0 || unit >= int(lay.units.size())) MT_FAIL(MT_E_INVAL, "unit %d out of range", unit);
    const mt::UnitLayout& u = lay.units[unit];
    if (idx < 0 || idx >= u.ntensors) MT_FAIL(MT_E_INVAL, "tensor %d out of range", idx);
    if (which < MT_W || which > MT_V) MT_FAIL(MT_E_INVAL, "bad `which` %d", which);
    const mt::TensorDesc& t = u.t[idx];
    const uint64_t n = uint64_t(t.rows * t.cols), es = which <= MT_G ? 2 : 4;
    if (bytes != n * es) MT_FAIL(MT_E_INVAL, "bytes %llu != %llu", (unsigned long long)bytes, (unsigned long long)(n * es));
    if (which == MT_G && !c->impl.opt.keep_grads)
        MT_FAIL(MT_E_STATE, "gradients are not kept in the store (keep_grads = 0)");
    const int ds = c->impl.drain_jobs();  // updates still queued by a cross-step train step
    if (ds != MT_OK) return ds;
    const int ls = c->impl.ensure_loaded(unit);  // a shard still pending after a lazy restore
    if (ls != MT_OK) return ls;
    const mt::TilePtrs p = mt::tile_ptrs(c->impl.store, lay, unit, c->impl.wblock);
    const void* src = which == MT_W ? static_cast<const void*>(p.w + t.off)
                    : which == MT_G ? static_cast<const void*>(p.g + t.off)
                    : which == MT_MASTER ? static_cast<const void*>(p.master + t.off)
                    : which == MT_M ? static_cast<const void*>(p.m + t.off)
                                    : static_cast<const void*>(p.v + t.off);
    memcpy(dst, src, bytes);
    return MT_OK;
}

int mt_set_tensor(mt_ctx* c, int32_t unit, int32_t idx, int32_t which, const void* srcp, uint64_t bytes) {
    if (!c || !srcp) {
        mt::set_error("ctx and host_src must not be NULL");
        return MT_E_INVAL;
    }
    const mt::Layout& lay = c->impl.lay;
    if (unit < 0 || unit >= int(lay.units.size())) MT_FAIL(MT_E_INVAL, "unit %d out of range", unit);
    const mt::UnitLayout& u = lay.units[unit];
    if (idx < 0 || idx >= u.ntensors) MT_FAIL(MT_E_INVAL, "tensor %d out of range", idx);
    if (which < MT_W || which > MT_V) MT_FAIL(MT_E_INVAL, "bad `which` %d", which);
    const mt::TensorDesc& t = u.t[idx];
    const uint64_t n = uint64_t(t.rows * t.cols), es = which <= MT_G ? 2 : 4;
    if (bytes != n * es) MT_FAIL(MT_E_INVAL, "bytes %llu != %llu", (unsigned long long)bytes, (unsigned long long)(n * es));
    const int ds = c->impl.drain_jobs();
    if (ds != MT_OK) return ds;
    const int ls = c->impl.ensure_loaded(unit);
    if (ls != MT_OK) return ls;
    const mt::TilePtrs p = mt::tile_ptrs(c->impl.store, lay, unit, c->impl.wblock);
    void* dst = which == MT_W ? static_cast<void*>(p.w + t.off)
              : which == MT_G ? static_cast<void*>(p.g + t.off)
              : which == MT_MASTER ? static_cast<void*>(p.master + t.off)
              : which == MT_M ? static_cast<void*>(p.m + t.off)
                              : static_cast<void*>(p.v + t.off);
    memcpy(dst, srcp, bytes);
    return MT_OK;
}

int mt_sync(mt_ctx* c) {
    if (!c) {
        mt::set_error("ctx is NULL");
        return MT_E_INVAL;
    }
    return c->impl.drain_jobs();
}

int mt_checkpoint_save(mt_ctx* c, const char* dir) {
    if (!c || !dir || !*dir) {
        mt::set_error("ctx and dir must not be NULL or empty");
        return MT_E_INVAL;
    }
    try {
        return c->impl.checkpoint_save(dir);
    } catch (...) {
        mt::set_error("unexpected exception in mt_checkpoint_save");
        return MT_E_INTERNAL;
    }
}

int mt_checkpoint_restore(mt_ctx* c, const char* dir, int32_t lazy) {
    if (!c || !dir || !*dir) {
        mt::set_error("ctx and dir must not be NULL or empty");
        return MT_E_INVAL;
    }
    try {
        return c->impl.checkpoint_restore(dir, lazy != 0);
    } catch (...) {
        c->impl.failed = true;
        mt::set_error("unexpected exception in mt_checkpoint_restore");
        return MT_E_INTERNAL;
    }
}

int64_t mt_abi_sizeof(int32_t which) {
    switch (which) {
        case 0: return int64_t(sizeof(mt_shape));
        case 1: return int64_t(sizeof(mt_options));
        case 2: return int64_t(sizeof(mt_stats));
        case 3: return int64_t(sizeof(mt_tensor_info));
        default: return -1;
    }
}

int mt_step_count(mt_ctx* c, int64_t* out) {
    if (!c || !out) return MT_E_INVAL;
    *out = c->impl.step;
    return MT_OK;
}

void mt_destroy(mt_ctx* c) { delete c; }

}  // extern "C"

