/*
 * mt.h -- C ABI of the layer-streamed decoder training step for MI355X.
 *
 * Pages the declarations below cite:
 *   [Review]  "MegaTrain: Full Precision Training of 100B+ Parameter Large
 *             Language Models on a Single GPU Review", dimensionstp.github.io
 *   [Hotdry]  MegaTrain checkpoint strategy and communication overlap,
 *             blog.hotdry.top (2026-04-09)
 *   [Lilting] "MegaTrainはシングルGPUで120BパラメータLLMをフル精度訓練する",
 *             lilting.ch
 *   [Peter]   MegaTrain translated abstract and technical details,
 *             peter-blog.pages.dev
 *
 * What the library does.  All persistent training state lives in a host
 * master store, one contiguous tile per unit holding BF16 W, BF16 G and the
 * FP32 master, m and v ([Review] 3-2 item 4 "Layer-contiguous tiling and
 * pinned slabs"; [Hotdry] host memory layout section; [Lilting] 16-byte per
 * parameter table).  A training step streams each unit's BF16 weights
 * through pinned staging into GPU weight slots, binds them to a stateless
 * block template, runs forward, then recompute and backward in reverse
 * order, streams BF16 gradients out to a pool of pinned slabs, and runs Adam
 * on the host as each unit's gradients land ([Review] 3-2 items 1-6;
 * [Hotdry] "三层 CUDA Stream 流水线与双缓冲调度" and "事件驱动同步协议";
 * [Peter] abstract).
 *
 * Units.  unit 0..L-1 are decoder layers, unit L is the LM head (final
 * RMSNorm gain gf and the output table E_out), unit L+1 is the input
 * embedding E_in, which never leaves the host: its gather and scatter run
 * on host memory.  Tensor order inside a decoder tile is
 *   0 g1[d]  1 wq[Hq*hd x d]  2 wk[Hkv*hd x d]  3 wv[Hkv*hd x d]
 *   4 wo[d x Hq*hd]  5 g2[d]  6 wg[F x d]  7 wu[F x d]  8 wd[d x F]
 * each row-major [out x in], so wq|wk|wv and wg|wu are contiguous; the head
 * tile is 0 gf[d]  1 e_out[V x d]; the embedding tile is 0 e_in[V x d].
 *
 * Conventions.  Every function returns MT_OK (0) or a negative MT_E_* code
 * and never aborts or throws across the ABI; mt_last_error() gives the
 * calling thread's detail text for its last failure.  Arguments are checked
 * before any device work.  A context is not re-entrant: one call at a time.
 * A failure inside a step marks the context failed (MT_E_STATE afterwards).
 */
#ifndef MT_H
#define MT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MT_OK 0
#define MT_E_INVAL (-1)    /* bad argument: shape, size, pointer, token id */
#define MT_E_NOMEM (-2)    /* host, pinned or device arena too small        */
#define MT_E_HIP (-3)      /* a HIP runtime call failed                     */
#define MT_E_STATE (-4)    /* the context failed earlier                    */
#define MT_E_INTERNAL (-5) /* a host worker failed                          */
#define MT_E_IO (-6)       /* a checkpoint file could not be written or read */

/* Which copy of a tensor mt_get_tensor / mt_set_tensor address. */
#define MT_W 0      /* BF16 weight (uint16 bit patterns)            */
#define MT_G 1      /* BF16 gradient of the last step              */
#define MT_MASTER 2 /* FP32 master weight                           */
#define MT_M 3      /* FP32 Adam first moment                       */
#define MT_V 4      /* FP32 Adam second moment                      */

#define MT_DTYPE_BF16 0
#define MT_DTYPE_F32 1

/* Model shape.  A pre-norm decoder: RMSNorm, causal GQA attention with
 * rotary positions, residual, RMSNorm, SwiGLU MLP, residual; no biases.
 * Constraints: d_model, head_dim, ffn_dim, vocab multiples of 8; head_dim
 * in {64, 128}; n_heads a multiple of n_kv_heads. */
typedef struct mt_shape {
    int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab;
    float rms_eps;   /* inside the square root, e.g. 1e-6 */
    float rope_base; /* e.g. 10000                        */
} mt_shape;

/* Run options.  mt_default_options() fills the defaults noted here. */
typedef struct mt_options {
    int32_t max_batch, max_seq;  /* size the device workspace: T <= max_batch*max_seq */
    int32_t n_weight_slots;      /* GPU weight buffers, 1..4 (2: ping-pong, [Review] 3-2 item 3) */
    int32_t n_grad_slabs;        /* pinned gradient slabs, 1..64 (12, [Hotdry] stream section) */
    int32_t slot_mode;           /* 0: W slots and G buffers separate; 1: one slot holds W and G,
                                    refilled only after its G left ([Hotdry] buffer-free event) */
    int32_t ckpt_on_host;        /* 1: layer inputs go to a pinned host ring; 0: kept on the GPU */
    int32_t resident;            /* 1: all units' weights copied to the GPU once per step, no
                                    per-layer streaming (the comparison run) */
    int32_t host_threads;        /* host worker threads; 0: all online CPUs */
    int32_t head_chunk;          /* token rows per LM-head chunk; 0: min(T, 8192) */
    int32_t profile_kernels;     /* 1: time every kernel site with HIP events (mt_stats.site_*) */
    int32_t pin_store;           /* 1: allocate the host store page-locked, so H2D reads it
                                    directly instead of packing into staging; 0 (default): pageable
                                    store plus two pinned staging buffers, as on the pages */
    int32_t cross_step;          /* 1: mt_train_step returns once the loss is known and every
                                    unit's Adam is queued; Adam runs on, lowest unit first, and the
                                    next step streams a unit only after its update has landed
                                    (the next forward overlaps the Adam tail).  The input
                                    embedding's update waits for the next step's tokens, whose
                                    rows it updates first.  Same results as 0.  mt_sync, and every
                                    entry that reads or writes the store, wait for the queued
                                    updates first.  0 (default): synchronous step */
    int32_t ckpt_interval;       /* k >= 1: the forward keeps every k-th layer input (layers 0, k,
                                    2k, ...); the backward restores a block's first input, re-runs
                                    the forward of the block's first k-1 layers to rebuild the
                                    others, then runs the block's backward ([Argon] block-wise
                                    recomputation).  1 (default): every layer's input.  k > 1 needs
                                    ckpt_on_host = 1 */
    int32_t pin_weights;         /* 1: the W regions of all units live in one page-locked block
                                    (2 B/param), so StreamIn copies straight from it with no pack;
                                    G and the optimizer state stay in the pageable tiles.  0
                                    (default): W inside each pageable tile, packed into staging */
    int32_t head_vocab_chunk;    /* the LM head streamed in chunks of E_out rows, so the weight
                                    slots are sized to the largest decoder layer instead of the
                                    head: a forward pass over the chunks keeps a running
                                    logsumexp per token, a backward pass (chunks in reverse order)
                                    recomputes each chunk's logits and forms its gradients; each
                                    chunk's gradient is offloaded and updated on its own ([Hotdry]
                                    staging buffers sized to the largest layer).  0 (default): the
                                    head is one unit; -1: rows per chunk chosen so a chunk fits the
                                    largest decoder layer's slot; k > 0 (a multiple of 8): k rows */
    int32_t poison_released;     /* debug, 1: fill every weight slot with bf16 NaN when its last
                                    compute visit releases it (the slot is then re-streamed even
                                    where it still held the unit), and every gradient area once
                                    its copy to a slab is done; a late reader of a released
                                    buffer then turns the step's results to NaN.  Needs
                                    slot_mode 0 and resident 0.  Same results as 0 */
    int32_t keep_grads;          /* 1 (default): the store's G region receives every unit's BF16
                                    gradient (the slab is unpacked into G, then Adam reads it:
                                    [Hotdry] the CPU thread that unpacks slabs and runs Adam).
                                    0: with one micro-batch per step Adam reads the slab itself
                                    and G is not written (2 B/param less host-DRAM traffic per
                                    step); G still accumulates micro-batches, and
                                    mt_get_tensor(MT_G) is refused.  Same W, master, m, v */
    int32_t ckpt_attn;           /* 1: the forward also checkpoints every layer's attention output
                                    (fp16) and log-sum-exp (fp32) to a second pinned host ring,
                                    and the backward's recompute restores them instead of running
                                    the attention forward again: long sequences, where that
                                    forward dominates the recompute, trade T*Hq*hd*2 + T*Hq*4
                                    bytes per layer each way over PCIe for it.  Needs
                                    ckpt_on_host = 1 and ckpt_interval = 1.  Same results as 0
                                    (default) */
    uint64_t slot_bytes_override;      /* 0: largest unit's weight bytes */
    uint64_t workspace_bytes_override; /* 0: computed from max_batch*max_seq */
    float lr, beta1, beta2, adam_eps;  /* 1e-4, 0.9, 0.999, 1e-8 */
    float init_std;                    /* 0.02: matrices N(0, init_std^2); gains 1.0 */
    uint64_t seed;                     /* weight init seed */
} mt_options;

#define MT_MAX_SITES 48

/* Per-step statistics (all times in milliseconds of wall or device time). */
typedef struct mt_stats {
    double step_ms;       /* wall time of mt_train_step, Adam tail included */
    double fwd_ms, head_ms, bwd_ms, adam_tail_ms; /* wall time per phase */
    double compute_busy_ms; /* sum of compute-stream visit spans (device clock) */
    double h2d_busy_ms, d2h_busy_ms;   /* sum of copy durations (device clock) */
    double pack_ms, adam_ms;           /* host worker busy time */
    double adam_wait_ms;               /* time this step waited for the previous step's Adam
                                          (cross_step) */
    double overlap_ratio;   /* |compute ∩ copies| / min(|compute|, |copies|) */
    double pcie_busy_frac;  /* |H2D| / step time */
    double overlap_phase[3];        /* overlap_ratio within the forward, the head, the backward */
    double exposed_transfer_ms[3];  /* |copies \ compute| per phase (device clock) */
    uint64_t h2d_bytes, d2h_bytes;
    uint64_t gpu_arena_bytes, pinned_bytes, host_store_bytes;
    int32_t n_sites;                       /* kernel sites timed (profile_kernels) */
    double site_ms[MT_MAX_SITES];          /* summed device time per site */
    uint64_t site_launches[MT_MAX_SITES];  /* launches per site */
    uint64_t fp16_saturated;  /* fp16 range guard: values of the attention operands (n1, Wqkv, Wo, q, k,
                                 v, o) whose magnitude exceeded the fp16 range in this step and were
                                 saturated to +-65504 (0 in a healthy run) */
    double compute_union_ms;  /* |C|: union of compute-stream visit spans (device clock) */
    double copy_union_ms;     /* |X|: union of H2D and D2H copy spans */
    double overlap_ms;        /* |C ∩ X|; |C ∩ X| / |X| is the share of transfer time hidden under compute */
    double switch_gap_ms[3];  /* median gap between the end of one compute visit and the start of the
                                 next, per phase (forward, head, backward): the double-buffer switch
                                 latency, including any wait for the next unit's weights ([Hotdry]
                                 monitoring section: switch latency) */
    double device_idle_ms[3]; /* per phase: time with neither a compute visit nor a copy running */
    /* Prefetch timing ([Peter] technical details, memory prefetch strategy):
     * the time the host-to-device link idles before a copy on the weight
     * stream, per phase and by what the copy waited for: [p][0] its slot
     * (the earliest any schedule over the same slots could issue it),
     * [p][1] the host (the update of its weights, or the pack), [p][2]
     * copies that are not weights (checkpoint restores, labels, inputs). */
    double h2d_idle_ms[3][3];
    /* Switch latency of the double buffer ([Hotdry] monitoring section):
     * start of a compute visit minus the end of the one before, over the
     * visits whose weights (and, writing gradients, whose gradient area)
     * were ready before the previous visit ended: median and 90th
     * percentile; ready_switches of switches visits were ready. */
    double ready_switch_ms[2];
    int32_t ready_switches, switches;
} mt_stats;

typedef struct mt_tensor_info {
    char name[16];
    uint64_t offset_elems; /* element offset inside the unit's BF16 weight region */
    int64_t rows, cols;    /* a gain vector has rows = 1 */
    int32_t dtype;         /* MT_DTYPE_BF16 for W and G; MT_MASTER/M/V are F32 */
} mt_tensor_info;

typedef struct mt_ctx mt_ctx;

/* Defaults for every field of *opt. */
int mt_default_options(mt_options* opt);

/* Bytes needed: device arena, pinned host memory, host master store. */
int mt_workspace_bytes(const mt_shape* shape, const mt_options* opt, uint64_t* gpu_arena,
                       uint64_t* pinned, uint64_t* host_store);

/* Create a context.  gpu_arena: caller-owned device memory of arena_bytes
 * (>= mt_workspace_bytes' gpu_arena), 256-byte aligned, owned by the caller
 * and outliving the context.  streams[3]: caller-owned hipStream_t for
 * compute, weight H2D and gradient D2H ([Peter] "CUDA Stream 管理"); NULL
 * entries make the library create its own.  The library allocates the host
 * store, pinned staging and slabs, events and host threads, initialises the
 * weights from opt->seed (matrices N(0, init_std^2) rounded to BF16, gains
 * 1.0, master = W, m = v = G = 0) and returns *out.  Errors: MT_E_INVAL,
 * MT_E_NOMEM, MT_E_HIP. */
int mt_init(const mt_shape* shape, const mt_options* opt, void* gpu_arena, uint64_t arena_bytes,
            void* const streams[3], mt_ctx** out);

/* One training step over host int32 tokens and labels [batch x seq]
 * (row t = b*seq + s; copied during the call).  Runs the streamed forward,
 * the fused LM head, the recomputing backward and the host Adam (step count
 * advanced by one), then returns the mean token cross-entropy in *loss_out.
 * Synchronous unless opt->cross_step: all Adam work has finished on return.
 * With cross_step the updates of this step may still be running on return
 * (mt_sync waits for them).  stats_out may be NULL.  Errors: MT_E_INVAL (shape beyond max_batch*max_seq, token or label
 * outside [0, vocab), NULL pointers), MT_E_HIP, MT_E_INTERNAL, MT_E_STATE.
 * Debugging aid: with the environment variable MT_TRACE=<path> set when the
 * context is created, every step appends its intervals (compute visits with
 * their kind and unit, H2D and D2H copies with their bytes; device-clock ms
 * from the step's first event) to <path> as CSV lines
 * step,kind,visit,unit,start_ms,end_ms,bytes.  Host-side spans follow with
 * the kind host_job (one update job; visit = mode*100 + slab), host_pick (the
 * worker's choice; visit = jobs queued*100 + whether its gradients had
 * landed), host_slab_wait, host_staging_wait and host_pack, on the host
 * clock from the step's start. */
int mt_train_step(mt_ctx* ctx, const int32_t* tokens, const int32_t* labels, int32_t batch,
                  int32_t seq, float* loss_out, mt_stats* stats_out);

#define MT_MAX_MICRO 4096

/* One optimizer step over n_micro micro-batches: tokens and labels are
 * [n_micro x batch x seq] int32 (micro-batch j at offset j*batch*seq).
 * The host keeps the accumulated gradient in each tile's BF16 G region
 * ([Review] 3-2 item 1: parameters, the accumulated gradient and the
 * optimizer state live on the host; [Hotdry] "三层 CUDA Stream 流水线与双缓冲调度":
 * the CPU thread unpacks each slab and accumulates it into the master store).
 * Every micro-batch runs the whole streamed forward, head and recomputing
 * backward with the step's weights; its gradient is that of the mean loss
 * over all n_micro*batch*seq tokens, streamed out in BF16; the host stores
 * the first micro-batch's gradient into G and adds each later one into G
 * (fp32 add, one BF16 rounding, in micro-batch order); after the last one,
 * each unit's Adam runs once on G.  *loss_out is the mean cross-entropy over
 * all tokens.  n_micro = 1 is mt_train_step.  Synchronicity, stats and
 * errors as mt_train_step, plus MT_E_INVAL for n_micro outside
 * [1, MT_MAX_MICRO]; stats phase times are summed over the micro-batches. */
int mt_train_step_accum(mt_ctx* ctx, const int32_t* tokens, const int32_t* labels, int32_t n_micro,
                        int32_t batch, int32_t seq, float* loss_out, mt_stats* stats_out);

/* Wait until every queued host Adam update has been applied to the store
 * (a no-op for synchronous steps).  Returns the first error a host worker
 * met since the last call (MT_E_HIP, MT_E_INTERNAL), else MT_OK. */
int mt_sync(mt_ctx* ctx);

/* Test entry: forward of decoder layer `layer` on caller-owned device
 * buffers x_dev, y_dev (BF16 [batch*seq x d_model] row-major).  Streams the
 * layer's current weights in through the same pack, copy, weights-ready and
 * bind path as a step, runs the forward kernels and synchronises the compute
 * stream.  This is one visit of the stateless block template: the layer's
 * streamed weights bound to a template that holds no parameters of its own
 * ([Lilting] "Stateless Layer Templates"; [Peter] stateless template
 * section; [Review] 3-2 item 5). */
int mt_layer_fwd(mt_ctx* ctx, int32_t layer, const void* x_dev, void* y_dev, int32_t batch,
                 int32_t seq);

/* Test entry: recompute and backward of decoder layer `layer`.  x_dev is the
 * layer input, dy_dev the gradient of its output; writes dx_dev (BF16
 * [batch*seq x d_model]) and grad_tile_dev (BF16, the unit's W-region
 * layout of mt_tensor_desc, caller-owned device memory).  No Adam runs and
 * the store is not touched.  The backward visit of one layer: its forward
 * recomputed from the stored input, then differentiated ([Review] 3-2 item 2
 * "Streaming forward and block-wise backward"; [Argon] "Block-Wise
 * Recomputation"), with the gradients in the tile layout they are streamed
 * out in ([Hotdry] pinned gradient slabs). */
int mt_layer_bwd(mt_ctx* ctx, int32_t layer, const void* x_dev, const void* dy_dev, void* dx_dev,
                 void* grad_tile_dev, int32_t batch, int32_t seq);

/* Describe tensor idx of unit (offsets in elements inside the unit's W
 * region).  Pure host function.  Errors: MT_E_INVAL.  The layout is the
 * layer-contiguous tile: one unit's tensors back to back in one flat region,
 * so a unit streams as a single copy ([Review] 3-2 item 4 "Layer-contiguous
 * tiling and pinned slabs"; [Hotdry] host memory layout section). */
int mt_tensor_desc(const mt_shape* shape, int32_t unit, int32_t idx, mt_tensor_info* out);

/* Number of tensors in a unit (9, 2 or 1), or a negative error. */
int mt_unit_tensors(const mt_shape* shape, int32_t unit);

/* Element count of a unit's weight region (all its tensors, padding
 * included), or 0 for a bad unit. */
uint64_t mt_unit_elems(const mt_shape* shape, int32_t unit);

/* Copy one tensor between the host store and caller host memory.  `which`
 * is MT_W/MT_G (BF16, 2 bytes per element) or MT_MASTER/MT_M/MT_V (FP32);
 * bytes must equal rows*cols*element size.  mt_set_tensor(MT_W) also
 * refreshes nothing else: set MT_MASTER too to keep them consistent.  The
 * store is the host master copy of all persistent state, BF16 W and G with
 * the FP32 master, m and v ([Review] 3-2 item 1; [Lilting] 16-byte per
 * parameter table).  Both wait for queued host updates first.  Errors:
 * MT_E_INVAL (unit, tensor, which or bytes out of range, NULL pointers),
 * MT_E_STATE for mt_get_tensor(MT_G) on a context with keep_grads = 0, or
 * a host worker's or a lazy restore's error. */
int mt_get_tensor(mt_ctx* ctx, int32_t unit, int32_t idx, int32_t which, void* host_dst,
                  uint64_t bytes);
int mt_set_tensor(mt_ctx* ctx, int32_t unit, int32_t idx, int32_t which, const void* host_src,
                  uint64_t bytes);

/* Adam step count already applied (0 after init). */
int mt_step_count(mt_ctx* ctx, int64_t* out);

/* Checkpoint shards ([Hotdry] checkpoint sharding and restore): write every
 * unit's whole tile (W, G, master, m, v) and the step count to one file per
 * unit, dir/unit_NNNNN.mtt, after waiting for queued host updates.  The
 * directory is created if missing; files are written under a temporary name
 * and renamed.  Errors: MT_E_INVAL, MT_E_IO, MT_E_STATE. */
int mt_checkpoint_save(mt_ctx* ctx, const char* dir);

/* Restore a context of the same shape from mt_checkpoint_save's files: every
 * header is checked (format, unit, shape, size, one step count for all) before
 * anything is read, then the tiles are loaded now (lazy = 0) or each when the
 * step first needs it (lazy = 1: the embedding before the gather, a layer or
 * the head before it is streamed, any unit before mt_get/set_tensor).  The
 * step count continues from the saved one.  A checksum mismatch found while
 * loading fails the context (MT_E_IO, then MT_E_STATE).  Errors: MT_E_INVAL
 * (NULL, other shape), MT_E_IO. */
int mt_checkpoint_restore(mt_ctx* ctx, const char* dir, int32_t lazy);

/* sizeof the ABI structs as this library was built, for bindings to check
 * their mirrors: which 0 mt_shape, 1 mt_options, 2 mt_stats,
 * 3 mt_tensor_info; -1 for another value. */
int64_t mt_abi_sizeof(int32_t which);

/* Name of a kernel timing site of mt_stats (NULL if out of range). */
const char* mt_site_name(int32_t site);

/* Join the host threads and free everything the library owns. */
void mt_destroy(mt_ctx* ctx);

const char* mt_strerror(int status);
const char* mt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MT_H */
