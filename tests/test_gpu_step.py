"""Layer- and step-level parity of the streamed GPU path against the oracle,
plus bit-identity of results across streaming configurations.

Weights come from the library's own seeded init and are read back through
mt_get_tensor, so the oracle computes on exactly the values the GPU used.
Bound: normwise relative error <= 1e-2 per tensor (loss, dx, every gradient).
"""
import numpy as np
import pytest

from layer_streaming_amd import synth
from oracle import step as ostep
from oracle.bf16 import round_bf16
from tests.gpu_util import TOL, assert_close, dev_bits, dev_zeros_bits, host_f32, log, widen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from layer_streaming_amd import mt  # noqa: E402

CFG1 = dict(n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64, ffn_dim=688, vocab=1024)
GQA = dict(n_layers=2, d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=688, vocab=1024)
HD128 = dict(n_layers=1, d_model=256, n_heads=2, n_kv_heads=1, head_dim=128, ffn_dim=512, vocab=512)


def make_ctx(shape_kw, max_batch, max_seq, **opts):
    sh = mt.make_shape(**shape_kw)
    opts.setdefault("host_threads", 8)
    o = mt.default_options(max_batch=max_batch, max_seq=max_seq, **opts)
    arena_bytes, _, _ = mt.workspace_bytes(sh, o)
    arena = torch.empty(arena_bytes, dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    ctx = mt.Context(sh, o, arena.data_ptr(), arena_bytes, [s.cuda_stream for s in streams])
    ctx._keep = (arena, streams)
    return ctx


def oracle_shape(kw):
    return ostep.Shape(**kw)


def read_params(ctx, kw):
    L = kw["n_layers"]
    layers = []
    for i in range(L):
        layers.append({n: widen(ctx.get_tensor(i, j, mt.MT_W)).astype(np.float64)
                       for j, n in enumerate(ostep.LAYER_TENSORS)})
    head = {n: widen(ctx.get_tensor(L, j, mt.MT_W)).astype(np.float64) for j, n in enumerate(ostep.HEAD_TENSORS)}
    return {"layers": layers, "head": head, "e_in": widen(ctx.get_tensor(L + 1, 0, mt.MT_W)).astype(np.float64)}


def read_all(ctx, kw, which):
    L = kw["n_layers"]
    out = []
    for u in range(L + 2):
        n = 9 if u < L else (2 if u == L else 1)
        for j in range(n):
            out.append(((u, j), ctx.get_tensor(u, j, which).copy()))
    return out


# ----------------------------------------------------------- layer level --
@pytest.mark.parametrize("kw,B,S", [(GQA, 2, 72), (HD128, 1, 130), (CFG1, 1, 1)])
def test_layer_fwd_bwd_parity(kw, B, S):
    log(f"layer fwd/bwd {kw} B={B} S={S}")
    ctx = make_ctx(kw, B, S)
    sh = oracle_shape(kw)
    T, d = B * S, kw["d_model"]
    rng = np.random.default_rng(99)
    x = synth.bf16_exact_normal(rng, (T, d))
    dy = synth.bf16_exact_normal(rng, (T, d), std=0.1)
    dx_, dy_ = dev_bits(x), dev_bits(dy)
    y_, dxo = dev_zeros_bits((T, d)), dev_zeros_bits((T, d))
    gtile = dev_zeros_bits((mt.unit_elems(ctx.shape, 0),))
    ctx.layer_fwd(0, dx_.data_ptr(), y_.data_ptr(), B, S)
    ctx.layer_bwd(0, dx_.data_ptr(), dy_.data_ptr(), dxo.data_ptr(), gtile.data_ptr(), B, S)
    torch.cuda.synchronize()
    w = read_params(ctx, kw)["layers"][0]
    y_ref, cache = ostep.layer_fwd(x.astype(np.float64), w, sh, B, S)
    assert_close(host_f32(y_), y_ref, "y")
    dx_ref, g_ref = ostep.layer_bwd(dy.astype(np.float64), cache, w, sh, B, S)
    assert_close(host_f32(dxo), dx_ref, "dx")
    gt = host_f32(gtile)
    for j, n in enumerate(ostep.LAYER_TENSORS):
        info = mt.tensor_desc(ctx.shape, 0, j)
        sl = gt[info["offset"]: info["offset"] + info["rows"] * info["cols"]].reshape(g_ref[n].shape)
        assert_close(sl, g_ref[n], f"d{n}")
    ctx.close()


# ------------------------------------------------------------ full step --
# Gradients are compared per tensor (every gradient of every unit, the input
# embedding's included) and per streamed unit (a layer's, the head's and the
# embedding's whole BF16 gradient tile, the granularity gradients leave the
# GPU in), all at normwise relative error <= 1e-2.
def _cmp_units(ctx, kw, g_ref):
    L = kw["n_layers"]
    units = [(i, ostep.LAYER_TENSORS, g_ref["layers"][i], f"L{i}") for i in range(L)]
    units += [(L, ostep.HEAD_TENSORS, g_ref["head"], "head"), (L + 1, ("e_in",), {"e_in": g_ref["e_in"]}, "emb")]
    worst = (0.0, "")
    for u, names, ref, tag in units:
        got_all, ref_all = [], []
        for j, n in enumerate(names):
            got = widen(ctx.get_tensor(u, j, mt.MT_G))
            e = assert_close(got, ref[n], f"{tag}.d{n}")
            worst = max(worst, (e, f"{tag}.d{n}"))
            got_all.append(got.reshape(-1))
            ref_all.append(np.asarray(ref[n]).reshape(-1))
        assert_close(np.concatenate(got_all), np.concatenate(ref_all), f"{tag} gradient tile")
    log(f"  worst gradient tensor: {worst[1]} {worst[0]:.3e}")
    return worst[0]


@pytest.mark.parametrize("kw,B,S", [(CFG1, 2, 128), (GQA, 3, 40), (HD128, 2, 100), (HD128, 1, 1)])
def test_train_step_parity(kw, B, S):
    log(f"train step {kw} B={B} S={S}")
    ctx = make_ctx(kw, B, S)
    sh = oracle_shape(kw)
    tokens, labels = synth.tokens_labels(synth.SEED_TOKENS, B, S, kw["vocab"])
    params = read_params(ctx, kw)
    masters0 = read_all(ctx, kw, mt.MT_MASTER)
    loss, st = ctx.train_step(tokens, labels)
    log(f"  loss gpu {loss:.6f}  step {st.step_ms:.1f} ms")
    loss_ref, g_ref = ostep.grads_monolithic(params, tokens, labels, sh)
    assert abs(loss - loss_ref) / abs(loss_ref) <= 1e-2, (loss, loss_ref)
    _cmp_units(ctx, kw, g_ref)
    # The host Adam consumed exactly the gradients the store now holds.
    for (u, j), m0 in masters0:
        g = widen(ctx.get_tensor(u, j, mt.MT_G))
        z = np.zeros_like(m0)
        mst, m, v, w = ostep.adam_update(m0, z, z, g, 1, 1e-4, 0.9, 0.999, 1e-8)
        got = ctx.get_tensor(u, j, mt.MT_MASTER)
        ulp = np.spacing(np.abs(mst)).astype(np.float64)
        err = np.abs(got.astype(np.float64) - mst.astype(np.float64))
        assert np.all(err <= np.maximum(2 * ulp, 1e-10)), (u, j, float(err.max()))
        np.testing.assert_allclose(ctx.get_tensor(u, j, mt.MT_M), m, rtol=1e-6, atol=1e-30)
        np.testing.assert_allclose(ctx.get_tensor(u, j, mt.MT_V), v, rtol=1e-6, atol=1e-30)
        assert np.array_equal(widen(ctx.get_tensor(u, j, mt.MT_W)), round_bf16(got))
    assert ctx.step_count() == 1
    ctx.close()


def test_multi_chunk_head_parity():
    """LM head over several token chunks (fp32 accumulation of dE_out)."""
    kw, B, S = CFG1, 2, 128
    log("multi-chunk head")
    ctx = make_ctx(kw, B, S, head_chunk=48)
    tokens, labels = synth.tokens_labels(7, B, S, kw["vocab"])
    params = read_params(ctx, kw)
    loss, _ = ctx.train_step(tokens, labels)
    loss_ref, g_ref = ostep.grads_monolithic(params, tokens, labels, oracle_shape(kw))
    assert abs(loss - loss_ref) / abs(loss_ref) <= 1e-2
    L = kw["n_layers"]
    assert_close(widen(ctx.get_tensor(L, 1, mt.MT_G)), g_ref["head"]["e_out"], "head.de_out")
    _cmp_units(ctx, kw, g_ref)
    ctx.close()


# ------------------------------------------- the benchmarked option set --
# The options the benchmark runs with: cross-step pipelining, the weight
# regions in one page-locked block, the LM head in layer-sized E_out chunks,
# 16 gradient slabs, per-kernel timing, every host thread, Adam reading the
# slabs without a copy into the store's G.  Three layers and a vocabulary of
# 8192 give three head chunks; three steps with distinct tokens run the split
# update of the input embedding twice.
BENCH_OPTS = dict(cross_step=1, pin_weights=1, head_vocab_chunk=-1, n_grad_slabs=16, profile_kernels=1,
                  host_threads=0, keep_grads=0)
BENCHLIKE = dict(n_layers=3, d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=688, vocab=8192)


def _oracle_store(ctx, kw):
    """The context's whole state in the oracle's store layout (float32 W
    values, master, m, v per tensor)."""
    L = kw["n_layers"]

    def unit(u, names):
        return {n: {"w": widen(ctx.get_tensor(u, j, mt.MT_W)), "master": ctx.get_tensor(u, j, mt.MT_MASTER).copy(),
                    "m": ctx.get_tensor(u, j, mt.MT_M).copy(), "v": ctx.get_tensor(u, j, mt.MT_V).copy()}
                for j, n in enumerate(names)}
    return {"layers": [unit(i, ostep.LAYER_TENSORS) for i in range(L)], "head": unit(L, ostep.HEAD_TENSORS),
            "e_in": unit(L + 1, ("e_in",))}


def _units(kw):
    L = kw["n_layers"]
    return ([(i, ostep.LAYER_TENSORS, lambda t, i=i: t["layers"][i], f"L{i}") for i in range(L)] +
            [(L, ostep.HEAD_TENSORS, lambda t: t["head"], "head"), (L + 1, ("e_in",), lambda t: t["e_in"], "emb")])


@pytest.mark.parametrize("opts", [BENCH_OPTS, dict(BENCH_OPTS, keep_grads=1)], ids=["bench", "bench,keep-grads"])
def test_bench_option_set_three_steps_against_oracle(opts):
    """Three steps with the benchmark's options, nothing read between them,
    against three steps of the oracle's streamed training (its gradients
    rounded to BF16, its Adam at t = 1, 2, 3) from the same initial state:
    the loss of every step, the Adam moments m and sqrt(v) (sqrt(v) has the
    gradient's units) per tensor within 1e-2, and, where the store keeps
    them, the last step's gradients.  Without them m still carries the last
    gradient at weight 0.1 against 0.081 and 0.09 for the two before, so a
    wrong last gradient shows in m."""
    kw, B, S = BENCHLIKE, 2, 64
    keep = opts.get("keep_grads", 1) == 1
    log(f"bench option set, 3 steps, vs the oracle's 3-step training {kw} {opts}")
    ctx = make_ctx(kw, B, S, **opts)
    store = _oracle_store(ctx, kw)
    batches = [synth.tokens_labels(700 + k, B, S, kw["vocab"]) for k in range(3)]
    losses = [ctx.train_step(t, lb)[0] for t, lb in batches]
    ctx.sync()
    assert ctx.step_count() == 3
    sh = oracle_shape(kw)
    for k, (t, lb) in enumerate(batches):
        loss_ref, g_ref = ostep.train_step(store, t, lb, sh, k + 1)
        log(f"  step {k + 1}: loss gpu {losses[k]:.6f} oracle {loss_ref:.6f}")
        assert abs(losses[k] - loss_ref) <= 1e-2 * abs(loss_ref)
    worst = 0.0
    for u, names, pick, tag in _units(kw):
        for j, n in enumerate(names):
            ref = pick(store)[n]
            if keep:
                worst = max(worst, assert_close(widen(ctx.get_tensor(u, j, mt.MT_G)), pick(g_ref)[n], f"{tag}.d{n}"))
            assert_close(ctx.get_tensor(u, j, mt.MT_M), ref["m"], f"{tag}.m({n})")
            assert_close(np.sqrt(ctx.get_tensor(u, j, mt.MT_V).astype(np.float64)),
                         np.sqrt(ref["v"].astype(np.float64)), f"{tag}.sqrt_v({n})")
    if keep:
        log(f"  worst step-3 gradient tensor {worst:.3e}")
    else:
        with pytest.raises(mt.MTError, match="not kept"):
            ctx.get_tensor(0, 0, mt.MT_G)
    ctx.close()


def _run_steps(kw, B, S, n, stats_out=None, with_g=True, **opts):
    ctx = make_ctx(kw, B, S, **opts)
    losses = []
    for k in range(n):
        tokens, labels = synth.tokens_labels(700 + k, B, S, kw["vocab"])
        loss, st = ctx.train_step(tokens, labels)
        losses.append(loss)
        if stats_out is not None:
            stats_out.append(st)
    # with_g=False: compared without G (a store that does not keep gradients)
    whiches = (mt.MT_W, mt.MT_G, mt.MT_MASTER, mt.MT_M, mt.MT_V) if with_g else \
        (mt.MT_W, mt.MT_MASTER, mt.MT_M, mt.MT_V)
    state = [(key, which, a) for which in whiches for key, a in read_all(ctx, kw, which)]
    ctx.close()
    return losses, state


@pytest.mark.parametrize("opts", [BENCH_OPTS, dict(BENCH_OPTS, pin_weights=0, n_grad_slabs=12, keep_grads=1)],
                         ids=["bench", "pages-pinned-footprint"])
def test_bench_option_set_bit_identical_to_synchronous_path(opts):
    """The benchmark's option set (and the pages' pinned footprint: two
    staging buffers and 12 slabs) against the plain synchronous streamed
    path with the same chunked head, over three steps: losses and the whole
    store (W, master, m, v, and G where the option set keeps it) bit for bit."""
    kw, B, S = BENCHLIKE, 2, 64
    log(f"bench option set vs synchronous path: {opts}")
    with_g = opts.get("keep_grads", 1) == 1
    base_losses, base_state = _run_steps(kw, B, S, 3, with_g=with_g, head_vocab_chunk=-1)
    losses, state = _run_steps(kw, B, S, 3, with_g=with_g, **opts)
    assert [np.float32(x).tobytes() for x in losses] == [np.float32(x).tobytes() for x in base_losses]
    for (k1, w1, a1), (k2, w2, a2) in zip(base_state, state):
        assert k1 == k2 and w1 == w2
        assert np.array_equal(a1.view(np.uint8), a2.view(np.uint8)), (k1, w1)


# ------------------------------------------------------- bit identity ----
VARIANTS = [dict(resident=1), dict(n_weight_slots=1), dict(n_weight_slots=3), dict(n_grad_slabs=1),
            dict(slot_mode=1), dict(ckpt_on_host=0), dict(host_threads=3), dict(pin_store=1),
            dict(cross_step=1), dict(cross_step=1, n_grad_slabs=1), dict(cross_step=1, resident=1),
            dict(pin_weights=1), dict(pin_weights=1, cross_step=1), dict(ckpt_attn=1),
            dict(ckpt_attn=1, cross_step=1, pin_weights=1), dict(ckpt_attn=1, resident=1, n_grad_slabs=1)]


def _run_two_steps(kw, B, S, **opts):
    ctx = make_ctx(kw, B, S, **opts)
    losses = []
    for k in range(2):
        tokens, labels = synth.tokens_labels(100 + k, B, S, kw["vocab"])
        losses.append(ctx.train_step(tokens, labels)[0])
    state = [(key, which, a) for which in (mt.MT_W, mt.MT_G, mt.MT_MASTER, mt.MT_M, mt.MT_V)
             for key, a in read_all(ctx, kw, which)]
    ctx.close()
    return losses, state


@pytest.fixture(scope="module")
def baseline_run():
    return _run_two_steps(GQA, 2, 64)


@pytest.mark.parametrize("opts", VARIANTS, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_streamed_configurations_bit_identical(baseline_run, opts):
    log(f"bit identity vs default streaming: {opts}")
    base_losses, base_state = baseline_run
    losses, state = _run_two_steps(GQA, 2, 64, **opts)
    assert [np.float32(x).tobytes() for x in losses] == [np.float32(x).tobytes() for x in base_losses]
    for (k1, w1, a1), (k2, w2, a2) in zip(base_state, state):
        assert k1 == k2 and w1 == w2
        assert np.array_equal(a1.view(np.uint8), a2.view(np.uint8)), (k1, w1)


DEEP = dict(n_layers=5, d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=688, vocab=1024)


@pytest.fixture(scope="module")
def deep_baseline_run():
    return _run_two_steps(DEEP, 2, 64)


@pytest.mark.parametrize("opts", [dict(ckpt_interval=2), dict(ckpt_interval=3), dict(ckpt_interval=5),
                                  dict(ckpt_interval=7), dict(ckpt_interval=2, n_weight_slots=1),
                                  dict(ckpt_interval=3, cross_step=1), dict(ckpt_attn=1),
                                  dict(ckpt_attn=1, n_weight_slots=1, slot_mode=1)],
                         ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_checkpoint_interval_bit_identical(deep_baseline_run, opts):
    """Block-wise recomputation (every k-th layer input kept, the block's
    other inputs rebuilt by re-running its forward) changes where the inputs
    come from, not their values: 5 layers in blocks of 2, 3, 5 and 7 (capped
    at the depth) give the per-layer-checkpoint results bit for bit; so does
    checkpointing each layer's attention output and log-sum-exp as well, so
    that the recompute skips the attention forward."""
    log(f"checkpoint interval vs every layer: {opts}")
    base_losses, base_state = deep_baseline_run
    losses, state = _run_two_steps(DEEP, 2, 64, **opts)
    assert [np.float32(x).tobytes() for x in losses] == [np.float32(x).tobytes() for x in base_losses]
    for (k1, w1, a1), (k2, w2, a2) in zip(base_state, state):
        assert k1 == k2 and w1 == w2
        assert np.array_equal(a1.view(np.uint8), a2.view(np.uint8)), (k1, w1)


@pytest.mark.parametrize("k", [2, 3])
def test_checkpoint_interval_step_parity(k):
    """Block-wise recomputation against the oracle: 5 layers in blocks of k
    (the block's first input kept, the others rebuilt in the backward), the
    loss and every gradient tensor within 1e-2 of the plain definition."""
    kw, B, S = DEEP, 2, 64
    log(f"checkpoint interval {k} vs the oracle")
    ctx = make_ctx(kw, B, S, ckpt_interval=k)
    tokens, labels = synth.tokens_labels(23, B, S, kw["vocab"])
    params = read_params(ctx, kw)
    loss, _ = ctx.train_step(tokens, labels)
    loss_ref, g_ref = ostep.grads_monolithic(params, tokens, labels, oracle_shape(kw))
    assert abs(loss - loss_ref) / abs(loss_ref) <= 1e-2, (loss, loss_ref)
    _cmp_units(ctx, kw, g_ref)
    ctx.close()


# ------------------------------------------- vocabulary-chunked head ----
BIGV = dict(n_layers=2, d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=688, vocab=8192)


@pytest.mark.parametrize("kw,B,S,opts", [(CFG1, 2, 128, dict(head_vocab_chunk=256)),
                                         (CFG1, 2, 128, dict(head_vocab_chunk=264, head_chunk=48)),
                                         (BIGV, 1, 96, dict(head_vocab_chunk=-1))],
                         ids=["4chunks", "ragged+tokenchunks", "auto"])
def test_vocab_chunked_head_step_parity(kw, B, S, opts):
    """The head streamed in E_out row chunks (online logsumexp over a forward
    pass, logits recomputed in a reverse backward pass, each chunk's gradient
    offloaded and updated on its own) against the oracle: loss, every
    gradient and the Adam update of the head."""
    log(f"vocab-chunked head {kw['vocab']} {opts}")
    ctx = make_ctx(kw, B, S, **opts)
    tokens, labels = synth.tokens_labels(17, B, S, kw["vocab"])
    params = read_params(ctx, kw)
    masters0 = read_all(ctx, kw, mt.MT_MASTER)
    loss, _ = ctx.train_step(tokens, labels)
    loss_ref, g_ref = ostep.grads_monolithic(params, tokens, labels, oracle_shape(kw))
    assert abs(loss - loss_ref) / abs(loss_ref) <= 1e-2, (loss, loss_ref)
    _cmp_units(ctx, kw, g_ref)
    L = kw["n_layers"]
    for (u, j), m0 in masters0:
        if u != L:
            continue
        g = widen(ctx.get_tensor(u, j, mt.MT_G))
        z = np.zeros_like(m0)
        mst, _, _, _ = ostep.adam_update(m0, z, z, g, 1, 1e-4, 0.9, 0.999, 1e-8)
        got = ctx.get_tensor(u, j, mt.MT_MASTER)
        err = np.abs(got.astype(np.float64) - mst.astype(np.float64))
        assert np.all(err <= np.maximum(2 * np.spacing(np.abs(mst)).astype(np.float64), 1e-10)), (u, j)
    ctx.close()


def test_vocab_chunked_head_slots_sized_to_the_layer():
    """With automatic chunking the weight slots (and so the arena) hold the
    largest decoder layer, not the head."""
    sh = mt.make_shape(**BIGV)
    whole = mt.workspace_bytes(sh, mt.default_options(max_batch=1, max_seq=96))
    chunked = mt.workspace_bytes(sh, mt.default_options(max_batch=1, max_seq=96, head_vocab_chunk=-1))
    assert chunked[1] < whole[1]  # pinned: staging and slabs are slot-sized


@pytest.fixture(scope="module")
def chunked_baseline_run():
    return _run_two_steps(BIGV, 1, 64, head_vocab_chunk=-1)


@pytest.mark.parametrize("opts", [dict(resident=1), dict(n_weight_slots=1), dict(n_weight_slots=3),
                                  dict(slot_mode=1), dict(cross_step=1, n_grad_slabs=1), dict(pin_weights=1),
                                  dict(ckpt_interval=2)],
                         ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_vocab_chunked_head_bit_identical_across_streaming_options(chunked_baseline_run, opts):
    log(f"chunked head vs default streaming: {opts}")
    base_losses, base_state = chunked_baseline_run
    losses, state = _run_two_steps(BIGV, 1, 64, head_vocab_chunk=-1, **opts)
    assert [np.float32(x).tobytes() for x in losses] == [np.float32(x).tobytes() for x in base_losses]
    for (k1, w1, a1), (k2, w2, a2) in zip(base_state, state):
        assert k1 == k2 and w1 == w2
        assert np.array_equal(a1.view(np.uint8), a2.view(np.uint8)), (k1, w1)


def test_vocab_chunked_head_with_micro_batches():
    """Chunked head under gradient accumulation: two identical micro-batches
    give the one-micro-batch step bit for bit."""
    kw, B, S = BIGV, 1, 64
    base_losses, base_state = _run_two_steps(kw, B, S, head_vocab_chunk=-1)
    ctx = make_ctx(kw, B, S, head_vocab_chunk=-1)
    losses = []
    for k in range(2):
        t, lb = synth.tokens_labels(100 + k, B, S, kw["vocab"])
        losses.append(ctx.train_step_accum(np.stack([t] * 2), np.stack([lb] * 2))[0])
    state = _state(ctx, kw)
    ctx.close()
    assert [np.float32(x).tobytes() for x in losses] == [np.float32(x).tobytes() for x in base_losses]
    for (k1, w1, a1), (k2, w2, a2) in zip(base_state, state):
        assert np.array_equal(a1.view(np.uint8), a2.view(np.uint8)), (k1, w1)


# -------------------------------------------- gradient accumulation ----
def _micro_batches(kw, n, B, S, seed0):
    tl = [synth.tokens_labels(seed0 + j, B, S, kw["vocab"]) for j in range(n)]
    return np.stack([t for t, _ in tl]), np.stack([lb for _, lb in tl])


@pytest.mark.parametrize("opts", [dict(), dict(head_vocab_chunk=256, ckpt_interval=2, cross_step=1, n_grad_slabs=3),
                                  dict(ckpt_attn=1, cross_step=1),
                                  dict(pin_weights=1, n_weight_slots=3, head_vocab_chunk=-1)],
                         ids=["default", "chunked-head,interval2,cross-step", "attn-ckpt,cross-step", "pinned,3slots"])
def test_poisoned_released_buffers_change_nothing(opts):
    """Race check of the streaming protocol: with poison_released every
    weight slot is filled with NaN when its last visit releases it, and every
    gradient area once its copy to a slab is done.  Three steps must give
    bit-identical losses and state to the same run without poisoning: no
    kernel reads a released slot or gradient area, and every visit writes
    its whole gradient area."""
    log(f"poisoned release vs plain: {opts}")
    st0, st1 = [], []
    base_losses, base_state = _run_steps(DEEP, 2, 48, 3, stats_out=st0, **opts)
    losses, state = _run_steps(DEEP, 2, 48, 3, stats_out=st1, poison_released=1, **opts)
    assert all(np.isfinite(losses))
    # the poison is live: a released slot is never reused, so a unit whose
    # slot the next visit could have reused is streamed again
    h0, h1 = st0[-1].h2d_bytes, st1[-1].h2d_bytes
    log(f"  h2d bytes per step: plain {h0}, poisoned {h1}")
    assert h1 > h0
    assert [np.float32(x).tobytes() for x in losses] == [np.float32(x).tobytes() for x in base_losses]
    for (k1, w1, a1), (k2, w2, a2) in zip(base_state, state):
        assert k1 == k2 and w1 == w2
        assert np.array_equal(a1.view(np.uint8), a2.view(np.uint8)), (k1, w1)


def test_accumulated_step_parity():
    """Three micro-batches, one optimizer step, against the oracle: the loss
    over every token, the accumulated gradients, and Adam run once on them."""
    kw, B, S, n = CFG1, 1, 96, 3
    log(f"accumulated step {n} x B={B} S={S}")
    ctx = make_ctx(kw, B, S)
    tokens, labels = _micro_batches(kw, n, B, S, 300)
    params = read_params(ctx, kw)
    masters0 = read_all(ctx, kw, mt.MT_MASTER)
    loss, st = ctx.train_step_accum(tokens, labels)
    log(f"  loss gpu {loss:.6f}  step {st.step_ms:.1f} ms")
    loss_ref, g_ref = ostep.grads_accumulated(params, tokens, labels, oracle_shape(kw))
    assert abs(loss - loss_ref) / abs(loss_ref) <= 1e-2, (loss, loss_ref)
    _cmp_units(ctx, kw, g_ref)
    for (u, j), m0 in masters0:
        g = widen(ctx.get_tensor(u, j, mt.MT_G))
        z = np.zeros_like(m0)
        mst, m, v, w = ostep.adam_update(m0, z, z, g, 1, 1e-4, 0.9, 0.999, 1e-8)
        got = ctx.get_tensor(u, j, mt.MT_MASTER)
        err = np.abs(got.astype(np.float64) - mst.astype(np.float64))
        assert np.all(err <= np.maximum(2 * np.spacing(np.abs(mst)).astype(np.float64), 1e-10)), (u, j)
        np.testing.assert_allclose(ctx.get_tensor(u, j, mt.MT_M), m, rtol=1e-6, atol=1e-30)
    assert ctx.step_count() == 1
    ctx.close()


def test_accumulation_is_the_bf16_sum_of_separate_micro_batch_gradients():
    """Two micro-batches give, bit for bit, the one-rounding BF16 sum of half
    the gradients two fresh contexts compute for each micro-batch alone (the
    loss scale 1/(2T) is exactly half of 1/T, and every gradient is linear in
    it), which pins the host accumulation of every unit, the input embedding
    included."""
    kw, B, S = GQA, 2, 48
    log("accumulation vs separate micro-batch gradients")
    tokens, labels = _micro_batches(kw, 2, B, S, 400)
    sep = []
    for j in range(2):
        c = make_ctx(kw, B, S)
        c.train_step(tokens[j], labels[j])
        sep.append([a for _, a in read_all(c, kw, mt.MT_G)])
        c.close()
    ctx = make_ctx(kw, B, S)
    ctx.train_step_accum(tokens, labels)
    got = read_all(ctx, kw, mt.MT_G)
    ctx.close()
    for (key, g), g0, g1 in zip(got, sep[0], sep[1]):
        want = ostep.accumulate_bf16(widen(g0) * 0.5, widen(g1) * 0.5)
        assert np.array_equal(widen(g), want), key


def test_identical_micro_batches_equal_one_micro_batch_bit_for_bit():
    kw, B, S = GQA, 2, 64
    log("n identical micro-batches vs one")
    base_losses, base_state = _run_two_steps(kw, B, S)
    for n in (2, 4):
        ctx = make_ctx(kw, B, S)
        losses = []
        for k in range(2):
            t, lb = synth.tokens_labels(100 + k, B, S, kw["vocab"])
            losses.append(ctx.train_step_accum(np.stack([t] * n), np.stack([lb] * n))[0])
        state = _state(ctx, kw)
        ctx.close()
        assert [np.float32(x).tobytes() for x in losses] == [np.float32(x).tobytes() for x in base_losses]
        for (k1, w1, a1), (k2, w2, a2) in zip(base_state, state):
            assert np.array_equal(a1.view(np.uint8), a2.view(np.uint8)), (n, k1, w1)


def _run_two_accum_steps(kw, B, S, n, **opts):
    ctx = make_ctx(kw, B, S, **opts)
    losses = []
    for k in range(2):
        t, lb = _micro_batches(kw, n, B, S, 500 + 10 * k)
        losses.append(ctx.train_step_accum(t, lb)[0])
    state = _state(ctx, kw)
    ctx.close()
    return losses, state


@pytest.fixture(scope="module")
def accum_baseline_run():
    return _run_two_accum_steps(DEEP, 1, 64, 3)


@pytest.mark.parametrize("opts", [dict(cross_step=1), dict(n_grad_slabs=1), dict(n_weight_slots=1),
                                  dict(ckpt_interval=2), dict(resident=1), dict(slot_mode=1),
                                  dict(cross_step=1, n_grad_slabs=1, ckpt_interval=3), dict(ckpt_attn=1)],
                         ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()))
def test_accumulated_steps_bit_identical_across_streaming_options(accum_baseline_run, opts):
    log(f"accumulated steps vs default streaming: {opts}")
    base_losses, base_state = accum_baseline_run
    losses, state = _run_two_accum_steps(DEEP, 1, 64, 3, **opts)
    assert [np.float32(x).tobytes() for x in losses] == [np.float32(x).tobytes() for x in base_losses]
    for (k1, w1, a1), (k2, w2, a2) in zip(base_state, state):
        assert k1 == k2 and w1 == w2
        assert np.array_equal(a1.view(np.uint8), a2.view(np.uint8)), (k1, w1)


def test_bad_micro_batch_count_rejected():
    kw, B, S = CFG1, 1, 16
    ctx = make_ctx(kw, B, S)
    t, lb = synth.tokens_labels(1, B, S, kw["vocab"])
    for n in (0, mt.MT_MAX_MICRO + 1):
        r = mt.lib.mt_train_step_accum(ctx._ptr, t.ctypes.data_as(mt.C.POINTER(mt.C.c_int32)),
                                       lb.ctypes.data_as(mt.C.POINTER(mt.C.c_int32)), n, B, S,
                                       mt.C.byref(mt.C.c_float()), None)
        assert r == mt.MT_E_INVAL
    assert ctx.step_count() == 0
    ctx.train_step(t, lb)  # the context is still usable
    ctx.close()


# ----------------------------------------------------- checkpoint shards --
def _state(ctx, kw):
    return [(key, which, a) for which in (mt.MT_W, mt.MT_G, mt.MT_MASTER, mt.MT_M, mt.MT_V)
            for key, a in read_all(ctx, kw, which)]


@pytest.mark.parametrize("lazy", [False, True], ids=["eager", "lazy"])
def test_checkpoint_shards_resume_bit_identical(tmp_path, lazy):
    """Save after step 1, restore into a context initialised from another
    seed, run step 2: the same loss and the same state, bit for bit, as the
    run that never stopped."""
    kw, B, S = DEEP, 2, 64
    t1 = synth.tokens_labels(100, B, S, kw["vocab"])
    t2 = synth.tokens_labels(101, B, S, kw["vocab"])
    a = make_ctx(kw, B, S)
    a.train_step(*t1)
    a.checkpoint_save(str(tmp_path / "ck"))
    loss_a, _ = a.train_step(*t2)
    state_a = _state(a, kw)
    a.close()
    b = make_ctx(kw, B, S, seed=999)
    b.checkpoint_restore(str(tmp_path / "ck"), lazy=lazy)
    assert b.step_count() == 1
    loss_b, _ = b.train_step(*t2)
    assert np.float32(loss_a).tobytes() == np.float32(loss_b).tobytes()
    for (k1, w1, x1), (k2, w2, x2) in zip(state_a, _state(b, kw)):
        assert k1 == k2 and w1 == w2
        assert np.array_equal(x1.view(np.uint8), x2.view(np.uint8)), (k1, w1)
    b.close()


def test_checkpoint_restore_errors(tmp_path):
    kw, B, S = CFG1, 1, 16
    tok = synth.tokens_labels(3, B, S, kw["vocab"])
    a = make_ctx(kw, B, S)
    a.train_step(*tok)
    ck = tmp_path / "ck"
    a.checkpoint_save(str(ck))
    # another model shape: rejected before anything is read, context usable
    other = make_ctx(GQA, B, S)
    with pytest.raises(mt.MTError) as e:
        other.checkpoint_restore(str(ck))
    assert e.value.status == mt.MT_E_INVAL
    other.train_step(*tok)
    other.close()
    # a missing shard: rejected up front, context usable
    with pytest.raises(mt.MTError) as e:
        a.checkpoint_restore(str(tmp_path / "nothing"))
    assert e.value.status == mt.MT_E_IO
    a.train_step(*tok)
    # a flipped byte in layer 1's master region: found by the checksum when
    # the shard is loaded; the context is then failed
    p = ck / "unit_00001.mtt"
    raw = bytearray(p.read_bytes())
    raw[256 + len(raw) // 2] ^= 0x40
    p.write_bytes(bytes(raw))
    with pytest.raises(mt.MTError) as e:
        a.checkpoint_restore(str(ck))
    assert e.value.status == mt.MT_E_IO
    with pytest.raises(mt.MTError) as e:
        a.train_step(*tok)
    assert e.value.status == mt.MT_E_STATE
    a.close()
    # lazily: the same corruption surfaces at the step that first needs layer 1
    c = make_ctx(kw, B, S)
    c.checkpoint_restore(str(ck), lazy=True)
    with pytest.raises(mt.MTError) as e:
        c.train_step(*tok)
    assert e.value.status == mt.MT_E_IO
    c.close()


def test_loss_decreases_over_steps_on_fixed_batch():
    log("loss decreases on a repeated batch")
    kw = CFG1
    ctx = make_ctx(kw, 2, 64, )
    tokens, labels = synth.tokens_labels(5, 2, 64, kw["vocab"])
    losses = [ctx.train_step(tokens, labels)[0] for _ in range(4)]
    log(f"  losses {losses}")
    assert losses[-1] < losses[0]
    ctx.close()


# ------------------------------------------------------------ errors ------
def test_invalid_tokens_rejected_before_device_work():
    ctx = make_ctx(CFG1, 1, 16)
    tokens, labels = synth.tokens_labels(1, 1, 16, 1024)
    tokens[0, 3] = 1024
    with pytest.raises(mt.MTError) as e:
        ctx.train_step(tokens, labels)
    assert e.value.status == mt.MT_E_INVAL
    # the context is still usable
    tokens[0, 3] = 5
    loss, _ = ctx.train_step(tokens, labels)
    assert np.isfinite(loss)
    with pytest.raises(mt.MTError) as e:
        ctx.train_step(np.zeros((2, 16), np.int32), np.zeros((2, 16), np.int32))
    assert e.value.status == mt.MT_E_INVAL
    ctx.close()


def test_arena_too_small_is_nomem():
    sh = mt.make_shape(**CFG1)
    o = mt.default_options(max_batch=1, max_seq=16)
    need, _, _ = mt.workspace_bytes(sh, o)
    arena = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(mt.MTError) as e:
        mt.Context(sh, o, arena.data_ptr(), need - 4096)
    assert e.value.status == mt.MT_E_NOMEM


def test_injected_slab_worker_fault_is_reported(monkeypatch):
    """A host worker failure (forced from the host) ends the step with an
    error, joins cleanly and marks the context failed."""
    monkeypatch.setenv("MT_FAULT", "slab:1")
    ctx = make_ctx(CFG1, 1, 16)
    tokens, labels = synth.tokens_labels(1, 1, 16, 1024)
    with pytest.raises(mt.MTError) as e:
        ctx.train_step(tokens, labels)
    assert e.value.status == mt.MT_E_INTERNAL
    with pytest.raises(mt.MTError) as e:
        ctx.train_step(tokens, labels)
    assert e.value.status == mt.MT_E_STATE
    ctx.close()


def test_injected_slab_worker_fault_with_cross_step(monkeypatch):
    """With cross_step the failing update may land after mt_train_step has
    returned: then mt_sync reports it; either way the context is failed."""
    monkeypatch.setenv("MT_FAULT", "slab:1")
    ctx = make_ctx(CFG1, 1, 16, cross_step=1)
    tokens, labels = synth.tokens_labels(1, 1, 16, 1024)
    statuses = []
    for call in (lambda: ctx.train_step(tokens, labels), ctx.sync):
        try:
            call()
            statuses.append(mt.MT_OK)
        except mt.MTError as e:
            statuses.append(e.status)
    log(f"  statuses {statuses}")
    assert mt.MT_E_INTERNAL in statuses
    with pytest.raises(mt.MTError) as e:
        ctx.train_step(tokens, labels)
    assert e.value.status == mt.MT_E_STATE
    ctx.close()


def test_injected_pack_fault_is_reported(monkeypatch):
    monkeypatch.setenv("MT_FAULT", "pack:0")
    ctx = make_ctx(CFG1, 1, 16)
    tokens, labels = synth.tokens_labels(1, 1, 16, 1024)
    with pytest.raises(mt.MTError) as e:
        ctx.train_step(tokens, labels)
    assert e.value.status == mt.MT_E_INTERNAL
    ctx.close()
