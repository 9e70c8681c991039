"""Pins for the oracle's whole-model gradients, streaming invariance and Adam.

All CPU.  Gradients are pinned by central finite differences of every
parameter element on a tiny LM and by torch float64 autograd at the tiny-LM
shape of the parity workload; the head and the layers by closed forms; the
streamed form by bit-equality with plain backprop; Adam by its closed forms.
"""
import math

import numpy as np
import pytest
import torch

from layer_streaming_amd import synth
from oracle import block, step
from oracle.bf16 import round_bf16

TINY = step.Shape(n_layers=2, d_model=16, n_heads=2, n_kv_heads=1, head_dim=8,
                  ffn_dim=24, vocab=37, rms_eps=1e-6, rope_base=10000.0)
CFG1 = step.Shape(n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64,
                  ffn_dim=688, vocab=1024, rms_eps=1e-6, rope_base=10000.0)


def random_params(sh, seed, std=0.3, gamma_noise=0.2):
    rng = np.random.default_rng(seed)
    layers = []
    for _ in range(sh.n_layers):
        u = {}
        for name, shp in sh.layer_shapes().items():
            if name.startswith("g"):
                u[name] = 1.0 + gamma_noise * rng.standard_normal(shp)
            else:
                u[name] = std * rng.standard_normal(shp)
        layers.append(u)
    head = {"gf": 1.0 + gamma_noise * rng.standard_normal(sh.d_model),
            "e_out": std * rng.standard_normal((sh.vocab, sh.d_model))}
    return {"layers": layers, "head": head,
            "e_in": rng.standard_normal((sh.vocab, sh.d_model))}


def _all_tensors(tree):
    for i, u in enumerate(tree["layers"]):
        for k in step.LAYER_TENSORS:
            yield ("layers", i, k), u[k]
    for k in step.HEAD_TENSORS:
        yield ("head", None, k), tree["head"][k]
    yield ("e_in", None, "e_in"), tree["e_in"]


def _get(tree, key):
    kind, i, k = key
    if kind == "layers":
        return tree["layers"][i][k]
    if kind == "head":
        return tree["head"][k]
    return tree["e_in"]


# ----------------------------------------------- finite differences (P1) --
def test_gradients_match_finite_differences_every_element():
    params = random_params(TINY, seed=1)
    tokens, labels = synth.tokens_labels(99, 2, 5, TINY.vocab)
    loss, grads = step.grads_monolithic(params, tokens, labels, TINY)
    h = 1e-5
    for key, w in _all_tensors(params):
        g = _get(grads, key)
        flat = w.reshape(-1)
        fd = np.zeros(flat.size)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + h
            lp = step.loss_only(params, tokens, labels, TINY)
            flat[i] = old - h
            lm = step.loss_only(params, tokens, labels, TINY)
            flat[i] = old
            fd[i] = (lp - lm) / (2 * h)
        err = np.linalg.norm(g.reshape(-1) - fd) / max(np.linalg.norm(fd), 1e-30)
        assert err < 1e-6, (key, err)
        assert np.max(np.abs(g.reshape(-1) - fd)) < 1e-8, key
    assert loss == pytest.approx(step.loss_only(params, tokens, labels, TINY), rel=1e-15)


# ------------------------------------------------ torch float64 autograd --
def _torch_loss(p, tokens, labels, sh):
    """The same model written with torch ops; autograd supplies the backward."""
    bsz, seq = tokens.shape
    t = bsz * seq
    hq, hkv, hd = sh.n_heads, sh.n_kv_heads, sh.head_dim

    def rms(x, g):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + sh.rms_eps) * g

    e = torch.arange(hd // 2, dtype=torch.float64)
    inv = sh.rope_base ** (-2.0 * e / hd)
    ang = torch.arange(seq, dtype=torch.float64)[:, None] * inv[None, :]
    cos = torch.cat([ang.cos(), ang.cos()], -1)[None, :, None, :]
    sin = torch.cat([ang.sin(), ang.sin()], -1)[None, :, None, :]

    def rope(z):
        lo, hi = z[..., : hd // 2], z[..., hd // 2:]
        return z * cos + torch.cat([-hi, lo], -1) * sin

    x = p["e_in"][torch.from_numpy(tokens.reshape(-1).astype(np.int64))]
    for w in p["layers"]:
        n1 = rms(x, w["g1"])
        q = rope((n1 @ w["wq"].T).view(bsz, seq, hq, hd)).transpose(1, 2)
        k = rope((n1 @ w["wk"].T).view(bsz, seq, hkv, hd)).transpose(1, 2)
        v = (n1 @ w["wv"].T).view(bsz, seq, hkv, hd).transpose(1, 2)
        k = k.repeat_interleave(hq // hkv, dim=1)
        v = v.repeat_interleave(hq // hkv, dim=1)
        s = (q @ k.transpose(-1, -2)) / math.sqrt(hd)
        mask = torch.ones(seq, seq, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
        o = (torch.softmax(s, -1) @ v).transpose(1, 2).reshape(t, hq * hd)
        h1 = x + o @ w["wo"].T
        n2 = rms(h1, w["g2"])
        x = h1 + (torch.nn.functional.silu(n2 @ w["wg"].T) * (n2 @ w["wu"].T)) @ w["wd"].T
    nf = rms(x, p["head"]["gf"])
    logits = nf @ p["head"]["e_out"].T
    return torch.nn.functional.cross_entropy(
        logits, torch.from_numpy(labels.reshape(-1).astype(np.int64)))


def test_gradients_match_torch_autograd_at_parity_shape():
    sh = CFG1
    params = random_params(sh, seed=2, std=0.05)
    tokens, labels = synth.tokens_labels(5678, 2, 128, sh.vocab)
    loss, grads = step.grads_monolithic(params, tokens, labels, sh)
    tp = {"layers": [{k: torch.from_numpy(v.copy()).requires_grad_(True) for k, v in u.items()}
                     for u in params["layers"]],
          "head": {k: torch.from_numpy(v.copy()).requires_grad_(True)
                   for k, v in params["head"].items()},
          "e_in": torch.from_numpy(params["e_in"].copy()).requires_grad_(True)}
    ref = _torch_loss(tp, tokens, labels, sh)
    ref.backward()
    assert loss == pytest.approx(ref.item(), rel=1e-12)
    for key, _ in _all_tensors(params):
        g = _get(grads, key)
        tg = _get(tp, key).grad.numpy()
        err = np.linalg.norm(g - tg) / np.linalg.norm(tg)
        assert err < 1e-10, (key, err)


# ------------------------------------------------------- head (P2) -------
def test_zero_head_gives_ln_vocab_and_closed_form_gradients():
    sh = step.Shape(2, 32, 2, 2, 16, 40, 1024)
    params = random_params(sh, seed=3)
    params["head"]["e_out"][:] = 0.0
    tokens, labels = synth.tokens_labels(4, 2, 6, sh.vocab)
    loss, grads = step.grads_monolithic(params, tokens, labels, sh)
    assert loss == pytest.approx(6.931471805599453, abs=1e-14)
    # dx into the last layer is zero, so every layer gradient is zero
    for u in grads["layers"]:
        for k, g in u.items():
            assert np.all(g == 0.0), k
    assert np.all(grads["head"]["gf"] == 0.0)
    # dE_out = dlogits^T nf with dlogits = (1/V - onehot)/T
    x = params["e_in"][tokens.reshape(-1)]
    for w in params["layers"]:
        x, _ = step.layer_fwd(x, w, sh, 2, 6)
    nf = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + sh.rms_eps) * params["head"]["gf"]
    t = 12
    onehot = np.zeros((t, sh.vocab))
    onehot[np.arange(t), labels.reshape(-1)] = 1.0
    expect = ((1.0 / sh.vocab - onehot) / t).T @ nf
    np.testing.assert_allclose(grads["head"]["e_out"], expect, rtol=1e-12, atol=1e-16)


def test_init_scale_loss_is_near_ln_vocab_plus_half_variance():
    """At N(0, 0.02^2) init the logits have variance 0.02^2 * d (unit-RMS
    inputs), so E[loss] ~ ln V + sigma^2/2."""
    sh = CFG1
    rng = np.random.default_rng(8)
    params = random_params(sh, seed=8, std=0.02, gamma_noise=0.0)
    params["e_in"] = 0.02 * rng.standard_normal((sh.vocab, sh.d_model))
    tokens, labels = synth.tokens_labels(5678, 2, 128, sh.vocab)
    loss = step.loss_only(params, tokens, labels, sh)
    expect = math.log(sh.vocab) + 0.02 ** 2 * sh.d_model / 2
    assert abs(loss - expect) < 0.03


# ---------------------------------------------- identity network (P7) ----
def test_identity_network_reduces_to_embedding_head():
    sh = TINY
    params = random_params(sh, seed=4)
    for u in params["layers"]:
        u["wo"][:] = 0.0
        u["wd"][:] = 0.0
    tokens, labels = synth.tokens_labels(12, 2, 5, sh.vocab)
    loss = step.loss_only(params, tokens, labels, sh)
    x = params["e_in"][tokens.reshape(-1)]
    nf = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + sh.rms_eps) * params["head"]["gf"]
    logits = nf @ params["head"]["e_out"].T
    lab = labels.reshape(-1)
    expect = np.mean([math.log(np.sum(np.exp(r))) - r[l] for r, l in zip(logits, lab)])
    assert loss == pytest.approx(expect, rel=1e-13)


def test_zero_gate_makes_mlp_vanish():
    sh = TINY
    w = random_params(sh, seed=6)["layers"][0]
    w["wg"][:] = 0.0
    x = np.random.default_rng(1).standard_normal((10, sh.d_model))
    y, c = step.layer_fwd(x, w, sh, 2, 5)
    np.testing.assert_array_equal(y, c["h1"])


# -------------------------------------------- streaming invariance (P8) --
@pytest.mark.parametrize("n_staging", [1, 2, 3])
def test_streamed_equals_monolithic_bit_for_bit(n_staging):
    sh = TINY
    params = random_params(sh, seed=5)
    tokens, labels = synth.tokens_labels(77, 2, 5, sh.vocab)
    l1, g1 = step.grads_monolithic(params, tokens, labels, sh)
    l2, g2 = step.grads_streamed(params, tokens, labels, sh, n_staging=n_staging)
    assert l1 == l2
    for key, _ in _all_tensors(params):
        assert np.array_equal(_get(g1, key), _get(g2, key)), key


def _store_from(params, sh):
    def t(w):
        wb = round_bf16(w.astype(np.float32))
        return {"w": wb.copy(), "master": wb.copy(), "m": np.zeros_like(wb),
                "v": np.zeros_like(wb)}
    return {"layers": [{k: t(v) for k, v in u.items()} for u in params["layers"]],
            "head": {k: t(v) for k, v in params["head"].items()},
            "e_in": {"e_in": t(params["e_in"])}}


def test_adam_order_does_not_change_the_step():
    sh = TINY
    params = random_params(sh, seed=9)
    tokens, labels = synth.tokens_labels(3, 2, 5, sh.vocab)
    s1, s2 = _store_from(params, sh), _store_from(params, sh)
    n_units = sh.n_layers + 2
    l1, _ = step.train_step(s1, tokens, labels, sh, step=1)
    l2, _ = step.train_step(s2, tokens, labels, sh, step=1, n_staging=3,
                            adam_order=list(reversed(range(n_units))))
    assert l1 == l2
    for a, b in zip(_leaves(s1), _leaves(s2)):
        assert np.array_equal(a, b)


def _leaves(store):
    for u in store["layers"]:
        for k in step.LAYER_TENSORS:
            yield from (u[k][f] for f in ("w", "master", "m", "v"))
    for k in step.HEAD_TENSORS:
        yield from (store["head"][k][f] for f in ("w", "master", "m", "v"))
    yield from (store["e_in"]["e_in"][f] for f in ("w", "master", "m", "v"))


# ------------------------------------------------------------- Adam (P9) --
def _ulp_diff(a, b):
    ia = a.astype(np.float32).view(np.int32).astype(np.int64)
    ib = b.astype(np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def test_adam_first_step_closed_form():
    rng = np.random.default_rng(21)
    n = 20000
    theta = rng.standard_normal(n).astype(np.float32)
    g = round_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
    g[:50] = 0.0
    lr, eps = 1e-4, 1e-8
    mast, m, v, w = step.adam_update(theta, np.zeros(n, np.float32), np.zeros(n, np.float32),
                                     g, 1, lr, 0.9, 0.999, eps)
    gd = g.astype(np.float64)
    expect = theta.astype(np.float64) - lr * gd / (np.abs(gd) + eps)
    # m/bc1 and sqrt(v/bc2) carry float32 rounding of ~1e-7 relative, so the
    # step itself is exact to ~1e-7 * lr; elsewhere within a few ulp of theta
    err = np.abs(mast.astype(np.float64) - expect)
    ulp = np.spacing(np.abs(expect).astype(np.float32)).astype(np.float64)
    assert np.all(err <= np.maximum(4 * ulp, 1e-6 * lr))
    assert np.array_equal(mast[:50], theta[:50])
    # (1 - beta) of the float32 hyper-parameters the library receives
    np.testing.assert_allclose(m, (1 - float(np.float32(0.9))) * gd, rtol=1e-6)
    np.testing.assert_allclose(v, (1 - float(np.float32(0.999))) * gd * gd, rtol=1e-6)
    assert np.array_equal(w, round_bf16(mast))


def test_adam_two_steps_closed_form():
    rng = np.random.default_rng(22)
    n = 1000
    theta = rng.standard_normal(n).astype(np.float32)
    g1 = round_bf16((rng.standard_normal(n) * 1e-2).astype(np.float32)).astype(np.float64)
    g2 = round_bf16((rng.standard_normal(n) * 1e-2).astype(np.float32)).astype(np.float64)
    # hyper-parameters as the float32 values the library receives
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    lr, eps = float(np.float32(1e-3)), float(np.float32(1e-8))
    st = (theta, np.zeros(n, np.float32), np.zeros(n, np.float32))
    st = step.adam_update(*st, g1.astype(np.float32), 1, lr, b1, b2, eps)[:3]
    mast, m, v, _ = step.adam_update(*st, g2.astype(np.float32), 2, lr, b1, b2, eps)
    m2 = (1 - b1) * (b1 * g1 + g2)
    v2 = (1 - b2) * (b2 * g1 * g1 + g2 * g2)
    d1 = lr * g1 / (np.abs(g1) + eps)
    d2 = lr * (m2 / (1 - b1 ** 2)) / (np.sqrt(v2 / (1 - b2 ** 2)) + eps)
    expect = theta.astype(np.float64) - d1 - d2
    np.testing.assert_allclose(mast, expect, rtol=2e-6, atol=1e-9)
    np.testing.assert_allclose(m, m2, rtol=1e-5, atol=1e-10)
    np.testing.assert_allclose(v, v2, rtol=1e-5, atol=1e-15)


def test_adam_zero_betas_is_sign_descent_every_step():
    rng = np.random.default_rng(23)
    n = 500
    theta = rng.standard_normal(n).astype(np.float32)
    st = (theta, np.zeros(n, np.float32), np.zeros(n, np.float32))
    cur = theta.astype(np.float64)
    for t in range(1, 4):
        g = round_bf16((rng.standard_normal(n) * 1e-2).astype(np.float32))
        st = step.adam_update(*st, g, t, 1e-3, 0.0, 0.0, 1e-8)[:3]
        cur = cur - 1e-3 * g / (np.abs(g.astype(np.float64)) + 1e-8)
        ulp = np.spacing(np.abs(cur).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(st[0] - cur) <= np.maximum(2 * ulp, 1e-9))
        cur = st[0].astype(np.float64)


# ------------------------------------------------ memory arithmetic (P11) --
def test_parameter_counts_and_host_store_bytes():
    qwen7 = step.Shape(28, 3584, 28, 4, 128, 18944, 152064)
    qwen14 = step.Shape(48, 5120, 40, 8, 128, 13824, 152064)
    assert qwen7.n_params() == 7_615_487_488
    assert qwen14.n_params() == 14_769_689_600
    # 16 bytes per parameter: ~122 GB and ~235 GB on the pages
    assert abs(qwen7.n_params() * 16 / 1e9 - 122) < 0.5
    assert abs(qwen14.n_params() * 16 / 1e9 - 235) < 1.5
    assert CFG1.n_params() == 2 * 791_040 + 256 + 2 * 1024 * 256


# ------------------------------------------- gradient accumulation (P10) --
def _bf16_grid_neighbours(x):
    """The two bf16 values around a float64 x (exact, via float32 bits)."""
    f = np.float32(x)
    bits = int(np.array(f).view(np.uint32))
    lo_bits = bits & 0xFFFF0000
    lo = float(np.array(lo_bits, dtype=np.uint32).view(np.float32))
    hi = float(np.array((lo_bits + 0x10000) & 0xFFFFFFFF, dtype=np.uint32).view(np.float32))
    return lo, hi


def test_accumulate_bf16_is_one_rounding_of_the_exact_sum():
    """Brute force against the definition: the exact sum (Fractions) rounded
    to the nearer bf16 neighbour, ties to the even one."""
    from fractions import Fraction
    rng = np.random.default_rng(4)
    a = round_bf16(rng.standard_normal(4000).astype(np.float32))
    b = round_bf16((rng.standard_normal(4000) * np.exp2(rng.integers(-30, 30, 4000))).astype(np.float32))
    # ties: b equal to half a bf16 unit of a, with a's last bit odd and even
    ta = round_bf16(np.float32(1.0) + np.arange(1, 33, dtype=np.float32) * np.float32(2.0 ** -7))
    tb = np.full(32, 2.0 ** -8, dtype=np.float32)
    a, b = np.concatenate([a, ta]), np.concatenate([b, tb])
    got = step.accumulate_bf16(a, b)
    for x, y, g in zip(a, b, got):
        s = Fraction(float(x)) + Fraction(float(y))
        lo, hi = _bf16_grid_neighbours(float(s))
        if s < 0:
            lo, hi = sorted(_bf16_grid_neighbours(float(s)))
        lo, hi = min(lo, hi), max(lo, hi)
        if Fraction(lo) == s:
            want = lo
        elif Fraction(hi) == s:
            want = hi
        else:
            dlo, dhi = s - Fraction(lo), Fraction(hi) - s
            if dlo != dhi:
                want = lo if dlo < dhi else hi
            else:
                lob = int(np.array(np.float32(lo)).view(np.uint32)) >> 16
                want = lo if lob % 2 == 0 else hi
        assert float(g) == want, (x, y, g, want)


def test_accumulated_gradient_equals_the_full_batch_gradient():
    """Two micro-batches of B sequences give the gradient of one batch of 2B
    sequences (the mean over every token), before any rounding."""
    sh = TINY
    params = random_params(sh, seed=31)
    ta, la = synth.tokens_labels(41, 2, 5, sh.vocab)
    tb, lb = synth.tokens_labels(42, 2, 5, sh.vocab)
    loss_acc, g_acc = step.grads_accumulated(params, np.stack([ta, tb]), np.stack([la, lb]), sh)
    loss_full, g_full = step.grads_monolithic(params, np.concatenate([ta, tb]), np.concatenate([la, lb]), sh)
    assert abs(loss_acc - loss_full) <= 1e-13 * abs(loss_full)
    for key, _ in _all_tensors(params):
        ga, gf = _get(g_acc, key), _get(g_full, key)
        assert np.max(np.abs(ga - gf)) <= 1e-12 * max(np.max(np.abs(gf)), 1e-300), key


def test_one_micro_batch_is_the_plain_step():
    sh = TINY
    params = random_params(sh, seed=12)
    tokens, labels = synth.tokens_labels(8, 2, 5, sh.vocab)
    s1, s2 = _store_from(params, sh), _store_from(params, sh)
    l1, g1 = step.train_step(s1, tokens, labels, sh, step=1)
    l2, g2 = step.train_step_accum(s2, tokens[None], labels[None], sh, step=1)
    assert l1 == l2
    for a, b in zip(_leaves(s1), _leaves(s2)):
        assert np.array_equal(a, b)


def test_identical_micro_batches_equal_one_step_bit_for_bit():
    """n copies of one micro-batch: each gradient is the plain one times 1/n
    (a power of two here, exact), the BF16 sums are exact, so the update is
    the plain step's bit for bit."""
    sh = TINY
    params = random_params(sh, seed=13)
    tokens, labels = synth.tokens_labels(9, 2, 5, sh.vocab)
    for n in (2, 4):
        s1, s2 = _store_from(params, sh), _store_from(params, sh)
        l1, g1 = step.train_step(s1, tokens, labels, sh, step=1)
        l2, g2 = step.train_step_accum(s2, np.stack([tokens] * n), np.stack([labels] * n), sh, step=1)
        assert l1 == l2
        for a, b in zip(_leaves(s1), _leaves(s2)):
            assert np.array_equal(a, b)


def test_accumulation_adds_in_micro_batch_order_with_one_rounding_each():
    """Planted values: the accumulated G of three micro-batches is
    bf16(bf16(g0 + g1) + g2) of the per-micro-batch BF16 gradients."""
    sh = TINY
    params = random_params(sh, seed=14)
    toks = [synth.tokens_labels(50 + j, 1, 6, sh.vocab) for j in range(3)]
    tokens = np.stack([t for t, _ in toks])
    labels = np.stack([l for _, l in toks])
    store = _store_from(params, sh)
    _, gacc = step.train_step_accum(store, tokens, labels, sh, step=1)
    p = step.params_from_store(_store_from(params, sh))
    per = [step.grads_streamed(p, tokens[j], labels[j], sh)[1] for j in range(3)]
    for key, _ in _all_tensors(params):
        gb = [round_bf16((_get(g, key) / 3).astype(np.float32)) for g in per]
        want = round_bf16((round_bf16((gb[0].astype(np.float64) + gb[1]).astype(np.float32))
                           .astype(np.float64) + gb[2]).astype(np.float32))
        kind, i, k = key
        got = gacc["layers"][i][k] if kind == "layers" else gacc[kind][k]
        assert np.array_equal(got, want), key
