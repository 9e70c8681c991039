"""One training step of the decoder LM in float64, plus the host Adam.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Pages cited in this file:
  [Review]  MegaTrain review, dimensionstp.github.io/study-concept/megatrain/
  [Argon]   "Training 100B models on a single GPU: what MegaTrain changes ...",
            argonsys.com
  [Hotdry]  MegaTrain checkpoint strategy and communication overlap,
            blog.hotdry.top
  [Lilting] MegaTrain article, lilting.ch

What a step computes.  Forward runs layer by layer and keeps each layer's
output; backward runs the layers in reverse order, recomputing each layer's
forward from its stored input before differentiating it ([Review] 3-2 item 2
"Streaming forward and block-wise backward"; [Argon] "Layer-Wise Streaming"
and "Block-Wise Recomputation").  Gradients are the exact derivatives of the
mean token cross-entropy.  The optimizer is Adam applied on the host to FP32
master weights, first and second moments, after which the BF16 weight is
refreshed from the master ([Review] 3-2 item 6 "CPU-side optimizer update";
[Hotdry] "三层 CUDA Stream 流水线与双缓冲调度", the background thread that
runs Adam; [Lilting] per-parameter byte table: BF16 W and G, FP32 m, v and
master).  Recomputation and streaming do not change any value
([Lilting] accuracy section: the same BF16/FP32 data is only copied between
CPU and GPU), so the monolithic and streamed forms below are equal bit for
bit, which the tests check.

Readings where the pages are silent (the same list is kept with the design
notes): Adam is Kingma-Ba with bias correction, eps added after the square
root, no weight decay, no clipping, no loss scaling; the gradient Adam consumes is the
BF16 gradient widened to FP32; the embedding and LM-head tables are untied and
both trained; RMSNorm gains start at 1.
"""
from dataclasses import dataclass

import numpy as np

from . import block
from .bf16 import round_bf16

LAYER_TENSORS = ("g1", "wq", "wk", "wv", "wo", "g2", "wg", "wu", "wd")
HEAD_TENSORS = ("gf", "e_out")


@dataclass(frozen=True)
class Shape:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rms_eps: float = 1e-6
    rope_base: float = 10000.0

    def layer_shapes(self):
        d, hq, hkv, hd, f = (self.d_model, self.n_heads, self.n_kv_heads,
                             self.head_dim, self.ffn_dim)
        return {"g1": (d,), "wq": (hq * hd, d), "wk": (hkv * hd, d),
                "wv": (hkv * hd, d), "wo": (d, hq * hd), "g2": (d,),
                "wg": (f, d), "wu": (f, d), "wd": (d, f)}

    def head_shapes(self):
        return {"gf": (self.d_model,), "e_out": (self.vocab, self.d_model)}

    def n_params(self):
        per_layer = sum(int(np.prod(s)) for s in self.layer_shapes().values())
        head = sum(int(np.prod(s)) for s in self.head_shapes().values())
        return self.n_layers * per_layer + head + self.vocab * self.d_model


# --------------------------------------------------------------------------
# Decoder layer
# --------------------------------------------------------------------------
def layer_fwd(x, w, sh, batch, seq):
    """y = layer(x) for x [T, d].  Returns (y, cache of intermediates)."""
    t = x.shape[0]
    hq, hkv, hd = sh.n_heads, sh.n_kv_heads, sh.head_dim
    n1, r1 = block.rmsnorm_fwd(x, w["g1"], sh.rms_eps)
    q = block.linear_fwd(n1, w["wq"]).reshape(batch, seq, hq, hd)
    k = block.linear_fwd(n1, w["wk"]).reshape(batch, seq, hkv, hd)
    v = block.linear_fwd(n1, w["wv"]).reshape(batch, seq, hkv, hd)
    qr = block.rope_fwd(q, sh.rope_base)
    kr = block.rope_fwd(k, sh.rope_base)
    o = block.attention_fwd(qr, kr, v).reshape(t, hq * hd)
    h1 = x + block.linear_fwd(o, w["wo"])
    n2, r2 = block.rmsnorm_fwd(h1, w["g2"], sh.rms_eps)
    a = block.linear_fwd(n2, w["wg"])
    b = block.linear_fwd(n2, w["wu"])
    m = block.swiglu_fwd(a, b)
    y = h1 + block.linear_fwd(m, w["wd"])
    cache = dict(x=x, n1=n1, r1=r1, qr=qr, kr=kr, v=v, o=o, h1=h1, n2=n2,
                 r2=r2, a=a, b=b, m=m)
    return y, cache


def layer_bwd(dy, c, w, sh, batch, seq):
    """Backward of ``layer_fwd`` from its cache.  Returns (dx, grads dict)."""
    t = dy.shape[0]
    hq, hkv, hd = sh.n_heads, sh.n_kv_heads, sh.head_dim
    g = {}
    dm, g["wd"] = block.linear_bwd(dy, c["m"], w["wd"])
    da, db = block.swiglu_bwd(dm, c["a"], c["b"])
    dn2a, g["wg"] = block.linear_bwd(da, c["n2"], w["wg"])
    dn2b, g["wu"] = block.linear_bwd(db, c["n2"], w["wu"])
    dh1_norm, g["g2"] = block.rmsnorm_bwd(dn2a + dn2b, c["h1"], w["g2"], c["r2"])
    dh1 = dy + dh1_norm
    do, g["wo"] = block.linear_bwd(dh1, c["o"], w["wo"])
    dqr, dkr, dv = block.attention_bwd(do.reshape(batch, seq, hq, hd),
                                       c["qr"], c["kr"], c["v"])
    dq = block.rope_bwd(dqr, sh.rope_base).reshape(t, hq * hd)
    dk = block.rope_bwd(dkr, sh.rope_base).reshape(t, hkv * hd)
    dv = dv.reshape(t, hkv * hd)
    dn1q, g["wq"] = block.linear_bwd(dq, c["n1"], w["wq"])
    dn1k, g["wk"] = block.linear_bwd(dk, c["n1"], w["wk"])
    dn1v, g["wv"] = block.linear_bwd(dv, c["n1"], w["wv"])
    dx_norm, g["g1"] = block.rmsnorm_bwd(dn1q + dn1k + dn1v, c["x"], w["g1"], c["r1"])
    return dh1 + dx_norm, g


# --------------------------------------------------------------------------
# LM head: final RMSNorm, logits, cross-entropy (forward and backward)
# --------------------------------------------------------------------------
def head_fwd_bwd(x_last, hw, labels, sh):
    """Returns (loss, dx_last, grads dict for gf and e_out)."""
    nf, rf = block.rmsnorm_fwd(x_last, hw["gf"], sh.rms_eps)
    logits = block.linear_fwd(nf, hw["e_out"])
    loss, dlogits = block.cross_entropy(logits, labels)
    dnf, de_out = block.linear_bwd(dlogits, nf, hw["e_out"])
    dx, dgf = block.rmsnorm_bwd(dnf, x_last, hw["gf"], rf)
    return loss, dx, {"gf": dgf, "e_out": de_out}


def embed_fwd(e_in, tokens):
    return e_in[tokens.reshape(-1)]


def embed_bwd(dx0, tokens, vocab):
    """dE_in[v] = sum of dx0 rows whose token is v."""
    de = np.zeros((vocab, dx0.shape[1]))
    np.add.at(de, tokens.reshape(-1), dx0)
    return de


# --------------------------------------------------------------------------
# Whole-model loss and gradients
# --------------------------------------------------------------------------
def loss_only(params, tokens, labels, sh):
    """Forward only: the mean token cross-entropy."""
    batch, seq = tokens.shape
    x = embed_fwd(params["e_in"], tokens)
    for w in params["layers"]:
        x, _ = layer_fwd(x, w, sh, batch, seq)
    nf, _ = block.rmsnorm_fwd(x, params["head"]["gf"], sh.rms_eps)
    loss, _ = block.cross_entropy(block.linear_fwd(nf, params["head"]["e_out"]),
                                  labels.reshape(-1))
    return loss


def grads_monolithic(params, tokens, labels, sh):
    """Standard backprop keeping every layer's intermediates.

    Returns (loss, grads) with grads = {"layers": [dict...], "head": dict,
    "e_in": array}."""
    batch, seq = tokens.shape
    x = embed_fwd(params["e_in"], tokens)
    caches = []
    for w in params["layers"]:
        x, c = layer_fwd(x, w, sh, batch, seq)
        caches.append(c)
    loss, dx, ghead = head_fwd_bwd(x, params["head"], labels.reshape(-1), sh)
    glayers = [None] * sh.n_layers
    for i in reversed(range(sh.n_layers)):
        dx, glayers[i] = layer_bwd(dx, caches[i], params["layers"][i], sh, batch, seq)
    ge = embed_bwd(dx, tokens, sh.vocab)
    return loss, {"layers": glayers, "head": ghead, "e_in": ge}


def grads_streamed(params, tokens, labels, sh, n_staging=2):
    """The same gradients computed the layer-streamed way.

    Forward keeps only each layer's input (checkpoint interval of one layer);
    every layer's weights are first copied into one of ``n_staging`` staging
    arrays, as the streamed engine copies them into its ping-pong buffers.
    Backward re-copies the weights, recomputes the layer forward from the
    stored input and differentiates it.
    """
    batch, seq = tokens.shape
    staging = [None] * n_staging

    def stream_in(i):
        slot = i % n_staging
        staging[slot] = {k: v.copy() for k, v in params["layers"][i].items()}
        return staging[slot]

    x = embed_fwd(params["e_in"], tokens)
    inputs = []
    for i in range(sh.n_layers):
        inputs.append(x.copy())
        x, _ = layer_fwd(x, stream_in(i), sh, batch, seq)
    loss, dx, ghead = head_fwd_bwd(x, params["head"], labels.reshape(-1), sh)
    glayers = [None] * sh.n_layers
    for i in reversed(range(sh.n_layers)):
        w = stream_in(i)
        _, c = layer_fwd(inputs[i], w, sh, batch, seq)
        dx, glayers[i] = layer_bwd(dx, c, w, sh, batch, seq)
    ge = embed_bwd(dx, tokens, sh.vocab)
    return loss, {"layers": glayers, "head": ghead, "e_in": ge}


# --------------------------------------------------------------------------
# Host Adam on FP32 master, m, v; BF16 weight refresh
# --------------------------------------------------------------------------
def adam_update(master, m, v, grad, step, lr, beta1, beta2, eps):
    """One Adam step.

    Inputs master, m, v are float32 arrays (the FP32 state), grad holds the
    BF16 gradient values (as float32), step t >= 1.  Hyper-parameters are
    the float32 values a caller hands the library (0.999 is 0.99900001287...);
    from those, everything (1 - beta, the bias corrections 1 - beta^t, the
    update) is computed in float64, and the new state is stored back in
    float32, the state's precision.  Returns (master, m, v, w) with
    w = bf16_RNE(master).

        m <- b1 m + (1 - b1) g
        v <- b2 v + (1 - b2) g^2
        master <- master - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
    """
    b1, b2 = float(np.float32(beta1)), float(np.float32(beta2))
    lr, eps = float(np.float32(lr)), float(np.float32(eps))
    bc1 = 1.0 - b1 ** step
    bc2 = 1.0 - b2 ** step
    g = grad.astype(np.float64)
    m_new = (b1 * m.astype(np.float64) + (1.0 - b1) * g).astype(np.float32)
    v_new = (b2 * v.astype(np.float64) + (1.0 - b2) * g * g).astype(np.float32)
    mhat = m_new.astype(np.float64) / bc1
    vhat = v_new.astype(np.float64) / bc2
    upd = lr * mhat / (np.sqrt(vhat) + eps)
    master_new = (master.astype(np.float64) - upd).astype(np.float32)
    return master_new, m_new, v_new, round_bf16(master_new)


# --------------------------------------------------------------------------
# Full step over a parameter store
# --------------------------------------------------------------------------
def params_from_store(store):
    """float64 weights from a store {unit: {name: {"w","master","m","v"}}}."""
    return {"layers": [{k: t["w"].astype(np.float64) for k, t in u.items()}
                       for u in store["layers"]],
            "head": {k: t["w"].astype(np.float64) for k, t in store["head"].items()},
            "e_in": store["e_in"]["e_in"]["w"].astype(np.float64)}


def train_step(store, tokens, labels, sh, step, lr=1e-4, beta1=0.9,
               beta2=0.999, eps=1e-8, n_staging=2, adam_order=None):
    """Layer-streamed step on ``store`` (modified in place).

    The store holds float32 arrays "w" (BF16 values), "master", "m", "v" per
    tensor.  Gradients come from ``grads_streamed`` and are rounded to BF16,
    the precision the pages stream gradients out in; Adam then updates every
    tensor.  ``adam_order`` permutes the order units are updated in (units
    are independent, so the result must not depend on it).  Returns
    (loss, bf16 gradients as float32 in store layout).
    """
    params = params_from_store(store)
    loss, gr = grads_streamed(params, tokens, labels, sh, n_staging)
    units = [("layers", i) for i in range(sh.n_layers)] + [("head", None), ("e_in", None)]
    gstore = {"layers": [dict() for _ in range(sh.n_layers)], "head": {}, "e_in": {}}

    def unit_of(tree, kind, i):
        return tree[kind][i] if kind == "layers" else tree[kind]

    for kind, i in units:
        g_unit = unit_of(gr, kind, i) if kind != "e_in" else {"e_in": gr["e_in"]}
        for name, g in g_unit.items():
            unit_of(gstore, kind, i)[name] = round_bf16(g.astype(np.float32))
    order = list(range(len(units))) if adam_order is None else list(adam_order)
    for u in order:
        kind, i = units[u]
        for name, t in unit_of(store, kind, i).items():
            g = unit_of(gstore, kind, i)[name]
            t["master"], t["m"], t["v"], t["w"] = adam_update(
                t["master"], t["m"], t["v"], g, step, lr, beta1, beta2, eps)
    return loss, gstore


# --------------------------------------------------------------------------
# Gradient accumulation over micro-batches
# --------------------------------------------------------------------------
def accumulate_bf16(acc, g):
    """acc + g for two arrays of BF16 values, rounded once to BF16 (RNE).

    The host keeps the accumulated gradient in the BF16 G region of each
    tile ([Review] 3-2 item 1: the host holds parameters, the accumulated
    gradient and the optimizer state; [Hotdry] "三层 CUDA Stream 流水线与双缓冲调度":
    the CPU thread unpacks each slab and accumulates it into the master
    store).  The sum of two BF16 values is computed exactly in float64;
    float32 then holds it exactly, or within far less than half a BF16 unit
    of the larger operand, so a single BF16 rounding follows."""
    s = acc.astype(np.float64) + g.astype(np.float64)
    return round_bf16(s.astype(np.float32))


def grads_accumulated(params, tokens, labels, sh, n_staging=2):
    """float64 gradients of the mean cross-entropy over every token of the
    micro-batches tokens[j] (shape [n, B, S]), without BF16 rounding: the
    sum over j of each micro-batch's gradient times 1/n.  Returns
    (loss, grads) like ``grads_streamed``."""
    n = tokens.shape[0]
    total, loss = None, 0.0
    for j in range(n):
        lj, gj = grads_streamed(params, tokens[j], labels[j], sh, n_staging)
        loss += lj / n
        gj = _scale_tree(gj, 1.0 / n)
        total = gj if total is None else _add_tree(total, gj)
    return loss, total


def _scale_tree(tree, s):
    return {"layers": [{k: v * s for k, v in u.items()} for u in tree["layers"]],
            "head": {k: v * s for k, v in tree["head"].items()},
            "e_in": tree["e_in"] * s}


def _add_tree(a, b):
    return {"layers": [{k: ua[k] + ub[k] for k in ua} for ua, ub in zip(a["layers"], b["layers"])],
            "head": {k: a["head"][k] + b["head"][k] for k in a["head"]},
            "e_in": a["e_in"] + b["e_in"]}


def train_step_accum(store, tokens, labels, sh, step, lr=1e-4, beta1=0.9,
                     beta2=0.999, eps=1e-8, n_staging=2):
    """One optimizer step over n micro-batches (tokens, labels [n, B, S]).

    Every micro-batch runs the whole streamed forward and backward with the
    weights of the step's start; its gradient of the mean loss over all
    n*B*S tokens (the micro-batch's own gradient times 1/n) is rounded to
    BF16, the precision gradients stream out in, and summed into the BF16
    accumulator in micro-batch order with one rounding per addition
    (``accumulate_bf16``).  Adam then runs once on the accumulated gradient.
    The loss is the mean over all tokens.  With n = 1 this is ``train_step``.
    Returns (loss, accumulated BF16 gradients as float32 in store layout)."""
    n = tokens.shape[0]
    params = params_from_store(store)
    units = [("layers", i) for i in range(sh.n_layers)] + [("head", None), ("e_in", None)]

    def unit_of(tree, kind, i):
        return tree[kind][i] if kind == "layers" else tree[kind]

    gstore = None
    loss = 0.0
    for j in range(n):
        lj, gr = grads_streamed(params, tokens[j], labels[j], sh, n_staging)
        loss += lj / n
        gj = {"layers": [dict() for _ in range(sh.n_layers)], "head": {}, "e_in": {}}
        for kind, i in units:
            g_unit = unit_of(gr, kind, i) if kind != "e_in" else {"e_in": gr["e_in"]}
            for name, g in g_unit.items():
                gb = round_bf16((g / n).astype(np.float32))
                if gstore is not None:
                    gb = accumulate_bf16(unit_of(gstore, kind, i)[name], gb)
                unit_of(gj, kind, i)[name] = gb
        gstore = gj
    for kind, i in units:
        for name, t in unit_of(store, kind, i).items():
            g = unit_of(gstore, kind, i)[name]
            t["master"], t["m"], t["v"], t["w"] = adam_update(
                t["master"], t["m"], t["v"], g, step, lr, beta1, beta2, eps)
    return loss, gstore
