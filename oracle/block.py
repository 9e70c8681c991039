"""Decoder-block operations in float64: forward and hand-written backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Pages cited in this file:
  [Review]  "MegaTrain: Full Precision Training of 100B+ Parameter Large
            Language Models on a Single GPU Review", dimensionstp.github.io
  [Lilting] "MegaTrainはシングルGPUで120BパラメータLLMをフル精度訓練する",
            lilting.ch

The pages train dense Qwen2.5 decoders ([Review] section 4-2, model list;
[Lilting] section "ベンチマーク結果") but never spell the block out.  The
reading taken is the standard pre-norm decoder those models use: RMSNorm ->
causal grouped-query attention with rotary positions -> residual -> RMSNorm
-> SwiGLU MLP -> residual, with no biases.  Conventions the pages leave open,
and the reading taken for each:
  * RMSNorm: eps inside the square root, statistics over the model dim.
  * RoPE: "rotate-half" pairs (e, e + hd/2), angle s * base^(-2e/hd), with
    s the position inside its own sequence.
  * GQA: query head h reads key/value head h // (Hq / Hkv).
  * attention: scale 1/sqrt(hd), causal mask s' <= s, no dropout.
  * SwiGLU: silu(gate) * up, silu(z) = z / (1 + exp(-z)).
  * loss: mean token cross-entropy over all B*S positions.

Every function takes and returns float64 numpy arrays.  Token row t = b*S+s.
"""
import numpy as np


# --------------------------------------------------------------------------
# RMSNorm
# --------------------------------------------------------------------------
def rmsnorm_fwd(x, gamma, eps):
    """n = gamma * x / sqrt(mean(x^2) + eps) per row.  Returns (n, rstd)."""
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    n = x * rstd[..., None] * gamma
    return n, rstd


def rmsnorm_bwd(dn, x, gamma, rstd):
    """Backward of ``rmsnorm_fwd``.  Returns (dx, dgamma).

    With nh = x * rstd:  dx = rstd * (g - nh * mean(g * nh)),  g = dn * gamma;
    dgamma = sum over rows of dn * nh.
    """
    nh = x * rstd[..., None]
    g = dn * gamma
    dx = rstd[..., None] * (g - nh * np.mean(g * nh, axis=-1, keepdims=True))
    dgamma = np.sum((dn * nh).reshape(-1, x.shape[-1]), axis=0)
    return dx, dgamma


# --------------------------------------------------------------------------
# Linear map y = x W^T with W stored [out x in]
# --------------------------------------------------------------------------
def linear_fwd(x, w):
    return x @ w.T


def linear_bwd(dy, x, w):
    """Returns (dx, dw) for y = x W^T."""
    return dy @ w, dy.T @ x


# --------------------------------------------------------------------------
# Rotary position embedding, rotate-half convention
# --------------------------------------------------------------------------
def rope_angles(seq, head_dim, base):
    """theta[s, e] = s * base^(-2e/hd) for s < seq, e < hd/2."""
    e = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * e / head_dim)
    s = np.arange(seq, dtype=np.float64)
    return s[:, None] * inv_freq[None, :]


def rope_rotate(z, theta):
    """Rotate pairs (e, e+hd/2) of z [B, S, H, hd] by angle theta [S, hd/2]."""
    half = z.shape[-1] // 2
    c = np.cos(theta)[None, :, None, :]
    s = np.sin(theta)[None, :, None, :]
    lo, hi = z[..., :half], z[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rope_fwd(z, base):
    """RoPE forward on z [B, S, H, hd]; position = index along S."""
    return rope_rotate(z, rope_angles(z.shape[1], z.shape[-1], base))


def rope_bwd(dz, base):
    """RoPE backward: the transpose of a rotation is the rotation by -theta."""
    return rope_rotate(dz, -rope_angles(dz.shape[1], dz.shape[-1], base))


# --------------------------------------------------------------------------
# Causal grouped-query attention, brute force S x S per head
# --------------------------------------------------------------------------
def _causal_mask(seq):
    return np.tril(np.ones((seq, seq), dtype=bool))


def _group_scores(q, k, b, j, group):
    """Scores of KV group j of sequence b: s[g, s, s'] = q[b,s,jG+g] . k[b,s',j]
    / sqrt(hd), causal (-inf above the diagonal).  [G, S, S]."""
    seq, hd = q.shape[1], q.shape[3]
    qg = np.ascontiguousarray(q[b, :, j * group:(j + 1) * group].transpose(1, 0, 2))   # [G, S, hd]
    s = (qg @ k[b, :, j].T) / np.sqrt(hd)
    return np.where(_causal_mask(seq)[None], s, -np.inf)


def _group_probs(q, k, b, j, group):
    s = _group_scores(q, k, b, j, group)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def attention_probs(q, k):
    """P[b, h, s, s'] = softmax_{s'<=s}(q[b,s,h] . k[b,s',h//G] / sqrt(hd))."""
    bsz, seq, hq, _ = q.shape
    hkv = k.shape[2]
    group = hq // hkv
    p = np.empty((bsz, hq, seq, seq))
    for b in range(bsz):
        for j in range(hkv):
            p[b, j * group:(j + 1) * group] = _group_probs(q, k, b, j, group)
    return p


def attention_lse(q, k):
    """lse[b, h, s] = log sum_{s'<=s} exp(q[b,s,h] . k[b,s',h//G] / sqrt(hd)),
    the softmax normaliser a streaming attention keeps per query row."""
    bsz, seq, hq, _ = q.shape
    hkv = k.shape[2]
    group = hq // hkv
    out = np.empty((bsz, hq, seq))
    for b in range(bsz):
        for j in range(hkv):
            s = _group_scores(q, k, b, j, group)
            mx = s.max(axis=-1, keepdims=True)
            out[b, j * group:(j + 1) * group] = (mx + np.log(np.exp(s - mx).sum(axis=-1, keepdims=True)))[..., 0]
    return out


def attention_fwd(q, k, v):
    """o [B, S, Hq, hd] for q [B,S,Hq,hd], k and v [B,S,Hkv,hd]."""
    bsz, seq, hq, hd = q.shape
    hkv = k.shape[2]
    group = hq // hkv
    o = np.empty((bsz, seq, hq, hd))
    for b in range(bsz):
        for j in range(hkv):
            p = _group_probs(q, k, b, j, group)                 # [G, S, S]
            o[b, :, j * group:(j + 1) * group] = (p @ v[b, :, j]).transpose(1, 0, 2)
    return o


def attention_bwd(do, q, k, v):
    """Returns (dq, dk, dv).

    dP = dO V^T, D = rowsum(dO * O) = rowsum(P * dP), dS = P (dP - D),
    dQ = dS K / sqrt(hd), dK = dS^T Q / sqrt(hd), dV = P^T dO; the key and
    value gradients of a KV head are summed over the query heads of its group.
    """
    bsz, seq, hq, hd = q.shape
    hkv = k.shape[2]
    group = hq // hkv
    scale = 1.0 / np.sqrt(hd)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(bsz):
        for j in range(hkv):
            hs = slice(j * group, (j + 1) * group)
            p = _group_probs(q, k, b, j, group)                 # [G, S, S]
            dog = np.ascontiguousarray(do[b, :, hs].transpose(1, 0, 2))      # [G, S, hd]
            qg = np.ascontiguousarray(q[b, :, hs].transpose(1, 0, 2))
            dp = dog @ v[b, :, j].T                              # [G, S, S]
            dsum = np.sum(p * dp, axis=-1, keepdims=True)
            ds = p * (dp - dsum)
            dq[b, :, hs] = (ds @ k[b, :, j]).transpose(1, 0, 2) * scale
            dk[b, :, j] = np.einsum("gst,gsd->td", ds, qg, optimize=True) * scale
            dv[b, :, j] = np.einsum("gst,gsd->td", p, dog, optimize=True)
    return dq, dk, dv


def attention_group_rows(q, k, v, do, rows_q, rows_k, block=1024):
    """The same attention, forward and backward, for one KV group of one
    sequence at lengths where the S x S matrices do not fit: q and do are
    [S, G, hd] (the group's G query heads), k and v [S, hd].  Returns o, lse
    and dq at query rows ``rows_q`` ([len, G, hd], [len, G], [len, G, hd]) and
    dk, dv at key rows ``rows_k`` ([len, hd], summed over the group).

    Exact float64 definition, computed in row blocks: pass 1 gets lse_s and
    o_s for every row s (softmax over keys s' <= s), hence D_s = do_s . o_s;
    then dq_s = sum_{s'<=s} P_ss' (dP_ss' - D_s) k_s' / sqrt(hd) and
    dk_j = sum_{s>=j} P_sj (dP_sj - D_s) q_s / sqrt(hd), dv_j = sum_{s>=j} P_sj do_s.
    """
    seq, grp, hd = q.shape
    sc = 1.0 / np.sqrt(hd)
    lse = np.empty((seq, grp))
    o = np.empty((seq, grp, hd))
    # Row s's lse and o depend on keys <= s only, so pass 1 is needed just for
    # the sampled query rows and for every row at or after the first sampled key.
    rows_q = np.asarray(rows_q)
    rows_k = np.asarray(rows_k)
    need = np.zeros(seq, dtype=bool)
    need[rows_q] = True
    if len(rows_k):
        need[int(rows_k.min()):] = True
    idx = np.nonzero(need)[0]
    for c0 in range(0, len(idx), block):
        rows = idx[c0:c0 + block]
        r1 = int(rows[-1]) + 1
        for g in range(grp):
            s = (q[rows, g] @ k[:r1].T) * sc                        # [rows, keys]
            s = np.where(np.arange(r1)[None, :] <= rows[:, None], s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            p = np.exp(s - mx)
            den = p.sum(axis=1, keepdims=True)
            lse[rows, g] = (mx + np.log(den))[:, 0]
            o[rows, g] = (p / den) @ v[:r1]
    dsum = np.einsum("sgd,sgd->sg", do, o)
    dq = np.zeros((len(rows_q), grp, hd))
    for i, s_ in enumerate(rows_q):
        for g in range(grp):
            p = np.exp(k[: s_ + 1] @ q[s_, g] * sc - lse[s_, g])
            dp = v[: s_ + 1] @ do[s_, g]
            dq[i, g] = (p * (dp - dsum[s_, g])) @ k[: s_ + 1] * sc
    dk = np.zeros((len(rows_k), hd))
    dv = np.zeros((len(rows_k), hd))
    for i, j in enumerate(rows_k):
        for g in range(grp):
            p = np.exp(q[j:, g] @ k[j] * sc - lse[j:, g])               # P_sj for s >= j
            dp = do[j:, g] @ v[j]
            dk[i] += (p * (dp - dsum[j:, g])) @ q[j:, g] * sc
            dv[i] += p @ do[j:, g]
    return o[rows_q], lse[rows_q], dq, dk, dv


# --------------------------------------------------------------------------
# SwiGLU
# --------------------------------------------------------------------------
def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    return z * sigmoid(z)


def silu_grad(z):
    """d silu / dz = sigma(z) * (1 + z * (1 - sigma(z)))."""
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def swiglu_fwd(a, b):
    """m = silu(a) * b, with a the gate projection and b the up projection."""
    return silu(a) * b


def swiglu_bwd(dm, a, b):
    """Returns (da, db)."""
    return dm * b * silu_grad(a), dm * silu(a)


# --------------------------------------------------------------------------
# Cross-entropy, mean over tokens
# --------------------------------------------------------------------------
def logsumexp(x):
    mx = x.max(axis=-1, keepdims=True)
    return (mx + np.log(np.sum(np.exp(x - mx), axis=-1, keepdims=True)))[..., 0]


def cross_entropy(logits, labels):
    """loss = mean_t [lse(logits_t) - logits_t[label_t]];
    dlogits = (softmax(logits) - onehot(labels)) / T.  Returns (loss, dlogits)."""
    t = logits.shape[0]
    lse = logsumexp(logits)
    picked = logits[np.arange(t), labels]
    loss = float(np.mean(lse - picked))
    dlogits = np.exp(logits - lse[:, None])
    dlogits[np.arange(t), labels] -= 1.0
    return loss, dlogits / t
