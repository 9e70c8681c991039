"""Pins for the oracle's block operations (CPU only).

Each oracle function is checked against something other than itself:
closed forms, identities, brute-force sums, finite differences, or a torch
float64 library routine.
"""
import math

import numpy as np
import pytest
import torch

from oracle import block


def _fd_grad(f, x, h=1e-6):
    """Central finite differences of scalar f at every element of x."""
    g = np.zeros_like(x)
    flat = x.reshape(-1)
    gf = g.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + h
        fp = f()
        flat[i] = old - h
        fm = f()
        flat[i] = old
        gf[i] = (fp - fm) / (2 * h)
    return g


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


rng = np.random.default_rng(11)


# ----------------------------------------------------------------- RMSNorm --
def test_rmsnorm_constant_row_closed_form():
    d, c, eps = 64, 0.37, 1e-6
    x = np.full((3, d), c)
    gamma = rng.standard_normal(d)
    n, rstd = block.rmsnorm_fwd(x, gamma, eps)
    np.testing.assert_allclose(rstd, 1.0 / math.sqrt(c * c + eps), rtol=1e-15)
    np.testing.assert_allclose(n, np.broadcast_to(c / math.sqrt(c * c + eps) * gamma, (3, d)),
                               rtol=1e-14)


def test_rmsnorm_scale_invariant_when_eps_zero():
    x = rng.standard_normal((4, 32))
    g = rng.standard_normal(32)
    n1, _ = block.rmsnorm_fwd(x, g, 0.0)
    n2, _ = block.rmsnorm_fwd(7.5 * x, g, 0.0)
    np.testing.assert_allclose(n1, n2, rtol=1e-13)


def test_rmsnorm_bwd_finite_differences():
    x = rng.standard_normal((3, 12))
    gamma = rng.standard_normal(12)
    w = rng.standard_normal((3, 12))            # loss = sum(w * n)
    eps = 1e-3

    def f():
        return float(np.sum(w * block.rmsnorm_fwd(x, gamma, eps)[0]))
    _, rstd = block.rmsnorm_fwd(x, gamma, eps)
    dx, dg = block.rmsnorm_bwd(w, x, gamma, rstd)
    assert _rel(dx, _fd_grad(f, x)) < 1e-8
    assert _rel(dg, _fd_grad(f, gamma)) < 1e-8


# -------------------------------------------------------------------- RoPE --
def test_rope_identity_at_position_zero_and_norm_preserved():
    z = rng.standard_normal((2, 9, 3, 16))
    r = block.rope_fwd(z, 10000.0)
    np.testing.assert_array_equal(r[:, 0], z[:, 0])
    half = 8
    n_in = z[..., :half] ** 2 + z[..., half:] ** 2
    n_out = r[..., :half] ** 2 + r[..., half:] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-12)


def test_rope_relative_position_property():
    hd, base = 32, 10000.0
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    theta = block.rope_angles(40, hd, base)
    rot = lambda z, s: block.rope_rotate(z[None, None, None, :], theta[s][None, :])[0, 0, 0]
    for m, n in [(5, 2), (17, 17), (39, 0), (21, 8)]:
        lhs = rot(q, m) @ rot(k, n)
        rhs = rot(q, m - n) @ k
        assert abs(lhs - rhs) < 1e-11 * (1 + abs(rhs))


def test_rope_bwd_is_inverse_and_transpose():
    z = rng.standard_normal((2, 7, 2, 8))
    w = rng.standard_normal((2, 7, 2, 8))
    np.testing.assert_allclose(block.rope_bwd(block.rope_fwd(z, 500.0), 500.0), z, atol=1e-13)
    # <R z, w> = <z, R^T w>
    lhs = np.sum(block.rope_fwd(z, 500.0) * w)
    rhs = np.sum(z * block.rope_bwd(w, 500.0))
    assert abs(lhs - rhs) < 1e-12


def test_rope_matches_complex_rotation():
    """Pair (e, e+hd/2) as a complex number rotated by exp(i theta)."""
    z = rng.standard_normal((1, 6, 1, 10))
    r = block.rope_fwd(z, 10000.0)
    for s in range(6):
        for e in range(5):
            th = s * 10000.0 ** (-2 * e / 10)
            c = complex(z[0, s, 0, e], z[0, s, 0, e + 5]) * complex(math.cos(th), math.sin(th))
            assert abs(r[0, s, 0, e] - c.real) < 1e-13
            assert abs(r[0, s, 0, e + 5] - c.imag) < 1e-13


# --------------------------------------------------------------- Attention --
def test_attention_single_position_returns_v():
    q = rng.standard_normal((2, 1, 4, 8))
    k = rng.standard_normal((2, 1, 2, 8))
    v = rng.standard_normal((2, 1, 2, 8))
    o = block.attention_fwd(q, k, v)
    np.testing.assert_allclose(o, np.repeat(v, 2, axis=2), rtol=1e-15)


def test_attention_zero_query_is_causal_prefix_mean():
    bsz, seq, hq, hkv, hd = 2, 9, 4, 2, 8
    q = np.zeros((bsz, seq, hq, hd))
    k = rng.standard_normal((bsz, seq, hkv, hd))
    v = rng.standard_normal((bsz, seq, hkv, hd))
    o = block.attention_fwd(q, k, v)
    for s in range(seq):
        expect = np.repeat(v[:, : s + 1].mean(axis=1), 2, axis=1)
        np.testing.assert_allclose(o[:, s], expect, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(o[:, 0], np.repeat(v[:, 0], 2, axis=1), rtol=1e-14)


def test_attention_lse_closed_forms():
    # zero queries: every visible score is 0, so lse = log(number of keys seen)
    q = np.zeros((1, 7, 2, 8))
    k = rng.standard_normal((1, 7, 1, 8))
    lse = block.attention_lse(q, k)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, 8)), rtol=1e-14)
    # position 0 sees only key 0: lse = q0 . k0 / sqrt(hd)
    q = rng.standard_normal((2, 5, 2, 16))
    k = rng.standard_normal((2, 5, 2, 16))
    lse = block.attention_lse(q, k)
    np.testing.assert_allclose(lse[:, :, 0], np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]) / 4.0, rtol=1e-13)
    # brute force on one row
    s = 4
    ref = math.log(sum(math.exp(float(q[1, s, 1] @ k[1, j, 1]) / 4.0) for j in range(s + 1)))
    assert abs(lse[1, 1, s] - ref) < 1e-12


def test_attention_brute_force_loops():
    bsz, seq, hq, hkv, hd = 1, 6, 3, 1, 4
    q = rng.standard_normal((bsz, seq, hq, hd))
    k = rng.standard_normal((bsz, seq, hkv, hd))
    v = rng.standard_normal((bsz, seq, hkv, hd))
    o = block.attention_fwd(q, k, v)
    for h in range(hq):
        for s in range(seq):
            w = [math.exp(sum(q[0, s, h, e] * k[0, j, 0, e] for e in range(hd)) / 2.0)
                 for j in range(s + 1)]
            tot = sum(w)
            ref = [sum(w[j] * v[0, j, 0, e] for j in range(s + 1)) / tot for e in range(hd)]
            np.testing.assert_allclose(o[0, s, h], ref, rtol=1e-12)


def test_attention_matches_torch_sdpa_float64():
    bsz, seq, hq, hkv, hd = 2, 33, 6, 2, 16
    q = rng.standard_normal((bsz, seq, hq, hd))
    k = rng.standard_normal((bsz, seq, hkv, hd))
    v = rng.standard_normal((bsz, seq, hkv, hd))
    o = block.attention_fwd(q, k, v)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.repeat(k, 3, axis=2)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.repeat(v, 3, axis=2)).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-13)


def test_attention_group_rows_equals_full_attention():
    """The blocked row-sampled form against the S x S form on one KV group."""
    seq, grp, hd = 70, 3, 16
    q = rng.standard_normal((1, seq, grp, hd))
    k = rng.standard_normal((1, seq, 1, hd))
    v = rng.standard_normal((1, seq, 1, hd))
    do = rng.standard_normal((1, seq, grp, hd))
    o = block.attention_fwd(q, k, v)[0]
    lse = block.attention_lse(q, k)[0]                     # [grp, seq]
    dq, dk, dv = block.attention_bwd(do, q, k, v)
    rq, rk = [0, 5, 31, 32, 69], [0, 1, 40, 69]
    o2, lse2, dq2, dk2, dv2 = block.attention_group_rows(q[0], k[0, :, 0], v[0, :, 0], do[0], rq, rk, block=16)
    np.testing.assert_allclose(o2, o[rq], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse[:, rq].T, rtol=1e-12)
    np.testing.assert_allclose(dq2, dq[0, rq], rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dk2, dk[0, rk, 0], rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dv2, dv[0, rk, 0], rtol=1e-10, atol=1e-13)


def test_attention_gqa_equals_mha_with_replicated_kv():
    bsz, seq, hq, hkv, hd = 1, 7, 6, 2, 8
    q = rng.standard_normal((bsz, seq, hq, hd))
    k = rng.standard_normal((bsz, seq, hkv, hd))
    v = rng.standard_normal((bsz, seq, hkv, hd))
    do = rng.standard_normal((bsz, seq, hq, hd))
    kr, vr = np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2)
    np.testing.assert_allclose(block.attention_fwd(q, k, v), block.attention_fwd(q, kr, vr),
                               rtol=1e-14)
    dq, dk, dv = block.attention_bwd(do, q, k, v)
    dq2, dkr, dvr = block.attention_bwd(do, q, kr, vr)
    np.testing.assert_allclose(dq, dq2, rtol=1e-13)
    np.testing.assert_allclose(dk, dkr.reshape(bsz, seq, 2, 3, hd).sum(3), rtol=1e-12)
    np.testing.assert_allclose(dv, dvr.reshape(bsz, seq, 2, 3, hd).sum(3), rtol=1e-12)


def test_attention_bwd_finite_differences():
    bsz, seq, hq, hkv, hd = 1, 5, 4, 2, 4
    q = rng.standard_normal((bsz, seq, hq, hd))
    k = rng.standard_normal((bsz, seq, hkv, hd))
    v = rng.standard_normal((bsz, seq, hkv, hd))
    w = rng.standard_normal((bsz, seq, hq, hd))

    def f():
        return float(np.sum(w * block.attention_fwd(q, k, v)))
    dq, dk, dv = block.attention_bwd(w, q, k, v)
    assert _rel(dq, _fd_grad(f, q)) < 1e-8
    assert _rel(dk, _fd_grad(f, k)) < 1e-8
    assert _rel(dv, _fd_grad(f, v)) < 1e-8


# ------------------------------------------------------------------ SwiGLU --
def test_silu_and_its_derivative():
    z = np.linspace(-8, 8, 41)
    np.testing.assert_allclose(block.silu(z), z / (1 + np.exp(-z)), rtol=1e-15)
    h = 1e-6
    fd = (block.silu(z + h) - block.silu(z - h)) / (2 * h)
    np.testing.assert_allclose(block.silu_grad(z), fd, rtol=1e-8, atol=1e-10)
    assert block.silu(np.array(0.0)) == 0.0


def test_swiglu_bwd_finite_differences():
    a = rng.standard_normal((3, 5))
    b = rng.standard_normal((3, 5))
    w = rng.standard_normal((3, 5))

    def f():
        return float(np.sum(w * block.swiglu_fwd(a, b)))
    da, db = block.swiglu_bwd(w, a, b)
    assert _rel(da, _fd_grad(f, a)) < 1e-8
    assert _rel(db, _fd_grad(f, b)) < 1e-8


# ----------------------------------------------------------- Cross-entropy --
def test_ce_zero_logits_is_ln_vocab():
    t, v = 6, 1024
    labels = rng.integers(0, v, size=t)
    loss, dl = block.cross_entropy(np.zeros((t, v)), labels)
    assert loss == pytest.approx(6.931471805599453, abs=1e-15)
    onehot = np.zeros((t, v))
    onehot[np.arange(t), labels] = 1
    np.testing.assert_allclose(dl, (1.0 / v - onehot) / t, rtol=1e-14, atol=1e-18)


def test_ce_matches_torch_and_fd():
    t, v = 5, 13
    logits = rng.standard_normal((t, v)) * 3
    labels = rng.integers(0, v, size=t)
    loss, dl = block.cross_entropy(logits, labels)
    tl = torch.from_numpy(logits.copy()).requires_grad_(True)
    ref = torch.nn.functional.cross_entropy(tl, torch.from_numpy(labels))
    ref.backward()
    assert loss == pytest.approx(ref.item(), rel=1e-14)
    np.testing.assert_allclose(dl, tl.grad.numpy(), rtol=1e-12, atol=1e-16)
    fd = _fd_grad(lambda: block.cross_entropy(logits, labels)[0], logits)
    assert _rel(dl, fd) < 1e-8


def test_ce_shift_invariance_and_large_logits():
    logits = rng.standard_normal((4, 9))
    labels = np.array([0, 3, 8, 2])
    l1, d1 = block.cross_entropy(logits, labels)
    l2, d2 = block.cross_entropy(logits + 1e4, labels)
    assert l2 == pytest.approx(l1, rel=1e-9)
    np.testing.assert_allclose(d2, d1, rtol=1e-8, atol=1e-14)


def test_linear_bwd_finite_differences():
    x = rng.standard_normal((4, 6))
    w = rng.standard_normal((3, 6))
    c = rng.standard_normal((4, 3))

    def f():
        return float(np.sum(c * block.linear_fwd(x, w)))
    dx, dw = block.linear_bwd(c, x, w)
    assert _rel(dx, _fd_grad(f, x)) < 1e-9
    assert _rel(dw, _fd_grad(f, w)) < 1e-9
