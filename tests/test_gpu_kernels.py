"""Kernel-level parity: each gfx950 kernel (through the C ABI test entries)
against the float64 oracle on the same seeded bf16 inputs, at sizes that span
several tiles with ragged tails.  Bound: normwise relative error <= 1e-2."""
import math

import numpy as np
import pytest

from layer_streaming_amd import synth
from oracle import block
from oracle.bf16 import bf16_bits
from tests.gpu_util import (assert_close, attn_inputs, dev_bits, dev_f16, dev_zeros_bits, host_f16, host_f32, log,
                            widen)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from layer_streaming_amd import mt  # noqa: E402

RNG = np.random.default_rng(1234)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------ GEMM --
GEMM_SHAPES = [(200, 136, 72), (520, 392, 264), (136, 264, 1000), (4096, 8192, 64), (64, 8, 8), (13, 24, 40)]


@pytest.mark.parametrize("layout", [0, 1, 2], ids=["NT", "NN", "TN"])
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_layouts(layout, M, N, K):
    if layout == 2 and M % 8:
        pytest.skip("TN reads A row-contiguous along M: M must be a multiple of 8")
    log(f"gemm layout={layout} M={M} N={N} K={K}")
    a_shape = (M, K) if layout in (0, 1) else (K, M)
    b_shape = (N, K) if layout == 0 else (K, N)
    A = synth.bf16_exact_normal(RNG, a_shape)
    B = synth.bf16_exact_normal(RNG, b_shape)
    opA = A if layout in (0, 1) else A.T
    opB = B.T if layout == 0 else B
    ref = opA.astype(np.float64) @ opB.astype(np.float64)
    dA, dB = dev_bits(A), dev_bits(B)
    dC = dev_zeros_bits((M, N))
    mt.check(mt.lib.mt_k_gemm(layout, 0, dA.data_ptr(), a_shape[1], dB.data_ptr(), b_shape[1], dC.data_ptr(), N,
                              None, 0, None, 0, M, N, K, _stream()), "gemm")
    _sync()
    assert_close(host_f32(dC), ref, "C")


def test_gemm_epilogues():
    M, N, K = 300, 264, 136
    log(f"gemm epilogues M={M} N={N} K={K}")
    A = synth.bf16_exact_normal(RNG, (M, K))
    B = synth.bf16_exact_normal(RNG, (N, K))
    R = synth.bf16_exact_normal(RNG, (M, N))
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    dA, dB, dR = dev_bits(A), dev_bits(B), dev_bits(R)
    s = _stream()
    # residual
    dC = dev_zeros_bits((M, N))
    mt.check(mt.lib.mt_k_gemm(0, 1, dA.data_ptr(), K, dB.data_ptr(), K, dC.data_ptr(), N, dR.data_ptr(), N,
                              None, 0, M, N, K, s))
    _sync()
    assert_close(host_f32(dC), ref + R, "C+R")
    # fp32 out, then fp32 accumulate twice, then bf16 from the fp32 partial
    c32 = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    mt.check(mt.lib.mt_k_gemm(0, 2, dA.data_ptr(), K, dB.data_ptr(), K, c32.data_ptr(), N, None, 0, None, 0,
                              M, N, K, s))
    _sync()
    assert_close(c32.cpu().numpy(), ref, "C f32", tol=1e-5)
    mt.check(mt.lib.mt_k_gemm(0, 3, dA.data_ptr(), K, dB.data_ptr(), K, c32.data_ptr(), N, None, 0, None, 0,
                              M, N, K, s))
    _sync()
    assert_close(c32.cpu().numpy(), 2 * ref, "C f32 += ", tol=1e-5)
    dC2 = dev_zeros_bits((M, N))
    mt.check(mt.lib.mt_k_gemm(0, 4, dA.data_ptr(), K, dB.data_ptr(), K, dC2.data_ptr(), N, None, 0,
                              c32.data_ptr(), N, M, N, K, s))
    _sync()
    assert_close(host_f32(dC2), 3 * ref, "C bf16 from f32 partial")
    # fp32 residual stream: C f32 = acc + R bf16, then C bf16 = acc + R f32
    h32 = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    mt.check(mt.lib.mt_k_gemm(0, 5, dA.data_ptr(), K, dB.data_ptr(), K, h32.data_ptr(), N, dR.data_ptr(), N,
                              None, 0, M, N, K, s))
    _sync()
    assert_close(h32.cpu().numpy(), ref + R, "C f32 = acc + R bf16", tol=1e-5)
    dC3 = dev_zeros_bits((M, N))
    mt.check(mt.lib.mt_k_gemm(0, 6, dA.data_ptr(), K, dB.data_ptr(), K, dC3.data_ptr(), N, h32.data_ptr(), N,
                              None, 0, M, N, K, s))
    _sync()
    assert_close(host_f32(dC3), 2 * ref + R, "C bf16 = acc + R f32")


# The NT kernel's 64-deep form runs when a grid has at least 120 tiles of
# 256 x 256.  These shapes reach it with ragged rows and columns and with k
# ending inside a tile (k-tile counts 1, 2, 3, 4, 16 and 42), with a grid
# smaller than the CU count (3080 x 3000: 156 tiles) and with several rounds
# of tiles (6152 x 5384: 550 tiles, 8200 x 8200: 1089).
GEMM_BIG = [(4104, 4040, 200), (4000, 4100, 1000), (4352, 3848, 72), (4100, 4104, 8), (4096, 4096, 136),
            (4104, 4096, 2632), (3080, 3000, 200), (6152, 5384, 200), (8200, 8200, 72)]


def _elementwise_check(got, ref, A, B, name, K):
    """Every output element within the bound of its own dot product:
    half a bf16 ulp of the result plus fp32 accumulation of K exact products,
    |err| <= 2^-8 |ref| + 4 K 2^-24 ||a_i|| ||b_j|| (Cauchy-Schwarz on the sum
    of |a_ik b_jk|).  A lost or misplaced 8-deep k-chunk, row or column moves
    most of the elements it touches well past it."""
    na = np.linalg.norm(A.astype(np.float64), axis=1)
    nb = np.linalg.norm(B.astype(np.float64), axis=1)
    bound = 2.0 ** -8 * np.abs(ref) + 4.0 * K * 2.0 ** -24 * np.outer(na, nb) + 1e-30
    err = np.abs(np.asarray(got, np.float64) - ref)
    bad = err > bound
    assert not bad.any(), (f"{name}: {int(bad.sum())} elements outside the bound, first at "
                           f"{tuple(int(x) for x in np.argwhere(bad)[0])}")


@pytest.mark.parametrize("M,N,K", GEMM_BIG)
def test_gemm_nt_large_tile_form(M, N, K):
    log(f"gemm NT large-tile form M={M} N={N} K={K}")
    A = synth.bf16_exact_normal(RNG, (M, K))
    B = synth.bf16_exact_normal(RNG, (N, K))
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    dA, dB = dev_bits(A), dev_bits(B)
    dC = dev_zeros_bits((M, N))
    mt.check(mt.lib.mt_k_gemm(0, 0, dA.data_ptr(), K, dB.data_ptr(), K, dC.data_ptr(), N, None, 0, None, 0,
                              M, N, K, _stream()), "gemm")
    _sync()
    got = host_f32(dC)
    assert_close(got, ref, "C")
    _elementwise_check(got, ref, A, B, "C", K)


# NN and TN grids of at least 120 tiles of 256 x 256 read their k-major
# operands straight (transposed fragments from LDS): ragged M, N and K,
# leading dimensions wider than the operands, the backward products' shapes.
KMAJOR_CASES = [(1, 4104, 4040, 200, 24, 8), (2, 4104, 4040, 997, 16, 8), (1, 2056, 7176, 520, 0, 0),
                (2, 3584, 4608, 1000, 0, 0), (2, 4608, 3584, 136, 8, 16)]


@pytest.mark.parametrize("layout,M,N,K,pa,pb", KMAJOR_CASES)
def test_gemm_kmajor_large_tile_form(layout, M, N, K, pa, pb):
    log(f"gemm k-major large-tile form layout={layout} M={M} N={N} K={K} pads {pa},{pb}")
    a_cols = K if layout == 1 else M
    A = synth.bf16_exact_normal(RNG, (M, K + pa) if layout == 1 else (K, M + pa))
    B = synth.bf16_exact_normal(RNG, (K, N + pb))
    opA = A[:, :K] if layout == 1 else A[:, :M].T
    opB = B[:, :N]
    ref = opA.astype(np.float64) @ opB.astype(np.float64)
    dA, dB = dev_bits(A), dev_bits(B)
    dC = dev_zeros_bits((M, N + 4))
    mt.check(mt.lib.mt_k_gemm(layout, 0, dA.data_ptr(), a_cols + pa, dB.data_ptr(), N + pb, dC.data_ptr(), N + 4,
                              None, 0, None, 0, M, N, K, _stream()), "gemm")
    _sync()
    full = host_f32(dC)
    got = full[:, :N]
    assert_close(got, ref, "C")
    _elementwise_check(got, ref, np.ascontiguousarray(opA), np.ascontiguousarray(opB.T), "C", K)
    assert np.all(full[:, N:] == 0), "columns past N written"


def test_gemm_kmajor_head_epilogues():
    """The TN epilogues the vocabulary-chunked head's dW runs on the k-major
    form: fp32 out, fp32 accumulate, bf16 from an fp32 partial."""
    M, N, K = 4104, 3584, 300
    log(f"gemm TN k-major epilogues M={M} N={N} K={K}")
    A = synth.bf16_exact_normal(RNG, (K, M))
    B = synth.bf16_exact_normal(RNG, (K, N))
    ref = A.T.astype(np.float64) @ B.astype(np.float64)
    dA, dB = dev_bits(A), dev_bits(B)
    s = _stream()
    c32 = torch.zeros((M, N), dtype=torch.float32, device="cuda")

    def run(epi, C, acc=None):
        mt.check(mt.lib.mt_k_gemm(2, epi, dA.data_ptr(), M, dB.data_ptr(), N, C.data_ptr(), N, None, 0, acc,
                                  N if acc else 0, M, N, K, s), f"gemm epi {epi}")
        _sync()

    run(2, c32)
    got32 = c32.cpu().numpy()
    assert_close(got32, ref, "C f32", tol=1e-5)
    _elementwise_check(got32, ref, np.ascontiguousarray(A.T), np.ascontiguousarray(B.T), "C f32", K)
    run(3, c32)
    assert_close(c32.cpu().numpy(), 2 * ref, "C f32 += ", tol=1e-5)
    dC = dev_zeros_bits((M, N))
    run(4, dC, acc=c32.data_ptr())
    assert_close(host_f32(dC), 3 * ref, "C bf16 from f32 partial")


@pytest.mark.parametrize("ldc", [4044, 4048])
def test_gemm_nt_large_tile_partial_column_chunk(ldc):
    """bf16 output whose last 8-column chunk is cut by N (N = 4044), with a
    leading dimension that does (4048) and does not (4044) allow 16-byte
    stores; columns from N to ldc stay untouched."""
    M, N, K = 4104, 4044, 136
    log(f"gemm NT large-tile partial chunk M={M} N={N} K={K} ldc={ldc}")
    A = synth.bf16_exact_normal(RNG, (M, K))
    B = synth.bf16_exact_normal(RNG, (N, K))
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    dA, dB = dev_bits(A), dev_bits(B)
    dC = dev_zeros_bits((M, ldc))
    mt.check(mt.lib.mt_k_gemm(0, 0, dA.data_ptr(), K, dB.data_ptr(), K, dC.data_ptr(), ldc, None, 0, None, 0,
                              M, N, K, _stream()), "gemm")
    _sync()
    full = host_f32(dC)
    got = full[:, :N]
    assert_close(got, ref, "C")
    _elementwise_check(got, ref, A, B, "C", K)
    assert np.all(full[:, N:] == 0), "columns past N written"


def test_gemm_nt_large_tile_epilogues():
    """Every epilogue of the 64-deep form on one ragged shape (partial last
    k-tile, partial row and column tiles), with leading dimensions wider than
    the operands."""
    M, N, K = 4104, 4040, 200
    lda, ldb, ldc = K + 24, K + 8, N + 12
    log(f"gemm NT large-tile epilogues M={M} N={N} K={K}")
    A = synth.bf16_exact_normal(RNG, (M, lda))
    B = synth.bf16_exact_normal(RNG, (N, ldb))
    R = synth.bf16_exact_normal(RNG, (M, ldc))
    ref = A[:, :K].astype(np.float64) @ B[:, :K].astype(np.float64).T
    dA, dB, dR = dev_bits(A), dev_bits(B), dev_bits(R)
    s = _stream()
    Rv = R[:, :N].astype(np.float64)

    def run(epi, C, Rp=None, ldr=0, acc=None):
        mt.check(mt.lib.mt_k_gemm(0, epi, dA.data_ptr(), lda, dB.data_ptr(), ldb, C.data_ptr(), ldc,
                                  Rp, ldr, acc, ldc if acc else 0, M, N, K, s), f"gemm epi {epi}")
        _sync()

    dC = dev_zeros_bits((M, ldc))
    run(1, dC, dR.data_ptr(), ldc)
    got = host_f32(dC)[:, :N]
    assert_close(got, ref + Rv, "C+R")
    _elementwise_check(got, ref + Rv, A[:, :K], B[:, :K], "C+R", K)
    assert np.all(host_f32(dC)[:, N:] == 0), "C+R: columns past N written"
    c32 = torch.zeros((M, ldc), dtype=torch.float32, device="cuda")
    run(2, c32)
    got32 = c32.cpu().numpy()[:, :N]
    assert_close(got32, ref, "C f32", tol=1e-5)
    _elementwise_check(got32, ref, A[:, :K], B[:, :K], "C f32", K)
    run(3, c32)
    assert_close(c32.cpu().numpy()[:, :N], 2 * ref, "C f32 += ", tol=1e-5)
    dC2 = dev_zeros_bits((M, ldc))
    run(4, dC2, acc=c32.data_ptr())
    assert_close(host_f32(dC2)[:, :N], 3 * ref, "C bf16 from f32 partial")
    h32 = torch.zeros((M, ldc), dtype=torch.float32, device="cuda")
    run(5, h32, dR.data_ptr(), ldc)
    assert_close(h32.cpu().numpy()[:, :N], ref + Rv, "C f32 = acc + R bf16", tol=1e-5)
    dC3 = dev_zeros_bits((M, ldc))
    run(6, dC3, h32.data_ptr(), ldc)
    assert_close(host_f32(dC3)[:, :N], 2 * ref + Rv, "C bf16 = acc + R f32")
    # fp16 operands
    A16 = RNG.standard_normal((M, lda)).astype(np.float16)
    B16 = (0.02 * RNG.standard_normal((N, ldb))).astype(np.float16)
    dA16, dB16 = dev_f16(A16), dev_f16(B16)
    c16 = torch.zeros((M, ldc), dtype=torch.float32, device="cuda")
    mt.check(mt.lib.mt_k_gemm(0, 7, dA16.data_ptr(), lda, dB16.data_ptr(), ldb, c16.data_ptr(), ldc, None, 0,
                              None, 0, M, N, K, s), "gemm f16")
    _sync()
    ref16 = A16[:, :K].astype(np.float64) @ B16[:, :K].astype(np.float64).T
    assert_close(c16.cpu().numpy()[:, :N], ref16, "C f16 operands", tol=1e-5)
    # fp16 operands with the bf16 residual (the O product of the attention)
    c16r = torch.zeros((M, ldc), dtype=torch.float32, device="cuda")
    mt.check(mt.lib.mt_k_gemm(0, 8, dA16.data_ptr(), lda, dB16.data_ptr(), ldb, c16r.data_ptr(), ldc, dR.data_ptr(),
                              ldc, None, 0, M, N, K, s), "gemm f16 + resid")
    _sync()
    assert_close(c16r.cpu().numpy()[:, :N], ref16 + Rv, "C f16 operands + R", tol=1e-5)


def test_gemm_rejects_misaligned_shapes():
    A = dev_zeros_bits((16, 16))
    r = mt.lib.mt_k_gemm(0, 0, A.data_ptr(), 12, A.data_ptr(), 16, A.data_ptr(), 16, None, 0, None, 0,
                         16, 16, 12, _stream())
    assert r == mt.MT_E_INVAL


@pytest.mark.parametrize("M,N,K", [(200, 136, 72), (520, 4608, 264), (8192, 1536, 512)])
def test_gemm_f16_operands(M, N, K):
    """Epilogue 7: fp16 operands (the QKV projection of the logit path), f32 out."""
    log(f"gemm f16 M={M} N={N} K={K}")
    A = RNG.standard_normal((M, K)).astype(np.float16)
    B = (0.02 * RNG.standard_normal((N, K))).astype(np.float16)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    dA, dB = dev_f16(A), dev_f16(B)
    dC = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    mt.check(mt.lib.mt_k_gemm(0, 7, dA.data_ptr(), K, dB.data_ptr(), K, dC.data_ptr(), N, None, 0, None, 0,
                              M, N, K, _stream()), "gemm f16")
    _sync()
    assert_close(dC.cpu().numpy(), ref, "C", tol=1e-5)
    r = mt.lib.mt_k_gemm(1, 7, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N, None, 0, None, 0,
                         M, N, K, _stream())
    assert r == mt.MT_E_INVAL
    # epilogue 8: the same with a bf16 residual (ragged N exercises the
    # element-wise tail of the residual read)
    R = synth.bf16_exact_normal(RNG, (M, N))
    dR = dev_bits(R)
    dC8 = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    mt.check(mt.lib.mt_k_gemm(0, 8, dA.data_ptr(), K, dB.data_ptr(), K, dC8.data_ptr(), N, dR.data_ptr(), N,
                              None, 0, M, N, K, _stream()), "gemm f16 + resid")
    _sync()
    assert_close(dC8.cpu().numpy(), ref + R, "C + R", tol=1e-5)
    assert mt.lib.mt_k_gemm(0, 8, dA.data_ptr(), K, dB.data_ptr(), K, dC8.data_ptr(), N, None, 0, None, 0,
                            M, N, K, _stream()) == mt.MT_E_INVAL  # no residual


# The tail split: the tiles of the last, partial round of 256 x 256 tiles run
# as several blocks over consecutive K ranges whose fp32 partials a second
# kernel adds in split order before the epilogue.  Forced split counts, on
# grids with whole rounds before the tail (306 and 272 tiles: 256 whole) and
# without (156 tiles: every tile split), ragged M, N and K (a last k-range
# shorter than the others), every layout.  Checked element by element against
# the float64 product, bit for bit against itself (deterministic), and bit for
# bit against the unsplit product outside the tail tiles.
def _tile_coords(pid, tiles_m, tiles_n, group=8):
    per_group = group * tiles_n
    first_m = (pid // per_group) * group
    gsz = min(tiles_m - first_m, group)
    return first_m + (pid % per_group) % gsz, (pid % per_group) // gsz


def _tail_mask(M, N, n_full):
    tm, tn = (M + 255) // 256, (N + 255) // 256
    mask = np.zeros((M, N), bool)
    for pid in range(n_full, tm * tn):
        i, j = _tile_coords(pid, tm, tn)
        mask[i * 256:(i + 1) * 256, j * 256:(j + 1) * 256] = True
    return mask


SPLIT_CASES = [(0, 4104, 4360, 520, 3), (0, 3080, 3000, 1000, 2), (1, 4104, 4360, 1000, 5), (2, 4104, 4040, 997, 4),
               (2, 3584, 3584, 1032, 7), (1, 4104, 4360, 200, 16)]


@pytest.mark.parametrize("layout,M,N,K,splits", SPLIT_CASES)
def test_gemm_tail_split(layout, M, N, K, splits):
    log(f"gemm tail split layout={layout} M={M} N={N} K={K} splits={splits}")
    a_shape = (M, K) if layout in (0, 1) else (K, M)
    b_shape = (N, K) if layout == 0 else (K, N)
    A = synth.bf16_exact_normal(RNG, a_shape)
    B = synth.bf16_exact_normal(RNG, b_shape)
    opA = A if layout in (0, 1) else A.T
    opB = B.T if layout == 0 else B
    ref = opA.astype(np.float64) @ opB.astype(np.float64)
    dA, dB = dev_bits(A), dev_bits(B)
    tiles = ((M + 255) // 256) * ((N + 255) // 256)
    n_full = (tiles // 256) * 256
    nk = (K + 63) // 64
    kper = -(-nk // splits)
    eff = -(-nk // kper)
    ws = torch.empty((tiles - n_full) * eff * 65536, dtype=torch.float32, device="cuda")

    def run(sp):
        dC = dev_zeros_bits((M, N))
        mt.check(mt.lib.mt_k_gemm_split(layout, 0, dA.data_ptr(), a_shape[1], dB.data_ptr(), b_shape[1],
                                        dC.data_ptr(), N, None, 0, None, 0, M, N, K, ws.data_ptr(),
                                        ws.numel() * 4, sp, _stream()), "gemm_split")
        _sync()
        return dC.cpu().numpy()

    got = run(splits)
    again = run(splits)
    plain = run(1)
    gotf = widen(got.view(np.uint16))
    assert_close(gotf, ref, "C split")
    _elementwise_check(gotf, ref, np.ascontiguousarray(opA), np.ascontiguousarray(opB.T), "C split", K)
    assert np.array_equal(got, again), "split product not deterministic"
    outside = ~_tail_mask(M, N, n_full)
    assert np.array_equal(got[outside], plain[outside]), "whole tiles changed by the split"
    assert not np.array_equal(got, plain), "split not taken"


def test_gemm_tail_split_epilogues():
    """The fixup kernel's epilogues: fp32 out and accumulate, bf16 from an fp32
    partial, the residual forms of the forward products, fp16 operands."""
    M, N, K = 4104, 4040, 600
    ldc = N + 12
    log(f"gemm tail split epilogues M={M} N={N} K={K}")
    A = synth.bf16_exact_normal(RNG, (M, K))
    B = synth.bf16_exact_normal(RNG, (N, K))
    R = synth.bf16_exact_normal(RNG, (M, ldc))
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    Rv = R[:, :N].astype(np.float64)
    dA, dB, dR = dev_bits(A), dev_bits(B), dev_bits(R)
    ws = torch.empty(16 * 3 * 65536, dtype=torch.float32, device="cuda")
    s = _stream()

    def run(epi, C, Rp=None, ldr=0, acc=None, a=dA, b=dB):
        mt.check(mt.lib.mt_k_gemm_split(0, epi, a.data_ptr(), K, b.data_ptr(), K, C.data_ptr(), ldc, Rp, ldr, acc,
                                        ldc if acc else 0, M, N, K, ws.data_ptr(), ws.numel() * 4, 3, s),
                 f"gemm split epi {epi}")
        _sync()

    dC = dev_zeros_bits((M, ldc))
    run(1, dC, dR.data_ptr(), ldc)
    assert_close(host_f32(dC)[:, :N], ref + Rv, "C+R")
    assert np.all(host_f32(dC)[:, N:] == 0), "columns past N written"
    c32 = torch.zeros((M, ldc), dtype=torch.float32, device="cuda")
    run(2, c32)
    got32 = c32.cpu().numpy()[:, :N]
    assert_close(got32, ref, "C f32", tol=1e-5)
    _elementwise_check(got32, ref, A, B, "C f32", K)
    run(3, c32)
    assert_close(c32.cpu().numpy()[:, :N], 2 * ref, "C f32 += ", tol=1e-5)
    dC2 = dev_zeros_bits((M, ldc))
    run(4, dC2, acc=c32.data_ptr())
    assert_close(host_f32(dC2)[:, :N], 3 * ref, "C bf16 from f32 partial")
    h32 = torch.zeros((M, ldc), dtype=torch.float32, device="cuda")
    run(5, h32, dR.data_ptr(), ldc)
    assert_close(h32.cpu().numpy()[:, :N], ref + Rv, "C f32 = acc + R bf16", tol=1e-5)
    dC3 = dev_zeros_bits((M, ldc))
    run(6, dC3, h32.data_ptr(), ldc)
    assert_close(host_f32(dC3)[:, :N], 2 * ref + Rv, "C bf16 = acc + R f32")
    A16 = RNG.standard_normal((M, K)).astype(np.float16)
    B16 = (0.02 * RNG.standard_normal((N, K))).astype(np.float16)
    dA16, dB16 = dev_f16(A16), dev_f16(B16)
    ref16 = A16.astype(np.float64) @ B16.astype(np.float64).T
    c16 = torch.zeros((M, ldc), dtype=torch.float32, device="cuda")
    run(7, c16, a=dA16, b=dB16)
    assert_close(c16.cpu().numpy()[:, :N], ref16, "C f16 operands", tol=1e-5)
    c16r = torch.zeros((M, ldc), dtype=torch.float32, device="cuda")
    run(8, c16r, dR.data_ptr(), ldc, a=dA16, b=dB16)
    assert_close(c16r.cpu().numpy()[:, :N], ref16 + Rv, "C f16 operands + R", tol=1e-5)


def test_gemm_tail_split_kmajor_accumulate():
    """The split k-major forms with the accumulating epilogues the chunked LM
    head runs: NN with fp32 out then fp32 accumulate (dX over vocabulary
    chunks), TN with fp32 accumulate and bf16 from an fp32 partial (dE_out)."""
    s = _stream()
    M, N, K = 4104, 4360, 1000       # NN: 17 x 18 = 306 tiles, 50 split
    log(f"gemm tail split NN accumulate M={M} N={N} K={K}")
    A = synth.bf16_exact_normal(RNG, (M, K))
    B = synth.bf16_exact_normal(RNG, (K, N))
    ref = A.astype(np.float64) @ B.astype(np.float64)
    dA, dB = dev_bits(A), dev_bits(B)
    ws = torch.empty(50 * 4 * 65536, dtype=torch.float32, device="cuda")
    c32 = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    for epi in (2, 3):
        mt.check(mt.lib.mt_k_gemm_split(1, epi, dA.data_ptr(), K, dB.data_ptr(), N, c32.data_ptr(), N, None, 0, None,
                                        0, M, N, K, ws.data_ptr(), ws.numel() * 4, 4, s), f"gemm split NN epi {epi}")
    _sync()
    assert_close(c32.cpu().numpy(), 2 * ref, "NN C f32 += (split)", tol=1e-5)
    M2, N2, K2 = 4104, 4040, 997     # TN: 17 x 16 = 272 tiles, 16 split
    log(f"gemm tail split TN accumulate M={M2} N={N2} K={K2}")
    A2 = synth.bf16_exact_normal(RNG, (K2, M2))
    B2 = synth.bf16_exact_normal(RNG, (K2, N2))
    ref2 = A2.T.astype(np.float64) @ B2.astype(np.float64)
    dA2, dB2 = dev_bits(A2), dev_bits(B2)
    acc = torch.zeros((M2, N2), dtype=torch.float32, device="cuda")
    mt.check(mt.lib.mt_k_gemm_split(2, 2, dA2.data_ptr(), M2, dB2.data_ptr(), N2, acc.data_ptr(), N2, None, 0, None, 0,
                                    M2, N2, K2, ws.data_ptr(), ws.numel() * 4, 3, s), "gemm split TN f32")
    mt.check(mt.lib.mt_k_gemm_split(2, 3, dA2.data_ptr(), M2, dB2.data_ptr(), N2, acc.data_ptr(), N2, None, 0, None, 0,
                                    M2, N2, K2, ws.data_ptr(), ws.numel() * 4, 3, s), "gemm split TN f32 +=")
    dC = dev_zeros_bits((M2, N2))
    mt.check(mt.lib.mt_k_gemm_split(2, 4, dA2.data_ptr(), M2, dB2.data_ptr(), N2, dC.data_ptr(), N2, None, 0,
                                    acc.data_ptr(), N2, M2, N2, K2, ws.data_ptr(), ws.numel() * 4, 3, s),
             "gemm split TN bf16 from f32")
    _sync()
    assert_close(acc.cpu().numpy(), 2 * ref2, "TN C f32 += (split)", tol=1e-5)
    assert_close(host_f32(dC), 3 * ref2, "TN C bf16 from f32 partial (split)")


def test_gemm_tail_split_refuses_small_scratch():
    M, N, K = 3080, 3000, 1000
    dA = dev_zeros_bits((M, K))
    dB = dev_zeros_bits((N, K))
    dC = dev_zeros_bits((M, N))
    ws = torch.empty(65536, dtype=torch.float32, device="cuda")
    rc = mt.lib.mt_k_gemm_split(0, 0, dA.data_ptr(), K, dB.data_ptr(), K, dC.data_ptr(), N, None, 0, None, 0,
                                M, N, K, ws.data_ptr(), ws.numel() * 4, 2, _stream())
    assert rc == mt.MT_E_INVAL


# The attention backward's scale from its producers (the step's form): the
# O dX product's epilogue adds max |dO| of the values it stores, the
# recompute's rotation max |v| of the fp16 v it stores, each into 16 partial
# maxima (float bit patterns) one 256-byte line apart.
def _amax_words():
    return torch.zeros(2048, dtype=torch.int32, device="cuda")


def _partial_max(words, first):
    w = words.cpu().numpy().view(np.uint32)[(16 * first + np.arange(16)) * 64]
    return float(np.max(w.view(np.float32)))


@pytest.mark.parametrize("layout,M,N,K,std", [(1, 4104, 3592, 520, 1.0), (1, 8192, 3584, 3584, 1e-4),
                                              (0, 4104, 4044, 200, 30.0), (0, 200, 136, 72, 1.0)])
def test_gemm_amax_epilogue(layout, M, N, K, std):
    """bf16 output bit-identical to the plain epilogue; max |C| exact (the max
    over the stored bf16 values, ragged columns included, none past N): NN on
    the 64-deep form (the O dX shape among them), NT with a last 8-column chunk
    cut by N and rows not 16-byte aligned (the 4-column stores), NT on the
    32-deep form of small grids."""
    log(f"gemm with max |C| layout={layout} M={M} N={N} K={K} std={std}")
    a_shape = (M, K)
    b_shape = (N, K) if layout == 0 else (K, N)
    A = synth.bf16_exact_normal(RNG, a_shape, std=std)
    B = synth.bf16_exact_normal(RNG, b_shape)
    dA, dB = dev_bits(A), dev_bits(B)
    ldc = N + 8
    C1 = torch.full((M, ldc), 0x7F80, dtype=torch.int16, device="cuda")   # +inf past N: must stay out of the max
    C0 = dev_zeros_bits((M, ldc))
    words = _amax_words()
    s = _stream()
    mt.check(mt.lib.mt_k_gemm_amax(layout, dA.data_ptr(), K, dB.data_ptr(), b_shape[1], C1.data_ptr(), ldc, M, N, K,
                                   words.data_ptr(), s), "gemm_amax")
    mt.check(mt.lib.mt_k_gemm(layout, 0, dA.data_ptr(), K, dB.data_ptr(), b_shape[1], C0.data_ptr(), ldc, None, 0,
                              None, 0, M, N, K, s), "gemm")
    _sync()
    c1 = C1.cpu().numpy()
    assert np.array_equal(c1[:, :N], C0.cpu().numpy()[:, :N]), "values differ from the plain epilogue"
    want = float(np.max(np.abs(widen(c1[:, :N].view(np.uint16)))))
    assert _partial_max(words, 0) == want
    assert _partial_max(words, 1) == 0.0, "|v| words touched"
    if layout == 1:  # NN grids below 120 tiles of 256 x 256 are refused (no direct form takes them)
        assert mt.lib.mt_k_gemm_amax(layout, dA.data_ptr(), K, dB.data_ptr(), b_shape[1], C1.data_ptr(), ldc, 200,
                                     136, K, words.data_ptr(), s) == mt.MT_E_INVAL


@pytest.mark.parametrize("hd,S", [(128, 1024), (64, 100)])
def test_qkv_rope_cvt_vmax(hd, S):
    """max |v| over the fp16 v heads the rotation stores, exactly; fp16 output
    bit-identical to the plain entry."""
    hq, hkv, B = 4, 2, 3
    log(f"qkv_rope_cvt with max |v| hd={hd} S={S}")
    ld = (hq + 2 * hkv) * hd
    T = B * S
    x = RNG.standard_normal((T, ld)).astype(np.float32)
    x[:, (hq + hkv) * hd:] *= 3.0
    dx = torch.from_numpy(x).cuda()
    out = dev_zeros_bits((T, ld))
    out0 = dev_zeros_bits((T, ld))
    tab = torch.zeros(S * hd, dtype=torch.float32, device="cuda")
    words = _amax_words()
    s = _stream()
    mt.check(mt.lib.mt_k_qkv_rope_cvt_vmax(dx.data_ptr(), ld, out.data_ptr(), ld, tab.data_ptr(), T, S, hq + hkv,
                                           hq + 2 * hkv, hd, 10000.0, None, words.data_ptr(), s))
    mt.check(mt.lib.mt_k_qkv_rope_cvt(dx.data_ptr(), ld, out0.data_ptr(), ld, None, 0, tab.data_ptr(), T, S,
                                      hq + hkv, hq + 2 * hkv, hd, 10000.0, None, s))
    _sync()
    assert torch.equal(out, out0)
    v = out.cpu().numpy().view(np.uint16)[:, (hq + hkv) * hd:].view(np.float16).astype(np.float32)
    assert _partial_max(words, 1) == float(np.max(np.abs(v)))
    assert _partial_max(words, 0) == 0.0, "|dO| words touched"


# --------------------------------------------------------------- RMSNorm --
@pytest.mark.parametrize("T,d,x_f32", [(37, 256, 0), (130, 3584, 0), (9, 8192, 0), (1, 64, 0), (130, 3584, 1),
                                       (21, 256, 1)])
def test_rmsnorm_fwd_bwd(T, d, x_f32):
    log(f"rmsnorm T={T} d={d} x_f32={x_f32}")
    eps = 1e-6
    if x_f32:
        x = RNG.standard_normal((T, d)).astype(np.float32)
        dx_ = torch.from_numpy(x).cuda()
    else:
        x = synth.bf16_exact_normal(RNG, (T, d))
        dx_ = dev_bits(x)
    g = synth.bf16_exact_normal(RNG, (d,), std=0.2, mean=1.0)
    dn = synth.bf16_exact_normal(RNG, (T, d))
    res = synth.bf16_exact_normal(RNG, (T, d))
    n_, dg_, nh_ = dev_zeros_bits((T, d)), dev_zeros_bits((d,)), dev_zeros_bits((T, d))
    rstd = torch.zeros(T, dtype=torch.float32, device="cuda")
    dgam, ddn, dres = dev_bits(g), dev_bits(dn), dev_bits(res)
    s = _stream()
    ovf = torch.zeros(4, dtype=torch.int32, device="cuda")
    mt.check(mt.lib.mt_k_rmsnorm_fwd(dx_.data_ptr(), x_f32, dgam.data_ptr(), n_.data_ptr(), nh_.data_ptr(),
                                     rstd.data_ptr(), T, d, eps, ovf.data_ptr(), s))
    scratch = torch.zeros(int(mt.lib.mt_k_rmsnorm_bwd_scratch_elems(T, d)), dtype=torch.float32, device="cuda")
    ddx = dev_zeros_bits((T, d))
    mt.check(mt.lib.mt_k_rmsnorm_bwd(ddn.data_ptr(), dx_.data_ptr(), x_f32, dgam.data_ptr(), rstd.data_ptr(),
                                     dres.data_ptr(), ddx.data_ptr(), dg_.data_ptr(), scratch.data_ptr(), T, d, s))
    _sync()
    xd = x.astype(np.float64)
    n_ref, r_ref = block.rmsnorm_fwd(xd, g.astype(np.float64), eps)
    assert_close(host_f32(n_), n_ref, "n")
    assert_close(host_f16(nh_), n_ref, "n (fp16)", tol=1e-3)
    assert ovf[0].item() == 0
    assert_close(rstd.cpu().numpy(), r_ref, "rstd", tol=1e-5)
    dx_ref, dg_ref = block.rmsnorm_bwd(dn.astype(np.float64), xd, g.astype(np.float64), r_ref)
    assert_close(host_f32(ddx), dx_ref + res, "dx")
    assert_close(host_f32(dg_), dg_ref, "dgamma")


# ------------------------------------------------------------------ RoPE --
@pytest.mark.parametrize("hd", [64, 128])
def test_rope_fwd_bwd(hd):
    B, S, hq, hkv = 2, 100, 4, 2
    log(f"rope hd={hd}")
    ld = (hq + 2 * hkv) * hd
    T = B * S
    qkv = synth.bf16_exact_normal(RNG, (T, ld))
    dq = dev_bits(qkv)
    tab = torch.zeros(S * hd // 2 * 2, dtype=torch.float32, device="cuda")
    mt.check(mt.lib.mt_k_rope(dq.data_ptr(), ld, tab.data_ptr(), T, S, hq + hkv, hd, 10000.0, 1, _stream()))
    _sync()
    got = host_f32(dq)
    rot = qkv[:, :(hq + hkv) * hd].astype(np.float64).reshape(B, S, hq + hkv, hd)
    ref = block.rope_fwd(rot, 10000.0).reshape(T, -1)
    assert_close(got[:, :(hq + hkv) * hd], ref, "rope fwd")
    np.testing.assert_array_equal(got[:, (hq + hkv) * hd:], qkv[:, (hq + hkv) * hd:])
    dq2 = dev_bits(qkv)
    mt.check(mt.lib.mt_k_rope(dq2.data_ptr(), ld, tab.data_ptr(), T, S, hq + hkv, hd, 10000.0, -1, _stream()))
    _sync()
    ref_b = block.rope_bwd(rot, 10000.0).reshape(T, -1)
    assert_close(host_f32(dq2)[:, :(hq + hkv) * hd], ref_b, "rope bwd")


def test_rope_long_positions():
    """Angles up to 131071 rad: the table is computed in float64."""
    B, S, h, hd = 1, 131072, 1, 128
    log("rope long S=131072")
    qkv = synth.bf16_exact_normal(RNG, (S, 3 * hd))
    dq = dev_bits(qkv)
    tab = torch.zeros(S * hd, dtype=torch.float32, device="cuda")
    mt.check(mt.lib.mt_k_rope(dq.data_ptr(), 3 * hd, tab.data_ptr(), S, S, 1, hd, 10000.0, 1, _stream()))
    _sync()
    got = host_f32(dq)[:, :hd]
    ref = block.rope_fwd(qkv[:, :hd].astype(np.float64).reshape(1, S, 1, hd), 10000.0).reshape(S, hd)
    assert_close(got, ref, "rope fwd long")


@pytest.mark.parametrize("hd,S", [(64, 100), (128, 100), (128, 131072)])
def test_qkv_rope_cvt(hd, S):
    """Forward RoPE on the f32 projection: q, k rotated, every head stored as
    fp16 (v bit-exact against round-to-nearest-even) and, in a second buffer,
    as bf16 (v bit-exact)."""
    hq, hkv = (4, 2) if S < 1000 else (1, 1)
    B = 2 if S < 1000 else 1
    log(f"qkv_rope_cvt hd={hd} S={S}")
    ld = (hq + 2 * hkv) * hd
    T = B * S
    x = RNG.standard_normal((T, ld)).astype(np.float32)
    dx = torch.from_numpy(x).cuda()
    out = dev_zeros_bits((T, ld))
    nr = (hq + hkv) * hd
    outb = dev_zeros_bits((T, ld))
    tab = torch.zeros(S * hd, dtype=torch.float32, device="cuda")
    ovf = torch.zeros(4, dtype=torch.int32, device="cuda")
    mt.check(mt.lib.mt_k_qkv_rope_cvt(dx.data_ptr(), ld, out.data_ptr(), ld, outb.data_ptr(), ld, tab.data_ptr(), T,
                                      S, hq + hkv, hq + 2 * hkv, hd, 10000.0, ovf.data_ptr(), _stream()))
    _sync()
    got_qk = host_f16(out)[:, :nr]
    rot = x[:, :nr].astype(np.float64).reshape(B, S, hq + hkv, hd)
    ref = block.rope_fwd(rot, 10000.0).reshape(T, nr)
    assert_close(got_qk, ref, "q, k (fp16)", tol=1e-3)
    got_v = out.cpu().numpy().view(np.uint16)[:, nr:]
    np.testing.assert_array_equal(got_v, x[:, nr:].astype(np.float16).view(np.uint16))
    # the bf16 copy is the bf16 rounding of the fp16 values, bit for bit
    np.testing.assert_array_equal(outb.cpu().numpy().view(np.uint16), bf16_bits(host_f16(out)))
    assert ovf[0].item() == 0
    # without the bf16 copy: same fp16 output
    out2 = dev_zeros_bits((T, ld))
    mt.check(mt.lib.mt_k_qkv_rope_cvt(dx.data_ptr(), ld, out2.data_ptr(), ld, None, 0, tab.data_ptr(), T, S,
                                      hq + hkv, hq + 2 * hkv, hd, 10000.0, None, _stream()))
    _sync()
    assert torch.equal(out, out2)
    # a bf16 copy narrower than every head is refused
    assert mt.lib.mt_k_qkv_rope_cvt(dx.data_ptr(), ld, out2.data_ptr(), ld, outb.data_ptr(), nr, tab.data_ptr(), T,
                                    S, hq + hkv, hq + 2 * hkv, hd, 10000.0, None, _stream()) == mt.MT_E_INVAL


# ------------------------------------------------------ fp16 range guard --
def _f16_sat_ref(x):
    """The guard's definition: |x| < 65520 rounds to nearest even (numpy's
    float16 cast), anything else saturates to +-65504 and counts; NaN stays
    NaN and counts."""
    x = np.asarray(x, np.float32)
    over = ~(np.abs(x) < 65520.0)
    y = np.where(over & ~np.isnan(x), np.copysign(np.float32(65504.0), x), x).astype(np.float16)
    return y, int(over.sum())


def test_fp16_range_guard_conversion():
    """bf16 -> fp16 of the weights of the fp16 products: values near and past
    the fp16 maximum, infinities, NaN, fp16 subnormals and values below them,
    against the guard's definition bit for bit, with the exact count."""
    edge = np.array([65504.0, -65504.0, 65280.0, 65536.0, -65536.0, 1e5, -3e38, np.inf, -np.inf, np.nan,
                     2.0 ** -14, 2.0 ** -15, 3 * 2.0 ** -24, 2.0 ** -25, 2.0 ** -26, -(2.0 ** -20), 0.0, -0.0,
                     1.0, 0.02], np.float32)
    x = np.concatenate([edge, synth.bf16_exact_normal(RNG, (4076,), std=3e4)])
    x = widen(bf16_bits(x))  # exactly bf16
    ref, n_over = _f16_sat_ref(x)
    dx = torch.from_numpy(bf16_bits(x).view(np.int16)).cuda()
    dy = dev_zeros_bits(x.shape)
    ovf = torch.zeros(4, dtype=torch.int32, device="cuda")
    mt.check(mt.lib.mt_k_bf16_to_f16(dx.data_ptr(), dy.data_ptr(), x.size, ovf.data_ptr(), _stream()))
    _sync()
    got = dy.cpu().numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref.view(np.uint16)[~nan])
    assert np.all(np.isnan(got[nan].view(np.float16)))
    assert ovf[0].item() == n_over and n_over > 5


def test_fp16_range_guard_norm_and_rope():
    """The fp16 copy of the norm output and the RoPE conversion saturate and
    count too: a gain of 2^20 drives n past the fp16 range."""
    T, d = 40, 256
    x = synth.bf16_exact_normal(RNG, (T, d))
    g = np.full(d, 2.0 ** 20, np.float32)
    dx_, dg = dev_bits(x), dev_bits(g)
    n_, nh_ = dev_zeros_bits((T, d)), dev_zeros_bits((T, d))
    rstd = torch.zeros(T, dtype=torch.float32, device="cuda")
    ovf = torch.zeros(4, dtype=torch.int32, device="cuda")
    mt.check(mt.lib.mt_k_rmsnorm_fwd(dx_.data_ptr(), 0, dg.data_ptr(), n_.data_ptr(), nh_.data_ptr(),
                                     rstd.data_ptr(), T, d, 1e-6, ovf.data_ptr(), _stream()))
    _sync()
    n_ref, _ = block.rmsnorm_fwd(x.astype(np.float64), g.astype(np.float64), 1e-6)
    got = nh_.cpu().numpy().view(np.float16).astype(np.float64)
    over = np.abs(n_ref) >= 65600.0  # clear of the boundary, where fp32 and fp64 may round apart
    assert np.all(got[over] == np.copysign(65504.0, n_ref[over]))
    assert np.all(np.isfinite(got))
    cnt = int(np.sum(np.abs(n_ref) >= 65520.0))
    assert abs(ovf[0].item() - cnt) <= 2 and cnt > T * d // 2
    # RoPE conversion of an out-of-range projection
    hd, S = 64, T
    ld = 3 * hd
    xp = (RNG.standard_normal((T, ld)) * 1e5).astype(np.float32)
    dxp = torch.from_numpy(xp).cuda()
    out = dev_zeros_bits((T, ld))
    tab = torch.zeros(S * hd, dtype=torch.float32, device="cuda")
    ovf.zero_()
    mt.check(mt.lib.mt_k_qkv_rope_cvt(dxp.data_ptr(), ld, out.data_ptr(), ld, None, 0, tab.data_ptr(), T, S, 2, 3,
                                      hd, 10000.0, ovf.data_ptr(), _stream()))
    _sync()
    h = out.cpu().numpy().view(np.float16)
    assert np.all(np.isfinite(h)) and np.max(np.abs(h)) == 65504.0
    _, cnt_v = _f16_sat_ref(xp[:, 2 * hd:])
    assert ovf[0].item() >= cnt_v > 0


# ---------------------------------------------------------------- SwiGLU --
@pytest.mark.parametrize("T,F", [(50, 688), (7, 18944)])
def test_swiglu_fwd_bwd(T, F):
    log(f"swiglu T={T} F={F}")
    gu = synth.bf16_exact_normal(RNG, (T, 2 * F), std=2.0)
    dm = synth.bf16_exact_normal(RNG, (T, F))
    dgu_, dm_, m_, dgo = dev_bits(gu), dev_bits(dm), dev_zeros_bits((T, F)), dev_zeros_bits((T, 2 * F))
    s = _stream()
    mt.check(mt.lib.mt_k_swiglu_fwd(dgu_.data_ptr(), m_.data_ptr(), T, F, s))
    mt.check(mt.lib.mt_k_swiglu_bwd(dm_.data_ptr(), dgu_.data_ptr(), dgo.data_ptr(), T, F, s))
    _sync()
    a, b = gu[:, :F].astype(np.float64), gu[:, F:].astype(np.float64)
    assert_close(host_f32(m_), block.swiglu_fwd(a, b), "m")
    da, db = block.swiglu_bwd(dm.astype(np.float64), a, b)
    got = host_f32(dgo)
    assert_close(got[:, :F], da, "dgate")
    assert_close(got[:, F:], db, "dup")


# ------------------------------------------------------------- Attention --
ATTN_CASES = [(2, 200, 4, 2, 64), (1, 300, 7, 1, 128), (2, 128, 4, 4, 128), (1, 1, 2, 1, 64),
              (1, 65, 2, 2, 128), (1, 1024, 28, 4, 128)]


@pytest.mark.parametrize("B,S,Hq,Hkv,hd", ATTN_CASES)
@pytest.mark.parametrize("f32_out", [False, True], ids=["bf16-dqk", "f32-dqk"])
@pytest.mark.parametrize("dq_form", [1, 2], ids=["dq-recomputed", "dq-stored-ds"])
def test_attention_fwd_bwd(B, S, Hq, Hkv, hd, f32_out, dq_form):
    """Forward and backward (fp16 products, scaled dO) against the float64
    oracle; dQ and dK written as bf16 into the qkv layout, or as fp32; dQ
    recomputing the scores and dP, or formed from the dS the dK/dV pass
    stored."""
    _attention_case(B, S, Hq, Hkv, hd, 1.0, f32_out, dq_form=dq_form)


@pytest.mark.parametrize("dq_form", [1, 2], ids=["dq-recomputed", "dq-stored-ds"])
def test_attention_sharp_logits(dq_form):
    """q, k with std 2 (logits of std 4): a peaked softmax, where the logit
    path's rounding matters most."""
    _attention_case(1, 700, 8, 2, 128, 2.0, True, dq_form=dq_form)


@pytest.mark.parametrize("do_std", [1e-9, 1e-4, 3e2])
def test_attention_bwd_scale_follows_gradient_size(do_std):
    """The backward's power-of-two scale follows max|dO|: gradients many
    orders of magnitude below fp16's normal range (the loss scale of a long
    sequence) and well above 1 give the same relative accuracy."""
    _attention_case(2, 130, 4, 2, 128, 1.0, True, do_std=do_std)


@pytest.mark.parametrize("B,S,Hq,Hkv,hd,splits,taken", [(1, 300, 7, 1, 128, 1, 1), (1, 300, 7, 1, 128, 3, 3),
                                                         (1, 1024, 28, 4, 128, 1, 1), (2, 200, 4, 2, 64, 1, 1),
                                                         (1, 1024, 28, 4, 128, 0, 7), (2, 200, 4, 2, 64, 0, 2),
                                                         (2, 256, 260, 130, 64, 2, 1)])
def test_attention_dkdv_head_split(B, S, Hq, Hkv, hd, splits, taken):
    """The dK/dV pass with each KV group's query heads split over several
    blocks (fp32 partials added in split order; 3 of 7 heads is uneven) and
    without a split: both against the oracle.  The backward runs twice on
    the same inputs and must repeat bit for bit.  A pass with 512 key-tile
    blocks or more has no partials in its scratch, so a requested split is
    not taken (the last case, 520 blocks)."""
    assert mt.lib.mt_k_attn_dkdv_splits(B, S, Hq, Hkv, hd, splits) == taken
    _attention_case(B, S, Hq, Hkv, hd, 1.0, True, splits=splits, repeat=True)


def _attention_case(B, S, Hq, Hkv, hd, qk_std, f32_out, do_std=1.0, splits=0, dq_form=0, repeat=False):
    log(f"attention B={B} S={S} Hq={Hq} Hkv={Hkv} hd={hd} qk_std={qk_std} f32_out={f32_out} do_std={do_std} "
        f"splits={splits} dq_form={dq_form}")
    T = B * S
    ld = (Hq + 2 * Hkv) * hd
    nq, nr = Hq * hd, (Hq + Hkv) * hd
    qkv, d_qkv, _ = attn_inputs(RNG, T, Hq, Hkv, hd, qk_std)
    dout = synth.bf16_exact_normal(RNG, (T, nq), std=do_std)
    d_do = dev_bits(dout)
    d_o = dev_zeros_bits((T, nq))
    lse = torch.zeros(B * Hq * S, dtype=torch.float32, device="cuda")
    work = torch.zeros(int(mt.lib.mt_k_attn_bwd_work_bytes(B, S, Hq, Hkv, hd)), dtype=torch.uint8, device="cuda")
    d_dqkv = dev_zeros_bits((T, ld))
    dqk32 = torch.zeros((T, nr), dtype=torch.float32, device="cuda") if f32_out else None
    ovf = torch.zeros(4, dtype=torch.int32, device="cuda")
    s = _stream()
    mt.check(mt.lib.mt_k_attn_fwd(d_qkv.data_ptr(), ld, d_o.data_ptr(), nq, lse.data_ptr(), B, S, Hq, Hkv, hd,
                                  ovf.data_ptr(), s))
    mt.check(mt.lib.mt_k_attn_bwd(d_qkv.data_ptr(), ld, d_o.data_ptr(), d_do.data_ptr(), nq, lse.data_ptr(),
                                  work.data_ptr(), d_dqkv.data_ptr(), ld, B, S, Hq, Hkv, hd,
                                  dqk32.data_ptr() if f32_out else None, nr if f32_out else 0, splits, dq_form,
                                  ovf.data_ptr(), s))
    _sync()
    assert ovf[0].item() == 0
    if repeat:
        d_dqkv2 = dev_zeros_bits((T, ld))
        dqk32_2 = torch.zeros((T, nr), dtype=torch.float32, device="cuda") if f32_out else None
        mt.check(mt.lib.mt_k_attn_bwd(d_qkv.data_ptr(), ld, d_o.data_ptr(), d_do.data_ptr(), nq, lse.data_ptr(),
                                      work.data_ptr(), d_dqkv2.data_ptr(), ld, B, S, Hq, Hkv, hd,
                                      dqk32_2.data_ptr() if f32_out else None, nr if f32_out else 0, splits,
                                      dq_form, ovf.data_ptr(), s))
        _sync()
        assert torch.equal(d_dqkv2, d_dqkv)
        if f32_out:
            assert torch.equal(dqk32_2.view(torch.int32), dqk32.view(torch.int32))
    x = qkv.astype(np.float64).reshape(B, S, Hq + 2 * Hkv, hd)
    q, k, v = x[:, :, :Hq], x[:, :, Hq:Hq + Hkv], x[:, :, Hq + Hkv:]
    o_ref = block.attention_fwd(q, k, v)
    o_gpu = host_f16(d_o)
    assert_close(o_gpu, o_ref.reshape(T, nq), "o (fp16)", tol=2e-3)
    lse_ref = block.attention_lse(q, k)   # [B, Hq, S]
    assert_close(lse.cpu().numpy().reshape(B, Hq, S), lse_ref, "lse", tol=1e-4)
    dq, dk, dv = block.attention_bwd(dout.astype(np.float64).reshape(B, S, Hq, hd), q, k, v)
    g = host_f32(d_dqkv).reshape(B, S, Hq + 2 * Hkv, hd)
    gqk = dqk32.cpu().numpy().reshape(B, S, Hq + Hkv, hd).astype(np.float64) if f32_out else g
    if S == 1:
        # one key: P = 1 and D = dP, so dS = 0 and dQ, dK vanish up to the
        # fp32 summation order of dP (MFMA) against D (a loop)
        bound = 1e-5 * do_std
        assert np.max(np.abs(gqk[:, :, :Hq + Hkv])) <= bound, np.max(np.abs(gqk[:, :, :Hq + Hkv]))
    assert_close(gqk[:, :, :Hq], dq, "dq", tol=5e-3)
    assert_close(gqk[:, :, Hq:Hq + Hkv], dk, "dk", tol=5e-3)
    assert_close(g[:, :, Hq + Hkv:], dv, "dv", tol=5e-3)
    if f32_out:  # dQ, dK only in the fp32 buffer
        assert np.all(g[:, :, :Hq + Hkv] == 0)


@pytest.mark.parametrize("B,S,Hq,Hkv,hd,dq_form,splits", [(2, 300, 8, 2, 128, 1, 1), (2, 300, 8, 2, 128, 2, 3),
                                                          (1, 1024, 28, 4, 128, 2, 0), (3, 77, 4, 2, 64, 1, 2),
                                                          (3, 77, 4, 2, 64, 2, 1)])
def test_attention_bwd_rope_fused(B, S, Hq, Hkv, hd, dq_form, splits):
    """The RoPE backward folded into the attention backward (the step's form):
    dQ and dK rotated by -theta where they are finished (dQ kernel; dK/dV
    kernel, or the reduction of a head-split pass) and rounded to bf16 once.
    Against the oracle's attention backward followed by its RoPE backward, and
    against the unfused path (fp32 dQ, dK, then the rotation kernel) to within
    one bf16 rounding; dV unchanged bit for bit."""
    log(f"attention bwd with RoPE bwd B={B} S={S} Hq={Hq} Hkv={Hkv} hd={hd} dq_form={dq_form} splits={splits}")
    T = B * S
    ld = (Hq + 2 * Hkv) * hd
    nq, nr = Hq * hd, (Hq + Hkv) * hd
    qkv, d_qkv, _ = attn_inputs(RNG, T, Hq, Hkv, hd, 1.0)
    dout = synth.bf16_exact_normal(RNG, (T, nq))
    d_do = dev_bits(dout)
    d_o = dev_zeros_bits((T, nq))
    lse = torch.zeros(B * Hq * S, dtype=torch.float32, device="cuda")
    work = torch.zeros(int(mt.lib.mt_k_attn_bwd_work_bytes(B, S, Hq, Hkv, hd)), dtype=torch.uint8, device="cuda")
    ovf = torch.zeros(4, dtype=torch.int32, device="cuda")
    tab = torch.zeros(S * hd, dtype=torch.float32, device="cuda")
    s = _stream()
    mt.check(mt.lib.mt_k_attn_fwd(d_qkv.data_ptr(), ld, d_o.data_ptr(), nq, lse.data_ptr(), B, S, Hq, Hkv, hd,
                                  ovf.data_ptr(), s))
    # unfused: fp32 dQ and dK, then both rotated by the rotation kernel
    g32 = torch.zeros((T, nr), dtype=torch.float32, device="cuda")
    g_un = dev_zeros_bits((T, ld))
    mt.check(mt.lib.mt_k_attn_bwd(d_qkv.data_ptr(), ld, d_o.data_ptr(), d_do.data_ptr(), nq, lse.data_ptr(),
                                  work.data_ptr(), g_un.data_ptr(), ld, B, S, Hq, Hkv, hd, g32.data_ptr(), nr, splits,
                                  dq_form, ovf.data_ptr(), s))
    rot_un = dev_zeros_bits((T, nr))
    mt.check(mt.lib.mt_k_rope_f32_bf16(g32.data_ptr(), nr, rot_un.data_ptr(), nr, tab.data_ptr(), T, S, Hq + Hkv, hd,
                                       10000.0, -1, s))
    # fused
    g_fu = dev_zeros_bits((T, ld))
    mt.check(mt.lib.mt_k_attn_bwd_rope(d_qkv.data_ptr(), ld, d_o.data_ptr(), d_do.data_ptr(), nq, lse.data_ptr(),
                                       work.data_ptr(), g_fu.data_ptr(), ld, B, S, Hq, Hkv, hd, None, 0, splits,
                                       dq_form, ovf.data_ptr(), tab.data_ptr(), 10000.0, 0, s))
    # again with the maxima left in the scratch by the call before (no maxima pass): bit-identical
    g_fu2 = dev_zeros_bits((T, ld))
    mt.check(mt.lib.mt_k_attn_bwd_rope(d_qkv.data_ptr(), ld, d_o.data_ptr(), d_do.data_ptr(), nq, lse.data_ptr(),
                                       work.data_ptr(), g_fu2.data_ptr(), ld, B, S, Hq, Hkv, hd, None, 0, splits,
                                       dq_form, ovf.data_ptr(), tab.data_ptr(), 0.0, 1, s))
    _sync()
    assert torch.equal(g_fu, g_fu2), "maxima taken before: results differ"
    assert ovf[0].item() == 0
    gf = g_fu.cpu().numpy()
    assert np.array_equal(gf[:, nr:], g_un.cpu().numpy()[:, nr:]), "dV changed"
    got = widen(gf[:, :nr].view(np.uint16))
    unf = widen(rot_un.cpu().numpy().view(np.uint16))
    # within one bf16 rounding of each other: the same fp32 rotation up to the
    # contraction of its products into FMAs (a few fp32 ulps of the row's
    # largest terms), then rounded once
    row_max = np.max(np.abs(unf), axis=1, keepdims=True)
    assert np.all(np.abs(got - unf) <= np.maximum(np.abs(unf), np.abs(got)) * 2.0 ** -7 + row_max * 2.0 ** -20)
    log(f"  fused vs unfused: {np.mean(got != unf):.2e} of dQ, dK elements differ")
    x = qkv.astype(np.float64).reshape(B, S, Hq + 2 * Hkv, hd)
    q, k, v = x[:, :, :Hq], x[:, :, Hq:Hq + Hkv], x[:, :, Hq + Hkv:]
    dq, dk, _ = block.attention_bwd(dout.astype(np.float64).reshape(B, S, Hq, hd), q, k, v)
    assert_close(got[:, :nq], block.rope_bwd(dq, 10000.0).reshape(T, nq), "dq rotated (bf16)", tol=5e-3)
    assert_close(got[:, nq:], block.rope_bwd(dk, 10000.0).reshape(T, nr - nq), "dk rotated (bf16)", tol=5e-3)


@pytest.mark.parametrize("hd", [64, 128])
def test_rope_f32_to_bf16_backward(hd):
    """The rotation by -theta of fp32 gradients, rounded to bf16 once."""
    B, S, h = 2, 100, 3
    log(f"rope f32 -> bf16 hd={hd}")
    T, ld = B * S, h * hd + 8
    x = RNG.standard_normal((T, ld)).astype(np.float32)
    dx = torch.from_numpy(x).cuda()
    out = dev_zeros_bits((T, h * hd))
    tab = torch.zeros(S * hd, dtype=torch.float32, device="cuda")
    mt.check(mt.lib.mt_k_rope_f32_bf16(dx.data_ptr(), ld, out.data_ptr(), h * hd, tab.data_ptr(), T, S, h, hd,
                                       10000.0, -1, _stream()))
    _sync()
    ref = block.rope_bwd(x[:, :h * hd].astype(np.float64).reshape(B, S, h, hd), 10000.0).reshape(T, h * hd)
    got = host_f32(out)
    assert_close(got, ref, "rope bwd (bf16 out)", tol=3e-3)
    # one rounding: every element within half a bf16 ulp of the fp32 rotation (plus fp32 slack)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)


# --------------------------------------------------------- Cross-entropy --
@pytest.mark.parametrize("Tc,V", [(37, 1024), (3, 152064)])
def test_cross_entropy(Tc, V):
    log(f"ce Tc={Tc} V={V}")
    logits = (RNG.standard_normal((Tc, V)) * 2).astype(np.float32)
    labels = RNG.integers(0, V, size=Tc).astype(np.int32)
    dl = torch.from_numpy(logits).cuda()
    dlab = torch.from_numpy(labels).cuda()
    rows = torch.zeros(Tc, dtype=torch.float32, device="cuda")
    dlog = dev_zeros_bits((Tc, V))
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    s = _stream()
    mt.check(mt.lib.mt_k_ce(dl.data_ptr(), dlab.data_ptr(), rows.data_ptr(), dlog.data_ptr(), Tc, V, 1.0 / Tc, s))
    mt.check(mt.lib.mt_k_mean(rows.data_ptr(), out.data_ptr(), Tc, s))
    _sync()
    loss, dref = block.cross_entropy(logits.astype(np.float64), labels)
    assert abs(out.item() - loss) / abs(loss) < 1e-5
    assert_close(host_f32(dlog), dref, "dlogits")


# ------------------------------------------------------ fp32 -> bf16 RNE --
def test_f32_to_bf16_round_to_nearest_even():
    """The device conversion used by every bf16 output against the IEEE
    definition (oracle bf16_bits): values over the whole exponent range, all
    rounding cases of the low half (below, at and above the tie, odd and even
    kept bit), signed zeros and infinities bit for bit; NaN stays NaN."""
    rng = np.random.default_rng(7)
    hi = rng.integers(0, 1 << 16, size=1 << 16, dtype=np.uint32)
    hi = hi[((hi >> 7) & 0xFF) != 0xFF]                          # finite high halves
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    u = ((hi[:, None] << 16) | lows[None, :]).reshape(-1)
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x00000001, 0x007FFFFF,
                        0x00800000, 0x7FC00000, 0x7F800001, 0xFFC12345], np.uint32)
    u = np.concatenate([u, special, np.zeros((-(u.size + special.size)) % 4, np.uint32)])
    x = u.view(np.float32)
    dx = torch.from_numpy(x).cuda()
    dy = torch.zeros(x.size, dtype=torch.int16, device="cuda")
    mt.check(mt.lib.mt_k_f32_to_bf16(dx.data_ptr(), dy.data_ptr(), x.size, _stream()))
    _sync()
    got = dy.cpu().numpy().view(np.uint16)
    ref = bf16_bits(x)
    nan = np.isnan(x)
    # below fp32's normal range the hardware may flush; everything else exact
    sub = (np.abs(x) < np.float32(1.1754944e-38)) & (x != 0)
    keep = ~nan & ~sub
    assert np.array_equal(got[keep], ref[keep]), int(np.sum(got[keep] != ref[keep]))
    assert np.all(np.isnan((got[nan].astype(np.uint32) << 16).view(np.float32)))


@pytest.mark.parametrize("R,C,pad_s,pad_d", [(64, 64, 0, 0), (130, 77, 3, 5), (1000, 520, 8, 0),
                                              (1, 1, 0, 0), (8192, 200, 0, 0), (200, 8192, 0, 8), (71, 64, 0, 1)])
def test_transpose16_bit_exact(R, C, pad_s, pad_d):
    """The transpose feeding the backward products moves bit patterns: exact,
    including ragged edges (vector interior, element-wise border) and leading
    dimensions that rule the vector path out; the padding is left alone."""
    log(f"transpose16 {R}x{C} pad {pad_s},{pad_d}")
    rng = np.random.default_rng(R * 7 + C)
    lds, ldd = C + pad_s, R + pad_d
    src = rng.integers(0, 1 << 16, size=(R, lds), dtype=np.uint16)
    dsrc = torch.from_numpy(src.view(np.int16)).cuda()
    ddst = torch.full((C, ldd), 0x1234, dtype=torch.int16, device="cuda")
    mt.check(mt.lib.mt_k_transpose16(dsrc.data_ptr(), lds, ddst.data_ptr(), ldd, R, C, 0, _stream()))
    _sync()
    got = ddst.cpu().numpy().view(np.uint16)
    assert np.array_equal(got[:, :R], src[:, :C].T)
    assert np.all(got[:, R:] == 0x1234)
    assert mt.lib.mt_k_transpose16(dsrc.data_ptr(), lds, ddst.data_ptr(), R - 1, R, C, 0, _stream()) == mt.MT_E_INVAL


@pytest.mark.parametrize("R,C", [(130, 77), (1000, 520)])
def test_transpose16_fp16_to_bf16(R, C):
    """The transpose that hands the fp16 attention output to the bf16 dW
    product: each element rounded to bf16 (RNE), bit for bit."""
    log(f"transpose16 fp16->bf16 {R}x{C}")
    rng = np.random.default_rng(R + C)
    src = (rng.standard_normal((R, C)) * 10.0 ** rng.uniform(-6, 4, (R, C))).astype(np.float16)
    dsrc = torch.from_numpy(src.view(np.int16)).cuda()
    ddst = dev_zeros_bits((C, R))
    mt.check(mt.lib.mt_k_transpose16(dsrc.data_ptr(), C, ddst.data_ptr(), R, R, C, 1, _stream()))
    _sync()
    got = ddst.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, bf16_bits(src.astype(np.float32)).T)
