"""Pin the oracle's float32 -> bf16 rounding against its IEEE definition.

Definition used here (no bit manipulation): bf16 keeps 8 significant bits, so
a finite float32 x with |x| in [2^(e-1), 2^e) lies between two consecutive
multiples of the quantum 2^(e-8) (2^-133 below the normal range); the result
is the nearer multiple, ties going to the even one, and anything that rounds
to 2^128 or beyond becomes infinity.  NaN stays NaN and is quiet.
"""
import numpy as np

from oracle.bf16 import bf16_bits, bf16_to_f32, round_bf16


def _reference_round(x32):
    x = x32.astype(np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    xf = x[finite]
    _, e = np.frexp(xf)                       # |x| = m 2^e with m in [0.5, 1)
    e = np.maximum(e, -125)                   # below 2^-126 the quantum is fixed
    q = np.ldexp(1.0, (e - 8).astype(np.int64))
    lo = np.floor(xf / q)
    hi = lo + 1.0
    dlo = xf - lo * q
    dhi = hi * q - xf
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (np.mod(hi, 2.0) == 0.0))
    r = np.where(pick_hi, hi, lo) * q
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    out[finite] = r
    out[~finite] = x[~finite]
    return out


def _patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = [0x0000, 0x0001, 0x3FFF, 0x4000, 0x7FFE, 0x7FFF, 0x8000, 0x8001,
            0xBFFF, 0xC000, 0xFFFE, 0xFFFF]
    rng = np.random.default_rng(7)
    lows += list(rng.integers(0, 1 << 16, size=12))
    return np.concatenate([hi | np.uint32(lo) for lo in lows])


def test_bf16_rne_matches_ieee_definition():
    bits = _patterns()
    x = bits.view(np.float32)
    got = round_bf16(x).astype(np.float64)
    ref = _reference_round(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # zeros keep their sign
    z = x == 0
    assert np.array_equal(np.signbit(got[z]), np.signbit(x[z]))


def test_bf16_nan_stays_quiet_nan_with_sign():
    bits = _patterns()
    x = bits.view(np.float32)
    nan = np.isnan(x)
    b = bf16_bits(x[nan])
    assert np.all((b & 0x7F80) == 0x7F80)
    assert np.all((b & 0x0040) == 0x0040)
    assert np.array_equal(b >> 15, (bits[nan] >> 31).astype(np.uint16))


def test_bf16_widening_is_exact_and_idempotent():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100000).astype(np.float32)
    r = round_bf16(x)
    assert np.array_equal(round_bf16(r), r)
    assert np.array_equal(bf16_to_f32(bf16_bits(r)), r)
    # relative rounding error of RNE to 8 significant bits is at most 2^-8
    assert np.max(np.abs(r - x) / np.abs(x)) <= 2.0 ** -8
