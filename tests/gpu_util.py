"""Helpers for the GPU parity tests: device buffers of bf16 bit patterns,
comparison metrics.  Arithmetic of the method lives in oracle/ (reference)
and libmt.so (under test), never here."""
import sys

import numpy as np

TOL = 1e-2  # normwise relative error bound on activations, loss and gradients


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits_of(x):
    """bf16 bit patterns of float32 values that are exactly representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def widen(bits):
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def dev_bits(x_f32):
    import torch
    return torch.from_numpy(bits_of(x_f32).view(np.int16)).cuda()


def dev_zeros_bits(shape):
    import torch
    return torch.zeros(shape, dtype=torch.int16, device="cuda")


def host_f32(t):
    """Device tensor of bf16 bits (int16) -> float32 numpy."""
    return widen(t.cpu().numpy().view(np.uint16))


def f16_exact(x):
    """The float32 values as float16, asserting that none changes."""
    h = np.asarray(x, dtype=np.float32).astype(np.float16)
    assert np.array_equal(h.astype(np.float32), np.asarray(x, dtype=np.float32)), "value not exact in fp16"
    return h


def dev_f16(x_f16):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_f16, dtype=np.float16).view(np.int16)).cuda()


def host_f16(t):
    """Device tensor of fp16 bits (int16) -> float32 numpy."""
    return t.cpu().numpy().view(np.float16).astype(np.float32)


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    if den == 0.0:
        return float(np.linalg.norm(got))
    return float(np.linalg.norm(got - ref) / den)


def assert_close(got, ref, name, tol=TOL):
    e = rel_err(got, ref)
    mx = float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)))) if np.size(ref) else 0.0
    log(f"  {name}: normwise rel err {e:.3e} (max abs {mx:.3e})")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert e <= tol, f"{name}: normwise relative error {e:.3e} > {tol}"
    return e


def attn_inputs(rng, T, Hq, Hkv, hd, qk_std=1.0):
    """qkv [T x (Hq+2Hkv)hd] as the attention kernels take it: q and k
    (normal, std qk_std) and v (standard normal) as fp16.  Returns the values
    (float32), the device fp16 bit patterns (int16), and the device bf16 copy
    of the same values that the backward's gradient products take (int16)."""
    import torch
    from oracle.bf16 import bf16_bits
    nr = (Hq + Hkv) * hd
    qk = (qk_std * rng.standard_normal((T, nr))).astype(np.float16)
    v = rng.standard_normal((T, Hkv * hd)).astype(np.float16)
    h = np.concatenate([qk, v], axis=1)
    vals = h.astype(np.float32)
    dev = torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).cuda()
    devb = torch.from_numpy(np.ascontiguousarray(bf16_bits(vals)).view(np.int16)).cuda()
    return vals, dev, devb
