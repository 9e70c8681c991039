"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the training step: it only draws token ids
and random arrays from numpy's PCG64 generator.  Both the HIP library's tests
and the CPU oracle's tests take their inputs from here.

Recipe (the measured workloads train on a math question/answer corpus; these
uniform ids stand in for it at the same batch and sequence shapes, since a
dense step's work does not depend on token values):
  * token ids [B, S+1] uniform in [0, V) from ``numpy.random.default_rng(seed)``;
    tokens = ids[:, :S] and labels = ids[:, 1:], so labels are next tokens.
  * random float arrays are N(0, std^2) float32 draws with the low 16 bits of
    each pattern cleared, so every value is exactly representable in bf16.
"""
import numpy as np

SEED_WEIGHTS = 1234
SEED_TOKENS = 5678


def tokens_labels(seed, batch, seq, vocab):
    """(tokens, labels) as int32 [batch, seq]; labels are the next tokens."""
    ids = np.random.default_rng(seed).integers(0, vocab, size=(batch, seq + 1),
                                               dtype=np.int64)
    return (np.ascontiguousarray(ids[:, :seq], dtype=np.int32),
            np.ascontiguousarray(ids[:, 1:], dtype=np.int32))


def bf16_exact_normal(rng, shape, std=1.0, mean=0.0):
    """float32 normal draws truncated to values exactly representable in bf16."""
    x = (rng.standard_normal(size=shape) * std + mean).astype(np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def normal(rng, shape, std=1.0):
    """float64 normal draws (for float64-only oracle checks)."""
    return rng.standard_normal(size=shape) * std
