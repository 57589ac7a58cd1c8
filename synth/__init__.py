"""Seeded synthetic inputs for the sparse-attention workloads.

This package is shared by the tests, the benchmark and the oracle's callers.
It only makes inputs: random tensors, needle placements and the fixed
dominant-pair sets.  It computes no step of the attention method itself.

Random numbers come from a counter-based generator so that any element of any
tensor can be regenerated on its own, on the host (this module, numpy) or on
the GPU (``synth/gen.hip``, a separate kernel written from the same published
definition).  Both produce bit-identical values.

Definition (one element, index ``n`` of tensor ``tid`` under seed ``seed``):

* key = seed * 2**40  XOR  tid * 2**36  XOR  n        (n < 2**36)
* three successive outputs w1, w2, w3 of SplitMix64 started at state = key
  (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014; the finaliser constants are those of the published
  SplitMix64 variant);
* the twelve 16-bit lanes u_j of (w1, w2, w3) are summed exactly as integers;
* z = float32(sum - 6*65535) * float32(1 / sqrt(65536**2 - 1)), one fp32
  multiply.  This is the Irwin-Hall(12) approximation of N(0, 1): mean 0,
  variance 1, tails cut at +-6;
* the value is stored as fp32, or rounded to bfloat16 with round-to-nearest-
  even.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
MIX1 = np.uint64(0xBF58476D1CE4E5B9)
MIX2 = np.uint64(0x94D049BB133111EB)
IH_OFFSET = 6 * 65535
IH_SCALE = np.float32(1.0 / np.sqrt(65536.0 ** 2 - 1.0))

# tensor ids used by the workloads
TID_Q, TID_K, TID_V, TID_NEEDLE, TID_DOM, TID_SCORES, TID_SEL = 1, 2, 3, 4, 5, 6, 7


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * MIX1
    z = (z ^ (z >> np.uint64(27))) * MIX2
    return z ^ (z >> np.uint64(31))


def counter_key(seed: int, tid: int, n: np.ndarray) -> np.ndarray:
    n = np.asarray(n, dtype=np.uint64)
    assert seed < (1 << 24) and tid < 16
    return (np.uint64(seed) << np.uint64(40)) ^ (np.uint64(tid) << np.uint64(36)) ^ n


def splitmix_words(seed: int, tid: int, n: np.ndarray, count: int = 3) -> list[np.ndarray]:
    """First ``count`` SplitMix64 outputs for the stream started at each key."""
    state = counter_key(seed, tid, n)
    out = []
    with np.errstate(over="ignore"):
        for _ in range(count):
            state = state + GAMMA
            out.append(_mix(state.copy()))
    return out


def gaussian_f32(seed: int, tid: int, n: np.ndarray) -> np.ndarray:
    """Irwin-Hall(12) normal variates (fp32) for element indices ``n``."""
    words = splitmix_words(seed, tid, np.asarray(n, dtype=np.uint64).ravel())
    # the twelve 16-bit lanes of (w1, w2, w3); the order of an integer sum is irrelevant
    lanes = np.stack(words, axis=-1).astype("<u8").view("<u2")
    total = lanes.sum(axis=-1, dtype=np.int64)
    centred = (total - IH_OFFSET).astype(np.float32)  # exact: |x| < 2**24
    z = centred * IH_SCALE
    return z.reshape(np.shape(n))


def uniform01(seed: int, tid: int, n: np.ndarray) -> np.ndarray:
    """Uniform doubles in [0, 1) from the top 53 bits of the first word."""
    w = splitmix_words(seed, tid, np.asarray(n, dtype=np.uint64).ravel(), 1)[0]
    u = (w >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
    return u.reshape(np.shape(n))


def uniform_int(seed: int, tid: int, n: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """Integers uniform on [lo, hi] (inclusive)."""
    u = uniform01(seed, tid, n)
    return lo + np.floor(u * (hi - lo + 1)).astype(np.int64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even); returns uint16 bits.

    NaN inputs map to a quiet NaN; infinities are kept.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    rounded = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    isnan = np.isnan(np.asarray(x, dtype=np.float32))
    out = rounded.astype(np.uint16)
    out[isnan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Value of ``x`` (any float dtype) after fp32 then bf16 rounding, as fp32.

    fp64 inputs are first rounded to fp32 (nearest), then to bf16.  Both
    roundings are deterministic, and every consumer reads the stored result,
    so the double rounding never matters for parity.
    """
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def gaussian_tensor(seed: int, tid: int, shape, dtype: str, base: int = 0) -> np.ndarray:
    """A whole tensor on the host: fp32 values, or bf16-rounded values as fp32.

    Element (i0, i1, ...) has counter index ``base + flat_index``.
    """
    count = int(np.prod(shape))
    z = gaussian_f32(seed, tid, np.arange(base, base + count, dtype=np.uint64))
    if dtype == "bf16":
        z = bf16_bits_to_f32(f32_to_bf16_bits(z))
    elif dtype != "f32":
        raise ValueError(dtype)
    return z.reshape(shape)
