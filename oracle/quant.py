"""Low-bit expert weights: MXFP4 (OCP Microscaling Formats v1.0), the
gfx950-native analogue of the 4-bit weight formats the pages list for
DiffusionGemma ([Experimental] "DiffusionGemma: Google's Experimental
Diffusion LLM" and [ParadigmShift] "Serving in Production": GGUF Q4_K_M to
Q8_0 and NVFP4 builds).

Test infrastructure only: the CPU oracle of the quantiser and of the
dequantised weights the GPU's expert GEMMs multiply by.

Format.  A block is 32 consecutive weights along the input (K) dimension of
one output column.  Each element is FP4 E2M1: a sign bit, two exponent bits
with bias 1 and one mantissa bit, subnormal at exponent 0, no infinity or NaN,
so the magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  The block shares one
E8M0 scale 2^s stored as s + 127.

Quantisation, following the specification's conversion rule: s =
floor(log2(max |x|)) - 2 (2 = the exponent of E2M1's largest normal, 6 =
1.5 * 2^2); every element becomes the E2M1 value nearest to x / 2^s, ties to
the even mantissa, magnitudes beyond 6 saturating to 6.  Reading taken here:
s is clamped to [-126, 127] (a block whose largest magnitude is below 2^-124,
all-zero blocks included, takes s = -126), so every scale is a normal float.
Code: sign << 3 | magnitude index; the sign bit is the sign bit of x.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

BLOCK = 32
EMAX_ELEM = 2  # exponent of the largest E2M1 normal (6 = 1.5 * 2^2)
S_MIN, S_MAX = -126, 127


def e2m1_value(code: int) -> float:
    """The value of a 4-bit E2M1 code from its bit fields."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e, m = (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return sign * mag


E2M1 = np.array([e2m1_value(c) for c in range(16)])
_MAG = E2M1[:8]  # magnitudes by index 0..7, increasing


def round_e2m1(y: np.ndarray) -> np.ndarray:
    """Codes of the E2M1 values nearest to ``y`` (ties to the even mantissa,
    saturating at 6)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), 6.0)
    d = np.abs(a[..., None] - _MAG)                 # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                 # one, or two at a midpoint
    even = cand & ((np.arange(8) & 1) == 0)          # the even mantissa wins a tie
    idx = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    return (idx | (np.signbit(y).astype(np.int64) << 3)).astype(np.uint8)


def shared_exponent(amax: np.ndarray) -> np.ndarray:
    """s = floor(log2(amax)) - 2, clamped to [-126, 127] (amax == 0 -> -126)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)                           # amax = f * 2^ex, f in [0.5, 1)
    s = np.where(amax > 0, ex - 1 - EMAX_ELEM, S_MIN)
    return np.clip(s, S_MIN, S_MAX).astype(np.int64)


def quantize_blocks(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """``x [..., 32]`` -> codes uint8 ``[..., 32]`` and scale bytes uint8 ``[...]`` (s + 127)."""
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == BLOCK
    s = shared_exponent(np.abs(x).max(axis=-1))
    codes = round_e2m1(np.ldexp(x, -s[..., None]))
    return codes, (s + 127).astype(np.uint8)


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return np.ldexp(E2M1[codes], scales.astype(np.int64)[..., None] - 127)


def quantize_weight(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """A weight ``[K, N]`` (math layout y = x @ W) quantised in blocks of 32
    along K per column: codes ``[K, N]``, scale bytes ``[K / 32, N]``."""
    K, N = w.shape
    assert K % BLOCK == 0
    blocks = np.asarray(w, dtype=np.float64).reshape(K // BLOCK, BLOCK, N).transpose(0, 2, 1)
    codes, scales = quantize_blocks(blocks)          # [K/32, N, 32], [K/32, N]
    return codes.transpose(0, 2, 1).reshape(K, N), scales


def dequantize_weight(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    K, N = codes.shape
    c = codes.reshape(K // BLOCK, BLOCK, N).transpose(0, 2, 1)
    return dequantize_blocks(c, scales).transpose(0, 2, 1).reshape(K, N)


def mxfp4_weight(w: np.ndarray) -> np.ndarray:
    """The float64 values an MXFP4-stored weight ``[K, N]`` stands for."""
    return dequantize_weight(*quantize_weight(w))
