"""FP8 E4M3 quantisation and Hadamard rotation in plain numpy -- test
infrastructure only.

* Block quantisation: one fp32 scale per block and x~ = clip(x / s, -448, 448)
  ("FlashAttention-3 Deep Dive", section 4 "FP8 Block Quantization & Numerical
  Incoherence Elimination", per-block scaling).  The block here is 128
  consecutive rows (tokens) of one (batch, head) across all d channels, for Q,
  K and V alike; s = amax / 448 so the block's largest magnitude lands on the
  format's largest finite value (448, the clip bound of that section), and
  s = 1 for an all-zero block.  The scale, the division and the rounding
  decision are taken in fp32, the precision the kernel uses.
* E4M3 is the OCP 8-bit float with 4 exponent bits (bias 7), 3 mantissa bits,
  no infinities and a largest finite value of 448 (0x7E); rounding is to
  nearest, ties to even.
* Rotation: Q' = Q H, K' = K H with an orthogonal Hadamard matrix, which
  leaves Q K^T unchanged (same section, the incoherence-processing identity
  (QH)(KH)^T = QK^T).  "Random" is read as H = diag(sigma) H_n / sqrt(n) with
  the Sylvester H_n and random signs sigma, the same sigma for Q and K and for
  every head.  V is not rotated.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6
E4M3_MANT_BITS = 3


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> fp64 values (0x7F / 0xFF decode to NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** (E4M3_MIN_NORMAL_EXP - E4M3_MANT_BITS)
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    val = np.where(e == 0, sub, nrm)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """Round values in [-448, 448] to E4M3 codes (nearest, ties to even).

    Raises on values outside the finite range: callers clip first, as the
    block quantiser does."""
    a64 = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(a64)) or np.any(np.abs(a64) > E4M3_MAX):
        raise ValueError("e4m3_encode expects finite values within [-448, 448]")
    sign = np.signbit(a64)
    a = np.abs(a64)
    codes = np.zeros(a.shape, dtype=np.int64)
    # subnormal range: multiples of 2^-9 below 2^-6 (a count of 8 is 2^-6 itself,
    # whose code 0x08 is the smallest normal, so the encoding stays continuous)
    sub = a < 2.0 ** E4M3_MIN_NORMAL_EXP
    codes[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        mant, ex = np.frexp(a[nrm])          # a = mant * 2^ex, mant in [0.5, 1)
        e = ex - 1                           # a = (2 mant) * 2^e, 2 mant in [1, 2)
        m = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)   # exact in fp64
        carry = m == 8
        e = np.where(carry, e + 1, e)
        m = np.where(carry, 0, m)
        codes[nrm] = ((e + 7) << 3) | m
    codes = codes | np.where(sign, 0x80, 0)
    return codes.astype(np.uint8)


def block_quantize(x, block: int = 128):
    """Per-(batch, head, 128-row block) quantisation of x [B, S, H, d] (fp32).

    Returns (codes uint8 [B, S, H, d], scale fp32 [B, H, ceil(S / block)]).
    Dequantised value = e4m3_decode(code) * scale."""
    x = np.asarray(x, dtype=np.float32)
    B, S, H, d = x.shape
    nb = (S + block - 1) // block
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.ones((B, H, nb), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for j in range(nb):
                blk = x[b, j * block:(j + 1) * block, h, :]
                amax = np.float32(np.max(np.abs(blk))) if blk.size else np.float32(0)
                s = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
                y = (blk / s).astype(np.float32)                  # fp32 division, as the kernel
                y = np.clip(y, -E4M3_MAX, E4M3_MAX)
                codes[b, j * block:(j + 1) * block, h, :] = e4m3_encode(y)
                scales[b, h, j] = s
    return codes, scales


def dequantize(codes, scales, block: int = 128) -> np.ndarray:
    """codes [B, S, H, d], scales [B, H, nb] -> fp64 [B, S, H, d]."""
    vals = e4m3_decode(codes)
    B, S, H, d = vals.shape
    row_block = np.arange(S) // block
    sc = np.asarray(scales, dtype=np.float64)[:, :, row_block]   # [B, H, S]
    return vals * np.transpose(sc, (0, 2, 1))[..., None]


def hadamard_matrix(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_n (entries +-1), n a power of two."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation(signs) -> np.ndarray:
    """Orthogonal R = diag(signs) H_n / sqrt(n), applied as x' = x R."""
    s = np.asarray(signs, dtype=np.float64)
    n = s.shape[0]
    return (s[:, None] * hadamard_matrix(n)) / np.sqrt(n)


def rotate(x, signs) -> np.ndarray:
    """x [..., n] -> x R in fp64 (callers round to fp32 before quantising,
    as the kernel rotates in fp32)."""
    return np.asarray(x, dtype=np.float64) @ rotation(signs)
