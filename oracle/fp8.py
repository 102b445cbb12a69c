"""FP8 (e4m3) dynamic quantisation of Q and K (oracle; test infrastructure only).

Source: the ParaAttention/HunyuanVideo post (WaveSpeed), section "FP8 dynamic
quantisation": activations are quantised to FP8 at run time, so that the
products run on 8-bit matrix units, with the precision loss kept small.  The
post fixes neither the 8-bit format nor the granularity of the scales; the
readings taken here:

* format: OCP FP8 E4M3 (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits; no infinities; the all-ones code of either sign is NaN; largest finite
  magnitude 1.75 * 2^8 = 448; subnormals m * 2^-9 for m = 1..7), the 8-bit
  type of gfx950's matrix cores.  Encoding rounds to nearest, ties to even;
  inputs are clamped to [-448, 448] first, so no code is NaN;
* "dynamic": each scale comes from the data of the call, as the largest
  magnitude of its group mapped to 448;
* groups: one scale per query token (its d values) for Q, and one per
  64-token tile of a (batch, head) for K (tile tau covers tokens
  64 tau .. min(64 tau + 64, N) - 1); only the S = Q K^T product is in FP8:
  V, the weights P and the output stay in the bf16 path.

Every quantisation decision is made in fp32, step by step, so that a
correctly rounded fp32 implementation reproduces each code bit for bit:

    a     = max |x| over the group              (exact)
    inv   = fp32(448 / a)                        (correctly rounded division)
    y     = fp32(x * inv)                        (one rounding)
    code  = e4m3(clamp(y, -448, 448))            (round to nearest even)
    scale = fp32(a / 448)                        (the dequantisation factor)

and a group whose largest magnitude is 0 gets inv = scale = 0 and all-zero
codes.  The dequantised value of a code c is value(c) * scale; the fp8
attention path is exact attention on dequantised Q and K (and the original V).

The fp32 steps use fp64 arithmetic followed by one rounding to fp32: the
exact quotient or product of two fp32 numbers rounded to fp64 and then to
fp32 is the correctly rounded fp32 result (fp64 carries more than 2 * 24 + 2
significand bits).
"""
from __future__ import annotations

import dataclasses

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9
QUANT_TILE = 64          # K tokens per scale


def e4m3_value(code) -> np.ndarray:
    """Value of E4M3 codes (uint8) as fp64; NaN for the two NaN codes."""
    c = np.asarray(code).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * E4M3_SUBNORMAL_STEP, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def _round_half_even(x: np.ndarray) -> np.ndarray:
    return np.rint(x)    # numpy rounds halves to even


def e4m3_encode(x) -> np.ndarray:
    """E4M3 code (uint8) of each value, rounded to nearest, ties to even.

    The values must be finite with |x| <= 448 (callers clamp).  The sign bit
    is the input's: a negative value that rounds to zero, and -0, give the
    negative zero code 0x80.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode expects finite values with |x| <= 448")
    a = np.abs(x)
    # Binade of a normal value: a = f * 2^k with f in [0.5, 1), so a lies in
    # [2^(k-1), 2^k) and its quantum is 2^(k-1-3).
    _, k = np.frexp(a)
    normal = a >= E4M3_MIN_NORMAL
    quantum = np.where(normal, np.exp2((k - 4).astype(np.float64)), E4M3_SUBNORMAL_STEP)
    q = _round_half_even(a / quantum) * quantum          # exact: divisions by powers of two
    # Rounding can carry into the next binade (or from subnormal to normal);
    # the code is recomputed from the rounded magnitude.
    _, kq = np.frexp(q)
    qnormal = q >= E4M3_MIN_NORMAL
    exp_field = np.where(qnormal, kq - 1 + 7, 0)
    mant = np.where(qnormal, q / np.exp2((kq - 1).astype(np.float64)) * 8.0 - 8.0, q / E4M3_SUBNORMAL_STEP)
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    code = np.where(q == 0, 0, code) | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def _f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def group_factors(group_amax) -> tuple[np.ndarray, np.ndarray]:
    """(inv, scale) of groups with the given largest magnitudes, both fp32
    values held in fp64: inv = fp32(448 / a), scale = fp32(a / 448); both 0
    when a = 0."""
    a = np.asarray(group_amax, dtype=np.float64)
    safe = np.where(a > 0, a, 1.0)
    inv = np.where(a > 0, _f32(E4M3_MAX / safe), 0.0)
    scale = np.where(a > 0, _f32(safe / E4M3_MAX), 0.0)
    return inv, scale


def quantize_groups(x, group_amax) -> np.ndarray:
    """E4M3 codes of x given the largest magnitude of each element's group
    (group_amax broadcastable to x)."""
    x = np.asarray(x, dtype=np.float64)
    inv, _ = group_factors(group_amax)
    y = _f32(x * inv)
    return e4m3_encode(np.clip(y, -E4M3_MAX, E4M3_MAX))


@dataclasses.dataclass
class QuantizedQK:
    q_codes: np.ndarray     # [B,H,N,d] uint8
    q_scale: np.ndarray     # [B,H,N] fp32, one per token
    k_codes: np.ndarray     # [B,H,N,d] uint8
    k_scale: np.ndarray     # [B,H,ceil(N/64)] fp32, one per 64-token tile
    q_deq: np.ndarray       # [B,H,N,d] fp64 dequantised Q
    k_deq: np.ndarray       # [B,H,N,d] fp64 dequantised K


def quantize_q(q) -> tuple[np.ndarray, np.ndarray]:
    """Per-token E4M3 quantisation of q [B,H,N,d]: codes and scales [B,H,N]."""
    q = np.asarray(q, dtype=np.float64)
    amax = np.abs(q).max(axis=-1)
    return quantize_groups(q, amax[..., None]), group_factors(amax)[1].astype(np.float32)


def tile_amax(k, tile: int = QUANT_TILE) -> np.ndarray:
    """Largest magnitude of each `tile`-token tile of each (b, h) of k
    [B,H,N,d]; the last tile holds the remaining N - tile*(nt-1) tokens."""
    k = np.asarray(k, dtype=np.float64)
    B, H, N, d = k.shape
    nt = -(-N // tile)
    amax = np.zeros((B, H, nt))
    for t in range(nt):
        amax[:, :, t] = np.abs(k[:, :, t * tile:min(N, (t + 1) * tile)]).max(axis=(-1, -2))
    return amax


def quantize_k(k, tile: int = QUANT_TILE) -> tuple[np.ndarray, np.ndarray]:
    """Per-tile E4M3 quantisation of k [B,H,N,d]: codes and one scale per
    `tile` tokens of each (b, h), [B,H,ceil(N/tile)]."""
    k = np.asarray(k, dtype=np.float64)
    amax = tile_amax(k, tile)
    tile_of_token = np.arange(k.shape[2]) // tile
    return quantize_groups(k, amax[:, :, tile_of_token][..., None]), group_factors(amax)[1].astype(np.float32)


def dequantize(codes, scale) -> np.ndarray:
    """value(code) * scale in fp64 (exact); scale broadcast against codes."""
    return e4m3_value(codes) * np.asarray(scale, dtype=np.float64)


def quantize_qk(q, k, tile: int = QUANT_TILE) -> QuantizedQK:
    """Q per token and K per tile, with their dequantised values."""
    qc, qs = quantize_q(q)
    kc, ks = quantize_k(k, tile)
    N = np.asarray(k).shape[2]
    tile_of_token = np.arange(N) // tile
    return QuantizedQK(qc, qs, kc, ks, dequantize(qc, qs[..., None]),
                       dequantize(kc, ks[:, :, tile_of_token][..., None]))
