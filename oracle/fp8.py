"""FP8 pieces of the oracle (test infrastructure only).

The pages say only that the FP8 variant keeps accuracy with outlier
activations through block quantisation -- every small tile gets its own scale
-- and through incoherent processing -- Q and K are multiplied by random
orthogonal matrices before quantisation (page "FlashAttention-Skalierung,
Multi-GPU-Training und Gewichtsquantisierung", section 1, FlashAttention-3
item on FP8).  Everything more specific is a reading, stated here and in
the design doc:

* format: OCP FP8 E4M3 ("e4m3fn": 1 sign, 4 exponent bits with bias 7,
  3 mantissa bits, subnormal step 2^-9, no infinities, NaN = S.1111.111,
  largest finite 448); conversion rounds to nearest, ties to even, and
  saturates to +-448;
* tile: 128 consecutive rows of one (batch, head), all d columns; its scale is
  amax / 448 (1 when the tile is all zero), so the largest entry maps to +-448;
  a tile whose amax is below 2^-96 (2^-96 / sqrt(d) for a rotated tile, whose
  device transform leaves out the 1/sqrt(d)) is treated as all zero -- scale 1,
  so its values round to codes of zero -- which keeps 448 / amax finite;
* rotation: the same R = diag(s) H_d / sqrt(d) for Q and K (H_d the Sylvester
  Hadamard matrix in natural order, s a random +-1 vector), which leaves
  Q K^T unchanged because R R^T = I; V is not rotated;
* the "mirrored" oracle: exact fp64 attention of the dequantised operands
  (code value x tile scale), decoded from the codes and scales the device
  produced.
"""
from __future__ import annotations

import numpy as np

from .attention import _as_f64, reference

E4M3_MAX = 448.0
TILE_ROWS = 128


# ----------------------------------------------------------------------------
# codec, from the OCP 8-bit floating point specification (E4M3 column)
# ----------------------------------------------------------------------------
def e4m3_decode(codes) -> np.ndarray:
    """Exact float64 value of each e4m3 code (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """Round float64 values to e4m3 codes: nearest, ties to even, saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    # binade exponent of a (a = f * 2^ex with f in [0.5, 1)); normal binades start at 2^-6
    _, ex = np.frexp(a)
    e_unb = np.maximum(ex - 1, -6)  # floor(log2 a), clamped into the subnormal range
    quantum = np.exp2(e_unb - 3.0)  # spacing of representable values in that binade
    steps = np.rint(a / quantum)  # exact division by a power of two, then RNE
    val = np.minimum(steps * quantum, E4M3_MAX)  # rounding up out of range saturates
    # value -> bit pattern
    _, vex = np.frexp(val)
    is_sub = val < 2.0 ** -6
    e_field = np.where(is_sub, 0, vex - 1 + 7)
    m_field = np.where(is_sub, np.rint(val / 2.0 ** -9), np.rint((val / np.exp2(vex - 1.0) - 1.0) * 8))
    code = (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    code = np.where(val == 0, 0, code)
    code = code | np.where(sign, 0x80, 0)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


# ----------------------------------------------------------------------------
# random orthogonal rotation (incoherent processing)
# ----------------------------------------------------------------------------
def sylvester_hadamard(d: int) -> np.ndarray:
    """H_1 = [1];  H_2n = [[H_n, H_n], [H_n, -H_n]]  (d a power of two)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_matrix(signs) -> np.ndarray:
    """R = diag(signs) H_d / sqrt(d): orthogonal, shared by Q and K."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.shape[0]
    return (s[:, None] * sylvester_hadamard(d)) / np.sqrt(d)


def rotate(x, signs) -> np.ndarray:
    """x R for every row of x ([..., d]); identity when signs is None."""
    x = _as_f64(x)
    if signs is None:
        return x
    return x @ rotation_matrix(signs)


# ----------------------------------------------------------------------------
# block quantisation
# ----------------------------------------------------------------------------
MIN_AMAX = 2.0 ** -96  # below this a tile counts as all zero


def quantize_tiles(y, tile: int = TILE_ROWS, min_amax: float = MIN_AMAX):
    """Per-tile e4m3 quantisation of y ([B, H, N, d], float64).

    Returns (codes uint8 [B,H,N,d], scales float64 [B,H,ceil(N/tile)],
    t float64 [B,H,N,d]) where t = y / scale is the exact value that was
    rounded to a code (used to recognise rounding ties in comparisons).
    A tile with amax < min_amax gets scale 1 (its values, all below 2^-96,
    then round to codes of zero).
    """
    y = np.asarray(y, dtype=np.float64)
    B, H, N, d = y.shape
    nt = -(-N // tile)
    scales = np.empty((B, H, nt))
    t = np.empty_like(y)
    for i in range(nt):
        blk = y[:, :, i * tile:(i + 1) * tile, :]
        amax = np.abs(blk).max(axis=(2, 3))
        sc = np.where(amax >= min_amax, amax / E4M3_MAX, 1.0)
        scales[:, :, i] = sc
        t[:, :, i * tile:(i + 1) * tile, :] = blk / sc[:, :, None, None]
    return e4m3_encode(t), scales, t


def quantize_rotate(x, signs, tile: int = TILE_ROWS):
    """Rotate (when signs is not None) then block-quantise; see quantize_tiles.
    The zero-tile bound applies to the unnormalised transform x diag(s) H_d,
    i.e. to sqrt(d) times the rotated values."""
    y = rotate(x, signs)
    bound = MIN_AMAX if signs is None else MIN_AMAX / np.sqrt(y.shape[-1])
    return quantize_tiles(y, tile, bound)


def quantize_tensor(y, tile: int = TILE_ROWS, min_amax: float = MIN_AMAX):
    """e4m3 quantisation of the whole tensor y ([B, H, N, d]) with ONE scale: the
    baseline of the block quantisation.  scale = amax over every entry / 448 (1 when
    amax < min_amax); returned like quantize_tiles, the scale repeated in every
    (b, h, tile) entry so that dequantize and the mirrored oracle apply unchanged."""
    y = np.asarray(y, dtype=np.float64)
    B, H, N, d = y.shape
    amax = float(np.abs(y).max()) if y.size else 0.0
    sc = amax / E4M3_MAX if amax >= min_amax else 1.0
    t = y / sc
    return e4m3_encode(t), np.full((B, H, -(-N // tile)), sc), t


def quantize_rotate_tensor(x, signs, tile: int = TILE_ROWS):
    """Rotate (when signs is not None) then quantise with one scale for the tensor;
    the zero bound applies as in quantize_rotate."""
    y = rotate(x, signs)
    bound = MIN_AMAX if signs is None else MIN_AMAX / np.sqrt(y.shape[-1])
    return quantize_tensor(y, tile, bound)


def dequantize(codes, scales, tile: int = TILE_ROWS) -> np.ndarray:
    """code value x tile scale, float64 [B, H, N, d]."""
    vals = e4m3_decode(codes)
    sc = np.repeat(np.asarray(scales, dtype=np.float64), tile, axis=2)[:, :, :vals.shape[2]]
    return vals * sc[..., None]


def mirrored_attention(q8, k8, v8, q_scale, k_scale, v_scale, causal, scale, rows=None, tile=TILE_ROWS):
    """Exact attention of the dequantised fp8 operands (in the rotated basis for Q, K)."""
    return reference(dequantize(q8, q_scale, tile), dequantize(k8, k_scale, tile),
                     dequantize(v8, v_scale, tile), causal, scale, rows)
