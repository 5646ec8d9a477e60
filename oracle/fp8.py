"""fp8 input preparation for attention (oracle; test infrastructure only).

Follows "8.3 FlashAttention-3" (booiljung.github.io):

* section 5.2 (incoherent processing): Q and K are multiplied by one random orthogonal
  matrix, taken to be a Hadamard matrix with a random sign per channel. Because it is
  orthogonal, (Q M)(K M)^T = Q K^T, so the scores are unchanged while outlier
  channels are spread over all d channels. The page stresses that the transform needs
  only additions and subtractions and costs O(d log d), i.e. the fast Walsh-Hadamard
  butterfly. Here M = diag(sigma) * H_d / sqrt(d) with H_d Sylvester's Hadamard
  matrix and sigma in {+1,-1}^d; V is not rotated (rotating V would rotate O).
* section 5.1 (block quantisation): one fp32 scale per block of 128 rows (all d
  columns of one (batch, head)), instead of one scale per tensor.

The 8-bit format is OCP FP8 E4M3FN ("E4M3" on the Triton 07 page's list of future
work): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
infinities, a single NaN pattern per sign (exponent and mantissa all ones), largest
finite value 448.

Precision. The attention oracle works in fp64, but the quantiser decides integer
codes, so it takes each rounding decision in fp32 exactly as a device kernel working
in fp32 would: the butterfly adds/subtracts in fp32, the 1/sqrt(d) factor is the fp32
value nearest to it, the scale is fp32(amax / 448) and each code is the E4M3 value
nearest to fp32(x / scale) after clamping to +-448, ties to even.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK_ROWS = 128


# --------------------------------------------------------------------------- E4M3 codec

def e4m3_decode(codes) -> np.ndarray:
    """Decode E4M3FN byte codes to fp64 from the format definition (NaN codes -> NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * np.ldexp(1.0 + m / 8.0, e - 7)
    subnormal = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (m == 7), np.nan, out)


_POS_CODES = np.arange(0x7F, dtype=np.uint8)          # 0x00 .. 0x7E: the finite non-negatives
_POS_VALUES = e4m3_decode(_POS_CODES)                  # strictly increasing


def e4m3_encode(x) -> np.ndarray:
    """Round fp32/fp64 values in [-448, 448] to the nearest E4M3FN code, ties to even.

    "Even" means the code with a zero least-significant mantissa bit, which is the
    usual round-half-to-even on the significand. The sign bit follows the sign of x,
    so -0.0 and negative values that round to zero give 0x80. Values outside
    [-448, 448] or NaN raise: callers clamp first.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or (np.abs(x) > E4M3_MAX).any():
        raise ValueError("e4m3_encode expects finite values within [-448, 448]")
    ax = np.abs(x)
    hi = np.searchsorted(_POS_VALUES, ax, side="left")   # first grid value >= ax
    hi = np.minimum(hi, _POS_VALUES.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = ax - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - ax
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


# ------------------------------------------------------------------------------ Hadamard

def sylvester_hadamard(d: int) -> np.ndarray:
    """Sylvester's Hadamard matrix H_d (d a power of two): H_1 = [1], H_2n = [[H, H], [H, -H]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht(x, dtype=np.float32) -> np.ndarray:
    """Fast Walsh-Hadamard transform along the last axis: returns x @ H_d.

    The butterfly runs log2(d) stages with spans 1, 2, 4, ..., d/2; in the stage of span
    h, positions j and j+h of every block of 2h become (x_j + x_{j+h}, x_j - x_{j+h}).
    Every output of a stage is one rounded add or subtract in ``dtype``.
    """
    y = np.array(x, dtype=dtype, copy=True)
    d = y.shape[-1]
    if d < 1 or d & (d - 1):
        raise ValueError("last axis must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        y = y.reshape(lead + (d // (2 * h), 2, h))
        a = y[..., 0, :]
        b = y[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(lead + (d,))
        h *= 2
    return y


def inv_sqrt_d_f32(d: int) -> np.float32:
    """The fp32 value nearest to 1/sqrt(d)."""
    return np.float32(1.0 / np.sqrt(np.float64(d)))


def rotate_f32(x, signs) -> np.ndarray:
    """x -> x * diag(signs) * H_d / sqrt(d), in fp32 (sign flip, fp32 butterfly, one fp32 multiply)."""
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(signs, dtype=np.float32)
    if not np.all(np.abs(s) == 1):
        raise ValueError("signs must be +-1")
    d = x.shape[-1]
    return fwht(x * s, np.float32) * inv_sqrt_d_f32(d)


# --------------------------------------------------------------------- block quantiser

def quantize_blocks(x, block_rows: int = BLOCK_ROWS):
    """Per-(b, h, 128-row block) E4M3 quantisation of an fp32 array [B, H, N, d].

    For each block: amax = max |x|; scale = fp32(amax / 448), or 1 when amax == 0;
    code = e4m3(clamp(fp32(x / scale), -448, 448)). The last block of a head may hold
    fewer than 128 rows.

    Returns (codes uint8 [B, H, N, d], scales fp32 [B, H, ceil(N / 128)]).
    """
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    nblk = -(-N // block_rows)
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty((B, H, nblk), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for t in range(nblk):
                blk = x[b, h, t * block_rows:(t + 1) * block_rows]
                amax = np.float32(np.abs(blk).max())
                s = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
                y = np.clip(blk / s, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
                codes[b, h, t * block_rows:(t + 1) * block_rows] = e4m3_encode(y)
                scales[b, h, t] = s
    return codes, scales


def dequantize_blocks(codes, scales, block_rows: int = BLOCK_ROWS) -> np.ndarray:
    """fp64 values decode(code) * scale of the code's block, shape [B, H, N, d]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float64)
    N = codes.shape[2]
    per_row = np.repeat(scales, block_rows, axis=2)[:, :, :N]
    return e4m3_decode(codes) * per_row[..., None]


def prepare_fp8(q, k, v, signs, rotate: bool = True):
    """fp8 inputs for attention: rotate Q and K (unless ``rotate`` is False), then
    block-quantise Q, K and V. Inputs are fp32 arrays [B, H, N, d] (bf16 activations
    upcast exactly) and ``signs`` is the shared +-1 vector of length d.

    Returns dict with codes q8/k8/v8 (uint8) and scales sq/sk/sv (fp32).
    """
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    if rotate:
        q = rotate_f32(q, signs)
        k = rotate_f32(k, signs)
    q8, sq = quantize_blocks(q)
    k8, sk = quantize_blocks(k)
    v8, sv = quantize_blocks(v)
    return {"q8": q8, "k8": k8, "v8": v8, "sq": sq, "sk": sk, "sv": sv}
