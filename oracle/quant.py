"""Per-block 8-bit quantization of the QK operands (fp64 oracle, TEST INFRASTRUCTURE ONLY).

The SpargeAttn notes, section 2.4, say the sparse kernel's QK path takes Q and K
quantized block by block, each block carrying its own dequantization scale
(the SageAttention scheme), while P V stays in the input precision.  The pages
fix neither the 8-bit format nor how a block's scale is chosen.  Readings taken
here (the plainest ones the rest supports):

* Format: OCP FP8 E4M3 (the 8-bit float the gfx950 matrix cores take): sign
  bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals m * 2^-9,
  largest finite value 448 (exponent field 15, mantissa 6), no infinities,
  0x7F / 0xFF are NaN.  Rounding is to nearest, ties to the even code.
* Scale: symmetric, one per block of rows: amax = max |x| over the block,
  s = amax / 448, and each element becomes the code nearest to
  clamp(x * (448 / amax), -448, 448); an all-zero block gets s = 1 and zero
  codes.  The dequantized element is value(code) * s.
* Blocks: Q in blocks of block_q rows (the query blocks), K in blocks of 64
  rows (the key tile), both in the reordered token order; the last block may
  be short.
* The steps that decide a code -- amax, the division 448 / amax, the scale
  amax / 448 and the product x * (448 / amax) -- are IEEE float32 operations
  (correctly rounded), the precision the kernel takes them in, so that both
  sides reach the same code; only the final rounding to E4M3 is written out
  here, from the format's definition (a table of the 127 non-negative finite
  values and a nearest-value search).
"""

import numpy as np

E4M3_MAX = 448.0
KEY_QUANT_ROWS = 64  # rows per K quantization block


def e4m3_values() -> np.ndarray:
    """Values of the non-negative codes 0x00 .. 0x7E, in code order (increasing)."""
    c = np.arange(0x7F)
    e = c >> 3
    m = (c & 7).astype(np.float64)
    sub = m * 2.0 ** -9
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    return np.where(e == 0, sub, nrm)


_VALS = e4m3_values()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes -> float64 (0x7F and 0xFF give NaN)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = c & 0x7F
    out = np.where(mag == 0x7F, np.nan, _VALS[np.minimum(mag, 0x7E)])
    return np.where(c & 0x80, -out, out)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """float values with |y| <= 448 -> uint8 E4M3 codes, round to nearest, ties to even.

    The sign is kept (a negative value that rounds to zero gives 0x80).
    """
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.isnan(y)) or np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values of magnitude at most 448")
    a = np.abs(y)
    hi = np.searchsorted(_VALS, a, side="left")  # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _VALS[lo]
    dhi = _VALS[hi] - a
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _VALS[hi], hi, code).astype(np.uint8)
    return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)


def quantize_blocks(x: np.ndarray, block: int):
    """Quantize the rows of x ([n, d], values exactly representable in float32, e.g.
    bf16 inputs) in consecutive blocks of ``block`` rows.

    Returns (codes uint8 [n, d], scales float32 [ceil(n / block)]).
    """
    x32 = np.asarray(x, dtype=np.float32)
    if not np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64)):
        raise ValueError("inputs must be float32 values")
    n = x32.shape[0]
    nb = -(-n // block)
    codes = np.zeros(x32.shape, dtype=np.uint8)
    scales = np.ones(nb, dtype=np.float32)
    m448 = np.float32(E4M3_MAX)
    for j in range(nb):
        blk = x32[j * block:(j + 1) * block]
        amax = np.float32(np.max(np.abs(blk))) if blk.size else np.float32(0)
        if amax == 0:
            codes[j * block:(j + 1) * block] = np.where(np.signbit(blk), 0x80, 0)
            continue
        inv = np.float32(m448 / amax)           # float32 division, correctly rounded
        scales[j] = np.float32(amax / m448)
        y = (blk * inv).astype(np.float32)      # float32 products, correctly rounded
        y = np.clip(y, -m448, m448)
        codes[j * block:(j + 1) * block] = e4m3_encode(y)
    return codes, scales


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray, block: int) -> np.ndarray:
    """value(code) * s of each row's block, in float64."""
    vals = e4m3_decode(codes)
    s = np.repeat(np.asarray(scales, dtype=np.float64), block)[:vals.shape[0]]
    return vals * s[:, None]


def score_error_bound(q: np.ndarray, k: np.ndarray, q_hat: np.ndarray, k_hat: np.ndarray, scale: float):
    """Bound on |scale * (q_hat . k_hat - q . k)| for every (query, key) pair.

    With q_hat = q + dq and k_hat = k + dk,
    q_hat.k_hat - q.k = dq.k + q.dk + dq.dk, so the error is at most
    sum |dq||k| + |q||dk| + |dq||dk|, taken elementwise here (exact errors of
    the given quantized operands, no model of the rounding).
    """
    dq = np.abs(q_hat - q)
    dk = np.abs(k_hat - k)
    return scale * (dq @ np.abs(k).T + np.abs(q) @ dk.T + dq @ dk.T)
