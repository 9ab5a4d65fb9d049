"""Pins of the oracle's per-block FP8 E4M3 quantizer (CPU only).

Source of the method: SpargeAttn notes, section 2.4 (the QK path takes Q and K
quantized per block with one dequantization scale each).  The format is OCP
FP8 E4M3; its values are fixed by the format's definition (bias 7, 3 mantissa
bits, subnormals m * 2^-9, largest finite 448, NaN at 0x7F / 0xFF).  Pins: the
format's landmark values, ties written out by hand, torch's own float32 ->
float8_e4m3fn cast (a library routine the oracle does not call), brute-force
nearest search, and invariants of absmax block scaling.
"""

import math

import numpy as np
import pytest
import torch

from oracle import quant as Q


def test_decode_landmarks():
    """Format definition: the largest finite value, the smallest subnormal and normal, 1.0, NaN."""
    d = Q.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x30, 0x3C, 0x7E, 0x80, 0x81, 0xFE], dtype=np.uint8))
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 0.5, 1.5, 448.0, -0.0, -(2.0 ** -9), -448.0]
    assert d.tolist() == want
    assert np.isnan(Q.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    vals = Q.e4m3_values()
    assert len(vals) == 127 and np.all(np.diff(vals) > 0)  # strictly increasing in code order


def test_encode_hand_ties():
    """Round to nearest, ties to the even code, at hand-picked midpoints."""
    cases = {
        1.0: 0x38,
        1.0625: 0x38,               # midpoint of 1.0 (0x38) and 1.125 (0x39): even is 0x38
        1.1875: 0x3A,               # midpoint of 1.125 (0x39) and 1.25 (0x3A)
        1.0625 + 2.0 ** -20: 0x39,  # just above the midpoint
        2.0 ** -10: 0x00,           # midpoint of 0 and 2^-9
        3 * 2.0 ** -10: 0x02,       # midpoint of 2^-9 (0x01) and 2^-8 (0x02)
        15 * 2.0 ** -10: 0x08,      # midpoint of 7*2^-9 (0x07) and 2^-6 (0x08): carry into the exponent
        432.0: 0x7E,                # midpoint of 416 (0x7D) and 448 (0x7E)
        448.0: 0x7E,
        -1.1875: 0xBA,
        -(2.0 ** -11): 0x80,        # a negative value that rounds to zero keeps its sign
    }
    got = Q.e4m3_encode(np.array(list(cases), dtype=np.float64))
    assert got.tolist() == list(cases.values())


def test_encode_roundtrip_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(Q.e4m3_encode(Q.e4m3_decode(codes)), codes)


def test_encode_matches_torch_float8_e4m3fn():
    """Library pin: torch's float32 -> float8_e4m3fn cast (RNE) on random values, every
    exact midpoint between neighbouring codes, and the float32 neighbours of each midpoint."""
    rng = np.random.default_rng(0)
    mag = np.exp2(rng.uniform(-14, math.log2(448.0), 20000))
    rnd = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    vals = Q.e4m3_values()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000))])
    y = np.concatenate([rnd, mids, -mids, near, -near, np.float32([0.0, -0.0, 448.0, -448.0])])
    y = np.clip(y, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(Q.e4m3_encode(y), ref)


def test_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(1)
    y = rng.uniform(-448, 448, 3000)
    got = Q.e4m3_decode(Q.e4m3_encode(y))
    allv = np.concatenate([Q.e4m3_values(), -Q.e4m3_values()])
    best = np.min(np.abs(y[:, None] - allv[None, :]), axis=1)
    assert np.array_equal(np.abs(got - y), best)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        Q.e4m3_encode(np.array([449.0]))
    with pytest.raises(ValueError):
        Q.e4m3_encode(np.array([np.nan]))


def _bf16_values(rng, shape, scale):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def test_block_scaling_invariants():
    """Absmax scaling: per block, the largest magnitude maps to +-448 (code 0x7E / 0xFE),
    s = float32(amax / 448), every dequantized element lies within half a code step (times s)
    of x, and blocks of very different magnitude keep their own scale (a per-tensor scale
    would flush the small block to zero)."""
    rng = np.random.default_rng(2)
    x = np.concatenate([_bf16_values(rng, (64, 32), 100.0), _bf16_values(rng, (64, 32), 1e-3),
                        _bf16_values(rng, (37, 32), 1.0)])
    codes, s = Q.quantize_blocks(x, 64)
    assert codes.shape == x.shape and s.shape == (3,)
    for j in range(3):
        blk = x[64 * j:64 * (j + 1)].astype(np.float64)
        c = codes[64 * j:64 * (j + 1)]
        amax = np.abs(blk).max()
        assert s[j] == np.float32(np.float32(amax) / np.float32(448.0))
        am = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
        assert (c[am] & 0x7F) == 0x7E
        assert np.all((c & 0x7F) <= 0x7E)
        y = blk * (448.0 / amax)
        val = Q.e4m3_decode(c)
        e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
        half_step = np.exp2(e - 3) / 2  # half the spacing of codes around |y|
        assert np.all(np.abs(val - y) <= half_step * (1 + 1e-6))
        assert np.count_nonzero(c & 0x7F) > 0.9 * c.size
    deq = Q.dequantize_blocks(codes, s, 64)
    # normal-range codes carry 3 mantissa bits: relative error at most 2^-4 (plus the
    # float32 rounding of the scale and of x * 448/amax)
    for j, sl in enumerate((slice(0, 64), slice(64, 128), slice(128, 165))):
        xb, db = x[sl].astype(np.float64), deq[sl]
        big = np.abs(xb) >= 2.0 ** -6 * float(s[j])
        assert np.all(np.abs(db - xb)[big] <= np.abs(xb)[big] * 2.0 ** -4 * (1 + 1e-6))


def test_zero_block_and_ragged_tail():
    x = np.zeros((70, 8), dtype=np.float32)
    x[65, 3] = -2.5
    codes, s = Q.quantize_blocks(x, 64)
    assert s.tolist() == [1.0, np.float32(2.5 / 448.0)]
    assert np.all(codes[:64] == 0)
    assert codes[65, 3] == 0xFE and np.count_nonzero(codes[64:]) == 1
    assert Q.dequantize_blocks(codes, s, 64)[65, 3] == -448.0 * np.float64(np.float32(2.5 / 448.0))


def test_score_error_bound_holds():
    """|q_hat.k_hat - q.k| <= sum |dq||k| + |q||dk| + |dq||dk| (triangle inequality), checked
    on quantized random blocks; the bound is also within a small factor of the true error."""
    rng = np.random.default_rng(3)
    q = _bf16_values(rng, (128, 64), 1.0)
    k = _bf16_values(rng, (64, 64), 1.0)
    cq, sq = Q.quantize_blocks(q, 128)
    ck, sk = Q.quantize_blocks(k, 64)
    qh, kh = Q.dequantize_blocks(cq, sq, 128), Q.dequantize_blocks(ck, sk, 64)
    q64, k64 = q.astype(np.float64), k.astype(np.float64)
    err = np.abs(qh @ kh.T - q64 @ k64.T) * 0.125
    bound = Q.score_error_bound(q64, k64, qh, kh, 0.125)
    assert np.all(err <= bound * (1 + 1e-12))
    assert np.median(bound / np.maximum(err, 1e-12)) < 100
