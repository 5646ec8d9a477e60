"""Pins for the fp8 oracle (CPU only): E4M3 codec, Hadamard transform, block quantiser.

The codec is checked against the format's published anchor values and against
PyTorch's float8_e4m3fn casts over all 256 codes and every rounding midpoint; the
transform against scipy's Hadamard matrix and the orthogonality identity; the
quantiser against a scalar brute-force nearest-value search and the E4M3 error bound.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import fp8
from oracle.attention import attention_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(99)


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn).float().numpy()


def torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32).copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.e4m3_decode(codes)
    ref = torch_decode(codes).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_decode_anchor_values():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_anchor_values.json")))
    for hexcode, val in g["codes"].items():
        got = fp8.e4m3_decode(np.array([int(hexcode, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hexcode


def test_encode_representables_roundtrip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = fp8.e4m3_decode(codes)
    np.testing.assert_array_equal(fp8.e4m3_encode(vals), codes)


def test_encode_midpoints_ties_to_even():
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2          # exactly representable in fp32
    got = fp8.e4m3_encode(np.float32(mids))
    lower = np.arange(0x7E, dtype=np.uint8)
    expect = np.where(lower % 2 == 0, lower, lower + 1).astype(np.uint8)
    np.testing.assert_array_equal(got, expect)
    np.testing.assert_array_equal(got, torch_encode(mids))
    np.testing.assert_array_equal(fp8.e4m3_encode(-np.float32(mids)), expect | 0x80)


def test_encode_random_matches_torch_after_clamp():
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 50,
        (rng.standard_normal(20000) * 2.0 ** -8).astype(np.float32),      # subnormal range
        np.float32(rng.uniform(-448, 448, 20000)),
        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -9 * 1.5], dtype=np.float32),
    ])
    np.testing.assert_array_equal(fp8.e4m3_encode(x), torch_encode(x))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([448.5], dtype=np.float32))
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([np.nan]))
    # why the quantiser clamps: PyTorch's cast turns 500 into NaN
    assert torch_encode(np.array([500.0]))[0] == 0x7F


def scalar_nearest_code(x):
    """Brute force: scan all finite non-negative codes, keep the nearest, ties to even code."""
    best = None
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        val = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        dist = abs(abs(x) - val)
        if best is None or dist < best[0] or (dist == best[0] and c % 2 == 0):
            best = (dist, c)
    return best[1] | (0x80 if math.copysign(1.0, x) < 0 else 0)


def test_encode_matches_scalar_brute_force():
    xs = np.float32(np.concatenate([rng.uniform(-448, 448, 300), rng.standard_normal(300) * 0.02]))
    got = fp8.e4m3_encode(xs)
    assert [scalar_nearest_code(float(x)) for x in xs] == list(got)


@pytest.mark.parametrize("d", [1, 2, 4, 16, 64, 128])
def test_sylvester_matches_scipy_and_is_orthogonal(d):
    h = fp8.sylvester_hadamard(d)
    np.testing.assert_array_equal(h, scipy.linalg.hadamard(d))
    np.testing.assert_array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_fwht_equals_matrix_product(d):
    xi = rng.integers(-50, 50, size=(3, 5, d))
    h = scipy.linalg.hadamard(d)
    np.testing.assert_array_equal(fp8.fwht(xi, np.float64), (xi @ h).astype(np.float64))
    xf = rng.standard_normal((7, d))
    np.testing.assert_allclose(fp8.fwht(xf, np.float64), xf @ h, atol=1e-12, rtol=0)
    # fp32 butterfly: log2(d) rounded stages, each within half an ulp of its exact result
    y32 = fp8.fwht(np.float32(xf), np.float32).astype(np.float64)
    exact = np.float32(xf).astype(np.float64) @ h
    bound = math.log2(d) * 2.0 ** -24 * (np.abs(np.float32(xf)).astype(np.float64) @ np.abs(h))
    assert (np.abs(y32 - exact) <= bound + 1e-30).all()


def test_rotation_preserves_scores():
    d = 128
    signs = np.where(rng.integers(0, 2, d) == 1, 1.0, -1.0)
    M = np.diag(signs) @ scipy.linalg.hadamard(d) / math.sqrt(d)
    np.testing.assert_allclose(M @ M.T, np.eye(d), atol=1e-14)
    q, k = rng.standard_normal((20, d)), rng.standard_normal((30, d))
    np.testing.assert_allclose((q @ M) @ (k @ M).T, q @ k.T, atol=1e-12)
    # the fp32 rotation the quantiser uses agrees with M to fp32 accuracy
    r32 = fp8.rotate_f32(np.float32(q), signs).astype(np.float64)
    np.testing.assert_allclose(r32, np.float32(q).astype(np.float64) @ M, atol=1e-5, rtol=0)
    assert fp8.inv_sqrt_d_f32(128) == np.float32(0.088388346)
    assert fp8.inv_sqrt_d_f32(64) == np.float32(0.125)


def test_quantize_blocks_properties():
    B, H, N, d = 2, 2, 300, 64                   # ragged: blocks of 128, 128, 44 rows
    x = (rng.standard_normal((B, H, N, d)) * rng.uniform(0.01, 30, (B, H, N, 1))).astype(np.float32)
    x[1, 1, 128:256] = 0.0                       # an all-zero block
    codes, scales = fp8.quantize_blocks(x)
    assert codes.shape == x.shape and scales.shape == (B, H, 3)
    assert scales.dtype == np.float32
    xh = fp8.dequantize_blocks(codes, scales)
    for b in range(B):
        for h in range(H):
            for t in range(3):
                blk = x[b, h, t * 128:(t + 1) * 128].astype(np.float64)
                cb = codes[b, h, t * 128:(t + 1) * 128]
                amax = np.abs(blk).max()
                s = scales[b, h, t]
                if amax == 0:
                    assert s == 1.0 and (cb & 0x7F).max() == 0
                    continue
                assert s == np.float32(np.float32(amax) / np.float32(448))
                assert (cb & 0x7F).max() == 0x7E                      # the block max maps to 448
                err = np.abs(xh[b, h, t * 128:(t + 1) * 128] - blk)
                y = np.abs(blk) / float(s)
                normal = y >= 2.0 ** -6
                # half an ulp of a 3-bit significand, plus the fp32 division's own rounding
                assert (err[normal] <= (2.0 ** -4 + 2.0 ** -23) * np.abs(blk[normal]) * 1.0000001).all()
                assert (err[~normal] <= 2.0 ** -10 * float(s) * 1.0001 + 1e-30).all()


def test_quantize_brute_force_tiny():
    x = np.float32(rng.standard_normal((1, 1, 5, 8)) * 3)
    codes, scales = fp8.quantize_blocks(x)
    amax = max(abs(float(t)) for t in x.ravel())
    s = np.float32(np.float32(amax) / np.float32(448.0))
    assert scales[0, 0, 0] == s
    for idx in np.ndindex(x.shape):
        y = float(np.float32(x[idx] / s))
        y = min(max(y, -448.0), 448.0)
        assert codes[idx] == scalar_nearest_code(y)


def test_prepare_fp8_attention_tracks_unquantised():
    # The dequantised fp8 inputs give attention close to the unquantised inputs, and the
    # rotation leaves the exact scores unchanged (so O differs only by quantisation error).
    B, H, N, d = 1, 2, 256, 128
    q, k, v = (rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(3))
    signs = np.where(rng.integers(0, 2, d) == 1, 1.0, -1.0).astype(np.float32)
    p = fp8.prepare_fp8(q, k, v, signs)
    qh, kh, vh = (fp8.dequantize_blocks(p[c], p[s]) for c, s in (("q8", "sq"), ("k8", "sk"), ("v8", "sv")))
    scale = 1 / math.sqrt(d)
    O_exact, _ = attention_forward(q, k, v, True, scale)
    O_q, _ = attention_forward(qh, kh, vh, True, scale)
    err = O_q - O_exact
    assert np.sqrt(np.mean(err ** 2)) < 0.02
    # causal row 0 attends to key 0 alone, so its error is V's own quantisation error
    np.testing.assert_allclose(O_q[:, :, 0], vh[:, :, 0], atol=1e-12)
    # V is not rotated: its dequantised values track V itself
    assert np.abs(vh - v).max() <= 2.0 ** -4 * np.abs(v).max() + 1e-6
