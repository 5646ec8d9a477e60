"""Pins for the attention oracle (CPU only).

Each test ties oracle.attention to something other than itself: brute-force scalar
loops on tiny inputs, PyTorch's own scaled-dot-product attention in float64, a
hand-worked example, closed forms (Q = 0, causal row 0) and invariants of the
definition (rows of the softmax sum to one, permutation, shift and affine
invariances). A dropped mask, a transposed operand, a wrong log base, a missing
max-subtraction or a wrong normaliser fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.attention import attention_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def brute_force(q, k, v, causal, scale):
    """Scalar loops with math.exp / math.fsum; no numpy arithmetic."""
    B, H, N, d = q.shape
    Nk = k.shape[2]
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                js = range(i + 1) if causal else range(Nk)
                s = [scale * math.fsum(float(q[b, h, i, t]) * float(k[b, h, j, t]) for t in range(d)) for j in js]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for t in range(d):
                    O[b, h, i, t] = math.fsum(e[n] * float(v[b, h, j, t]) for n, j in enumerate(js)) / tot
                L[b, h, i] = m + math.log(tot)
    return O, L


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (1, 2, 5, 3), (2, 1, 16, 8), (1, 3, 9, 4)])
def test_brute_force_tiny(shape, causal):
    q, k, v = (rng.standard_normal(shape) * 2 for _ in range(3))
    scale = 0.7
    O, L = attention_forward(q, k, v, causal, scale)
    Ob, Lb = brute_force(q, k, v, causal, scale)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("nq,nk", [(1, 9), (3, 16), (5, 2)])
def test_brute_force_fewer_queries_than_keys(nq, nk):
    # decoding shape: q [B, H, Nq, d] against a key/value cache [B, H, Nk, d], no mask
    q = rng.standard_normal((2, 2, nq, 4))
    k, v = rng.standard_normal((2, 2, nk, 4)), rng.standard_normal((2, 2, nk, 4))
    O, L = attention_forward(q, k, v, False, 0.6)
    Ob, Lb = brute_force(q, k, v, False, 0.6)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


def test_decode_shape_against_torch_sdpa_and_causal_rejected():
    q = rng.standard_normal((2, 3, 4, 32))
    k, v = rng.standard_normal((2, 3, 300, 32)), rng.standard_normal((2, 3, 300, 32))
    O, L = attention_forward(q, k, v, False, 0.17)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    To = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.17)
    TL = torch.logsumexp(0.17 * torch.matmul(tq, tk.transpose(-1, -2).contiguous()), dim=-1)
    np.testing.assert_allclose(O, To.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, TL.numpy(), rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        attention_forward(q, k, v, True, 0.17)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 37, 16), (1, 2, 130, 64)])
def test_against_torch_sdpa_float64(shape, causal):
    q, k, v = (rng.standard_normal(shape) for _ in range(3))
    scale = 1.0 / math.sqrt(shape[-1])
    O, L = attention_forward(q, k, v, causal, scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    To = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    S = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    if causal:
        n = shape[2]
        S = S.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    TL = torch.logsumexp(S, dim=-1)
    np.testing.assert_allclose(O, To.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, TL.numpy(), rtol=0, atol=1e-12)


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "attention_hand_example.json")))
    q, k, v = (np.array(g[x], dtype=np.float64)[None, None] for x in ("q", "k", "v"))
    for mode, causal in (("noncausal", False), ("causal", True)):
        O, L = attention_forward(q, k, v, causal, g["scale"])
        np.testing.assert_allclose(O[0, 0], np.array(g[mode]["O"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(L[0, 0], np.array(g[mode]["LSE"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_is_mean_of_allowed_values(causal):
    B, H, N, d = 1, 2, 50, 8
    q = np.zeros((B, H, N, d))
    k, v = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d))
    O, L = attention_forward(q, k, v, causal, 0.3)
    if causal:
        expect = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
        expect_l = np.log(np.arange(1, N + 1, dtype=np.float64))[None, None].repeat(H, 1)
    else:
        expect = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        expect_l = np.full((B, H, N), math.log(N))
    np.testing.assert_allclose(O, expect, atol=1e-13, rtol=0)
    np.testing.assert_allclose(L, expect_l, atol=1e-13, rtol=0)


def test_causal_row0_returns_v0():
    B, H, N, d = 2, 2, 33, 16
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    scale = 0.125
    O, L = attention_forward(q, k, v, True, scale)
    np.testing.assert_array_equal(O[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(L[:, :, 0], scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    # With V = identity (d = N) the output rows are the softmax rows themselves.
    N = 24
    q, k = rng.standard_normal((1, 1, N, N)), rng.standard_normal((1, 1, N, N))
    v = np.eye(N)[None, None]
    P, _ = attention_forward(q, k, v, causal, 0.5)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-14)
    assert (P >= 0).all()
    if causal:
        assert np.all(P[0, 0][np.triu_indices(N, 1)] == 0)
        assert np.all(P[0, 0][np.tril_indices(N)] > 0)


def test_noncausal_permutation_invariance():
    B, H, N, d = 1, 3, 40, 8
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    perm = rng.permutation(N)
    O1, L1 = attention_forward(q, k, v, False, 0.4)
    O2, L2 = attention_forward(q, k[:, :, perm], v[:, :, perm], False, 0.4)
    np.testing.assert_allclose(O1, O2, atol=1e-13)
    np.testing.assert_allclose(L1, L2, atol=1e-13)
    # the causal result is NOT invariant: the mask follows key positions
    O3, _ = attention_forward(q, k[:, :, perm], v[:, :, perm], True, 0.4)
    O4, _ = attention_forward(q, k, v, True, 0.4)
    assert np.abs(O3 - O4).max() > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    # K_j <- K_j + u adds s*q_i.u to every score of row i: O unchanged, LSE shifted.
    B, H, N, d = 1, 2, 30, 8
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    u = rng.standard_normal(d) * 300.0
    s = 0.25
    O1, L1 = attention_forward(q, k, v, causal, s)
    O2, L2 = attention_forward(q, k + u, v, causal, s)
    np.testing.assert_allclose(O1, O2, atol=1e-9)
    np.testing.assert_allclose(L2, L1 + s * q @ u, atol=1e-9)
    assert np.isfinite(L2).all()


@pytest.mark.parametrize("causal", [False, True])
def test_value_affine(causal):
    B, H, N, d = 1, 2, 21, 4
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    O, L = attention_forward(q, k, v, causal, 0.5)
    O_c, L_c = attention_forward(q, k, v + 3.0, causal, 0.5)
    O_a, L_a = attention_forward(q, k, -2.5 * v, causal, 0.5)
    np.testing.assert_allclose(O_c, O + 3.0, atol=1e-13)
    np.testing.assert_allclose(O_a, -2.5 * O, atol=1e-13)
    np.testing.assert_array_equal(L, L_c)
    np.testing.assert_array_equal(L, L_a)


def test_one_hot_key_selects_its_value():
    B, H, N, d = 1, 1, 16, 8
    q = np.zeros((B, H, N, d))
    q[..., 0] = 1.0
    k = rng.standard_normal((B, H, N, d)) * 0.01
    k[0, 0, 7, 0] = 100.0
    v = rng.standard_normal((B, H, N, d))
    O, L = attention_forward(q, k, v, False, 1.0)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0, 7], (N, d)), atol=1e-30 + 1e-12)
    np.testing.assert_allclose(L[0, 0], 100.0, atol=1e-6)


def test_row_and_head_subsets_match_full():
    B, H, N, d = 2, 2, 70, 8
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    O, L = attention_forward(q, k, v, True, 0.3, row_chunk=16)
    rows = np.array([0, 5, 69, 33])
    Os, Ls = attention_forward(q, k, v, True, 0.3, rows=rows, heads=[(1, 0)])
    np.testing.assert_array_equal(Os[1, 0], O[1, 0, rows])
    np.testing.assert_array_equal(Ls[1, 0], L[1, 0, rows])
    assert np.isnan(Os[0]).all()


def test_accepts_low_precision_torch_inputs():
    x = torch.randn(1, 1, 8, 4).to(torch.bfloat16)
    O, L = attention_forward(x, x, x, False, 0.5)
    O2, L2 = attention_forward(x.float().numpy(), x.float().numpy(), x.float().numpy(), False, 0.5)
    np.testing.assert_array_equal(O, O2)
