"""Pins for the backward-pass oracle (CPU only).

oracle.attention.attention_backward is tied to things other than itself: central finite
differences of the (separately pinned) forward oracle, PyTorch autograd through its own
scaled-dot-product attention in float64, closed forms (Q = 0) and invariants of the
softmax gradient (dK sums to zero over keys, dV sums to the summed dO, causal row 0
has no dQ). A transposed P, a dropped row-sum term in dS, a missing scale factor or a
dropped causal mask fails at least one of them.
"""

import math

import numpy as np
import pytest
import torch

from oracle.attention import attention_backward, attention_forward

rng = np.random.default_rng(4321)


def loss(q, k, v, dout, causal, scale):
    O, _ = attention_forward(q, k, v, causal, scale)
    return float(np.sum(O * dout))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 2), (1, 2, 5, 3), (2, 1, 6, 2)])
def test_finite_differences(shape, causal):
    q, k, v, dout = (rng.standard_normal(shape) for _ in range(4))
    scale = 0.8
    grads = attention_backward(q, k, v, dout, causal, scale)
    h = 1e-6
    for which, g in zip(range(3), grads):
        args = [q, k, v]
        fd = np.zeros(shape)
        for idx in np.ndindex(*shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (loss(*plus, dout, causal, scale) - loss(*minus, dout, causal, scale)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=0, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 37, 16), (1, 2, 130, 64)])
def test_against_torch_autograd_float64(shape, causal):
    q, k, v, dout = (rng.standard_normal(shape) for _ in range(4))
    scale = 1.0 / math.sqrt(shape[-1])
    dQ, dK, dV = attention_backward(q, k, v, dout, causal, scale, row_chunk=32)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    To = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    To.backward(torch.from_numpy(dout))
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_closed_form(causal):
    # Q = 0: uniform weights over the allowed keys. dV_j sums dO_i / n_i over the rows i
    # that see key j (n_i = number of keys row i sees), and dK = scale * dS^T Q = 0.
    B, H, N, d = 1, 2, 40, 8
    q = np.zeros((B, H, N, d))
    k, v, dout = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    _, dK, dV = attention_backward(q, k, v, dout, causal, 0.3)
    if causal:
        w = dout / np.arange(1, N + 1)[None, None, :, None]
        expect = np.flip(np.cumsum(np.flip(w, axis=2), axis=2), axis=2)     # sum over i >= j
    else:
        expect = np.broadcast_to(dout.sum(axis=2, keepdims=True) / N, dout.shape)
    np.testing.assert_allclose(dV, expect, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(dK, 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_gradient_invariants(causal):
    B, H, N, d = 2, 2, 33, 8
    q, k, v, dout = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    dQ, dK, dV = attention_backward(q, k, v, dout, causal, 0.5, row_chunk=8)
    # scores of a row are shift invariant along K: the key gradients sum to zero
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-12)
    # every softmax row sums to one: the value gradients sum to the summed dO
    np.testing.assert_allclose(dV.sum(axis=2), dout.sum(axis=2), atol=1e-12)
    if causal:
        # row 0 sees only key 0 (P = 1), so its scores carry no gradient
        np.testing.assert_array_equal(dQ[:, :, 0], 0.0)
        # the last key is seen by the last row only: dV[N-1] = P[N-1, N-1] * dO[N-1]
        _, L = attention_forward(q, k, v, True, 0.5)
        p_last = np.exp(0.5 * np.einsum("bhd,bhd->bh", q[:, :, -1], k[:, :, -1]) - L[:, :, -1])
        np.testing.assert_allclose(dV[:, :, -1], p_last[..., None] * dout[:, :, -1], atol=1e-13)


def test_linear_in_dout_and_chunking():
    B, H, N, d = 1, 2, 50, 4
    q, k, v, g1, g2 = (rng.standard_normal((B, H, N, d)) for _ in range(5))
    a = attention_backward(q, k, v, g1, True, 0.4, row_chunk=7)
    b = attention_backward(q, k, v, g2, True, 0.4, row_chunk=50)
    c = attention_backward(q, k, v, 2.0 * g1 - g2, True, 0.4, row_chunk=13)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(z, 2.0 * x - y, atol=1e-12)


def test_head_subset_leaves_others_nan():
    B, H, N, d = 2, 1, 9, 4
    q, k, v, g = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    full = attention_backward(q, k, v, g, False, 0.5)
    part = attention_backward(q, k, v, g, False, 0.5, heads=[(1, 0)])
    for f, p in zip(full, part):
        np.testing.assert_array_equal(p[1, 0], f[1, 0])
        assert np.isnan(p[0]).all()
