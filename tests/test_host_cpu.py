"""Host-side pieces outside the oracle (CPU only): the FLOP conventions of the
throughput figures, and the pooled runner of the oracle."""

import itertools

import numpy as np
import pytest

from exact_attention_78_amd.flops import counted_flops, counted_flops_backward
from oracle.attention import attention_backward, attention_forward
from oracle.pool import backward_pooled, forward_pooled, host_cores


def _terms(N, d, causal):
    """Multiply-add terms of one N x N x d contraction, counted by enumerating (i, j, c)
    over all pairs (the convention counts the full N^2 and halves it for causal)."""
    return sum(1 for _i, _j, _c in itertools.product(range(N), range(N), range(d)))


@pytest.mark.parametrize("B,H,N,d", [(1, 1, 4, 2), (2, 3, 5, 4), (1, 2, 8, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_flops_count_two_contractions(B, H, N, d, causal):
    # two contractions (QK^T, PV), two FLOPs (multiply, add) per term, halved for causal
    expect = B * H * 2 * 2 * _terms(N, d, causal) / (2 if causal else 1)
    assert counted_flops(B, H, N, d, causal) == expect


def test_headline_shape_flops():
    # bf16 causal B2 H16 N8192 d128: 549.8 GFLOP
    assert round(counted_flops(2, 16, 8192, 128, True) / 1e9, 1) == 549.8
    assert counted_flops(2, 16, 8192, 128, False) == 2 * counted_flops(2, 16, 8192, 128, True)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_flops_count_five_contractions(causal):
    # QK^T again, then dV = P^T dO, dP = dO V^T, dQ = dS K, dK = dS^T Q
    B, H, N, d = 1, 2, 6, 4
    assert counted_flops_backward(B, H, N, d, causal) == 5 * 2 * B * H * _terms(N, d, causal) / (2 if causal else 1)


@pytest.mark.parametrize("causal", [False, True])
def test_pooled_oracle_matches_the_oracle(causal):
    # the pool only distributes (b, h, row chunk) units: same values in the same places
    rng = np.random.default_rng(4)
    B, H, N, d = 2, 3, 70, 8
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    O, L = attention_forward(q, k, v, causal, 0.4)
    Op, Lp = forward_pooled(q, k, v, causal, 0.4, workers=4, row_chunk=16)
    np.testing.assert_allclose(Op, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Lp, L, rtol=0, atol=1e-13)
    rows, heads = np.array([3, 69, 0, 17]), [(1, 2), (0, 1)]
    Os, Ls = attention_forward(q, k, v, causal, 0.4, rows=rows, heads=heads)
    Ops, Lps = forward_pooled(q, k, v, causal, 0.4, rows=rows, heads=heads, workers=3, row_chunk=3)
    np.testing.assert_allclose(Ops, Os, rtol=0, atol=1e-13, equal_nan=True)
    np.testing.assert_allclose(Lps, Ls, rtol=0, atol=1e-13, equal_nan=True)
    assert np.isnan(Ops[0, 0]).all()
    assert host_cores() >= 1






@pytest.mark.parametrize("causal", [False, True])
def test_pooled_backward_matches_the_oracle(causal):
    # one head per unit: the same gradients in the same places, NaN for heads left out
    rng = np.random.default_rng(5)
    B, H, N, d = 2, 2, 50, 8
    q, k, v, g = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    ref = attention_backward(q, k, v, g, causal, 0.3, row_chunk=7)
    got = backward_pooled(q, k, v, g, causal, 0.3, workers=3, row_chunk=7)
    for x, r in zip(got, ref):
        np.testing.assert_allclose(x, r, rtol=0, atol=1e-13)
    part = backward_pooled(q, k, v, g, causal, 0.3, heads=[(1, 0)], workers=2)
    for x, r in zip(part, ref):
        np.testing.assert_allclose(x[1, 0], r[1, 0], rtol=0, atol=1e-12)
        assert np.isnan(x[0]).all() and np.isnan(x[1, 1]).all()
