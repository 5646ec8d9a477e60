"""FLOP conventions of the throughput figures (host arithmetic on sizes only).

The pages quote attention throughput as FLOPs counted from the two N x N x d
contractions of the forward pass (QK^T and PV, one multiply and one add per term):
4 * B * H * N^2 * d, halved for a causal mask (the masked half is not counted; the
diagonal is not added back). The backward pass recomputes QK^T and adds four more
contractions of the same size (dV, dP, dQ, dK), so its count is 2.5 times the forward
count.
"""


def counted_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Forward FLOPs: 4*B*H*N^2*d, halved when causal."""
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def counted_flops_backward(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Backward FLOPs: five N x N x d contractions, 2.5 times the forward count."""
    return 2.5 * counted_flops(B, H, N, d, causal)
