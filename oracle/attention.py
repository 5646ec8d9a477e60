"""Plain fp64 definition of exact attention, forward and backward (oracle; test infrastructure only).

The forward also takes fewer query rows than keys without a mask (one decoding step
against a key/value cache: the digest's discussion points ask whether such steps
need a kernel of their own); it is the same definition with Nq rows.

What is computed (FlashAttention-2 digest, "Method — framework overview" flowchart and
glossary): for each batch b and head h independently,

    S   = scale * Q K^T                      (N x N scores)
    S_ij = -inf  for j > i                   (causal only; the diagonal stays allowed)
    m_i = max_j S_ij,  P_ij = exp(S_ij - m_i),  l_i = sum_j P_ij
    O_i = (sum_j P_ij V_j) / l_i             (one division per row, at the end)
    LSE_i = m_i + ln(l_i)                    (natural log of the sum of exponentials)

The tiled, online-softmax algorithm on the pages reaches this same result up to
rounding order (FlashAttention is exact attention, per the digest's title and
findings), so the oracle is the definition itself: it materialises the full score
rows in fp64 and never tiles the key axis. Rows are independent, so the work is
split by query rows only (``row_chunk``) to bound memory; each chunk holds complete
rows.
"""

from __future__ import annotations

import numpy as np


def _as_f64(x) -> np.ndarray:
    """Upcast a numpy array or a CPU torch tensor (any float dtype) to fp64 numpy."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        import torch  # local: the oracle works on numpy and only accepts torch inputs

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def attention_forward(q, k, v, causal: bool, scale: float, rows=None, heads=None,
                      row_chunk: int = 1024):
    """Exact attention forward in fp64.

    Parameters
    ----------
    q, k, v : arrays of shape [B, H, N, d] (numpy or CPU torch, any float dtype). When
              causal is False, q may have its own row count: q [B, H, Nq, d] against
              k, v [B, H, Nk, d] (every query row sees all Nk keys, as one decoding
              step does against a key/value cache).
    causal  : mask keys j > i (query i may see keys 0..i); needs Nq == Nk.
    scale   : the softmax scale, used as given (callers pass the same fp32 value the
              device uses, upcast exactly).
    rows    : optional 1-D array of query-row indices to evaluate (default: all rows).
    heads   : optional list of (b, h) pairs to evaluate (default: all B*H heads).
    row_chunk : number of query rows materialised at once.

    Returns
    -------
    O   : fp64 array [B, H, R, d] (R = len(rows)); heads not requested are NaN.
    LSE : fp64 array [B, H, R]; natural-log log-sum-exp of the scaled, masked scores.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q [B, H, Nq, d], k and v [B, H, Nk, d] with matching B, H, d")
    if causal and q.shape != k.shape:
        raise ValueError("the causal mask needs as many query rows as keys")
    B, H, Nq, d = q.shape
    N = k.shape[2]
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    if rows.ndim != 1 or (rows.size and (rows.min() < 0 or rows.max() >= Nq)):
        raise ValueError("rows must be a 1-D array of indices in [0, Nq)")
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    scale = float(scale)

    O = np.full((B, H, rows.size, d), np.nan)
    LSE = np.full((B, H, rows.size), np.nan)
    key_index = np.arange(N)
    for b, h in heads:
        for c0 in range(0, rows.size, row_chunk):
            r = rows[c0:c0 + row_chunk]
            S = scale * (q[b, h, r, :] @ k[b, h].T)          # [len(r), N]
            if causal:
                S[key_index[None, :] > r[:, None]] = -np.inf
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            l = P.sum(axis=1, keepdims=True)
            O[b, h, c0:c0 + r.size] = (P @ v[b, h]) / l
            LSE[b, h, c0:c0 + r.size] = (m + np.log(l))[:, 0]
    return O, LSE


def attention_backward(q, k, v, dout, causal: bool, scale: float, heads=None, row_chunk: int = 512):
    """Gradients of the exact attention forward in fp64 (oracle; test infrastructure only).

    The FlashAttention-2 digest (key technical points and method summary) has the
    backward pass recompute the attention from the stored log-sum-exp and produce dQ, dK
    and dV with the same query-split partition; it prints no formulas. What such a pass
    must reach is the gradient of O = softmax(scale * Q K^T [+ causal mask]) V, which
    the chain rule fixes. Per (b, h), with P the softmax rows of the forward pass:

        dV   = P^T dO
        dP   = dO V^T
        dS_ij = P_ij * (dP_ij - sum_k P_ik dP_ik)     (Jacobian of a softmax row)
        dQ   = scale * dS K
        dK   = scale * dS^T Q

    The oracle materialises P from its definition (max-subtracted exponentials divided
    by their row sum), never from a stored LSE, so a wrong LSE on the device side cannot
    hide. Query rows are processed in chunks of complete rows (``row_chunk``) to bound
    memory; dK and dV sum the chunks' contributions.

    Returns dQ, dK, dV as fp64 arrays [B, H, N, d]; heads not requested are NaN.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    dout = _as_f64(dout)
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, k, v, dout must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    scale = float(scale)

    dQ = np.full(q.shape, np.nan)
    dK = np.full(q.shape, np.nan)
    dV = np.full(q.shape, np.nan)
    key_index = np.arange(N)
    for b, h in heads:
        dK[b, h] = 0.0
        dV[b, h] = 0.0
        for c0 in range(0, N, row_chunk):
            r = np.arange(c0, min(N, c0 + row_chunk))
            S = scale * (q[b, h, r, :] @ k[b, h].T)          # [len(r), N]
            if causal:
                S[key_index[None, :] > r[:, None]] = -np.inf
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P = E / E.sum(axis=1, keepdims=True)
            g = dout[b, h, r, :]
            dV[b, h] += P.T @ g
            dP = g @ v[b, h].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dQ[b, h, r] = scale * (dS @ k[b, h])
            dK[b, h] += scale * (dS.T @ q[b, h, r, :])
    return dQ, dK, dV
