"""Run the attention oracle over many heads on the host's cores (test infrastructure only).

This module holds no arithmetic of its own. Heads and query rows of exact attention are
independent (each output row depends only on its own query row and the head's K and V),
so a forward call is split into units of (b, h, chunk of query rows) and every unit is
handed, unchanged, to ``attention.attention_forward`` on a worker thread; a backward call
(whose dK and dV sum over all query rows of a head) into units of one head, each handed
to ``attention.attention_backward``. NumPy releases the
interpreter lock inside its array kernels, so the units run in parallel; each worker
keeps BLAS to one thread so that the workers do not oversubscribe the cores.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .attention import _as_f64, attention_backward, attention_forward


def host_cores() -> int:
    """Cores this process may run on (its CPU affinity set)."""
    return len(os.sched_getaffinity(0))


def forward_pooled(q, k, v, causal: bool, scale: float, rows=None, heads=None, workers=None,
                   row_chunk: int = 1024):
    """``attention_forward`` with the same arguments and result, computed unit by unit on
    ``workers`` threads (default: every core of the affinity set).

    Returns (O, LSE) exactly as ``attention_forward`` would: fp64 [B, H, R, d] and
    [B, H, R], NaN for heads not requested.
    """
    from threadpoolctl import threadpool_limits

    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, Nq, d = q.shape
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    O = np.full((B, H, rows.size, d), np.nan)
    LSE = np.full((B, H, rows.size), np.nan)
    units = [(b, h, c0) for b, h in heads for c0 in range(0, rows.size, row_chunk)]

    def run(unit):
        b, h, c0 = unit
        r = rows[c0:c0 + row_chunk]
        o, lse = attention_forward(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], causal, scale,
                                   rows=r, row_chunk=row_chunk)
        O[b, h, c0:c0 + r.size] = o[0, 0]
        LSE[b, h, c0:c0 + r.size] = lse[0, 0]

    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers or host_cores()) as ex:
        list(ex.map(run, units))
    return O, LSE


def backward_pooled(q, k, v, dout, causal: bool, scale: float, heads=None, workers=None, row_chunk: int = 1024):
    """``attention_backward`` with the same arguments and result, one head per unit on
    ``workers`` threads (default: every core of the affinity set).

    Returns (dQ, dK, dV) exactly as ``attention_backward`` would: fp64 [B, H, N, d], NaN
    for heads not requested.
    """
    from threadpoolctl import threadpool_limits

    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    heads = [(b, h) for b in range(q.shape[0]) for h in range(q.shape[1])] if heads is None else list(heads)
    out = [np.full(q.shape, np.nan) for _ in range(3)]

    def run(unit):
        b, h = unit
        sl = (slice(b, b + 1), slice(h, h + 1))
        grads = attention_backward(q[sl], k[sl], v[sl], dout[sl], causal, scale, row_chunk=row_chunk)
        for o, g in zip(out, grads):
            o[b, h] = g[0, 0]

    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers or host_cores()) as ex:
        list(ex.map(run, heads))
    return tuple(out)
