"""CPU oracle for exact attention (forward and backward) and its fp8 input preparation.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it, to check and to time the GPU library against a plain, slow,
obviously correct implementation written from the pages:

* "FlashAttention-2: faster attention with better parallelism and work partitioning"
  (digest, irregular6612.github.io) — the method's framework-overview flowchart and
  its glossary entries for online softmax and log-sum-exp;
* "8.3 FlashAttention-3" (booiljung.github.io) — section 5.1 (block quantisation) and
  section 5.2 (incoherent processing with a Hadamard transform);
* "Triton 07: Flash Attention v3" (wonbeomjang.kr) — section "Method", which fixes
  low-precision inputs with fp32 accumulation.

The oracle shares no code, constant or table with the HIP path. It computes in fp64
except where a floating-point result decides an integer code (the fp8 quantiser),
where it takes that decision in fp32, the precision the device kernel works in.

Modules
-------
attention : plain definition of softmax(scale * Q K^T [+ causal mask]) V and its LSE,
            and its gradients dQ, dK, dV by the chain rule.
fp8       : OCP E4M3 codec, Sylvester Hadamard / fast Walsh-Hadamard transform,
            per-128-row block quantiser, and the fp8 input preparation.

Every function here is pinned by ``tests/test_oracle_*.py`` against brute force,
closed forms, invariants and independent library routines; none is "parity unpinned".
"""

from . import attention, fp8  # noqa: F401
