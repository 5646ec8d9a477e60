"""attn_decode_bf16_noalloc (partials in the library's static device scratch, no
workspace) against attn_decode_bf16 (caller workspace), through the C ABI.

Both run the same split and combine kernels with the same key chunking, so their
outputs must agree bit for bit; both are also held to the oracle's 16-bit gates (O
max-abs <= 2e-2, |dLSE| <= 1e-3 * max(1, |LSE|)). Two calls in a row, the second with
a smaller input, check that nothing from the first call's scratch contents leaks into
the second.
"""

import sys

import numpy as np
import pytest
import torch

from exact_attention_78_amd import attn_decode_bf16, attn_decode_bf16_noalloc, inputs
from oracle.attention import attention_forward

pytestmark = pytest.mark.gpu


def test_noalloc_decode_matches_workspace_decode_twice():
    for B, H, Nq, Nk, d in ((4, 16, 32, 5000, 128), (2, 3, 1, 777, 64)):
        print(f"case noalloc decode B{B} H{H} Nq{Nq} Nk{Nk} d{d}", flush=True)
        sys.stdout.flush()
        q = inputs.to_torch(inputs.normal_f32(95, inputs.Q_ID, (B, H, Nq, d)), "bf16")
        k = inputs.to_torch(inputs.normal_f32(95, inputs.K_ID, (B, H, Nk, d)), "bf16")
        v = inputs.to_torch(inputs.normal_f32(95, inputs.V_ID, (B, H, Nk, d)), "bf16")
        gq, gk, gv = q.cuda(), k.cuda(), v.cuda()
        o2 = torch.full_like(gq, float("nan"))
        l2 = torch.full((B, H, Nq), float("nan"), device="cuda")
        attn_decode_bf16_noalloc(gq, gk, gv, out=o2, lse=l2)
        o1, l1 = attn_decode_bf16(gq, gk, gv)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        Oref, Lref = attention_forward(q, k, v, False, inputs.softmax_scale(d))
        eo = np.abs(o2.double().cpu().numpy() - Oref).max()
        el = (np.abs(l2.double().cpu().numpy() - Lref) / np.maximum(1, np.abs(Lref))).max()
        print(f"  bit-identical to the workspace entry point; max|dO|={eo:.3e} max rel dLSE={el:.3e}", flush=True)
        assert eo <= 2e-2 and el <= 1e-3
