"""GPU parity of the split-KV decoding path (attn_decode_*) against the fp64 oracle.

A few query rows attend, with no mask, to a key/value cache of Nk rows. The oracle is
the plain definition with Nq != Nk (pinned on the CPU by brute force and float64 SDPA);
it sees exactly the rounded values the GPU sees. Tolerances are those of the forward
pass: O max-abs <= 2e-2, |dLSE| <= 1e-3 * max(1, |LSE|). The decode-sized workload of
the benchmark (B16 H16 Nq1 Nk8192 d128) is checked in full: its oracle cost is small.
"""

import sys

import numpy as np
import pytest
import torch

from exact_attention_78_amd import attn_decode_bf16, attn_decode_f16, inputs
from oracle.attention import attention_forward

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_REL = 1e-3
FN = {"bf16": attn_decode_bf16, "f16": attn_decode_f16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def draw(wid, B, H, Nq, Nk, d, dtype):
    q = inputs.normal_f32(wid, inputs.Q_ID, (B, H, Nq, d))
    k = inputs.normal_f32(wid, inputs.K_ID, (B, H, Nk, d))
    v = inputs.normal_f32(wid, inputs.V_ID, (B, H, Nk, d))
    return tuple(inputs.to_torch(x, dtype) for x in (q, k, v))


def check(cpu, dtype, label):
    tq, tk, tv = cpu
    scale = inputs.softmax_scale(tq.shape[-1])
    o, lse = FN[dtype](*(t.cuda() for t in cpu), scale=scale)
    torch.cuda.synchronize()
    O = o.double().cpu().numpy()
    L = lse.double().cpu().numpy()
    Oref, Lref = attention_forward(tq, tk, tv, False, scale)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    eo = np.abs(O - Oref).max()
    el = (np.abs(L - Lref) / np.maximum(1, np.abs(Lref))).max()
    say(f"  {label}: max|dO|={eo:.3e} max rel dLSE={el:.3e}")
    assert eo <= O_TOL and el <= LSE_REL


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 2, 1, 1, 128), (2, 3, 1, 1000, 128), (1, 2, 4, 333, 64), (2, 2, 32, 2048, 128),
                                   (1, 1, 7, 65, 64), (3, 5, 2, 4097, 128), (1, 1, 1, 31, 64), (1, 1, 16, 100000, 128)])
def test_decode_shapes(shape, dtype):
    B, H, Nq, Nk, d = shape
    say(f"case decode {dtype} B{B} H{H} Nq{Nq} Nk{Nk} d{d}")
    check(draw(80 + Nk % 13, B, H, Nq, Nk, d, dtype), dtype, f"{dtype} {shape}")


def test_decode_bench_workload_full():
    B, H, Nq, Nk, d = 16, 16, 1, 8192, 128
    say(f"case decode full workload B{B} H{H} Nq{Nq} Nk{Nk} d{d}")
    check(draw(7, B, H, Nq, Nk, d, "bf16"), "bf16", "decode workload")


def test_decode_peaked_rows():
    # one key per row far above the rest: the chunk holding it must dominate the merge
    B, H, Nq, Nk, d = 1, 2, 3, 5000, 128
    tq, tk, tv = draw(81, B, H, Nq, Nk, d, "bf16")
    tk = tk.clone()
    tk[:, :, 4321] = (tq[:, :, 0] * 4).to(torch.bfloat16)
    say("case decode peaked rows")
    check((tq, tk, tv), "bf16", "peaked")


def test_decode_reuses_caller_buffers_and_is_deterministic():
    tq, tk, tv = (t.cuda() for t in draw(82, 2, 2, 3, 777, 64, "bf16"))
    o1, l1 = attn_decode_bf16(tq, tk, tv)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    ws = torch.full((1 << 20,), float("nan"), device="cuda")
    attn_decode_bf16(tq, tk, tv, out=o2, lse=l2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_cache_over_2_31_elements():
    # B16 H16, one query row against Nk = 66000 keys, d128 bf16: K and V each hold 2.16e9
    # elements (> 2^31, 4.3 GB), so the last heads' cache rows sit beyond 32-bit element
    # offsets. Inputs are drawn on the device; three heads (first, middle, last) are read
    # back and checked in full.
    B, H, Nq, Nk, d = 16, 16, 1, 66000, 128
    assert B * H * Nk * d > 2**31
    say(f"case >2^31 elements decode: B{B} H{H} Nq{Nq} Nk{Nk} d{d} bf16")
    q = inputs.normal_on_device(42, inputs.Q_ID, (B, H, Nq, d), torch.bfloat16)
    k = inputs.normal_on_device(42, inputs.K_ID, (B, H, Nk, d), torch.bfloat16)
    v = inputs.normal_on_device(42, inputs.V_ID, (B, H, Nk, d), torch.bfloat16)
    scale = inputs.softmax_scale(d)
    o, lse = attn_decode_bf16(q, k, v, scale=scale)
    torch.cuda.synchronize()
    heads = [(0, 0), (B // 2, H // 2), (B - 1, H - 1)]
    O = np.stack([o[b, h].double().cpu().numpy() for b, h in heads])[None]
    L = np.stack([lse[b, h].double().cpu().numpy() for b, h in heads])[None]
    cpu = [torch.stack([t[b, h] for b, h in heads])[None].cpu() for t in (q, k, v)]
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    Oref, Lref = attention_forward(*cpu, False, scale)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    eo = np.abs(O - Oref).max()
    el = (np.abs(L - Lref) / np.maximum(1, np.abs(Lref))).max()
    say(f"  heads {heads}: max|dO|={eo:.3e} max rel dLSE={el:.3e}")
    assert eo <= O_TOL and el <= LSE_REL
