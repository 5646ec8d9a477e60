"""GPU parity of the 16-bit forward pass's launch variants against the fp64 oracle.

attn_fwd_variant runs the same kernels as attn_fwd_bf16 / attn_fwd_f16 with another
mapping of query tiles to workgroups (six tile orders of a one-workgroup-per-tile grid,
and two persistent grids of one workgroup per CU: a fixed stride, or XCD-local tile
queues in caller memory) or another pass selection (the running-max pass alone, or the
first-tile-reference pass followed by the running-max pass at any size). Every variant
must give O and LSE within the 16-bit gates (O max-abs <= 2e-2, |dLSE| <= 1e-3 *
max(1, |LSE|)), checked on every head and every row.
"""

import functools
import sys

import numpy as np
import pytest
import torch

from exact_attention_78_amd import _binding, attn_fwd_variant, inputs, queue_workspace
from oracle.pool import forward_pooled

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_REL = 1e-3
SCHEDS = list(_binding.SCHEDULES)
DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make(wid, B, H, N, d, dtype, key_factor=None):
    q, k, v = inputs.draw_qkv(wid, B, H, N, d)
    if key_factor is not None:
        k = k.copy()
        k[:, :, 300:] *= np.float32(key_factor)
    cpu = tuple(inputs.to_torch(x, dtype) for x in (q, k, v))
    return cpu, tuple(t.cuda() for t in cpu)


def compare(o, lse, ref, label):
    O = o.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    Oref, Lref = ref
    assert np.isfinite(O).all() and np.isfinite(L).all(), label
    eo = np.max(np.abs(O - Oref))
    el = np.max(np.abs(L - Lref) / np.maximum(1.0, np.abs(Lref)))
    say(f"  {label}: max|dO|={eo:.3e} max rel dLSE={el:.3e}")
    assert eo <= O_TOL, (label, eo)
    assert el <= LSE_REL, (label, el)


def run(gpu, causal, scale, queue, **kw):
    o, lse = attn_fwd_variant(*gpu, causal=causal, scale=scale, queue=queue, **kw)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(2, 16, 1000, 128), (1, 3, 777, 64), (3, 8, 256, 128), (1, 1, 65, 64)])
def test_every_schedule_small(shape, causal):
    # ragged sequence lengths; head counts that are and are not multiples of 8 (the XCD
    # orders group heads per XCD only then); fewer tiles than a persistent grid's workgroups
    B, H, N, d = shape
    say(f"case schedules shape={shape} causal={causal}")
    cpu, gpu = make(60 + N % 17, B, H, N, d, "bf16")
    scale = inputs.softmax_scale(d)
    ref = forward_pooled(*cpu, causal, scale)
    queue = queue_workspace()
    for sched in SCHEDS:
        for passes in ("auto", "two"):
            o, lse = run(gpu, causal, scale, queue, sched=sched, passes=passes)
            compare(o, lse, ref, f"{sched} passes={passes}")
    assert int(queue.abs().sum()) == 0     # every call returned its queue to zero


@pytest.mark.parametrize("name,causal", [("H", True), ("C4", True), ("C3", False)])
def test_every_schedule_full_size(name, causal):
    # The benchmarked shapes under every schedule (both passes, as the default call runs
    # them), against one oracle result; the queue schedule runs twice in
    # a row on one queue array.
    w = inputs.WORKLOADS[name]
    say(f"case schedules {name} causal={causal}")
    cpu, gpu = make(w.wid, w.B, w.H, w.N, w.d, "bf16")
    ref = forward_pooled(*cpu, causal, w.scale)
    queue = queue_workspace()
    for sched in SCHEDS + ["persistent_queue"]:
        o, lse = run(gpu, causal, w.scale, queue, sched=sched)
        compare(o, lse, ref, f"{name} {sched}")
    assert int(queue.abs().sum()) == 0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 2, 1000, 128), (2, 3, 333, 64), (1, 1, 1, 64), (1, 2, 17, 128),
                                   (1, 4, 2048, 64)])
def test_two_passes_at_any_size(shape, causal, dtype):
    # The first-tile-reference pass and the marked-tile redo on small shapes, d = 64 and 128
    B, H, N, d = shape
    say(f"case passes=two shape={shape} causal={causal} dtype={dtype}")
    cpu, gpu = make(70 + N % 13, B, H, N, d, dtype)
    scale = inputs.softmax_scale(d)
    ref = forward_pooled(*cpu, causal, scale)
    o, lse = run(gpu, causal, scale, None, passes="two")
    compare(o, lse, ref, "passes=two")
    o, lse = run(gpu, causal, scale, None, passes="exact")
    compare(o, lse, ref, "passes=exact")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("factor", [8.0, 30.0])
@pytest.mark.parametrize("d", [64, 128])
def test_two_passes_with_marked_tiles(d, factor, causal, dtype):
    # Keys from 300 on scaled up: their scores outgrow the first tile's row max by ~25 (x8)
    # or by far more than 64 (x30) log2 units, so the first pass must mark those rows and
    # the second redo their query tiles; also under the persistent queue.
    B, H, N = 2, 4, 1500
    say(f"case marked tiles d={d} x{factor} causal={causal} dtype={dtype}")
    cpu, gpu = make(80, B, H, N, d, dtype, key_factor=factor)
    scale = inputs.softmax_scale(d)
    ref = forward_pooled(*cpu, causal, scale)
    queue = queue_workspace()
    for sched in ("default", "persistent_queue", "persistent_stride"):
        o, lse = run(gpu, causal, scale, queue, sched=sched, passes="two")
        compare(o, lse, ref, f"{sched} passes=two")
    assert int(queue.abs().sum()) == 0


def test_exact_pass_alone_on_the_metric_workload():
    # The running-max pass alone on bf16 causal B2 H16 N8192 d128: every head, every row.
    w = inputs.WORKLOADS["H"]
    say("case H passes=exact")
    cpu, gpu = make(w.wid, w.B, w.H, w.N, w.d, "bf16")
    ref = forward_pooled(*cpu, True, w.scale)
    o, lse = run(gpu, True, w.scale, None, passes="exact")
    compare(o, lse, ref, "H passes=exact")


def test_variant_matches_plain_entry_point_bitwise():
    # The default variant is the plain entry point: identical bits.
    cpu, gpu = make(90, 2, 16, 2048, 128, "f16")
    from exact_attention_78_amd import attn_fwd_f16

    o1, l1 = attn_fwd_f16(*gpu, causal=True)
    o2, l2 = attn_fwd_variant(*gpu, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_binding_requires_queue_for_the_queue_schedule():
    _, gpu = make(91, 1, 1, 64, 64, "bf16")
    with pytest.raises(ValueError):
        attn_fwd_variant(*gpu, sched="persistent_queue")
    with pytest.raises(ValueError):
        attn_fwd_variant(*gpu, sched="no_such_schedule")
    functools.partial(attn_fwd_variant, sched="default")(*gpu)
    torch.cuda.synchronize()
