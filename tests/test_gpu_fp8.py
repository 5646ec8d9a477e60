"""GPU parity of the fp8 path: the Hadamard + E4M3 block quantiser (bit-exact against
the oracle's quantiser) and the fp8 attention forward (against the fp64 oracle run on
the dequantised inputs, O max-abs error <= 1e-1 and |dLSE| <= 1e-3 * max(1, |LSE|)).

The quantiser decides integer codes, so it must match the oracle exactly: both take the
same fp32 roundings (butterfly adds, the 1/sqrt(d) product, amax/448 and x/scale).
"""

import sys

import numpy as np
import pytest
import torch

from exact_attention_78_amd import (attn_fwd_fp8, attn_fwd_fp8_rotq, attn_quant_fp8, attn_quant_fp8_kv,
                                   attn_quant_fp8_qkv, inputs)
from oracle import fp8 as ofp8
from oracle.attention import attention_forward
from oracle.pool import forward_pooled

pytestmark = pytest.mark.gpu

O_TOL_FP8 = 1e-1
LSE_REL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_activations(x32):
    """Round fp32 draws to the bf16 activations both sides consume."""
    t = inputs.to_torch(x32, "bf16")
    return t, t.float().numpy()


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("rotate", [True, False])
@pytest.mark.parametrize("N", [300, 128, 1])
def test_quantiser_bit_exact(d, rotate, N):
    say(f"case quant d={d} rotate={rotate} N={N}")
    q, _, _, signs = inputs.draw_fp8_workload(20 + N % 13, 2, 3, N, d)
    tx, x = bf16_activations(q)
    if N >= 256:
        tx[1, 2, 128:256] = 0                     # an all-zero block
        x = tx.float().numpy()
    sg = torch.from_numpy(signs).cuda() if rotate else None
    codes, scales = attn_quant_fp8(tx.cuda(), sg)
    torch.cuda.synchronize()
    xr = ofp8.rotate_f32(x, signs) if rotate else x
    ref_codes, ref_scales = ofp8.quantize_blocks(xr)
    np.testing.assert_array_equal(scales.cpu().numpy(), ref_scales)
    got = codes.cpu().numpy()
    bad = np.count_nonzero(got != ref_codes)
    say(f"  codes differing: {bad} of {got.size}")
    assert bad == 0


@pytest.mark.parametrize("rotate", [True, False])
def test_quantiser_tiny_block_scales_bit_exact(rotate):
    # Blocks whose scale amax/448 is tiny: below 2^-64, at the bottom of the fp32 normal
    # range, and subnormal (bf16 inputs that are themselves subnormal). The division by
    # such a scale must still be the correctly rounded quotient of every element.
    B, H, N, d = 1, 2, 640, 128
    say(f"case quant tiny scales rotate={rotate}")
    x = inputs.normal_f32(61, 0, (B, H, N, d))
    for blk, f in enumerate([1e-37, 1e-30, 1e-39, 3e-41, 1.0]):
        x[:, :, blk * 128:(blk + 1) * 128] *= np.float32(f)
    tx, xf = bf16_activations(x)
    signs = np.where(inputs.generator(61, inputs.SIGN_ID).integers(0, 2, size=d) == 1, 1.0, -1.0).astype(np.float32)
    codes, scales = attn_quant_fp8(tx.cuda(), torch.from_numpy(signs).cuda() if rotate else None)
    torch.cuda.synchronize()
    xr = ofp8.rotate_f32(xf, signs) if rotate else xf
    ref_codes, ref_scales = ofp8.quantize_blocks(xr)
    say(f"  scales {ref_scales[0, 0]}")
    assert (ref_scales[0, 0, :3] < 2.0 ** -64).all() and ref_scales[0, 0, 2] < np.finfo(np.float32).tiny
    np.testing.assert_array_equal(scales.cpu().numpy(), ref_scales)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_codes)


def test_quantiser_full_size_c5_sampled_heads():
    w = inputs.WORKLOADS["C5"]
    say("case quant C5 full size")
    q, k, v, signs = inputs.draw_fp8_workload(w.wid, w.B, w.H, w.N, w.d)
    sg = torch.from_numpy(signs).cuda()
    for name, x32, rot in (("q", q, True), ("k", k, True), ("v", v, False)):
        tx, x = bf16_activations(x32)
        codes, scales = attn_quant_fp8(tx.cuda(), sg if rot else None)
        torch.cuda.synchronize()
        for b, h in ((0, 0), (w.B - 1, w.H - 1), (1, 5)):
            xs = x[b:b + 1, h:h + 1]
            xr = ofp8.rotate_f32(xs, signs) if rot else xs
            rc, rs = ofp8.quantize_blocks(xr)
            np.testing.assert_array_equal(scales[b:b + 1, h:h + 1].cpu().numpy(), rs)
            np.testing.assert_array_equal(codes[b:b + 1, h:h + 1].cpu().numpy(), rc)
        say(f"  {name}: sampled heads bit-exact")


def oracle_inputs(wid, B, H, N, d):
    q, k, v, signs = inputs.draw_fp8_workload(wid, B, H, N, d)
    xs = [bf16_activations(t)[1] for t in (q, k, v)]
    p = ofp8.prepare_fp8(*xs, signs)
    deq = [ofp8.dequantize_blocks(p[c], p[s]) for c, s in (("q8", "sq"), ("k8", "sk"), ("v8", "sv"))]
    return p, deq, xs, signs


def run_fp8(p, causal, scale):
    t = {key: torch.from_numpy(np.ascontiguousarray(val)).cuda() for key, val in p.items()}
    o, lse = attn_fwd_fp8(t["q8"], t["k8"], t["v8"], t["sq"], t["sk"], t["sv"], causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def compare(O, L, Oref, Lref, label):
    assert np.isfinite(O).all() and np.isfinite(L).all()
    eo = np.abs(O - Oref).max()
    el = (np.abs(L - Lref) / np.maximum(1, np.abs(Lref))).max()
    say(f"  {label}: max|dO|={eo:.3e} max rel dLSE={el:.3e}")
    assert eo <= O_TOL_FP8
    assert el <= LSE_REL


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 2, 1000, 128), (2, 2, 256, 128), (1, 1, 77, 128), (1, 1, 1, 128),
                                   (1, 2, 1000, 64), (2, 2, 256, 64), (1, 1, 77, 64), (1, 1, 1, 64)])
def test_fp8_attention_small(shape, causal):
    B, H, N, d = shape
    say(f"case fp8 attention shape={shape} causal={causal}")
    p, deq, _, _ = oracle_inputs(30 + N % 11, B, H, N, d)
    scale = inputs.softmax_scale(d)
    O, L = run_fp8(p, causal, scale)
    Oref, Lref = attention_forward(*deq, causal, scale)
    compare(O, L, Oref, Lref, f"fp8 {shape} causal={causal}")


def test_fp8_attention_c5_every_row():
    # The fp8 workload on every one of its 32 heads and every row (the oracle runs on the
    # dequantised codes the device reads).
    w = inputs.WORKLOADS["C5"]
    say("case fp8 attention C5: every head, every row")
    p, deq, _, _ = oracle_inputs(w.wid, w.B, w.H, w.N, w.d)
    O, L = run_fp8(p, True, w.scale)
    Oref, Lref = forward_pooled(*deq, True, w.scale)
    compare(O, L, Oref, Lref, "C5 every row")


def test_fp8_end_to_end_gpu_quantiser():
    # GPU quantiser -> GPU fp8 attention, against oracle quantiser -> oracle attention.
    B, H, N, d = 1, 2, 640, 128
    p, deq, xs, signs = oracle_inputs(41, B, H, N, d)
    sg = torch.from_numpy(signs).cuda()
    tq, tk, tv = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in xs)
    q8, sq = attn_quant_fp8(tq, sg)
    k8, sk = attn_quant_fp8(tk, sg)
    v8, sv = attn_quant_fp8(tv, None)
    o, lse = attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=True)
    torch.cuda.synchronize()
    Oref, Lref = attention_forward(*deq, True, inputs.softmax_scale(d))
    compare(o.double().cpu().numpy(), lse.double().cpu().numpy(), Oref, Lref, "end-to-end")


def test_binding_rejects_bad_output_tensors():
    # The binding checks caller-provided outputs before any call into the library.
    x = torch.zeros((1, 1, 256, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        attn_quant_fp8(x, None, out=torch.empty((1, 1, 256, 128), dtype=torch.int8, device="cuda"))
    with pytest.raises(ValueError):
        attn_quant_fp8(x, None, scales=torch.empty((1, 1, 1), dtype=torch.float32, device="cuda"))
    q8, sq = attn_quant_fp8(x, None)
    with pytest.raises(ValueError):
        attn_fwd_fp8(q8, q8, q8, sq, sq, sq, out=torch.empty((1, 1, 256, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        attn_fwd_fp8(q8, q8, q8, sq, sq, sq, lse=torch.empty((1, 1, 256), dtype=torch.float32))
    torch.cuda.synchronize()


def test_rotation_lowers_fp8_error_with_outliers():
    # Direction of the incoherent-processing claim ("8.3 FlashAttention-3", section 5.2):
    # with outlier channels shared by Q and K, the fp8 path's error against exact
    # attention on the unquantised inputs is lower with the Hadamard rotation than without.
    B, H, N, d = 1, 4, 1024, 128
    q, k, v, signs = inputs.draw_fp8_workload(50, B, H, N, d)
    xs = [bf16_activations(t)[1] for t in (q, k, v)]
    scale = inputs.softmax_scale(d)
    Oexact, _ = attention_forward(*xs, True, scale)
    errs = {}
    for rot in (True, False):
        p = ofp8.prepare_fp8(*xs, signs, rotate=rot)
        O, _ = run_fp8(p, True, scale)
        errs[rot] = np.sqrt(np.mean((O - Oexact) ** 2))
    say(f"  RMSE with rotation {errs[True]:.4e}, without {errs[False]:.4e}, ratio {errs[False] / errs[True]:.2f}")
    assert errs[True] < errs[False]


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("factor", [1.5, 4.0, 30.0])
def test_fp8_scores_jumping_past_the_first_tile_max(factor, causal, d):
    # K activations from key 300 on are scaled up before quantisation, so their scores rise
    # far above the first key tile's row max (x4, x30), or a little above it for some rows
    # (x1.5). The running max must then move, with the accumulators rescaled, so that the
    # E4M3 codes of the probabilities stay in range.
    B, H, N = 1, 2, 700
    say(f"case fp8 jumping scores x{factor} causal={causal} d={d}")
    q, k, v, signs = inputs.draw_fp8_workload(52, B, H, N, d)
    k = k.copy()
    k[:, :, 300:] *= np.float32(factor)
    xs = [bf16_activations(t)[1] for t in (q, k, v)]
    p = ofp8.prepare_fp8(*xs, signs)
    deq = [ofp8.dequantize_blocks(p[c], p[s]) for c, s in (("q8", "sq"), ("k8", "sk"), ("v8", "sv"))]
    scale = inputs.softmax_scale(d)
    O, L = run_fp8(p, causal, scale)
    Oref, Lref = attention_forward(*deq, causal, scale)
    compare(O, L, Oref, Lref, f"fp8 jump x{factor} causal={causal}")


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_v_block_scales_far_apart(causal):
    # V's 128-row blocks are scaled by factors between 1/64 and 5/4 before quantisation, so
    # neighbouring V block scales differ by up to 64x: where the ratio of a block's scale to
    # the accumulator's unit leaves [1/4, 3/2] the accumulator changes unit, elsewhere the
    # ratio rides in the exp2 argument. Both must give the weights the oracle uses.
    B, H, N, d = 1, 2, 1300, 128
    say(f"case fp8 V block scales far apart causal={causal}")
    q, k, v, signs = inputs.draw_fp8_workload(53, B, H, N, d)
    v = v.copy()
    f = np.array([1, 1 / 16, 1, 0.5, 1 / 64, 0.75, 1, 1 / 8, 1.25, 1 / 32, 1, 0.3], dtype=np.float32)
    for b in range((N + 127) // 128):
        v[:, :, b * 128:(b + 1) * 128] *= f[b % len(f)]
    xs = [bf16_activations(t)[1] for t in (q, k, v)]
    p = ofp8.prepare_fp8(*xs, signs)
    sv = p["sv"][0, 0]
    assert sv.max() / sv.min() > 32
    deq = [ofp8.dequantize_blocks(p[c], p[s]) for c, s in (("q8", "sq"), ("k8", "sk"), ("v8", "sv"))]
    scale = inputs.softmax_scale(d)
    O, L = run_fp8(p, causal, scale)
    Oref, Lref = attention_forward(*deq, causal, scale)
    compare(O, L, Oref, Lref, f"fp8 V block scales far apart causal={causal}")


def test_rotation_study_across_outlier_layouts():
    # fp8 error against exact attention on the unquantised inputs, with and without the
    # Hadamard rotation, for four outlier layouts ("8.3 FlashAttention-3", section 5.2
    # claims lower error with the rotation; its workload is unspecified). The GPU path
    # runs end to end (quantiser and attention); only the shared-channel layout, the
    # setting the section describes, must show the claimed direction. The ratios are
    # printed for the record.
    B, H, N, d = 1, 4, 1024, 128
    scale = inputs.softmax_scale(d)
    layouts = {
        "shared channels": inputs.draw_fp8_workload(53, B, H, N, d),
        "independent channels": inputs.draw_fp8_workload(53, B, H, N, d, shared_channels=False),
        "1% of entries": inputs.draw_fp8_entry_outliers(53, B, H, N, d),
        "no outliers": inputs.draw_fp8_workload(53, B, H, N, d, mult=1.0),
    }
    ratios = {}
    for name, (q, k, v, signs) in layouts.items():
        xs = [bf16_activations(t) for t in (q, k, v)]
        Oexact, _ = attention_forward(*[x[1] for x in xs], True, scale)
        sg = torch.from_numpy(signs).cuda()
        errs = {}
        for rot in (True, False):
            q8, sq = attn_quant_fp8(xs[0][0].cuda(), sg if rot else None)
            k8, sk = attn_quant_fp8(xs[1][0].cuda(), sg if rot else None)
            v8, sv = attn_quant_fp8(xs[2][0].cuda(), None)
            o, _ = attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=True, scale=scale)
            torch.cuda.synchronize()
            errs[rot] = float(np.sqrt(np.mean((o.double().cpu().numpy() - Oexact) ** 2)))
        ratios[name] = errs[False] / errs[True]
        say(f"  {name}: RMSE rotated {errs[True]:.4e}, unrotated {errs[False]:.4e}, "
            f"unrotated/rotated {ratios[name]:.2f}")
    assert ratios["shared channels"] > 1.0


def test_tensors_over_2_31_elements():
    # B1 H4100 N4096 d128: the bf16 activations and the E4M3 codes each hold 2.15e9
    # elements (> 2^31), so the heads past 4096 sit beyond 32-bit element offsets. Q and K
    # are rotated and quantised on the device, V quantised, then fp8 attention (causal).
    # Three heads (first, middle, last) are read back: codes and scales bit-exact against
    # the oracle's quantiser, O and LSE against the oracle on sampled rows.
    B, H, N, d = 1, 4100, 4096, 128
    assert B * H * N * d > 2**31
    say(f"case >2^31 elements fp8: B{B} H{H} N{N} d{d} causal")
    xs = [inputs.normal_on_device(43, t, (B, H, N, d), torch.bfloat16) for t in range(3)]
    signs = np.where(inputs.generator(43, inputs.SIGN_ID).integers(0, 2, size=d) == 1, 1.0, -1.0).astype(np.float32)
    sg = torch.from_numpy(signs).cuda()
    q8, sq = attn_quant_fp8(xs[0], sg)
    k8, sk = attn_quant_fp8(xs[1], sg)
    v8, sv = attn_quant_fp8(xs[2], None)
    scale = inputs.softmax_scale(d)
    o, lse = attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=True, scale=scale)
    torch.cuda.synchronize()
    hs = [0, H // 2, H - 1]
    acts = [x[:, hs].float().cpu().numpy() for x in xs]
    got = {n: t[:, hs].cpu().numpy() for n, t in (("q8", q8), ("sq", sq), ("k8", k8), ("sk", sk), ("v8", v8), ("sv", sv))}
    O = o[:, hs].double().cpu().numpy()
    L = lse[:, hs].double().cpu().numpy()
    del xs, q8, k8, v8, sq, sk, sv, o, lse
    torch.cuda.empty_cache()
    p = ofp8.prepare_fp8(*acts, signs)
    for n in ("q8", "sq", "k8", "sk", "v8", "sv"):
        np.testing.assert_array_equal(got[n], p[n])
    deq = [ofp8.dequantize_blocks(p[c], p[s]) for c, s in (("q8", "sq"), ("k8", "sk"), ("v8", "sv"))]
    rows = np.unique(np.concatenate([np.arange(0, 4), [255, 256, N - 1], np.random.default_rng(13).integers(0, N, 24)]))
    Oref, Lref = attention_forward(*deq, True, scale, rows=rows)
    compare(O[:, :, rows], L[:, :, rows], Oref, Lref, f"heads {hs}: quantiser bit-exact")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("N", [300, 1000, 1])
def test_quant_kv_one_launch_bit_exact(N, d):
    # K rotated and V unrotated in one launch: the codes and scales of the oracle's quantiser
    say(f"case quant kv N={N} d={d}")
    _, k, v, signs = inputs.draw_fp8_workload(24 + N % 7, 2, 3, N, d)
    tk, kx = bf16_activations(k)
    tv, vx = bf16_activations(v)
    k8, sk, v8, sv = attn_quant_fp8_kv(tk.cuda(), tv.cuda(), torch.from_numpy(signs).cuda())
    torch.cuda.synchronize()
    rk, rsk = ofp8.quantize_blocks(ofp8.rotate_f32(kx, signs))
    rv, rsv = ofp8.quantize_blocks(vx)
    for got, ref in ((k8, rk), (sk, rsk), (v8, rv), (sv, rsv)):
        np.testing.assert_array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("N", [300, 1000, 1])
def test_quant_qkv_one_launch_bit_exact(N, d):
    # Q and K rotated and V unrotated in one launch: the codes and scales of the oracle's
    # quantiser for each
    say(f"case quant qkv N={N} d={d}")
    q, k, v, signs = inputs.draw_fp8_workload(31 + N % 5, 2, 3, N, d)
    (tq, qx), (tk, kx), (tv, vx) = (bf16_activations(t) for t in (q, k, v))
    outs = attn_quant_fp8_qkv(tq.cuda(), tk.cuda(), tv.cuda(), torch.from_numpy(signs).cuda())
    torch.cuda.synchronize()
    refs = (*ofp8.quantize_blocks(ofp8.rotate_f32(qx, signs)), *ofp8.quantize_blocks(ofp8.rotate_f32(kx, signs)),
            *ofp8.quantize_blocks(vx))
    for got, ref in zip(outs, refs):
        np.testing.assert_array_equal(got.cpu().numpy(), ref)


def test_quant_qkv_full_size_equals_three_launches():
    # The fp8 workload's shape: one launch gives the bytes of the three single-tensor calls
    w = inputs.WORKLOADS["C5"]
    say("case quant qkv C5 vs three attn_quant_fp8 calls")
    q, k, v, signs = inputs.draw_fp8_workload(w.wid, w.B, w.H, w.N, w.d)
    tq, tk, tv = (inputs.to_torch(x, "bf16").cuda() for x in (q, k, v))
    sg = torch.from_numpy(signs).cuda()
    one = attn_quant_fp8_qkv(tq, tk, tv, sg)
    three = (*attn_quant_fp8(tq, sg), *attn_quant_fp8(tk, sg), *attn_quant_fp8(tv, None))
    torch.cuda.synchronize()
    for a, b in zip(one, three):
        assert torch.equal(a, b)


def fused_case(wid, B, H, N, d, tweak=None):
    q, k, v, signs = inputs.draw_fp8_workload(wid, B, H, N, d)
    if tweak is not None:
        tweak(q)
    xs = [bf16_activations(t) for t in (q, k, v)]
    sg = torch.from_numpy(signs).cuda()
    gq, gk, gv = (x[0].cuda() for x in xs)
    k8, sk, v8, sv = attn_quant_fp8_kv(gk, gv, sg)
    return xs, signs, sg, gq, (k8, sk, v8, sv)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 2, 1000, 128), (2, 2, 256, 128), (1, 1, 77, 128), (1, 1, 1, 128),
                                   (1, 3, 300, 128), (1, 2, 1000, 64), (1, 3, 300, 64), (1, 1, 1, 64)])
def test_fused_q_preparation(shape, causal):
    # The attention kernel rotates and quantises Q itself: its codes and scales equal the
    # oracle's quantiser bit for bit (also for an all-zero block and a block whose scale is
    # subnormal), its O and LSE equal attn_fwd_fp8's on the separately quantised Q bit for
    # bit, and both meet the fp8 gate against the oracle.
    B, H, N, d = shape
    say(f"case fused Q shape={shape} causal={causal}")

    def tweak(q):
        if N >= 256 and H >= 3:
            q[0, 2, 128:256] = 0.0
            q[0, 1, 0:128] *= np.float32(1e-39)
    xs, signs, sg, gq, (k8, sk, v8, sv) = fused_case(34 + N % 5, B, H, N, d, tweak)
    scale = inputs.softmax_scale(d)
    nblk = (N + 127) // 128
    q8o = torch.full((B, H, N, d), 0x7F, dtype=torch.uint8, device="cuda")
    sqo = torch.full((B, H, nblk), float("nan"), dtype=torch.float32, device="cuda")
    o_f, l_f = attn_fwd_fp8_rotq(gq, sg, k8, v8, sk, sv, causal=causal, scale=scale, q8_out=q8o, q_scale_out=sqo)
    q8, sq = attn_quant_fp8(gq, sg)
    o_s, l_s = attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rsq = ofp8.quantize_blocks(ofp8.rotate_f32(xs[0][1], signs))
    np.testing.assert_array_equal(q8o.cpu().numpy(), rq)
    np.testing.assert_array_equal(sqo.cpu().numpy(), rsq)
    assert torch.equal(o_f, o_s) and torch.equal(l_f, l_s)
    p = {"q8": rq, "sq": rsq, "k8": k8.cpu().numpy(), "sk": sk.cpu().numpy(), "v8": v8.cpu().numpy(),
         "sv": sv.cpu().numpy()}
    deq = [ofp8.dequantize_blocks(p[c], p[s_]) for c, s_ in (("q8", "sq"), ("k8", "sk"), ("v8", "sv"))]
    Oref, Lref = attention_forward(*deq, causal, scale)
    compare(o_f.double().cpu().numpy(), l_f.double().cpu().numpy(), Oref, Lref, f"fused Q {shape} causal={causal}")


def test_fused_fp8_path_c5_every_row():
    # The fp8 workload through the two-launch path (K/V quantiser, attention with fused Q
    # preparation) against the oracle on every head and every row.
    w = inputs.WORKLOADS["C5"]
    say("case fused fp8 path C5: every head, every row")
    xs, signs, sg, gq, (k8, sk, v8, sv) = fused_case(w.wid, w.B, w.H, w.N, w.d)
    o, lse = attn_fwd_fp8_rotq(gq, sg, k8, v8, sk, sv, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    p = ofp8.prepare_fp8(*[x[1] for x in xs], signs)
    for name, t in (("k8", k8), ("sk", sk), ("v8", v8), ("sv", sv)):
        np.testing.assert_array_equal(t.cpu().numpy(), p[name])
    deq = [ofp8.dequantize_blocks(p[c], p[s_]) for c, s_ in (("q8", "sq"), ("k8", "sk"), ("v8", "sv"))]
    Oref, Lref = forward_pooled(*deq, True, w.scale)
    compare(o.double().cpu().numpy(), lse.double().cpu().numpy(), Oref, Lref, "C5 fused path, every row")


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_head_dim_64_every_row(causal):
    # fp8 at head dim 64 on B2 H16 N8192 (the fp8 workload's shape with d = 64, the same
    # outlier recipe): the separate path and the fused-Q path, every head and every row.
    B, H, N, d = 2, 16, 8192, 64
    say(f"case fp8 d64 B{B} H{H} N{N} causal={causal}: every head, every row")
    xs, signs, sg, gq, (k8, sk, v8, sv) = fused_case(15, B, H, N, d)
    scale = inputs.softmax_scale(d)
    q8, sq = attn_quant_fp8(gq, sg)
    o_s, l_s = attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=causal, scale=scale)
    o_f, l_f = attn_fwd_fp8_rotq(gq, sg, k8, v8, sk, sv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_s) and torch.equal(l_f, l_s)
    p = ofp8.prepare_fp8(*[x[1] for x in xs], signs)
    for name, t in (("q8", q8), ("sq", sq), ("k8", k8), ("sk", sk), ("v8", v8), ("sv", sv)):
        np.testing.assert_array_equal(t.cpu().numpy(), p[name])
    deq = [ofp8.dequantize_blocks(p[c], p[s_]) for c, s_ in (("q8", "sq"), ("k8", "sk"), ("v8", "sv"))]
    Oref, Lref = forward_pooled(*deq, causal, scale)
    compare(o_f.double().cpu().numpy(), l_f.double().cpu().numpy(), Oref, Lref, f"fp8 d64 causal={causal}")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_row_dominated_by_one_key(causal, d):
    # Closed form, no oracle. Key k is +-16 (E4M3) on channel k % d (+ for k < d, - above);
    # query i is +-16 on the channel of its chosen key kappa(i) (kappa(i) <= i when causal),
    # so kappa(i) scores 256, its sign twin -256 and every other key 0. Softmax then gives
    # V's dequantised row kappa(i) up to N * exp(-256 * scale) * max|V| (every other key's
    # weight is at most exp(-256 * scale) of kappa's), and LSE = 256 * scale. The kernel
    # codes kappa's probability exactly (2^6) and carries keys seen before the row max
    # reached kappa's tile down by the same rescale, so it meets that bound; a denominator
    # summed over another row's codes would scale the row instead.
    B, H, N = 1, 2, 2 * d - 3                      # d = 128: two V scale blocks, ragged tail
    say(f"case fp8 row dominated by one key causal={causal} d={d} N={N}")
    rng = np.random.default_rng(7800 + d + int(causal))
    keys = np.arange(N)
    q8 = np.zeros((B, H, N, d), np.uint8)
    k8 = np.zeros((B, H, N, d), np.uint8)
    v8 = rng.integers(0, 256, size=(B, H, N, d)).astype(np.uint8)
    v8[(v8 & 0x7F) == 0x7F] = 0                    # no NaN codes
    kappa = np.zeros((H, N), np.int64)
    for h in range(H):
        k8[0, h, keys, keys % d] = np.where(keys < d, 0x58, 0xD8).astype(np.uint8)
        kappa[h] = (rng.random(N) * (keys + 1)).astype(np.int64) if causal else rng.integers(0, N, size=N)
        q8[0, h, keys, kappa[h] % d] = np.where(kappa[h] < d, 0x58, 0xD8).astype(np.uint8)
    nblk = (N + 127) // 128
    ones = torch.ones((B, H, nblk), dtype=torch.float32)
    sv = (0.5 * 6.0 ** torch.arange(nblk, dtype=torch.float32)).expand(B, H, nblk).contiguous()
    scale = inputs.softmax_scale(d)
    dev = lambda a: torch.from_numpy(a).cuda()
    O, L = attn_fwd_fp8(dev(q8), dev(k8), dev(v8), ones.cuda(), ones.cuda(), sv.cuda(), causal=causal,
                        scale=scale)
    torch.cuda.synchronize()
    vdq = torch.from_numpy(v8).view(torch.float8_e4m3fn).double() * sv.double().repeat_interleave(128, dim=2)[:, :, :N, None]
    expect = np.stack([vdq[0, h].numpy()[kappa[h]] for h in range(H)])[None]
    got = O.double().cpu().numpy()
    err = np.abs(got - expect).max()
    bound = N * np.exp(-256.0 * float(scale)) * float(vdq.abs().max())
    say(f"  max |O - V[kappa]| = {err:.3e} (softmax's own distance from V[kappa] <= {bound:.1e})")
    assert np.all(np.abs(got - expect) <= 2.0 ** -8 * np.abs(expect) + bound), err
    lse_expect = 256.0 * float(scale)
    lerr = np.abs(L.double().cpu().numpy() - lse_expect).max()
    say(f"  max |LSE - 256 scale| = {lerr:.3e}")
    assert lerr <= LSE_REL * lse_expect, lerr
