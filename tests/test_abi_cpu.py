"""The C-ABI library loads on the host, exports every symbol include/attn.h declares,
and rejects bad arguments on the host before any HIP call (CPU only).

Every call below carries at least one defect that the host-side validation must catch,
so no kernel is ever launched: the fake addresses are never dereferenced.
"""

import ctypes
import math
import os
import re

import pytest
import torch

import exact_attention_78_amd as ea
from exact_attention_78_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, INVALID, UNSUPPORTED, SCRATCH = 0, 1, 2, 4

# These calls use fake addresses: run them only where no GPU is present, so that a
# validation bug can never turn one into a real launch.
no_gpu_only = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake-pointer validation runs on GPU-less hosts")
# distinct, 16-byte aligned, far-apart fake device addresses (never dereferenced)
A = [(i + 1) << 40 for i in range(10)]


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:attn_status_t|const char\*|int|int64_t)\s+(attn_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return ea.library()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = header_functions()
    assert set(names) == {"attn_fwd_bf16", "attn_fwd_f16", "attn_fwd_f32", "attn_fwd_fp8", "attn_quant_fp8",
                          "attn_fwd_variant", "attn_calibrate", "attn_calibrate_ops", "attn_decode_bf16_noalloc",
                          "attn_quant_fp8_kv", "attn_quant_fp8_qkv", "attn_fwd_fp8_rotq",
                          "attn_bwd_bf16", "attn_bwd_f16", "attn_decode_bf16", "attn_decode_f16",
                          "attn_decode_workspace_floats", "attn_status_string", "attn_abi_version"}
    for n in names:
        assert hasattr(lib, n), n
        assert n in _binding.SIGNATURES, n


def test_abi_version_and_status_strings(lib):
    ver = int(re.search(r"#define ATTN_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.attn_abi_version() == ver
    for s in range(5):
        assert lib.attn_status_string(s) and lib.attn_status_string(s) != b"unknown status"
    assert lib.attn_status_string(99) == b"unknown status"


FWD16 = ["attn_fwd_bf16", "attn_fwd_f16", "attn_fwd_f32"]


def call_fwd(lib, fn, q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], B=1, H=2, N=64, d=64, causal=1, scale=0.125):
    return getattr(lib, fn)(q, k, v, o, lse, B, H, N, d, causal, scale, None)


@no_gpu_only
@pytest.mark.parametrize("fn", FWD16)
@pytest.mark.parametrize("defect,expect", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(o=None), INVALID),
    (dict(lse=None), INVALID), (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(N=0), INVALID),
    (dict(d=0), INVALID), (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(d=32), UNSUPPORTED),
    (dict(scale=0.0), INVALID), (dict(scale=-0.5), INVALID), (dict(scale=math.nan), INVALID),
    (dict(scale=math.inf), INVALID), (dict(q=A[0] + 2), INVALID), (dict(o=A[3] + 8), INVALID),
    (dict(lse=A[4] + 4), INVALID), (dict(o=A[0]), INVALID), (dict(o=A[2] + 16), INVALID),
    (dict(lse=A[1]), INVALID), (dict(lse=A[3] + 64), INVALID),
    (dict(B=1 << 31, H=1 << 31, N=1 << 20), INVALID), (dict(N=(1 << 31) + 64), INVALID),
])
def test_fwd_validation(lib, fn, defect, expect):
    assert call_fwd(lib, fn, **defect) == expect


@no_gpu_only
@pytest.mark.parametrize("defect,expect", [
    (dict(q=None), INVALID), (dict(N=0), INVALID), (dict(d=96), UNSUPPORTED), (dict(scale=0.0), INVALID),
    (dict(o=A[0]), INVALID), (dict(dtype=2), INVALID), (dict(dtype=-1), INVALID), (dict(sched=9), INVALID),
    (dict(sched=-1), INVALID), (dict(passes=3), INVALID), (dict(passes=-1), INVALID),
    (dict(sched=7, queue=None), INVALID), (dict(sched=7, queue=A[5] + 4), INVALID),
    (dict(sched=7, queue=A[3] + 64), INVALID), (dict(sched=7, queue=A[4]), INVALID),
    (dict(sched=7, queue=A[5], N=0), INVALID),
])
def test_fwd_variant_validation(lib, defect, expect):
    args = dict(q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], B=1, H=2, N=64, d=64, causal=1, scale=0.125, dtype=0,
                sched=0, passes=0, queue=A[5])
    args.update(defect)
    assert lib.attn_fwd_variant(*args.values(), None) == expect


@no_gpu_only
@pytest.mark.parametrize("defect,expect", [
    (dict(q8=None), INVALID), (dict(sk=None), INVALID), (dict(o=None), INVALID), (dict(d=96), UNSUPPORTED),
    (dict(d=32), UNSUPPORTED),
    (dict(N=0), INVALID), (dict(scale=0.0), INVALID), (dict(sv=A[5] + 4), INVALID), (dict(o=A[0]), INVALID),
    (dict(lse=A[3]), INVALID), (dict(o=A[7] - 16), INVALID),
])
def test_fp8_validation(lib, defect, expect):
    args = dict(q8=A[0], k8=A[1], v8=A[2], sq=A[3], sk=A[4], sv=A[5], o=A[6], lse=A[7], B=1, H=1, N=256, d=128,
                causal=1, scale=0.0884)
    args.update(defect)
    assert lib.attn_fwd_fp8(*args.values(), None) == expect


@no_gpu_only
@pytest.mark.parametrize("defect,expect", [
    (dict(k=None), INVALID), (dict(signs=None), INVALID), (dict(v8=None), INVALID), (dict(sv=None), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(N=0), INVALID), (dict(k8=A[0]), INVALID), (dict(v8=A[3]), INVALID),
    (dict(sk=A[6]), INVALID), (dict(sv=A[5] + 4), INVALID), (dict(signs=A[2] + 4), INVALID),
])
def test_quant_kv_validation(lib, defect, expect):
    args = dict(k=A[0], v=A[1], signs=A[2], k8=A[3], v8=A[4], sk=A[5], sv=A[6], B=1, H=1, N=256, d=128)
    args.update(defect)
    assert lib.attn_quant_fp8_kv(*args.values(), None) == expect


@no_gpu_only
@pytest.mark.parametrize("defect,expect", [
    (dict(q=None), INVALID), (dict(v=None), INVALID), (dict(signs=None), INVALID), (dict(q8=None), INVALID),
    (dict(sv=None), INVALID), (dict(d=96), UNSUPPORTED), (dict(N=0), INVALID), (dict(q8=A[0]), INVALID),
    (dict(k8=A[1]), INVALID), (dict(v8=A[4]), INVALID), (dict(sq=A[8]), INVALID), (dict(sk=A[7] + 4), INVALID),
    (dict(signs=A[3] + 4), INVALID), (dict(sv=A[3]), INVALID),
])
def test_quant_qkv_validation(lib, defect, expect):
    args = dict(q=A[0], k=A[1], v=A[2], signs=A[3], q8=A[4], k8=A[5], v8=A[6], sq=A[7], sk=A[8], sv=A[9], B=1, H=1,
                N=256, d=128)
    args.update(defect)
    assert lib.attn_quant_fp8_qkv(*args.values(), None) == expect


@no_gpu_only
@pytest.mark.parametrize("defect,expect", [
    (dict(q=None), INVALID), (dict(signs=None), INVALID), (dict(k8=None), INVALID), (dict(o=None), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(N=0), INVALID), (dict(scale=0.0), INVALID), (dict(o=A[0]), INVALID),
    (dict(q8o=A[2]), INVALID), (dict(sqo=A[4] + 8), INVALID), (dict(q8o=A[6]), INVALID),
    (dict(q8o=A[8] + 4), INVALID), (dict(sqo=A[7]), INVALID),
])
def test_fp8_rotq_validation(lib, defect, expect):
    args = dict(q=A[0], signs=A[1], k8=A[2], v8=A[3], sk=A[4], sv=A[5], o=A[6], lse=A[7], q8o=A[8], sqo=A[9],
                B=1, H=1, N=256, d=128, causal=1, scale=0.0884)
    args.update(defect)
    assert lib.attn_fwd_fp8_rotq(*args.values(), None) == expect


@no_gpu_only
@pytest.mark.parametrize("defect,expect", [
    (dict(x=None), INVALID), (dict(x8=None), INVALID), (dict(sc=None), INVALID), (dict(d=32), UNSUPPORTED),
    (dict(d=96), UNSUPPORTED), (dict(B=0), INVALID), (dict(signs=A[3] + 4), INVALID), (dict(x8=A[0]), INVALID),
    (dict(sc=A[1] + 32), INVALID),
])
def test_quant_validation(lib, defect, expect):
    args = dict(x=A[0], x8=A[1], sc=A[2], signs=A[3], B=1, H=1, N=256, d=128)
    args.update(defect)
    assert lib.attn_quant_fp8(*args.values(), None) == expect


@no_gpu_only
@pytest.mark.parametrize("fn", ["attn_bwd_bf16", "attn_bwd_f16"])
@pytest.mark.parametrize("defect,expect", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(lse=None), INVALID), (dict(dout=None), INVALID),
    (dict(dq=None), INVALID), (dict(dv=None), INVALID), (dict(ws=None), INVALID), (dict(N=0), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=32), UNSUPPORTED), (dict(scale=0.0), INVALID), (dict(scale=math.nan), INVALID),
    (dict(dk=A[5] + 8), INVALID), (dict(ws=A[9] + 4), INVALID),
    (dict(dq=A[0]), INVALID), (dict(dk=A[3] + 64), INVALID), (dict(dv=A[5] + 16), INVALID), (dict(ws=A[4]), INVALID),
    (dict(ws=A[6] + 32), INVALID), (dict(dq=A[7]), INVALID),
    (dict(B=1 << 31, H=1 << 31, N=1 << 20), INVALID),
])
def test_bwd_validation(lib, fn, defect, expect):
    args = dict(q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], dout=A[5], dq=A[6], dk=A[7], dv=A[8], ws=A[9],
                B=1, H=2, N=64, d=64, causal=1, scale=0.125)
    args.update(defect)
    assert getattr(lib, fn)(*args.values(), None) == expect


@no_gpu_only
@pytest.mark.parametrize("fn", ["attn_decode_bf16", "attn_decode_f16"])
@pytest.mark.parametrize("defect,expect", [
    (dict(q=None), INVALID), (dict(v=None), INVALID), (dict(ws=None), INVALID), (dict(Nq=0), INVALID),
    (dict(Nq=33), INVALID), (dict(Nk=0), INVALID), (dict(d=96), UNSUPPORTED), (dict(scale=0.0), INVALID),
    (dict(o=A[0]), INVALID), (dict(lse=A[1] + 64), INVALID), (dict(ws=A[3]), INVALID), (dict(ws=A[4] + 8), INVALID),
    (dict(B=1 << 40, H=1 << 40), INVALID),
])
def test_decode_validation(lib, fn, defect, expect):
    args = dict(q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], ws=A[5], B=2, H=2, Nq=1, Nk=1000, d=128, scale=0.0884)
    args.update(defect)
    assert getattr(lib, fn)(*args.values(), None) == expect


@no_gpu_only
@pytest.mark.parametrize("defect", [dict(kind=9), dict(kind=-1), dict(seed=None), dict(out=None), dict(wg=0),
                                    dict(iters=0), dict(seed=A[0] + 4), dict(wg=1 << 33)])
def test_calibrate_validation(lib, defect):
    args = dict(kind=0, seed=A[0], out=A[1], wg=256, iters=10)
    args.update(defect)
    assert lib.attn_calibrate(*args.values(), None) == INVALID


def test_calibrate_ops(lib):
    # 8 waves x iters x 8 chains x 32x32x16x2 FLOPs; 512 lanes x iters x 16 exponentials
    assert lib.attn_calibrate_ops(0, 10) == 8 * 10 * 8 * 32768
    assert lib.attn_calibrate_ops(1, 10) == 512 * 10 * 16
    assert lib.attn_calibrate_ops(2, 10) == 8 * 10 * 16 * 32768 and lib.attn_calibrate_ops(4, 10) == 4 * 10 * 16 * 32768
    # kind 6: 256 threads x iters x 16 bytes read
    assert lib.attn_calibrate_ops(6, 10) == 256 * 10 * 16
    # kinds 7, 8: 512 lanes x iters x 16 reads of 16 or 8 bytes
    assert lib.attn_calibrate_ops(7, 10) == 512 * 10 * 16 * 16 and lib.attn_calibrate_ops(8, 10) == 512 * 10 * 16 * 8
    assert lib.attn_calibrate_ops(9, 10) == -1 and lib.attn_calibrate_ops(0, 0) == -1


@no_gpu_only
@pytest.mark.parametrize("defect,expect", [
    (dict(q=None), INVALID), (dict(lse=None), INVALID), (dict(Nq=0), INVALID), (dict(Nq=33), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(scale=0.0), INVALID), (dict(o=A[0]), INVALID), (dict(lse=A[1] + 64), INVALID),
    # partials beyond the 2^24-float static scratch: B*H = 4096 heads at Nq = 32, d = 128
    (dict(B=64, H=64, Nq=32), SCRATCH), (dict(B=2048, H=2, Nq=32, Nk=64), SCRATCH),
])
def test_decode_noalloc_validation(lib, defect, expect):
    args = dict(q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], B=2, H=2, Nq=1, Nk=1000, d=128, scale=0.0884)
    args.update(defect)
    assert lib.attn_decode_bf16_noalloc(*args.values(), None) == expect


def test_decode_noalloc_scratch_limit(lib):
    # the largest decode sizes the static scratch holds, by the workspace formula
    assert lib.attn_decode_workspace_floats(2016, 1, 32, 1 << 20, 128) <= 1 << 24
    assert lib.attn_decode_workspace_floats(64, 64, 32, 1000, 128) > 1 << 24


def test_decode_workspace_size(lib):
    # B*H*n_split*Nq*(d+1): one partial O row and LSE per (head, key chunk, query row)
    n = lib.attn_decode_workspace_floats(2, 16, 1, 8192, 128)
    assert n > 0 and n % (2 * 16 * 1 * 129) == 0
    assert lib.attn_decode_workspace_floats(2, 16, 0, 8192, 128) == -1
    assert lib.attn_decode_workspace_floats(2, 16, 33, 8192, 128) == -1


def test_binding_rejects_host_tensors_before_calling():
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ea.attn_fwd_bf16(x, x, x)
    with pytest.raises(ValueError):
        ea.fwd(x.double(), x.double(), x.double())
    with pytest.raises(ValueError):
        ea.attn_quant_fp8(x)


def test_binding_raises_when_library_missing(monkeypatch):
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", "/nonexistent/libattn.so")
    with pytest.raises(RuntimeError):
        _binding.library()
