"""ctypes binding of libattn.so: the C entry points under the same names.

Argument marshalling only: each function checks that the torch tensors it is given
match what the C ABI expects (device, dtype, shape, contiguity), hands their device
pointers and the current HIP stream to the library, and raises ``AttnError`` on a
non-OK status. No step of the attention computation happens here, and there is no
fallback: if the library is missing the calls raise.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

_lib = None

STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED", 3: "ATTN_ERR_LAUNCH",
          4: "ATTN_ERR_SCRATCH_TOO_SMALL"}

# Exported symbols and their C signatures (mirrors include/attn.h).
_P, _I64, _INT, _F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
SIGNATURES = {
    "attn_fwd_bf16": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _INT, _F32, _P],
    "attn_fwd_f16": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _INT, _F32, _P],
    "attn_fwd_f32": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _INT, _F32, _P],
    "attn_fwd_variant": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _INT, _F32, _INT, _INT, _INT, _P, _P],
    "attn_fwd_fp8": [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _INT, _F32, _P],
    "attn_quant_fp8": [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P],
    "attn_quant_fp8_kv": [_P] * 7 + [_I64, _I64, _I64, _I64, _P],
    "attn_quant_fp8_qkv": [_P] * 10 + [_I64, _I64, _I64, _I64, _P],
    "attn_fwd_fp8_rotq": [_P] * 10 + [_I64, _I64, _I64, _I64, _INT, _F32, _P],
    "attn_bwd_bf16": [_P] * 10 + [_I64, _I64, _I64, _I64, _INT, _F32, _P],
    "attn_bwd_f16": [_P] * 10 + [_I64, _I64, _I64, _I64, _INT, _F32, _P],
    "attn_decode_bf16": [_P] * 6 + [_I64, _I64, _I64, _I64, _I64, _F32, _P],
    "attn_decode_f16": [_P] * 6 + [_I64, _I64, _I64, _I64, _I64, _F32, _P],
    "attn_decode_workspace_floats": [_I64, _I64, _I64, _I64, _I64],
    "attn_decode_bf16_noalloc": [_P] * 5 + [_I64, _I64, _I64, _I64, _I64, _F32, _P],
    "attn_calibrate": [_INT, _P, _P, _I64, _INT, _P],
    "attn_calibrate_ops": [_INT, _INT],
    "attn_status_string": [_INT],
    "attn_abi_version": [],
}


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({library().attn_status_string(status).decode()})")


def library():
    """Load libattn.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with exact_attention_78_amd.build.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = {"attn_status_string": ctypes.c_char_p, "attn_decode_workspace_floats": ctypes.c_int64,
                          "attn_calibrate_ops": ctypes.c_int64}.get(name, ctypes.c_int)
        _lib = lib
    return _lib


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise AttnError(fn, status)


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _qkv_checks(q, k, v, dtype):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
        _require(t.is_cuda, f"{name} must be on a GPU")
        _require(t.dtype == dtype, f"{name} must be {dtype}")
        _require(t.dim() == 4 and t.shape == q.shape, f"{name} must be [B, H, N, d] like q")
        _require(t.is_contiguous(), f"{name} must be contiguous")
        _require(t.device == q.device, f"{name} must be on q's device")


def _fwd(fn: str, dtype, q, k, v, causal: bool, scale, out=None, lse=None):
    _qkv_checks(q, k, v, dtype)
    B, H, N, d = q.shape
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    o = torch.empty_like(q) if out is None else out
    L = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _require(o.shape == q.shape and o.dtype == dtype and o.is_contiguous() and o.device == q.device, "bad out")
    _require(L.shape == (B, H, N) and L.dtype == torch.float32 and L.is_contiguous() and L.device == q.device,
             "bad lse")
    with torch.cuda.device(q.device):
        st = getattr(library(), fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), L.data_ptr(),
                                    B, H, N, d, int(bool(causal)), float(scale), _stream(q))
    _check(fn, st)
    return o, L


def attn_fwd_bf16(q, k, v, causal=False, scale=None, out=None, lse=None):
    """bf16 exact attention forward; returns (O bf16 [B,H,N,d], LSE fp32 [B,H,N])."""
    return _fwd("attn_fwd_bf16", torch.bfloat16, q, k, v, causal, scale, out, lse)


def attn_fwd_f16(q, k, v, causal=False, scale=None, out=None, lse=None):
    """fp16 exact attention forward; returns (O fp16, LSE fp32)."""
    return _fwd("attn_fwd_f16", torch.float16, q, k, v, causal, scale, out, lse)


def attn_fwd_f32(q, k, v, causal=False, scale=None, out=None, lse=None):
    """fp32 exact attention forward; returns (O fp32, LSE fp32)."""
    return _fwd("attn_fwd_f32", torch.float32, q, k, v, causal, scale, out, lse)


# attn_sched_t / attn_passes_t / attn_dtype_t of attn.h
SCHEDULES = {"default": 0, "xcd_all_heads": 1, "xcd_head": 2, "xcd_natural": 3, "linear_longest": 4,
             "linear_natural": 5, "persistent_stride": 6, "persistent_queue": 7, "persistent_snake": 8}
PASSES = {"auto": 0, "exact": 1, "two": 2}


def queue_workspace(device=None):
    """Zeroed queue memory for the persistent-queue schedule (16 int32 values); each call
    returns it to zero, so one tensor serves every call on one stream."""
    return torch.zeros(16, dtype=torch.int32, device=device if device is not None else "cuda")


def attn_fwd_variant(q, k, v, causal=False, scale=None, sched="default", passes="auto", queue=None, out=None,
                     lse=None):
    """16-bit forward with a chosen tile schedule and pass selection (same O and LSE as
    attn_fwd_bf16 / attn_fwd_f16). ``queue`` (from ``queue_workspace``) is required for
    sched="persistent_queue"."""
    _require(q.dtype in (torch.bfloat16, torch.float16), "q must be bf16 or fp16")
    _qkv_checks(q, k, v, q.dtype)
    _require(sched in SCHEDULES, f"sched must be one of {sorted(SCHEDULES)}")
    _require(passes in PASSES, f"passes must be one of {sorted(PASSES)}")
    B, H, N, d = q.shape
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    o = torch.empty_like(q) if out is None else out
    L = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _require(o.shape == q.shape and o.dtype == q.dtype and o.is_contiguous() and o.device == q.device, "bad out")
    _require(L.shape == (B, H, N) and L.dtype == torch.float32 and L.is_contiguous() and L.device == q.device,
             "bad lse")
    qp = None
    if sched == "persistent_queue":
        _require(isinstance(queue, torch.Tensor) and queue.dtype == torch.int32 and queue.numel() >= 16
                 and queue.is_contiguous() and queue.device == q.device,
                 "persistent_queue needs queue = queue_workspace(device)")
        qp = queue.data_ptr()
    with torch.cuda.device(q.device):
        st = library().attn_fwd_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), L.data_ptr(),
                                        B, H, N, d, int(bool(causal)), float(scale),
                                        0 if q.dtype == torch.bfloat16 else 1, SCHEDULES[sched], PASSES[passes], qp,
                                        _stream(q))
    _check("attn_fwd_variant", st)
    return o, L


# attn_calibrate kinds (see attn.h): the dense loops, and MFMA loops with the kernels' mix
# of work between MFMAs (one fma, exp and add each; LDS reads per MFMA; waves per SIMD)
CALIBRATION_KINDS = {"mfma": 0, "exp": 1, "mix_lds1_2w": 2, "mix_lds0.5_2w": 3, "mix_lds0.5_1w": 4,
                     "mix_nolds_2w": 5, "read": 6, "lds_b128": 7, "lds_tr_b64": 8}


def attn_calibrate(kind, workgroups, iters, seed=None, out=None):
    """Launch a calibration loop (a key of CALIBRATION_KINDS) on the current stream; returns
    the output tensor and the operations it performs (FLOPs, exponentials for "exp", bytes
    read for "read" and the LDS kinds). For "read", ``seed`` is the buffer the loop streams through
    (workgroups * 256 * iters 16-byte elements; zeros of that size by default)."""
    k = CALIBRATION_KINDS[kind]
    dev = torch.device("cuda", torch.cuda.current_device())
    if seed is None:
        seed = torch.zeros(workgroups * 256 * iters * 4, dtype=torch.int32, device=dev) if kind == "read" else \
            torch.tensor([0x3F803F80, 0x3F003F00, 0x3F403F40, 0x3E803E80], dtype=torch.int64).to(torch.int32).to(dev)
    need = workgroups * 256 * iters * 16 if kind == "read" else 16
    _require(seed.is_cuda and seed.is_contiguous() and seed.numel() * seed.element_size() >= need,
             f"seed: a contiguous GPU buffer of at least {need} bytes")
    out = torch.empty(workgroups * 512, dtype=torch.float32, device=dev) if out is None else out
    _require(out.numel() >= workgroups * 512 and out.dtype == torch.float32, "out: workgroups * 512 fp32 values")
    st = library().attn_calibrate(k, seed.data_ptr(), out.data_ptr(), workgroups, iters,
                                  torch.cuda.current_stream(dev).cuda_stream)
    _check("attn_calibrate", st)
    return out, library().attn_calibrate_ops(k, iters) * workgroups


def fwd(q, k, v, causal=False, scale=None, out=None, lse=None):
    """Dispatch on q.dtype to attn_fwd_{bf16,f16,f32}."""
    fn = {torch.bfloat16: attn_fwd_bf16, torch.float16: attn_fwd_f16, torch.float32: attn_fwd_f32}.get(q.dtype)
    _require(fn is not None, f"unsupported dtype {q.dtype}")
    return fn(q, k, v, causal, scale, out, lse)


def _bwd(fn: str, dtype, q, k, v, o, lse, dout, causal: bool, scale, dq=None, dk=None, dv=None, workspace=None):
    _qkv_checks(q, k, v, dtype)
    B, H, N, d = q.shape
    for name, t in (("o", o), ("dout", dout)):
        _require(isinstance(t, torch.Tensor) and t.dtype == dtype and t.shape == q.shape and t.is_contiguous()
                 and t.device == q.device, f"{name} must be a contiguous {dtype} [B, H, N, d] tensor on q's device")
    _require(isinstance(lse, torch.Tensor) and lse.dtype == torch.float32 and lse.shape == (B, H, N)
             and lse.is_contiguous() and lse.device == q.device, "lse must be fp32 [B, H, N] on q's device")
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    grads = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        t = torch.empty_like(q) if t is None else t
        _require(t.shape == q.shape and t.dtype == dtype and t.is_contiguous() and t.device == q.device, f"bad {name}")
        grads.append(t)
    ws = torch.empty((2, B, H, N), dtype=torch.float32, device=q.device) if workspace is None else workspace
    _require(ws.dtype == torch.float32 and ws.numel() >= 2 * B * H * N and ws.is_contiguous()
             and ws.device == q.device, "workspace must be a contiguous fp32 tensor of 2*B*H*N elements")
    with torch.cuda.device(q.device):
        st = getattr(library(), fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    dout.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
                                    ws.data_ptr(), B, H, N, d, int(bool(causal)), float(scale), _stream(q))
    _check(fn, st)
    return tuple(grads)


def attn_bwd_bf16(q, k, v, o, lse, dout, causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None):
    """Backward pass of attn_fwd_bf16 (o, lse from that call); returns (dq, dk, dv), bf16."""
    return _bwd("attn_bwd_bf16", torch.bfloat16, q, k, v, o, lse, dout, causal, scale, dq, dk, dv, workspace)


def attn_bwd_f16(q, k, v, o, lse, dout, causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None):
    """Backward pass of attn_fwd_f16; returns (dq, dk, dv), fp16."""
    return _bwd("attn_bwd_f16", torch.float16, q, k, v, o, lse, dout, causal, scale, dq, dk, dv, workspace)


def bwd(q, k, v, o, lse, dout, causal=False, scale=None):
    """Dispatch on q.dtype to attn_bwd_{bf16,f16}."""
    fn = {torch.bfloat16: attn_bwd_bf16, torch.float16: attn_bwd_f16}.get(q.dtype)
    _require(fn is not None, f"unsupported dtype {q.dtype}")
    return fn(q, k, v, o, lse, dout, causal, scale)


def _decode(fn: str, dtype, q, k, v, scale, out=None, lse=None, workspace=None):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype and t.dim() == 4
                 and t.is_contiguous() and t.device == q.device, f"{name} must be a contiguous {dtype} GPU tensor")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _require(k.shape == (B, H, Nk, d) and v.shape == k.shape, "k and v must be [B, H, Nk, d] with q's B, H, d")
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    n_ws = library().attn_decode_workspace_floats(B, H, Nq, Nk, d)
    _require(n_ws > 0, "unsupported decode sizes (1 <= Nq <= 32)")
    o = torch.empty_like(q) if out is None else out
    L = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    ws = torch.empty(n_ws, dtype=torch.float32, device=q.device) if workspace is None else workspace
    _require(o.shape == q.shape and o.dtype == dtype and o.is_contiguous() and o.device == q.device, "bad out")
    _require(L.shape == (B, H, Nq) and L.dtype == torch.float32 and L.is_contiguous() and L.device == q.device,
             "bad lse")
    _require(ws.dtype == torch.float32 and ws.is_contiguous() and ws.numel() >= n_ws and ws.device == q.device,
             f"workspace must be a contiguous fp32 tensor of at least {n_ws} elements")
    with torch.cuda.device(q.device):
        st = getattr(library(), fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), L.data_ptr(),
                                    ws.data_ptr(), B, H, Nq, Nk, d, float(scale), _stream(q))
    _check(fn, st)
    return o, L


def attn_decode_bf16(q, k, v, scale=None, out=None, lse=None, workspace=None):
    """Split-KV decoding step: bf16 q [B,H,Nq<=32,d] against k, v [B,H,Nk,d], no mask.
    Returns (O bf16 [B,H,Nq,d], LSE fp32 [B,H,Nq])."""
    return _decode("attn_decode_bf16", torch.bfloat16, q, k, v, scale, out, lse, workspace)


def attn_decode_bf16_noalloc(q, k, v, scale=None, out=None, lse=None):
    """attn_decode_bf16 with the partials in the library's static device scratch (no
    workspace; the library allocates nothing). Pass ``out`` and ``lse`` to allocate
    nothing here either. Calls that overlap in time on one GPU race."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.bfloat16 and t.dim() == 4
                 and t.is_contiguous() and t.device == q.device, f"{name} must be a contiguous bf16 GPU tensor")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _require(k.shape == (B, H, Nk, d) and v.shape == k.shape, "k and v must be [B, H, Nk, d] with q's B, H, d")
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    o = torch.empty_like(q) if out is None else out
    L = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _require(o.shape == q.shape and o.dtype == torch.bfloat16 and o.is_contiguous() and o.device == q.device,
             "bad out")
    _require(L.shape == (B, H, Nq) and L.dtype == torch.float32 and L.is_contiguous() and L.device == q.device,
             "bad lse")
    with torch.cuda.device(q.device):
        st = library().attn_decode_bf16_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), L.data_ptr(),
                                                B, H, Nq, Nk, d, float(scale), _stream(q))
    _check("attn_decode_bf16_noalloc", st)
    return o, L


def attn_decode_f16(q, k, v, scale=None, out=None, lse=None, workspace=None):
    """fp16 variant of attn_decode_bf16."""
    return _decode("attn_decode_f16", torch.float16, q, k, v, scale, out, lse, workspace)


def attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal=False, scale=None, out=None, lse=None):
    """fp8 (E4M3FN codes, uint8 tensors) attention forward with per-128-row block scales.
    Returns (O bf16 [B,H,N,d], LSE fp32 [B,H,N])."""
    _qkv_checks(q8, k8, v8, torch.uint8)
    B, H, N, d = q8.shape
    nblk = (N + 127) // 128
    for name, s in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _require(s.dtype == torch.float32 and s.shape == (B, H, nblk) and s.is_contiguous() and s.device == q8.device,
                 f"{name} must be fp32 [B, H, ceil(N/128)] on q8's device")
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device) if out is None else out
    L = torch.empty((B, H, N), dtype=torch.float32, device=q8.device) if lse is None else lse
    _require(o.shape == (B, H, N, d) and o.dtype == torch.bfloat16 and o.is_contiguous() and o.device == q8.device,
             "bad out")
    _require(L.shape == (B, H, N) and L.dtype == torch.float32 and L.is_contiguous() and L.device == q8.device,
             "bad lse")
    with torch.cuda.device(q8.device):
        st = library().attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), q_scale.data_ptr(),
                                    k_scale.data_ptr(), v_scale.data_ptr(), o.data_ptr(), L.data_ptr(), B, H, N, d,
                                    int(bool(causal)), float(scale), _stream(q8))
    _check("attn_fwd_fp8", st)
    return o, L


def attn_quant_fp8(x, signs=None, out=None, scales=None):
    """Rotate (if ``signs`` is given) and block-quantise bf16 x [B,H,N,d] to E4M3FN codes.
    Returns (codes uint8 [B,H,N,d], scales fp32 [B,H,ceil(N/128)])."""
    _require(isinstance(x, torch.Tensor) and x.is_cuda and x.dtype == torch.bfloat16 and x.dim() == 4
             and x.is_contiguous(), "x must be a contiguous bf16 [B, H, N, d] GPU tensor")
    B, H, N, d = x.shape
    nblk = (N + 127) // 128
    if signs is not None:
        _require(signs.dtype == torch.float32 and signs.shape == (d,) and signs.is_contiguous()
                 and signs.device == x.device, "signs must be fp32 [d] on x's device")
    x8 = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device) if out is None else out
    sc = torch.empty((B, H, nblk), dtype=torch.float32, device=x.device) if scales is None else scales
    _require(x8.shape == (B, H, N, d) and x8.dtype == torch.uint8 and x8.is_contiguous() and x8.device == x.device,
             "out must be a contiguous uint8 [B, H, N, d] tensor on x's device")
    _require(sc.shape == (B, H, nblk) and sc.dtype == torch.float32 and sc.is_contiguous() and sc.device == x.device,
             "scales must be a contiguous fp32 [B, H, ceil(N/128)] tensor on x's device")
    with torch.cuda.device(x.device):
        st = library().attn_quant_fp8(x.data_ptr(), x8.data_ptr(), sc.data_ptr(),
                                      None if signs is None else signs.data_ptr(), B, H, N, d, _stream(x))
    _check("attn_quant_fp8", st)
    return x8, sc


def attn_quant_fp8_kv(k, v, signs, k8=None, v8=None, k_scale=None, v_scale=None):
    """Quantise K (rotated with ``signs``) and V (unrotated) in one launch; returns
    (k8, k_scale, v8, v_scale) as two attn_quant_fp8 calls would."""
    for name, t in (("k", k), ("v", v)):
        _require(isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.bfloat16 and t.dim() == 4
                 and t.is_contiguous() and t.shape == k.shape and t.device == k.device,
                 f"{name} must be a contiguous bf16 [B, H, N, d] GPU tensor like k")
    B, H, N, d = k.shape
    nblk = (N + 127) // 128
    _require(isinstance(signs, torch.Tensor) and signs.dtype == torch.float32 and signs.shape == (d,)
             and signs.is_contiguous() and signs.device == k.device, "signs must be fp32 [d] on k's device")
    outs = []
    for name, t, shape, dt in (("k8", k8, (B, H, N, d), torch.uint8), ("v8", v8, (B, H, N, d), torch.uint8),
                               ("k_scale", k_scale, (B, H, nblk), torch.float32),
                               ("v_scale", v_scale, (B, H, nblk), torch.float32)):
        t = torch.empty(shape, dtype=dt, device=k.device) if t is None else t
        _require(t.shape == shape and t.dtype == dt and t.is_contiguous() and t.device == k.device, f"bad {name}")
        outs.append(t)
    with torch.cuda.device(k.device):
        st = library().attn_quant_fp8_kv(k.data_ptr(), v.data_ptr(), signs.data_ptr(), outs[0].data_ptr(),
                                         outs[1].data_ptr(), outs[2].data_ptr(), outs[3].data_ptr(), B, H, N, d,
                                         _stream(k))
    _check("attn_quant_fp8_kv", st)
    return outs[0], outs[2], outs[1], outs[3]


def attn_quant_fp8_qkv(q, k, v, signs, q8=None, k8=None, v8=None, q_scale=None, k_scale=None, v_scale=None):
    """Quantise Q and K (rotated with ``signs``) and V (unrotated) in one launch; returns
    (q8, q_scale, k8, k_scale, v8, v_scale) as three attn_quant_fp8 calls would."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.bfloat16 and t.dim() == 4
                 and t.is_contiguous() and t.shape == q.shape and t.device == q.device,
                 f"{name} must be a contiguous bf16 [B, H, N, d] GPU tensor like q")
    B, H, N, d = q.shape
    nblk = (N + 127) // 128
    _require(isinstance(signs, torch.Tensor) and signs.dtype == torch.float32 and signs.shape == (d,)
             and signs.is_contiguous() and signs.device == q.device, "signs must be fp32 [d] on q's device")
    outs = []
    for name, t, shape, dt in (("q8", q8, (B, H, N, d), torch.uint8), ("k8", k8, (B, H, N, d), torch.uint8),
                               ("v8", v8, (B, H, N, d), torch.uint8),
                               ("q_scale", q_scale, (B, H, nblk), torch.float32),
                               ("k_scale", k_scale, (B, H, nblk), torch.float32),
                               ("v_scale", v_scale, (B, H, nblk), torch.float32)):
        t = torch.empty(shape, dtype=dt, device=q.device) if t is None else t
        _require(t.shape == shape and t.dtype == dt and t.is_contiguous() and t.device == q.device, f"bad {name}")
        outs.append(t)
    with torch.cuda.device(q.device):
        st = library().attn_quant_fp8_qkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), signs.data_ptr(),
                                          *(t.data_ptr() for t in outs), B, H, N, d, _stream(q))
    _check("attn_quant_fp8_qkv", st)
    return outs[0], outs[3], outs[1], outs[4], outs[2], outs[5]


def attn_fwd_fp8_rotq(q, signs, k8, v8, k_scale, v_scale, causal=False, scale=None, out=None, lse=None,
                      q8_out=None, q_scale_out=None):
    """fp8 attention that rotates and quantises bf16 q itself (codes and scales optionally
    written to q8_out / q_scale_out). Returns (O bf16 [B,H,N,d], LSE fp32 [B,H,N])."""
    _require(isinstance(q, torch.Tensor) and q.is_cuda and q.dtype == torch.bfloat16 and q.dim() == 4
             and q.is_contiguous(), "q must be a contiguous bf16 [B, H, N, d] GPU tensor")
    B, H, N, d = q.shape
    nblk = (N + 127) // 128
    for name, t in (("k8", k8), ("v8", v8)):
        _require(isinstance(t, torch.Tensor) and t.dtype == torch.uint8 and t.shape == q.shape and t.is_contiguous()
                 and t.device == q.device, f"{name} must be uint8 [B, H, N, d] on q's device")
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _require(isinstance(t, torch.Tensor) and t.dtype == torch.float32 and t.shape == (B, H, nblk)
                 and t.is_contiguous() and t.device == q.device, f"{name} must be fp32 [B, H, ceil(N/128)]")
    _require(isinstance(signs, torch.Tensor) and signs.dtype == torch.float32 and signs.shape == (d,)
             and signs.is_contiguous() and signs.device == q.device, "signs must be fp32 [d] on q's device")
    if q8_out is not None:
        _require(q8_out.dtype == torch.uint8 and q8_out.shape == q.shape and q8_out.is_contiguous()
                 and q8_out.device == q.device, "bad q8_out")
    if q_scale_out is not None:
        _require(q_scale_out.dtype == torch.float32 and q_scale_out.shape == (B, H, nblk)
                 and q_scale_out.is_contiguous() and q_scale_out.device == q.device, "bad q_scale_out")
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device) if out is None else out
    L = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _require(o.shape == (B, H, N, d) and o.dtype == torch.bfloat16 and o.is_contiguous() and o.device == q.device,
             "bad out")
    _require(L.shape == (B, H, N) and L.dtype == torch.float32 and L.is_contiguous() and L.device == q.device,
             "bad lse")
    with torch.cuda.device(q.device):
        st = library().attn_fwd_fp8_rotq(q.data_ptr(), signs.data_ptr(), k8.data_ptr(), v8.data_ptr(),
                                         k_scale.data_ptr(), v_scale.data_ptr(), o.data_ptr(), L.data_ptr(),
                                         None if q8_out is None else q8_out.data_ptr(),
                                         None if q_scale_out is None else q_scale_out.data_ptr(),
                                         B, H, N, d, int(bool(causal)), float(scale), _stream(q))
    _check("attn_fwd_fp8_rotq", st)
    return o, L
