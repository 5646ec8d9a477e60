"""Exact attention (forward, backward, fp8 path) for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind a C ABI (``include/attn.h``,
built as ``libattn.so``); this package is the thin Python binding over it plus the
seeded workload generators (``inputs``). PyTorch supplies device memory and streams.
"""

from ._binding import (  # noqa: F401
    AttnError,
    LIB_PATH,
    SIGNATURES,
    attn_bwd_bf16,
    attn_calibrate,
    attn_bwd_f16,
    attn_decode_bf16,
    attn_decode_bf16_noalloc,
    attn_decode_f16,
    attn_fwd_bf16,
    attn_fwd_f16,
    attn_fwd_f32,
    attn_fwd_fp8,
    attn_fwd_fp8_rotq,
    attn_fwd_variant,
    queue_workspace,
    attn_quant_fp8,
    attn_quant_fp8_kv,
    attn_quant_fp8_qkv,
    bwd,
    fwd,
    library,
)
