"""Seeded synthetic workloads for the attention forward pass.

This module only draws inputs; it holds none of the attention or quantisation
arithmetic, and both the device library's tests/bench and the CPU oracle consume what
it returns. Every draw comes from numpy's PCG64 generator seeded by
``SeedSequence([78, workload_id, tensor_id])`` with tensor ids 0, 1, 2 for Q, K, V,
3 for the Hadamard sign vector, 4 for the outlier channels and 6 for the output
gradient dO of the backward pass.

The named workloads mirror the shapes the pages benchmark (heads = 16, head dims 64
and 128, sequence lengths 1k-16k, causal and non-causal; "Triton 07: Flash Attention
v3", benchmark section, and the FlashAttention-2 digest's results table). There is no
dataset behind those figures: the pages measure on random tensors of these shapes.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

SEED_ROOT = 78
Q_ID, K_ID, V_ID, SIGN_ID, OUTLIER_ID, DO_ID = 0, 1, 2, 3, 4, 6


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int           # workload id used in the seed
    B: int
    H: int
    N: int
    d: int
    dtype: str         # "f32", "bf16", "f16" or "fp8"
    causal: tuple      # the causal flags this workload is run with

    @property
    def scale(self) -> float:
        return softmax_scale(self.d)


WORKLOADS = {
    "C1": Workload("C1", 1, 1, 2, 128, 64, "f32", (False, True)),
    "C2": Workload("C2", 2, 4, 16, 1024, 64, "bf16", (True,)),
    "C3": Workload("C3", 3, 2, 16, 4096, 128, "bf16", (True, False)),
    "C4": Workload("C4", 4, 1, 16, 16384, 128, "bf16", (True,)),
    "C5": Workload("C5", 5, 2, 16, 8192, 128, "fp8", (True,)),
    # the headline shape: bf16, causal, d=128, N=8192 with B=2, H=16
    "H": Workload("H", 6, 2, 16, 8192, 128, "bf16", (True,)),
}


def softmax_scale(d: int) -> float:
    """The fp32 value nearest to 1/sqrt(d), returned as a Python float (exactly)."""
    return float(np.float32(1.0 / math.sqrt(d)))


def generator(wid: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, wid, tensor_id])))


def normal_f32(wid: int, tensor_id: int, shape) -> np.ndarray:
    """Standard-normal fp32 draws of the given shape."""
    return generator(wid, tensor_id).standard_normal(size=shape, dtype=np.float32)


def draw_qkv(wid: int, B: int, H: int, N: int, d: int):
    """Q, K, V ~ N(0, 1) as fp32 arrays [B, H, N, d]."""
    shape = (B, H, N, d)
    return normal_f32(wid, Q_ID, shape), normal_f32(wid, K_ID, shape), normal_f32(wid, V_ID, shape)


def draw_dout(wid: int, B: int, H: int, N: int, d: int):
    """The output gradient dO ~ N(0, 1) as an fp32 array [B, H, N, d]."""
    return normal_f32(wid, DO_ID, (B, H, N, d))


def outlier_channels(wid: int, d: int, frac: float = 0.01) -> np.ndarray:
    """ceil(frac * d) distinct channel indices, sorted."""
    n = max(1, math.ceil(frac * d))
    return np.sort(generator(wid, OUTLIER_ID).choice(d, size=n, replace=False))


def draw_fp8_workload(wid: int, B: int, H: int, N: int, d: int, frac: float = 0.01,
                      mult: float = 20.0, shared_channels: bool = True, v_outliers: bool = False):
    """Inputs of the fp8 workload: Q, K, V ~ N(0, 1) in fp32 with the channels returned by
    ``outlier_channels`` multiplied by ``mult`` in Q and K (one shared channel set), and
    V left plain unless ``v_outliers``. With ``shared_channels=False`` K gets its own
    channel set (drawn with tensor id 5). Also returns the +-1 sign vector of length d.
    """
    q, k, v = draw_qkv(wid, B, H, N, d)
    ch = outlier_channels(wid, d, frac)
    q[..., ch] *= np.float32(mult)
    if shared_channels:
        k[..., ch] *= np.float32(mult)
    else:
        n = ch.size
        ch_k = np.sort(generator(wid, 5).choice(d, size=n, replace=False))
        k[..., ch_k] *= np.float32(mult)
    if v_outliers:
        v[..., ch] *= np.float32(mult)
    signs = np.where(generator(wid, SIGN_ID).integers(0, 2, size=d) == 1, 1.0, -1.0).astype(np.float32)
    return q, k, v, signs


def draw_fp8_entry_outliers(wid: int, B: int, H: int, N: int, d: int, frac: float = 0.01, mult: float = 20.0):
    """Like ``draw_fp8_workload`` but the outliers are scattered entries instead of whole
    channels: a seeded ``frac`` of the entries of Q and of K (independent positions,
    tensor ids 8 and 9) is multiplied by ``mult``; V is plain."""
    q, k, v = draw_qkv(wid, B, H, N, d)
    for x, tid in ((q, 8), (k, 9)):
        mask = generator(wid, tid).random(size=x.shape) < frac
        x[mask] *= np.float32(mult)
    signs = np.where(generator(wid, SIGN_ID).integers(0, 2, size=d) == 1, 1.0, -1.0).astype(np.float32)
    return q, k, v, signs


def normal_on_device(wid: int, tensor_id: int, shape, dtype, device="cuda"):
    """Seeded N(0,1) tensor drawn directly on the device in the given torch dtype (torch's
    Philox generator, seeded from SeedSequence([78, workload_id, tensor_id])), for
    workloads too large to draw on the host. The oracle reads back the values drawn."""
    import torch

    seed = int(np.random.SeedSequence([SEED_ROOT, wid, tensor_id]).generate_state(1, dtype=np.uint64)[0] >> 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=dtype, device=device)


def to_torch(x: np.ndarray, dtype: str):
    """Round an fp32 array to the named dtype on the CPU (round-to-nearest-even) as a
    contiguous CPU torch tensor. fp8 workloads carry bf16 activations."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x))
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "fp8": torch.bfloat16}[dtype]
    return t.to(tdt).contiguous()
