"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to the storage dtype; it holds
none of the attention arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it without sharing any of the method's code.

Workloads are shaped like the video-DiT layers the ReHyAt pages evaluate on: a
Wan2.1-1.3B attention layer at 480x832 (latent grid 30x52 = 1560 tokens per latent
frame, 12 heads of dim 128), 5 s / 10 s / 20 s clips (21 / 41 / 81 latent frames), and a
14B-shaped layer at 720x1280 (45x80 = 3600 tokens per frame, 40 heads).  The pages use
chunks of Tc = 3 frames with To = 1 overlap frame and a degree-2 polynomial feature map.

Recipe: numpy PCG64 ``default_rng(seed)``; Q, K, V ~ N(0, 1) with shape [B, H, N, D],
then W_q, W_k ~ N(0, 1/D) with shape [H, Dphi, D], drawn in that order as float32;
for bf16 workloads every value is rounded to the nearest bfloat16 (ties to even) and
kept as float32 holding that exact value.  No bias (the API accepts one).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    T: int
    n: int
    Tc: int
    To: int
    Dphi: int
    P: int
    dtype: str          # "fp32" or "bf16": storage/compute input type
    linear_only: int = 0

    @property
    def N(self) -> int:
        return self.T * self.n

    @property
    def F(self) -> int:
        return self.P * self.Dphi


WORKLOADS = {
    # tiny parity case: 7 frames of 4x4 tokens
    "tiny_fp32": Workload("tiny_fp32", B=1, H=2, D=32, T=7, n=16, Tc=3, To=1, Dphi=32, P=2,
                          dtype="fp32"),
    # Wan2.1-1.3B layer, 5 s of 480x832: 21 latent frames of 30x52 tokens
    "wan_5s": Workload("wan_5s", B=1, H=12, D=128, T=21, n=1560, Tc=3, To=1, Dphi=128, P=2,
                       dtype="bf16"),
    # 10 s clip, processed chunk by chunk through the streaming entry points
    "wan_10s_stream": Workload("wan_10s_stream", B=1, H=12, D=128, T=41, n=1560, Tc=3, To=1,
                               Dphi=128, P=2, dtype="bf16"),
    # 20 s clip, batch of two, chunk-parallel form
    "wan_20s": Workload("wan_20s", B=2, H=12, D=128, T=81, n=1560, Tc=3, To=1, Dphi=128, P=2,
                        dtype="bf16"),
    # 14B-shaped layer at 720x1280: 45x80 tokens per frame, 40 heads, phi with 3 parts
    "wan14b_720p": Workload("wan14b_720p", B=1, H=40, D=128, T=21, n=3600, Tc=3, To=1,
                            Dphi=128, P=3, dtype="bf16"),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def make_inputs(w: Workload, seed: int):
    """Returns dict q, k, v [B,H,N,D] and wq, wk [H,Dphi,D] as float32 arrays."""
    rng = np.random.default_rng(seed)
    shape = (w.B, w.H, w.N, w.D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    wshape = (w.H, w.Dphi, w.D)
    sd = np.float32(1.0 / np.sqrt(w.D))
    wq = rng.standard_normal(wshape, dtype=np.float32) * sd
    wk = rng.standard_normal(wshape, dtype=np.float32) * sd
    out = dict(q=q, k=k, v=v, wq=wq, wk=wk)
    if w.dtype == "bf16":
        out = {key: round_bf16(val) for key, val in out.items()}
    return out
