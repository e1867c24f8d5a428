"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to the storage dtype; it holds
none of the attention arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it without sharing any of the method's code.

Workloads are shaped like the video-DiT layers the ReHyAt pages evaluate on: a
Wan2.1-1.3B attention layer at 480x832 (latent grid 30x52 = 1560 tokens per latent
frame, 12 heads of dim 128), 5 s / 10 s / 20 s clips (21 / 41 / 81 latent frames), and a
14B-shaped layer at 720x1280 (45x80 = 3600 tokens per frame, 40 heads).  The pages use
chunks of Tc = 3 frames with To = 1 overlap frame and a degree-2 polynomial feature map.

Recipe: numpy PCG64 with one independent stream per tensor slab, so that any (batch,
head) slab can be regenerated on its own: Q, K, V[b, h] ~ N(0, 1) of shape [N, D] from
``default_rng([seed, t, b, h])`` with t = 0, 1, 2; W_q[h], W_k[h] ~ N(0, 1/D) of shape
[Dphi, D] from ``default_rng([seed, t, h])`` with t = 3, 4; all drawn as float32.  For bf16
workloads every value is rounded to the nearest bfloat16 (ties to even) and kept as
float32 holding that exact value.  No bias (the API accepts one).  The seed of a workload
is its index in the list of measured workloads (tiny 0, 5 s 1, 10 s 2, 20 s 3, 14B 4).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
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
    """Round finite float32 values to the nearest bfloat16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _slab(seed: int, t: int, idx, shape, scale, bf16: bool) -> np.ndarray:
    a = np.random.default_rng([seed, t, *idx]).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return round_bf16(a) if bf16 else a


def make_inputs(w: Workload, seed: int, slabs=None):
    """Returns dict q, k, v [B,H,N,D] and wq, wk [H,Dphi,D] as float32 arrays.

    With ``slabs`` = list of (b, h), q/k/v hold only those slabs, stacked as
    [len(slabs), 1, N, D], and wq/wk the matching heads as [len(slabs), Dphi, D]."""
    bf = w.dtype == "bf16"
    sd = 1.0 / np.sqrt(w.D)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)] if slabs is None else list(slabs)
    out = {}
    for t, key in enumerate(("q", "k", "v")):
        if slabs is None:
            a = np.empty((w.B, w.H, w.N, w.D), dtype=np.float32)

            def fill(bh, t=t, a=a):
                a[bh[0], bh[1]] = _slab(seed, t, bh, (w.N, w.D), 1.0, bf)
            # slabs are independent streams, so filling them on several threads (numpy
            # drops the interpreter lock while it draws) gives the same values
            with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
                list(ex.map(fill, pairs))
        else:
            a = np.stack([_slab(seed, t, (b, h), (w.N, w.D), 1.0, bf)[None] for b, h in pairs])
        out[key] = a
    heads = range(w.H) if slabs is None else [h for _, h in pairs]
    for t, key in ((3, "wq"), (4, "wk")):
        out[key] = np.stack([_slab(seed, t, (h,), (w.Dphi, w.D), sd, bf) for h in heads])
    return out
