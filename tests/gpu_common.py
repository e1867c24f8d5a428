"""Helpers shared by the GPU parity tests: device copies of the seeded inputs and the
tolerance rule.

Tolerance (the bar stated for this path): per (batch, head) slab,
max_i |gpu_i - ref_i| / max_i |ref_i| <= 1e-5 for fp32 inputs and <= 2e-2 for bf16 inputs
with fp32 accumulation.  A purely elementwise relative error is ill-posed where outputs
cross zero, so the slab maximum is the scale.
"""
import numpy as np
import torch

import hybrid_softmax_linear_chunked_amd as rh
import oracle

TOL = {rh.FP32: 1e-5, rh.BF16: 2e-2}


def oracle_params(p: rh.Params) -> oracle.Params:
    return oracle.Params(p.B, p.H, p.D, p.T, p.n, p.Tc, p.To, p.Dphi, p.P, p.linear_only)


def rand_inputs(p: rh.Params, seed: int, bias: bool = False):
    """Seeded N(0,1) activations and N(0,1/D) weights, rounded to the input dtype."""
    from synth_inputs import round_bf16
    rng = np.random.default_rng(seed)
    shape = (p.B, p.H, p.N, p.D)
    x = dict(q=rng.standard_normal(shape, dtype=np.float32),
             k=rng.standard_normal(shape, dtype=np.float32),
             v=rng.standard_normal(shape, dtype=np.float32),
             wq=rng.standard_normal((p.H, p.Dphi, p.D), dtype=np.float32) / np.float32(np.sqrt(p.D)),
             wk=rng.standard_normal((p.H, p.Dphi, p.D), dtype=np.float32) / np.float32(np.sqrt(p.D)))
    if p.in_dtype == rh.BF16:
        x = {key: round_bf16(val) for key, val in x.items()}
    if bias:
        x["bq"] = (rng.standard_normal((p.H, p.Dphi)) * 0.5).astype(np.float32)
        x["bk"] = (rng.standard_normal((p.H, p.Dphi)) * 0.5).astype(np.float32)
    else:
        x["bq"] = x["bk"] = None
    return x


def to_dev(x: dict, p: rh.Params) -> dict:
    dt = rh.torch_dtype(p.in_dtype)
    out = {}
    for key, val in x.items():
        if val is None:
            out[key] = None
        elif key in ("bq", "bk"):
            out[key] = torch.from_numpy(val).to("cuda", torch.float32).contiguous()
        else:
            out[key] = torch.from_numpy(val).to("cuda", dt).contiguous()
    return out


def slab_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over (b,h) slabs of max|g - r| / max|r| (arrays [B,H,...])."""
    g = gpu.reshape(gpu.shape[0] * gpu.shape[1], -1).astype(np.float64)
    r = ref.reshape(ref.shape[0] * ref.shape[1], -1).astype(np.float64)
    num = np.abs(g - r).max(axis=1)
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((num / den).max())


def run_parallel(p: rh.Params, d: dict, aux=True):
    return rh.forward_parallel(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], d["bq"], d["bk"], aux=aux)
