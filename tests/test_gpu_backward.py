"""GPU parity of rehyat_backward (dq, dk, dv, dW_q, dW_k, db_q, db_k of the chunk-parallel
forward for an upstream gradient; ReHyAt blog, maplevalley.com.cn, 2.2.1-2.3 and 2.2.2 by
the chain rule) against the fp64 brute-force oracle, through the C ABI.

Bar: per (batch, head) slab for dq, dk, dv and per head for the parameter gradients,
max |gpu - oracle| / max |oracle| <= 1e-5 for fp32 inputs and 2e-2 for bf16 inputs (fp32
inputs: products on the fp32 matrix core; bf16 inputs: products on the bf16 matrix core with
fp32 accumulation, the softmax branch flash style with P and dS recomputed per tile and
rounded to bf16 as operands, the linear branch's float operands as hi + lo bf16 parts).
Repeated calls give identical bits.  Shapes span several
64-row tiles with ragged tails, To = 0 and To > Tc, a window with no linear region (one
chunk) and one with no softmax window (linear_only), batches and biases.
"""
import numpy as np
import pytest
import torch

import hybrid_softmax_linear_chunked_amd as rh
import oracle
from gpu_common import TOL, oracle_params, rand_inputs, slab_err, to_dev  # noqa: F401

pytestmark = pytest.mark.gpu

SHAPES = [
    # B, H, D, T, n, Tc, To, Dphi, P, linear_only, dtype, bias
    (1, 2, 32, 7, 16, 3, 1, 32, 2, 0, rh.FP32, False),
    (2, 2, 64, 6, 37, 2, 1, 64, 3, 0, rh.FP32, True),
    (1, 2, 32, 5, 40, 2, 1, 32, 2, 1, rh.FP32, False),
    (1, 2, 64, 4, 45, 4, 1, 64, 2, 0, rh.FP32, False),     # one chunk: softmax attention
    (1, 2, 128, 6, 50, 3, 1, 128, 2, 0, rh.BF16, False),
    (2, 2, 64, 8, 29, 3, 0, 64, 1, 0, rh.BF16, True),
    (1, 3, 128, 9, 45, 2, 3, 96, 4, 0, rh.BF16, False),
    (1, 2, 128, 6, 300, 3, 1, 128, 2, 0, rh.BF16, False),  # 1,800 tokens, windows of 1,200 keys
    (1, 2, 32, 1, 1, 1, 0, 32, 2, 0, rh.FP32, False),      # one token: o = v, dq = dk = 0, dv = G
    (2, 1, 64, 9, 1, 2, 1, 32, 3, 0, rh.FP32, True),       # one-token frames
    (1, 2, 64, 5, 70, 1, 0, 64, 2, 0, rh.BF16, False),     # Tc = 1, To = 0: spatial-only softmax
    (1, 2, 32, 7, 70, 3, 2, 32, 2, 0, rh.BF16, True),      # D = 32; key blocks across windows
    (1, 1, 128, 2, 33, 3, 1, 64, 2, 0, rh.BF16, False),    # T < Tc: one short chunk, ragged tiles
    (1, 2, 64, 6, 40, 3, 1, 128, 4, 0, rh.BF16, True),     # fused feature-map backward, P = 4
    (1, 2, 64, 4, 8, 2, 1, 32, 2, 0, rh.BF16, False),      # windows of 16 and 24 keys: one key half, one slot
    (1, 1, 128, 2, 32, 2, 0, 64, 2, 0, rh.BF16, True),     # one chunk of 64 queries and keys: one full slot
]


def input_grad_err(gpu, ref, x, g, key, p):
    """Per slab max |gpu - ref| / max |ref|; a slab whose exact gradient vanishes (one key in
    the window: the softmax has no score gradient) is measured against the natural scale of
    that gradient, |G| |v| |k or q| / sqrt(D) (|G| |v| for dv), since its reference is zero up
    to fp64 rounding."""
    worst = 0.0
    other = {"dq": "k", "dk": "q", "dv": None}[key]
    for b in range(p.B):
        for h in range(p.H):
            r, gg = ref[b, h].astype(np.float64), gpu[b, h].astype(np.float64)
            nat = np.abs(g[b, h]).max() * np.abs(x["v"][b, h]).max()
            if other:
                nat *= np.abs(x[other][b, h]).max() / np.sqrt(p.D)
            den = np.abs(r).max()
            if den < 1e-9 * nat:
                den = nat
            worst = max(worst, float(np.abs(gg - r).max() / den))
    return worst


@pytest.mark.parametrize("shape", SHAPES)
def test_backward_matches_oracle(shape):
    *pp, bias = shape
    p = rh.Params(*pp, out_dtype=rh.BF16)
    print(f"backward {shape}", flush=True)
    x = rand_inputs(p, seed=sum(pp[:9]) + 7, bias=bias)
    d = to_dev(x, p)
    g = np.random.default_rng(99).standard_normal((p.B, p.H, p.N, p.D)).astype(np.float32)
    dout = torch.from_numpy(g).cuda()
    got = rh.backward(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], dout, d["bq"], d["bk"])
    again = rh.backward(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], dout, d["bq"], d["bk"])
    torch.cuda.synchronize()
    for key in got:
        assert torch.equal(got[key], again[key]), key
    ref = oracle.backward(oracle_params(p), x["q"], x["k"], x["v"], x["wq"], x["wk"], g, x["bq"], x["bk"])
    tol = TOL[p.in_dtype]
    for key in ("dq", "dk", "dv"):
        e = input_grad_err(got[key].cpu().numpy(), ref[key], x, g, key, p)
        print(f"  {key}: max slab rel err {e:.2e}", flush=True)
        assert e <= tol, (key, e)
    for key in ("dwq", "dwk", "dbq", "dbk"):
        gk = got[key].cpu().numpy().astype(np.float64)
        if not ref[key].any():
            assert not gk.any(), key
            continue
        e = max(float(np.abs(gk[h] - ref[key][h]).max() / np.abs(ref[key][h]).max()) for h in range(p.H))
        print(f"  {key}: max head rel err {e:.2e}", flush=True)
        assert e <= tol, (key, e)


def test_backward_fullsize_head0():
    """Wan 5 s layer (12 heads x 32,760 tokens, bf16, B = 1) with a seeded upstream
    gradient: dq, dk, dv of slab (0, 0) and the parameter gradients of head 0 against the
    oracle's chunked form over the whole slab."""
    from synth_inputs import WORKLOADS, make_inputs
    w = WORKLOADS["wan_5s"]
    p = rh.Params(w.B, w.H, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P, 0, rh.BF16, rh.BF16)
    print("[backward wan_5s] inputs", flush=True)
    x = make_inputs(w, seed=1)
    d = {key: torch.from_numpy(val).to("cuda", torch.bfloat16).contiguous() for key, val in x.items()}
    del x
    g = np.random.default_rng(5).standard_normal((w.B, w.H, w.N, w.D), dtype=np.float32)
    got = rh.backward(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], torch.from_numpy(g).cuda(), biases=False)
    torch.cuda.synchronize()
    for key in got:
        assert torch.isfinite(got[key]).all(), key
    xs = make_inputs(w, seed=1, slabs=[(0, 0)])
    p1 = oracle.Params(1, 1, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P)
    print("[backward wan_5s] oracle (chunked form, slab 0, 0)", flush=True)
    ref = oracle.backward_chunked(p1, xs["q"], xs["k"], xs["v"], xs["wq"], xs["wk"], g[:, :1])
    tol = TOL[rh.BF16]
    for key in ("dq", "dk", "dv"):
        e = slab_err(got[key][:1, :1].cpu().numpy(), ref[key])
        print(f"  {key}: slab rel err {e:.2e}", flush=True)
        assert e <= tol, (key, e)
    for key in ("dwq", "dwk"):
        gk = got[key][0].cpu().numpy().astype(np.float64)
        e = float(np.abs(gk - ref[key][0]).max() / np.abs(ref[key][0]).max())
        print(f"  {key}: head 0 rel err {e:.2e}", flush=True)
        assert e <= tol, (key, e)
