"""GPU parity of rehyat_distill_grad (gradients of the distillation objective with respect
to W_q, W_k, b_q, b_k; ReHyAt blog, maplevalley.com.cn, 3.1.1) against the fp64 oracle,
through the C ABI.

Bar: per head, max |gpu - oracle| / max |oracle| over the [Dphi, D] matrix (and the
[Dphi] bias vector) <= the path's floating-point bar, 1e-5 for fp32 inputs and 2e-2 for
bf16 inputs with fp32 accumulation (fp32 inputs: gradient products on the fp32 matrix core;
bf16 inputs: on the bf16 matrix core with every float operand as hi + lo bf16 parts, about
2^-15 relative error per product, so the bf16 error still comes mostly from the student's
output, whose P and phi operands are bf16).  The shapes cover both the fused feature-map
backward (P = 1, 2, 4 with Dphi a multiple of 64) and its separate pass.  The loss
equals rehyat_distill_loss bit for bit, repeated calls give identical bits, and without a
linear region every gradient is exactly zero.
"""
import numpy as np
import pytest
import torch

import hybrid_softmax_linear_chunked_amd as rh
import oracle
from gpu_common import oracle_params, rand_inputs, to_dev
from synth_inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

GRAD_TOL = {rh.FP32: 1e-5, rh.BF16: 2e-2}

SHAPES = [
    # B, H, D, T, n, Tc, To, Dphi, P, linear_only, dtype, bias
    (1, 2, 32, 7, 16, 3, 1, 32, 2, 0, rh.FP32, False),
    (2, 2, 64, 6, 37, 2, 1, 64, 3, 0, rh.FP32, True),
    (1, 2, 32, 5, 40, 2, 1, 32, 2, 1, rh.FP32, False),
    (1, 2, 128, 6, 50, 3, 1, 128, 2, 0, rh.BF16, False),
    (2, 2, 64, 8, 29, 3, 0, 64, 1, 0, rh.BF16, True),
    (1, 3, 128, 9, 45, 2, 3, 96, 4, 0, rh.BF16, False),
    (1, 2, 64, 6, 40, 3, 1, 128, 4, 0, rh.BF16, True),    # fused feature-map backward, P = 4
    (1, 1, 64, 7, 30, 3, 2, 128, 3, 0, rh.BF16, False),   # P = 3 (parts 43/43/42): separate pass
]


def rel(g, r):
    return float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-30))


def compare(got, ref, heads, tol, label):
    for key in ("dwq", "dwk", "dbq", "dbk"):
        if key not in got or ref.get(key) is None:
            continue
        g = got[key].cpu().numpy().astype(np.float64)
        for h in heads:
            e = rel(g[h], ref[key][h])
            print(f"{label} {key} head {h}: rel err {e:.2e}", flush=True)
            assert e <= tol, (label, key, h, e)


@pytest.mark.parametrize("shape", SHAPES)
def test_distill_grad_matches_oracle(shape):
    *pp, bias = shape
    p = rh.Params(*pp, out_dtype=rh.BF16)
    print(f"distill_grad {shape}", flush=True)
    x = rand_inputs(p, seed=sum(pp[:9]) + 1, bias=bias)
    d = to_dev(x, p)
    got = rh.distill_grad(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], d["bq"], d["bk"])
    again = rh.distill_grad(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], d["bq"], d["bk"])
    loss = rh.distill_loss(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], d["bq"], d["bk"])
    torch.cuda.synchronize()
    for key in got:
        assert torch.equal(got[key], again[key]), key
    assert torch.equal(got["loss"], loss)
    ref = oracle.distill_phi_grads(oracle_params(p), x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"])
    compare(got, ref, range(p.H), GRAD_TOL[p.in_dtype], str(shape[:10]))


def test_distill_grad_zero_without_linear_region():
    p = rh.Params(1, 2, 64, 4, 33, 4, 1, 64, 2, 0, rh.BF16, rh.BF16)
    x = rand_inputs(p, seed=3, bias=True)
    d = to_dev(x, p)
    got = rh.distill_grad(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], d["bq"], d["bk"])
    torch.cuda.synchronize()
    for key in ("dwq", "dwk", "dbq", "dbk"):
        assert not got[key].any(), key
    assert (got["loss"] == 0).all()


def test_distill_grad_fullsize_head0():
    """Wan 5 s layer (12 heads x 32,760 tokens, bf16, B = 1): the gradients of head 0 against
    the oracle's chunked-state form over the whole slab."""
    w = WORKLOADS["wan_5s"]
    p = rh.Params(w.B, w.H, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P, 0, rh.BF16, rh.BF16)
    print("[distill_grad wan_5s] inputs", flush=True)
    x = make_inputs(w, seed=1)
    d = {key: torch.from_numpy(val).to("cuda", torch.bfloat16).contiguous() for key, val in x.items()}
    del x
    got = rh.distill_grad(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], biases=False)
    torch.cuda.synchronize()
    for key in got:
        assert torch.isfinite(got[key]).all(), key
    xs = make_inputs(w, seed=1, slabs=[(0, 0)])
    p1 = oracle.Params(1, 1, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P)
    print("[distill_grad wan_5s] oracle (chunked form, head 0)", flush=True)
    ref = oracle.distill_phi_grads_chunked(p1, xs["q"], xs["k"], xs["v"], xs["wq"], xs["wk"])
    got0 = {key: got[key][:1] for key in ("dwq", "dwk")}
    compare(got0, ref, [0], GRAD_TOL[rh.BF16], "wan_5s")
    assert abs(float(got["loss"][0, 0]) - ref["loss"][0, 0]) <= 1e-3 * ref["loss"][0, 0]
