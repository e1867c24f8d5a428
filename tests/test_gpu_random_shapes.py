"""Seeded random-shape sweep on the GPU, through the C ABI, against the fp64 oracle (ReHyAt
blog, maplevalley.com.cn, 2.2.1-2.3 and 2.2.2): batches, heads, head dims 32/64/128, frame
counts 1-9 of 1-70 tokens (ragged 64-token tiles), chunk sizes 1-5 with overlaps 0-3, feature
sizes 32-128 with 1-4 powers (uneven parts), fp32 and bf16 inputs, biases, and the empty
softmax window.  Per shape: the chunk-parallel forward at the output bar, the streamed form
against the parallel form (bit for bit), and the backward for a seeded upstream gradient at the same bars
(vanishing score gradients against their natural scale, as in test_gpu_backward), and the
distillation loss and feature-map gradients (blog 3.1.1) on the same shapes."""
import numpy as np
import pytest
import torch

import hybrid_softmax_linear_chunked_amd as rh
import oracle
from gpu_common import TOL, oracle_params, rand_inputs, slab_err, to_dev
from test_gpu_backward import input_grad_err

pytestmark = pytest.mark.gpu


def random_shapes(count, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        D = int(rng.choice([32, 64, 128]))
        shape = (int(rng.integers(1, 3)), int(rng.integers(1, 4)), D, int(rng.integers(1, 10)),
                 int(rng.integers(1, 71)), int(rng.integers(1, 6)), int(rng.integers(0, 4)),
                 int(rng.choice([32, 64, 96, 128])), int(rng.integers(1, 5)),
                 int(rng.random() < 0.2), int(rng.choice([rh.FP32, rh.BF16])), bool(rng.random() < 0.3))
        out.append(shape)
    return out


SHAPES = random_shapes(16)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"s{i}" for i in range(len(SHAPES))])
def test_random_shape(shape):
    *pp, bias = shape
    p = rh.Params(*pp, out_dtype=rh.FP32)
    print(f"random shape {shape}", flush=True)
    x = rand_inputs(p, seed=sum(pp[:9]) * 7 + 1, bias=bias)
    d = to_dev(x, p)
    po = oracle_params(p)
    tol = TOL[p.in_dtype]

    out = rh.forward_parallel(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], d["bq"], d["bk"])
    st = rh.Stream(p, d["wq"], d["wk"], d["bq"], d["bk"])
    outs = []
    for f0 in range(0, p.T, p.Tc):
        f1 = min(f0 + p.Tc, p.T)
        sl = slice(f0 * p.n, f1 * p.n)
        outs.append(st.step(d["q"][:, :, sl].contiguous(), d["k"][:, :, sl].contiguous(),
                            d["v"][:, :, sl].contiguous(), f1 - f0))
    torch.cuda.synchronize()
    ref = oracle.parallel(po, x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"])
    e = slab_err(out.cpu().numpy(), ref)
    print(f"  forward: {e:.2e}", flush=True)
    assert e <= tol
    s_out = torch.cat(outs, dim=2)
    assert torch.equal(s_out, out)

    g = np.random.default_rng(11).standard_normal((p.B, p.H, p.N, p.D)).astype(np.float32)
    got = rh.backward(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], torch.from_numpy(g).cuda(), d["bq"], d["bk"])
    torch.cuda.synchronize()
    bref = oracle.backward(po, x["q"], x["k"], x["v"], x["wq"], x["wk"], g, x["bq"], x["bk"])
    for key in ("dq", "dk", "dv"):
        e = input_grad_err(got[key].cpu().numpy(), bref[key], x, g, key, p)
        print(f"  {key}: {e:.2e}", flush=True)
        assert e <= tol, (key, e)
    for key in ("dwq", "dwk", "dbq", "dbk"):
        gk = got[key].cpu().numpy().astype(np.float64)
        if not bref[key].any():
            assert not gk.any(), key
            continue
        e = max(float(np.abs(gk[h] - bref[key][h]).max() / np.abs(bref[key][h]).max()) for h in range(p.H))
        print(f"  {key}: {e:.2e}", flush=True)
        assert e <= tol, (key, e)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"s{i}" for i in range(len(SHAPES))])
def test_random_shape_distill(shape):
    """The distillation objective and its feature-map gradients on the same random shapes
    (blog 3.1.1), against the oracle's loss and its brute-force gradients."""
    from test_gpu_distill import check_loss
    from test_gpu_distill_grad import GRAD_TOL, compare
    *pp, bias = shape
    p = rh.Params(*pp, out_dtype=rh.BF16)
    print(f"random shape distill {shape}", flush=True)
    x = rand_inputs(p, seed=sum(pp[:9]) * 7 + 2, bias=bias)
    d = to_dev(x, p)
    po = oracle_params(p)
    loss, stu, tea = rh.distill_loss(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], d["bq"], d["bk"], outputs=True)
    got = rh.distill_grad(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], d["bq"], d["bk"])
    torch.cuda.synchronize()
    assert torch.equal(got["loss"], loss)
    hyb = oracle.parallel(po, x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"])
    soft = oracle.full_softmax(po, x["q"], x["k"], x["v"])
    BH = p.B * p.H
    check_loss(loss.cpu().numpy().reshape(BH).astype(np.float64),
               stu.cpu().numpy().reshape(BH, -1).astype(np.float64),
               tea.cpu().numpy().reshape(BH, -1).astype(np.float64),
               hyb.reshape(BH, -1), soft.reshape(BH, -1), TOL[p.in_dtype])
    ref = oracle.distill_phi_grads(po, x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"])
    if not any(ref[key].any() for key in ("dwq", "dwk", "dbq", "dbk")):
        for key in ("dwq", "dwk", "dbq", "dbk"):
            assert not got[key].any(), key
        return
    compare(got, ref, range(p.H), GRAD_TOL[p.in_dtype], str(shape[:10]))
