"""Pins of the oracle's backward of the hybrid attention (dq, dk, dv and the feature-map
parameter gradients for an upstream gradient G; ReHyAt blog, maplevalley.com.cn, 2.2.1-2.3
and 2.2.2, chain rule).  Pinned to central finite differences of <G, o> computed with the
C chunk-parallel oracle (a different code path), along random directions in every input;
to the distillation gradients when G = 2 (o - t); and to the two reductions the pages fix:
with one chunk over the clip the inputs' gradients are those of softmax attention (torch
autograd in fp64), and without a linear region the feature-map gradients vanish.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def rand(p, seed, bias):
    rng = np.random.default_rng(seed)
    sh = (p.B, p.H, p.N, p.D)
    x = dict(q=rng.standard_normal(sh), k=rng.standard_normal(sh), v=rng.standard_normal(sh),
             wq=rng.standard_normal((p.H, p.Dphi, p.D)) / math.sqrt(p.D),
             wk=rng.standard_normal((p.H, p.Dphi, p.D)) / math.sqrt(p.D), g=rng.standard_normal(sh))
    x["bq"] = rng.standard_normal((p.H, p.Dphi)) * 0.5 if bias else None
    x["bk"] = rng.standard_normal((p.H, p.Dphi)) * 0.5 if bias else None
    return x


def bwd(p, x):
    return oracle.backward(p, x["q"], x["k"], x["v"], x["wq"], x["wk"], x["g"], x["bq"], x["bk"])


def objective(p, x):
    o = oracle.parallel(p, x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"])
    return float((o * x["g"]).sum())


@pytest.mark.parametrize("shape,bias", [
    ((1, 2, 8, 5, 4, 2, 1, 8, 2, 0), True),
    ((2, 1, 6, 6, 3, 3, 0, 6, 3, 0), False),
    ((1, 1, 4, 5, 3, 2, 1, 4, 2, 1), True),
    ((1, 1, 8, 7, 3, 2, 3, 8, 1, 0), False),
])
def test_backward_matches_finite_differences(shape, bias):
    p = oracle.Params(*shape)
    x = rand(p, 21, bias)
    gr = bwd(p, x)
    rng = np.random.default_rng(8)
    names = ["q", "k", "v", "wq", "wk"] + (["bq", "bk"] if bias else [])
    scale = sum(float(np.abs(gr["d" + n]).sum()) for n in names)
    for name in names:
        E = rng.standard_normal(x[name].shape)
        eps = 1e-5
        fd = (objective(p, dict(x, **{name: x[name] + eps * E}))
              - objective(p, dict(x, **{name: x[name] - eps * E}))) / (2 * eps)
        an = float((gr["d" + name] * E).sum())
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3 * scale), (name, fd, an)


def test_backward_with_distillation_gradient_equals_distill_grads():
    p = oracle.Params(1, 2, 8, 7, 4, 3, 1, 8, 2)
    x = rand(p, 4, bias=True)
    o = oracle.parallel(p, x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"])
    t = oracle.full_softmax(p, x["q"], x["k"], x["v"])
    gr = bwd(p, dict(x, g=2 * (o - t)))
    dg = oracle.distill_phi_grads(p, x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"])
    for key in ("dwq", "dwk", "dbq", "dbk"):
        assert np.abs(gr[key] - dg[key]).max() <= 1e-12 * np.abs(dg[key]).max()


def test_one_chunk_is_softmax_attention_backward():
    p = oracle.Params(1, 2, 8, 4, 5, 4, 1, 8, 2)
    x = rand(p, 6, bias=False)
    gr = bwd(p, x)
    tq, tk, tv = (torch.tensor(x[n], requires_grad=True) for n in ("q", "k", "v"))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    (o * torch.from_numpy(x["g"])).sum().backward()
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        ref = t.grad.numpy()
        assert np.abs(gr[name] - ref).max() <= 1e-12 * np.abs(ref).max(), name
    for key in ("dwq", "dwk", "dbq", "dbk"):
        assert not gr[key].any()


@pytest.mark.parametrize("shape,bias", [
    ((1, 2, 8, 7, 4, 3, 1, 8, 2, 0), True),
    ((2, 1, 6, 6, 5, 2, 0, 9, 3, 0), False),
    ((1, 1, 8, 8, 3, 2, 3, 8, 2, 0), True),      # To > Tc
    ((1, 2, 4, 5, 4, 2, 1, 8, 4, 1), False),     # empty softmax window
    ((1, 1, 8, 9, 2, 1, 0, 8, 1, 0), True),      # Tc = 1, To = 0, P = 1
    ((1, 1, 8, 4, 5, 4, 1, 8, 2, 0), False),     # one chunk
])
def test_chunked_backward_equals_brute_force(shape, bias):
    p = oracle.Params(*shape)
    x = rand(p, 12, bias)
    a = bwd(p, x)
    b = oracle.backward_chunked(p, x["q"], x["k"], x["v"], x["wq"], x["wk"], x["g"], x["bq"], x["bk"])
    for key in a:
        scale = max(np.abs(a[key]).max(), 1e-300)
        assert np.abs(a[key] - b[key]).max() <= 1e-10 * scale, key
