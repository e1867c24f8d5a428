"""Pins of the oracle's distillation gradients with respect to the feature-map parameters
W_q, W_k, b_q, b_k (ReHyAt blog, maplevalley.com.cn, 3.1.1: only phi_q and phi_k are
trained).  The brute-force form is pinned to central finite differences of the oracle's
distillation loss (a different code path: the C chunk-parallel forward and the numpy
teacher); the chunked-state form must equal the brute force; the feature layout the
backward uses must reproduce the C oracle's phi; and without a linear region (one chunk
over the clip, or an overlap reaching the first frame) every gradient is zero.
"""
import math

import numpy as np
import pytest

import oracle


def rand(p, seed, bias):
    rng = np.random.default_rng(seed)
    sh = (p.B, p.H, p.N, p.D)
    x = dict(q=rng.standard_normal(sh), k=rng.standard_normal(sh), v=rng.standard_normal(sh),
             wq=rng.standard_normal((p.H, p.Dphi, p.D)) / math.sqrt(p.D),
             wk=rng.standard_normal((p.H, p.Dphi, p.D)) / math.sqrt(p.D))
    x["bq"] = rng.standard_normal((p.H, p.Dphi)) * 0.5 if bias else None
    x["bk"] = rng.standard_normal((p.H, p.Dphi)) * 0.5 if bias else None
    return x


def args(x):
    return x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"]


@pytest.mark.parametrize("Dphi,P", [(8, 1), (8, 2), (10, 3), (12, 4)])
def test_feature_map_reproduces_phi(Dphi, P):
    p = oracle.Params(1, 2, 4, 2, 3, 1, 0, Dphi, P)
    x = rand(p, 3, bias=True)
    elem, power = oracle.feature_map(p)
    for h in range(p.H):
        pre = x["q"][0, h] @ x["wq"][h].T + x["bq"][h]
        u = np.logaddexp(0.0, pre)
        p1 = oracle.Params(1, 1, p.D, p.T, p.n, p.Tc, p.To, p.Dphi, p.P)
        ref = oracle.phi(p1, x["q"][:, h:h + 1], x["wq"][h:h + 1], x["bq"][h:h + 1])[0, 0]
        assert np.allclose(u[:, elem] ** power, ref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("shape,bias", [
    ((1, 2, 8, 5, 4, 2, 1, 8, 2, 0), True),
    ((2, 1, 6, 6, 3, 3, 0, 6, 3, 0), False),
    ((1, 1, 4, 5, 3, 2, 1, 4, 2, 1), True),
])
def test_brute_gradients_match_finite_differences(shape, bias):
    p = oracle.Params(*shape)
    x = rand(p, 11, bias)
    gr = oracle.distill_phi_grads(p, *args(x))
    base = oracle.distill_loss(p, *args(x))
    assert np.allclose(gr["loss"], base, rtol=1e-12)
    rng = np.random.default_rng(5)
    names = ["wq", "wk"] + (["bq", "bk"] if bias else [])
    for name in names:
        E = rng.standard_normal(x[name].shape)
        eps = 1e-5
        lp = oracle.distill_loss(p, *args(dict(x, **{name: x[name] + eps * E}))).sum()
        lm = oracle.distill_loss(p, *args(dict(x, **{name: x[name] - eps * E}))).sum()
        fd = (lp - lm) / (2 * eps)
        an = float((gr["d" + name] * E).sum())
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3 * base.sum()), (name, fd, an)


@pytest.mark.parametrize("shape,bias", [
    ((1, 2, 8, 7, 4, 3, 1, 8, 2, 0), True),
    ((2, 2, 6, 6, 5, 2, 0, 9, 3, 0), False),
    ((1, 1, 8, 8, 3, 2, 3, 8, 2, 0), True),      # To > Tc
    ((1, 2, 4, 5, 4, 2, 1, 8, 4, 1), False),     # empty softmax window
    ((1, 1, 8, 9, 2, 1, 0, 8, 1, 0), True),      # Tc = 1, To = 0, P = 1
])
def test_chunked_form_equals_brute_force(shape, bias):
    p = oracle.Params(*shape)
    x = rand(p, 7, bias)
    a = oracle.distill_phi_grads(p, *args(x))
    b = oracle.distill_phi_grads_chunked(p, *args(x))
    for key in ("loss", "dwq", "dwk", "dbq", "dbk"):
        scale = max(np.abs(a[key]).max(), 1e-300)
        assert np.abs(a[key] - b[key]).max() <= 1e-10 * scale, key


@pytest.mark.parametrize("Tc,To", [(6, 1), (9, 0), (2, 6)])
def test_no_linear_region_no_gradient(Tc, To):
    p = oracle.Params(1, 2, 4, 6, 3, Tc, To, 8, 2)
    x = rand(p, 2, bias=True)
    for fn in (oracle.distill_phi_grads, oracle.distill_phi_grads_chunked):
        g = fn(p, *args(x))
        for key in ("dwq", "dwk", "dbq", "dbk"):
            assert not g[key].any(), (fn.__name__, key)
