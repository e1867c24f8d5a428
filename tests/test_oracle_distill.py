"""Pins of the distillation objective in the oracle (ReHyAt blog, maplevalley.com.cn,
3.1.1: the hybrid block is trained towards the frozen softmax teacher's output on the
same inputs, in L2).  Reading: per (batch, head) slab, the sum over tokens and channels of
(hybrid - full softmax)^2.

The teacher is pinned to torch's scaled_dot_product_attention in fp64 (a library
routine); the whole loss to a two-token case evaluated by hand from the definitions
(blog 2.1.1, 2.2.1, 2.2.2); and to invariants the definitions fix: zero when one chunk
covers the clip, zero for constant values, a^2 scaling and shift invariance in V.
"""
import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def rand(p, seed, bias=False):
    rng = np.random.default_rng(seed)
    sh = (p.B, p.H, p.N, p.D)
    x = dict(q=rng.standard_normal(sh), k=rng.standard_normal(sh), v=rng.standard_normal(sh),
             wq=rng.standard_normal((p.H, p.Dphi, p.D)) / math.sqrt(p.D),
             wk=rng.standard_normal((p.H, p.Dphi, p.D)) / math.sqrt(p.D))
    x["bq"] = rng.standard_normal((p.H, p.Dphi)) * 0.5 if bias else None
    x["bk"] = rng.standard_normal((p.H, p.Dphi)) * 0.5 if bias else None
    return x


def loss(p, x):
    return oracle.distill_loss(p, x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"])


def test_teacher_is_sdpa():
    p = oracle.Params(2, 3, 16, 5, 7, 2, 1, 8, 2)
    x = rand(p, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x[key]) for key in ("q", "k", "v"))).numpy()
    got = oracle.full_softmax(p, x["q"], x["k"], x["v"])
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    rows = np.array([0, 4, 20, 34])
    assert np.array_equal(oracle.full_softmax(p, x["q"], x["k"], x["v"], rows=rows), got[:, :, rows])


def test_two_tokens_by_hand():
    """T = 2 frames of one token, Tc = 1, To = 0, D = 2, Dphi = 1, P = 2.  Token 0 sees only
    itself in softmax; token 1 sees itself in softmax and token 0 through the polynomial
    kernel kappa = (u w) + (u w)^2 with u = softplus(W_q q_1), w = softplus(W_k k_0)."""
    p = oracle.Params(1, 1, 2, 2, 1, 1, 0, 1, 2)
    q = np.array([[0.3, -1.1], [0.8, 0.5]])
    k = np.array([[-0.4, 0.9], [1.2, -0.7]])
    v = np.array([[1.5, -2.0], [0.25, 3.0]])
    wq, wk = np.array([[0.6, -0.2]]), np.array([[-0.5, 0.7]])
    sp = lambda t: math.log1p(math.exp(t))
    dot = lambda a, b: float(a @ b)
    s = lambda i, j: dot(q[i], k[j]) / math.sqrt(2.0)
    # student
    o0 = v[0]
    u, w = sp(dot(wq[0], q[1])), sp(dot(wk[0], k[0]))
    kap = u * w + (u * w) ** 2
    e11 = math.exp(s(1, 1))
    o1 = (e11 * v[1] + kap * v[0]) / (e11 + kap)
    # teacher
    t = [(math.exp(s(i, 0)) * v[0] + math.exp(s(i, 1)) * v[1]) / (math.exp(s(i, 0)) + math.exp(s(i, 1)))
         for i in range(2)]
    want = float(((o0 - t[0]) ** 2).sum() + ((o1 - t[1]) ** 2).sum())
    got = oracle.distill_loss(p, q[None, None], k[None, None], v[None, None], wq[None], wk[None])
    assert got.shape == (1, 1)
    assert abs(got[0, 0] - want) <= 1e-13 * want


@pytest.mark.parametrize("shape", [
    (1, 2, 8, 7, 4, 3, 1, 8, 2), (2, 1, 16, 6, 5, 2, 0, 16, 3), (1, 1, 32, 9, 3, 4, 2, 32, 1)])
def test_invariants(shape):
    p = oracle.Params(*shape)
    x = rand(p, 1, bias=True)
    base = loss(p, x)
    assert base.shape == (p.B, p.H) and (base > 0).all()
    # one chunk over the clip: the hybrid output is the teacher's
    one = oracle.Params(*shape[:5], p.T, shape[6], *shape[7:])
    assert (loss(one, x) <= 1e-24 * np.abs(x["v"]).max() ** 2 * p.N * p.D).all()
    # constant values: every output is that constant
    c = dict(x, v=np.broadcast_to(np.arange(p.D, dtype=np.float64), x["v"].shape).copy())
    assert (loss(p, c) <= 1e-22 * p.N * p.D ** 3).all()
    # V -> a V + b: both outputs move the same way (convex combinations)
    a, b = -2.5, 0.75
    y = dict(x, v=a * x["v"] + b)
    assert np.allclose(loss(p, y), a * a * base, rtol=1e-10)
    # slabs are independent: a change in one slab moves only its loss
    z = dict(x, v=x["v"].copy())
    z["v"][0, 0] *= 3.0
    lz = loss(p, z)
    assert np.array_equal(lz.reshape(-1)[1:], base.reshape(-1)[1:])
