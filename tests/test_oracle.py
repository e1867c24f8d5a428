"""Pins for the fp64 oracle against what the ReHyAt pages and plain mathematics fix.

The pages print no worked numeric example, so the pins are: hand-derived schedules and
feature layouts (tests/golden), reductions to textbook routines (softmax attention when
one chunk covers the clip, normalised linear attention when the softmax window is empty),
closed forms (constant feature maps, known softplus values), invariants of the map
(causality, convex combination, affine equivariance, permutation within a frame, slab
independence), and agreement of five constructions of the same map (brute force in C,
brute force in numpy, recurrent, chunk-parallel, streaming).

Citations: ReHyAt blog (maplevalley.com.cn) sections 2.1.1, 2.2.1, 2.2.2, 2.3, 5.2;
mind-verse.de summary (overlapping chunks, recurrent reformulation).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import Params

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(p: Params, seed=0, bias=False, scale_w=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((p.B, p.H, p.N, p.D))
    k = rng.standard_normal((p.B, p.H, p.N, p.D))
    v = rng.standard_normal((p.B, p.H, p.N, p.D))
    sw = 1.0 / math.sqrt(p.D) if scale_w is None else scale_w
    wq = rng.standard_normal((p.H, p.Dphi, p.D)) * sw
    wk = rng.standard_normal((p.H, p.Dphi, p.D)) * sw
    bq = rng.standard_normal((p.H, p.Dphi)) * 0.5 if bias else None
    bk = rng.standard_normal((p.H, p.Dphi)) * 0.5 if bias else None
    return q, k, v, wq, wk, bq, bk


def rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


# ---------------------------------------------------------------- schedule / masks ---

def _parse_tiny():
    chunks, frames = [], {}
    for line in open(os.path.join(GOLDEN, "schedule_tiny.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tok = line.split()
        if tok[0] == "chunk":
            chunks.append([int(t) for t in tok[2:]])
        elif tok[0] == "frame":
            f = int(tok[1])
            rest = line.split(":", 1)[1]
            soft, lin = rest.split("|")
            frames[f] = ([int(t) for t in soft.split()], [int(t) for t in lin.split()])
    return np.array(chunks), frames


def _parse_edge():
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "schedule_edge.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = ([int(t) for t in tok[1:]], [])
            cases.append(cur)
        else:
            cur[1].append([int(t) for t in tok[2:]])
    return cases


TINY = Params(B=1, H=2, D=32, T=7, n=16, Tc=3, To=1, Dphi=32, P=2)


def test_schedule_tiny_golden():
    chunks, _ = _parse_tiny()
    np.testing.assert_array_equal(oracle.schedule(TINY), chunks)


@pytest.mark.parametrize("case", range(len(_parse_edge())))
def test_schedule_edge_golden(case):
    (T, Tc, To, lin), rows = _parse_edge()[case]
    p = Params(1, 1, 32, T, 1, Tc, To, 32, 2, lin)
    np.testing.assert_array_equal(oracle.schedule(p), np.array(rows))


def test_regions_behave_as_golden_masks():
    """Perturbing one frame changes exactly the queries whose softmax or linear region holds
    it, per the hand-derived table (blog 2.2.1 regions, 2.3 causality)."""
    _, frames = _parse_tiny()
    p = TINY.with_(H=1, n=3)
    q, k, v, wq, wk, _, _ = rand_inputs(p, seed=1)
    base = oracle.bruteforce(p, q, k, v, wq, wk)
    for g in range(p.T):
        k2, v2 = k.copy(), v.copy()
        sl = slice(g * p.n, (g + 1) * p.n)
        k2[:, :, sl] += 0.37
        v2[:, :, sl] -= 0.81
        out = oracle.bruteforce(p, q, k2, v2, wq, wk)
        for f in range(p.T):
            soft, lin = frames[f]
            d = np.abs(out[0, 0, f * p.n:(f + 1) * p.n] - base[0, 0, f * p.n:(f + 1) * p.n]).max()
            if g in soft or g in lin:
                assert d > 1e-6, (g, f)
            else:
                assert d == 0.0, (g, f)


def test_numpy_masks_match_golden():
    _, frames = _parse_tiny()
    soft, lin = oracle.numpy_masks(TINY)
    n = TINY.n
    for f, (sf, lf) in frames.items():
        i = f * n + 5
        assert sorted(set(np.nonzero(soft[i])[0] // n)) == sf
        assert sorted(set(np.nonzero(lin[i])[0] // n)) == lf


# ------------------------------------------------------------------------------ phi ---

def _parse_phi():
    info, feats = {}, {}
    for line in open(os.path.join(GOLDEN, "phi_layout.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tok = line.split()
        if tok[0] == "P":
            feats[int(tok[1])] = [float(t) for t in tok[3:]]
        else:
            info[tok[0]] = [float(t) for t in tok[1:]]
    return info, feats


@pytest.mark.parametrize("P", [1, 2, 3])
@pytest.mark.parametrize("via_bias", [False, True])
def test_phi_layout_golden(P, via_bias):
    """blog 2.2.2: split into P parts, powers 1..P per part, concatenated."""
    info, feats = _parse_phi()
    perm = [int(t) for t in info["perm"]]
    a = np.array(info["a"])
    p = Params(1, 1, 4, 1, 1, 1, 0, 4, P)
    if via_bias:
        w = np.zeros((1, 4, 4))
        bias = np.log(np.expm1(np.array(info["u"])))[None]
        x = np.zeros((1, 1, 1, 4))
    else:
        w = np.zeros((1, 4, 4))
        for j, d in enumerate(perm):
            w[0, j, d] = 1.0
        bias = None
        x = np.log(np.expm1(a))[None, None, None]
    f = oracle.phi(p, x, w, bias)
    np.testing.assert_allclose(f[0, 0, 0], feats[P], rtol=1e-13, atol=1e-13)


def test_phi_p1_is_softplus():
    p = Params(2, 3, 32, 2, 5, 1, 0, 32, 1)
    q, _, _, wq, _, bq, _ = rand_inputs(p, seed=2, bias=True)
    f = oracle.phi(p, q, wq, bq)
    ref = torch.nn.functional.softplus(
        torch.einsum("bhnd,hjd->bhnj", torch.tensor(q), torch.tensor(wq)) + torch.tensor(bq)[None, :, None])
    np.testing.assert_allclose(f, ref.numpy(), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("P,Dphi", [(2, 32), (3, 32), (3, 7), (4, 10)])
def test_kappa_closed_form(P, Dphi):
    """phi_q(q).phi_k(k) = sum_j sum_p (u_j w_j)^p for every split (blog 2.2.2)."""
    p = Params(1, 2, 16, 1, 9, 1, 0, Dphi, P)
    q, k, _, wq, wk, bq, bk = rand_inputs(p, seed=3, bias=True)
    fq, fk = oracle.phi(p, q, wq, bq), oracle.phi(p, k, wk, bk)
    sp = torch.nn.functional.softplus
    uq = sp(torch.einsum("bhnd,hjd->bhnj", torch.tensor(q), torch.tensor(wq)) + torch.tensor(bq)[None, :, None]).numpy()
    uk = sp(torch.einsum("bhnd,hjd->bhnj", torch.tensor(k), torch.tensor(wk)) + torch.tensor(bk)[None, :, None]).numpy()
    kap = np.einsum("bhif,bhjf->bhij", fq, fk)
    ref = sum(np.einsum("bhij,bhkj->bhik", uq ** e, uk ** e) for e in range(1, P + 1))
    np.testing.assert_allclose(kap, ref, rtol=1e-12)


# ---------------------------------------------------------------- reductions ---------

@pytest.mark.parametrize("T,Tc,To", [(5, 5, 1), (4, 9, 0), (6, 6, 3)])
def test_one_chunk_is_softmax_attention(T, Tc, To):
    """Tc >= T: one chunk, no linear region: plain softmax attention (blog 2.1.1)."""
    p = Params(2, 2, 32, T, 7, Tc, To, 32, 2)
    q, k, v, wq, wk, _, _ = rand_inputs(p, seed=4)
    out = oracle.bruteforce(p, q, k, v, wq, wk)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q), torch.tensor(k), torch.tensor(v))
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def _linear_closed_form(p, q, k, v, wq, wk, chunk_causal):
    sp = torch.nn.functional.softplus
    uq = sp(torch.einsum("bhnd,hjd->bhnj", torch.tensor(q), torch.tensor(wq))).numpy()
    uk = sp(torch.einsum("bhnd,hjd->bhnj", torch.tensor(k), torch.tensor(wk))).numpy()
    kap = sum(np.einsum("bhij,bhkj->bhik", uq ** e, uk ** e) for e in range(1, p.P + 1))
    if chunk_causal:
        ch = (np.arange(p.N) // p.n) // p.Tc
        kap = kap * (ch[None, :] <= ch[:, None])
    return np.einsum("bhij,bhjd->bhid", kap, v) / kap.sum(-1)[..., None]


def test_empty_window_one_chunk_is_linear_attention():
    """linear_only with Tc >= T: phi_q(Q)[phi_k(K)^T V] / phi_q(Q)[phi_k(K)^T 1]."""
    p = Params(1, 2, 32, 4, 6, 4, 1, 32, 2, linear_only=1)
    q, k, v, wq, wk, _, _ = rand_inputs(p, seed=5)
    out = oracle.bruteforce(p, q, k, v, wq, wk)
    np.testing.assert_allclose(out, _linear_closed_form(p, q, k, v, wq, wk, False), rtol=1e-11)


def test_empty_window_is_chunk_causal_linear_attention():
    p = Params(1, 2, 32, 7, 5, 3, 1, 32, 3, linear_only=1)
    q, k, v, wq, wk, _, _ = rand_inputs(p, seed=6)
    out = oracle.parallel(p, q, k, v, wq, wk)
    np.testing.assert_allclose(out, _linear_closed_form(p, q, k, v, wq, wk, True), rtol=1e-11)


@pytest.mark.parametrize("P", [1, 2, 3])
def test_constant_feature_map_closed_form(P):
    """q = 0 and W = 0: every softmax weight is e^0 = 1 and every linear weight is the
    constant kappa = Dphi * sum_p (ln 2)^(2p) (softplus(0) = ln 2), so each output is a
    weighted mean of the visible values with region sizes from the golden table."""
    _, frames = _parse_tiny()
    p = TINY.with_(P=P)
    _, _, v, _, _, _, _ = rand_inputs(p, seed=7)
    q = np.zeros_like(v)
    k = np.random.default_rng(8).standard_normal(v.shape)
    w0 = np.zeros((p.H, p.Dphi, p.D))
    out = oracle.bruteforce(p, q, k, v, w0, w0)
    kappa = p.Dphi * sum(math.log(2.0) ** (2 * e) for e in range(1, P + 1))
    n = p.n
    for f, (sf, lf) in frames.items():
        vs = sum(v[:, :, g * n:(g + 1) * n].sum(2) for g in sf)
        vl = sum(v[:, :, g * n:(g + 1) * n].sum(2) for g in lf) if lf else 0.0
        ref = (vs + kappa * vl) / (len(sf) * n + kappa * len(lf) * n)
        for i in range(f * n, (f + 1) * n):
            np.testing.assert_allclose(out[:, :, i], ref, rtol=1e-12)


def test_bias_only_feature_map_closed_form():
    """W = 0 with biases b = log(expm1(a)): u = a exactly, kappa = sum_j sum_p (a_j c_j)^p."""
    p = TINY.with_(H=1)
    rng = np.random.default_rng(9)
    a = rng.uniform(0.2, 1.5, p.Dphi)
    c = rng.uniform(0.2, 1.5, p.Dphi)
    v = rng.standard_normal((1, 1, p.N, p.D))
    q = np.zeros_like(v)
    k = rng.standard_normal(v.shape)
    w0 = np.zeros((1, p.Dphi, p.D))
    out = oracle.parallel(p, q, k, v, w0, w0, np.log(np.expm1(a))[None], np.log(np.expm1(c))[None])
    kappa = sum(((a * c) ** e).sum() for e in range(1, p.P + 1))
    _, frames = _parse_tiny()
    n = p.n
    f = 6
    sf, lf = frames[f]
    vs = sum(v[0, 0, g * n:(g + 1) * n].sum(0) for g in sf)
    vl = sum(v[0, 0, g * n:(g + 1) * n].sum(0) for g in lf)
    ref = (vs + kappa * vl) / (len(sf) * n + kappa * len(lf) * n)
    np.testing.assert_allclose(out[0, 0, f * n], ref, rtol=1e-12)


# -------------------------------------------------------- five constructions agree ---

EDGE = [
    TINY,
    TINY.with_(B=2, H=1),
    Params(1, 2, 32, 10, 3, 4, 2, 32, 2),          # To=2, uneven tail
    Params(1, 1, 32, 6, 4, 2, 0, 32, 2),           # To=0
    Params(1, 1, 32, 7, 3, 2, 3, 32, 2),           # To > Tc
    Params(1, 1, 32, 2, 5, 3, 1, 32, 2),           # T < Tc
    Params(1, 1, 32, 1, 6, 3, 1, 32, 2),           # T = 1
    Params(1, 2, 32, 8, 1, 3, 1, 32, 2),           # n = 1
    Params(1, 1, 32, 7, 4, 3, 1, 32, 1),           # P = 1
    Params(1, 1, 64, 7, 4, 3, 1, 32, 3),           # P = 3, uneven split 11/11/10
    Params(1, 2, 32, 7, 4, 3, 1, 32, 2, 1),        # linear_only
    Params(2, 1, 16, 9, 3, 1, 1, 8, 2),            # Tc = 1 (spatial-only softmax)
]


@pytest.mark.parametrize("p", EDGE, ids=lambda p: f"T{p.T}n{p.n}Tc{p.Tc}To{p.To}P{p.P}L{p.linear_only}B{p.B}")
@pytest.mark.parametrize("bias", [False, True])
def test_constructions_agree(p, bias):
    """recurrent == chunk-parallel == streaming == brute force (C) == brute force (numpy):
    the recurrent and streaming forms are reformulations of the same map (abstract;
    mind-verse.de 'Rekurrente Formulierung'; blog 2.3 and 5.2)."""
    q, k, v, wq, wk, bq, bk = rand_inputs(p, seed=10, bias=bias)
    ref, aux = oracle.bruteforce(p, q, k, v, wq, wk, bq, bk, aux=True)
    assert rel(oracle.numpy_bruteforce(p, q, k, v, wq, wk, bq, bk), ref) < 1e-12
    r2, aux2 = oracle.recurrent(p, q, k, v, wq, wk, bq, bk, aux=True)
    r3, aux3 = oracle.parallel(p, q, k, v, wq, wk, bq, bk, aux=True)
    assert rel(r2, ref) < 1e-12
    assert rel(r3, ref) < 1e-12
    assert rel(oracle.stream(p, q, k, v, wq, wk, bq, bk), ref) < 1e-12
    for key in ("osoft", "y", "z"):
        assert rel(aux2[key], aux[key]) < 1e-12
        assert rel(aux3[key], aux[key]) < 1e-12
    fin = np.isfinite(aux["lse"])
    np.testing.assert_array_equal(fin, np.isfinite(aux3["lse"]))
    np.testing.assert_allclose(aux3["lse"][fin], aux["lse"][fin], rtol=1e-12)


def test_aux_parts_recompose_and_match_libraries():
    """osoft is softmax over the window, lse its log-sum-exp, and the output is the shared
    normalisation (e^lse osoft + y) / (e^lse + z) (blog 2.2.1)."""
    from scipy.special import logsumexp, softmax
    p = TINY
    q, k, v, wq, wk, _, _ = rand_inputs(p, seed=11)
    out, aux = oracle.parallel(p, q, k, v, wq, wk, aux=True)
    sched = oracle.schedule(p)
    for b in range(p.B):
        for h in range(p.H):
            for i in [0, 17, 47, 48, 60, 95, 96, 111]:
                f0, f1, ws, we, ls = sched[(i // p.n) // p.Tc]
                s = k[b, h, ws * p.n:we * p.n] @ q[b, h, i] / math.sqrt(p.D)
                np.testing.assert_allclose(aux["lse"][b, h, i], logsumexp(s), rtol=1e-13)
                np.testing.assert_allclose(aux["osoft"][b, h, i], softmax(s) @ v[b, h, ws * p.n:we * p.n],
                                           rtol=1e-11, atol=1e-13)
                e = math.exp(aux["lse"][b, h, i])
                rec = (e * aux["osoft"][b, h, i] + aux["y"][b, h, i]) / (e + aux["z"][b, h, i])
                np.testing.assert_allclose(out[b, h, i], rec, rtol=1e-12, atol=1e-14)


def test_parallel_rows_matches_full():
    p = Params(2, 2, 32, 7, 9, 3, 1, 32, 2)
    q, k, v, wq, wk, bq, bk = rand_inputs(p, seed=12, bias=True)
    full, aux = oracle.parallel(p, q, k, v, wq, wk, bq, bk, aux=True)
    rows = np.array([0, 8, 26, 27, 62, 63 + 1, p.N + 5, 3 * p.N + p.N - 1])
    out, ax = oracle.parallel_rows(p, q, k, v, wq, wk, rows, bq, bk)
    np.testing.assert_allclose(out, full.reshape(-1, p.D)[rows], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(ax["y"], aux["y"].reshape(-1, p.D)[rows], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(ax["z"], aux["z"].reshape(-1)[rows], rtol=1e-13)


# ------------------------------------------------------------------ invariants -------

def test_causality_future_frames_do_not_matter():
    """blog 2.3: a chunk attends only to earlier chunks (and its own window)."""
    p = Params(1, 2, 32, 9, 4, 3, 1, 32, 2)
    q, k, v, wq, wk, _, _ = rand_inputs(p, seed=13)
    base = oracle.parallel(p, q, k, v, wq, wk)
    cut = 6 * p.n  # chunk 2 starts at frame 6
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    rng = np.random.default_rng(14)
    for a in (q2, k2, v2):
        a[:, :, cut:] = rng.standard_normal(a[:, :, cut:].shape)
    out = oracle.parallel(p, q2, k2, v2, wq, wk)
    np.testing.assert_array_equal(out[:, :, :cut], base[:, :, :cut])
    assert np.abs(out[:, :, cut:] - base[:, :, cut:]).max() > 1e-3


def test_outputs_are_convex_combinations():
    p = Params(1, 2, 32, 7, 6, 3, 1, 32, 2)
    q, k, v, wq, wk, _, _ = rand_inputs(p, seed=15)
    out = oracle.bruteforce(p, q, k, v, wq, wk)
    soft, lin = oracle.numpy_masks(p)
    vis = soft | lin
    for b in range(p.B):
        for h in range(p.H):
            for i in range(p.N):
                vv = v[b, h][vis[i]]
                assert np.all(out[b, h, i] <= vv.max(0) + 1e-12)
                assert np.all(out[b, h, i] >= vv.min(0) - 1e-12)


def test_affine_equivariance_in_values():
    p = Params(1, 1, 32, 7, 5, 3, 1, 32, 2)
    q, k, v, wq, wk, _, _ = rand_inputs(p, seed=16)
    base = oracle.parallel(p, q, k, v, wq, wk)
    shift = np.random.default_rng(17).standard_normal(p.D)
    out = oracle.parallel(p, q, k, -2.5 * v + shift, wq, wk)
    np.testing.assert_allclose(out, -2.5 * base + shift, rtol=1e-11, atol=1e-12)


def test_permutation_within_frames():
    p = Params(1, 1, 32, 7, 6, 3, 1, 32, 2)
    q, k, v, wq, wk, _, _ = rand_inputs(p, seed=18)
    base = oracle.parallel(p, q, k, v, wq, wk)
    rng = np.random.default_rng(19)
    perm = np.concatenate([f * p.n + rng.permutation(p.n) for f in range(p.T)])
    out = oracle.parallel(p, q[:, :, perm], k[:, :, perm], v[:, :, perm], wq, wk)
    np.testing.assert_allclose(out, base[:, :, perm], rtol=1e-12, atol=1e-13)


def test_slabs_are_independent():
    p = Params(2, 3, 32, 7, 4, 3, 1, 32, 2)
    q, k, v, wq, wk, _, _ = rand_inputs(p, seed=20)
    out = oracle.parallel(p, q, k, v, wq, wk)
    p1 = p.with_(B=1, H=1)
    for b in range(p.B):
        for h in range(p.H):
            o1 = oracle.parallel(p1, q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                 wq[h:h + 1], wk[h:h + 1])
            np.testing.assert_allclose(out[b, h], o1[0, 0], rtol=1e-14, atol=1e-15)


def test_stream_rejects_bad_calls():
    p = TINY
    q, k, v, wq, wk, _, _ = rand_inputs(p, seed=21)
    st = oracle.Stream(p, wq, wk)
    sl = slice(0, 4 * p.n)
    with pytest.raises(ValueError):
        st.step(q[:, :, sl], k[:, :, sl], v[:, :, sl], 4)     # more than Tc frames
    sl = slice(0, 2 * p.n)
    st.step(q[:, :, sl], k[:, :, sl], v[:, :, sl], 2)         # short chunk closes the stream
    with pytest.raises(ValueError):
        st.step(q[:, :, sl], k[:, :, sl], v[:, :, sl], 2)
