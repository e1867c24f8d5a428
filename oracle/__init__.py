"""fp64 CPU oracle for ReHyAt chunk-wise hybrid attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code with
the HIP library and never imports it.

Two independent implementations live here:

* ``librehyat_oracle.so`` (``rehyat_oracle.c``): the brute-force definition plus the
  recurrent, chunk-parallel and streaming forms, all in fp64;
* ``numpy_bruteforce`` below: a second brute force written from the same pages with a
  different construction (explicit N x N masks and the closed form of the polynomial
  kernel), used to cross-check the C code.

Sources: the ReHyAt blog post (maplevalley.com.cn) sections 2.1.1, 2.2.1, 2.2.2, 2.3
and 5.2; the mind-verse.de summary sections on overlapping chunks and the recurrent
formulation.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rehyat_oracle.c")
_LIB_PATH = os.path.join(_HERE, "librehyat_oracle.so")
# A test may point the loader at a deliberately mutated build of the same source, to
# show that the pins fail on plausible mistakes.
_OVERRIDE = os.environ.get("REHYAT_ORACLE_LIB")


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(out_dir: str) -> str:
    """The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (clang, the runtime
    the sanitized librehyat uses; no OpenMP, so the pragmas are ignored).  Test tooling."""
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, "librehyat_oracle_san.so")
    tmp = path + ".tmp"
    subprocess.run(
        ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-shared-libsan", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
         "-Wno-unknown-pragmas", "-o", tmp, _SRC, "-lm"],
        check=True,
    )
    os.replace(tmp, path)
    return path


class _Params(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int) for name in
                ("B", "H", "D", "T", "n", "Tc", "To", "Dphi", "P", "linear_only")]


@dataclass(frozen=True)
class Params:
    B: int
    H: int
    D: int
    T: int
    n: int
    Tc: int
    To: int
    Dphi: int
    P: int
    linear_only: int = 0

    @property
    def N(self) -> int:
        return self.T * self.n

    @property
    def F(self) -> int:
        return self.P * self.Dphi

    def with_(self, **kw) -> "Params":
        return replace(self, **kw)

    def _c(self) -> _Params:
        return _Params(self.B, self.H, self.D, self.T, self.n, self.Tc, self.To, self.Dphi,
                       self.P, int(self.linear_only))


_lib = None
_D = ctypes.POINTER(ctypes.c_double)


def lib():
    global _lib
    if _lib is None:
        path = _OVERRIDE or _LIB_PATH
        if not _OVERRIDE and not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.POINTER(_Params)
        L.orc_schedule.argtypes = [P, ctypes.POINTER(ctypes.c_int)]
        L.orc_schedule.restype = ctypes.c_int
        L.orc_features.argtypes = [P]
        L.orc_features.restype = ctypes.c_int
        L.orc_phi.argtypes = [P, _D, _D, _D, _D]
        L.orc_phi.restype = None
        six = [P, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D]
        for name in ("orc_bruteforce", "orc_recurrent", "orc_parallel"):
            getattr(L, name).argtypes = six
            getattr(L, name).restype = None
        L.orc_parallel_rows.argtypes = [P, _D, _D, _D, _D, _D, _D, _D, ctypes.c_int64,
                                        ctypes.POINTER(ctypes.c_int64), _D, _D, _D, _D, _D]
        L.orc_parallel_rows.restype = None
        L.orc_stream_state_doubles.argtypes = [P]
        L.orc_stream_state_doubles.restype = ctypes.c_int64
        L.orc_stream_init.argtypes = [P, _D]
        L.orc_stream_init.restype = None
        L.orc_stream_step.argtypes = [P, _D, _D, _D, _D, ctypes.c_int, _D, _D, _D, _D, _D]
        L.orc_stream_step.restype = ctypes.c_int
        _lib = L
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return ctypes.cast(None, _D)
    return a.ctypes.data_as(_D)


def schedule(p: Params) -> np.ndarray:
    """[nc, 5] int table of (f0, f1, ws, we, ls) per chunk."""
    nc = lib().orc_schedule(ctypes.byref(p._c()), None)
    out = np.zeros((nc, 5), dtype=np.int32)
    lib().orc_schedule(ctypes.byref(p._c()), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int)))
    return out


def phi(p: Params, x, w, bias=None) -> np.ndarray:
    """Feature map over [B,H,N,D] -> [B,H,N,F] (fp64)."""
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    feat = np.empty(x.shape[:-1] + (p.F,), dtype=np.float64)
    lib().orc_phi(ctypes.byref(p._c()), _ptr(x), _ptr(w), _ptr(bias), _ptr(feat))
    return feat


def _run(name, p: Params, q, k, v, wq, wk, bq=None, bk=None, aux=False):
    q, k, v, wq, wk, bq, bk = map(_f64, (q, k, v, wq, wk, bq, bk))
    shape = (p.B, p.H, p.N, p.D)
    for a in (q, k, v):
        assert a.shape == shape, (a.shape, shape)
    out = np.empty(shape)
    ax = None
    if aux:
        ax = dict(osoft=np.empty(shape), lse=np.empty(shape[:-1]), y=np.empty(shape),
                  z=np.empty(shape[:-1]))
    getattr(lib(), name)(ctypes.byref(p._c()), _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk),
                         _ptr(bq), _ptr(bk), _ptr(out),
                         *(_ptr(ax[key]) if ax else _ptr(None) for key in ("osoft", "lse", "y", "z")))
    return (out, ax) if aux else out


def bruteforce(p, q, k, v, wq, wk, bq=None, bk=None, aux=False):
    return _run("orc_bruteforce", p, q, k, v, wq, wk, bq, bk, aux)


def recurrent(p, q, k, v, wq, wk, bq=None, bk=None, aux=False):
    return _run("orc_recurrent", p, q, k, v, wq, wk, bq, bk, aux)


def parallel(p, q, k, v, wq, wk, bq=None, bk=None, aux=False):
    return _run("orc_parallel", p, q, k, v, wq, wk, bq, bk, aux)


def parallel_rows(p, q, k, v, wq, wk, rows, bq=None, bk=None):
    """Outputs (and aux parts) for selected flattened rows of [B*H*N]; states in full."""
    q, k, v, wq, wk, bq, bk = map(_f64, (q, k, v, wq, wk, bq, bk))
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    R = rows.shape[0]
    out, osoft, y = (np.empty((R, p.D)) for _ in range(3))
    lse, z = np.empty(R), np.empty(R)
    lib().orc_parallel_rows(ctypes.byref(p._c()), _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk),
                            _ptr(bq), _ptr(bk), R,
                            rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                            _ptr(out), _ptr(osoft), _ptr(lse), _ptr(y), _ptr(z))
    return out, dict(osoft=osoft, lse=lse, y=y, z=z)


class Stream:
    """Chunk-by-chunk form with carried state (blog section 5.2 streaming loop)."""

    def __init__(self, p: Params, wq, wk, bq=None, bk=None):
        self.p = p
        self.wq, self.wk, self.bq, self.bk = map(_f64, (wq, wk, bq, bk))
        self.state = np.zeros(lib().orc_stream_state_doubles(ctypes.byref(p._c())))
        lib().orc_stream_init(ctypes.byref(p._c()), _ptr(self.state))

    def step(self, q, k, v, frames: int) -> np.ndarray:
        q, k, v = map(_f64, (q, k, v))
        out = np.empty_like(q)
        rc = lib().orc_stream_step(ctypes.byref(self.p._c()), _ptr(self.state), _ptr(q), _ptr(k),
                                   _ptr(v), frames, _ptr(self.wq), _ptr(self.wk), _ptr(self.bq),
                                   _ptr(self.bk), _ptr(out))
        if rc != 0:
            raise ValueError("oracle stream step rejected (frames out of range or stream closed)")
        return out


def stream(p, q, k, v, wq, wk, bq=None, bk=None):
    """Run the streaming form over the whole sequence, Tc frames per call."""
    st = Stream(p, wq, wk, bq, bk)
    q, k, v = map(_f64, (q, k, v))
    out = np.empty_like(q)
    for f0 in range(0, p.T, p.Tc):
        f1 = min(f0 + p.Tc, p.T)
        sl = slice(f0 * p.n, f1 * p.n)
        out[:, :, sl] = st.step(q[:, :, sl], k[:, :, sl], v[:, :, sl], f1 - f0)
    return out


# ---------------------------------------------------------------------------------------
# Second, independent brute force (numpy).  Built from the same definitions but a
# different construction: explicit frame-interval masks, dense score matrices, and the
# polynomial kernel in its closed form kappa(q,k) = sum_j sum_{p=1..P} (u_j w_j)^p, which
# holds because every part of phi carries every power 1..P (blog 2.2.2).
# ---------------------------------------------------------------------------------------

def _softplus(x):
    return np.logaddexp(0.0, x)


def numpy_masks(p: Params):
    """Boolean [N, N] masks (softmax region, linear region) from the frame rules."""
    frame = np.arange(p.N) // p.n
    chunk = frame // p.Tc
    f0 = chunk * p.Tc
    f1 = np.minimum(f0 + p.Tc, p.T)
    if p.linear_only:
        lo, hi, lin_end = f1, f1, f1
    else:
        lo, hi = np.maximum(f0 - p.To, 0), f1
        lin_end = lo
    kf = frame[None, :]
    soft = (kf >= lo[:, None]) & (kf < hi[:, None])
    lin = kf < lin_end[:, None]
    return soft, lin


def numpy_bruteforce(p: Params, q, k, v, wq, wk, bq=None, bk=None):
    q, k, v, wq, wk = map(_f64, (q, k, v, wq, wk))
    soft, lin = numpy_masks(p)
    out = np.empty_like(q)
    for b in range(p.B):
        for h in range(p.H):
            uq = np.einsum("jd,nd->nj", wq[h], q[b, h])
            uk = np.einsum("jd,nd->nj", wk[h], k[b, h])
            if bq is not None:
                uq = uq + np.asarray(bq, dtype=np.float64)[h]
            if bk is not None:
                uk = uk + np.asarray(bk, dtype=np.float64)[h]
            uq, uk = _softplus(uq), _softplus(uk)
            prod = uq[:, None, :] * uk[None, :, :]            # [N, N, Dphi]
            kappa = sum((prod ** e).sum(-1) for e in range(1, p.P + 1))
            s = q[b, h] @ k[b, h].T / np.sqrt(p.D)
            smax = np.where(soft, s, -np.inf).max(axis=1, keepdims=True)
            shift = np.maximum(np.where(np.isfinite(smax), smax, 0.0), 0.0)
            w = np.where(soft, np.exp(s - shift), 0.0) + np.where(lin, kappa * np.exp(-shift), 0.0)
            out[b, h] = (w @ v[b, h]) / w.sum(axis=1, keepdims=True)
    return out


# ---------------------------------------------------------------------------------------
# Attention distillation objective (blog 3.1.1): with the softmax teacher frozen, only
# phi_q and phi_k are trained, so that the hybrid block's output approaches the teacher's
# in L2 on the same inputs.  Reading taken: the squared Euclidean distance per
# (batch, head) slab, between the hybrid output and full softmax attention over the
# whole clip.
# ---------------------------------------------------------------------------------------

def full_softmax(p: Params, q, k, v, rows=None):
    """Teacher: softmax(q k^T / sqrt(D)) v over all N tokens of the clip (blog 2.1.1),
    for every query, or only for the given token indices of each slab."""
    q, k, v = map(_f64, (q, k, v))
    if rows is not None:
        q = q[:, :, np.asarray(rows)]
    out = np.empty(q.shape)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            s = q[b, h] @ k[b, h].T / np.sqrt(p.D)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, h] = (e @ v[b, h]) / e.sum(axis=1, keepdims=True)
    return out


def distill_loss(p: Params, q, k, v, wq, wk, bq=None, bk=None):
    """[B, H]: sum over tokens and channels of (hybrid - full softmax)^2, fp64."""
    hyb = parallel(p, q, k, v, wq, wk, bq, bk)
    soft = full_softmax(p, q, k, v)
    return ((hyb - soft) ** 2).sum(axis=(2, 3))


# ---------------------------------------------------------------------------------------
# Gradients of the distillation objective with respect to the feature-map parameters
# (blog 3.1.1: only phi_q and phi_k are trained; the teacher does not depend on them).
# With L = sum over slabs of distill_loss, g_i = dL/do_i = 2 (o_i - t_i), and the hybrid
# output o_i = num_i / den_i of blog 2.2.1:
#   dL/dkappa_ij = a_i . v_j - h_i   for j in the linear region of i, where
#   a_i = g_i / den_i and h_i = (g_i . o_i) / den_i;
#   kappa_ij = phi_q(q_i) . phi_k(k_j), so dL/dphi_q(q_i) = sum_j dL/dkappa_ij phi_k(k_j)
#   and dL/dphi_k(k_j) = sum_i dL/dkappa_ij phi_q(q_i);
#   phi = per-part powers u^p of u = softplus(pre), pre = W x + b (blog 2.2.2), so
#   dL/du_j = sum_p p u_j^(p-1) dL/dphi_(j,p), dL/dpre = dL/du * sigmoid(pre),
#   dL/dW = sum over tokens of dL/dpre x^T, dL/db = sum over tokens of dL/dpre.
# ---------------------------------------------------------------------------------------

def feature_map(p: Params):
    """(element, power) of every feature in phi's layout: parts are contiguous ranges of
    the Dphi elements (the first Dphi mod P parts one longer) and each part lists all its
    elements at power 1, then at power 2, ..., then P (blog 2.2.2)."""
    q, r = divmod(p.Dphi, p.P)
    elem, power = [], []
    start = 0
    for part in range(p.P):
        ln = q + (1 if part < r else 0)
        for pw in range(1, p.P + 1):
            elem += list(range(start, start + ln))
            power += [pw] * ln
        start += ln
    return np.array(elem), np.array(power)


def _phi_parts(p, x, w, b):
    """pre = W x + b, u = softplus(pre), phi [N, F] for one slab."""
    pre = x @ w.T
    if b is not None:
        pre = pre + b
    u = _softplus(pre)
    elem, power = feature_map(p)
    return pre, u, u[:, elem] ** power


def _phi_backward(p, pre, u, x, dphi):
    """dL/dW and dL/db of one slab from dL/dphi [N, F]."""
    elem, power = feature_map(p)
    du = np.zeros_like(u)
    for f in range(elem.size):
        du[:, elem[f]] += power[f] * u[:, elem[f]] ** (power[f] - 1) * dphi[:, f]
    dpre = du / (1.0 + np.exp(-pre))
    return dpre.T @ x, dpre.sum(axis=0)


def distill_phi_grads(p: Params, q, k, v, wq, wk, bq=None, bk=None):
    """Brute force: explicit masks and the N x N matrix dL/dkappa.  Returns dict with
    loss [B,H], dwq, dwk [H,Dphi,D], dbq, dbk [H,Dphi] of the summed loss."""
    q, k, v, wq, wk = map(_f64, (q, k, v, wq, wk))
    bq = None if bq is None else np.asarray(bq, dtype=np.float64)
    bk = None if bk is None else np.asarray(bk, dtype=np.float64)
    soft, lin = numpy_masks(p)
    t = full_softmax(p, q, k, v)
    res = dict(loss=np.zeros((p.B, p.H)), dwq=np.zeros(wq.shape), dwk=np.zeros(wk.shape),
               dbq=np.zeros(wq.shape[:2]), dbk=np.zeros(wk.shape[:2]))
    for b in range(p.B):
        for h in range(p.H):
            prq, uq, fq = _phi_parts(p, q[b, h], wq[h], None if bq is None else bq[h])
            prk, uk, fk = _phi_parts(p, k[b, h], wk[h], None if bk is None else bk[h])
            s = q[b, h] @ k[b, h].T / np.sqrt(p.D)
            smax = np.where(soft, s, -np.inf).max(axis=1, keepdims=True)
            shift = np.maximum(np.where(np.isfinite(smax), smax, 0.0), 0.0)
            kap = fq @ fk.T
            wgt = np.where(soft, np.exp(s - shift), 0.0) + np.where(lin, kap * np.exp(-shift), 0.0)
            den = wgt.sum(axis=1, keepdims=True)             # true denominator times e^-shift
            o = (wgt @ v[b, h]) / den
            g = 2.0 * (o - t[b, h])
            res["loss"][b, h] = ((o - t[b, h]) ** 2).sum()
            scale = np.exp(-shift) / den                      # 1 / true denominator
            a = g * scale
            hv = (g * o).sum(axis=1, keepdims=True) * scale
            dkap = np.where(lin, a @ v[b, h].T - hv, 0.0)
            dwq, dbq = _phi_backward(p, prq, uq, q[b, h], dkap @ fk)
            dwk, dbk = _phi_backward(p, prk, uk, k[b, h], dkap.T @ fq)
            res["dwq"][h] += dwq
            res["dbq"][h] += dbq
            res["dwk"][h] += dwk
            res["dbk"][h] += dbk
    return res


def distill_phi_grads_chunked(p: Params, q, k, v, wq, wk, bq=None, bk=None, heads=None):
    """The same gradients through the recurrent states (blog 2.3): per chunk c the state
    S_c = sum phi_k(k_j) v_j^T and Z_c = sum phi_k(k_j) over the frames [0, ls(c)), so
    dL/dphi_q(q_i) = S_c a_i - h_i Z_c; per chunk R_c = sum_i phi_q(q_i) a_i^T and
    r_c = sum_i phi_q(q_i) h_i over its queries, and key frame f receives the sum of R_c,
    r_c over the chunks whose linear region holds it, dL/dphi_k(k_j) = R v_j - r.  The
    outputs come from the chunk-parallel oracle (with its per-part outputs, so the
    denominator is exp(lse) + z), the teacher from full_softmax.  Memory O(N F) per slab,
    so whole Wan-sized slabs fit.  heads: restrict to these heads (others left zero)."""
    q, k, v, wq, wk = map(_f64, (q, k, v, wq, wk))
    bq = None if bq is None else np.asarray(bq, dtype=np.float64)
    bk = None if bk is None else np.asarray(bk, dtype=np.float64)
    sch = schedule(p)
    n = p.n
    res = dict(loss=np.zeros((p.B, p.H)), dwq=np.zeros(wq.shape), dwk=np.zeros(wk.shape),
               dbq=np.zeros(wq.shape[:2]), dbk=np.zeros(wk.shape[:2]))
    p1 = replace(p, B=1, H=1)
    for b in range(p.B):
        for h in (range(p.H) if heads is None else heads):
            sl = lambda a: a[b:b + 1, h:h + 1]
            o, ax = parallel_rows(p1, sl(q), sl(k), sl(v), wq[h:h + 1], wk[h:h + 1], np.arange(p.N),
                                  None if bq is None else bq[h:h + 1], None if bk is None else bk[h:h + 1])
            t = np.empty_like(o)
            for r0 in range(0, p.N, 4096):
                rows = np.arange(r0, min(r0 + 4096, p.N))
                t[rows] = full_softmax(p1, sl(q), sl(k), sl(v), rows=rows)[0, 0]
            den = np.exp(ax["lse"]) + ax["z"]
            g = 2.0 * (o - t)
            res["loss"][b, h] = ((o - t) ** 2).sum()
            a = g / den[:, None]
            hv = (g * o).sum(axis=1) / den
            prq, uq, fq = _phi_parts(p, q[b, h], wq[h], None if bq is None else bq[h])
            prk, uk, fk = _phi_parts(p, k[b, h], wk[h], None if bk is None else bk[h])
            dfq = np.zeros_like(fq)
            dfk = np.zeros_like(fk)
            R = np.zeros((fq.shape[1], p.D))
            r = np.zeros(fq.shape[1])
            # chunks from the last: R, r accumulate the chunks whose region reaches further
            for c in range(len(sch) - 1, -1, -1):
                f0, f1, ws, we, ls = sch[c]
                lo, hi = f0 * n, f1 * n
                if ls > 0:
                    keys = slice(0, ls * n)
                    S = fk[keys].T @ v[b, h][keys]
                    Z = fk[keys].sum(axis=0)
                    dfq[lo:hi] = a[lo:hi] @ S.T - hv[lo:hi, None] * Z[None, :]
                R += fq[lo:hi].T @ a[lo:hi]
                r += fq[lo:hi].T @ hv[lo:hi]
                # key frames whose earliest linear reader is chunk c: [ls(c-1), ls(c))
                lprev = sch[c - 1][4] if c > 0 else 0
                ks = slice(lprev * n, ls * n)
                dfk[ks] = v[b, h][ks] @ R.T - r[None, :]
            dwq, dbq = _phi_backward(p, prq, uq, q[b, h], dfq)
            dwk, dbk = _phi_backward(p, prk, uk, k[b, h], dfk)
            res["dwq"][h] += dwq
            res["dbq"][h] += dbq
            res["dwk"][h] += dwk
            res["dbk"][h] += dbk
    return res


# ---------------------------------------------------------------------------------------
# Backward of the hybrid attention for an upstream gradient G = dL/do (blog 2.2.1-2.3 with
# the chain rule): for a weight w_ij of key j in query i (exp(s_ij) in the softmax region,
# kappa_ij in the linear region), dL/dw_ij = a_i . v_j - h_i with a_i = G_i / den_i and
# h_i = (G_i . o_i) / den_i, and dL/dv_j = sum_i (w_ij / den_i) G_i.  Softmax weights give
# dL/ds_ij = exp(s_ij) (a_i . v_j - h_i) on the scaled score s_ij = q_i . k_j / sqrt(D), so
# dq_i += sum_j dL/ds_ij k_j / sqrt(D) and dk_j += sum_i dL/ds_ij q_i / sqrt(D); linear
# weights reach q and k through phi: dq += W_q^T dpre_q, dk += W_k^T dpre_k.
# ---------------------------------------------------------------------------------------

def backward(p: Params, q, k, v, wq, wk, dout, bq=None, bk=None):
    """Brute force with explicit masks.  Returns dict dq, dk, dv [B,H,N,D], dwq, dwk
    [H,Dphi,D], dbq, dbk [H,Dphi]."""
    q, k, v, wq, wk, G = map(_f64, (q, k, v, wq, wk, dout))
    bq = None if bq is None else np.asarray(bq, dtype=np.float64)
    bk = None if bk is None else np.asarray(bk, dtype=np.float64)
    soft, lin = numpy_masks(p)
    res = dict(dq=np.zeros(q.shape), dk=np.zeros(k.shape), dv=np.zeros(v.shape), dwq=np.zeros(wq.shape),
               dwk=np.zeros(wk.shape), dbq=np.zeros(wq.shape[:2]), dbk=np.zeros(wk.shape[:2]))
    rs = 1.0 / np.sqrt(p.D)
    for b in range(p.B):
        for h in range(p.H):
            prq, uq, fq = _phi_parts(p, q[b, h], wq[h], None if bq is None else bq[h])
            prk, uk, fk = _phi_parts(p, k[b, h], wk[h], None if bk is None else bk[h])
            s = q[b, h] @ k[b, h].T * rs
            smax = np.where(soft, s, -np.inf).max(axis=1, keepdims=True)
            shift = np.maximum(np.where(np.isfinite(smax), smax, 0.0), 0.0)
            ws_ = np.where(soft, np.exp(s - shift), 0.0)
            wl = np.where(lin, (fq @ fk.T) * np.exp(-shift), 0.0)
            den = (ws_ + wl).sum(axis=1, keepdims=True)
            o = ((ws_ + wl) @ v[b, h]) / den
            g = G[b, h]
            a = g / den                                       # G_i / den_i (shifted units)
            hv = (g * o).sum(axis=1, keepdims=True) / den
            dw = a @ v[b, h].T - hv                           # dL/dw_ij in shifted units
            ds = ws_ * dw                                     # dL/ds_ij
            res["dq"][b, h] += ds @ k[b, h] * rs
            res["dk"][b, h] += ds.T @ q[b, h] * rs
            res["dv"][b, h] += (ws_ + wl).T @ a
            dkap = np.where(lin, dw * np.exp(-shift), 0.0)
            dwq, dbq, dxq = _phi_backward_x(p, prq, uq, q[b, h], wq[h], dkap @ fk)
            dwk, dbk, dxk = _phi_backward_x(p, prk, uk, k[b, h], wk[h], dkap.T @ fq)
            res["dq"][b, h] += dxq
            res["dk"][b, h] += dxk
            res["dwq"][h] += dwq
            res["dbq"][h] += dbq
            res["dwk"][h] += dwk
            res["dbk"][h] += dbk
    return res


def _phi_backward_x(p, pre, u, x, w, dphi):
    """dL/dW, dL/db and dL/dx of one slab from dL/dphi (pre = x W^T + b)."""
    elem, power = feature_map(p)
    du = np.zeros_like(u)
    for f in range(elem.size):
        du[:, elem[f]] += power[f] * u[:, elem[f]] ** (power[f] - 1) * dphi[:, f]
    dpre = du / (1.0 + np.exp(-pre))
    return dpre.T @ x, dpre.sum(axis=0), dpre @ w


def backward_chunked(p: Params, q, k, v, wq, wk, dout, bq=None, bk=None, heads=None):
    """The backward through the chunk structure (blog 2.2.1-2.3): the outputs and their
    per-part outputs from the chunk-parallel oracle (den = exp(lse) + z); the softmax branch
    one chunk window at a time (scores of the chunk's queries against the window's keys);
    the linear branch through the chunk states S_c, Z_c for the queries and the reverse sums
    of R_c, r_c over chunks for the keys, dv_j += R^T phi_k(k_j).  Memory O(N F + Lq Lk) per
    slab, so whole Wan-sized slabs fit.  heads: restrict to these heads (others zero)."""
    q, k, v, wq, wk, G = map(_f64, (q, k, v, wq, wk, dout))
    bq = None if bq is None else np.asarray(bq, dtype=np.float64)
    bk = None if bk is None else np.asarray(bk, dtype=np.float64)
    sch = schedule(p)
    n = p.n
    rs = 1.0 / np.sqrt(p.D)
    res = dict(dq=np.zeros(q.shape), dk=np.zeros(k.shape), dv=np.zeros(v.shape), dwq=np.zeros(wq.shape),
               dwk=np.zeros(wk.shape), dbq=np.zeros(wq.shape[:2]), dbk=np.zeros(wk.shape[:2]))
    p1 = replace(p, B=1, H=1)
    for b in range(p.B):
        for h in (range(p.H) if heads is None else heads):
            sl = lambda a: a[b:b + 1, h:h + 1]
            o, ax = parallel_rows(p1, sl(q), sl(k), sl(v), wq[h:h + 1], wk[h:h + 1], np.arange(p.N),
                                  None if bq is None else bq[h:h + 1], None if bk is None else bk[h:h + 1])
            den = np.exp(ax["lse"]) + ax["z"]
            qq, kk, vv, g = q[b, h], k[b, h], v[b, h], G[b, h]
            a = g / den[:, None]
            delta = (g * o).sum(axis=1)
            hv = delta / den
            # softmax branch per chunk window
            for f0, f1, ws, we, ls in sch:
                if we <= ws:
                    continue
                qs, ks = slice(f0 * n, f1 * n), slice(ws * n, we * n)
                pr = np.exp(qq[qs] @ kk[ks].T * rs - np.log(den[qs])[:, None])   # w_ij / den_i
                res["dv"][b, h][ks] += pr.T @ g[qs]
                ds = pr * (g[qs] @ vv[ks].T - delta[qs][:, None]) * rs
                res["dq"][b, h][qs] += ds @ kk[ks]
                res["dk"][b, h][ks] += ds.T @ qq[qs]
            # linear branch
            prq, uq, fq = _phi_parts(p, qq, wq[h], None if bq is None else bq[h])
            prk, uk, fk = _phi_parts(p, kk, wk[h], None if bk is None else bk[h])
            dfq = np.zeros_like(fq)
            dfk = np.zeros_like(fk)
            R = np.zeros((fq.shape[1], p.D))
            r = np.zeros(fq.shape[1])
            for c in range(len(sch) - 1, -1, -1):
                f0, f1, ws, we, ls = sch[c]
                lo, hi = f0 * n, f1 * n
                if ls > 0:
                    keys = slice(0, ls * n)
                    S = fk[keys].T @ vv[keys]
                    Z = fk[keys].sum(axis=0)
                    dfq[lo:hi] = a[lo:hi] @ S.T - hv[lo:hi, None] * Z[None, :]
                R += fq[lo:hi].T @ a[lo:hi]
                r += fq[lo:hi].T @ hv[lo:hi]
                lprev = sch[c - 1][4] if c > 0 else 0
                ks = slice(lprev * n, ls * n)
                dfk[ks] = vv[ks] @ R.T - r[None, :]
                res["dv"][b, h][ks] += fk[ks] @ R
            dwq, dbq, dxq = _phi_backward_x(p, prq, uq, qq, wq[h], dfq)
            dwk, dbk, dxk = _phi_backward_x(p, prk, uk, kk, wk[h], dfk)
            res["dq"][b, h] += dxq
            res["dk"][b, h] += dxk
            res["dwq"][h] += dwq
            res["dbq"][h] += dbq
            res["dwk"][h] += dwk
            res["dbk"][h] += dbk
    return res
