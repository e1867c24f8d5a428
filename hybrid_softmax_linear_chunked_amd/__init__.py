"""Python binding of librehyat.so, the gfx950 library for ReHyAt chunk-wise recurrent
hybrid attention (ReHyAt blog, maplevalley.com.cn, sections 2.2-2.3 and 5.2).

Argument marshalling only: every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  The functions
mirror the C ABI in include/rehyat.h and raise RehyatError on a non-OK status.  Importing
the package does not need a GPU; calling into the library needs the built librehyat.so
(``python -m hybrid_softmax_linear_chunked_amd.build``) and raises if it is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, replace
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librehyat.so")
# the host-sanitized build of the same sources (build_sanitized), for the sanitizer test
if os.environ.get("REHYAT_LIB"):
    LIB_PATH = os.environ["REHYAT_LIB"]

FP32, BF16 = 0, 1
_STATUS = {0: "REHYAT_OK", 1: "REHYAT_EINVAL", 2: "REHYAT_ESHAPE", 3: "REHYAT_EALIGN",
           4: "REHYAT_EWORKSPACE", 5: "REHYAT_ESTATE", 6: "REHYAT_EHIP", 7: "REHYAT_ESCRATCH"}

EXPORTS = (
    "rehyat_status_string", "rehyat_features", "rehyat_phi", "rehyat_workspace_bytes",
    "rehyat_forward_parallel", "rehyat_forward_parallel_aux", "rehyat_forward_parallel_noalloc",
    "rehyat_state_bytes",
    "rehyat_stream_workspace_bytes", "rehyat_state_init", "rehyat_chunk_step",
    "rehyat_parallel_states", "rehyat_parallel_attend", "rehyat_distill_workspace_bytes",
    "rehyat_distill_loss", "rehyat_distill_grad_workspace_bytes", "rehyat_distill_grad",
    "rehyat_backward_workspace_bytes", "rehyat_backward",
)


class RehyatError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({status_string(status)})")


class _CParams(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in
                ("B", "H", "D", "T", "frame_tokens", "Tc", "To", "Dphi", "P", "linear_only",
                 "in_dtype", "out_dtype")]


class _CStream(ctypes.Structure):
    _fields_ = [("frames_seen", ctypes.c_int64), ("frames_absorbed", ctypes.c_int64),
                ("closed", ctypes.c_int32), ("overlap_slot", ctypes.c_int32),
                ("magic", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _CAux(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in ("o_soft", "lse", "y", "z")]


_lib = None


def lib():
    """Load librehyat.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m hybrid_softmax_linear_chunked_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, P = ctypes.c_void_p, ctypes.POINTER(_CParams)
        L.rehyat_status_string.argtypes = [ctypes.c_int]
        L.rehyat_status_string.restype = ctypes.c_char_p
        L.rehyat_features.argtypes = [P]
        L.rehyat_features.restype = ctypes.c_int32
        L.rehyat_phi.argtypes = [P, vp, vp, vp, vp, vp]
        L.rehyat_phi.restype = ctypes.c_int
        for name in ("rehyat_workspace_bytes", "rehyat_state_bytes", "rehyat_stream_workspace_bytes"):
            getattr(L, name).argtypes = [P]
            getattr(L, name).restype = ctypes.c_size_t
        L.rehyat_forward_parallel.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.rehyat_forward_parallel.restype = ctypes.c_int
        L.rehyat_forward_parallel_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.rehyat_forward_parallel_noalloc.restype = ctypes.c_int
        L.rehyat_forward_parallel_aux.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp,
                                                  ctypes.POINTER(_CAux), vp, ctypes.c_size_t, vp]
        L.rehyat_forward_parallel_aux.restype = ctypes.c_int
        L.rehyat_parallel_states.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.rehyat_parallel_states.restype = ctypes.c_int
        L.rehyat_parallel_attend.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.POINTER(_CAux), vp,
                                             ctypes.c_size_t, vp]
        L.rehyat_parallel_attend.restype = ctypes.c_int
        L.rehyat_state_init.argtypes = [P, vp, ctypes.POINTER(_CStream), vp]
        L.rehyat_state_init.restype = ctypes.c_int
        L.rehyat_chunk_step.argtypes = [P, vp, ctypes.POINTER(_CStream), vp, vp, vp, ctypes.c_int32,
                                        vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.rehyat_chunk_step.restype = ctypes.c_int
        L.rehyat_distill_workspace_bytes.argtypes = [P]
        L.rehyat_distill_workspace_bytes.restype = ctypes.c_size_t
        L.rehyat_distill_loss.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.rehyat_distill_loss.restype = ctypes.c_int
        L.rehyat_distill_grad_workspace_bytes.argtypes = [P]
        L.rehyat_distill_grad_workspace_bytes.restype = ctypes.c_size_t
        L.rehyat_distill_grad.argtypes = [P] + [vp] * 13 + [ctypes.c_size_t, vp]
        L.rehyat_distill_grad.restype = ctypes.c_int
        L.rehyat_backward_workspace_bytes.argtypes = [P]
        L.rehyat_backward_workspace_bytes.restype = ctypes.c_size_t
        L.rehyat_backward.argtypes = [P] + [vp] * 16 + [ctypes.c_size_t, vp]
        L.rehyat_backward.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().rehyat_status_string(status).decode()


@dataclass(frozen=True)
class Params:
    B: int
    H: int
    D: int
    T: int
    n: int            # tokens per latent frame
    Tc: int
    To: int
    Dphi: int
    P: int
    linear_only: int = 0
    in_dtype: int = BF16
    out_dtype: int = BF16

    @property
    def N(self) -> int:
        return self.T * self.n

    @property
    def F(self) -> int:
        return self.P * self.Dphi

    def with_(self, **kw) -> "Params":
        return replace(self, **kw)

    def c(self) -> _CParams:
        return _CParams(self.B, self.H, self.D, self.T, self.n, self.Tc, self.To, self.Dphi, self.P,
                        int(self.linear_only), self.in_dtype, self.out_dtype)


def torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == BF16 else torch.float32


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(t: torch.Tensor, shape, dtype, name: str):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def _raise(status: int, where: str):
    if status != 0:
        raise RehyatError(status, where)


def features(p: Params) -> int:
    return lib().rehyat_features(ctypes.byref(p.c()))


def workspace_bytes(p: Params) -> int:
    return lib().rehyat_workspace_bytes(ctypes.byref(p.c()))


def state_bytes(p: Params) -> int:
    return lib().rehyat_state_bytes(ctypes.byref(p.c()))


def stream_workspace_bytes(p: Params) -> int:
    return lib().rehyat_stream_workspace_bytes(ctypes.byref(p.c()))


def alloc_bytes(nbytes: int, device="cuda") -> torch.Tensor:
    """Device byte buffer for workspaces and states (at least 1 byte)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def phi(p: Params, x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None,
        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    dt = torch_dtype(p.in_dtype)
    _check(x, (p.B, p.H, p.N, p.D), dt, "x")
    _check(w, (p.H, p.Dphi, p.D), dt, "w")
    if bias is not None:
        _check(bias, (p.H, p.Dphi), torch.float32, "bias")
    if out is None:
        out = torch.empty((p.B, p.H, p.N, p.F), dtype=dt, device=x.device)
    _check(out, (p.B, p.H, p.N, p.F), dt, "out")
    _raise(lib().rehyat_phi(ctypes.byref(p.c()), _ptr(x), _ptr(w), _ptr(bias), _ptr(out),
                            _stream_handle()), "rehyat_phi")
    return out


def forward_parallel_noalloc(p: Params, q, k, v, wq, wk, bq=None, bk=None, out=None):
    """rehyat_forward_parallel_noalloc: the chunk-parallel forward with the library's static
    scratch area as workspace (64 MiB per GPU; raises REHYAT_ESCRATCH beyond).  Calls on one
    GPU that overlap race on that area."""
    dt = torch_dtype(p.in_dtype)
    shape = (p.B, p.H, p.N, p.D)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, shape, dt, name)
    for name, t in (("wq", wq), ("wk", wk)):
        _check(t, (p.H, p.Dphi, p.D), dt, name)
    for name, t in (("bq", bq), ("bk", bk)):
        if t is not None:
            _check(t, (p.H, p.Dphi), torch.float32, name)
    if out is None:
        out = torch.empty(shape, dtype=torch_dtype(p.out_dtype), device=q.device)
    _check(out, shape, torch_dtype(p.out_dtype), "out")
    c = p.c()
    _raise(lib().rehyat_forward_parallel_noalloc(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk),
                                                 _ptr(bq), _ptr(bk), _ptr(out), _stream_handle()),
           "rehyat_forward_parallel_noalloc")
    return out


def forward_parallel(p: Params, q, k, v, wq, wk, bq=None, bk=None, out=None, ws=None,
                     aux: bool = False):
    """Chunk-parallel hybrid attention over the whole clip.  With aux=True also returns a
    dict of the per-part outputs (o_soft, lse, y, z), all float32."""
    dt = torch_dtype(p.in_dtype)
    shape = (p.B, p.H, p.N, p.D)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, shape, dt, name)
    for name, t in (("wq", wq), ("wk", wk)):
        _check(t, (p.H, p.Dphi, p.D), dt, name)
    for name, t in (("bq", bq), ("bk", bk)):
        if t is not None:
            _check(t, (p.H, p.Dphi), torch.float32, name)
    if out is None:
        out = torch.empty(shape, dtype=torch_dtype(p.out_dtype), device=q.device)
    _check(out, shape, torch_dtype(p.out_dtype), "out")
    need = workspace_bytes(p)
    if ws is None:
        ws = alloc_bytes(need, q.device)
    c = p.c()
    if not aux:
        _raise(lib().rehyat_forward_parallel(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(wq),
                                             _ptr(wk), _ptr(bq), _ptr(bk), _ptr(out), _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream_handle()),
               "rehyat_forward_parallel")
        return out
    ax = dict(o_soft=torch.empty(shape, dtype=torch.float32, device=q.device),
              lse=torch.empty(shape[:-1], dtype=torch.float32, device=q.device),
              y=torch.empty(shape, dtype=torch.float32, device=q.device),
              z=torch.empty(shape[:-1], dtype=torch.float32, device=q.device))
    caux = _CAux(*(ax[key].data_ptr() for key in ("o_soft", "lse", "y", "z")))
    _raise(lib().rehyat_forward_parallel_aux(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(wq),
                                             _ptr(wk), _ptr(bq), _ptr(bk), _ptr(out),
                                             ctypes.byref(caux), _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream_handle()),
           "rehyat_forward_parallel_aux")
    return out, ax


def distill_workspace_bytes(p: Params) -> int:
    return int(lib().rehyat_distill_workspace_bytes(ctypes.byref(p.c())))


def distill_loss(p: Params, q, k, v, wq, wk, bq=None, bk=None, loss=None, ws=None, outputs=False):
    """Per-(batch, head) squared L2 distance between the hybrid output and full softmax
    attention on the same inputs (rehyat_distill_loss).  Returns float32 [B, H]; with
    outputs=True also the float32 student and teacher outputs it left in ws."""
    dt = torch_dtype(p.in_dtype)
    shape = (p.B, p.H, p.N, p.D)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, shape, dt, name)
    for name, t in (("wq", wq), ("wk", wk)):
        _check(t, (p.H, p.Dphi, p.D), dt, name)
    for name, t in (("bq", bq), ("bk", bk)):
        if t is not None:
            _check(t, (p.H, p.Dphi), torch.float32, name)
    if loss is None:
        loss = torch.empty((p.B, p.H), dtype=torch.float32, device=q.device)
    _check(loss, (p.B, p.H), torch.float32, "loss")
    need = distill_workspace_bytes(p)
    if need == 0:
        raise RehyatError(1, "rehyat_distill_workspace_bytes")
    if ws is None:
        ws = alloc_bytes(need, q.device)
    _raise(lib().rehyat_distill_loss(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk),
                                     _ptr(bq), _ptr(bk), _ptr(loss), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream_handle()),
           "rehyat_distill_loss")
    if not outputs:
        return loss
    n = p.B * p.H * p.N * p.D
    off = (n * 4 + 255) // 256 * 256
    flat = ws.view(torch.uint8)
    stu = flat[:n * 4].view(torch.float32).view(shape)
    tea = flat[off:off + n * 4].view(torch.float32).view(shape)
    return loss, stu, tea


def distill_grad_workspace_bytes(p: Params) -> int:
    return int(lib().rehyat_distill_grad_workspace_bytes(ctypes.byref(p.c())))


def distill_grad(p: Params, q, k, v, wq, wk, bq=None, bk=None, ws=None, biases=True):
    """Distillation loss and its gradients with respect to W_q, W_k (and b_q, b_k) through
    rehyat_distill_grad.  Returns a dict of float32 tensors: loss [B,H], dwq, dwk
    [H,Dphi,D], and dbq, dbk [H,Dphi] when biases=True."""
    dt = torch_dtype(p.in_dtype)
    shape = (p.B, p.H, p.N, p.D)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, shape, dt, name)
    for name, t in (("wq", wq), ("wk", wk)):
        _check(t, (p.H, p.Dphi, p.D), dt, name)
    for name, t in (("bq", bq), ("bk", bk)):
        if t is not None:
            _check(t, (p.H, p.Dphi), torch.float32, name)
    dev = q.device
    out = dict(loss=torch.empty((p.B, p.H), dtype=torch.float32, device=dev),
               dwq=torch.empty((p.H, p.Dphi, p.D), dtype=torch.float32, device=dev),
               dwk=torch.empty((p.H, p.Dphi, p.D), dtype=torch.float32, device=dev))
    if biases:
        out["dbq"] = torch.empty((p.H, p.Dphi), dtype=torch.float32, device=dev)
        out["dbk"] = torch.empty((p.H, p.Dphi), dtype=torch.float32, device=dev)
    need = distill_grad_workspace_bytes(p)
    if need == 0:
        raise RehyatError(1, "rehyat_distill_grad_workspace_bytes")
    if ws is None:
        ws = alloc_bytes(need, dev)
    _raise(lib().rehyat_distill_grad(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk),
                                     _ptr(bq), _ptr(bk), _ptr(out["loss"]), _ptr(out["dwq"]), _ptr(out["dwk"]),
                                     _ptr(out.get("dbq")), _ptr(out.get("dbk")), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream_handle()),
           "rehyat_distill_grad")
    return out


def backward_workspace_bytes(p: Params) -> int:
    return int(lib().rehyat_backward_workspace_bytes(ctypes.byref(p.c())))


def backward(p: Params, q, k, v, wq, wk, dout, bq=None, bk=None, ws=None, biases=True):
    """Gradients of the chunk-parallel forward for the upstream gradient dout (float32
    [B,H,N,D]) through rehyat_backward.  Returns a dict of float32 tensors dq, dk, dv
    [B,H,N,D], dwq, dwk [H,Dphi,D], and dbq, dbk [H,Dphi] when biases=True."""
    dt = torch_dtype(p.in_dtype)
    shape = (p.B, p.H, p.N, p.D)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, shape, dt, name)
    _check(dout, shape, torch.float32, "dout")
    for name, t in (("wq", wq), ("wk", wk)):
        _check(t, (p.H, p.Dphi, p.D), dt, name)
    for name, t in (("bq", bq), ("bk", bk)):
        if t is not None:
            _check(t, (p.H, p.Dphi), torch.float32, name)
    dev = q.device
    out = {key: torch.empty(shape, dtype=torch.float32, device=dev) for key in ("dq", "dk", "dv")}
    out["dwq"] = torch.empty((p.H, p.Dphi, p.D), dtype=torch.float32, device=dev)
    out["dwk"] = torch.empty((p.H, p.Dphi, p.D), dtype=torch.float32, device=dev)
    if biases:
        out["dbq"] = torch.empty((p.H, p.Dphi), dtype=torch.float32, device=dev)
        out["dbk"] = torch.empty((p.H, p.Dphi), dtype=torch.float32, device=dev)
    need = backward_workspace_bytes(p)
    if need == 0:
        raise RehyatError(1, "rehyat_backward_workspace_bytes")
    if ws is None:
        ws = alloc_bytes(need, dev)
    _raise(lib().rehyat_backward(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), _ptr(bq),
                                 _ptr(bk), _ptr(dout), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                 _ptr(out["dwq"]), _ptr(out["dwk"]), _ptr(out.get("dbq")), _ptr(out.get("dbk")),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream_handle()),
           "rehyat_backward")
    return out


def parallel_states(p: Params, k, v, wk, bk, ws):
    """First stage of forward_parallel: per-frame state partials and their prefix into ws."""
    _raise(lib().rehyat_parallel_states(ctypes.byref(p.c()), _ptr(k), _ptr(v), _ptr(wk), _ptr(bk),
                                        _ptr(ws), ws.numel() * ws.element_size(), _stream_handle()),
           "rehyat_parallel_states")


def parallel_attend(p: Params, q, k, v, wq, bq, out, ws):
    """Second stage of forward_parallel: windowed softmax with the fused linear part."""
    _raise(lib().rehyat_parallel_attend(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(wq),
                                        _ptr(bq), _ptr(out), None, _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream_handle()),
           "rehyat_parallel_attend")


class Stream:
    """Constant-memory streaming form: one call per chunk of Tc frames (a final call may be
    shorter), with S, Z and the overlap frames carried in a device state buffer."""

    def __init__(self, p: Params, wq, wk, bq=None, bk=None, device="cuda"):
        self.p = p
        self.wq, self.wk, self.bq, self.bk = wq, wk, bq, bk
        self.state = alloc_bytes(state_bytes(p), device)
        self.ws = alloc_bytes(stream_workspace_bytes(p), device)
        self.handle = _CStream()
        self.init()

    def init(self):
        _raise(lib().rehyat_state_init(ctypes.byref(self.p.c()), _ptr(self.state),
                                       ctypes.byref(self.handle), _stream_handle()), "rehyat_state_init")

    def step(self, q, k, v, frames: int, out=None):
        p = self.p
        dt = torch_dtype(p.in_dtype)
        shape = (p.B, p.H, frames * p.n, p.D)
        for name, t in (("q", q), ("k", k), ("v", v)):
            _check(t, shape, dt, name)
        if out is None:
            out = torch.empty(shape, dtype=torch_dtype(p.out_dtype), device=q.device)
        _check(out, shape, torch_dtype(p.out_dtype), "out")
        _raise(lib().rehyat_chunk_step(ctypes.byref(p.c()), _ptr(self.state), ctypes.byref(self.handle),
                                       _ptr(q), _ptr(k), _ptr(v), frames, _ptr(self.wq), _ptr(self.wk),
                                       _ptr(self.bq), _ptr(self.bk), _ptr(out), _ptr(self.ws),
                                       self.ws.numel(), _stream_handle()), "rehyat_chunk_step")
        return out

    # the device state plus the host handle is the whole checkpoint of a stream
    def save(self):
        h = self.handle
        return (self.state.clone(), (h.frames_seen, h.frames_absorbed, h.closed, h.overlap_slot,
                                     h.magic, h.reserved))

    def restore(self, snap):
        state, fields = snap
        self.state.copy_(state)
        self.handle = _CStream(*fields)
