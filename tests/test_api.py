"""Host-side checks of the C ABI (no GPU needed): the library loads and exports every
entry point include/rehyat.h declares, sizes follow the documented layouts, and every
invalid call is rejected with its status code before any HIP call is made."""
import ctypes
import os
import re
import subprocess

import pytest

import hybrid_softmax_linear_chunked_amd as rh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rehyat.h")

OK, EINVAL, ESHAPE, EALIGN, EWORKSPACE, ESTATE, EHIP = range(7)
WAN = rh.Params(1, 12, 128, 21, 1560, 3, 1, 128, 2, 0, rh.BF16, rh.BF16)
FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10004)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rh.LIB_PATH):
        from hybrid_softmax_linear_chunked_amd.build import build
        build()
    return rh.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(rehyat_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(rh.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", rh.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (rehyat_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def test_status_strings(L):
    for s in range(7):
        assert rh.status_string(s)
    assert rh.status_string(0) == "ok"


def test_sizes_follow_layouts(L):
    a = lambda x: (x + 255) // 256 * 256
    F = WAN.P * WAN.Dphi
    assert rh.features(WAN) == 256
    # chunk-parallel: per-frame partials for the 17 frames that enter some chunk's state,
    # then one state image (S in the input dtype, operand order, Z in float) per chunk,
    # followed by the attention stage's tail-split scratch (bf16 inputs): per XCD (8
    # contiguous shares of the 12 * 19 chunk-0 query tiles of 256 queries) the last 8 tiles
    # are split, each with an arrival counter and two halves x 8 waves x 64 lanes x
    # (4 * 16 O values + reference + row sum) floats
    ns = 12 * 19
    splits = sum(min(ns * (x + 1) // 8 - ns * x // 8, 8) for x in range(8))
    assert splits == 64
    split_bytes = a(splits * 4) + splits * 2 * 8 * 64 * (4 * 16 + 2) * 4
    assert rh.workspace_bytes(WAN) == (a(12 * 17 * F * 128 * 4) + a(12 * 17 * F * 4)
                                       + a(12 * 7 * F * 128 * 2) + a(12 * 7 * F * 4) + split_bytes)
    # fp32 inputs run the other tile kernel, which does not split
    assert rh.workspace_bytes(WAN.with_(in_dtype=0)) == (a(12 * 17 * F * 128 * 4) + a(12 * 17 * F * 4)
                                                         + a(12 * 7 * F * 128 * 4) + a(12 * 7 * F * 4))
    # streaming: S, Z, the image of the current state and two overlap buffers of K and V
    # with To frames and 64 spare rows, independent of T
    ov = 12 * (1 * 1560 + 64) * 128 * 2
    assert rh.state_bytes(WAN) == (a(12 * F * 128 * 4) + a(12 * F * 4) + a(12 * F * 128 * 2)
                                   + a(12 * F * 4) + 4 * a(ov))
    assert rh.state_bytes(WAN.with_(T=81)) == rh.state_bytes(WAN)
    # the step's workspace: partials of up to Tc frames, then the first chunk's split
    # scratch (the same tiles as the chunk-parallel grid splits)
    assert rh.stream_workspace_bytes(WAN) == a(12 * 3 * F * 128 * 4) + a(12 * 3 * F * 4) + split_bytes
    assert rh.stream_workspace_bytes(WAN.with_(in_dtype=0)) == a(12 * 3 * F * 128 * 4) + a(12 * 3 * F * 4)
    # one chunk covering the clip has no linear region; bf16 inputs need only the split
    # scratch (12 * 128 tiles, 8 split per XCD), fp32 inputs nothing
    assert rh.workspace_bytes(WAN.with_(Tc=21)) == a(64 * 4) + 64 * 2 * 8 * 64 * (4 * 16 + 2) * 4
    assert rh.workspace_bytes(WAN.with_(Tc=21, in_dtype=0)) == 0
    # a clip shorter than one chunk splits the tiles of its T frames (2 frames: 12 * 13 tiles,
    # still 8 per XCD); a window under four tiles splits nothing
    assert rh.workspace_bytes(WAN.with_(T=2)) == a(64 * 4) + 64 * 2 * 8 * 64 * (4 * 16 + 2) * 4
    assert rh.workspace_bytes(WAN.with_(n=50, Tc=3, T=3)) == 0


@pytest.mark.parametrize("change,status", [
    (dict(D=48), ESHAPE), (dict(D=256), ESHAPE), (dict(Dphi=48), ESHAPE), (dict(Dphi=160), ESHAPE),
    (dict(P=0), ESHAPE), (dict(P=5), ESHAPE), (dict(Tc=0), EINVAL), (dict(To=-1), EINVAL),
    (dict(T=0), EINVAL), (dict(n=0), EINVAL), (dict(B=0), EINVAL), (dict(linear_only=2), EINVAL),
    (dict(in_dtype=7), EINVAL), (dict(out_dtype=-1), EINVAL),
])
def test_invalid_params_rejected(L, change, status):
    p = WAN.with_(**change).c()
    f = L.rehyat_forward_parallel
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 1 << 40, None) == status
    assert L.rehyat_workspace_bytes(ctypes.byref(p)) == 0
    # features and state sizes do not depend on the clip length T
    t_only = list(change) == ["T"]
    assert L.rehyat_features(ctypes.byref(p)) == (256 if t_only else -1)


def test_pointer_checks(L):
    p = WAN.c()
    f = L.rehyat_forward_parallel
    args = [FAKE] * 5
    for i in range(5):
        bad = list(args)
        bad[i] = None
        assert f(ctypes.byref(p), *bad, None, None, FAKE, FAKE, 1 << 40, None) == EALIGN
        bad[i] = MISALIGNED
        assert f(ctypes.byref(p), *bad, None, None, FAKE, FAKE, 1 << 40, None) == EALIGN
    assert f(ctypes.byref(p), *args, None, None, None, FAKE, 1 << 40, None) == EALIGN
    assert f(ctypes.byref(p), *args, ctypes.c_void_p(0x10002), None, FAKE, FAKE, 1 << 40, None) == EALIGN
    assert L.rehyat_phi(ctypes.byref(p), None, FAKE, None, FAKE, None) == EALIGN


def test_workspace_checks(L):
    p = WAN.c()
    need = L.rehyat_workspace_bytes(ctypes.byref(p))
    f = L.rehyat_forward_parallel
    assert f(ctypes.byref(p), *[FAKE] * 5, None, None, FAKE, FAKE, need - 1, None) == EWORKSPACE
    assert f(ctypes.byref(p), *[FAKE] * 5, None, None, FAKE, None, need, None) == EWORKSPACE
    assert f(ctypes.byref(p), *[FAKE] * 5, None, None, FAKE, ctypes.c_void_p(0x10010), need, None) == EWORKSPACE


def test_stream_contract(L):
    p = WAN.c()
    st = rh._CStream()
    step = L.rehyat_chunk_step
    ws = L.rehyat_stream_workspace_bytes(ctypes.byref(p))
    call = lambda handle, frames: step(ctypes.byref(p), FAKE, ctypes.byref(handle), FAKE, FAKE, FAKE, frames,
                                       FAKE, FAKE, None, None, FAKE, FAKE, ws, None)
    assert call(st, 3) == ESTATE                    # never initialised
    st.magic = 0x52485954
    assert call(st, 4) == ESTATE                    # more than Tc frames
    assert call(st, 0) == ESTATE
    st.closed = 1
    assert call(st, 2) == ESTATE                    # after a short final chunk
    st.closed = 0
    assert step(ctypes.byref(p), FAKE, ctypes.byref(st), FAKE, FAKE, FAKE, 3, FAKE, FAKE, None, None, FAKE,
                FAKE, ws - 1, None) == EWORKSPACE
    assert step(ctypes.byref(p), ctypes.c_void_p(0x10010), ctypes.byref(st), FAKE, FAKE, FAKE, 3, FAKE, FAKE,
                None, None, FAKE, FAKE, ws, None) == EALIGN
    assert L.rehyat_state_init(ctypes.byref(p), FAKE, None, None) == ESTATE
    assert L.rehyat_state_init(ctypes.byref(p), ctypes.c_void_p(0x10010), ctypes.byref(st), None) == EALIGN


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(rh, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(rh, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        rh.lib()


def test_distill_sizes_and_checks(L):
    """Distillation workspace: student and teacher outputs (float32), per-segment partial
    sums (16,384 floats per segment), then the larger of the two forwards' workspaces."""
    a = lambda x: (x + 255) // 256 * 256
    p = WAN.c()
    out = a(12 * 32760 * 128 * 4)
    nseg = -(-32760 * 128 // 16384)
    student = rh.workspace_bytes(WAN.with_(out_dtype=rh.FP32))
    teacher = rh.workspace_bytes(WAN.with_(Tc=21, To=0, out_dtype=rh.FP32))
    need = L.rehyat_distill_workspace_bytes(ctypes.byref(p))
    assert need == 2 * out + a(12 * nseg * 4) + max(student, teacher)
    f = L.rehyat_distill_loss
    assert f(ctypes.byref(p), *[FAKE] * 5, None, None, FAKE, FAKE, need - 1, None) == EWORKSPACE
    assert f(ctypes.byref(p), *[FAKE] * 5, None, None, FAKE, ctypes.c_void_p(0x10010), need, None) == EWORKSPACE
    assert f(ctypes.byref(p), *[FAKE] * 5, None, None, None, FAKE, need, None) == EALIGN
    assert f(ctypes.byref(p), *[FAKE] * 5, None, None, ctypes.c_void_p(0x10002), FAKE, need, None) == EALIGN
    assert f(ctypes.byref(p), FAKE, MISALIGNED, *[FAKE] * 3, None, None, FAKE, FAKE, need, None) == EALIGN
    # the teacher's one window must stay within 2^28 tokens
    big = WAN.with_(T=2 ** 28 // 1560 + 1, Tc=3).c()
    assert L.rehyat_distill_workspace_bytes(ctypes.byref(big)) == 0
    assert f(ctypes.byref(big), *[FAKE] * 5, None, None, FAKE, FAKE, 1 << 50, None) == EINVAL
    bad = WAN.with_(D=48).c()
    assert f(ctypes.byref(bad), *[FAKE] * 5, None, None, FAKE, FAKE, 1 << 40, None) == ESHAPE


def test_distill_grad_checks(L):
    p = WAN.c()
    need = L.rehyat_distill_grad_workspace_bytes(ctypes.byref(p))
    assert need > L.rehyat_distill_workspace_bytes(ctypes.byref(p))
    # bf16 inputs with P = 2 fuse the feature map's backward into the feature gradients, so
    # the float [B*H, N, F] dphi buffer (403 MB here) is not part of the workspace; fp32
    # inputs keep it (the two layouts otherwise differ by tens of MB: image dtypes, the
    # bf16 attention's tail-split scratch)
    dphi = 12 * 32760 * 256 * 4
    need32 = L.rehyat_distill_grad_workspace_bytes(ctypes.byref(WAN.with_(in_dtype=0).c()))
    assert need32 - need > dphi // 2
    f = L.rehyat_distill_grad
    outs = [FAKE, FAKE, FAKE, None, None]            # loss, dwq, dwk, dbq, dbk
    assert f(ctypes.byref(p), *[FAKE] * 5, None, None, *outs, FAKE, need - 1, None) == EWORKSPACE
    assert f(ctypes.byref(p), *[FAKE] * 5, None, None, *outs, ctypes.c_void_p(0x10010), need, None) == EWORKSPACE
    for i in range(3):
        bad = list(outs)
        bad[i] = None
        assert f(ctypes.byref(p), *[FAKE] * 5, None, None, *bad, FAKE, need, None) == EALIGN
    assert f(ctypes.byref(p), *[FAKE] * 5, None, None, FAKE, FAKE, FAKE, ctypes.c_void_p(0x10002), None, FAKE,
             need, None) == EALIGN
    big = WAN.with_(T=2 ** 28 // 1560 + 1).c()
    assert L.rehyat_distill_grad_workspace_bytes(ctypes.byref(big)) == 0
    assert f(ctypes.byref(big), *[FAKE] * 5, None, None, *outs, FAKE, 1 << 50, None) == EINVAL


def test_backward_checks(L):
    p = WAN.c()
    need = L.rehyat_backward_workspace_bytes(ctypes.byref(p))
    # bf16: no score-sized buffer (the softmax branch recomputes P and dS tile by tile), so a
    # longer chunk window leaves the workspace nearly unchanged; float32 inputs keep two
    # chunk-window buffers (4,680 queries x 6,240 keys per slab)
    window = 2 * 12 * 4680 * 6240 * 4
    need7 = L.rehyat_backward_workspace_bytes(ctypes.byref(WAN.with_(Tc=7).c()))
    assert need < window and abs(need7 - need) < need // 10
    assert L.rehyat_backward_workspace_bytes(ctypes.byref(WAN.with_(in_dtype=0).c())) > window
    f = L.rehyat_backward
    ins = [FAKE] * 5 + [None, None, FAKE]             # q, k, v, wq, wk, bq, bk, dout
    outs = [FAKE] * 5 + [None, None]                 # dq, dk, dv, dwq, dwk, dbq, dbk
    assert f(ctypes.byref(p), *ins, *outs, FAKE, need - 1, None) == EWORKSPACE
    assert f(ctypes.byref(p), *ins, *outs, ctypes.c_void_p(0x10010), need, None) == EWORKSPACE
    for i in range(5):
        bad = list(outs)
        bad[i] = None
        assert f(ctypes.byref(p), *ins, *bad, FAKE, need, None) == EALIGN
    bad = list(ins)
    bad[7] = MISALIGNED
    assert f(ctypes.byref(p), *bad, *outs, FAKE, need, None) == EALIGN
    assert L.rehyat_backward_workspace_bytes(ctypes.byref(WAN.with_(D=48).c())) == 0
