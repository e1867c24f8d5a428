"""rehyat_forward_parallel_noalloc, the allocation-free variant of rehyat_forward_parallel (its
workspace is the library's static scratch area), called through the C ABI and compared with
rehyat_forward_parallel on the same inputs: bit for bit, since both run the same kernels on
the same inputs, over three calls in a row whose shapes shrink (the area keeps the previous
call's contents), plus the fp64 oracle bar on each, and the size limit."""
import ctypes

import numpy as np
import pytest
import torch

import hybrid_softmax_linear_chunked_amd as rh
import oracle
from gpu_common import TOL, oracle_params, rand_inputs, slab_err, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # bf16 with several chunks (chunk-0 window of 15 key tiles)
    rh.Params(1, 3, 128, 7, 300, 3, 1, 128, 2, 0, rh.BF16, rh.BF16),
    # smaller: fewer heads and frames, other head dim and feature map, biases
    rh.Params(1, 2, 64, 4, 100, 3, 1, 64, 3, 0, rh.BF16, rh.FP32),
    # smaller still, fp32 inputs
    rh.Params(1, 1, 32, 5, 48, 2, 1, 32, 2, 0, rh.FP32, rh.FP32),
]


def _noalloc(p, d, out):
    c = p.c()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)
    st = rh.lib().rehyat_forward_parallel_noalloc(ctypes.byref(c), ptr(d["q"]), ptr(d["k"]), ptr(d["v"]),
                                                  ptr(d["wq"]), ptr(d["wk"]), ptr(d["bq"]), ptr(d["bk"]), ptr(out),
                                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_equals_forward_parallel_on_shrinking_calls():
    for i, p in enumerate(CASES):
        x = rand_inputs(p, seed=20 + i, bias=(i == 1))
        d = to_dev(x, p)
        ref = rh.forward_parallel(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], d["bq"], d["bk"])
        out = torch.full_like(ref, float("nan"))
        assert _noalloc(p, d, out) == 0
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"case {i}: differs from rehyat_forward_parallel"
        orc = oracle.parallel(oracle_params(p), x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"])
        assert slab_err(out.float().cpu().numpy(), orc) <= TOL[p.in_dtype]


def test_noalloc_rejects_workspace_above_the_scratch_area():
    # the 14B-shaped layer (40 heads, 75,600 tokens, P = 3) needs about 138 MB of workspace
    p = rh.Params(1, 40, 128, 21, 3600, 3, 1, 128, 3, 0, rh.BF16, rh.BF16)
    assert rh.lib().rehyat_workspace_bytes(ctypes.byref(p.c())) > 64 << 20
    dummy = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    c = p.c()
    vp = ctypes.c_void_p(dummy.data_ptr())
    st = rh.lib().rehyat_forward_parallel_noalloc(ctypes.byref(c), vp, vp, vp, vp, vp, None, None, vp,
                                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rh._STATUS[st] == "REHYAT_ESCRATCH"
    assert b"static scratch" in rh.lib().rehyat_status_string(st)
