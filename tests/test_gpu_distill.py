"""GPU parity of rehyat_distill_loss (ReHyAt blog, maplevalley.com.cn, 3.1.1: the hybrid
block is distilled towards the frozen softmax teacher's output in L2) against the fp64
oracle, through the C ABI.

Three checks per case:
  * the student and teacher outputs the call leaves in its workspace match the oracle's
    hybrid output and full softmax attention at the output bar (1e-5 fp32, 2e-2 bf16 of
    the slab maximum);
  * the loss equals an fp64 re-summation of those same two outputs to 1e-5 relative (the
    reduction itself: fixed-order fp32 sums);
  * the loss is within what the observed output deviations allow around the oracle's
    loss: with e = max|student - hybrid| + max|teacher - softmax| over the slab and
    d = hybrid - softmax, |loss - sum d^2| <= 2 e sum|d| + N D e^2 (plus the reduction's
    1e-5).
Repeated calls give identical bits.
"""
import numpy as np
import pytest
import torch

import hybrid_softmax_linear_chunked_amd as rh
import oracle
from gpu_common import TOL, oracle_params, rand_inputs, to_dev
from synth_inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

SHAPES = [
    # B, H, D, T, n, Tc, To, Dphi, P, linear_only, dtype
    (1, 2, 32, 7, 16, 3, 1, 32, 2, 0, rh.FP32),
    (2, 3, 64, 5, 37, 2, 1, 64, 2, 0, rh.FP32),
    (1, 2, 128, 6, 50, 3, 1, 128, 2, 0, rh.BF16),
    (1, 3, 128, 9, 45, 2, 2, 128, 3, 0, rh.BF16),
    (2, 2, 64, 8, 29, 3, 0, 64, 1, 0, rh.BF16),
    (1, 2, 32, 6, 40, 2, 1, 32, 2, 1, rh.BF16),
    (1, 1, 128, 4, 100, 5, 1, 96, 2, 0, rh.BF16),   # one chunk: student = teacher
    (2, 1, 64, 9, 1, 2, 1, 32, 3, 0, rh.FP32),      # one-token frames
    (1, 2, 64, 5, 70, 1, 0, 64, 2, 0, rh.BF16),     # Tc = 1, To = 0
]


def check_loss(loss, stu, tea, hyb, soft, tol):
    """Assertions shared by the small and the full-size cases, per slab."""
    for s in range(loss.shape[0]):
        g_h, g_t, r_h, r_t = stu[s], tea[s], hyb[s], soft[s]
        assert np.abs(g_h - r_h).max() <= tol * np.abs(r_h).max()
        assert np.abs(g_t - r_t).max() <= tol * np.abs(r_t).max()
        own = float(((g_h - g_t) ** 2).sum())
        assert abs(loss[s] - own) <= 1e-5 * own + 1e-30
        d = r_h - r_t
        ref = float((d ** 2).sum())
        e = np.abs(g_h - r_h).max() + np.abs(g_t - r_t).max()
        bound = 2 * e * np.abs(d).sum() + d.size * e * e + 1e-5 * ref
        assert abs(loss[s] - ref) <= bound, (s, loss[s], ref, bound)
        print(f"slab {s}: loss {loss[s]:.6e} oracle {ref:.6e} rel {abs(loss[s] - ref) / ref:.2e}", flush=True)


@pytest.mark.parametrize("shape", SHAPES)
def test_distill_loss_matches_oracle(shape):
    p = rh.Params(*shape, out_dtype=rh.BF16)
    print(f"distill {shape}", flush=True)
    x = rand_inputs(p, seed=sum(shape[:9]), bias=shape[3] == 9)
    d = to_dev(x, p)
    loss, stu, tea = rh.distill_loss(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], d["bq"], d["bk"], outputs=True)
    torch.cuda.synchronize()
    again = rh.distill_loss(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], d["bq"], d["bk"])
    torch.cuda.synchronize()
    assert torch.equal(loss, again)
    po = oracle_params(p)
    hyb = oracle.parallel(po, x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"])
    soft = oracle.full_softmax(po, x["q"], x["k"], x["v"])
    BH = p.B * p.H
    check_loss(loss.cpu().numpy().reshape(BH).astype(np.float64),
               stu.cpu().numpy().reshape(BH, -1).astype(np.float64),
               tea.cpu().numpy().reshape(BH, -1).astype(np.float64),
               hyb.reshape(BH, -1), soft.reshape(BH, -1), TOL[p.in_dtype])
    if p.Tc >= p.T:
        assert float(loss.abs().max()) <= 1e-6 * float((stu.double() ** 2).sum())


def test_distill_loss_fullsize_slab():
    """Wan 5 s layer (12 heads x 32,760 tokens, bf16): the slab of head 0 against the oracle
    over every query row (hybrid by the chunk-parallel form, teacher by the definition)."""
    w = WORKLOADS["wan_5s"]
    p = rh.Params(w.B, w.H, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P, 0, rh.BF16, rh.BF16)
    print("[distill wan_5s] inputs", flush=True)
    x = make_inputs(w, seed=1)
    d = {key: torch.from_numpy(val).to("cuda", torch.bfloat16).contiguous() for key, val in x.items()}
    del x
    loss, stu, tea = rh.distill_loss(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], outputs=True)
    torch.cuda.synchronize()
    assert torch.isfinite(loss).all() and (loss > 0).all()
    xs = make_inputs(w, seed=1, slabs=[(0, 0)])
    p1 = oracle.Params(1, 1, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P)
    print("[distill wan_5s] oracle hybrid rows", flush=True)
    hyb, _ = oracle.parallel_rows(p1, xs["q"], xs["k"], xs["v"], xs["wq"], xs["wk"], np.arange(w.N))
    soft = np.empty_like(hyb)
    for r0 in range(0, w.N, 4096):
        rows = np.arange(r0, min(r0 + 4096, w.N))
        print(f"[distill wan_5s] oracle teacher rows {r0}..", flush=True)
        soft[rows] = oracle.full_softmax(p1, xs["q"], xs["k"], xs["v"], rows=rows)[0, 0]
    check_loss(loss[0, :1].cpu().numpy().astype(np.float64),
               stu[0, :1].cpu().numpy().reshape(1, -1).astype(np.float64),
               tea[0, :1].cpu().numpy().reshape(1, -1).astype(np.float64),
               hyb.reshape(1, -1), soft.reshape(1, -1), TOL[rh.BF16])
