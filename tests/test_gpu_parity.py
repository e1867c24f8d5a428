"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle on the same
seeded inputs, element by element, at sizes that span several 64-token tiles and ragged
tails; plus the per-part outputs (softmax part, log-sum-exp, phi(q) S, phi(q) Z), the
reductions (one chunk = softmax attention, empty window = linear attention), streaming
against the chunk-parallel form, determinism and state checkpoint/restore.

References: ReHyAt blog (maplevalley.com.cn) sections 2.2.1, 2.2.2, 2.3, 5.2.
"""
import numpy as np
import pytest
import torch

import hybrid_softmax_linear_chunked_amd as rh
import oracle
from gpu_common import TOL, oracle_params, rand_inputs, run_parallel, slab_err, to_dev

pytestmark = pytest.mark.gpu

FP32, BF16 = rh.FP32, rh.BF16

CASES = [
    # tiny workload: 7 frames of 4x4 tokens, D=32, phi 32 -> 64 features
    rh.Params(1, 2, 32, 7, 16, 3, 1, 32, 2, 0, FP32, FP32),
    # several tiles per window with ragged tails (n=40: window of 160 keys = 2.5 tiles)
    rh.Params(2, 2, 32, 7, 40, 3, 1, 32, 2, 0, FP32, FP32),
    rh.Params(1, 2, 64, 9, 50, 3, 1, 64, 2, 0, FP32, FP32),
    rh.Params(1, 1, 128, 7, 70, 3, 1, 128, 2, 0, FP32, FP32),
    # overlap variants and uneven tails
    rh.Params(1, 1, 32, 10, 24, 4, 2, 32, 2, 0, FP32, FP32),
    rh.Params(1, 1, 32, 6, 33, 2, 0, 32, 2, 0, FP32, FP32),
    rh.Params(1, 1, 32, 7, 20, 2, 3, 32, 2, 0, FP32, FP32),
    rh.Params(1, 1, 32, 2, 30, 3, 1, 32, 2, 0, FP32, FP32),
    rh.Params(1, 1, 32, 1, 45, 3, 1, 32, 2, 0, FP32, FP32),
    rh.Params(1, 2, 32, 8, 1, 3, 1, 32, 2, 0, FP32, FP32),
    rh.Params(1, 1, 64, 9, 17, 1, 1, 32, 2, 0, FP32, FP32),
    # P = 1, P = 3 (uneven split 11/11/10 and 43/43/42), P = 4
    rh.Params(1, 1, 32, 7, 20, 3, 1, 32, 1, 0, FP32, FP32),
    rh.Params(1, 1, 64, 7, 20, 3, 1, 32, 3, 0, FP32, FP32),
    rh.Params(1, 1, 128, 7, 20, 3, 1, 128, 3, 0, FP32, FP32),
    rh.Params(1, 1, 32, 7, 20, 3, 1, 64, 4, 0, FP32, FP32),
    # empty softmax window
    rh.Params(1, 2, 32, 7, 20, 3, 1, 32, 2, 1, FP32, FP32),
    # bf16 inputs, fp32 accumulation
    rh.Params(1, 2, 128, 7, 100, 3, 1, 128, 2, 0, BF16, BF16),
    rh.Params(2, 1, 128, 8, 90, 3, 1, 128, 2, 0, BF16, FP32),
    rh.Params(1, 2, 128, 7, 60, 3, 1, 128, 3, 0, BF16, BF16),
    rh.Params(1, 2, 64, 7, 75, 3, 1, 64, 2, 0, BF16, BF16),
    rh.Params(1, 2, 32, 7, 80, 3, 1, 32, 2, 0, BF16, BF16),
    rh.Params(1, 2, 128, 7, 50, 3, 1, 128, 2, 1, BF16, BF16),
    rh.Params(1, 1, 128, 10, 64, 4, 2, 96, 2, 0, BF16, BF16),
    # bf16, P = 4 at Dphi = D = 128: W_q and all four state-image powers exceed the LDS, so the
    # epilogue stages one power at a time
    rh.Params(1, 1, 128, 7, 70, 3, 1, 128, 4, 0, BF16, BF16),
]


def _id(p):
    return (f"{'bf16' if p.in_dtype else 'f32'}-B{p.B}H{p.H}D{p.D}T{p.T}n{p.n}Tc{p.Tc}To{p.To}"
            f"F{p.Dphi}x{p.P}{'-lin' if p.linear_only else ''}")


@pytest.mark.parametrize("p", CASES, ids=_id)
def test_forward_parallel_matches_oracle(p):
    x = rand_inputs(p, seed=1, bias=(p.B == 2))
    d = to_dev(x, p)
    out, aux = run_parallel(p, d)
    # the production call, without per-part outputs
    out_only = run_parallel(p, d, aux=False)
    torch.cuda.synchronize()
    op = oracle_params(p)
    ref, rax = oracle.parallel(op, x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"], aux=True)
    tol = TOL[p.in_dtype]
    assert slab_err(out.float().cpu().numpy(), ref) <= tol
    assert slab_err(out_only.float().cpu().numpy(), ref) <= tol
    # per-part outputs: each one is checked at the same bar where it is defined
    if not p.linear_only:
        assert slab_err(aux["o_soft"].cpu().numpy(), rax["osoft"]) <= tol
        assert slab_err(aux["lse"].cpu().numpy(), rax["lse"]) <= tol
    lin = rax["z"].reshape(-1) > 0
    if lin.any():
        gy = aux["y"].cpu().numpy().reshape(-1, p.D)[lin]
        ry = rax["y"].reshape(-1, p.D)[lin]
        assert np.abs(gy - ry).max() / np.abs(ry).max() <= tol
        gz = aux["z"].cpu().numpy().reshape(-1)[lin]
        rz = rax["z"].reshape(-1)[lin]
        assert np.abs(gz / rz - 1).max() <= tol
    # rows without a linear region report exactly zero linear parts
    if (~lin).any():
        assert np.all(aux["z"].cpu().numpy().reshape(-1)[~lin] == 0)


@pytest.mark.parametrize("p", [CASES[0], CASES[13], CASES[16], CASES[18]], ids=_id)
def test_phi_matches_oracle(p):
    x = rand_inputs(p, seed=2, bias=True)
    d = to_dev(x, p)
    f = rh.phi(p, d["q"], d["wq"], d["bq"])
    torch.cuda.synchronize()
    ref = oracle.phi(oracle_params(p), x["q"], x["wq"], x["bq"])
    assert slab_err(f.float().cpu().numpy(), ref) <= TOL[p.in_dtype]


@pytest.mark.parametrize("dt", [FP32, BF16])
def test_one_chunk_is_softmax_attention(dt):
    """Tc >= T: one chunk, no linear region: softmax attention (the full-softmax comparator)."""
    p = rh.Params(1, 2, 128 if dt == BF16 else 64, 5, 70, 8, 1, 128 if dt == BF16 else 64, 2, 0, dt, FP32)
    x = rand_inputs(p, seed=3)
    d = to_dev(x, p)
    out = run_parallel(p, d, aux=False)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x[key]).double() for key in ("q", "k", "v"))).numpy()
    assert slab_err(out.cpu().numpy(), ref) <= TOL[dt]


@pytest.mark.parametrize("p", [CASES[0], CASES[4], CASES[6], CASES[15], CASES[16], CASES[18], CASES[22]], ids=_id)
def test_stream_equals_parallel_bitwise(p):
    """The streaming form adds the same per-frame partials in the same order and sweeps the
    same window tiles in the same order, so it reproduces the chunk-parallel output bit for
    bit, first chunk included."""
    x = rand_inputs(p, seed=4)
    d = to_dev(x, p)
    par = run_parallel(p, d, aux=False)
    st = rh.Stream(p, d["wq"], d["wk"])
    outs = []
    for f0 in range(0, p.T, p.Tc):
        f1 = min(f0 + p.Tc, p.T)
        sl = slice(f0 * p.n, f1 * p.n)
        outs.append(st.step(d["q"][:, :, sl].contiguous(), d["k"][:, :, sl].contiguous(),
                            d["v"][:, :, sl].contiguous(), f1 - f0))
    torch.cuda.synchronize()
    s_out = torch.cat(outs, dim=2)
    assert torch.equal(s_out, par)
    ref = oracle.stream(oracle_params(p), x["q"], x["k"], x["v"], x["wq"], x["wk"])
    assert slab_err(s_out.float().cpu().numpy(), ref) <= TOL[p.in_dtype]


@pytest.mark.parametrize("T,Tc", [(3, 5), (3, 3)], ids=["T<Tc", "T=Tc"])
def test_one_chunk_clip_same_bits_in_every_form(T, Tc):
    """A clip that one chunk covers is plain softmax attention over all its frames.  The bf16
    kernel splits the last query tiles of each XCD over two workgroups by a rule that looks at
    that chunk alone (its frames and its tiles), so running the clip with Tc >= T, with
    Tc = T (the distillation teacher's form) or streamed in one step gives the same bits; the
    output matches the oracle.  The window spans 300 keys (five tiles), so the split engages."""
    p = rh.Params(1, 2, 128, T, 100, Tc, 1, 128, 2, 0, BF16, BF16)
    x = rand_inputs(p, seed=11)
    d = to_dev(x, p)
    par = run_parallel(p, d, aux=False)
    teacher = p.with_(Tc=T)
    par_t = run_parallel(teacher, d, aux=False)
    st = rh.Stream(p, d["wq"], d["wk"])
    s_out = st.step(d["q"].contiguous(), d["k"].contiguous(), d["v"].contiguous(), T)
    torch.cuda.synchronize()
    assert rh.workspace_bytes(p) > 0 and rh.workspace_bytes(teacher) == rh.workspace_bytes(p)
    assert torch.equal(par, par_t)
    assert torch.equal(s_out, par)
    ref = oracle.parallel(oracle_params(p), x["q"], x["k"], x["v"], x["wq"], x["wk"])
    assert slab_err(par.float().cpu().numpy(), ref) <= TOL[BF16]


def test_stream_rejects_calls_after_short_chunk():
    p = CASES[0]
    x = rand_inputs(p, seed=5)
    d = to_dev(x, p)
    st = rh.Stream(p, d["wq"], d["wk"])
    sl = slice(0, 2 * p.n)
    st.step(d["q"][:, :, sl].contiguous(), d["k"][:, :, sl].contiguous(), d["v"][:, :, sl].contiguous(), 2)
    with pytest.raises(rh.RehyatError) as e:
        st.step(d["q"][:, :, sl].contiguous(), d["k"][:, :, sl].contiguous(), d["v"][:, :, sl].contiguous(), 2)
    assert e.value.status == 5


def test_attend_repeats_after_one_states_call():
    """The attention stage only reads the workspace that rehyat_parallel_states wrote:
    repeated attention calls on one workspace agree bit for bit."""
    p = CASES[16]
    x = rand_inputs(p, seed=7)
    d = to_dev(x, p)
    ws = rh.alloc_bytes(rh.workspace_bytes(p))
    rh.parallel_states(p, d["k"], d["v"], d["wk"], d["bk"], ws)
    outs = []
    for _ in range(3):
        o = torch.empty_like(d["q"])
        rh.parallel_attend(p, d["q"], d["k"], d["v"], d["wq"], d["bq"], o, ws)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    ref = oracle.parallel(oracle_params(p), x["q"], x["k"], x["v"], x["wq"], x["wk"], x["bq"], x["bk"])
    assert slab_err(outs[2].float().cpu().numpy(), ref) <= TOL[p.in_dtype]


@pytest.mark.parametrize("p", [CASES[1], CASES[16]], ids=_id)
def test_deterministic(p):
    x = rand_inputs(p, seed=6)
    d = to_dev(x, p)
    a = run_parallel(p, d, aux=False).clone()
    b = run_parallel(p, d, aux=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_stream_checkpoint_restore():
    """The device state plus the host handle is the whole checkpoint (blog 5.2 `states`)."""
    p = rh.Params(1, 2, 128, 10, 50, 3, 1, 128, 2, 0, BF16, BF16)
    x = rand_inputs(p, seed=7)
    d = to_dev(x, p)

    def chunk(f0):
        f1 = min(f0 + p.Tc, p.T)
        sl = slice(f0 * p.n, f1 * p.n)
        return d["q"][:, :, sl].contiguous(), d["k"][:, :, sl].contiguous(), d["v"][:, :, sl].contiguous(), f1 - f0

    a = rh.Stream(p, d["wq"], d["wk"])
    a.step(*chunk(0))
    a.step(*chunk(3))
    snap = a.save()
    ref = [a.step(*chunk(6)).clone(), a.step(*chunk(9)).clone()]
    b = rh.Stream(p, d["wq"], d["wk"])
    b.restore(snap)
    got = [b.step(*chunk(6)), b.step(*chunk(9))]
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert torch.equal(r, g)


def _far_score_inputs(p, seed):
    """Queries sharing a large positive mean and one all-3 key per frame at frame offset 45,
    past the first 32 keys of every window: those keys score about 2^90 (log2 units) above
    the keys at the start of their windows."""
    from synth_inputs import round_bf16
    x = rand_inputs(p, seed=seed)
    q = x["q"] * np.float32(0.3) + np.float32(2.0)
    k = x["k"].copy()
    for f in range(p.T):
        k[:, :, f * p.n + 45, :] = 3.0
    if p.in_dtype == BF16:
        q = round_bf16(q)
    x["q"], x["k"] = q, k
    return x


@pytest.mark.parametrize("dt", [BF16, FP32], ids=["bf16", "f32"])
def test_scores_far_above_window_start(dt):
    """The bf16 kernel takes its softmax reference from the first 32 keys of a window; with
    the planted keys every row sum overflows its range check and the window is swept again
    against the exact row maximum.  The fp32 kernel rescales its running maximum instead.
    Both must match the oracle, the log-sum-exp included (ReHyAt blog, maplevalley.com.cn,
    2.2.1)."""
    p = rh.Params(1, 2, 128, 7, 100, 3, 1, 128, 2, 0, dt, dt)
    x = _far_score_inputs(p, seed=5)
    q, k = x["q"], x["k"]
    d = to_dev(x, p)
    out, aux = run_parallel(p, d)
    torch.cuda.synchronize()
    op = oracle_params(p)
    ref, rax = oracle.parallel(op, x["q"], x["k"], x["v"], x["wq"], x["wk"], None, None, aux=True)
    # the planted keys' margin over the window start exceeds 64 log2 units
    s = (q[0, 0, 0].astype(np.float64) @ k[0, 0, 45].astype(np.float64)) / np.sqrt(p.D) * np.log2(np.e)
    s0 = (k[0, 0, :32].astype(np.float64) @ q[0, 0, 0].astype(np.float64)).max() / np.sqrt(p.D) * np.log2(np.e)
    assert s - s0 > 64
    tol = TOL[dt]
    assert slab_err(out.float().cpu().numpy(), ref) <= tol
    assert slab_err(aux["o_soft"].cpu().numpy(), rax["osoft"]) <= tol
    assert np.abs(aux["lse"].cpu().numpy() - rax["lse"]).max() <= tol * np.abs(rax["lse"]).max()


def test_stream_equals_parallel_far_scores():
    """The streaming kernel takes the same second sweep on the same windows: bitwise equal to
    the chunk-parallel output on the planted far-score inputs."""
    p = rh.Params(1, 2, 128, 7, 100, 3, 1, 128, 2, 0, BF16, BF16)
    x = _far_score_inputs(p, seed=6)
    d = to_dev(x, p)
    par = run_parallel(p, d, aux=False)
    st = rh.Stream(p, d["wq"], d["wk"])
    outs = []
    for f0 in range(0, p.T, p.Tc):
        f1 = min(f0 + p.Tc, p.T)
        sl = slice(f0 * p.n, f1 * p.n)
        outs.append(st.step(d["q"][:, :, sl].contiguous(), d["k"][:, :, sl].contiguous(),
                            d["v"][:, :, sl].contiguous(), f1 - f0))
    torch.cuda.synchronize()
    s_out = torch.cat(outs, dim=2)
    assert torch.equal(s_out, par)
