#!/usr/bin/env python3
"""Throughput of ReHyAt chunk-wise hybrid attention on one MI355X.

One step = one chunk-parallel forward of the whole hot path on a Wan2.1-1.3B-shaped
attention layer, 5 s of 480x832 video: B=1, 12 heads, D=128, 21 latent frames of 30x52 =
1560 tokens (32,760 tokens), bf16 inputs, Tc=3, To=1, phi = per-head 128->128 map,
2 parts, powers 1..2 (256 features).  A step runs the per-frame state kernel, the frame
scan and the windowed softmax tile kernel with the fused linear combine, all in
librehyat.so, on device-resident synthetic inputs.

Printed as one JSON line: tokens/s (value), TFLOP/s and the fraction of the bf16 MFMA
peak, the roofline of the dominant kernel (attention tile kernel, timed with HIP events
on the stream it runs on), the full-softmax comparator on the same shapes, the 10 s
streaming form with its peak memory at 21/41/81 frames, the chunking and feature-map
variants the pages discuss (Tc/To presets and ablations, higher polynomial degree) on the
same inputs, the distillation objective (hybrid vs full-softmax teacher, squared L2 per
slab) and its gradients with respect to the feature-map weights, the backward for an
upstream gradient (dq, dk, dv and the feature-map gradients), the 20 s clip at batch 2 and
the 14B-shaped 720x1280 layer with P = 3 (each with its own oracle sample and spot check),
and the CPU oracle timed on a bounded sample of the same workload (which also serves as a
parity spot check).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0
METRIC = "hybrid-attn tokens/s & TFLOP/s (% bf16 MFMA peak), 32760-token 12-head layer"
KERNEL_SOURCES = ["attn_wide.hip", "attn_common.hpp", "dma.hpp", "tiles.hpp", "common.hpp", "kernels.hpp",
                  "state16.hpp", "wide_substep.inc", "gen_wide_substep.py"]
COUNTER_FILE = os.path.join(ROOT, "profiles", "attn_kernel_wan_5s_counters.txt")


LEGS = ("comparator", "stream", "variants", "distill_loss", "distill_grad", "backward", "wan_20s", "wan14b_720p")


def progress(msg):
    """One line per finished leg on stderr, so that a long run shows it is alive."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def schedule(T, Tc, To, linear_only=0):
    out = []
    for c in range((T + Tc - 1) // Tc):
        f0 = c * Tc
        f1 = min(f0 + Tc, T)
        ws = f1 if linear_only else max(0, f0 - To)
        out.append((f0, f1, ws, f1, ws))
    return out


def flop_model(B, H, D, T, n, Tc, To, Dphi, P, linear_only=0):
    """Algorithmic FLOPs (2 per multiply-add, elementwise work not counted)."""
    F = P * Dphi
    sch = schedule(T, Tc, To, linear_only)
    soft = sum((f1 - f0) * n * (we - ws) * n for f0, f1, ws, we, ls in sch)
    n_s = sch[-1][4] * n                                        # tokens entering some state
    n_c = sum((f1 - f0) * n for f0, f1, ws, we, ls in sch if ls > 0)  # queries with a linear part
    N = T * n
    total = B * H * (4 * D * soft + 4 * N * D * Dphi + 2 * n_s * F * D + 2 * n_c * F * (D + 1))
    attn = B * H * (4 * D * soft + 2 * n_c * D * Dphi + 2 * n_c * F * (D + 1))
    state = B * H * (2 * n_s * D * Dphi + 2 * n_s * F * D)
    return dict(total=total, attn_kernel=attn, state_kernel=state)


def sources_digest():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "hybrid_softmax_linear_chunked_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch of the attention kernel from the committed counter summary (two
    rocprofv3 passes, FETCH_SIZE and WRITE_SIZE, scaled by a copy kernel's readings), and
    where they come from.  The value is None unless the summary was taken on the current
    kernel sources (same sha256 over KERNEL_SOURCES)."""
    src = {"profile": os.path.relpath(COUNTER_FILE, ROOT), "sources_sha256": None,
           "current_sources_sha256": sources_digest(), "measured_in_this_run": False}
    if not os.path.exists(COUNTER_FILE):
        return None, src
    kv = {}
    for line in open(COUNTER_FILE):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    src["sources_sha256"] = kv.get("sources_sha256")
    try:
        if kv.get("sources_sha256") != src["current_sources_sha256"]:
            return None, src
        return float(kv["hbm_bytes_per_dispatch"]), src
    except (KeyError, ValueError):
        return None, src


def cpu_baseline(w, x, out_gpu, budget_s=12.0):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload: whole heads,
    every query row with the fp64 states built in full, head after head until about
    budget_s of wall time has passed (at least one head); extrapolated linearly to every
    head.  Also returns the parity of the GPU output on the heads computed."""
    import numpy as np
    import oracle
    p1 = oracle.Params(1, 1, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P)
    N = w.N
    rows = np.arange(N)
    done, spent, err = 0, 0.0, 0.0
    while done < w.H and (done == 0 or spent < budget_s):
        h = done
        sl = {key: (x[key][:, h:h + 1] if key in ("q", "k", "v") else x[key][h:h + 1]).astype(np.float64)
              for key in ("q", "k", "v", "wq", "wk")}
        t0 = time.perf_counter()
        ref, _ = oracle.parallel_rows(p1, sl["q"], sl["k"], sl["v"], sl["wq"], sl["wk"], rows)
        spent += time.perf_counter() - t0
        g = out_gpu[0, h].float().cpu().numpy()
        err = max(err, float(np.abs(g - ref).max() / np.abs(ref).max()))
        done += 1
    per_head = spent / done
    full_s = w.B * w.H * per_head
    cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    return dict(value=round(w.B * N / full_s, 3), unit="tokens/s", cores=cores, kind="oracle",
                sample=(f"{done} of {w.H} heads (batch 0) in full: fp64 states over all {w.T} frames and all "
                        f"{N} query rows, {spent:.1f} s ({per_head:.2f} s per head); extrapolated linearly "
                        f"to {w.B * w.H} heads = {full_s:.1f} s per layer")), \
        dict(max_rel_err=err, rows=int(N * done), heads=done, tol=2e-2)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip every leg after the main step")
    ap.add_argument("--legs", default="all",
                    help="comma-separated legs to run after the main step (comparator, stream, variants, "
                         "distill_loss, distill_grad, backward, wan_20s, wan14b_720p), or all")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="only time a plain bf16 library GEMM (torch.matmul, 8192 x 8192 x 8192) and print its "
                         "TFLOP/s: what a dense product reaches on this part under the same clock limits")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (3 dispatches): the reference for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import hybrid_softmax_linear_chunked_amd as rh
    from synth_inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.gemm_reference:
        n = 8192
        g = torch.Generator(device=dev)
        g.manual_seed(3)
        a_ = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
        b_ = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
        c_ = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
        for _ in range(5):
            torch.matmul(a_, b_, out=c_)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record()
        for _ in range(reps):
            torch.matmul(a_, b_, out=c_)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
        print(json.dumps({"gemm_reference": {"m": n, "n": n, "k": n, "dtype": "bf16", "ms": round(ms, 4),
                                             "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}}),
              flush=True)
        return
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_dispatch": src.numel() * 4}), flush=True)
        return
    w = WORKLOADS["wan_5s"]
    p = rh.Params(w.B, w.H, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P, 0, rh.BF16, rh.BF16)
    x = make_inputs(w, seed=1)
    d = {key: torch.from_numpy(val).to(dev, torch.bfloat16).contiguous() for key, val in x.items()}
    out = torch.empty((p.B, p.H, p.N, p.D), dtype=torch.bfloat16, device=dev)
    ws = rh.alloc_bytes(rh.workspace_bytes(p), dev)

    def step(ev_mid=None):
        rh.parallel_states(p, d["k"], d["v"], d["wk"], None, ws)
        if ev_mid is not None:
            ev_mid.record()
        rh.parallel_attend(p, d["q"], d["k"], d["v"], d["wq"], None, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record()
    for i in range(args.steps):
        starts[i].record()
        step(mids[i])
        ends[i].record()
    t_end.record()
    torch.cuda.synchronize()
    ms = t_begin.elapsed_time(t_end) / args.steps
    attn_ms = sum(mids[i].elapsed_time(ends[i]) for i in range(args.steps)) / args.steps
    state_ms = sum(starts[i].elapsed_time(mids[i]) for i in range(args.steps)) / args.steps

    fl = flop_model(w.B, w.H, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P)
    traffic, traffic_src = stored_traffic()
    tokens = w.B * w.N
    tflops = fl["total"] / (ms * 1e-3) / 1e12
    attn_tflops = fl["attn_kernel"] / (attn_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V and N(0,1/D) phi weights, bf16",
        "config": {"workload": "wan_5s", "B": w.B, "heads": w.H, "head_dim": w.D, "frames": w.T,
                   "frame_tokens": w.n, "tokens": w.N, "Tc": w.Tc, "To": w.To, "Dphi": w.Dphi, "P": w.P,
                   "form": "chunk-parallel"},
        "tflops": round(tflops, 2), "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "flops_per_step": fl["total"],
        "stages_ms": {"state_and_scan": round(state_ms, 4), "attn_kernel": round(attn_ms, 4)},
        "roofline": {"kernel": "attn_kernel (windowed softmax + fused linear combine)", "bound": "mfma",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "traffic_source": traffic_src, "algorithmic_flops_per_launch": fl["attn_kernel"]},
    }

    want = set(LEGS) if args.legs == "all" else set(args.legs.split(","))
    if args.no_extras:
        want = set()
    unknown = want - set(LEGS)
    if unknown:
        print(f"unknown legs: {sorted(unknown)}", file=sys.stderr)
        sys.exit(2)
    if "distill_grad" in want:
        want.add("distill_loss")
    if "comparator" in want:
        # full-softmax comparator: the same tile kernel with one window over all frames
        pc = p.with_(Tc=w.T)
        outc = torch.empty_like(out)
        rh.forward_parallel(pc, d["q"], d["k"], d["v"], d["wq"], d["wk"], out=outc)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record()
        for _ in range(reps):
            rh.forward_parallel(pc, d["q"], d["k"], d["v"], d["wq"], d["wk"], out=outc)
        e1.record()
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / reps
        cfl = flop_model(w.B, w.H, w.D, w.T, w.n, w.T, w.To, w.Dphi, w.P)["total"]
        res["full_softmax_comparator"] = {"ms": round(cms, 3), "tflops": round(cfl / (cms * 1e-3) / 1e12, 2),
                                          "speedup_of_hybrid": round(cms / ms, 2)}
        del outc
    if want:
        legs = [("stream", lambda: stream_leg(rh, torch, WORKLOADS["wan_10s_stream"], dev)),
                ("variants", lambda: variants_leg(rh, torch, p, d, ms)),
                ("distill_loss", lambda: distill_leg(rh, torch, p, d, w)),
                ("distill_grad", lambda: distill_grad_leg(rh, torch, p, d, w, res["distill_loss"]["ms"])),
                ("backward", lambda: backward_leg(rh, torch, p, d, w, ms))]
        for name, seed in (("wan_20s", 3), ("wan14b_720p", 4)):
            legs.append((name, lambda name=name, seed=seed: workload_leg(
                rh, torch, WORKLOADS[name], seed, dev, with_cpu=not args.no_cpu_baseline)))
        for name, leg in legs:
            if name not in want:
                continue
            t0 = time.perf_counter()
            res[name] = leg()
            progress(f"{name} leg done in {time.perf_counter() - t0:.1f} s")

    if not args.no_cpu_baseline:
        cb, parity = cpu_baseline(w, x, out)
        res["cpu_baseline"] = cb
        res["parity_spot_check"] = parity
        progress("cpu baseline done")
    print(json.dumps(res), flush=True)


def workload_leg(rh, torch, w, seed, dev, with_cpu=True, reps=5):
    """Chunk-parallel forward of a further measured workload (the 20 s clip at batch 2, the
    14B-shaped layer with P = 3) on its own seeded inputs: ms per forward, state/scan and
    attention stages, tokens/s, TFLOP/s of the FLOP model and fractions of the bf16 peak;
    then the CPU oracle on a bounded sample of it, which is also a parity spot check."""
    from synth_inputs import make_inputs
    p = rh.Params(w.B, w.H, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P, 0, rh.BF16, rh.BF16)
    x = make_inputs(w, seed=seed)
    d = {key: torch.from_numpy(val).to(dev, torch.bfloat16).contiguous() for key, val in x.items()}
    out = torch.empty((p.B, p.H, p.N, p.D), dtype=torch.bfloat16, device=dev)
    ws = rh.alloc_bytes(rh.workspace_bytes(p), dev)

    def step(ev_mid=None):
        rh.parallel_states(p, d["k"], d["v"], d["wk"], None, ws)
        if ev_mid is not None:
            ev_mid.record()
        rh.parallel_attend(p, d["q"], d["k"], d["v"], d["wq"], None, out, ws)

    step()
    step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        step(e[1])
        e[2].record()
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[2]) for e in ev) / reps
    state_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / reps
    fl = flop_model(w.B, w.H, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P)
    tf = fl["total"] / (ms * 1e-3) / 1e12
    atf = fl["attn_kernel"] / (attn_ms * 1e-3) / 1e12
    res = {"workload": w.name, "B": w.B, "heads": w.H, "frames": w.T, "frame_tokens": w.n,
           "tokens_per_sample": w.N, "Tc": w.Tc, "To": w.To, "Dphi": w.Dphi, "P": w.P,
           "ms": round(ms, 4), "stages_ms": {"state_and_scan": round(state_ms, 4), "attn_kernel": round(attn_ms, 4)},
           "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1), "tflops": round(tf, 2),
           "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
           "attn_kernel_frac_of_bf16_peak": round(atf / PEAK_BF16_TFLOPS, 4), "flops": fl["total"]}
    del ws, d
    if with_cpu:
        cb, parity = cpu_baseline(w, x, out, budget_s=6.0)
        res["cpu_baseline"] = cb
        res["parity_spot_check"] = parity
    del out, x
    torch.cuda.empty_cache()
    return res


# chunking and feature-map variants the pages discuss (ReHyAt blog 3.2, 5.2, 5.3, 6;
# mind-verse.de ablations), on the same Wan 5 s inputs
VARIANTS = {"tc5_to2": dict(Tc=5, To=2), "tc1_to0": dict(Tc=1, To=0), "tc3_to0": dict(Tc=3, To=0),
            "tc3_to2": dict(Tc=3, To=2), "tc7_to1": dict(Tc=7, To=1), "p3": dict(P=3), "p4": dict(P=4)}


def variants_leg(rh, torch, p, d, base_ms, reps=5):
    """Whole chunk-parallel forward (states, scan, attention) per variant: ms, tokens/s,
    TFLOP/s of the FLOP model and its fraction of the bf16 peak."""
    res = {}
    for name, kw in VARIANTS.items():
        pv = p.with_(**kw)
        ws = rh.alloc_bytes(rh.workspace_bytes(pv), d["q"].device)
        out = torch.empty((p.B, p.H, p.N, p.D), dtype=torch.bfloat16, device=d["q"].device)

        def call(ev_mid=None):
            rh.parallel_states(pv, d["k"], d["v"], d["wk"], None, ws)
            if ev_mid is not None:
                ev_mid.record()
            rh.parallel_attend(pv, d["q"], d["k"], d["v"], d["wq"], None, out, ws)
        call()
        call()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        for e in ev:
            e[0].record()
            call(e[1])
            e[2].record()
        torch.cuda.synchronize()
        vms = sum(e[0].elapsed_time(e[2]) for e in ev) / reps
        sms = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
        fl = flop_model(pv.B, pv.H, pv.D, pv.T, pv.n, pv.Tc, pv.To, pv.Dphi, pv.P)["total"]
        tf = fl / (vms * 1e-3) / 1e12
        res[name] = {"Tc": pv.Tc, "To": pv.To, "P": pv.P, "ms": round(vms, 4), "state_and_scan_ms": round(sms, 4),
                     "tokens_per_s": round(pv.B * pv.N / (vms * 1e-3), 1), "tflops": round(tf, 2),
                     "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2), "flops": fl}
        del ws, out
    fl1 = flop_model(p.B, p.H, p.D, p.T, p.n, p.Tc, p.To, p.Dphi, p.P)["total"]
    res["to2_vs_to1"] = {"flop_ratio": round(res["tc3_to2"]["flops"] / fl1, 4),
                         "time_ratio": round(res["tc3_to2"]["ms"] / base_ms, 4)}
    return res


def distill_leg(rh, torch, p, d, w, reps=3):
    """Distillation objective on the same inputs (student forward with float32 output,
    full-softmax teacher, squared distance per slab): ms per call and TFLOP/s over the two
    forwards' FLOPs."""
    ws = rh.alloc_bytes(rh.distill_workspace_bytes(p), d["q"].device)
    loss = torch.empty((p.B, p.H), dtype=torch.float32, device=d["q"].device)
    call = lambda: rh.distill_loss(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], loss=loss, ws=ws)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    dms = e0.elapsed_time(e1) / reps
    fl = (flop_model(w.B, w.H, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P)["total"]
          + flop_model(w.B, w.H, w.D, w.T, w.n, w.T, 0, w.Dphi, w.P)["total"])
    res = {"ms": round(dms, 3), "tflops": round(fl / (dms * 1e-3) / 1e12, 2),
           "loss_mean_per_element": float(loss.double().sum() / (p.B * p.H * p.N * p.D))}
    del ws
    return res


def grad_flops(B, H, D, T, n, Tc, To, Dphi, P, linear_only=0):
    """Algorithmic FLOPs of the feature-map gradients after the two forwards: phi of every
    query and key, dphi_q over the queries with a linear region, the per-chunk sums
    R = phi_q^T [a|h], dphi_k over the keys that enter a state, dW_q over all queries and
    dW_k over those keys (2 per multiply-add)."""
    F = P * Dphi
    sch = schedule(T, Tc, To, linear_only)
    N = T * n
    n_s = sch[-1][4] * n
    n_c = sum((f1 - f0) * n for f0, f1, ws, we, ls in sch if ls > 0)
    return B * H * (4 * N * D * Dphi + 4 * n_c * F * (D + 1) + 2 * n_s * F * (D + 1)
                    + 2 * N * Dphi * D + 2 * n_s * Dphi * D)


def distill_grad_leg(rh, torch, p, d, w, loss_ms, reps=3):
    """Distillation loss and its gradients with respect to W_q, W_k, b_q, b_k: ms per call,
    the gradient stages' share (call minus the loss-only call) and their TFLOP/s."""
    ws = rh.alloc_bytes(rh.distill_grad_workspace_bytes(p), d["q"].device)
    call = lambda: rh.distill_grad(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], ws=ws)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    gms = e0.elapsed_time(e1) / reps
    gfl = grad_flops(w.B, w.H, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P)
    bw = max(gms - loss_ms, 1e-6)
    res = {"ms": round(gms, 3), "gradient_stages_ms": round(bw, 3), "gradient_flops": gfl,
           "gradient_tflops": round(gfl / (bw * 1e-3) / 1e12, 2),
           "bound": "products on the bf16 matrix core (a float operand as hi + lo bf16 parts: up to three "
                    "products per algorithmic one; 2.5 PFLOP/s dense bf16) and HBM passes over float "
                    "per-token rows; fp32 inputs take the fp32 matrix core (157.3 TFLOP/s)",
           "workspace_bytes": int(ws.numel())}
    del ws
    return res


def backward_flops(B, H, D, T, n, Tc, To, Dphi, P, linear_only=0):
    """Algorithmic FLOPs of rehyat_backward after its forward recompute: five products per
    chunk window in the softmax branch (scores, dP, dV, dK, dQ), the feature-map gradients,
    and the linear branch's input gradients (dq, dk through W, dv through the chunk sums)."""
    F = P * Dphi
    sch = schedule(T, Tc, To, linear_only)
    soft = sum((f1 - f0) * n * (we - ws) * n for f0, f1, ws, we, ls in sch)
    n_s = sch[-1][4] * n
    N = T * n
    return (B * H * (10 * D * soft + 4 * N * Dphi * D + 2 * n_s * F * D)
            + grad_flops(B, H, D, T, n, Tc, To, Dphi, P, linear_only))


def backward_leg(rh, torch, p, d, w, fwd_ms, reps=2):
    """rehyat_backward for a seeded upstream gradient: ms per call (forward recompute
    included), the backward stages' share (call minus the forward step) and their TFLOP/s."""
    g = torch.Generator(device=d["q"].device)
    g.manual_seed(7)
    dout = torch.randn((p.B, p.H, p.N, p.D), generator=g, device=d["q"].device)
    ws = rh.alloc_bytes(rh.backward_workspace_bytes(p), d["q"].device)
    call = lambda: rh.backward(p, d["q"], d["k"], d["v"], d["wq"], d["wk"], dout, ws=ws)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    bms = e0.elapsed_time(e1) / reps
    fl = backward_flops(w.B, w.H, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P)
    st = max(bms - fwd_ms, 1e-6)
    tf = fl / (st * 1e-3) / 1e12
    res = {"ms": round(bms, 3), "backward_stages_ms": round(st, 3), "backward_flops": fl,
           "backward_tflops": round(tf, 2), "peak_tflops": PEAK_BF16_TFLOPS,
           "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
           "bound": "mfma: every product on the bf16 matrix core for bf16 inputs (the linear branch's float "
                    "operands as hi + lo bf16 parts)",
           "workspace_bytes": int(ws.numel())}
    del ws, dout
    return res


def stream_leg(rh, torch, w, dev):
    """10 s clip chunk by chunk through rehyat_chunk_step: time per clip, and peak device
    memory for 21, 41 and 81 frames with chunks generated on the fly (constant memory)."""
    p = rh.Params(w.B, w.H, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P, 0, rh.BF16, rh.BF16)
    g = torch.Generator(device=dev)
    g.manual_seed(2)
    sd = 1.0 / math.sqrt(w.D)
    wq = (torch.randn((w.H, w.Dphi, w.D), generator=g, device=dev) * sd).to(torch.bfloat16)
    wk = (torch.randn((w.H, w.Dphi, w.D), generator=g, device=dev) * sd).to(torch.bfloat16)
    chunks = []
    for f0 in range(0, w.T, w.Tc):
        fr = min(w.Tc, w.T - f0)
        shape = (w.B, w.H, fr * w.n, w.D)
        chunks.append((fr, *(torch.randn(shape, generator=g, device=dev).to(torch.bfloat16) for _ in range(3))))
    outs = [torch.empty_like(c[1]) for c in chunks]
    st = rh.Stream(p, wq, wk)

    def clip():
        st.init()
        for (fr, q, k, v), o in zip(chunks, outs):
            st.step(q, k, v, fr, out=o)

    clip()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        clip()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del chunks, outs, st
    torch.cuda.empty_cache()

    # one short warm-up stream first: the HIP runtime loads code objects and sizes its
    # scratch area on the first launch of each kernel, once per process
    full = w.B * w.H * w.Tc * w.n * w.D
    warm = [torch.zeros(full, dtype=torch.bfloat16, device=dev) for _ in range(4)]
    ws_ = rh.Stream(p, wq, wk)
    for fr in (w.Tc, w.Tc, w.Tc - 1):
        q, k, v, o = (t[:w.B * w.H * fr * w.n * w.D].view(w.B, w.H, fr * w.n, w.D) for t in warm)
        ws_.step(q, k, v, fr, out=o)
    torch.cuda.synchronize()
    del warm, ws_, q, k, v, o
    def measure(T):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        # one chunk of q, k, v, out (a shorter final chunk uses the front of the same
        # storage), the streaming state and its workspace: allocated once, up front
        bufs = [torch.empty(full, dtype=torch.bfloat16, device=dev) for _ in range(4)]
        for buf in bufs[:3]:
            buf.normal_(generator=g)
        s = rh.Stream(p.with_(T=T), wq, wk)
        torch.cuda.synchronize()
        footprint = torch.cuda.memory_allocated() - base
        torch.cuda.reset_peak_memory_stats()
        free0 = torch.cuda.mem_get_info()[0]
        low = free0
        for f0 in range(0, T, w.Tc):
            fr = min(w.Tc, T - f0)
            q, k, v, o = (t[:w.B * w.H * fr * w.n * w.D].view(w.B, w.H, fr * w.n, w.D) for t in bufs)
            s.step(q, k, v, fr, out=o)
            low = min(low, torch.cuda.mem_get_info()[0])
        torch.cuda.synchronize()
        return {"footprint_bytes": int(footprint),
                "peak_allocated_bytes": int(torch.cuda.max_memory_allocated() - base),
                "device_free_drop_during_steps": int(free0 - low)}

    peak = {str(T): measure(T) for T in (21, 41, 81)}
    # the streamed clip does the work of the chunk-parallel form on the same clip (the same
    # windows, the same state partials)
    fl = flop_model(w.B, w.H, w.D, w.T, w.n, w.Tc, w.To, w.Dphi, w.P)["total"]
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": "wan_10s_stream", "frames": w.T, "tokens": w.N, "ms_per_clip": round(ms, 3),
            "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1), "flops_per_clip": fl, "tflops": round(tf, 2),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "chunk_steps": (w.T + w.Tc - 1) // w.Tc, "peak_memory_by_frames": peak}


if __name__ == "__main__":
    main()
