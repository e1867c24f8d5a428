"""The FLOP model behind every TFLOP/s the benchmark reports, checked against a brute-force
count of the same quantities from the explicit region masks of the oracle (ReHyAt blog,
maplevalley.com.cn, 2.2.1 and 2.3): softmax (query, key) pairs, queries with a linear
region, keys that enter some query's linear region.  Work per item (2 flops per
multiply-add): softmax 4 D per pair (scores and values), feature map 2 D Dphi per query and
per key, state 2 F D per key that enters a state, combine 2 F (D + 1) per query with a
linear region; the backward adds 10 D per pair (scores, dP, dV, dK, dQ)."""
import numpy as np
import pytest

import bench
import oracle

SHAPES = [
    # B, H, D, T, n, Tc, To, Dphi, P, linear_only
    (1, 2, 32, 7, 16, 3, 1, 32, 2, 0),
    (2, 3, 64, 10, 5, 4, 2, 64, 3, 0),
    (1, 1, 128, 9, 7, 2, 3, 96, 4, 0),      # To > Tc
    (1, 2, 32, 8, 6, 3, 1, 32, 2, 1),       # empty softmax window
    (1, 1, 64, 5, 9, 1, 0, 32, 1, 0),       # Tc = 1, To = 0
    (1, 1, 32, 4, 6, 6, 1, 32, 2, 0),       # one chunk over the clip
]


def counts(p):
    soft, lin = oracle.numpy_masks(p)
    pairs = int(soft.sum())
    n_c = int(lin.any(axis=1).sum())
    n_s = int(lin.any(axis=0).sum())
    return pairs, n_c, n_s


@pytest.mark.parametrize("shape", SHAPES)
def test_flop_model_matches_mask_counts(shape):
    B, H, D, T, n, Tc, To, Dphi, P, lo = shape
    p = oracle.Params(*shape)
    pairs, n_c, n_s = counts(p)
    F, N = P * Dphi, T * n
    want = B * H * (4 * D * pairs + 4 * N * D * Dphi + 2 * n_s * F * D + 2 * n_c * F * (D + 1))
    assert bench.flop_model(B, H, D, T, n, Tc, To, Dphi, P, lo)["total"] == want
    g_want = B * H * (4 * N * D * Dphi + 4 * n_c * F * (D + 1) + 2 * n_s * F * (D + 1)
                      + 2 * N * Dphi * D + 2 * n_s * Dphi * D)
    assert bench.grad_flops(B, H, D, T, n, Tc, To, Dphi, P, lo) == g_want
    b_want = B * H * (10 * D * pairs + 4 * N * Dphi * D + 2 * n_s * F * D) + g_want
    assert bench.backward_flops(B, H, D, T, n, Tc, To, Dphi, P, lo) == b_want


def test_documented_workload_totals():
    tf = lambda *a: bench.flop_model(*a)["total"] / 1e12
    assert round(tf(1, 12, 128, 21, 1560, 3, 1, 128, 2), 4) == 1.2800
    assert round(tf(1, 12, 128, 41, 1560, 3, 1, 128, 2), 4) == 2.5213
    assert round(tf(2, 12, 128, 81, 1560, 3, 1, 128, 2), 3) == 10.180
    assert round(tf(1, 40, 128, 21, 3600, 3, 1, 128, 3), 3) == 22.195
