"""Pins of the oracle's V-Smooth grouping (k-means + stable label sort) and
preprocessing (block means, residual quantisation) against brute force,
library routines and invariants."""
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import oracle as O
import vc_workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bf16_vals(x):
    return O.bf16_to_f32(O.bf16_round(np.asarray(x, np.float32)))


def test_assign_matches_brute_force_fp64_when_margin_is_clear():
    rng = np.random.default_rng(0)
    for trial in range(40):
        N, k, d = rng.integers(1, 13), rng.integers(1, 4), 128
        V = _bf16_vals(rng.standard_normal((N, d)) * rng.uniform(0.1, 10))
        C = rng.standard_normal((k, d)).astype(np.float32)
        lab = O.kmeans_assign(V, C)
        dist = ((V[:, None, :].astype(np.float64) - C[None].astype(np.float64)) ** 2).sum(-1)
        order = np.sort(dist, axis=1)
        for j in range(N):
            if k == 1 or order[j, 1] - order[j, 0] > 1e-3 * max(1.0, order[j, 0]):
                assert lab[j] == int(np.argmin(dist[j]))


def test_assign_ties_go_to_lowest_centroid():
    V = _bf16_vals(np.ones((3, 128)))
    C = np.stack([np.full(128, 2.0), np.zeros(128), np.full(128, 2.0), np.zeros(128)]).astype(np.float32)
    assert list(O.kmeans_assign(V, C)) == [0, 0, 0]


def test_planted_clusters_recovered():
    rng = np.random.default_rng(1)
    k, d, N = 6, 128, 600
    centers = rng.standard_normal((k, d)) * 20
    lab = rng.integers(0, k, N)
    V = _bf16_vals(centers[lab] + rng.standard_normal((N, d)) * 0.5)
    # init draws centroid c from token floor(c*N/k): make every cluster appear there
    for c in range(k):
        lab[(c * N) // k] = c
        V[(c * N) // k] = _bf16_vals(centers[c])
    labels, cent, counts = O.kmeans(V, k, 5)
    # same partition up to relabelling
    for c in range(k):
        members = np.unique(labels[lab == c])
        assert len(members) == 1
    assert counts.sum() == N


def test_lloyd_objective_non_increasing_and_fixed_point():
    Q, K, V = W.custom_inputs(1, 1, 3000, seed=9)
    v = O.bf16_to_f32(V[0, 0].view(dtype=__import__("torch").int16).numpy().view(np.uint16))
    prev = np.inf
    vd = v.astype(np.float64)
    for it in range(1, 9):
        lab, cent, _ = O.kmeans(v, 16, it)
        # objective of the assignment against the centroids it was assigned to
        _, cent_prev, _ = O.kmeans(v, 16, it - 1) if it > 1 else (None, None, None)
        if it > 1:
            obj = float(((vd - cent_prev.astype(np.float64)[lab]) ** 2).sum())
            assert obj <= prev * (1 + 1e-9)
            prev = obj
        else:
            prev = np.inf
    # a converged run is a fixed point: labels = argmin, centroids = fixed-point means
    lab, cent, counts = O.kmeans(v, 16, 60)
    assert (O.kmeans_assign(v, cent) == lab).all()
    for c in range(16):
        if counts[c]:
            s = np.rint(v[lab == c].astype(np.float64) * 2 ** 24).astype(np.int64).sum(0)
            np.testing.assert_array_equal(cent[c], ((s.astype(np.float64) * 2 ** -24) / counts[c]).astype(np.float32))


def test_kmeans_is_independent_of_thread_count():
    code = ("import sys,numpy as np; sys.path.insert(0,%r); from oracle import oracle as O; import vc_workloads as W;"
            "Q,K,V=W.custom_inputs(1,1,5000,seed=3); v=O.bf16_to_f32(V[0,0].view(dtype=__import__('torch').int16).numpy().view(np.uint16));"
            "l,c,_=O.kmeans(v,32,6); import hashlib; sys.stdout.write(hashlib.md5(l.tobytes()+c.tobytes()).hexdigest())") % ROOT
    outs = set()
    for t in ("1", "3", "8"):
        env = dict(os.environ, OMP_NUM_THREADS=t)
        outs.add(subprocess.check_output([sys.executable, "-c", code], env=env).decode())
    assert len(outs) == 1


def test_stable_sort_matches_library_and_brute_force():
    rng = np.random.default_rng(2)
    for N, k in [(1, 1), (7, 3), (1000, 8), (5000, 64), (300, 256)]:
        lab = rng.integers(0, k, N)
        perm = O.stable_label_sort(lab, k)
        np.testing.assert_array_equal(perm, np.argsort(lab, kind="stable"))
        if N <= 300:
            brute = sorted(range(N), key=lambda j: (lab[j], j))
            assert list(perm) == brute


def test_block_means_reconstruct_values_exactly():
    Q, K, V = W.custom_inputs(1, 1, 1000, seed=4)
    v16 = V[0, 0].view(dtype=__import__("torch").int16).numpy().view(np.uint16)
    k16 = K[0, 0].view(dtype=__import__("torch").int16).numpy().view(np.uint16)
    perm = np.random.default_rng(0).permutation(1000).astype(np.int32)
    prep = O.preprocess_head(None, k16, v16, perm)
    vp = O.bf16_to_f32(v16)[perm]
    mu = np.repeat(O.bf16_to_f32(prep["means"]), 128, axis=0)[:1000]
    R = (vp - mu).astype(np.float32)
    bad = (mu + R) != vp
    assert bad.sum() <= 2          # only where the exponent gap exceeds 16 bits
    # the mean is the bf16 rounding of the fp32 block average (within fp32 error)
    exact = np.array([vp[t * 128:(t + 1) * 128].astype(np.float64).mean(0) for t in range(8)])
    m = O.bf16_to_f32(prep["means"]).astype(np.float64)
    assert np.all(np.abs(m - exact) <= np.abs(exact) * 2 ** -8 + 1e-6)
    # last block is partial: 1000 - 7*128 = 104 rows
    np.testing.assert_allclose(m[7], vp[896:].astype(np.float64).mean(0), rtol=2 ** -7, atol=1e-6)


def test_constant_blocks_give_zero_residual_codes():
    N = 384
    rows = _bf16_vals(np.random.default_rng(5).standard_normal((3, 128)) * 3)
    v = np.repeat(rows, 128, axis=0)
    v16 = O.bf16_round(v)
    perm = np.arange(N, dtype=np.int32)
    prep = O.preprocess_head(None, v16, v16, perm)
    np.testing.assert_array_equal(O.bf16_to_f32(prep["means"]), rows)
    assert not prep["v_codes"].any() and not prep["v_scales"].any()


def test_residual_quantisation_error_is_half_a_step():
    Q, K, V = W.custom_inputs(1, 1, 2000, seed=6)
    v16 = V[0, 0].view(dtype=__import__("torch").int16).numpy().view(np.uint16)
    perm = np.arange(2000, dtype=np.int32)
    prep = O.preprocess_head(None, v16, v16, perm)
    vp = O.bf16_to_f32(v16)
    mu = np.repeat(O.bf16_to_f32(prep["means"]), 128, axis=0)[:2000]
    R = (vp - mu).astype(np.float64)
    sv = prep["v_scales"].astype(np.float64)
    y = R / sv                                   # code units
    dec = O.e4m3_decode(prep["v_codes"][:2000])
    a = np.abs(y)
    step = np.where(a < 2 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2 ** -6))) - 3))
    assert np.all(np.abs(dec - y) <= step / 2 * (1 + 1e-6) + 1e-6)
    assert np.isclose(np.abs(y).max(axis=0), 448, rtol=1e-6).all()


def test_mean_storage_is_an_eighth_bit_per_element():
    facts = __import__("json").load(open(os.path.join(ROOT, "tests", "golden", "page_facts.json")))
    N, d = 75600, 128
    prep_bits = O.n_blocks(N) * d * 16
    assert abs(prep_bits / (N * d) - facts["mean_storage_bits_per_element"]["value"]) < 0.0002


def test_block_energy_rises_after_sorting_in_kind():
    # pages: 8% of block energy in sequence order, 36% after sorting (real heads)
    Q, K, V = W.custom_inputs(1, 1, 8192, seed=2)
    v = O.bf16_to_f32(V[0, 0].view(dtype=__import__("torch").int16).numpy().view(np.uint16))
    lab, _, _ = O.kmeans(v, 64, 8)
    seq = O.block_energy_fraction(v)
    srt = O.block_energy_fraction(v, O.stable_label_sort(lab, 64))
    assert srt > 3 * seq


def test_nvfp4_residual_within_half_step_of_group_grid():
    Q, K, V = W.custom_inputs(1, 1, 1000, seed=8)
    v16 = V[0, 0].view(dtype=__import__("torch").int16).numpy().view(np.uint16)
    perm = np.arange(1000, dtype=np.int32)
    prep = O.preprocess_head(None, v16, v16, perm, "nvfp4")
    vp = O.bf16_to_f32(v16)
    mu = np.repeat(O.bf16_to_f32(prep["means"]), 128, axis=0)[:1000]
    R = (vp - mu).astype(np.float64)
    St = float(prep["v_scales"][0])
    gs = O.e4m3_decode(np.repeat(prep["v_group_scales"], 16, axis=0)[:1000]) * St
    y = R / gs
    assert np.all(np.abs(y) <= 6 * (1 + 2 ** -3) + 1e-9)    # group scale rounding allowance
    dec = O.e2m1_decode(prep["v_nibbles"][:1000])
    a = np.minimum(np.abs(y), 6)
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    ok = (np.abs(dec - np.clip(y, -6, 6)) <= step / 2 + 1e-9)
    assert ok.mean() > 0.999
    assert prep["v_nibbles"][1000:].sum() == 0
