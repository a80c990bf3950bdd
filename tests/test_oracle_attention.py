"""Pins of the oracle's attention: the blockwise online softmax with mean
restore equals brute-force softmax when nothing is quantised, exact attention
is invariant under a joint K/V permutation, the mean restore is exact algebra,
and the quantised VC path stays close to exact attention."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
import vc_workloads as W

SCALE = 1.0 / np.sqrt(128.0)


def _u16(t):
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("N", [1, 77, 128, 300, 1024])
def test_online_softmax_with_mean_restore_is_exact_softmax(N):
    rng = np.random.default_rng(N)
    d = 128
    Q = rng.standard_normal((N, d))
    K = rng.standard_normal((N, d)) * 2
    V = rng.standard_normal((N, d)) + 5
    nb = O.n_blocks(N)
    # arbitrary per-block "means": restore must add them back exactly
    means = rng.standard_normal((nb, d)) * 3
    Vres = V - np.repeat(means, 128, axis=0)[:N]
    out = O.online_attention(Q, K, Vres, means, N, np.ones(N, np.float32), np.ones(nb, np.float32),
                             np.float32(1.0), "exact", np.arange(N))
    S = Q @ K.T * float(np.float32(1.0)) * np.log(2.0)      # log2 units -> natural
    P = np.exp(S - S.max(1, keepdims=True))
    want = P @ V / P.sum(1, keepdims=True)
    np.testing.assert_allclose(out, want, rtol=1e-10, atol=1e-10)


def test_exact_attention_is_invariant_under_joint_kv_permutation():
    Q, K, V = W.custom_inputs(1, 1, 700, seed=1)
    q, k, v = _u16(Q[0, 0]), _u16(K[0, 0]), _u16(V[0, 0])
    base = O.exact_attention(q, k, v, SCALE)
    pi = np.random.default_rng(3).permutation(700)
    np.testing.assert_allclose(O.exact_attention(q, k[pi], v[pi], SCALE), base, rtol=1e-12, atol=1e-12)
    lab, _, _ = O.kmeans(O.bf16_to_f32(v), 16, 5)
    pk = O.stable_label_sort(lab, 16)
    np.testing.assert_allclose(O.exact_attention(q, k[pk], v[pk], SCALE), base, rtol=1e-12, atol=1e-12)


def test_mean_restore_identity():
    rng = np.random.default_rng(4)
    P = np.abs(rng.standard_normal((16, 128)))
    mu = rng.standard_normal(128)
    V = rng.standard_normal((128, 128)) + mu
    R = V - mu
    np.testing.assert_allclose(P.sum(1)[:, None] * mu[None] + P @ R, P @ V, rtol=1e-12, atol=1e-12)


def _prep_cfg(N, H=1, seed=0, recipe="gauss", k=8, iters=10, fmt="e4m3"):
    Q, K, V = W.custom_inputs(1, H, N, seed=seed, recipe=recipe)
    q, kk, v = _u16(Q), _u16(K), _u16(V)
    perm, _, _ = O.vsmooth_group(v, k, iters)
    preps = O.preprocess(q, kk, v, perm, fmt)
    return q, kk, v, perm, preps


def test_vc_attention_close_to_exact_and_better_than_sequence_order():
    q, k, v, perm, preps = _prep_cfg(1024, seed=0)
    out = O.vc_attention_head(preps[0][0], SCALE, "expcast")
    ex = O.exact_attention(q[0, 0], k[0, 0], v[0, 0], SCALE)
    err = O.rel_l2(out, ex)
    assert err < 0.15
    conv = O.vc_attention_head(preps[0][0], SCALE, "fp32exp_e4m3")
    assert O.rel_l2(conv, ex) < err + 0.02


def test_constant_blocks_reduce_to_mean_only_formula():
    N = 256
    rng = np.random.default_rng(6)
    rows = O.bf16_round(rng.standard_normal((2, 128)).astype(np.float32) * 4)
    v = np.repeat(rows, 128, axis=0)
    Q, K, _ = W.custom_inputs(1, 1, N, seed=6)
    q, k = _u16(Q[0, 0]), _u16(K[0, 0])
    prep = O.preprocess_head(q, k, v, np.arange(N, dtype=np.int32))
    rec = []
    out = O.vc_attention_head(prep, SCALE, "expcast", record=rec)
    P = np.concatenate([O.e4m3_decode(r["codes"]) for r in rec], axis=1)
    # rescale each tile's P to the final running max
    mx_final = rec[-1]["mx"].astype(np.float64)
    w = np.concatenate([np.repeat(np.exp2(r["mx"].astype(np.float64) - mx_final)[:, None], 128, 1) for r in rec], 1)
    Pw = P * w
    mu = O.bf16_to_f32(rows).astype(np.float64)
    s = np.stack([Pw[:, :128].sum(1), Pw[:, 128:].sum(1)], 1)
    want = (s @ mu) / s.sum(1, keepdims=True)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)


def test_expcast_replay_given_scores_matches_the_pipeline():
    q, k, v, perm, preps = _prep_cfg(600, seed=3)
    rec = []
    O.vc_attention_head(preps[0][0], SCALE, "expcast", record=rec)
    S_tiles = [np.pad(r["S"], ((0, 0), (0, 128 - r["S"].shape[1]))) for r in rec]
    replay = O.expcast_given_scores(S_tiles, [r["kap"] for r in rec], 600)
    for r, c in zip(rec, replay):
        np.testing.assert_array_equal(c[:, :r["codes"].shape[1]], r["codes"])


def test_score_scale_constant():
    assert np.float32(O.score_scale(1 / np.sqrt(128))).view(np.uint32) == 0x3E0293EE
    assert np.float32(O.EXPCAST_OFFSET).view(np.uint32) == 0x425E999A


def test_nvfp4_path_runs_and_tracks_exact():
    q, k, v, perm, preps = _prep_cfg(1000, seed=4, recipe="clustered", k=16, iters=4, fmt="nvfp4")
    out = O.vc_attention_head(preps[0][0], SCALE, "fp32_bf16")
    ex = O.exact_attention(q[0, 0], k[0, 0], v[0, 0], SCALE)
    assert O.rel_l2(out, ex) < 0.2


def test_replay_with_given_scores_equals_computed_scores():
    q, k, v, perm, preps = _prep_cfg(400, seed=7)
    pr = preps[0][0]
    rec = []
    base = O.vc_attention_head(pr, SCALE, "expcast", record=rec)
    S = np.concatenate([np.pad(r["S"], ((0, 0), (0, 128 - r["S"].shape[1]))) for r in rec], axis=1)
    np.testing.assert_array_equal(O.vc_attention_head(pr, SCALE, "expcast", scores=S), base)
