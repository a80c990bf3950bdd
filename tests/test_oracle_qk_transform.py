"""Pins of the oracle's Q/K transforms of the fused preprocessing: RoPE and the
Walsh-Hadamard transform (paper digest, preprocessing paragraph: RoPE, mean,
gather, Hadamard and quantisation run in one kernel; results paragraph: a
Hadamard on Q and K moves PSNR by at most 0.1-0.3 dB).

Each pin is fixed by mathematics independent of the oracle's code: an explicit
Sylvester matrix built by Kronecker products, H H = 128 I, exactness on small
integers, the rotation group's properties (identity, quarter turn, norm, and
relative-position invariance of dot products)."""
import numpy as np
import pytest

from oracle import oracle as O


def _sylvester(d):
    H = np.array([[1.0]])
    while H.shape[0] < d:
        H = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), H)
    return H


def test_fwht_matches_the_sylvester_matrix_exactly_on_integers():
    rng = np.random.default_rng(0)
    x = rng.integers(-100, 101, size=(37, 128)).astype(np.float32)
    H = _sylvester(128)
    assert np.array_equal(O.fwht_f32(x).astype(np.float64), x.astype(np.float64) @ H.T)
    # small sizes as well (index and sign order at every stage)
    for d in (2, 4, 8, 16):
        xs = rng.integers(-9, 10, size=(5, d)).astype(np.float32)
        assert np.array_equal(O.fwht_f32(xs).astype(np.float64), xs.astype(np.float64) @ _sylvester(d).T)


def test_fwht_twice_is_128_times_identity():
    rng = np.random.default_rng(1)
    x = rng.integers(-50, 51, size=(8, 128)).astype(np.float32)
    assert np.array_equal(O.fwht_f32(O.fwht_f32(x)), np.float32(128) * x)


def test_fwht_error_bound_on_reals():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-4, 4, (64, 128)))).astype(np.float32)
    ref = x.astype(np.float64) @ _sylvester(128).T
    bound = 7 * 2.0 ** -24 * np.abs(x.astype(np.float64)).sum(axis=1, keepdims=True) * 1.01
    assert np.all(np.abs(O.fwht_f32(x) - ref) <= bound)


def test_hadamard_keeps_the_scores():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((20, 128)).astype(np.float32)
    k = rng.standard_normal((30, 128)).astype(np.float32)
    qh = O.qk_transform(q, hadamard=True, k_side=False).astype(np.float64)
    kh = O.qk_transform(k, hadamard=True, k_side=True).astype(np.float64)
    exact = q.astype(np.float64) @ k.astype(np.float64).T
    assert np.max(np.abs(qh @ kh.T - exact)) < 1e-4 * np.max(np.abs(exact))


def _table(pos, base=10000.0):
    i = np.arange(64)
    ang = np.asarray(pos, np.float64)[:, None] * base ** (-2.0 * i / 128.0)[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def test_rope_identity_and_quarter_turn():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    ident = np.zeros((6, 64, 2), np.float32)
    ident[..., 0] = 1
    assert np.array_equal(O.rope_f32(x, ident), x)
    quarter = np.zeros((6, 64, 2), np.float32)
    quarter[..., 1] = 1                        # angle pi/2: (x0, x1) -> (-x1, x0)
    y = O.rope_f32(x, quarter)
    assert np.array_equal(y[:, 0::2], -x[:, 1::2]) and np.array_equal(y[:, 1::2], x[:, 0::2])


def test_rope_keeps_pair_norms_and_depends_on_relative_position():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 128)).astype(np.float32)
    k = rng.standard_normal((1, 128)).astype(np.float32)
    for m, n in ((7, 3), (1000, 990), (50, 50)):
        qm = O.rope_f32(q, _table([m])).astype(np.float64)
        kn = O.rope_f32(k, _table([n])).astype(np.float64)
        qr = O.rope_f32(q, _table([m - n])).astype(np.float64)
        assert abs((qm @ kn.T).item() - (qr @ k.astype(np.float64).T).item()) < 1e-4 * np.abs(q).sum()
        pn = qm[:, 0::2] ** 2 + qm[:, 1::2] ** 2
        pq = q[:, 0::2].astype(np.float64) ** 2 + q[:, 1::2].astype(np.float64) ** 2
        assert np.allclose(pn, pq, rtol=1e-5, atol=1e-7)


def test_preprocess_with_rope_and_hadamard_keeps_scores_within_quantisation_error():
    rng = np.random.default_rng(6)
    N = 300
    qf = rng.standard_normal((N, 128)).astype(np.float32)
    kf = rng.standard_normal((N, 128)).astype(np.float32)
    vf = rng.standard_normal((N, 128)).astype(np.float32)
    q16, k16, v16 = (O.bf16_round(a) for a in (qf, kf, vf))
    perm = rng.permutation(N).astype(np.int64)
    cs = _table(np.arange(N))
    out = O.preprocess_head(q16, k16, v16, perm, "e4m3", rope_cs=cs, hadamard=True)
    nb = O.n_blocks(N)
    qd = O.e4m3_decode(out["q_codes"][:N]) * np.repeat(out["q_scales"], 128)[:N, None]
    kd = O.e4m3_decode(out["k_codes"][:N]) * np.repeat(out["k_scales"], 128)[:N, None]
    # reference: rotate in float64, no Hadamard (it leaves dot products alone)
    def rot(x, tab):
        x = x.astype(np.float64)
        c, s = tab[..., 0].astype(np.float64), tab[..., 1].astype(np.float64)
        y = np.empty_like(x)
        y[:, 0::2] = x[:, 0::2] * c - x[:, 1::2] * s
        y[:, 1::2] = x[:, 0::2] * s + x[:, 1::2] * c
        return y
    ref = rot(O.bf16_to_f32(q16), cs) @ rot(O.bf16_to_f32(k16), cs)[perm].T
    got = qd @ kd.T
    assert nb == 3
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err < 0.1, err        # E4M3 on both operands: a few percent
    # and the same codes' scores match the untransformed path's within the same error
    out0 = O.preprocess_head(q16, k16, v16, perm, "e4m3")
    assert np.array_equal(out["v_codes"], out0["v_codes"])   # V is untouched
