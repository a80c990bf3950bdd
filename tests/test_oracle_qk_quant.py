"""Pins of the oracle's per-128-row-block E4M3 quantiser of Q and K and of its
exact attention (the fidelity yardstick), against properties the reading fixes
and against brute force.

The pages leave the Q/K scheme to prior methods (insight article, section
"Value Is the Error Source Earlier Methods Underestimated"); the reading is one
scale per 128-row block, s = amax/448, codes E4M3(x * 448/amax), Q blocks in
original order, K blocks in permuted order.  Each pin below is chosen so that a
plausible mistake fails it: a per-row or per-tensor scale, a wrong format
maximum, a last block aligned to the end of the sequence instead of to the
128-row grid, or Q and K taking each other's order.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
import vc_workloads as W

SCALE = 1.0 / math.sqrt(128.0)


def _u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _blocks(N, seed, d=128):
    """float32 [N, d] with block magnitudes spread over six binades and distinct values."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, d)).astype(np.float32)
    for t in range(O.n_blocks(N)):
        x[t * 128:(t + 1) * 128] *= np.float32(2.0 ** rng.uniform(-3, 3))
    return x


def _torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("N", [128, 300, 1000, 1024])
def test_block_max_maps_to_448_and_scale_times_448_is_the_block_max(N):
    x = _blocks(N, N)
    codes, s = O._block_scaled_e4m3(x, N)
    assert codes.shape == (O.n_blocks(N) * 128, 128) and s.shape == (O.n_blocks(N),)
    for t in range(O.n_blocks(N)):
        blk = x[t * 128:min(N, (t + 1) * 128)]
        amax = float(np.abs(blk).max())
        # 448 * s is the block's own largest magnitude (one fp32 division apart)
        assert abs(448.0 * float(s[t]) - amax) <= amax * 2.0 ** -23
        # the element holding that magnitude is coded +-448 (0x7E / 0xFE)
        r, c = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
        assert codes[t * 128 + r, c] & 0x7F == 0x7E


def test_every_code_is_the_e4m3_rounding_of_the_scaled_value():
    # the encoder itself is pinned to torch; here: codes = E4M3(x * fl(448/amax)) per block
    N = 700
    x = _blocks(N, 3)
    codes, s = O._block_scaled_e4m3(x, N)
    for t in range(O.n_blocks(N)):
        blk = x[t * 128:min(N, (t + 1) * 128)]
        inv = np.float32(448.0) / np.float32(np.abs(blk).max())
        np.testing.assert_array_equal(codes[t * 128:t * 128 + blk.shape[0]], _torch_e4m3(blk * inv))


def test_scale_is_shared_by_every_row_of_a_block():
    # row 0 holds the block max; row 1 is 64x smaller: with one scale per block
    # its largest code decodes to 448/64 = 7, with one scale per row it would be 448
    x = np.zeros((128, 128), np.float32)
    x[0, 5] = 64.0
    x[1, 9] = -1.0
    x[2:, :] = np.float32(0.25)
    codes, s = O._block_scaled_e4m3(x, 128)
    dec = O.e4m3_decode(codes)
    assert dec[0, 5] == 448.0 and dec[1, 9] == -7.0 and np.all(dec[2:] == 1.75)
    assert float(s[0]) == np.float32(64.0) / np.float32(448.0)
    # only the rows holding the block maximum reach the format maximum
    x2 = _blocks(1000, 9)
    c2, _ = O._block_scaled_e4m3(x2, 1000)
    for t in range(8):
        rows = np.abs(x2[t * 128:min(1000, (t + 1) * 128)])
        at448 = np.nonzero((c2[t * 128:t * 128 + rows.shape[0]] & 0x7F).max(axis=1) == 0x7E)[0]
        assert set(at448) <= set(np.nonzero(rows.max(axis=1) >= rows.max() * (1 - 2.0 ** -4))[0])


def test_blocks_are_independent():
    # scaling one block by a power of two moves only that block's scale
    N = 600
    x = _blocks(N, 4)
    c0, s0 = O._block_scaled_e4m3(x, N)
    y = x.copy()
    y[128:256] *= np.float32(8.0)
    c1, s1 = O._block_scaled_e4m3(y, N)
    np.testing.assert_array_equal(c1, c0)
    assert s1[1] == np.float32(s0[1] * np.float32(8.0))
    np.testing.assert_array_equal(np.delete(s1, 1), np.delete(s0, 1))


def test_partial_last_block_uses_its_own_rows_only():
    # N = 300: the last block holds rows 256..299 (44 rows) on the 128-row grid
    N = 300
    x = _blocks(N, 5)
    x[200, 7] = np.float32(1000.0)       # block 1's max, far above everything else
    x[299, 3] = np.float32(-3.0)
    x[256:299] = np.clip(x[256:299], -2.0, 2.0)
    codes, s = O._block_scaled_e4m3(x, N)
    assert float(s[2]) == np.float32(3.0) / np.float32(448.0)       # not 1000/448
    assert codes[299, 3] == 0xFE                                       # -448
    assert not codes[N:].any()                                          # padding rows are zero bytes
    assert float(s[1]) == np.float32(1000.0) / np.float32(448.0)


def test_zero_block_gives_zero_scale_and_zero_codes():
    N = 384
    x = _blocks(N, 6)
    x[128:256] = 0.0
    codes, s = O._block_scaled_e4m3(x, N)
    assert s[1] == 0.0 and not codes[128:256].any()
    assert np.all(np.isfinite(s)) and s[0] > 0 and s[2] > 0


def test_q_blocks_in_original_order_k_blocks_in_permuted_order():
    N = 512
    Q, K, V = W.custom_inputs(1, 1, N, seed=12)
    q, k, v = _u16(Q[0, 0]), _u16(K[0, 0]), _u16(V[0, 0])
    kf = O.bf16_to_f32(k).copy()
    qf = O.bf16_to_f32(q)
    # a permutation that sends original block 0 to permuted block 3
    perm = np.concatenate([np.arange(128, 512), np.arange(0, 128)]).astype(np.int32)
    pr = O.preprocess_head(q, k, v, perm)
    for t in range(4):
        qa = float(np.abs(qf[t * 128:(t + 1) * 128]).max())
        ka = float(np.abs(kf[perm[t * 128:(t + 1) * 128]]).max())
        assert abs(448.0 * float(pr["q_scales"][t]) - qa) <= qa * 2.0 ** -23
        assert abs(448.0 * float(pr["k_scales"][t]) - ka) <= ka * 2.0 ** -23
    # K row j of permuted block 3 is original row j of block 0, coded with block 3's scale
    inv = np.float32(448.0) / np.float32(np.abs(kf[0:128]).max())
    np.testing.assert_array_equal(pr["k_codes"][384:512], _torch_e4m3(kf[0:128] * inv))
    # Q is not permuted
    invq = np.float32(448.0) / np.float32(np.abs(qf[0:128]).max())
    np.testing.assert_array_equal(pr["q_codes"][0:128], _torch_e4m3(qf[0:128] * invq))


# ---- exact attention ---------------------------------------------------------

def _brute_attention(q, k, v, scale):
    """softmax(q k^T * scale) v by explicit loops with math.exp (tiny inputs only)."""
    n, d = len(q), len(q[0])
    out = []
    for i in range(n):
        s = [sum(float(q[i][c]) * float(k[j][c]) for c in range(d)) * scale for j in range(n)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        out.append([sum(w[j] * float(v[j][c]) for j in range(n)) / z for c in range(d)])
    return np.array(out)


@pytest.mark.parametrize("N,seed", [(1, 0), (3, 1), (7, 2)])
def test_exact_attention_matches_explicit_loops(N, seed):
    Q, K, V = W.custom_inputs(1, 1, N, seed=seed, recipe="qk_outlier")
    q, k, v = _u16(Q[0, 0]), _u16(K[0, 0]), _u16(V[0, 0])
    got = O.exact_attention(q, k, v, SCALE)
    want = _brute_attention(O.bf16_to_f32(q), O.bf16_to_f32(k), O.bf16_to_f32(v), float(np.float32(SCALE)))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_exact_attention_two_keys_is_a_logistic_mix():
    # q = a e0, k_0 = 0, k_1 = b e0: the weight of v_1 is 1 / (1 + exp(-a b scale))
    a, b = 3.0, 2.5
    q = np.zeros((1, 128), np.float32)
    q[0, 0] = a
    k = np.zeros((2, 128), np.float32)
    k[1, 0] = b
    v = np.zeros((2, 128), np.float32)
    v[0, :] = 1.0
    v[1, :] = -2.0
    got = O.exact_attention(O.bf16_round(q), O.bf16_round(k), O.bf16_round(v), SCALE)
    w1 = 1.0 / (1.0 + math.exp(-a * b * float(np.float32(SCALE))))
    np.testing.assert_allclose(got[0], (1 - w1) * 1.0 + w1 * -2.0, rtol=1e-14)


def test_exact_attention_zero_query_averages_the_values():
    Q, K, V = W.custom_inputs(1, 1, 50, seed=8)
    q = np.zeros((4, 128), np.uint16)
    k, v = _u16(K[0, 0]), _u16(V[0, 0])
    got = O.exact_attention(q, k, v, SCALE)
    np.testing.assert_allclose(got, np.tile(O.bf16_to_f32(v).astype(np.float64).mean(0), (4, 1)), rtol=1e-13,
                               atol=1e-13)


def test_exact_attention_rows_subset_equals_full():
    Q, K, V = W.custom_inputs(1, 1, 90, seed=10)
    q, k, v = _u16(Q[0, 0]), _u16(K[0, 0]), _u16(V[0, 0])
    full = O.exact_attention(q, k, v, SCALE)
    rows = np.array([0, 17, 89])
    np.testing.assert_allclose(O.exact_attention(q, k, v, SCALE, rows=rows), full[rows], rtol=1e-12, atol=1e-14)
