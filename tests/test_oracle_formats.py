"""Pins of the oracle's number formats against independent definitions:
torch's own casts (E4M3FN, bfloat16), brute-force nearest search (E2M1) and
exact rational arithmetic (fused multiply-add)."""
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O


def _patterns_near_ties(lo_exp, hi_exp, shift):
    """float32 bit patterns around every rounding boundary of a format keeping
    (23 - shift) fewer mantissa bits, plus random mantissas, over a range of binades."""
    rng = np.random.default_rng(7)
    out = []
    for e in range(lo_exp, hi_exp + 1):
        base = np.uint32((e + 127) << 23)
        kept = np.arange(1 << (23 - shift), dtype=np.uint32) << shift if shift < 23 else np.array([0], np.uint32)
        half = np.uint32(1 << (shift - 1))
        for delta in (-1, 0, 1):
            out.append(base + kept + np.uint32(half + delta) if delta >= 0 else base + kept + half - np.uint32(1))
        out.append(base + rng.integers(0, 1 << 23, 4096, dtype=np.uint32))
    u = np.concatenate(out).astype(np.uint32)
    return np.concatenate([u, u | np.uint32(0x80000000)]).view(np.float32)


def test_e4m3_encode_matches_torch():
    # normal binades 2^-6..2^8 keep 3 mantissa bits (shift 20); subnormal range checked below
    x = _patterns_near_ties(-6, 8, 20)
    x = x[np.abs(x) <= 464.0]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(x), want)


def test_e4m3_encode_subnormals_and_tiny_match_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        (np.arange(0, 4096) * 2.0 ** -14).astype(np.float32),        # dense grid under 2^-2
        rng.uniform(-2 ** -5, 2 ** -5, 200000).astype(np.float32),
        np.float32([2 ** -10, 3 * 2 ** -11, 5 * 2 ** -11, 1e-30, -1e-30, 0.0, -0.0]),
    ])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(x), want)


def test_e4m3_saturates_and_keeps_signs():
    x = np.float32([448, 449, 463.9, 464.1, 1000, np.inf, -np.inf, -1e9, -0.0])
    assert list(O.e4m3_encode(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x80]
    assert O.e4m3_encode(np.float32([np.nan]))[0] & 0x7F == 0x7F


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    np.testing.assert_array_equal(got[~nan], want[~nan])
    # a round trip of every finite code
    fin = codes[~nan]
    np.testing.assert_array_equal(O.e4m3_encode(O.e4m3_decode(fin).astype(np.float32)), fin)


def test_bf16_round_matches_torch():
    x = _patterns_near_ties(-20, 20, 16)
    rng = np.random.default_rng(3)
    x = np.concatenate([x, rng.standard_normal(500000).astype(np.float32) * 30,
                        np.float32([3.4e38, -3.4e38, 1e-40, -1e-42, 0.0, -0.0, np.inf])])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.bf16_round(x), want)


def test_e2m1_encode_is_nearest_even_on_grid():
    grid = O.E2M1_GRID
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-8, 8, 20000), np.arange(-700, 701) / 100.0,
                        (grid[:-1] + grid[1:]) / 2, -(grid[:-1] + grid[1:]) / 2]).astype(np.float32)
    got = O.e2m1_encode(x)
    for xi, gi in zip(x, got):
        a = min(abs(float(xi)), 6.0)
        dist = np.abs(grid - a)
        cand = np.flatnonzero(dist == dist.min())
        idx = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
        assert int(gi) & 7 == idx, (xi, gi)
        if xi != 0:
            assert bool(int(gi) & 8) == (xi < 0)
    np.testing.assert_array_equal(O.e2m1_decode(np.arange(8)), grid)


def _exact_fma_f32(a, b, c):
    v = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    # round the exact value to float32, ties to even, via neighbours
    f = np.float32(float(v))
    lo, hi = (np.nextafter(f, np.float32(-np.inf)), f) if Fraction(float(f)) > v else (f, np.nextafter(f, np.float32(np.inf)))
    dl, dh = v - Fraction(float(lo)), Fraction(float(hi)) - v
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if (np.float32(lo).view(np.uint32) & 1) == 0 else hi


def test_fma_f32_is_one_rounding():
    rng = random.Random(11)
    cases = []
    for _ in range(3000):
        a = np.float32(rng.uniform(-100, 100))
        b = np.float32(rng.uniform(-100, 100))
        c = np.float32(-float(a) * float(b) + rng.uniform(-1e-3, 1e-3))   # heavy cancellation
        cases.append((a, b, c))
    for _ in range(3000):
        cases.append(tuple(np.float32(rng.uniform(-60, 60)) for _ in range(3)))
    # products landing exactly on float32 half-ulps
    cases += [(np.float32(1 + 2 ** -12), np.float32(1 + 2 ** -12), np.float32(-1.0)),
              (np.float32(1 + 2 ** -23), np.float32(1 - 2 ** -23), np.float32(0.0))]
    a, b, c = (np.array(v, np.float32) for v in zip(*cases))
    got = O.fma_f32(a, b, c)
    for i in range(len(cases)):
        assert got[i] == _exact_fma_f32(a[i], b[i], c[i]), cases[i]


# ---- MXFP4 residual (E2M1 values, E8M0 scale per 32) -------------------------

def test_mxfp4_groups_are_the_lane_sets_of_32():
    g = O.mxfp4_groups(256)
    assert np.bincount(g).tolist() == [32] * 8
    blk = g[:128]
    assert set(np.nonzero(blk == 0)[0]) == set(range(0, 16)) | set(range(32, 48))
    assert set(np.nonzero(blk == 1)[0]) == set(range(16, 32)) | set(range(48, 64))
    assert set(np.nonzero(blk == 2)[0]) == set(range(64, 80)) | set(range(96, 112))
    assert set(np.nonzero(blk == 3)[0]) == set(range(80, 96)) | set(range(112, 128))
    assert np.array_equal(g[128:], g[:128] + 4)


def _one_group(vals, d=1):
    """A 128-row residual whose group 0 (rows 0..15, 32..47) holds vals."""
    R = np.zeros((128, d), np.float32)
    rows = list(range(16)) + list(range(32, 48))
    R[rows[:len(vals)], 0] = vals
    return R


@pytest.mark.parametrize("amax,code", [(6.0, 127), (7.9, 127), (8.0, 128), (0.75, 124), (1.0, 125),
                                       (2.0 ** -20, 105), (448.0, 133)])
def test_mxfp4_scale_is_floor_log2_minus_two(amax, code):
    out = O._mxfp4_encode(_one_group([amax, -amax / 3]), 128)
    assert int(out["v_mx_scales"][0, 0, 0, 0]) == code
    # the other groups of the block are empty: code 0, zero values
    assert not out["v_mx_scales"][0, 1].any() and not out["v_mx_scales"][0, 0, 1].any()


def test_mxfp4_saturates_and_round_trips_the_grid():
    X = 2.0 ** -3                              # amax 0.75 -> scale 2^-3
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    vals = np.concatenate([grid * X, -grid[1:] * X, [0.75]]).astype(np.float32)
    out = O._mxfp4_encode(_one_group(vals), 128)
    rows = list(range(16)) + list(range(32, 48))
    got = out["v_res"][rows[:len(vals)], 0]
    assert np.array_equal(got, vals.astype(np.float64))
    # 7.9 with scale 1 saturates to 6
    sat = O._mxfp4_encode(_one_group([7.9]), 128)
    assert sat["v_res"][0, 0] == 6.0


def test_mxfp4_matches_brute_force_nearest_even():
    rng = np.random.default_rng(3)
    N = 200
    R = (rng.standard_normal((N, 4)) * np.exp(rng.uniform(-3, 3, (1, 4)))).astype(np.float32)
    out = O._mxfp4_encode(R, N)
    gid = O.mxfp4_groups(256)[:N]
    codes = out["v_mx_scales"].reshape(-1, 4)          # [4 nb, d] in index 4t + 2h + g
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    for j in range(N):
        for c in range(4):
            X = 2.0 ** (int(codes[gid[j], c]) - 127)
            a = abs(float(R[j, c])) / X
            dist = np.abs(grid - min(a, 6.0))
            best = np.nonzero(dist == dist.min())[0]
            k = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]   # ties to the even code
            want = np.copysign(grid[k] * X, R[j, c]) if grid[k] > 0 else 0.0
            assert out["v_res"][j, c] == want or (want == 0 and out["v_res"][j, c] == 0)
    # and every group's scale code is floor(log2 amax) - 2 + 127
    amax = np.zeros((8, 4))
    np.maximum.at(amax, gid, np.abs(R.astype(np.float64)))
    for q in range(8):
        for c in range(4):
            if amax[q, c] > 0:
                assert int(codes[q, c]) == int(np.floor(np.log2(amax[q, c]))) - 2 + 127
