"""Planted mistakes in the oracle (on the CPU) must each fail a pin: evidence
that the pins constrain the oracle and do not merely restate it."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import test_oracle_expcast as TE
from tests import test_oracle_attention as TA


def test_flipped_beta_fails_the_agreement_pin(monkeypatch):
    monkeypatch.setattr(O, "EXPCAST_OFFSET", np.float32(56.35))
    with pytest.raises(AssertionError):
        TE.test_agreement_per_doubling_is_79_6_percent()


def test_wrong_code_offset_fails_the_p_equals_one_pin(monkeypatch):
    monkeypatch.setattr(O, "EXPCAST_OFFSET", np.float32(47.65))   # as if the exponent bias were 6
    with pytest.raises(AssertionError):
        TE.test_probability_one_is_the_e4m3_byte_of_one()


def test_dropped_mean_restore_fails_the_softmax_pin(monkeypatch):
    real = O.online_attention

    def no_restore(Qd, Kd, Vres, means, *a, **k):
        return real(Qd, Kd, Vres, np.zeros_like(means), *a, **k)

    monkeypatch.setattr(O, "online_attention", no_restore)
    with pytest.raises(AssertionError):
        TA.test_online_softmax_with_mean_restore_is_exact_softmax(300)


def test_ties_away_from_zero_fail_the_e4m3_pin(monkeypatch):
    real_rint = np.rint

    def round_half_away(x):
        return np.sign(x) * np.floor(np.abs(x) + 0.5)

    monkeypatch.setattr(O.np, "rint", round_half_away)
    x = np.float32([1.0625, 1.1875, 3 * 2 ** -11])          # exact ties of E4M3
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(x)
    monkeypatch.setattr(O.np, "rint", real_rint)
    assert (got != want).any()


def test_missing_running_max_rescale_fails_the_softmax_pin(monkeypatch):
    real_exp2 = np.exp2
    calls = {"n": 0}

    def stale_alpha(x, *a, **k):
        return real_exp2(x, *a, **k)

    src = O.online_attention

    def no_rescale(Qd, Kd, Vres, means, N, sq, ks, c0, p_mode, rows, record=None):
        # run block by block but never rescale the accumulators
        nb = O.n_blocks(N)
        q = Qd[rows]
        U = 0
        l = 0
        for t in range(nb):
            k0, k1 = t * 128, min(N, (t + 1) * 128)
            x = q @ Kd[k0:k1].T * float(c0)
            P = np.exp2(x - x.max(1, keepdims=True))
            l = l + P.sum(1)
            U = U + P @ Vres[k0:k1] + P.sum(1)[:, None] * means[t][None]
        return U / l[:, None]

    monkeypatch.setattr(O, "online_attention", no_rescale)
    with pytest.raises(AssertionError):
        TA.test_online_softmax_with_mean_restore_is_exact_softmax(300)


def test_swapped_butterfly_fails_the_sylvester_pin(monkeypatch):
    from tests import test_oracle_qk_transform as TQ

    def fwht_swapped(x):
        y = O.f32(x).copy()
        d = y.shape[-1]
        lead = y.shape[:-1]
        h = 1
        while h < d:
            z = y.reshape(*lead, d // (2 * h), 2, h)
            a, b = z[..., 0, :], z[..., 1, :]
            y = np.stack([O.f32(a + b), O.f32(b - a)], axis=-2).reshape(*lead, d)   # wrong sign
            h *= 2
        return y

    monkeypatch.setattr(O, "fwht_f32", fwht_swapped)
    with pytest.raises(AssertionError):
        TQ.test_fwht_matches_the_sylvester_matrix_exactly_on_integers()


def test_wrong_rotation_sense_fails_the_quarter_turn_pin(monkeypatch):
    from tests import test_oracle_qk_transform as TQ
    real = O.rope_f32

    def rope_inverse(x, cs):
        cs = np.array(cs, np.float32, copy=True)
        cs[..., 1] = -cs[..., 1]          # rotates the other way
        return real(x, cs)

    monkeypatch.setattr(O, "rope_f32", rope_inverse)
    with pytest.raises(AssertionError):
        TQ.test_rope_identity_and_quarter_turn()


# ---- the per-block Q/K quantiser and exact attention ------------------------

def _quantiser(kind):
    """_block_scaled_e4m3 with one planted mistake."""
    def q(x, N):
        d = x.shape[1]
        nb = O.n_blocks(N)
        codes = np.zeros((nb * 128, d), np.uint8)
        scales = np.zeros(nb, np.float32)
        fmax = np.float32(240.0 if kind == "fnuz_max" else 448.0)
        for t in range(nb):
            lo, hi = t * 128, min(N, (t + 1) * 128)
            if kind == "end_aligned" and hi == N:
                lo = max(0, N - 128)                      # last block taken as the final 128 rows
            blk = x[lo:hi]
            if kind == "per_row":
                amax = np.abs(blk).max(axis=1, keepdims=True).astype(np.float32)
            elif kind == "per_tensor":
                amax = np.float32(np.abs(x[:N]).max())
            else:
                amax = np.float32(np.abs(blk).max())
            amax = np.where(amax > 0, amax, np.float32(1)).astype(np.float32)
            scales[t] = np.float32(np.max(amax) / fmax)
            codes[hi - blk.shape[0]:hi] = O.e4m3_encode(O.f32(blk * O.f32(fmax / amax)))
        return codes, scales
    return q


@pytest.mark.parametrize("kind,pin", [
    ("per_row", "test_scale_is_shared_by_every_row_of_a_block"),
    ("per_tensor", "test_blocks_are_independent"),
    ("end_aligned", "test_partial_last_block_uses_its_own_rows_only"),
    ("fnuz_max", "test_block_max_maps_to_448_and_scale_times_448_is_the_block_max"),
])
def test_planted_quantiser_mistakes_fail_a_pin(monkeypatch, kind, pin):
    from tests import test_oracle_qk_quant as TQ
    monkeypatch.setattr(O, "_block_scaled_e4m3", _quantiser(kind))
    fn = getattr(TQ, pin)
    with pytest.raises(AssertionError):
        fn(300) if pin.startswith("test_block_max") else fn()


def test_q_permuted_like_k_fails_the_order_pin(monkeypatch):
    from tests import test_oracle_qk_quant as TQ
    real = O.preprocess_head

    def q_permuted(q, k, v, perm, *a, **kw):
        return real(None if q is None else q[perm], k, v, perm, *a, **kw)

    monkeypatch.setattr(O, "preprocess_head", q_permuted)
    with pytest.raises(AssertionError):
        TQ.test_q_blocks_in_original_order_k_blocks_in_permuted_order()


def test_base_two_softmax_fails_the_logistic_pin(monkeypatch):
    from tests import test_oracle_qk_quant as TQ
    monkeypatch.setattr(O.np, "exp", np.exp2)
    with pytest.raises(AssertionError):
        TQ.test_exact_attention_two_keys_is_a_logistic_mix()


def test_unscaled_scores_fail_the_brute_force_pin(monkeypatch):
    from tests import test_oracle_qk_quant as TQ
    real = O.exact_attention

    def unscaled(q, k, v, softmax_scale, rows=None):
        return real(q, k, v, 1.0, rows)

    monkeypatch.setattr(O, "exact_attention", unscaled)
    with pytest.raises(AssertionError):
        TQ.test_exact_attention_matches_explicit_loops(7, 2)


def test_nvfp4_values_with_the_next_groups_scale_fail_the_4bit_pins(monkeypatch):
    from tests import test_oracle_4bit_attention as TN
    real = O._nvfp4_encode

    def shifted(R, N):
        out = real(R, N)
        sg = np.roll(out["v_group_scales"], 1, axis=0)          # each group decoded with its neighbour's scale
        res = O.e2m1_decode(out["v_nibbles"][:N]) * O.e4m3_decode(np.repeat(sg, 16, axis=0)[:N])
        out["v_res"] = res * np.float64(out["v_scales"][0])
        return out

    monkeypatch.setattr(O, "_nvfp4_encode", shifted)
    with pytest.raises(AssertionError):
        TN.test_uniform_scores_average_the_rebuilt_values("nvfp4", "fp32_bf16")


def test_dropped_mean_restore_fails_the_4bit_dominant_key_pin(monkeypatch):
    from tests import test_oracle_4bit_attention as TN
    real = O.online_attention

    def no_restore(Qd, Kd, Vres, means, *a, **k):
        return real(Qd, Kd, Vres, np.zeros_like(means), *a, **k)

    monkeypatch.setattr(O, "online_attention", no_restore)
    with pytest.raises(AssertionError):
        TN.test_one_dominant_key_returns_its_rebuilt_value("nvfp4", "fp32_bf16")


def test_mxfp4_groups_of_consecutive_rows_fail_the_4bit_pins(monkeypatch):
    from tests import test_oracle_4bit_attention as TN
    monkeypatch.setattr(O, "mxfp4_groups", lambda Np: np.arange(Np) // 32)   # 32 consecutive rows per group
    with pytest.raises(AssertionError):
        TN.test_uniform_scores_average_the_rebuilt_values("mxfp4", "expcast")
