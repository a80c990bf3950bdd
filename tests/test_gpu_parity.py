"""GPU parity: every entry point of libvc.so against the CPU oracle, element by
element, on seeded inputs (tiny configuration, the ExpCast ablation, ragged and
degenerate shapes, and sampled outputs of the full Wan2.2-shaped run).

Bar: bit-exact for labels, permutations, means, scales and every code byte.
The FP8 matrix instructions do not return the exactly rounded dot product (each
group of 8 products keeps 13 bits below its largest exponent; see
test_gpu_device_facts.py), so the kernel's scores differ from the oracle's
exact ones by up to 2^-10 of the sum of |products| (measured: 1e-5 to 5e-4).
Hence the P contract: P bit-exact GIVEN the kernel's scores (ExpCast; the
exp2 paths within one step at a rate <= 1e-4), and the output within relative
L2 1e-4 of the oracle replayed on those scores.

End to end against the exact-score oracle the score differences flip about one
P code in 5,000-50,000 (never by more than one step), and the benchmark spec bar of
rel-L2 <= 1e-3 holds on the Wan2.2 shape (measured 1.6e-4 to 1.8e-4) and on the
ragged 4-bit workload (3.4e-5 to 3.5e-5) but NOT on the N(0,1) / outlier Q,K
shapes of the tiny and ExpCast-ablation workloads (measured 1.1e-3 to 3.2e-3:
near-uniform attention rows whose output is much smaller than V, so a few
flipped codes show).  Those are held to 6e-3 end to end and to the given-S bar
above, and the mismatch rates are printed."""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
import vc_workloads as W

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128.0)
TOL_OUT = 1e-3          # output vs the exact-score oracle (the parity bar for fp32 outputs)
TOL_GIVEN_S = 1e-4      # output vs the oracle replayed on the kernel's own scores
TOL_GAUSS_QK = 6e-3     # output vs the exact-score oracle on N(0,1) / outlier Q,K
S_ERR_L1 = 2.0 ** -10   # |S - exact| <= 2^-10 * sum_c |q_c k_c| (FP8 MFMA accumulation)


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def vc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_attention_video_vc_amd as vc
    vc.lib()
    return vc


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _run_all(vc, Q, K, V, k, iters, fmt="e4m3"):
    dev = torch.device("cuda:0")
    Qd, Kd, Vd = (t.to(dev) for t in (Q, K, V))
    perm, labels, cents = vc.vsmooth_group(Vd, k, iters, want_labels=True, want_centroids=True)
    prep = vc.preprocess_quant(Qd, Kd, Vd, perm, fmt)
    torch.cuda.synchronize()
    return Qd, Kd, Vd, perm, labels, cents, prep


def _check_group_and_codes(vc, Q, K, V, k, iters, heads=None, fmt="e4m3"):
    """Runs the GPU grouping + preprocessing and checks the listed heads bit for bit."""
    Qd, Kd, Vd, perm, labels, cents, prep = _run_all(vc, Q, K, V, k, iters, fmt)
    B, H, N, _ = Q.shape
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    q16, k16, v16 = _u16(Q), _u16(K), _u16(V)
    perm_c, lab_c, cent_c = perm.cpu().numpy(), labels.cpu().numpy(), cents.cpu().numpy()
    vcodes = (vc.unswizzle_v_codes(prep["v_codes"], N) if fmt == "e4m3" else prep["v_codes"]).cpu().numpy()
    preps = {}
    for (b, h) in heads:
        lab, cen, _ = O.kmeans(O.bf16_to_f32(v16[b, h]), k, iters)
        np.testing.assert_array_equal(lab_c[b, h], lab, err_msg=f"labels b{b} h{h}")
        np.testing.assert_array_equal(cent_c[b, h], cen, err_msg=f"centroids b{b} h{h}")
        pm = O.stable_label_sort(lab, k)
        np.testing.assert_array_equal(perm_c[b, h], pm, err_msg=f"perm b{b} h{h}")
        pr = O.preprocess_head(q16[b, h], k16[b, h], v16[b, h], pm, fmt)
        np.testing.assert_array_equal(_u16(prep["v_means"][b, h]), pr["means"], err_msg="means")
        np.testing.assert_array_equal(prep["k_codes"][b, h].cpu().numpy(), pr["k_codes"], err_msg="k codes")
        np.testing.assert_array_equal(prep["k_scales"][b, h].cpu().numpy(), pr["k_scales"], err_msg="k scales")
        np.testing.assert_array_equal(prep["q_codes"][b, h].cpu().numpy(), pr["q_codes"], err_msg="q codes")
        np.testing.assert_array_equal(prep["q_scales"][b, h].cpu().numpy(), pr["q_scales"], err_msg="q scales")
        if fmt == "e4m3":
            np.testing.assert_array_equal(vcodes[b, h], pr["v_codes"], err_msg="v codes")
            np.testing.assert_array_equal(prep["v_scales"][b, h].cpu().numpy(), pr["v_scales"], err_msg="v scales")
        else:
            nib = vcodes[b, h]                                  # [nb, 128, 64] packed along rows
            lo, hi = nib & 15, nib >> 4
            rows = np.stack([lo, hi], axis=-1).reshape(nib.shape[0], 128, 128)   # [nb, ch, row]
            rows = rows.transpose(0, 2, 1).reshape(-1, 128)
            np.testing.assert_array_equal(rows, pr["v_nibbles"], err_msg="nvfp4 nibbles")
            np.testing.assert_array_equal(prep["v_group_scales"][b, h].cpu().numpy(), pr["v_group_scales"],
                                          err_msg="nvfp4 group scales")
            np.testing.assert_array_equal(prep["v_scales"][b, h].cpu().numpy(), pr["v_scales"][0],
                                          err_msg="nvfp4 St")
        preps[(b, h)] = pr
    return prep, preps, (Qd, Kd, Vd)


def _check_attention(vc, prep, preps, p_mode, rows_per_head=None, tol=TOL_OUT):
    """End to end: kernel output vs the oracle with exact scores."""
    out = vc.attn_fp8_fwd(prep, SCALE, p_mode).cpu().numpy()
    errs = []
    for (b, h), pr in preps.items():
        N = pr["N"]
        rows = np.arange(N) if rows_per_head is None else rows_per_head
        ref = O.vc_attention_head(pr, SCALE, p_mode, rows=rows)
        e = O.rel_l2(out[b, h][rows], ref)
        errs.append(e)
        _say(f"  b{b} h{h} {p_mode}: output rel-L2 vs exact-score oracle {e:.2e}")
        assert e <= tol, f"rel-L2 {e:.2e} vs oracle, b{b} h{h} {p_mode}"
    return out, max(errs)


def _head_prep(prep, b, h):
    """The preprocessed tensors of one (batch, head) as a B = H = 1 problem
    (views into the same memory), so that a score dump holds one head only."""
    sub = dict(prep, B=1, H=1)
    for k, v in prep.items():
        if isinstance(v, torch.Tensor):
            sub[k] = v[b:b + 1, h:h + 1]
    return sub


def _p_steps(got, want, p_mode):
    """Distance in format steps between two P tiles: E4M3 codes are positive
    bytes whose integer order is the value order; bf16 P bits likewise."""
    return np.abs(got.astype(np.int64) - want.astype(np.int64))


def _check_given_scores(vc, prep, preps, p_mode, rows=None, report_e2e=False):
    """Dump the kernel's scores and P values (vc_attn_fwd_dump): P bit-exact
    given S for ExpCast (one fmaf and a rounding), within one step for the paths
    through the hardware exp2 (within 1 ulp of exp2); scores within the FP8
    accumulation bound; output equal to the oracle replayed on S (rel-L2 1e-4).
    With report_e2e, also the end-to-end P mismatch against the exact-score
    oracle: rate, largest step, and flips across the flush boundary
    (a code 8 on one side and 0 on the other).  Returns the per-head stats."""
    stats = {}
    for (b, h), pr in preps.items():
        out, S, P = vc.attn_fwd_dump(_head_prep(prep, b, h), SCALE, p_mode)
        torch.cuda.synchronize()
        N = pr["N"]
        nb = O.n_blocks(N)
        Np = nb * 128
        rws = np.arange(N) if rows is None else np.asarray(rows)
        ridx = torch.from_numpy(rws).to(S.device)
        S_rows = S[0, 0].index_select(0, ridx).cpu().numpy()
        P_rows = P[0, 0].index_select(0, ridx).cpu().numpy()
        if p_mode == "fp32_bf16":
            P_rows = P_rows.view(np.uint16)
        out_rows = out[0, 0].index_select(0, ridx).cpu().numpy()
        del out, S, P
        S_full = np.zeros((N, Np), np.float32)      # untouched pages stay unallocated
        S_full[rws] = S_rows
        rec = []
        ref_s = O.vc_attention_head(pr, SCALE, p_mode, rows=rws, scores=S_full, record=rec)
        off = 0
        for t, r in enumerate(rec):
            k1 = r["codes"].shape[1]
            got = P_rows[:, t * 128:t * 128 + k1]
            if p_mode == "expcast":   # one fmaf + RNE: bit-exact given S
                np.testing.assert_array_equal(got, r["codes"], err_msg=f"P given S, b{b} h{h} tile {t}")
            else:                     # hardware exp2 is within 1 ulp: P may move one step at boundaries
                d = _p_steps(got, r["codes"], p_mode)
                assert d.max() <= 1, f"P given S off by {d.max()} steps, b{b} h{h} tile {t}"
                off += int((d > 0).sum())
            assert not P_rows[:, t * 128 + k1:(t + 1) * 128].any()
        if p_mode != "expcast":
            rate = off / float(len(rws) * N)
            _say(f"  b{b} h{h} {p_mode}: P off by one step given S: rate {rate:.1e}")
            assert rate <= 1e-4
        Qd = O.e4m3_decode(pr["q_codes"][rws])
        Kd = O.e4m3_decode(pr["k_codes"][:N])
        exact = Qd @ Kd.T
        l1 = np.abs(Qd) @ np.abs(Kd).T
        dS = np.abs(S_rows[:, :N].astype(np.float64) - exact)
        worst = float((dS / np.maximum(l1, 1e-30)).max())
        rne = float((S_rows[:, :N] == exact.astype(np.float32)).mean())
        _say(f"  b{b} h{h} {p_mode}: max |S - exact| / L1 = {worst:.2e}; S == RNE(exact) on {rne:.4f}")
        assert worst <= S_ERR_L1
        e = O.rel_l2(out_rows, ref_s)
        _say(f"  b{b} h{h} {p_mode}: output rel-L2 vs oracle on the kernel's scores {e:.2e}")
        assert e <= TOL_GIVEN_S
        assert np.isfinite(out_rows).all()
        st = dict(replay_rel_l2=e, s_err_l1=worst, s_rne_frac=rne)
        if report_e2e:
            rec_x = []
            ref_x = O.vc_attention_head(pr, SCALE, p_mode, rows=rws, record=rec_x)
            n_diff = n_flush = 0
            dmax = 0
            for t, r in enumerate(rec_x):
                k1 = r["codes"].shape[1]
                got = P_rows[:, t * 128:t * 128 + k1]
                d = _p_steps(got, r["codes"], p_mode)
                if p_mode != "fp32_bf16":
                    fl = ((got == 0) & (r["codes"] >= 8)) | ((got >= 8) & (r["codes"] == 0))
                    n_flush += int(fl.sum())
                    d = np.where(fl, 0, d)
                n_diff += int((d > 0).sum())
                dmax = max(dmax, int(d.max()))
            tot = float(len(rws) * N)
            e2e = O.rel_l2(out_rows, ref_x)
            _say(f"  b{b} h{h} {p_mode}: end to end vs exact-score oracle: P differs on {n_diff / tot:.2e} "
                 f"(max {dmax} step), flush-boundary flips {n_flush / tot:.2e}, output rel-L2 {e2e:.2e}")
            assert dmax <= 1
            st.update(p_mismatch=n_diff / tot, flush_flips=n_flush / tot, e2e_rel_l2=e2e)
        stats[(b, h)] = st
    return stats


def test_tiny_8bit_end_to_end(vc):
    _say("tiny 8-bit: B1 H2 N1024 k8 T10, E4M3 + ExpCast")
    c = W.WORKLOADS["tiny-8bit"]
    Q, K, V = W.make_inputs("tiny-8bit")
    prep, preps, _ = _check_group_and_codes(vc, Q, K, V, c["k"], c["iters"])
    _check_given_scores(vc, prep, preps, "expcast", report_e2e=True)
    _check_given_scores(vc, prep, preps, "fp32exp_e4m3", report_e2e=True)
    _check_attention(vc, prep, preps, "expcast", tol=TOL_GAUSS_QK)


def test_expcast_ablation_both_p_paths(vc):
    """The ExpCast ablation at its full shape (B1 H8 N8192, k32 T10, one cached
    permutation for both P paths): codes of two heads in full, then on 227
    sampled query rows of each the P bytes given the kernel's scores, the
    output replayed on those scores, and the end-to-end P mismatch and output
    error against the exact-score oracle."""
    _say("ExpCast ablation: B1 H8 N8192 k32 T10, conventional and ExpCast P paths")
    c = W.WORKLOADS["expcast-ablation"]
    Q, K, V = W.make_inputs("expcast-ablation")
    heads = [(0, 0), (0, 5)]
    prep, preps, _ = _check_group_and_codes(vc, Q, K, V, c["k"], c["iters"], heads=heads)
    rows = np.concatenate([np.arange(0, 8192, 61), np.arange(8100, 8192)])
    _check_attention(vc, prep, preps, "fp32exp_e4m3", rows, tol=TOL_GAUSS_QK)
    _check_attention(vc, prep, preps, "expcast", rows, tol=TOL_GAUSS_QK)
    _check_given_scores(vc, prep, preps, "expcast", rows, report_e2e=True)
    _check_given_scores(vc, prep, preps, "fp32exp_e4m3", rows, report_e2e=True)


def test_expcast_ablation_recipe_given_scores(vc):
    _say("ExpCast-ablation recipe at N=2048, H=2: scores and P bytes dumped")
    Q, K, V = W.custom_inputs(1, 2, 2048, seed=1, recipe="qk_outlier")
    prep, preps, _ = _check_group_and_codes(vc, Q, K, V, 32, 10)
    _check_given_scores(vc, prep, preps, "expcast")
    _check_given_scores(vc, prep, preps, "fp32exp_e4m3")


# block counts 1..8 cover every fill of the attention kernel's four-block
# mean-restore batches (nb = 5: one full batch and one block; nb = 6, 8 ...)
@pytest.mark.parametrize("B,H,N,k,iters", [(1, 3, 1000, 8, 4), (2, 1, 129, 3, 2), (1, 1, 1, 1, 1),
                                           (1, 2, 127, 5, 3), (1, 1, 300, 256, 2), (1, 1, 700, 100, 3),
                                           (1, 2, 600, 16, 3), (1, 1, 850, 12, 2)])
def test_ragged_and_degenerate_shapes(vc, B, H, N, k, iters):
    _say(f"ragged: B{B} H{H} N{N} k{k} T{iters}")
    Q, K, V = W.custom_inputs(B, H, N, seed=N + k, recipe="clustered")
    prep, preps, _ = _check_group_and_codes(vc, Q, K, V, k, iters)
    _check_given_scores(vc, prep, preps, "expcast")
    _check_given_scores(vc, prep, preps, "fp32exp_e4m3")
    _check_attention(vc, prep, preps, "expcast", tol=TOL_GAUSS_QK)
    _check_attention(vc, prep, preps, "fp32exp_e4m3", tol=TOL_GAUSS_QK)


def test_constant_value_blocks(vc):
    _say("degenerate: V constant per 128-row block (zero residual, zero V scales)")
    N = 384
    Q, K, _ = W.custom_inputs(1, 1, N, seed=5)
    rows = torch.randn(3, 128, generator=torch.Generator().manual_seed(1)) * 4
    V = rows.repeat_interleave(128, dim=0).reshape(1, 1, N, 128).to(torch.bfloat16)
    dev = torch.device("cuda:0")
    perm = torch.arange(N, dtype=torch.int32, device=dev).reshape(1, 1, N)
    prep = vc.preprocess_quant(Q.to(dev), K.to(dev), V.to(dev), perm)
    assert not prep["v_codes"].any() and not prep["v_scales"].any()
    pr = O.preprocess_head(_u16(Q[0, 0]), _u16(K[0, 0]), _u16(V[0, 0]), np.arange(N, dtype=np.int32))
    out = vc.attn_fp8_fwd(prep, SCALE, "expcast").cpu().numpy()[0, 0]
    assert O.rel_l2(out, O.vc_attention_head(pr, SCALE, "expcast")) <= TOL_OUT


def test_deterministic_bitwise(vc):
    _say("determinism: two runs of the tiny 8-bit workload compared bit for bit")
    c = W.WORKLOADS["tiny-8bit"]
    Q, K, V = W.make_inputs("tiny-8bit")
    r1 = _run_all(vc, Q, K, V, c["k"], c["iters"])
    r2 = _run_all(vc, Q, K, V, c["k"], c["iters"])
    assert torch.equal(r1[3], r2[3])
    o1 = vc.attn_fp8_fwd(r1[6], SCALE)
    o2 = vc.attn_fp8_fwd(r2[6], SCALE)
    assert torch.equal(o1, o2)


def test_permutation_alone_matches_oracle(vc):
    """Asked for the permutation only, the grouping skips the update after the
    last assignment; the permutation must not change (oracle, and the call that
    also returns labels and centroids)."""
    _say("permutation alone: B1 H3 N2000 k16 T5, with and without centroids")
    Q, K, V = W.custom_inputs(1, 3, 2000, seed=21, recipe="clustered")
    dev = torch.device("cuda:0")
    Vd = V.to(dev)
    perm_only, _, _ = vc.vsmooth_group(Vd, 16, 5)
    perm_full, labels, _ = vc.vsmooth_group(Vd, 16, 5, want_labels=True, want_centroids=True)
    torch.cuda.synchronize()
    assert torch.equal(perm_only, perm_full)
    v16 = _u16(V)
    for h in range(3):
        lab, _, _ = O.kmeans(O.bf16_to_f32(v16[0, h]), 16, 5)
        np.testing.assert_array_equal(labels[0, h].cpu().numpy(), lab, err_msg=f"labels h{h}")
        np.testing.assert_array_equal(perm_only[0, h].cpu().numpy(), O.stable_label_sort(lab, 16),
                                      err_msg=f"perm h{h}")


def test_grouping_large_values(vc):
    """Rows with |v| >= 128 take the accumulation's int64 conversion path (the
    others its int32 path); labels and centroids must match the oracle either way."""
    _say("grouping, large values: B1 H2 N5000 k8 T3, tokens 1000..1299 scaled by 700")
    g = torch.Generator().manual_seed(33)
    V = torch.randn(1, 2, 5000, 128, generator=g)
    V[:, :, 1000:1300] *= 700.0
    V[:, 1, 4090:4100] = -300.0
    V = V.to(torch.bfloat16)
    dev = torch.device("cuda:0")
    perm, labels, cents = vc.vsmooth_group(V.to(dev), 8, 3, want_labels=True, want_centroids=True)
    torch.cuda.synchronize()
    v16 = _u16(V)
    for h in range(2):
        lab, cen, _ = O.kmeans(O.bf16_to_f32(v16[0, h]), 8, 3)
        np.testing.assert_array_equal(labels[0, h].cpu().numpy(), lab, err_msg=f"labels h{h}")
        np.testing.assert_array_equal(cents[0, h].cpu().numpy(), cen, err_msg=f"centroids h{h}")
        np.testing.assert_array_equal(perm[0, h].cpu().numpy(), O.stable_label_sort(lab, 8), err_msg=f"perm h{h}")


def test_bf16_comparator_matches_exact_attention(vc):
    """The comparator's only rounding of note is P -> bf16: each weight moves by
    at most 2^-9 relative (the row sum is taken of the rounded weights, so the
    normalisation follows), and the output of row i moves by at most
    2^-9 / (1 - 2^-9) * sum_j w_ij |v_j - o_i| <= 2^-9 (1 + 2^-8) (sum_j w_ij |v_j| + |o_i|)
    in L2 norm (w = exact softmax weights).  The bf16 products of the two MFMAs
    are exact in fp32; the fp32 accumulation, the scaling of S and exp2 add
    relative errors of order 2^-20, covered by a slack of 1e-5.  Each row is held
    to that bound.  On these inputs the bf16 rounding of exact P alone (float64
    otherwise) gives rel-L2 8.6e-4 and 9.0e-4 for the two heads, so the whole
    output is held to 1.5e-3."""
    _say("bf16 comparator: B1 H2 N1000 against exact fp64 attention")
    Q, K, V = W.custom_inputs(1, 2, 1000, seed=11, recipe="clustered")
    dev = torch.device("cuda:0")
    out = vc.attn_bf16_fwd(Q.to(dev), K.to(dev), V.to(dev), SCALE).cpu().numpy()
    for h in range(2):
        q16, k16, v16 = _u16(Q[0, h]), _u16(K[0, h]), _u16(V[0, h])
        ex = O.exact_attention(q16, k16, v16, SCALE)
        q, k, v = (O.bf16_to_f32(t).astype(np.float64) for t in (q16, k16, v16))
        s = (q @ k.T) * SCALE
        w = np.exp(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        wv = w @ np.linalg.norm(v, axis=1)
        bound = 2.0 ** -9 * (1 + 2.0 ** -8) * (wv + np.linalg.norm(ex, axis=1)) + 1e-5 * wv
        err = np.linalg.norm(out[0, h].astype(np.float64) - ex, axis=1)
        assert np.all(err <= bound), f"h{h}: worst row {np.max(err / bound):.3f} of its bound"
        rel = O.rel_l2(out[0, h], ex)
        _say(f"bf16 comparator h{h}: rel-L2 {rel:.3e}, worst row at {np.max(err / bound):.3f} of its bound")
        assert rel < 1.5e-3


def test_wan22_full_size_sampled(vc):
    """Full Wan2.2 shape (B1 H40 N75600, k64, T8) in the launch configuration the
    bench times; the oracle checks two heads' grouping and codes in full and 48
    sampled query rows of each against its attention output."""
    _say("Wan2.2 shape: B1 H40 N75600 k64 T8 full size, sampled oracle heads 0 and 39")
    c = W.WORKLOADS["wan22-attention"]
    Q, K, V = W.make_inputs("wan22-attention")
    heads = [(0, 0), (0, 39)]
    prep, preps, _ = _check_group_and_codes(vc, Q, K, V, c["k"], c["iters"], heads=heads)
    rows = np.concatenate([np.arange(0, 75600, 1601), np.arange(75590, 75600)])
    _check_attention(vc, prep, preps, "expcast", rows)


def test_nvfp4_small_ragged(vc):
    _say("4-bit path: B1 H2 N1000 k8 T4, NVFP4 residual, fp32 softmax, bf16 P")
    Q, K, V = W.custom_inputs(1, 2, 1000, seed=41, recipe="clustered")
    prep, preps, _ = _check_group_and_codes(vc, Q, K, V, 8, 4, fmt="nvfp4")
    _check_given_scores(vc, prep, preps, "fp32_bf16", report_e2e=True)
    _check_attention(vc, prep, preps, "fp32_bf16", tol=TOL_GAUSS_QK)


def test_ragged_4bit_sampled(vc):
    """The ragged 4-bit workload at full size (B2 H24 N32760, last block 120 rows, k64 T8,
    NVFP4); two heads checked in full for grouping and codes, 48 rows each for
    the output."""
    _say("ragged 4-bit: B2 H24 N32760 k64 T8 NVFP4, sampled heads (0,0) and (1,23)")
    c = W.WORKLOADS["ragged-4bit"]
    Q, K, V = W.make_inputs("ragged-4bit")
    heads = [(0, 0), (1, 23)]
    prep, preps, _ = _check_group_and_codes(vc, Q, K, V, c["k"], c["iters"], heads=heads, fmt="nvfp4")
    rows = np.concatenate([np.arange(0, 32760, 701), np.arange(32750, 32760)])
    _check_attention(vc, prep, preps, "fp32_bf16", rows, tol=TOL_GAUSS_QK)
    # bf16 P given the kernel's scores, output replayed on them (1e-4), and the
    # end-to-end P mismatch, on the same sampled rows of the two heads
    _check_given_scores(vc, prep, preps, "fp32_bf16", rows, report_e2e=True)


@pytest.mark.parametrize("fmt,p_mode", [("e4m3", "expcast"), ("e4m3", "fp32exp_e4m3"), ("mxfp4", "expcast"),
                                        ("mxfp4", "fp32exp_e4m3"), ("nvfp4", "fp32_bf16")])
def test_masked_keys_with_zero_scale_blocks(vc, fmt, p_mode):
    """Ragged N with an all-zero Q block and an all-zero last K block: their
    scales are 0, so the score scale kap is 0 for those tiles, and the keys past
    N in the last tile must still take no part (no NaN from -inf * 0)."""
    _say(f"masked keys, zero-scale blocks: B1 H1 N300, {fmt} / {p_mode}")
    N = 300
    Q, K, V = W.custom_inputs(1, 1, N, seed=77, recipe="clustered")
    Q[:, :, 128:256] = 0
    K[:, :, 256:300] = 0        # identity permutation: this is the last permuted K block
    dev = torch.device("cuda:0")
    perm = torch.arange(N, dtype=torch.int32, device=dev).reshape(1, 1, N)
    prep = vc.preprocess_quant(Q.to(dev), K.to(dev), V.to(dev), perm, fmt)
    torch.cuda.synchronize()
    assert prep["q_scales"][0, 0, 1].item() == 0.0 and prep["k_scales"][0, 0, 2].item() == 0.0
    pr = O.preprocess_head(_u16(Q[0, 0]), _u16(K[0, 0]), _u16(V[0, 0]), np.arange(N, dtype=np.int32), fmt)
    out = vc.attn_fp8_fwd(prep, SCALE, p_mode).cpu().numpy()[0, 0]
    assert np.isfinite(out).all()
    e = O.rel_l2(out, O.vc_attention_head(pr, SCALE, p_mode))
    _say(f"  output rel-L2 vs exact-score oracle {e:.2e}")
    assert e <= TOL_GAUSS_QK
    _check_given_scores(vc, prep, {(0, 0): pr}, p_mode, report_e2e=True)


def test_preprocess_quant_entry_point_itself(vc):
    """vc_preprocess_quant (no RoPE, no Hadamard) called through the C ABI
    directly: every output bit-identical to the _ex call the binding makes,
    which the other tests hold to the oracle bit for bit."""
    import ctypes
    _say("vc_preprocess_quant called directly: B1 H2 N1000 k8 T4, E4M3")
    Q, K, V = W.custom_inputs(1, 2, 1000, seed=52, recipe="clustered")
    prep_ex, preps, (Qd, Kd, Vd) = _check_group_and_codes(vc, Q, K, V, 8, 4)
    perm, _, _ = vc.vsmooth_group(Vd, 8, 4)
    direct = {k: torch.full_like(v, 0x5A if v.dtype == torch.uint8 else 7) for k, v in prep_ex.items()
              if isinstance(v, torch.Tensor)}
    L = vc.lib()
    ws_bytes = L.vc_preprocess_workspace(1, 2, 1000, 128, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=Qd.device)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = L.vc_preprocess_quant(P(Qd), P(Kd), P(Vd), P(perm), 1, 2, 1000, 128, 0,
                               P(direct["q_codes"]), P(direct["q_scales"]), P(direct["k_codes"]),
                               P(direct["k_scales"]), P(direct["v_codes"]), P(direct["v_scales"]), None,
                               P(direct["v_means"]), P(ws), ws_bytes,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    assert set(direct) == {"q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales", "v_means"}
    for k, v in direct.items():
        assert torch.equal(v, prep_ex[k]), k


@pytest.mark.parametrize("case", ["uniform", "dominant"])
@pytest.mark.parametrize("fmt,p_mode", [("e4m3", "expcast"), ("e4m3", "fp32exp_e4m3"), ("mxfp4", "expcast"),
                                        ("mxfp4", "fp32exp_e4m3"), ("nvfp4", "fp32_bf16")])
def test_closed_form_score_patterns(vc, fmt, p_mode, case):
    """Two score patterns whose outputs have closed forms (the oracle is pinned
    to them on the CPU): Q = 0, so every P is exactly 1 and each row is the mean
    of the value tokens; and one key about 2^16 log2 units above every other,
    so each row is that key's token and every tile before it is rescaled by 0.
    Scores are exact in both (all partial sums are small multiples of one
    product), so the kernel meets the oracle within the given-S bar."""
    _say(f"closed-form scores ({case}): B1 H1 N300, {fmt} / {p_mode}")
    N = 300
    _, _, V = W.custom_inputs(1, 1, N, seed=91, recipe="clustered")
    if case == "uniform":
        Q = torch.zeros(1, 1, N, 128, dtype=torch.bfloat16)
        K = W.custom_inputs(1, 1, N, seed=92, recipe="clustered")[1]
    else:
        Q = torch.full((1, 1, N, 128), 64.0, dtype=torch.bfloat16)
        K = torch.zeros(1, 1, N, 128, dtype=torch.bfloat16)
        K[0, 0, 137] = 64.0
    dev = torch.device("cuda:0")
    perm_np = np.random.default_rng(93).permutation(N).astype(np.int32)
    perm = torch.from_numpy(perm_np).to(dev).reshape(1, 1, N)
    prep = vc.preprocess_quant(Q.to(dev), K.to(dev), V.to(dev), perm, fmt)
    out = vc.attn_fp8_fwd(prep, SCALE, p_mode).cpu().numpy()[0, 0]
    pr = O.preprocess_head(_u16(Q[0, 0]), _u16(K[0, 0]), _u16(V[0, 0]), perm_np, fmt)
    want = O.vc_attention_head(pr, SCALE, p_mode)
    e = O.rel_l2(out, want)
    _say(f"  output rel-L2 vs oracle {e:.2e}")
    assert np.isfinite(out).all() and e <= TOL_GIVEN_S
