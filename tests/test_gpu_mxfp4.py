"""GPU parity of the MXFP4 4-bit path: V residual as E2M1 values with one E8M0
scale per 32 rows, fed to the block-scaled FP4 MFMA (P in E4M3, by ExpCast or
by fp32 exp2 + convert).  Codes and scales bit-exact against the oracle; the
output within 1e-4 of the oracle replayed on the kernel's own scores, P bytes
bit-exact given them (ExpCast), and within the Gaussian-QK tolerance of the
oracle on exact scores."""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import test_gpu_parity as GP
import vc_workloads as W

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128.0)
TOL_GIVEN_S = 1e-4
TOL_GAUSS_QK = 6e-3


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


def _rows_of_kernel_nibbles(vb):
    """[nb, 128(ch), 64] bytes of the kernel layout -> [nb*128, 128] nibbles in row order."""
    nb = vb.shape[0]
    out = np.zeros((nb * 128, 128), np.uint8)
    for h in range(2):
        for g in range(2):
            seg = vb[:, :, 32 * h + 16 * g: 32 * h + 16 * g + 16]          # [nb, ch, 16]
            nib = np.stack([seg & 15, seg >> 4], axis=-1).reshape(nb, 128, 32)
            for j in range(32):
                u = 64 * h + 16 * g + (j if j < 16 else 16 + j)
                out[np.arange(nb) * 128 + u, :] = nib[:, :, j]
    return out


def _check(vc, Q, K, V, k, iters, heads, rows=None):
    dev = torch.device("cuda:0")
    Qd, Kd, Vd = (t.to(dev) for t in (Q, K, V))
    perm, _, _ = vc.vsmooth_group(Vd, k, iters)
    prep = vc.preprocess_quant(Qd, Kd, Vd, perm, "mxfp4")
    torch.cuda.synchronize()
    q16, k16, v16 = _u16(Q), _u16(K), _u16(V)
    perm_c = perm.cpu().numpy()
    N = Q.shape[2]
    outs = {pm: vc.attn_fp8_fwd(prep, SCALE, pm).cpu().numpy() for pm in ("expcast", "fp32exp_e4m3")}
    preps = {}
    for (b, h) in heads:
        pr = O.preprocess_head(q16[b, h], k16[b, h], v16[b, h], perm_c[b, h].astype(np.int64), "mxfp4")
        np.testing.assert_array_equal(prep["k_codes"][b, h].cpu().numpy(), pr["k_codes"], err_msg="k codes")
        np.testing.assert_array_equal(_u16(prep["v_means"][b, h]), pr["means"], err_msg="means")
        nib = _rows_of_kernel_nibbles(prep["v_codes"][b, h].cpu().numpy())
        np.testing.assert_array_equal(nib, pr["v_nibbles"], err_msg=f"mxfp4 nibbles b{b} h{h}")
        sc = prep["v_group_scales"][b, h].cpu().numpy()                 # [nb, ch, g, h]
        np.testing.assert_array_equal(sc.transpose(0, 3, 2, 1), pr["v_mx_scales"], err_msg="mxfp4 scales")
        assert np.all(prep["v_scales"][b, h].cpu().numpy() == 1.0)
        for pm in ("expcast", "fp32exp_e4m3"):
            ref = O.vc_attention_head(pr, SCALE, pm, rows=rows)
            got = outs[pm][b, h] if rows is None else outs[pm][b, h][rows]
            e = O.rel_l2(got, ref)
            _say(f"  b{b} h{h} {pm}: rel-L2 vs exact-score oracle {e:.2e}")
            assert e <= TOL_GAUSS_QK
        preps[(b, h)] = pr
    # P bytes given the MXFP4 kernel's own scores, output replayed on them (1e-4)
    for pm in ("expcast", "fp32exp_e4m3"):
        GP._check_given_scores(vc, prep, preps, pm, rows, report_e2e=True)


# N = 600: five 128-row blocks, one full four-block mean-restore batch and one more
@pytest.mark.parametrize("N", [1000, 600, 300, 128, 77])
def test_mxfp4_small(vc, N):
    _say(f"MXFP4 path: B1 H2 N{N} k8 T4")
    Q, K, V = W.custom_inputs(1, 2, N, seed=43, recipe="clustered")
    _check(vc, Q, K, V, 8, 4, [(0, 0), (0, 1)])


def test_mxfp4_ragged_4bit_shape_sampled(vc):
    """The ragged 4-bit workload's shape (B2 H24 N32760, last block 120 rows,
    k64 T8) on the MXFP4 path; two heads, 48 rows each."""
    _say("MXFP4 path at B2 H24 N32760 k64 T8, sampled heads (0,0) and (1,23)")
    c = W.WORKLOADS["ragged-4bit"]
    Q, K, V = W.make_inputs("ragged-4bit")
    rows = np.concatenate([np.arange(0, 32760, 701), np.arange(32750, 32760)])
    _check(vc, Q, K, V, c["k"], c["iters"], [(0, 0), (1, 23)], rows=rows)
