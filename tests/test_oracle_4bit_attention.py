"""Pins of the oracle's 4-bit attention outputs, from closed forms that hold
whatever the rounding order: the NVFP4 residual with fp32 softmax and P rounded
to bf16, and the MXFP4 residual with ExpCast or fp32 exp2 -> E4M3 P.

Paper digest "VC-Attention: Value Smoothing and Softmax Casting for Low-bit
Attention", V-Smooth paragraph: the 4-bit path quantises the residual to NVFP4
(E2M1 values with one E4M3 scale per 16 values) and restores each block mean from
the row sums.  The value tokens are rebuilt here from the stored codes with a
decoder of this file's own (the public E2M1 table, E8M0 = 2^(code - 127),
torch's E4M3 and bf16 casts), independent of the oracle's decoders.
"""
import pytest
import numpy as np
import torch

from oracle import oracle as O

SCALE = 1.0 / np.sqrt(128.0)
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rebuilt_values(prep, N, fmt):
    """V in permuted order as the 4-bit path stores it: E2M1 nibble (sign in bit
    3) x its group's scale, plus the bf16 mean of its 128-token block.  NVFP4:
    the E4M3 scale of the 16-token group x the head's second-level scale; MXFP4:
    the E8M0 scale of the 32-token group (t, h, g) that holds rows 64h + 16g +
    [0, 16) and 64h + 32 + 16g + [0, 16) of block t."""
    nib = prep["v_nibbles"][:N].astype(np.int64)
    val = np.where(nib & 8, -1.0, 1.0) * E2M1[nib & 7]
    if fmt == "nvfp4":
        sg = torch.from_numpy(np.ascontiguousarray(prep["v_group_scales"])).view(torch.float8_e4m3fn)
        sg = sg.to(torch.float64).numpy()
        scale = np.repeat(sg, 16, axis=0)[:N] * float(prep["v_scales"][0])
    else:
        rows = np.arange(N)
        t, u = rows // 128, rows % 128
        code = prep["v_mx_scales"][t, u // 64, (u % 64) // 16 % 2].astype(np.float64)
        scale = 2.0 ** (code - 127.0)
    means = torch.from_numpy(np.ascontiguousarray(prep["means"]).view(np.int16)).view(torch.bfloat16)
    means = means.to(torch.float64).numpy()
    return val * scale + np.repeat(means, 128, axis=0)[:N]


def _inputs(N, seed):
    rng = np.random.default_rng(seed)
    v = _bf16(rng.standard_normal((N, 128)) * np.linspace(0.2, 3.0, 128)[None, :] + rng.standard_normal(128))
    perm = rng.permutation(N).astype(np.int32)
    return v, perm


CASES = [("nvfp4", "fp32_bf16"), ("mxfp4", "expcast"), ("mxfp4", "fp32exp_e4m3")]


@pytest.mark.parametrize("fmt,p_mode", CASES)
def test_uniform_scores_average_the_rebuilt_values(fmt, p_mode):
    """Q = 0: every score is 0 and every P is exactly 1 (bf16 1.0; ExpCast code
    RNE(55.65) = 56 = E4M3 1.0; E4M3 of 2^0), so each output row is the plain mean
    of the rebuilt value tokens (ragged N: the padding rows of the last block take
    no part)."""
    N = 300
    v, perm = _inputs(N, 11)
    k = _bf16(np.random.default_rng(12).standard_normal((N, 128)))
    q = _bf16(np.zeros((N, 128)))
    prep = O.preprocess_head(q, k, v, perm, fmt)
    out = O.vc_attention_head(prep, SCALE, p_mode, rows=np.array([0, 131, 299]))
    want = _rebuilt_values(prep, N, fmt).mean(axis=0)
    np.testing.assert_allclose(out, np.broadcast_to(want, out.shape), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmt,p_mode", CASES)
def test_one_dominant_key_returns_its_rebuilt_value(fmt, p_mode):
    """One key aligned with every query and about 2^16 log2 units above the rest:
    its P is 1, every other P is 0 (and the blocks before it are rescaled by 0),
    so every output row is that key's rebuilt value token, which also checks
    which permuted row the P.V product pairs with which key."""
    N = 300
    v, perm = _inputs(N, 21)
    j = 137                                             # source index of the dominant key
    kk = np.zeros((N, 128))
    kk[j] = 64.0
    k = _bf16(kk)
    q = _bf16(np.full((N, 128), 64.0))
    prep = O.preprocess_head(q, k, v, perm, fmt)
    out = O.vc_attention_head(prep, SCALE, p_mode, rows=np.array([0, 5, 299]))
    pos = int(np.argsort(perm)[j])                      # its slot in the permuted order
    want = _rebuilt_values(prep, N, fmt)[pos]
    np.testing.assert_allclose(out, np.broadcast_to(want, out.shape), rtol=1e-12, atol=1e-12)
