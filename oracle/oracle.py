"""CPU oracle for the VC-Attention hot path.

TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously-correct reference of what the
HIP path computes.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it; the product path never does, and this module
imports nothing from the product package (the two share no code).

Sources (the four web pages about the method; cited by title and section):
  [digest]  "VC-Attention: Value Smoothing and Softmax Casting for Low-bit
            Attention" (paper digest page): V-Smooth paragraph, ExpCast-FP8
            paragraph, preprocessing paragraph, results table, limitations.
  [insight] "Nunchux AI Introduces VC-Attention" (insight article, English and
            Chinese editions): sections "Value Is the Error Source Earlier Methods
            Underestimated" and "Softmax Has to Be Designed for Low-Bit Execution
            Too".
  [news]    "Nunchux open-sources VC-Attention" (news article): sections
            "V-Smooth" (items Group / Demean / Restore) and "ExpCast-FP8".

Number formats follow their public definitions: OCP FP8 E4M3 (E4M3FN), OCP FP4
E2M1, bfloat16.  Contractions whose result is exact in float64 use numpy's
matmul as a step.  Where the pages leave the arithmetic open the reading taken is
stated in the function's docstring.

Parity status: every function here is pinned by a `-m "not gpu"` test.  No page
gives a number for the 4-bit attention outputs (NVFP4 and MXFP4 residuals); they
are pinned by closed forms (uniform scores average the value tokens rebuilt
from the stored codes; one dominant key returns its own rebuilt token).
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
BLOCK = 128          # block size of the method (V-Smooth demeans 128-token blocks)
LOG2E = 1.4426950408889634
E4M3_MAX = 448.0
E2M1_MAX = 6.0
F32 = np.float32

_lib = None


def build_lib(force: bool = False) -> str:
    """Compile vc_oracle.c with gcc (no fused multiply-add unless written)."""
    src = os.path.join(HERE, "vc_oracle.c")
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(src):
        import subprocess
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O3", "-mavx2", "-mfma", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build_lib()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.vco_fmaf.argtypes = [P, P, P, P, ctypes.c_int64]
        L.vco_kmeans.argtypes = [P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P]
        L.vco_kmeans.restype = ctypes.c_int
        L.vco_assign.argtypes = [P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, P, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def f32(x):
    return np.asarray(x, dtype=np.float32)


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest, ties to even."""
    x = f32(x)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    nan = np.isnan(x)
    r = np.where(nan, ((u >> 16) & 0x8000) | 0x7FC0, r)
    return r.astype(np.uint16)


def e4m3_decode(code) -> np.ndarray:
    """OCP E4M3 byte -> float64.  1 sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 holds subnormals m * 2^-9; 0x7F / 0xFF are NaN."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return s * mag


def e4m3_encode(x) -> np.ndarray:
    """float32 -> OCP E4M3 byte: round to nearest, ties to even, magnitudes above
    448 (and infinities) saturate to 448, NaN -> 0x7F with its sign, -0 -> 0x80."""
    x = f32(x).astype(np.float64)
    neg = np.signbit(x)
    nan = np.isnan(x)
    a = np.minimum(np.where(nan, 0.0, np.abs(x)), E4M3_MAX)
    _, fe = np.frexp(a)                       # a = mant * 2^fe, mant in [0.5, 1)
    e = np.maximum(fe - 1, -6)                # binade; subnormals use the 2^-6 binade
    quantum = np.ldexp(1.0, e - 3)            # three mantissa bits
    q = np.minimum(np.rint(a / quantum) * quantum, E4M3_MAX)   # rint: ties to even
    _, qe = np.frexp(q)
    qexp = qe - 1
    sub = q < 2.0 ** -6
    code_sub = np.rint(q / 2.0 ** -9)
    mant = np.rint((q / np.ldexp(1.0, qexp) - 1.0) * 8.0)
    code_norm = (qexp + 7) * 8 + mant
    code = np.where(sub, code_sub, code_norm).astype(np.int64)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(nib) -> np.ndarray:
    """OCP FP4 E2M1 nibble -> float64: bit 3 sign, 2 exponent bits (bias 1),
    1 mantissa bit; magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}."""
    n = np.asarray(nib, dtype=np.uint8).astype(np.int64)
    return np.where(n & 8, -1.0, 1.0) * E2M1_GRID[n & 7]


def e2m1_encode(x) -> np.ndarray:
    """float32 -> E2M1 nibble: round to nearest, ties to even mantissa,
    saturating at 6 (the pages' 4-bit path uses NVFP4, whose values are E2M1)."""
    x = f32(x).astype(np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(np.nan_to_num(x)), E2M1_MAX)
    quantum = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    q = np.minimum(np.rint(a / quantum) * quantum, E2M1_MAX)
    idx = np.searchsorted(E2M1_GRID, q)
    return (idx | np.where(neg, 8, 0)).astype(np.uint8)


def fma_f32(a, b, c) -> np.ndarray:
    """float32 fused multiply-add (one rounding of the exact a*b+c), element-wise
    with numpy broadcasting; evaluated by C99 fmaf."""
    a, b, c = np.broadcast_arrays(f32(a), f32(b), f32(c))
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    c = np.ascontiguousarray(c)
    out = np.empty(a.shape, np.float32)
    lib().vco_fmaf(_ptr(a), _ptr(b), _ptr(c), _ptr(out), out.size)
    return out


# ---------------------------------------------------------------------------
# V-Smooth grouping: k-means and the stable label sort
# ---------------------------------------------------------------------------

def kmeans(v_f32: np.ndarray, k: int, iters: int):
    """k-means over the Value tokens of one (batch, head).

    [digest] V-Smooth paragraph: each batch and head runs online k-means over its
    Value tokens.  [news] "V-Smooth", item Group.  Online is read as run at
    inference time on every call (Lloyd iterations, as the configurations state).
    The fixed arithmetic (see vc_oracle.c) is the reading taken.
    Returns (labels int32 [N], centroids float32 [k, d], counts int64 [k]).
    """
    v = np.ascontiguousarray(f32(v_f32))
    N, d = v.shape
    labels = np.empty(N, np.int32)
    cent = np.empty((k, d), np.float32)
    counts = np.empty(k, np.int64)
    rc = lib().vco_kmeans(_ptr(v), N, d, k, iters, _ptr(labels), _ptr(cent), _ptr(counts))
    if rc != 0:
        raise ValueError("bad k-means arguments")
    return labels, cent, counts


def kmeans_assign(v_f32: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(f32(v_f32))
    c = np.ascontiguousarray(f32(centroids))
    labels = np.empty(v.shape[0], np.int32)
    lib().vco_assign(_ptr(v), v.shape[0], v.shape[1], c.shape[0], _ptr(c), _ptr(labels))
    return labels


def stable_label_sort(labels: np.ndarray, k: int) -> np.ndarray:
    """Counting sort of tokens by cluster label: clusters in index order, tokens
    of one cluster in their original order.  perm[j'] = source token of permuted
    slot j'.  [digest] V-Smooth paragraph: Key and Value are reordered by
    cluster label.  Cluster order and tie order are not on the pages; ascending
    label and ascending token index are the reading taken."""
    labels = np.asarray(labels, dtype=np.int64)
    N = labels.shape[0]
    onehot = (labels[:, None] == np.arange(k)[None, :]).astype(np.int64)
    counts = onehot.sum(axis=0)
    start = np.concatenate([[0], np.cumsum(counts)[:-1]])
    before = np.cumsum(onehot, axis=0) - onehot          # same-label tokens earlier in order
    rank = before[np.arange(N), labels]
    perm = np.empty(N, np.int32)
    perm[start[labels] + rank] = np.arange(N, dtype=np.int32)
    return perm


def vsmooth_group(V_bf16: np.ndarray, k: int, iters: int):
    """V [B, H, N, d] bfloat16 bits -> perm, labels [B, H, N] int32, centroids [B, H, k, d]."""
    B, H, N, d = V_bf16.shape
    perm = np.empty((B, H, N), np.int32)
    labels = np.empty((B, H, N), np.int32)
    cents = np.empty((B, H, k, d), np.float32)
    for b in range(B):
        for h in range(H):
            lab, cen, _ = kmeans(bf16_to_f32(V_bf16[b, h]), k, iters)
            labels[b, h] = lab
            cents[b, h] = cen
            perm[b, h] = stable_label_sort(lab, k)
    return perm, labels, cents


# ---------------------------------------------------------------------------
# Preprocessing: gather, block mean, residual quantisation
# ---------------------------------------------------------------------------

def n_blocks(N: int) -> int:
    return -(-N // BLOCK)


def block_means(vp: np.ndarray) -> np.ndarray:
    """16-bit mean of every 128-token block of the permuted Values.

    [digest] V-Smooth paragraph: each 128-row hardware block subtracts its block
    mean; the mean is a 16-bit vector (about 0.125 bit per element).  [news]
    "V-Smooth", item Demean.  Reading: bfloat16 (the inputs' format), computed
    as a float32 sum over ascending permuted positions, divided in float32 by the
    block's row count (the last block may be partial), rounded to nearest even.
    Returns bf16 bits [nb, d]."""
    N, d = vp.shape
    nb = n_blocks(N)
    pad = np.zeros((nb * BLOCK, d), np.float32)
    pad[:N] = vp
    blocks = pad.reshape(nb, BLOCK, d)
    valid = (np.arange(nb * BLOCK).reshape(nb, BLOCK) < N)
    acc = np.zeros((nb, d), np.float32)
    for r in range(BLOCK):
        acc = np.where(valid[:, r:r + 1], f32(acc + blocks[:, r]), acc)
    n_t = valid.sum(axis=1).astype(np.float32)
    return bf16_round(f32(acc / n_t[:, None]))


def _block_scaled_e4m3(x: np.ndarray, N: int):
    """Per-128-row-block E4M3 quantisation (used for Q and K).

    The pages leave the Q/K scheme to prior methods ([insight] "Value Is the
    Error Source..."); the reading is one scale per 128-row block:
    s = amax / 448 and codes = E4M3(x * (448 / amax)), both in float32; an
    all-zero block gets s = 0 and zero codes.  Returns codes [Np, d], s [nb]."""
    d = x.shape[1]
    nb = n_blocks(N)
    codes = np.zeros((nb * BLOCK, d), np.uint8)
    scales = np.zeros(nb, np.float32)
    for t in range(nb):
        blk = x[t * BLOCK: min(N, (t + 1) * BLOCK)]
        amax = F32(np.max(np.abs(blk)))
        if amax > 0:
            scales[t] = F32(amax / F32(E4M3_MAX))
            inv = F32(F32(E4M3_MAX) / amax)
            codes[t * BLOCK: t * BLOCK + blk.shape[0]] = e4m3_encode(f32(blk * inv))
    return codes, scales


def rope_f32(x: np.ndarray, cs: np.ndarray) -> np.ndarray:
    """Rotary position embedding of Q or K rows, as a step of the fused
    preprocessing.

    [digest] preprocessing paragraph: RoPE is one of the steps fused into the
    quantisation kernel.  The pages do not define the rotation; the reading is
    the usual pairwise one, with the angles supplied by the caller: `cs` is a
    float32 table [rows, 64, 2] of (cos, sin) for each row and channel pair
    (2i, 2i+1), and in float32
        y_2i   = fmaf(x_2i, c, -(x_2i+1 * s))
        y_2i+1 = fmaf(x_2i, s,   x_2i+1 * c)
    with each inner product rounded once.  x: float32 [rows, 128].
    """
    x = f32(x)
    cs = f32(cs)
    x0, x1 = x[:, 0::2], x[:, 1::2]
    c, s = cs[..., 0], cs[..., 1]
    out = np.empty_like(x)
    out[:, 0::2] = fma_f32(x0, c, -f32(x1 * s))
    out[:, 1::2] = fma_f32(x0, s, f32(x1 * c))
    return out


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform along the last axis, y = H x with
    H[i][j] = (-1)^popcount(i & j) (Sylvester order), in float32 stage by stage:
    for h = 1, 2, 4, ..., d/2 the pair (i, i + h) with i & h == 0 becomes
    (a + b, a - b), each rounded once.

    [digest] preprocessing paragraph (Hadamard is one of the fused steps) and
    results paragraph (a Hadamard on Q and K moves PSNR by 0.1-0.3 dB at most).
    """
    y = f32(x).copy()
    d = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < d:
        z = y.reshape(*lead, d // (2 * h), 2, h)
        a, b = z[..., 0, :], z[..., 1, :]
        y = np.stack([f32(a + b), f32(a - b)], axis=-2).reshape(*lead, d)
        h *= 2
    return y


def qk_transform(x: np.ndarray, cs=None, hadamard: bool = False, k_side: bool = False) -> np.ndarray:
    """RoPE (when a table is given) then the Hadamard (when asked) of Q or K rows
    in float32, before the per-block E4M3 quantisation.  Reading for the
    Hadamard: Q' = H q and K' = 2^-7 H k (an exact power-of-two scale), so that
    Q'.K' = q.k exactly in real arithmetic (H H^T = 128 I)."""
    y = f32(x)
    if cs is not None:
        y = rope_f32(y, cs)
    if hadamard:
        y = fwht_f32(y)
        if k_side:
            y = f32(y * F32(2.0 ** -7))
    return y


def preprocess_head(q_bf16, k_bf16, v_bf16, perm, v_format: str = "e4m3", rope_cs=None, hadamard: bool = False):
    """Gather, demean and quantise one (batch, head).

    [digest] V-Smooth paragraph (reorder K and V by label; subtract each 128-row
    block's mean; quantise only the residual: per-channel E4M3 on the 8-bit
    path, NVFP4 on the 4-bit path) and preprocessing paragraph (mean, gather and
    quantisation fused in one kernel).  [news] "V-Smooth", items Group/Demean.

    Readings: "per-channel" = one scale per (batch, head, channel) over all N
    tokens, sv = amax/448; residual R = fp32(v) - fp32(mean) in float32;
    codes = E4M3(R * (448/amax)) in float32.  Q stays in the original order.
    With `rope_cs` ([N, 64, 2], original token order) and/or `hadamard`, Q and
    K rows go through qk_transform first (K rows keep their original position).
    """
    N = v_bf16.shape[0]
    qf = bf16_to_f32(q_bf16) if q_bf16 is not None else None
    if rope_cs is not None or hadamard:
        if qf is not None:
            qf = qk_transform(qf, rope_cs, hadamard, k_side=False)
        kp = qk_transform(bf16_to_f32(k_bf16), rope_cs, hadamard, k_side=True)[perm]
    else:
        kp = bf16_to_f32(k_bf16)[perm]
    vp = bf16_to_f32(v_bf16)[perm]
    nb = n_blocks(N)
    means = block_means(vp)
    mu = bf16_to_f32(means)
    R = f32(vp - np.repeat(mu, BLOCK, axis=0)[:N])
    out = dict(N=N, means=means)
    if qf is not None:
        out["q_codes"], out["q_scales"] = _block_scaled_e4m3(qf, N)
    out["k_codes"], out["k_scales"] = _block_scaled_e4m3(kp, N)
    if v_format == "e4m3":
        amax = np.max(np.abs(R), axis=0).astype(np.float32)
        pos = amax > 0
        sv = np.where(pos, f32(amax / F32(E4M3_MAX)), F32(0))
        inv = np.where(pos, f32(F32(E4M3_MAX) / np.where(pos, amax, F32(1))), F32(0))
        codes = np.zeros((nb * BLOCK, R.shape[1]), np.uint8)
        codes[:N] = e4m3_encode(f32(R * inv[None, :]))
        out.update(v_codes=codes, v_scales=sv.astype(np.float32))
        out["v_res"] = e4m3_decode(codes[:N]) * sv.astype(np.float64)[None, :]
    elif v_format == "nvfp4":
        out.update(_nvfp4_encode(R, N))
    elif v_format == "mxfp4":
        out.update(_mxfp4_encode(R, N))
    else:
        raise ValueError(v_format)
    return out


def _nvfp4_encode(R: np.ndarray, N: int):
    """NVFP4 residual (4-bit path): E2M1 values with one E4M3 scale per 16 values.

    [digest] V-Smooth paragraph: the 4-bit path quantises the residual to NVFP4;
    NVFP4 = E2M1 values + an E4M3 scale per 16 elements.  Readings: the 16-value
    groups run along the token axis (16 consecutive permuted tokens of one
    channel, inside one block; a partial group's amax is over its valid tokens);
    a per-(batch, head) float32 second-level scale St = amax_all / (6 * 448);
    group scale code sg = E4M3(g_amax / (6 * St)); value codes
    E2M1(R / (dec(sg) * St)); a zero divisor gives zero codes."""
    d = R.shape[1]
    nb = n_blocks(N)
    Np = nb * BLOCK
    amax_all = F32(np.max(np.abs(R))) if N > 0 else F32(0)
    St = F32(amax_all / F32(6.0 * E4M3_MAX))
    Rp = np.zeros((Np, d), np.float32)
    Rp[:N] = R
    G = Np // 16
    g_amax = np.max(np.abs(Rp.reshape(G, 16, d)), axis=1)            # [G, d]
    if St > 0:
        sg = e4m3_encode(f32(g_amax / F32(F32(6.0) * St)))
    else:
        sg = np.zeros((G, d), np.uint8)
    dsg = f32(f32(e4m3_decode(sg)) * St)                                # [G, d]
    den = np.repeat(dsg, 16, axis=0)                                    # [Np, d]
    safe = np.where(den > 0, den, F32(1))
    vals = np.where(den > 0, f32(Rp / safe), F32(0))
    nib = e2m1_encode(vals)
    nib[N:] = 0
    res = e2m1_decode(nib[:N]) * e4m3_decode(np.repeat(sg, 16, axis=0)[:N]) * np.float64(St)
    return dict(v_nibbles=nib, v_group_scales=sg, v_scales=np.array([St], np.float32), v_res=res)


def mxfp4_groups(Np: int) -> np.ndarray:
    """Group index of every padded permuted row for the MXFP4 residual: within
    each 128-row block, half h (rows 64h .. 64h+63) and g = bit 4 of the row
    offset in that half, so group (t, h, g) holds rows 64h + 16g + [0, 16) and
    64h + 32 + 16g + [0, 16): the 32 values one lane of the block-scaled FP4
    matrix instruction holds against the P operand layout.  Index 4t + 2h + g."""
    u = np.arange(Np) % BLOCK
    h = u // 64
    g = (u % 64 // 16) % 2
    return (np.arange(Np) // BLOCK) * 4 + 2 * h + g


def _mxfp4_encode(R: np.ndarray, N: int):
    """MXFP4 residual: E2M1 values with one E8M0 (power-of-two) scale per 32.

    Not a format of the pages: their 4-bit path is NVFP4 ([digest] V-Smooth
    paragraph and preprocessing paragraph), whose per-16 scales would have to
    be applied in the softmax; MI355X's block-scaled FP4 matrix instruction
    applies E8M0 scales itself, so this is the 4-bit V-Smooth residual in the
    hardware's own format.  Readings: the OCP MX rule for the shared scale,
    X = 2^(floor(log2 amax) - 2) (2 = the largest E2M1 exponent), E8M0 code
    clamped to [0, 254]; an all-zero group gets code 0 and zero values; values
    E2M1_RNE_SAT(R / X) (saturating at 6).  Groups: mxfp4_groups; padding rows
    count as zero.  V carries no per-channel scale on this path (v_scales = 1).
    Returns v_nibbles [Np, d] (row order), v_mx_scales [nb, 2(h), 2(g), d]
    (E8M0 codes), v_scales ones [d], v_res (decoded residual [N, d], float64)."""
    d = R.shape[1]
    nb = n_blocks(N)
    Np = nb * BLOCK
    Rp = np.zeros((Np, d), np.float32)
    Rp[:N] = R
    gid = mxfp4_groups(Np)
    amax = np.zeros((4 * nb, d), np.float32)
    np.maximum.at(amax, gid, np.abs(Rp))
    _, ex = np.frexp(amax.astype(np.float64))          # amax = m * 2^ex, m in [0.5, 1)
    code = np.clip(ex - 1 - 2 + 127, 0, 254).astype(np.int64)
    code = np.where(amax > 0, code, 0)
    X = np.ldexp(np.float64(1.0), code - 127)           # exact powers of two
    vals = f32(Rp.astype(np.float64) / X[gid])          # power-of-two division, then float32
    nib = e2m1_encode(vals)
    nib[N:] = 0
    res = e2m1_decode(nib[:N]) * X[gid][:N]
    scales = code.reshape(nb, 2, 2, d).astype(np.uint8)
    return dict(v_nibbles=nib, v_mx_scales=scales, v_scales=np.ones(d, np.float32), v_res=res)


# ---------------------------------------------------------------------------
# P tile: ExpCast-FP8 and the conventional paths
# ---------------------------------------------------------------------------

EXPCAST_OFFSET = F32(55.65)   # 56 + beta, beta = -0.35; float32 0x425E999A


def score_scale(softmax_scale: float) -> np.float32:
    """c0 = float32(softmax_scale * log2(e)): turns a score into log2 units."""
    return F32(np.float64(F32(softmax_scale)) * LOG2E)


def expcast_codes(S: np.ndarray, kap: np.ndarray, mx: np.ndarray, octave_offset: int = 0) -> np.ndarray:
    """ExpCast-FP8: the E4M3 byte of p = 2^(S*kap - mx) written straight from
    the log-domain score.

    [digest] ExpCast-FP8 paragraph: the map from log-domain score to the E4M3
    byte is affine: one fused multiply-add, round to nearest even, clip to the
    normal range; beta = -0.35 centres the mantissa error and the constants come
    from the format.  [news] "ExpCast-FP8": read as an integer an E4M3 byte is
    about 8*log2(v) + 56.
    Exact reading: A = 8*kap, Bc = float32(55.65 - 8*mx),
    code = RNE(fmaf(S, A, Bc)); codes below 8 (under the normal range) -> 0x00;
    codes above 56 cannot occur and are clamped as a guard.
    S: float32 [R, T]; kap, mx: float32 [R].
    octave_offset (a fidelity diagnostic only, never the method's default):
    P pre-scaled by 2^octave_offset, i.e. 8*octave_offset added to the
    constant; the row maximum then maps to code 56 + 8*octave_offset (at most
    8 octaves keeps every code finite), so fewer small probabilities fall below
    the normal range; the normalisation cancels the scale."""
    kap = f32(kap)
    A = f32(F32(8.0) * kap)
    Bc = f32(f32(EXPCAST_OFFSET + F32(8 * octave_offset)) - f32(F32(8.0) * f32(mx)))
    code_f = fma_f32(S, A[:, None], Bc[:, None])
    c = np.rint(code_f.astype(np.float64))
    c = np.where(c < 8, 0, np.minimum(c, 56 + 8 * octave_offset))
    return c.astype(np.uint8)


def exp2_probs_f32(S: np.ndarray, kap: np.ndarray, mx: np.ndarray) -> np.ndarray:
    """Conventional softmax numerator in float32: p = exp2(float32(S*kap) - mx),
    the stage ExpCast replaces ([insight] "The Bottleneck...": FP32 exponent then
    conversion).  exp2 is evaluated in float64 and rounded once to float32."""
    x = f32(S * f32(kap)[:, None])
    d = f32(x - f32(mx)[:, None])
    return f32(np.exp2(d.astype(np.float64)))


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def online_attention(Qd, Kd, Vres, means, N, qscale_rows, kscales, c0, p_mode, rows,
                     record=None, scores=None, octave_offset=0):
    """Blockwise non-causal attention with online softmax and block-mean restore.

    For each KV block t in permuted order (the order matters: P codes depend on
    the running max):
      S   = Q_codes . K_codes_t^T        (exact in float64, rounded once to float32)
      kap = float32(float32(sq*sk_t) * c0)
      mx' = max(mx, float32(max_j S * kap))
      P   = decoded P codes (ExpCast or conventional), masked keys absent
      a   = 2^(mx - mx')  (0 on the first block)
      s   = sum_j P            (the row sum online softmax already keeps)
      l   = a*l + s
      U   = a*U + P @ Vres_t + s (x) mean_t       (mean restore: one outer product)
    O = U / l.
    [digest] V-Smooth paragraph: the block means are added back through the row
    sums online softmax already accumulates, with one outer product and no second
    pass over V.  [news] "V-Smooth", item Restore.
    Qd, Kd: decoded codes (float64); Vres: residual in real units (float64 [N, d]);
    means: float64 [nb, d].  rows: the query rows to compute.
    scores: optional float32 [N, >= N] scores to use in place of Q.K^T (to replay
    the method on a device's own scores, key index in permuted order)."""
    nb = n_blocks(N)
    R = len(rows)
    d = Vres.shape[1]
    q = Qd[rows]
    sq = f32(qscale_rows)
    mx = np.full(R, -np.inf)          # float64 holder; float32 values in the quantised modes
    l = np.zeros(R)
    U = np.zeros((R, d))
    srows = None if scores is None else np.asarray(scores)[rows]
    for t in range(nb):
        k0, k1 = t * BLOCK, min(N, (t + 1) * BLOCK)
        S64 = q @ Kd[k0:k1].T if scores is None else f32(srows[:, k0:k1]).astype(np.float64)
        kap = f32(f32(sq * F32(kscales[t])) * F32(c0))
        if p_mode == "exact":          # no rounding anywhere (used to pin the algebra)
            x = S64 * kap.astype(np.float64)[:, None]
            mx_new = np.maximum(mx, x.max(axis=1))
            codes = None
            P = np.exp2(x - mx_new[:, None])
        else:
            S = S64.astype(np.float32)
            xmax = f32(S.max(axis=1) * kap)
            mx_new = np.maximum(mx, xmax.astype(np.float64))
            m32 = mx_new.astype(np.float32)
            if p_mode == "expcast":
                codes = expcast_codes(S, kap, m32, octave_offset)
                P = e4m3_decode(codes)
            elif p_mode == "fp32exp_e4m3":
                codes = e4m3_encode(exp2_probs_f32(S, kap, m32))
                P = e4m3_decode(codes)
            elif p_mode == "fp32_bf16":
                codes = bf16_round(exp2_probs_f32(S, kap, m32))
                P = bf16_to_f32(codes).astype(np.float64)
            else:
                raise ValueError(p_mode)
        alpha = np.where(np.isneginf(mx), 0.0, np.exp2(mx - mx_new))
        s = P.sum(axis=1)
        l = alpha * l + s
        U = alpha[:, None] * U + P @ Vres[k0:k1] + s[:, None] * means[t][None, :]
        if record is not None:
            record.append(dict(t=t, S=None if p_mode == "exact" else S, kap=kap,
                               mx=mx_new.astype(np.float32), codes=codes))
        mx = mx_new
    return U / l[:, None]


def vc_attention_head(prep: dict, softmax_scale: float, p_mode: str, rows=None, record=None, scores=None,
                      octave_offset: int = 0):
    """VC attention output (float64 [rows, d], original query order) for one
    (batch, head) from the preprocessed codes of preprocess_head().  `scores`
    optionally replaces the exact Q.K^T (see online_attention); octave_offset
    is the ExpCast fidelity diagnostic of expcast_codes (0 = the method)."""
    N = prep["N"]
    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows)
    Qd = e4m3_decode(prep["q_codes"])
    Kd = e4m3_decode(prep["k_codes"])
    means = bf16_to_f32(prep["means"]).astype(np.float64)
    sq = prep["q_scales"][rows // BLOCK]
    return online_attention(Qd, Kd, prep["v_res"], means, N, sq, prep["k_scales"],
                            score_scale(softmax_scale), p_mode, rows, record, scores, octave_offset)


def expcast_given_scores(S_tiles, kap_tiles, N):
    """Replay ExpCast on given float32 score tiles (rows x 128 per KV block, in
    permuted block order) with the running max of the method; returns the P codes
    per tile.  Used to check P bytes "given S" against a device's own scores."""
    out = []
    mx = None
    for t, (S, kap) in enumerate(zip(S_tiles, kap_tiles)):
        k1 = min(N, (t + 1) * BLOCK) - t * BLOCK
        Sv = f32(S)[:, :k1]
        kap = f32(kap)
        xmax = f32(Sv.max(axis=1) * kap)
        mx = xmax if mx is None else np.maximum(mx, xmax)
        c = np.zeros(f32(S).shape, np.uint8)
        c[:, :k1] = expcast_codes(Sv, kap, mx)
        out.append(c)
    return out


def exact_attention(q_bf16, k_bf16, v_bf16, softmax_scale: float, rows=None) -> np.ndarray:
    """softmax(Q K^T * scale) V in float64 from the bf16 inputs (fidelity yardstick)."""
    q = bf16_to_f32(q_bf16).astype(np.float64)
    k = bf16_to_f32(k_bf16).astype(np.float64)
    v = bf16_to_f32(v_bf16).astype(np.float64)
    if rows is not None:
        q = q[np.asarray(rows)]
    S = (q @ k.T) * float(F32(softmax_scale))
    S -= S.max(axis=1, keepdims=True)
    P = np.exp(S)
    return (P @ v) / P.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# Whole-tensor drivers and diagnostics
# ---------------------------------------------------------------------------

def preprocess(Q, K, V, perm, v_format="e4m3", rope_cs=None, hadamard=False):
    """[B, H, N, d] bf16 bits (Q may be None) -> list of per-head dicts.  One
    RoPE table [N, 64, 2] serves every (batch, head)."""
    B, H = K.shape[:2]
    return [[preprocess_head(None if Q is None else Q[b, h], K[b, h], V[b, h], perm[b, h], v_format,
                             rope_cs, hadamard)
             for h in range(H)] for b in range(B)]


def block_energy_fraction(v_f32: np.ndarray, order: np.ndarray | None = None) -> float:
    """Share of the Values' energy the 128-token block means carry:
    sum_t n_t |mean_t|^2 / sum_j |v_j|^2 (float64, exact means).  [digest]
    V-Smooth paragraph quotes 8% in sequence order and 36% after sorting on
    Wan2.2 heads; synthetic inputs compare only in kind."""
    v = np.asarray(v_f32, np.float64)
    if order is not None:
        v = v[order]
    N = v.shape[0]
    tot = 0.0
    for t in range(n_blocks(N)):
        blk = v[t * BLOCK: (t + 1) * BLOCK]
        tot += blk.shape[0] * float(np.sum(blk.mean(axis=0) ** 2))
    return tot / float(np.sum(v * v))


def total_variation(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Per-row total variation between two nonnegative row vectors, each
    normalised to sum 1."""
    p = np.asarray(p, np.float64)
    q = np.asarray(q, np.float64)
    return 0.5 * np.abs(p / p.sum(axis=-1, keepdims=True) - q / q.sum(axis=-1, keepdims=True)).sum(axis=-1)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
