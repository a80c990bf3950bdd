"""ctypes binding of libvc.so (include/vc.h).  Argument marshalling only: every
step of the path runs in the HIP kernels.  Tensors must live on the GPU; the
library is required (there is no fallback).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(HERE, "libvc.so")

P_EXPCAST, P_FP32EXP_E4M3, P_FP32_BF16 = 0, 1, 2
V_E4M3, V_NVFP4, V_MXFP4 = 0, 1, 2
_PMODES = {"expcast": P_EXPCAST, "fp32exp_e4m3": P_FP32EXP_E4M3, "fp32_bf16": P_FP32_BF16}
_VFMTS = {"e4m3": V_E4M3, "nvfp4": V_NVFP4, "mxfp4": V_MXFP4}
D = 128
BLOCK = 128

_lib = None


class VcError(RuntimeError):
    pass


def lib():
    """Load libvc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise VcError(f"{lib_path} is missing: build it with `python -m bit_attention_video_vc_amd.build`")
        L = ctypes.CDLL(lib_path)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.vc_vsmooth_group_workspace.argtypes = [I, I, I, I, I]
        L.vc_vsmooth_group_workspace.restype = Z
        L.vc_vsmooth_group.argtypes = [P, I, I, I, I, I, I, P, P, P, P, Z, P]
        L.vc_preprocess_workspace.argtypes = [I, I, I, I, I]
        L.vc_preprocess_workspace.restype = Z
        L.vc_preprocess_quant.argtypes = [P, P, P, P, I, I, I, I, I, P, P, P, P, P, P, P, P, P, Z, P]
        L.vc_preprocess_quant_ex.argtypes = [P, P, P, P, I, I, I, I, I, P, I, P, P, P, P, P, P, P, P, P, Z, P]
        L.vc_attn_fp8_fwd.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, F, I, I, P, P]
        L.vc_attn_bf16_workspace.argtypes = [I, I, I, I]
        L.vc_attn_bf16_workspace.restype = Z
        L.vc_attn_bf16_fwd.argtypes = [P, P, P, I, I, I, I, F, P, P, Z, P]
        L.vc_attn_fp8_fwd_dump.argtypes = [P, P, P, P, P, P, P, I, I, I, I, F, I, P, P, P, P]
        L.vc_attn_fwd_dump.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, F, I, I, P, P, P, P]
        L.vc_device_probe.argtypes = [I, P, P, I, P]
        L.vc_preprocess_quant_noalloc.argtypes = [P, P, P, P, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
        L.vc_preprocess_noalloc_max_scratch.restype = Z
        for f in ("vc_vsmooth_group", "vc_preprocess_quant", "vc_preprocess_quant_ex", "vc_attn_fp8_fwd", "vc_attn_bf16_fwd",
                  "vc_attn_fp8_fwd_dump", "vc_attn_fwd_dump", "vc_device_probe", "vc_preprocess_quant_noalloc"):
            getattr(L, f).restype = I
        for f in ("vc_group_due", "vc_group_source"):
            getattr(L, f).argtypes = [I, I, I, F]
            getattr(L, f).restype = I
        L.vc_group_count.argtypes = [I, I, F]
        L.vc_group_count.restype = I
        L.vc_status_string.argtypes = [I]
        L.vc_status_string.restype = ctypes.c_char_p
        L.vc_version.restype = ctypes.c_char_p
        L.vc_last_hip_error.restype = I
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        raise VcError(f"{what} failed: {rc} ({lib().vc_status_string(rc).decode()})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t):
    if not t.is_cuda:
        raise VcError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise VcError("tensors must be contiguous")
    return t.device


def _bits(t):
    """bf16 tensor -> same memory viewed as int16 (the ABI takes uint16 bits)."""
    if t.dtype != torch.bfloat16:
        raise VcError("expected a bfloat16 tensor")
    return t


def vsmooth_group(V: torch.Tensor, k: int, iters: int, want_labels=False, want_centroids=False):
    """V [B,H,N,128] bf16 -> perm int32 [B,H,N] (and labels, centroids if asked)."""
    dev = _dev(_bits(V))
    B, H, N, d = V.shape
    L = lib()
    ws_bytes = L.vc_vsmooth_group_workspace(B, H, N, d, k)
    if ws_bytes == 0:
        raise VcError("bad V-Smooth shape")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    perm = torch.empty(B, H, N, dtype=torch.int32, device=dev)
    labels = torch.empty(B, H, N, dtype=torch.int32, device=dev) if want_labels else None
    cents = torch.empty(B, H, k, d, dtype=torch.float32, device=dev) if want_centroids else None
    _check(L.vc_vsmooth_group(_ptr(V), B, H, N, d, k, iters, _ptr(perm), _ptr(labels), _ptr(cents),
                              _ptr(ws), ws_bytes, _stream(dev)), "vc_vsmooth_group")
    return perm, labels, cents


def preprocess_quant(Q, K, V, perm, v_format="e4m3", rope_cs=None, hadamard=False):
    """Gather, block means and quantisation.  Q may be None.  Returns a dict of
    device tensors in the layouts of include/vc.h.  rope_cs (fp32 [N, 64, 2]
    cos/sin table on the GPU) and hadamard select the Q/K transforms of
    vc_preprocess_quant_ex."""
    fmt = _VFMTS[v_format] if isinstance(v_format, str) else v_format
    dev = _dev(_bits(K))
    _dev(_bits(V))
    _dev(perm)
    if Q is not None:
        _dev(_bits(Q))
    B, H, N, d = K.shape
    nb = -(-N // BLOCK)
    Np = nb * BLOCK
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(N=N, B=B, H=H, v_format=fmt)
    out["q_codes"] = torch.empty(B, H, Np, d, **u8) if Q is not None else None
    out["q_scales"] = torch.empty(B, H, nb, **f32) if Q is not None else None
    out["k_codes"] = torch.empty(B, H, Np, d, **u8)
    out["k_scales"] = torch.empty(B, H, nb, **f32)
    if fmt == V_E4M3:
        out["v_codes"] = torch.empty(B, H, nb, d, BLOCK, **u8)
        out["v_scales"] = torch.empty(B, H, d, **f32)
        out["v_group_scales"] = None
    elif fmt == V_MXFP4:
        out["v_codes"] = torch.empty(B, H, nb, d, BLOCK // 2, **u8)
        out["v_scales"] = torch.empty(B, H, d, **f32)
        out["v_group_scales"] = torch.empty(B, H, nb, d, 2, 2, **u8)
    else:
        out["v_codes"] = torch.empty(B, H, nb, d, BLOCK // 2, **u8)
        out["v_scales"] = torch.empty(B, H, **f32)
        out["v_group_scales"] = torch.empty(B, H, Np // 16, d, **u8)
    out["v_means"] = torch.empty(B, H, nb, d, dtype=torch.bfloat16, device=dev)
    L = lib()
    ws_bytes = L.vc_preprocess_workspace(B, H, N, d, fmt)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    if rope_cs is not None:
        _dev(rope_cs)
        if rope_cs.dtype != torch.float32 or tuple(rope_cs.shape) != (N, 64, 2):
            raise VcError("rope_cs must be float32 [N, 64, 2]")
    _check(L.vc_preprocess_quant_ex(_ptr(Q), _ptr(K), _ptr(V), _ptr(perm), B, H, N, d, fmt, _ptr(rope_cs),
                                    1 if hadamard else 0,
                                    _ptr(out["q_codes"]), _ptr(out["q_scales"]), _ptr(out["k_codes"]),
                                    _ptr(out["k_scales"]), _ptr(out["v_codes"]), _ptr(out["v_scales"]),
                                    _ptr(out["v_group_scales"]), _ptr(out["v_means"]), _ptr(ws), ws_bytes,
                                    _stream(dev)), "vc_preprocess_quant_ex")
    return out


def attn_fp8_fwd(prep: dict, softmax_scale: float | None = None, p_mode="expcast", out=None):
    """VC attention from the preprocessed codes; returns fp32 [B,H,N,128]."""
    pm = _PMODES[p_mode] if isinstance(p_mode, str) else p_mode
    B, H, N = prep["B"], prep["H"], prep["N"]
    dev = prep["k_codes"].device
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty(B, H, N, D, dtype=torch.float32, device=dev)
    _check(lib().vc_attn_fp8_fwd(_ptr(prep["q_codes"]), _ptr(prep["q_scales"]), _ptr(prep["k_codes"]),
                                 _ptr(prep["k_scales"]), _ptr(prep["v_codes"]), _ptr(prep["v_scales"]),
                                 _ptr(prep["v_group_scales"]), _ptr(prep["v_means"]), B, H, N, D,
                                 float(softmax_scale), pm, prep["v_format"], _ptr(out), _stream(dev)),
           "vc_attn_fp8_fwd")
    return out


def attn_fp8_fwd_dump(prep: dict, softmax_scale: float | None = None, p_mode="expcast"):
    """attn_fp8_fwd plus the per-(query, key) scores and P bytes (small N only)."""
    pm = _PMODES[p_mode] if isinstance(p_mode, str) else p_mode
    B, H, N = prep["B"], prep["H"], prep["N"]
    Np = -(-N // BLOCK) * BLOCK
    dev = prep["k_codes"].device
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    out = torch.empty(B, H, N, D, dtype=torch.float32, device=dev)
    s = torch.empty(B, H, N, Np, dtype=torch.float32, device=dev)
    p = torch.empty(B, H, N, Np, dtype=torch.uint8, device=dev)
    _check(lib().vc_attn_fp8_fwd_dump(_ptr(prep["q_codes"]), _ptr(prep["q_scales"]), _ptr(prep["k_codes"]),
                                      _ptr(prep["k_scales"]), _ptr(prep["v_codes"]), _ptr(prep["v_scales"]),
                                      _ptr(prep["v_means"]), B, H, N, D, float(softmax_scale), pm,
                                      _ptr(out), _ptr(s), _ptr(p), _stream(dev)), "vc_attn_fp8_fwd_dump")
    return out, s, p


def attn_fwd_dump(prep: dict, softmax_scale: float | None = None, p_mode="expcast"):
    """vc_attn_fwd_dump: the attention output plus the per-(query, key) scores
    and P values of any pairing (E4M3 bytes as uint8, bf16 P bits as int16)."""
    pm = _PMODES[p_mode] if isinstance(p_mode, str) else p_mode
    B, H, N = prep["B"], prep["H"], prep["N"]
    Np = -(-N // BLOCK) * BLOCK
    dev = prep["k_codes"].device
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    out = torch.empty(B, H, N, D, dtype=torch.float32, device=dev)
    s = torch.empty(B, H, N, Np, dtype=torch.float32, device=dev)
    p = torch.empty(B, H, N, Np, dtype=torch.int16 if pm == P_FP32_BF16 else torch.uint8, device=dev)
    _check(lib().vc_attn_fwd_dump(_ptr(prep["q_codes"]), _ptr(prep["q_scales"]), _ptr(prep["k_codes"]),
                                  _ptr(prep["k_scales"]), _ptr(prep["v_codes"]), _ptr(prep["v_scales"]),
                                  _ptr(prep["v_group_scales"]), _ptr(prep["v_means"]), B, H, N, D,
                                  float(softmax_scale), pm, prep["v_format"], _ptr(out), _ptr(s), _ptr(p),
                                  _stream(dev)), "vc_attn_fwd_dump")
    return out, s, p


_PROBES = {"cvt_fp8": 0, "cvt_u8": 1, "exp2": 2, "mfma_32x32x64": 3, "mfma_16x16x128": 4,
           "hbm_read": 5, "hbm_copy": 6, "hbm_read2_write1": 7, "mfma_fp8_rate": 8,
           "valu_rate": 9, "lds_copy_rate": 10}


def device_probe(what: str, inp: torch.Tensor, out: torch.Tensor, n: int):
    """vc_device_probe: run one gfx950 instruction on `inp` into `out` (device tensors)."""
    _dev(inp)
    _dev(out)
    _check(lib().vc_device_probe(_PROBES[what], _ptr(inp), _ptr(out), int(n), _stream(inp.device)),
           "vc_device_probe")
    return out


def attn_bf16_fwd(Q, K, V, softmax_scale: float | None = None, out=None, workspace=None):
    """bf16 flash-attention comparator; returns fp32 [B,H,N,128]."""
    dev = _dev(_bits(Q))
    _dev(_bits(K))
    _dev(_bits(V))
    B, H, N, d = Q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
    L = lib()
    ws_bytes = L.vc_attn_bf16_workspace(B, H, N, d)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(L.vc_attn_bf16_fwd(_ptr(Q), _ptr(K), _ptr(V), B, H, N, d, float(softmax_scale), _ptr(out),
                              _ptr(workspace), ws_bytes, _stream(dev)), "vc_attn_bf16_fwd")
    return out


def unswizzle_v_codes(v_codes: torch.Tensor, N: int) -> torch.Tensor:
    """E4M3 V codes from the per-block transposed layout [B,H,nb,128(ch),128(row)]
    to row-major permuted order [B,H,Np,128] (host-side helper for checks)."""
    B, H, nb, d, r = v_codes.shape
    return v_codes.permute(0, 1, 2, 4, 3).reshape(B, H, nb * r, d)


def group_due(step: int, total_steps: int, reuse: int = 4, fraction: float = 0.25) -> bool:
    """True if denoising step `step` computes a new V-Smooth permutation (include/vc.h)."""
    r = lib().vc_group_due(step, total_steps, reuse, fraction)
    _check(min(r, 0), "vc_group_due")
    return bool(r)


def group_source(step: int, total_steps: int, reuse: int = 4, fraction: float = 0.25) -> int:
    """The step whose permutation denoising step `step` uses."""
    r = lib().vc_group_source(step, total_steps, reuse, fraction)
    _check(min(r, 0), "vc_group_source")
    return r


def group_count(total_steps: int, reuse: int = 4, fraction: float = 0.25) -> int:
    """Number of regrouping steps over a trajectory of `total_steps`."""
    r = lib().vc_group_count(total_steps, reuse, fraction)
    _check(min(r, 0), "vc_group_count")
    return r


class PermutationCache:
    """One V-Smooth permutation per attention layer across a denoising trajectory.

    `perm(layer, step, V)` regroups when the cadence says so (vc_group_due) and
    otherwise returns the permutation cached for that layer, after checking that
    it came from the step the cadence names (vc_group_source).  `group_fn` is
    vsmooth_group unless given (it must return the permutation first).
    """

    def __init__(self, total_steps: int, reuse: int = 4, fraction: float = 0.25, k: int = 64, iters: int = 8,
                 group_fn=None):
        group_count(total_steps, reuse, fraction)   # validates the cadence
        self.total_steps, self.reuse, self.fraction = total_steps, reuse, fraction
        self.k, self.iters = k, iters
        self.group_fn = group_fn if group_fn is not None else (lambda V, k, it: vsmooth_group(V, k, it))
        self._perms = {}
        self.group_calls = 0

    def perm(self, layer, step: int, V):
        if group_due(step, self.total_steps, self.reuse, self.fraction):
            self._perms[layer] = (step, self.group_fn(V, self.k, self.iters)[0])
            self.group_calls += 1
            return self._perms[layer][1]
        src = group_source(step, self.total_steps, self.reuse, self.fraction)
        cached = self._perms.get(layer)
        if cached is None or cached[0] != src:
            have = None if cached is None else cached[0]
            raise VcError(f"layer {layer!r}, step {step}: needs the permutation of step {src}, cache holds {have}")
        return cached[1]
