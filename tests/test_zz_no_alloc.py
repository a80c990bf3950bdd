"""The allocation-free preprocessing entry point (vc_preprocess_quant_noalloc),
called through the C ABI, against vc_preprocess_quant with a caller workspace:
every output bit-identical, on two calls in a row, the second smaller and with
smaller residuals (so amax accumulators left over from the first call would show
in its V scales)."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import vc_workloads as W

pytestmark = pytest.mark.gpu


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


def _outputs_like(ref):
    return {k: torch.full_like(v, 0x5A if v.dtype == torch.uint8 else 3) for k, v in ref.items()
            if isinstance(v, torch.Tensor)}


def _noalloc(vc, Qd, Kd, Vd, perm, fmt):
    B, H, N, d = Kd.shape
    ref = vc.preprocess_quant(Qd, Kd, Vd, perm, fmt)        # the workspace entry point
    got = _outputs_like(ref)
    P = lambda k: None if got.get(k) is None else ctypes.c_void_p(got[k].data_ptr())
    T = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = vc.lib().vc_preprocess_quant_noalloc(T(Qd), T(Kd), T(Vd), T(perm), B, H, N, d, ref["v_format"],
                                              P("q_codes"), P("q_scales"), P("k_codes"), P("k_scales"),
                                              P("v_codes"), P("v_scales"), P("v_group_scales"), P("v_means"),
                                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, vc.lib().vc_status_string(rc)
    torch.cuda.synchronize()
    for k, v in got.items():
        assert torch.equal(v, ref[k]), f"{k} differs ({fmt}, B{B} H{H} N{N})"


@pytest.mark.parametrize("fmt", ["e4m3", "nvfp4"])
def test_allocation_free_preprocessing_matches_the_workspace_call(vc, fmt):
    dev = torch.device("cuda:0")
    _say(f"allocation-free preprocessing, {fmt}: B1 H8 N3000 (V x 10), then B1 H2 N300")
    Q, K, V = W.custom_inputs(1, 8, 3000, seed=91, recipe="clustered")
    V = (V.float() * 10).to(torch.bfloat16)
    Qd, Kd, Vd = Q.to(dev), K.to(dev), V.to(dev)
    perm, _, _ = vc.vsmooth_group(Vd, 16, 3)
    _noalloc(vc, Qd, Kd, Vd, perm, fmt)
    Q2, K2, V2 = W.custom_inputs(1, 2, 300, seed=92, recipe="clustered")
    Qd2, Kd2, Vd2 = Q2.to(dev), K2.to(dev), V2.to(dev)
    perm2, _, _ = vc.vsmooth_group(Vd2, 8, 3)
    _noalloc(vc, Qd2, Kd2, Vd2, perm2, fmt)
