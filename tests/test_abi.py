"""CPU checks of the C ABI: libvc.so loads, exports every function include/vc.h
declares, and rejects bad arguments synchronously (no GPU call is made: the
library validates before it launches anything)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vc.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(vc_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    import bit_attention_video_vc_amd as vc
    return vc.lib()


def test_header_declares_the_four_entry_points():
    names = _declared()
    for n in ("vc_vsmooth_group", "vc_preprocess_quant", "vc_attn_fp8_fwd", "vc_attn_bf16_fwd"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings(L):
    assert L.vc_status_string(0) == b"ok"
    assert b"argument" in L.vc_status_string(-1)
    assert b"unsupported" in L.vc_status_string(-2)
    assert b"workspace" in L.vc_status_string(-3)
    assert L.vc_version().startswith(b"vc-attn")


def test_workspace_sizes(L):
    assert L.vc_vsmooth_group_workspace(1, 40, 75600, 128, 64) > 0
    assert L.vc_vsmooth_group_workspace(1, 1, 10, 64, 8) == 0       # d != 128
    assert L.vc_vsmooth_group_workspace(1, 1, 10, 128, 300) == 0    # k > 256
    assert L.vc_preprocess_workspace(1, 40, 75600, 128, 0) == 40 * 128 * 4
    assert L.vc_preprocess_workspace(2, 24, 32760, 128, 1) == 48 * 4


def test_argument_errors_are_synchronous(L):
    p = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    null = None
    # vsmooth: d, k, iters, null pointers, workspace
    assert L.vc_vsmooth_group(p, 1, 1, 8, 64, 4, 2, p, null, null, p, 1 << 20, null) == -2
    assert L.vc_vsmooth_group(p, 1, 1, 8, 128, 0, 2, p, null, null, p, 1 << 20, null) == -1
    assert L.vc_vsmooth_group(p, 1, 1, 8, 128, 257, 2, p, null, null, p, 1 << 20, null) == -1
    assert L.vc_vsmooth_group(p, 1, 1, 8, 128, 4, 0, p, null, null, p, 1 << 20, null) == -1
    assert L.vc_vsmooth_group(null, 1, 1, 8, 128, 4, 2, p, null, null, p, 1 << 20, null) == -1
    assert L.vc_vsmooth_group(p, 1, 1, 0, 128, 4, 2, p, null, null, p, 1 << 20, null) == -1
    assert L.vc_vsmooth_group(p, 1, 1, 8, 128, 4, 2, p, null, null, p, 8, null) == -3
    assert L.vc_vsmooth_group(p, 1, 1, 8, 128, 4, 2, p, null, null, null, 1 << 20, null) == -3
    # preprocess: unknown format, missing outputs, workspace
    args = [p, p, p, p, 1, 1, 8, 128]
    outs = [p, p, p, p, p, p, null, p]
    assert L.vc_preprocess_quant(*args, 7, *outs, p, 1 << 20, null) == -2
    assert L.vc_preprocess_quant(*args, 1, *outs, p, 1 << 20, null) == -1      # NVFP4 needs group scales
    assert L.vc_preprocess_quant(*args, 2, *outs, p, 1 << 20, null) == -1      # so does MXFP4
    assert L.vc_preprocess_quant(*args, 0, *outs, p, 4, null) == -3
    assert L.vc_preprocess_quant(p, p, p, p, 1, 1, 8, 96, 0, *outs, p, 1 << 20, null) == -2
    assert L.vc_preprocess_quant(p, null, p, p, 1, 1, 8, 128, 0, *outs, p, 1 << 20, null) == -1
    # the Q/K-transform variant: hadamard must be 0 or 1; the rest as above
    assert L.vc_preprocess_quant_ex(*args, 0, null, 2, *outs, p, 1 << 20, null) == -1
    assert L.vc_preprocess_quant_ex(*args, 7, p, 1, *outs, p, 1 << 20, null) == -2
    assert L.vc_preprocess_quant_ex(*args, 0, p, 1, *outs, p, 4, null) == -3
    # attention: pairing of modes, d, null out
    a = [p] * 8 + [1, 1, 8, 128, 0.1]
    assert L.vc_attn_fp8_fwd(*a, 2, 0, p, null) == -2       # bf16 P with E4M3 V: not a built pairing
    assert L.vc_attn_fp8_fwd(*a, 0, 1, p, null) == -2       # ExpCast with NVFP4: the pages exclude it
    assert L.vc_attn_fp8_fwd(*a, 2, 2, p, null) == -2       # bf16 P with MXFP4 V: not a built pairing
    a6 = [p] * 6 + [null, p] + [1, 1, 8, 128, 0.1]
    assert L.vc_attn_fp8_fwd(*a6, 0, 2, p, null) == -1      # MXFP4 needs its group scales
    assert L.vc_attn_fp8_fwd(*[p] * 8, 1, 1, 8, 64, 0.1, 0, 0, p, null) == -2
    assert L.vc_attn_fp8_fwd(*a, 0, 0, null, null) == -1
    assert L.vc_attn_bf16_fwd(p, p, p, 1, 1, 8, 64, 0.1, p, p, 1 << 20, null) == -2
    assert L.vc_attn_bf16_fwd(p, p, null, 1, 1, 8, 128, 0.1, p, p, 1 << 20, null) == -1
    assert L.vc_attn_bf16_fwd(p, p, p, 1, 1, 8, 128, 0.1, p, p, 16, null) == -3
    assert L.vc_attn_bf16_workspace(1, 2, 300, 128) == 2 * 3 * 128 * 256
    # a head's bytes must fit one 32-bit buffer record count: longer sequences are refused
    assert L.vc_attn_fp8_fwd(*[p] * 8, 1, 1, (1 << 25) + 1, 128, 0.1, 0, 0, p, null) == -1
    assert L.vc_attn_bf16_fwd(p, p, p, 1, 1, 1 << 24, 128, 0.1, p, p, 1 << 40, null) == -1
    assert L.vc_preprocess_quant(p, p, p, p, 1, 1, 1 << 24, 128, 0, *outs, p, 1 << 40, null) == -1
    assert L.vc_attn_fp8_fwd_dump(*[p] * 7, 1, 1, 8, 128, 0.1, 2, p, p, p, null) == -2


def test_test_hooks_reject_bad_arguments(L):
    p = ctypes.c_void_p(16)
    null = None
    a = [p] * 8 + [1, 1, 8, 128, 0.1]
    assert L.vc_attn_fwd_dump(*a, 0, 1, p, p, p, null) == -2          # ExpCast with NVFP4
    assert L.vc_attn_fwd_dump(*a, 2, 0, p, p, p, null) == -2          # bf16 P with E4M3 V
    assert L.vc_attn_fwd_dump(*a, 0, 0, p, null, p, null) == -1       # no score dump
    a6 = [p] * 6 + [null, p] + [1, 1, 8, 128, 0.1]
    assert L.vc_attn_fwd_dump(*a6, 0, 2, p, p, p, null) == -1         # MXFP4 needs its group scales
    assert L.vc_attn_fwd_dump(*a6, 2, 1, p, p, p, null) == -1         # so does NVFP4
    assert L.vc_attn_fwd_dump(*[p] * 8, 1, 1, 8, 64, 0.1, 0, 0, p, p, p, null) == -2
    assert L.vc_device_probe(11, p, p, 4, null) == -2
    assert L.vc_device_probe(0, p, p, 0, null) == -1
    assert L.vc_device_probe(0, null, p, 4, null) == -1


def test_allocation_free_preprocessing_rejects_problems_beyond_its_scratch(L):
    p = ctypes.c_void_p(16)
    null = None
    outs = [p, p, p, p, p, p, null, p]
    assert L.vc_preprocess_noalloc_max_scratch() == 1 << 20
    # E4M3 needs B*H*128 floats: 2049 heads exceed 1 MiB; checked before any GPU call
    assert L.vc_preprocess_quant_noalloc(p, p, p, p, 1, 2049, 8, 128, 0, *outs, null) == -5
    assert L.vc_preprocess_quant_noalloc(p, p, p, p, 3, 700, 8, 128, 2, *outs, null) == -5
    assert L.vc_preprocess_quant_noalloc(p, p, p, p, 1, 1, 8, 96, 0, *outs, null) == -2
    assert L.vc_preprocess_quant_noalloc(p, null, p, p, 1, 1, 8, 128, 0, *outs, null) == -1
    assert L.vc_preprocess_quant_noalloc(p, p, p, p, 1, 1, 8, 128, 7, *outs, null) == -2
    assert b"scratch" in L.vc_status_string(-5)
