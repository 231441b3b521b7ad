"""The roofline's calibration library (libattn_ceilings.so): exports, argument checks, and on the
GPU that the measured rates are positive and physically possible."""
import ctypes
import math
import os
import re

import pytest

from attention_forward_06_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_ceilings.h")
HIP_ERROR_INVALID_VALUE = 1
# dense bf16 MFMA at the top clock: 256 CUs x 4 SIMDs x 1024 FLOP per clock x 2.4 GHz
PHYSICAL_MFMA_TFLOPS = 256 * 4 * 1024 * 2.4e9 / 1e12


@pytest.fixture(scope="module")
def lib():
    return binding.load_ceilings()


def _declared_functions():
    with open(HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_declares_both_ceilings():
    assert _declared_functions() == ["attn_ceiling_hbm_3r1w", "attn_ceiling_mfma_bf16"]


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value, name


@pytest.mark.parametrize("warmup,launches", [(-1, 1), (0, 0)])
def test_mfma_rejects_bad_counts_before_any_hip_call(lib, warmup, launches):
    out = ctypes.c_double(-7.0)
    assert lib.attn_ceiling_mfma_bf16(warmup, launches, ctypes.byref(out)) == HIP_ERROR_INVALID_VALUE
    assert out.value == -7.0
    assert lib.attn_ceiling_mfma_bf16(0, 1, None) == HIP_ERROR_INVALID_VALUE


@pytest.mark.parametrize("warmup,launches,nbytes", [(-1, 1, 1024), (0, 0, 1024), (0, 1, 0), (0, 1, 24)])
def test_hbm_rejects_bad_arguments_before_any_hip_call(lib, warmup, launches, nbytes):
    out = ctypes.c_double(-7.0)
    assert lib.attn_ceiling_hbm_3r1w(warmup, launches, nbytes, ctypes.byref(out)) == HIP_ERROR_INVALID_VALUE
    assert out.value == -7.0


@pytest.mark.gpu
def test_measured_ceilings_are_physical():
    mfma = binding.ceiling_mfma_bf16(warmup=20, launches=50)
    assert math.isfinite(mfma) and 100.0 < mfma <= PHYSICAL_MFMA_TFLOPS * 1.001
    hbm = binding.ceiling_hbm_3r1w(warmup=2, launches=5, bytes_per_array=256 << 20)
    assert math.isfinite(hbm) and 100.0 < hbm < 20000.0
