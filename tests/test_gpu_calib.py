"""The benchmark's MFMA-rate calibration kernel (libmla_calib.so) does the
matrix work its FLOP count assumes: on a table of ones every MFMA adds K
(16 for 32x32x16, 32 for 16x16x32) to each accumulator element, so the
per-thread sum of the accumulators after `iters` iterations of 64 MFMAs per
wave is exact and known in closed form."""

import ctypes
import os

import pytest
import torch

from mla_latent_kv_attn_amd import build as _b
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def calib():
    if not os.path.exists(_b.CALIB_LIB):
        pytest.fail("libmla_calib.so not built")
    lib = ctypes.CDLL(_b.CALIB_LIB)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.mla_calib_mfma_rate.argtypes = [vp, vp, i, i, i, vp]
    lib.mla_calib_mfma_rate.restype = i
    return lib


def _run(lib, table, blocks, iters, shape):
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    assert lib.mla_calib_mfma_rate(table.data_ptr(), out.data_ptr(), blocks, iters, shape, st) == 0
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("shape,per_iter", [(32, 64 * 16 * 16), (16, 32 * 8 * 32)])
def test_calibration_kernel_sum_on_ones_is_exact(calib, shape, per_iter):
    # 32x32x16: 4 chains x 16 elements per lane, 16 MFMAs per chain and
    # iteration, +16 each; 16x16x32: 8 chains x 4 elements, 8 MFMAs per
    # chain and iteration, +32 each.  Both give 64 MFMAs per wave and
    # iteration.
    say(f"calibration kernel shape {shape}")
    ones = torch.ones(65536 * 8, dtype=torch.bfloat16, device=DEV)
    iters = 3
    out = _run(calib, ones, 2, iters, shape)
    assert torch.all(out == float(per_iter * iters)), out[:8]
    zeros = torch.zeros_like(ones)
    assert torch.all(_run(calib, zeros, 2, iters, shape) == 0)
