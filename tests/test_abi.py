"""The C ABI: the library loads, exports every function include/mla_attn.h
declares, and rejects bad arguments on the host before touching a device.
No compute call is made here (these run without a GPU)."""

import ctypes
import os
import re

import pytest

from mla_latent_kv_attn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_header_declares_the_expected_api():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_strings(lib):
    for s in range(8):
        txt = lib.mla_status_string(s).decode()
        assert txt.startswith("MLA_"), txt
    assert lib.mla_status_string(99).decode() == "unknown mla_status_t"


P = 0x10000          # a 16-byte aligned fake device address (never dereferenced)
BAD = 0x10008        # misaligned


def _attn(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=2, N=256, D=64, scale=0.125, causal=0, dt=0):
    return lib.attn_fwd(q, k, v, o, lse, B, H, N, D, scale, causal, dt, None)


def test_attn_validation_codes(lib):
    assert _attn(lib, q=None) == binding.MLA_ERR_NULL
    assert _attn(lib, o=None) == binding.MLA_ERR_NULL
    assert _attn(lib, B=0) == binding.MLA_ERR_SHAPE
    assert _attn(lib, N=-1) == binding.MLA_ERR_SHAPE
    assert _attn(lib, N=(1 << 20) + 1) == binding.MLA_ERR_SHAPE
    assert _attn(lib, scale=0.0) == binding.MLA_ERR_SHAPE
    assert _attn(lib, scale=float("nan")) == binding.MLA_ERR_SHAPE
    assert _attn(lib, causal=2) == binding.MLA_ERR_SHAPE
    assert _attn(lib, D=128, dt=0) == binding.MLA_ERR_UNSUPPORTED
    assert _attn(lib, D=64, dt=1) == binding.MLA_ERR_UNSUPPORTED
    assert _attn(lib, dt=7) == binding.MLA_ERR_UNSUPPORTED
    assert _attn(lib, k=BAD) == binding.MLA_ERR_ALIGN
    assert _attn(lib, lse=BAD) == binding.MLA_ERR_ALIGN
    assert _attn(lib, N=0) == binding.MLA_OK        # nothing to do, nothing enqueued


def _chunk(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=64, Nk=256, D=64, scale=0.125, causal=1, dt=0):
    return lib.attn_fwd_chunk(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, dt, None)


def test_attn_chunk_validation_codes(lib):
    assert _chunk(lib, v=None) == binding.MLA_ERR_NULL
    assert _chunk(lib, Nq=-1) == binding.MLA_ERR_SHAPE
    assert _chunk(lib, Nk=-1) == binding.MLA_ERR_SHAPE
    assert _chunk(lib, Nk=(1 << 20) + 1) == binding.MLA_ERR_SHAPE
    assert _chunk(lib, causal=3) == binding.MLA_ERR_SHAPE
    assert _chunk(lib, D=128, dt=0) == binding.MLA_ERR_UNSUPPORTED
    assert _chunk(lib, o=BAD) == binding.MLA_ERR_ALIGN
    assert _chunk(lib, Nq=0) == binding.MLA_OK      # nothing to do, nothing enqueued


def _dec(lib, ql=P, qr=P, c=P, sl=P, o=P, lse=P, B=2, H=128, S=64, scale=0.04, ns=4, ws=P, wsb=1 << 30):
    return lib.mla_decode_fwd(ql, qr, c, sl, o, lse, B, H, S, scale, ns, ws, wsb, None)


def test_decode_validation_codes(lib):
    assert _dec(lib, c=None) == binding.MLA_ERR_NULL
    assert _dec(lib, sl=None) == binding.MLA_ERR_NULL
    assert _dec(lib, H=8) == binding.MLA_ERR_SHAPE
    assert _dec(lib, H=40) == binding.MLA_ERR_SHAPE
    assert _dec(lib, ns=0) == binding.MLA_ERR_SHAPE
    assert _dec(lib, ns=33) == binding.MLA_ERR_SHAPE
    assert _dec(lib, S=0) == binding.MLA_ERR_SHAPE
    assert _dec(lib, B=(1 << 16) + 1) == binding.MLA_ERR_SHAPE
    assert _dec(lib, B=4096, S=4096) == binding.MLA_ERR_SHAPE   # B*S_max*576 beyond int32 rows
    assert _dec(lib, scale=-1.0) == binding.MLA_ERR_SHAPE
    assert _dec(lib, ql=BAD) == binding.MLA_ERR_ALIGN
    assert _dec(lib, ws=None) == binding.MLA_ERR_WORKSPACE


def test_combine_and_absorb_validation_codes(lib):
    assert lib.mla_combine(None, P, P, P, 1, 1, 2, None) == binding.MLA_ERR_NULL
    assert lib.mla_combine(P, P, P, P, 1, 1, 0, None) == binding.MLA_ERR_SHAPE
    assert lib.mla_combine(P, P, P, P, 1, 1, 33, None) == binding.MLA_ERR_SHAPE
    assert lib.mla_combine(P, BAD, P, P, 1, 1, 2, None) == binding.MLA_ERR_ALIGN
    assert lib.mla_absorb_q(P, None, P, 4, 8, 128, 512, None) == binding.MLA_ERR_NULL
    assert lib.mla_absorb_q(P, P, P, 0, 8, 128, 512, None) == binding.MLA_ERR_SHAPE
    assert lib.mla_absorb_q(P, P, P, 4, 8, 100, 512, None) == binding.MLA_ERR_UNSUPPORTED
    assert lib.mla_absorb_q(P, P, P, 4, 8, 128, 500, None) == binding.MLA_ERR_UNSUPPORTED
    assert lib.mla_absorb_q(BAD, P, P, 4, 8, 128, 512, None) == binding.MLA_ERR_ALIGN


def test_up_proj_validation_codes(lib):
    assert lib.mla_up_proj_v(None, P, P, 4, 8, 512, 128, None) == binding.MLA_ERR_NULL
    assert lib.mla_up_proj_v(P, P, None, 4, 8, 512, 128, None) == binding.MLA_ERR_NULL
    assert lib.mla_up_proj_v(P, P, P, 4, 0, 512, 128, None) == binding.MLA_ERR_SHAPE
    assert lib.mla_up_proj_v(P, P, P, 4, 8, 1024, 128, None) == binding.MLA_ERR_UNSUPPORTED
    assert lib.mla_up_proj_v(P, P, P, 4, 8, 500, 128, None) == binding.MLA_ERR_UNSUPPORTED
    assert lib.mla_up_proj_v(P, P, P, 4, 8, 512, 100, None) == binding.MLA_ERR_UNSUPPORTED
    assert lib.mla_up_proj_v(P, P, BAD, 4, 8, 512, 128, None) == binding.MLA_ERR_ALIGN


def test_workspace_size_rejects_bad_shapes(lib):
    assert lib.mla_decode_workspace_size(0, 128, 4) == 0
    assert lib.mla_decode_workspace_size(4, 17, 4) == 0
    assert lib.mla_decode_workspace_size(4, 128, 40) == 0


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


@pytest.mark.skipif(_gpu_visible(), reason="would launch with fake pointers on a real device")
def test_valid_call_without_device_reports_hip_error(lib):
    # Validation passes; the HIP runtime then reports that there is no device.
    assert _attn(lib) == binding.MLA_ERR_HIP
    assert _dec(lib) == binding.MLA_ERR_HIP
    assert lib.mla_decode_workspace_size(4, 128, 4) == 0


def test_decode_noalloc_validation_codes(lib):
    def call(ql=P, qr=P, c=P, sl=P, o=P, lse=P, B=2, H=128, S=64, scale=0.04, ns=4):
        return lib.mla_decode_fwd_noalloc(ql, qr, c, sl, o, lse, B, H, S, scale, ns, None)
    assert call(ql=None) == binding.MLA_ERR_NULL
    assert call(sl=None) == binding.MLA_ERR_NULL
    assert call(B=0) == binding.MLA_ERR_SHAPE
    assert call(H=24) == binding.MLA_ERR_SHAPE
    assert call(ns=33) == binding.MLA_ERR_SHAPE
    assert call(S=0) == binding.MLA_ERR_SHAPE
    assert call(scale=-1.0) == binding.MLA_ERR_SHAPE
    assert call(c=BAD) == binding.MLA_ERR_ALIGN
    assert call(lse=BAD) == binding.MLA_ERR_ALIGN


INT_MIN, INT_MAX = -(1 << 31), (1 << 31) - 1
EXTREMES = (INT_MIN, -1, 0, 1, 15, 16, 17, 1 << 16, (1 << 20) + 1, INT_MAX)


def _sweep(fn, base, positions, allowed):
    """Each listed int argument takes every extreme value in turn; a misaligned
    pointer in `base` keeps every call from reaching a launch, so the status
    is a validation code and never MLA_OK or MLA_ERR_HIP."""
    for pos in positions:
        for val in EXTREMES:
            args = list(base)
            args[pos] = val
            st = fn(*args)
            assert st in allowed, (fn.__name__, pos, val, st)


def test_extreme_integer_arguments_are_rejected_before_any_launch(lib):
    # Under the host sanitizer build these also check that no validation
    # expression overflows or reads an out-of-range value.
    shape = {binding.MLA_ERR_SHAPE, binding.MLA_ERR_UNSUPPORTED, binding.MLA_ERR_ALIGN}
    _sweep(lib.attn_fwd, [P, P, P, BAD, P, 1, 2, 256, 64, 0.125, 0, 0, None], (5, 6, 7, 8, 10, 11), shape)
    _sweep(lib.attn_fwd_chunk, [P, P, P, BAD, P, 1, 2, 128, 256, 128, 0.125, 1, 1, None], (5, 6, 7, 8, 9, 11, 12),
           shape)
    _sweep(lib.mla_decode_fwd, [BAD, P, P, P, P, P, 2, 128, 64, 0.04, 4, P, 1 << 30, None], (6, 7, 8, 10), shape)
    _sweep(lib.mla_decode_fwd_v, [BAD, P, P, P, P, P, P, 2, 128, 64, 512, 0.04, 4, P, 1 << 30, None],
           (7, 8, 9, 10, 12), shape)
    _sweep(lib.mla_decode_fwd_noalloc, [BAD, P, P, P, P, P, 2, 128, 64, 0.04, 4, None], (6, 7, 8, 10), shape)
    _sweep(lib.mla_combine, [BAD, P, P, P, 2, 128, 4, None], (4, 5, 6), shape)
    _sweep(lib.mla_absorb_q, [BAD, P, P, 4, 8, 128, 512, None], (3, 4, 5, 6), shape)
    _sweep(lib.mla_up_proj_v, [BAD, P, P, 4, 8, 512, 128, None], (3, 4, 5, 6), shape)


def test_extreme_workspace_queries_and_status_codes(lib):
    for fn in (lib.mla_decode_workspace_size, lib.mla_decode_v_workspace_size):
        for pos in range(3):
            for val in EXTREMES:
                args = [4, 128, 4]
                args[pos] = val
                n = fn(*args)
                valid = 1 <= args[0] <= 1 << 16 and args[1] >= 16 and args[1] % 16 == 0 and args[1] <= 1024 \
                    and 1 <= args[2] <= 32
                if not valid:
                    assert n == 0, (fn.__name__, args, n)
    for s in (INT_MIN, -1, 8, INT_MAX):
        assert lib.mla_status_string(s).decode() == "unknown mla_status_t"


def test_calibration_library_exports_its_kernel_and_checks_arguments():
    # The benchmark's MFMA-rate calibration kernel lives in its own library,
    # next to (not inside) the attention library.
    from mla_latent_kv_attn_amd import build as _b
    if not os.path.exists(_b.CALIB_LIB):
        pytest.skip("libmla_calib.so not built")
    cal = ctypes.CDLL(_b.CALIB_LIB)
    f = cal.mla_calib_mfma_rate
    vp, i = ctypes.c_void_p, ctypes.c_int
    f.argtypes = [vp, vp, i, i, i, vp]
    f.restype = i
    bad = 1  # hipErrorInvalidValue
    p = ctypes.c_void_p(16)
    assert f(None, p, 1, 1, 16, None) == bad
    assert f(p, None, 1, 1, 16, None) == bad
    assert f(p, p, 0, 1, 16, None) == bad
    assert f(p, p, 1, 0, 32, None) == bad
    assert f(p, p, 1, 1, 8, None) == bad
    assert not hasattr(binding.load(), "mla_calib_mfma_rate")
