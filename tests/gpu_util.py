"""Helpers shared by the GPU parity tests (comparison and tolerances)."""

import math
import sys

import numpy as np
import torch

from oracle import attention as OA

# Tolerances (stated for this library's outputs):
#   fp32 path: max |O - O_ref| <= 1e-5;
#   bf16-in / fp32-accumulate: max |O - O_ref| <= 2e-2 and
#     ||O - O_ref||_2 / ||O_ref||_2 <= 2e-2 (element-wise relative error is
#     meaningless for outputs near zero);
#   LSE (both paths): max |LSE - LSE_ref| <= 1e-3.
TOL_F32 = 1e-5
TOL_BF16_ABS = 2e-2
TOL_BF16_REL = 2e-2
TOL_LSE = 1e-3


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_bf16(o_gpu, o_ref, what):
    og, orf = np64(o_gpu), np.asarray(o_ref, dtype=np.float64)
    assert og.shape == orf.shape, (og.shape, orf.shape)
    assert np.isfinite(og).all(), f"{what}: non-finite output"
    d = np.abs(og - orf)
    mx = float(d.max()) if d.size else 0.0
    rel = float(np.linalg.norm(og - orf) / max(np.linalg.norm(orf), 1e-30)) if d.size else 0.0
    say(f"  {what}: max|d|={mx:.3e} rel={rel:.3e}")
    assert mx <= TOL_BF16_ABS, f"{what}: max abs {mx}"
    assert rel <= TOL_BF16_REL, f"{what}: rel norm {rel}"
    return mx, rel


def check_f32(o_gpu, o_ref, what, tol=TOL_F32):
    og, orf = np64(o_gpu), np.asarray(o_ref, dtype=np.float64)
    assert og.shape == orf.shape
    d = float(np.abs(og - orf).max()) if og.size else 0.0
    say(f"  {what}: max|d|={d:.3e}")
    assert np.isfinite(og).all()
    assert d <= tol, f"{what}: max abs {d}"
    return d


def check_lse(l_gpu, l_ref, what):
    lg, lr = np64(l_gpu), np.asarray(l_ref, dtype=np.float64)
    both_inf = np.isneginf(lg) & np.isneginf(lr)
    assert np.array_equal(np.isneginf(lg), np.isneginf(lr)), f"{what}: -inf pattern differs"
    with np.errstate(invalid="ignore"):
        d = np.abs(np.where(both_inf, 0.0, lg - lr))
    mx = float(d.max()) if d.size else 0.0
    say(f"  {what}: max|dLSE|={mx:.3e}")
    assert mx <= TOL_LSE, f"{what}: LSE max abs {mx}"
    return mx


def attn_rows_ref(q, k, v, scale, causal, picks):
    """Oracle O and LSE for selected (b, h, row) triples only (CPU, fp64).
    q, k, v are CPU tensors; each row is the definition over its visible keys."""
    O, L = [], []
    for b, h, i in picks:
        lim = i + 1 if causal else k.shape[2]
        qi = np64(q[b, h, i:i + 1])[None, None]
        kk = np64(k[b, h, :lim])[None, None]
        vv = np64(v[b, h, :lim])[None, None]
        o, l = OA.attn_ref(qi, kk, vv, scale, False)
        O.append(o[0, 0, 0])
        L.append(l[0, 0, 0])
    return np.array(O), np.array(L)


def pick_rows(B, H, N, n, seed, tile=128):
    """Sampled (b, h, row) triples: tile boundaries, the ends, and random rows."""
    rng = np.random.default_rng(seed)
    rows = {0, 1, N - 1, min(N - 1, tile - 1), min(N - 1, tile), N // 2}
    while len(rows) < n:
        rows.add(int(rng.integers(0, N)))
    return [(int(rng.integers(0, B)), int(rng.integers(0, H)), r) for r in sorted(rows)]


def sync():
    torch.cuda.synchronize()
