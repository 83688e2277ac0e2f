"""Pins of the prefill oracle against facts independent of it.

Each test would fail for a plausible slip in ``oracle.attention`` (a dropped
scale, a transposed operand, a wrong mask direction, a missing max shift,
LSE in the wrong base): brute-force scalar loops, torch's fp64 CPU attention,
closed forms, invariants, and the numbers the blog prints.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force(q, k, v, scale, causal):
    """Scalar loops with math.exp / math.fsum for one (b, h); independent of numpy."""
    N, Nk, D, Dv = len(q), len(k), len(q[0]), len(v[0])
    O, LSE = [], []
    for i in range(N):
        s = []
        for j in range(Nk):
            if causal and j > i:
                continue
            s.append((j, scale * math.fsum(float(q[i][d]) * float(k[j][d]) for d in range(D))))
        mx = max(x for _, x in s)
        w = [(j, math.exp(x - mx)) for j, x in s]
        tot = math.fsum(x for _, x in w)
        O.append([math.fsum(x * float(v[j][c]) for j, x in w) / tot for c in range(Dv)])
        LSE.append(mx + math.log(tot))
    return np.array(O), np.array(LSE)


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("N,D,Dv", [(1, 1, 1), (3, 4, 2), (8, 4, 4), (7, 3, 5)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force(N, D, Dv, causal):
    q, k, v = rnd((1, 1, N, D), 1), rnd((1, 1, N, D), 2), rnd((1, 1, N, Dv), 3)
    scale = 0.37
    O, L = A.attn_ref(q, k, v, scale, causal)
    Ob, Lb = brute_force(q[0, 0], k[0, 0], v[0, 0], scale, causal)
    np.testing.assert_allclose(O[0, 0], Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L[0, 0], Lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_fp64(causal):
    B, H, N, D = 2, 3, 37, 16
    q, k, v = rnd((B, H, N, D), 4), rnd((B, H, N, D), 5), rnd((B, H, N, D), 6)
    scale = 1 / math.sqrt(D)
    O, _ = A.attn_ref(q, k, v, scale, causal, row_block=8)
    Ot = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=scale).numpy()
    np.testing.assert_allclose(O, Ot, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(9, 9), (4, 9), (9, 4)])
def test_rows_of_P_sum_to_one_and_mask(causal, Nq, Nk):
    # With V = I (Dv = Nk) attn_ref returns P itself; with V = ones, the row
    # sums.  P is checked against scalar softmax loops, its rows must sum to
    # one, and the causal zero pattern is the bottom-right one.
    q, k = rnd((2, 2, Nq, 5), 7), rnd((2, 2, Nk, 5), 8)
    eye = np.broadcast_to(np.eye(Nk), (2, 2, Nk, Nk))
    P, _ = A.attn_ref(q, k, eye, 0.5, causal)
    off = Nk - Nq
    for b in range(2):
        for h in range(2):
            for i in range(Nq):
                lim = min(i + off + 1, Nk) if causal else Nk
                if lim <= 0:
                    assert np.all(P[b, h, i] == 0.0)
                    continue
                s = [0.5 * math.fsum(q[b, h, i, d] * k[b, h, j, d] for d in range(5)) for j in range(lim)]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = math.fsum(e)
                np.testing.assert_allclose(P[b, h, i, :lim], [x / tot for x in e], rtol=0, atol=1e-14)
                assert np.all(P[b, h, i, lim:] == 0.0)
    seen = np.array([min(i + off + 1, Nk) > 0 if causal else Nk > 0 for i in range(Nq)])
    np.testing.assert_allclose(P.sum(-1)[..., seen], 1.0, rtol=0, atol=1e-12)
    ones = np.ones((2, 2, Nk, 3))
    R, _ = A.attn_ref(q, k, ones, 0.5, causal)
    np.testing.assert_allclose(R[..., seen, :], 1.0, rtol=0, atol=1e-12)
    if causal and Nq == Nk:
        assert np.all(P[..., 0, 0] == 1.0)  # row 0 puts all its mass on key 0


def test_causal_row0_is_v0_exactly():
    q, k, v = rnd((2, 3, 11, 6), 9), rnd((2, 3, 11, 6), 10), rnd((2, 3, 11, 6), 11)
    O, L = A.attn_ref(q, k, v, 0.8, True)
    assert np.array_equal(O[:, :, 0], v[:, :, 0])
    s00 = 0.8 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    np.testing.assert_allclose(L[:, :, 0], s00, rtol=0, atol=1e-14)


def test_identical_keys_give_mean_of_v():
    N, D = 10, 4
    q = rnd((1, 1, N, D), 12)
    k = np.broadcast_to(rnd((1, 1, 1, D), 13), (1, 1, N, D)).copy()
    v = rnd((1, 1, N, 3), 14)
    O, L = A.attn_ref(q, k, v, 0.6, False)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0].mean(0), (N, 3)), atol=1e-12)
    s = 0.6 * q[0, 0] @ k[0, 0, 0]
    np.testing.assert_allclose(L[0, 0], s + math.log(N), atol=1e-12)
    Oc, Lc = A.attn_ref(q, k, v, 0.6, True)
    for i in range(N):
        np.testing.assert_allclose(Oc[0, 0, i], v[0, 0, : i + 1].mean(0), atol=1e-12)
        np.testing.assert_allclose(Lc[0, 0, i], s[i] + math.log(i + 1), atol=1e-12)


def test_two_keys_sigmoid_closed_form():
    q, k, v = rnd((1, 1, 4, 3), 15), rnd((1, 1, 2, 3), 16), rnd((1, 1, 2, 5), 17)
    O, L = A.attn_ref(q, k, v, 1.3, False)
    for i in range(4):
        s0, s1 = 1.3 * q[0, 0, i] @ k[0, 0, 0], 1.3 * q[0, 0, i] @ k[0, 0, 1]
        w0 = 1 / (1 + math.exp(s1 - s0))
        np.testing.assert_allclose(O[0, 0, i], w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, 1], atol=1e-12)
        np.testing.assert_allclose(L[0, 0, i], math.log(math.exp(s0) + math.exp(s1)), atol=1e-12)


def test_joint_key_value_permutation_invariance():
    q, k, v = rnd((1, 2, 6, 4), 18), rnd((1, 2, 9, 4), 19), rnd((1, 2, 9, 4), 20)
    perm = np.random.default_rng(21).permutation(9)
    O, L = A.attn_ref(q, k, v, 0.7, False)
    Op, Lp = A.attn_ref(q, k[:, :, perm], v[:, :, perm], 0.7, False)
    np.testing.assert_allclose(O, Op, atol=1e-12)
    np.testing.assert_allclose(L, Lp, atol=1e-12)


@pytest.mark.parametrize("N,Br,Bc", [(64, 16, 16), (67, 16, 8), (100, 32, 16), (33, 8, 32), (256, 128, 32)])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_equals_definition(N, Br, Bc, causal):
    q, k, v = rnd((1, 2, N, 8), 22), rnd((1, 2, N, 8), 23), rnd((1, 2, N, 8), 24)
    O, L = A.attn_ref(q, k, v, 0.35, causal)
    Oo, Lo = A.online_attn_ref(q, k, v, 0.35, causal, Br, Bc, guard=True)
    np.testing.assert_allclose(Oo, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Lo, L, rtol=0, atol=1e-13)


def test_unguarded_recurrence_hits_the_nan_trap():
    # Br > Bc: the diagonal tiles hold rows whose every key is masked.
    N, Br, Bc = 256, 128, 32
    q, k, v = rnd((1, 1, N, 8), 25), rnd((1, 1, N, 8), 26), rnd((1, 1, N, 8), 27)
    O, _ = A.online_attn_ref(q, k, v, 0.35, True, Br, Bc, guard=False)
    nan_rows = int(np.isnan(O[0, 0]).any(axis=1).sum())
    # rows r of a query tile are NaN when a visited tile starts past r:
    # 96 of each 128-row tile (tiles 1..3 of the diagonal block).
    assert nan_rows == 192
    Og, _ = A.online_attn_ref(q, k, v, 0.35, True, Br, Bc, guard=True)
    assert np.isfinite(Og).all()
    # Br == Bc never leaves a row with an all-masked visited tile.
    O2, _ = A.online_attn_ref(q, k, v, 0.35, True, 32, 32, guard=False)
    assert np.isfinite(O2).all()


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_blog_block_skip_worked_example():
    g = _golden("fa2_v2_block_skip.json")
    ex = g["example"]
    q_start = ex["q_block"] * ex["Br"]
    assert [q_start, q_start + ex["Br"]] == ex["rows"]
    kv_limit, Tc = A.causal_kv_tiles(q_start, ex["Br"], ex["N"], ex["Bc"], True)
    assert kv_limit == ex["kv_limit"]
    assert Tc == ex["tiles_visited"]
    assert -(-ex["N"] // ex["Bc"]) - Tc == ex["tiles_skipped"]
    # only the last visited tile straddles the diagonal
    diag = [j for j in range(Tc) if A.is_diagonal_tile(j * ex["Bc"], ex["Bc"], q_start, True)]
    assert diag == ex["diagonal_tiles"]
    # non-causal visits all tiles
    assert A.causal_kv_tiles(q_start, ex["Br"], ex["N"], ex["Bc"], False) == (ex["N"], ex["N"] // ex["Bc"])


def test_blog_launch_and_shared_memory_arithmetic():
    g = _golden("fa2_v2_launch_shape.json")
    s = g["shape"]
    shp = A.v2_launch_shape(s["B"], s["H"], s["N"], s["D"], s["Br"], s["Bc"])
    assert shp["blocks"] == g["blocks"]
    assert list(shp["grid"]) == g["grid"]
    assert shp["nvec"] == g["nvec"]
    total, qo = A.v2_shared_bytes(s["Br"], s["Bc"], s["D"])
    assert round(total / 1024) == g["shared_total_KiB"]
    assert total == g["shared_total_bytes"]
    assert int(qo / 1000) == g["qs_oacc_kB"]


# ---------------------------------------------------------------------------
# Non-square causal attention (a prefill chunk of Nq queries over Nk keys)
# ---------------------------------------------------------------------------
def brute_force_chunk(q, k, v, scale):
    """Scalar loops, bottom-right causal: row i sees keys j <= i + Nk - Nq."""
    N, Nk, D, Dv = len(q), len(k), len(q[0]), len(v[0])
    off = Nk - N
    O, LSE = [], []
    for i in range(N):
        s = [(j, scale * math.fsum(float(q[i][d]) * float(k[j][d]) for d in range(D)))
             for j in range(Nk) if j <= i + off]
        if not s:
            O.append([0.0] * Dv)
            LSE.append(-math.inf)
            continue
        mx = max(x for _, x in s)
        w = [(j, math.exp(x - mx)) for j, x in s]
        tot = math.fsum(x for _, x in w)
        O.append([math.fsum(x * float(v[j][c]) for j, x in w) / tot for c in range(Dv)])
        LSE.append(mx + math.log(tot))
    return np.array(O), np.array(LSE)


@pytest.mark.parametrize("Nq,Nk", [(3, 7), (5, 5), (7, 3), (1, 6), (6, 1)])
def test_chunk_brute_force(Nq, Nk):
    D, Dv = 4, 3
    q, k, v = rnd((1, 1, Nq, D), 11), rnd((1, 1, Nk, D), 12), rnd((1, 1, Nk, Dv), 13)
    O, L = A.attn_ref(q, k, v, 0.41, True)
    Ob, Lb = brute_force_chunk(q[0, 0], k[0, 0], v[0, 0], 0.41)
    np.testing.assert_allclose(O[0, 0], Ob, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(L[0, 0]), np.isneginf(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(L[0, 0][fin], Lb[fin], rtol=0, atol=1e-12)


def test_chunk_equals_last_rows_of_square_causal():
    # The queries of a chunk are the last Nq positions of the key sequence:
    # their rows of a full square causal attention are the chunk's result.
    B, H, Nk, D = 2, 2, 50, 8
    q, k, v = rnd((B, H, Nk, D), 14), rnd((B, H, Nk, D), 15), rnd((B, H, Nk, D), 16)
    O, L = A.attn_ref(q, k, v, 0.3, True)
    for Nq in (1, 17, 50):
        Oc, Lc = A.attn_ref(q[:, :, Nk - Nq:], k, v, 0.3, True, row_block=7)
        np.testing.assert_allclose(Oc, O[:, :, Nk - Nq:], rtol=0, atol=1e-12)
        np.testing.assert_allclose(Lc, L[:, :, Nk - Nq:], rtol=0, atol=1e-12)


def test_chunk_single_query_sees_every_key_and_empty_rows():
    q, k, v = rnd((1, 2, 1, 8), 17), rnd((1, 2, 30, 8), 18), rnd((1, 2, 30, 5), 19)
    O, L = A.attn_ref(q, k, v, 0.5, True)
    On, Ln = A.attn_ref(q, k, v, 0.5, False)
    np.testing.assert_allclose(O, On, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, Ln, rtol=0, atol=1e-13)
    # Nq > Nk: the first Nq - Nk rows see no key
    q2 = rnd((1, 1, 9, 8), 20)
    O2, L2 = A.attn_ref(q2, k[:, :1, :4], v[:, :1, :4], 0.5, True)
    assert np.all(O2[0, 0, :5] == 0) and np.all(np.isneginf(L2[0, 0, :5]))
    assert np.all(np.isfinite(L2[0, 0, 5:]))


def test_chunk_against_torch_sdpa_with_explicit_mask():
    B, H, Nq, Nk, D = 2, 3, 21, 45, 16
    q, k, v = rnd((B, H, Nq, D), 21), rnd((B, H, Nk, D), 22), rnd((B, H, Nk, D), 23)
    scale = 1 / math.sqrt(D)
    O, _ = A.attn_ref(q, k, v, scale, True, row_block=8)
    allowed = torch.from_numpy(np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq))
    Ot = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=allowed, scale=scale).numpy()
    np.testing.assert_allclose(O, Ot, rtol=0, atol=1e-12)
