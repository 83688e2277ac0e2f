"""Pins of the MLA decode oracle against facts independent of it.

A dropped RoPE term, a value slice that includes the RoPE dims, a transposed
W_UK, a wrong sign in the LSE merge or a missing empty-split rule each fail
one of these.
"""

import math

import numpy as np
import pytest
import torch

from oracle import mla as M


def rnd(shape, seed, s=1.0):
    return s * np.random.default_rng(seed).standard_normal(shape)


def brute_decode(q_lat, q_rope, cache, L, scale):
    """Scalar loops for one sequence: returns (O [H][512], LSE [H])."""
    H = len(q_lat)
    O, LSE = [], []
    for h in range(H):
        qv = list(q_lat[h]) + list(q_rope[h])
        s = [scale * math.fsum(float(qv[d]) * float(cache[t][d]) for d in range(576)) for t in range(L)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = math.fsum(w)
        O.append([math.fsum(w[t] * float(cache[t][c]) for t in range(L)) / tot for c in range(512)])
        LSE.append(mx + math.log(tot))
    return np.array(O), np.array(LSE)


def make(B, H, S_max, seed):
    q_lat, q_rope = rnd((B, H, 512), seed), rnd((B, H, 64), seed + 1)
    cache = rnd((B, S_max, 576), seed + 2)
    return q_lat, q_rope, cache


def test_brute_force_small():
    q_lat, q_rope, cache = make(2, 3, 5, 100)
    lens = [5, 2]
    O, L = M.mla_decode_ref(q_lat, q_rope, cache, lens, 0.05)
    for b in range(2):
        Ob, Lb = brute_decode(q_lat[b], q_rope[b], cache[b], lens[b], 0.05)
        np.testing.assert_allclose(O[b], Ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[b], Lb, rtol=0, atol=1e-12)


def test_rope_term_and_value_slice():
    # Only the RoPE part differs between tokens: scores must come from it,
    # and the output must be built from the latent part only.
    H, Lt = 2, 4
    q_lat, q_rope = np.zeros((1, H, 512)), rnd((1, H, 64), 3)
    cache = np.zeros((1, Lt, 576))
    cache[0, :, :512] = rnd((Lt, 512), 4)
    cache[0, :, 512:] = rnd((Lt, 64), 5)
    O, L = M.mla_decode_ref(q_lat, q_rope, cache, [Lt], 0.3)
    s = 0.3 * q_rope[0] @ cache[0, :, 512:].T
    w = np.exp(s - s.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    np.testing.assert_allclose(O[0], w @ cache[0, :, :512], atol=1e-12)


def test_against_torch_sdpa_fp64():
    B, H, S = 3, 4, 17
    q_lat, q_rope, cache = make(B, H, S, 200)
    lens = [17, 9, 1]
    scale = 1 / math.sqrt(576)
    O, _ = M.mla_decode_ref(q_lat, q_rope, cache, lens, scale)
    for b in range(B):
        q = torch.from_numpy(np.concatenate([q_lat[b], q_rope[b]], 1))[:, None, :]   # [H,1,576]
        kk = torch.from_numpy(cache[b, : lens[b]])[None].expand(H, -1, -1)          # [H,L,576]
        vv = torch.from_numpy(cache[b, : lens[b], :512])[None].expand(H, -1, -1)
        ot = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, scale=scale)[:, 0].numpy()
        np.testing.assert_allclose(O[b], ot, rtol=0, atol=1e-12)


def test_identical_rows_and_single_token():
    H, Lt = 3, 7
    q_lat, q_rope = rnd((1, H, 512), 6), rnd((1, H, 64), 7)
    row = rnd((576,), 8)
    cache = np.broadcast_to(row, (1, Lt, 576)).copy()
    O, L = M.mla_decode_ref(q_lat, q_rope, cache, [Lt], 0.04)
    np.testing.assert_allclose(O[0], np.broadcast_to(row[:512], (H, 512)), atol=1e-12)
    s = 0.04 * (q_lat[0] @ row[:512] + q_rope[0] @ row[512:])
    np.testing.assert_allclose(L[0], s + math.log(Lt), atol=1e-12)
    O1, L1 = M.mla_decode_ref(q_lat, q_rope, rnd((1, 3, 576), 9), [1], 0.04)
    c0 = rnd((1, 3, 576), 9)[0, 0]
    assert np.array_equal(O1[0], np.broadcast_to(c0[:512], (H, 512)))
    np.testing.assert_allclose(L1[0], 0.04 * (q_lat[0] @ c0[:512] + q_rope[0] @ c0[512:]), atol=1e-14)


def test_empty_sequence_and_unread_padding():
    q_lat, q_rope, cache = make(2, 2, 6, 300)
    cache[0, 3:] = np.nan
    O, L = M.mla_decode_ref(q_lat, q_rope, cache, [3, 0], 0.05)
    assert np.isfinite(O[0]).all() and np.isfinite(L[0]).all()
    assert np.all(O[1] == 0.0) and np.all(np.isneginf(L[1]))
    O3, L3 = M.mla_decode_ref(q_lat[:1], q_rope[:1], cache[:1, :3], [3], 0.05)
    np.testing.assert_array_equal(O[0], O3[0])


def test_absorption_identity_against_explicit_decompression():
    # q_nope . (W_UK c)  ==  (q_nope W_UK) . c, the absorption equation.
    H, Dn, T = 4, 128, 16
    q_nope, w_uk, c = rnd((2, H, Dn), 10), rnd((H, Dn, 512), 11, 0.02), rnd((T, 512), 12)
    K = M.decompress_k_ref(c, w_uk)                                  # [T,H,Dn]
    explicit = np.einsum("bhd,thd->bht", q_nope, K)
    absorbed = np.einsum("bhl,tl->bht", M.absorb_ref(q_nope, w_uk), c)
    rel = np.abs(explicit - absorbed).max() / np.abs(explicit).max()
    assert rel <= 1e-12
    # independent restatement of the two products on one entry
    h, d, t = 2, 5, 7
    assert math.isclose(K[t, h, d], math.fsum(w_uk[h, d, l] * c[t, l] for l in range(512)), rel_tol=1e-12)
    ql = M.absorb_ref(q_nope, w_uk)
    assert math.isclose(ql[1, h, 9], math.fsum(q_nope[1, h, i] * w_uk[h, i, 9] for i in range(Dn)),
                        rel_tol=1e-12, abs_tol=1e-15)


def test_explicit_decode_equals_absorbed_decode():
    B, H, Dn, S = 2, 4, 128, 12
    q_nope, w_uk = rnd((B, H, Dn), 13), rnd((H, Dn, 512), 14, 0.02)
    q_rope, cache = rnd((B, H, 64), 15), rnd((B, S, 576), 16)
    lens = [12, 5]
    scale = 1 / math.sqrt(576)
    Oe, Le = M.mla_decode_explicit_ref(q_nope, q_rope, w_uk, cache, lens, scale)
    Oa, La = M.mla_decode_ref(M.absorb_ref(q_nope, w_uk), q_rope, cache, lens, scale)
    np.testing.assert_allclose(Oa, Oe, rtol=0, atol=1e-12)
    np.testing.assert_allclose(La, Le, rtol=0, atol=1e-12)


def _random_ranges(L, S, rng):
    cuts = sorted(rng.integers(0, L + 1, size=S - 1).tolist())
    b = [0] + cuts + [L]
    return [(b[i], b[i + 1]) for i in range(S)]


@pytest.mark.parametrize("S", [1, 2, 7, 32])
def test_split_invariance(S):
    B, H, Smax = 3, 4, 40
    q_lat, q_rope, cache = make(B, H, Smax, 400 + S)
    lens = [40, 13, 3]
    rng = np.random.default_rng(S)
    ranges = [_random_ranges(L, S, rng) for L in lens]
    op, lp = M.split_partials_ref(q_lat, q_rope, cache, ranges, 0.05)
    O, L = M.combine_ref(op, lp)
    Or, Lr = M.mla_decode_ref(q_lat, q_rope, cache, lens, 0.05)
    np.testing.assert_allclose(O, Or, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lr, rtol=0, atol=1e-12)


def test_combine_closed_forms():
    o = rnd((1, 2, 3, 8), 17)
    lse = np.array([[[0.3, 0.3, -np.inf], [-np.inf, -np.inf, -np.inf]]])
    O, L = M.combine_ref(o, lse)
    np.testing.assert_allclose(O[0, 0], 0.5 * (o[0, 0, 0] + o[0, 0, 1]), atol=1e-15)
    np.testing.assert_allclose(L[0, 0], 0.3 + math.log(2), atol=1e-15)
    assert np.all(O[0, 1] == 0.0) and np.isneginf(L[0, 1])
    lse2 = np.array([[[-np.inf, 1.5, -np.inf], [2.0, -1.0, 0.5]]])
    O2, L2 = M.combine_ref(o, lse2)
    np.testing.assert_array_equal(O2[0, 0], o[0, 0, 1])
    assert L2[0, 0] == 1.5
    w = np.exp([2.0, -1.0, 0.5])
    np.testing.assert_allclose(L2[0, 1], math.log(w.sum()), atol=1e-14)
    np.testing.assert_allclose(O2[0, 1], (w[:, None] * o[0, 1]).sum(0) / w.sum(), atol=1e-14)


# ---------------------------------------------------------------------------
# Value up-projection W_UV
# ---------------------------------------------------------------------------
def test_up_projection_equals_attention_over_decompressed_values():
    # Attention is linear in its values: projecting the latent output equals
    # attending over V_h = c W_UV[h].  The two sides share only the scores.
    B, H, S_max, Dv = 2, 3, 40, 16
    q_lat, q_rope, cache = make(B, H, S_max, 71)
    w_uv = rnd((H, 512, Dv), 72, 0.05)
    lens = np.array([40, 17])
    scale = 1 / math.sqrt(576)
    O, _ = M.mla_decode_ref(q_lat, q_rope, cache, lens, scale)
    got = M.up_project_v_ref(O, w_uv)
    ref = M.mla_decode_values_explicit_ref(q_lat, q_rope, w_uv, cache, lens, scale)
    assert np.abs(got - ref).max() < 1e-12 * max(1.0, np.abs(ref).max())


def test_up_projection_selection_matrix_copies_dims():
    # W_UV[h] = columns of the identity picking latent dims sel[h]: the
    # projection returns exactly those dims of the latent output.
    B, H, Dv = 3, 2, 8
    o = rnd((B, H, 512), 73)
    sel = [np.arange(Dv) * 7 + 3, np.arange(Dv)[::-1] * 5 + 100]
    w = np.zeros((H, 512, Dv))
    for h in range(H):
        w[h, sel[h], np.arange(Dv)] = 1.0
    got = M.up_project_v_ref(o, w)
    for h in range(H):
        assert np.array_equal(got[:, h, :], o[:, h, sel[h]])


def test_up_projection_brute_force_tiny():
    B, H, Dl, Dv = 2, 2, 6, 3
    o = rnd((B, H, Dl), 74)
    w = rnd((H, Dl, Dv), 75)
    got = M.up_project_v_ref(o, w)
    for b in range(B):
        for h in range(H):
            for d in range(Dv):
                ref = math.fsum(float(o[b, h, c]) * float(w[h, c, d]) for c in range(Dl))
                assert abs(got[b, h, d] - ref) < 1e-12


# ---------------------------------------------------------------------------
# bfloat16 rounding and the end-to-end (absorb -> round -> decode) reference
# ---------------------------------------------------------------------------
def test_round_bf16_matches_torch_on_float32_values():
    # For float32-representable inputs torch's float32 -> bfloat16 conversion
    # is one round-to-nearest-even, the same operation.
    x = np.concatenate([rnd((20000,), 80), rnd((2000,), 81, 1e-30), rnd((2000,), 82, 1e30),
                        rnd((500,), 83, 1e-39)]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = M.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_round_bf16_ties_go_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 (even: 1); 1 + 3*2^-8 lies
    # halfway between 1 + 2^-7 (odd mantissa) and 1 + 2^-6 (even).
    assert M.round_bf16(1 + 2.0 ** -8) == 1.0
    assert M.round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert M.round_bf16(-(1 + 3 * 2.0 ** -8)) == -(1 + 2.0 ** -6)
    assert M.round_bf16(1 + 2.0 ** -8 + 2.0 ** -30) == 1 + 2.0 ** -7   # just above the tie
    assert M.round_bf16(0.0) == 0.0
    # bfloat16 values are fixed points
    v = np.array([1.0, -3.5, 2.0 ** -126, 2.0 ** -133, 1.9921875 * 2.0 ** 100])
    np.testing.assert_array_equal(M.round_bf16(v), v)


def test_absorb_decode_ref_composition_and_explicit_path():
    B, H, Dn, S = 2, 3, 128, 10
    q_nope, w_uk = rnd((B, H, Dn), 84), rnd((H, Dn, 512), 85, 0.02)
    q_rope, cache = rnd((B, H, 64), 86), rnd((B, S, 576), 87)
    lens = [10, 4]
    scale = 1 / math.sqrt(576)
    O, L = M.absorb_decode_ref(q_nope, w_uk, q_rope, cache, lens, scale)
    ql = M.absorb_ref(q_nope, w_uk)
    qlr = torch.from_numpy(ql.astype(np.float32)).to(torch.bfloat16).double().numpy()
    # the rounding matters: the unrounded query gives visibly different scores
    assert np.abs(qlr - ql).max() > 1e-5
    Or, Lr = M.mla_decode_ref(qlr, q_rope, cache, lens, scale)
    # torch rounds via float32 (two roundings); a double rounding can only
    # differ from the single one on near-ties, which these draws do not hit.
    np.testing.assert_allclose(O, Or, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, Lr, rtol=0, atol=1e-13)
    # and against scores taken through explicitly decompressed keys with the
    # rounding error of q_lat moved into q_nope's side: both are within the
    # score perturbation that the bf16 rounding of q_lat causes
    Oe, Le = M.mla_decode_explicit_ref(q_nope, q_rope, w_uk, cache, lens, scale)
    ds = scale * np.abs(qlr - ql).max() * np.abs(cache[..., :512]).sum(-1).max()
    assert np.abs(L - Le).max() <= ds
