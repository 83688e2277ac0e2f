"""Latent-cache MLA decode oracle: float64 numpy, test infrastructure only.

What the fused decode computes ([MLA-FA3 article]): every cached token t holds
a 512-dim compressed latent c_t^KV and a 64-dim decoupled RoPE key k_t^R,
stored side by side as one 576-wide row (fused dataflow figure; section 1,
where one row of the cache is latent_dim = 512 + 64 = 576 elements).  With the
key up-projection W_UK absorbed into the query (section 2, absorption
equation), one head's score against token t is

    s_t = scale * ( (q_nope W_UK) . c_t^KV  +  q_rope . k_t^R )
        = scale * [q_lat || q_rope] . [c_t^KV || k_t^R]

so a single 576-wide dot product per (head, token) against the cache as
stored, with no decompressed key ever formed.  The value side stays in
latent space: O = softmax(s) . c^KV (the first 512 dims of the same rows);
W_UV is not applied on this path.

Readings of what the pages leave open (each also listed in the design notes):
  * the extracted absorption equation lost its '=' and '+'; it is read as
    Q K^T = (Q W_UK)(c^KV)^T + Q^R (k^R)^T;
  * k^R is cached already rotated and q_rope arrives rotated: no rotation is
    computed here;
  * W_UK is laid out [H, Dn, Dl] (per head, nope dim x latent dim);
  * cache rows are padded per sequence, [B, S_max, 576]; rows >= len_b are
    never read; len_b = 0 gives O = 0 and LSE = -inf;
  * LSE is the natural log of the sum of exponentiated scaled scores.

The value up-projection W_UV (named with W_UK in the article's fused
dataflow figure, in the in-place absorption stage) maps the latent output to
the per-head value space: o_v[b, h] = O[b, h] W_UV[h].  Because attention is
linear in the values, applying it after the softmax-weighted sum equals
attending over explicitly decompressed values V_h = c^KV W_UV[h]; that is the
value-side counterpart of the absorption equation.  W_UV is laid out
[H, 512, Dv] (per head, latent dim x value dim), the row-vector form of the
column-vector W^UV blocks.

Pinned by (tests/test_oracle_mla.py): pure-Python brute force on tiny
inputs, identical cache rows (O = latent row, LSE = s + ln len), len = 1,
the absorption identity against explicit decompression (sampled), decode
through explicit decompression versus the absorbed decode, split invariance of
the combine over arbitrary split plans, combine closed forms; for the value
up-projection, attention over explicitly decompressed values versus the
latent output projected afterwards, a selection matrix (exact copy of chosen
latent dims), and pure-Python loops on tiny inputs; for the bfloat16
rounding, torch's float32 -> bfloat16 conversion (a single rounding for
float32-representable values), hand-made ties that must go to the even
neighbour, and the set of representable values being fixed points; the
end-to-end reference is its two pinned parts composed, checked once more
against explicit key decompression on a bf16-rounded query.
"""

import numpy as np

__all__ = [
    "LATENT_DIM",
    "ROPE_DIM",
    "mla_decode_ref",
    "absorb_ref",
    "decompress_k_ref",
    "mla_decode_explicit_ref",
    "split_partials_ref",
    "combine_ref",
    "up_project_v_ref",
    "decompress_v_ref",
    "mla_decode_values_explicit_ref",
    "round_bf16",
    "absorb_decode_ref",
]

LATENT_DIM = 512
ROPE_DIM = 64


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _softmax_rows(S):
    """Row softmax pieces (m, E, l) of a score matrix with finite rows."""
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    return m, E, E.sum(axis=1, keepdims=True)


def mla_decode_ref(q_lat, q_rope, cache, seqlens, scale):
    """Absorbed decode against the latent cache, one query token per sequence.

    q_lat [B, H, 512], q_rope [B, H, 64], cache [B, S_max, 576] (columns
    0..511 = c^KV, 512..575 = k^R), seqlens [B] integers.
    Returns (O [B, H, 512] float64, LSE [B, H] float64).

    Per sequence b with L = seqlens[b] > 0:
      Q = [q_lat[b] || q_rope[b]] (H x 576), C = cache[b, :L] (L x 576)
      S = scale Q C^T;  P = softmax_row(S);  O = P C[:, :512];  LSE = m + ln l
    ([MLA-FA3 article] section 2 absorption equation, fused dataflow figure.)
    """
    q_lat, q_rope, cache = _f64(q_lat), _f64(q_rope), _f64(cache)
    B, H, Dl = q_lat.shape
    O = np.zeros((B, H, Dl))
    LSE = np.full((B, H), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        if L == 0:
            continue
        Q = np.concatenate([q_lat[b], q_rope[b]], axis=1)
        C = cache[b, :L]
        m, E, l = _softmax_rows(scale * (Q @ C.T))
        O[b] = (E / l) @ C[:, :Dl]
        LSE[b] = (m + np.log(l))[:, 0]
    return O, LSE


def absorb_ref(q_nope, w_uk):
    """Weight absorption: q_lat[b, h, :] = q_nope[b, h, :] @ W_UK[h].

    q_nope [B, H, Dn], w_uk [H, Dn, Dl] -> q_lat [B, H, Dl] float64.
    ([MLA-FA3 article] section 2: the factor Q W_UK of the absorption
    equation, formed once per query instead of once per cached token.)
    """
    q_nope, w_uk = _f64(q_nope), _f64(w_uk)
    B, H, Dn = q_nope.shape
    out = np.empty((B, H, w_uk.shape[2]))
    for h in range(H):
        out[:, h, :] = q_nope[:, h, :] @ w_uk[h]
    return out


def round_bf16(x):
    """Round float64 values to bfloat16 (1-8-7), round to nearest, ties to even.

    bfloat16 keeps 8 significant bits.  For x = m 2^e with 0.5 <= |m| < 1
    (numpy's frexp), the spacing of bfloat16 values around x is 2^(e-8),
    never finer than 2^-133 (the subnormal spacing below the smallest
    normal, 2^-126).  x / spacing is exact in float64, np.rint rounds it to
    the nearest integer with ties to even, and the product is exact again.
    Values beyond the largest finite bfloat16 are not expected here and are
    not clamped.  Returns float64 arrays holding bfloat16 values.
    (The precision the decode's query is stored in after absorption:
    q_lat is kept in bf16 before the decode.)
    """
    x = _f64(x)
    _, e = np.frexp(x)
    spacing = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.rint(x / spacing) * spacing


def absorb_decode_ref(q_nope, w_uk, q_rope, cache, seqlens, scale):
    """The decode step end to end from the un-absorbed query.

    q_lat = round_bf16(absorb_ref(q_nope, W_UK)) -- the absorption in float64,
    then the one rounding to bfloat16 that storing q_lat implies -- followed
    by ``mla_decode_ref`` on [q_lat || q_rope] against the cache.
    Returns (O [B, H, 512], LSE [B, H]).
    ([MLA-FA3 article] section 2: absorb W_UK into the query once, then take
    the 576-wide dot products against the cache as stored.)
    """
    q_lat = round_bf16(absorb_ref(q_nope, w_uk))
    return mla_decode_ref(q_lat, q_rope, cache, seqlens, scale)


def decompress_k_ref(c_latent, w_uk):
    """Explicit key decompression (the step fusion avoids).

    c_latent [T, 512], w_uk [H, Dn, 512] -> K_nope [T, H, Dn] with
    K_nope[t, h, :] = W_UK[h] c_t.  This is the separate restore-to-HBM
    kernel of the unfused path ([MLA-FA3 article] introduction, scheme A of
    the benchmark section).
    """
    c_latent, w_uk = _f64(c_latent), _f64(w_uk)
    T = c_latent.shape[0]
    H, Dn, _ = w_uk.shape
    K = np.empty((T, H, Dn))
    for h in range(H):
        K[:, h, :] = c_latent @ w_uk[h].T
    return K


def mla_decode_explicit_ref(q_nope, q_rope, w_uk, cache, seqlens, scale):
    """Decode through explicitly decompressed keys (scheme A's arithmetic).

    Scores are scale * (q_nope . K_nope_t + q_rope . k_t^R) with
    K_nope = decompress_k_ref(c^KV, W_UK); the value side is the latent
    c^KV as in ``mla_decode_ref``.  Equal to the absorbed decode up to
    rounding, which is the content of the absorption equation.
    Returns (O [B, H, 512], LSE [B, H]).
    """
    q_nope, q_rope, cache, w_uk = _f64(q_nope), _f64(q_rope), _f64(cache), _f64(w_uk)
    B, H, _ = q_nope.shape
    O = np.zeros((B, H, LATENT_DIM))
    LSE = np.full((B, H), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        if L == 0:
            continue
        C = cache[b, :L]
        K = decompress_k_ref(C[:, :LATENT_DIM], w_uk)           # [L, H, Dn]
        S = np.einsum("hd,thd->ht", q_nope[b], K) + q_rope[b] @ C[:, LATENT_DIM:].T
        m, E, l = _softmax_rows(scale * S)
        O[b] = (E / l) @ C[:, :LATENT_DIM]
        LSE[b] = (m + np.log(l))[:, 0]
    return O, LSE


def split_partials_ref(q_lat, q_rope, cache, ranges, scale):
    """Per-split partial results of the decode over given token ranges.

    ranges: list over b of lists of (t0, t1) token ranges; every list is
    padded to the same length S with empty ranges.  Returns
    (o_part [B, H, S, 512], lse_part [B, H, S]) where split s of sequence b
    holds the attention of the tokens [t0, t1) alone, normalised over that
    range (O_s = softmax-weighted latent rows), and lse_s = m_s + ln l_s.
    An empty range gives O_s = 0 and lse_s = -inf.
    (Split-KV partials that the [MLA-FA3 article] dataflow figure merges in
    its "online softmax scaling and partial reduction" stage.)
    """
    q_lat, q_rope, cache = _f64(q_lat), _f64(q_rope), _f64(cache)
    B, H, Dl = q_lat.shape
    S_n = max(len(r) for r in ranges) if ranges else 0
    o_part = np.zeros((B, H, S_n, Dl))
    lse_part = np.full((B, H, S_n), -np.inf)
    for b in range(B):
        Q = np.concatenate([q_lat[b], q_rope[b]], axis=1)
        for s, (t0, t1) in enumerate(ranges[b]):
            if t1 <= t0:
                continue
            C = cache[b, t0:t1]
            m, E, l = _softmax_rows(scale * (Q @ C.T))
            o_part[b, :, s] = (E / l) @ C[:, :Dl]
            lse_part[b, :, s] = (m + np.log(l))[:, 0]
    return o_part, lse_part


def combine_ref(o_part, lse_part):
    """Log-sum-exp merge of split partials.

    o_part [B, H, S, Dv], lse_part [B, H, S] (-inf marks an empty split).
      LSE = log sum_s exp(lse_s)                (-inf if every split is empty)
      O   = sum_s exp(lse_s - LSE) O_s          (0 if every split is empty)
    Each O_s is normalised over its own range, so exp(lse_s - LSE) is the
    share of the total softmax mass that range carries.
    """
    o_part, lse_part = _f64(o_part), _f64(lse_part)
    M = lse_part.max(axis=2, keepdims=True)
    alive = np.isfinite(M)
    Msafe = np.where(alive, M, 0.0)
    w = np.where(np.isneginf(lse_part), 0.0, np.exp(lse_part - Msafe))
    tot = w.sum(axis=2, keepdims=True)
    LSE = np.where(alive, Msafe + np.log(np.where(alive, tot, 1.0)), -np.inf)[..., 0]
    frac = np.where(alive, w / np.where(alive, tot, 1.0), 0.0)
    O = np.einsum("bhs,bhsd->bhd", frac, o_part)
    return O, LSE


def up_project_v_ref(o_lat, w_uv):
    """Value up-projection of the latent output: o_v[b, h, :] = O[b, h, :] @ W_UV[h].

    o_lat [B, H, Dl], w_uv [H, Dl, Dv] -> [B, H, Dv] float64.
    ([MLA-FA3 article] fused dataflow figure: the W_UK / W_UV projections of
    the in-place absorption stage; here the W_UV one, applied once per query
    after the softmax-weighted sum over the latent cache.)
    """
    o_lat, w_uv = _f64(o_lat), _f64(w_uv)
    B, H, _ = o_lat.shape
    out = np.empty((B, H, w_uv.shape[2]))
    for h in range(H):
        out[:, h, :] = o_lat[:, h, :] @ w_uv[h]
    return out


def decompress_v_ref(c_latent, w_uv):
    """Explicit value decompression (the step the latent path avoids).

    c_latent [T, 512], w_uv [H, 512, Dv] -> V [T, H, Dv] with
    V[t, h, :] = c_t W_UV[h].
    """
    c_latent, w_uv = _f64(c_latent), _f64(w_uv)
    T = c_latent.shape[0]
    H, _, Dv = w_uv.shape
    V = np.empty((T, H, Dv))
    for h in range(H):
        V[:, h, :] = c_latent @ w_uv[h]
    return V


def mla_decode_values_explicit_ref(q_lat, q_rope, w_uv, cache, seqlens, scale):
    """Decode whose values are explicitly decompressed, V_h = c^KV W_UV[h].

    Scores as in ``mla_decode_ref``; output o_v[b, h] = softmax(s) V_h.
    Equal to up_project_v_ref(mla_decode_ref(...)[0], w_uv) up to rounding
    (attention is linear in its values).  Returns o_v [B, H, Dv] (zeros for
    an empty sequence).
    """
    q_lat, q_rope, cache, w_uv = _f64(q_lat), _f64(q_rope), _f64(cache), _f64(w_uv)
    B, H, Dl = q_lat.shape
    out = np.zeros((B, H, w_uv.shape[2]))
    for b in range(B):
        L = int(seqlens[b])
        if L == 0:
            continue
        Q = np.concatenate([q_lat[b], q_rope[b]], axis=1)
        C = cache[b, :L]
        m, E, l = _softmax_rows(scale * (Q @ C.T))
        P = E / l                                           # [H, L]
        V = decompress_v_ref(C[:, :Dl], w_uv)               # [L, H, Dv]
        out[b] = np.einsum("ht,thd->hd", P, V)
    return out
