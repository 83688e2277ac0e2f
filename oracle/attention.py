"""Prefill attention oracle: float64 numpy, test infrastructure only.

What the fused forward computes, per (batch b, head h), is the plain
definition restated in [FA2-v2 blog] section 1.3 and section 3.3:

    S = scale * Q K^T            (scale applied before the row max, section 3.3)
    S[i, j] = -inf  for j > i    (causal, top-left aligned: row i sees keys <= i,
                                  section 3.4)
    P = softmax_row(S),  O = P V
    LSE_i = m_i + ln l_i  with m_i = max_j S_ij, l_i = sum_j exp(S_ij - m_i)

The online-softmax kernel reaches this result exactly up to rounding order
(the rescaling in section 1.3 is an exact rewrite), so ``attn_ref`` is the
definition written out.  ``online_attn_ref`` restates the blog's tiled
algorithm step by step (tile loop, running m and l, unnormalised accumulator,
one division at the end) so that the tiled recurrence itself can be pinned
against the definition, including the fully-masked-tile case where the
printed recurrence produces NaN unless guarded.

LSE is this library's addition: the blog writes only O.  It is the natural
logarithm of the row's sum of exponentiated scaled scores.

Pinned by (tests/test_oracle_attention.py): pure-Python brute force on tiny
inputs, torch's fp64 CPU scaled_dot_product_attention, row sums of P = 1,
causal row 0 = V[0], identical keys -> mean of V (closed form, also per causal
prefix), two-key sigmoid closed form, joint permutation invariance of (K, V),
and the blog's printed worked example and launch arithmetic.  The
non-square causal form (Nq != Nk) is pinned by chunk consistency (the last
Nq rows of a square causal attention, run as a chunk against all keys),
Nq = 1 (sees every key), rows with no key (Nq > Nk), pure-Python loops, and
torch's fp64 SDPA with an explicit boolean mask.
"""

import numpy as np

__all__ = [
    "attn_ref",
    "online_attn_ref",
    "causal_kv_tiles",
    "is_diagonal_tile",
    "v2_shared_bytes",
    "v2_launch_shape",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def attn_ref(q, k, v, scale, causal, row_block=256):
    """Explicit softmax attention and per-row LSE.

    q: [B, H, Nq, D]; k: [B, H, Nk, D]; v: [B, H, Nk, Dv] (any real dtype,
    upcast to float64).  Returns (O [B, H, Nq, Dv] float64, LSE [B, H, Nq]).

    Rows are processed in blocks of ``row_block`` only to bound memory; each
    block's softmax is over the full key range, so blocking changes nothing.
    Definition: [FA2-v2 blog] section 1.3 (O = softmax(S) V, deferred
    normalisation being an exact rewrite of it) and section 3.4 (causal:
    row i sees keys 0..i).  With Nq != Nk the causal mask is aligned at the
    bottom right (the queries are the last Nq positions of the key sequence,
    as in a prefill chunk over an existing cache): row i sees keys
    0..i + (Nk - Nq).  A row that sees no key (Nq > Nk) gives O = 0 and
    LSE = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, _ = q.shape
    Nk = k.shape[2]
    Dv = v.shape[3]
    off = Nk - N
    O = np.zeros((B, H, N, Dv))
    LSE = np.full((B, H, N), -np.inf)
    keys = np.arange(Nk)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, row_block):
                r1 = min(N, r0 + row_block)
                S = scale * (q[b, h, r0:r1] @ k[b, h].T)
                if causal:
                    rows = np.arange(r0, r1)[:, None]
                    S = np.where(keys[None, :] > rows + off, -np.inf, S)
                seen = np.isfinite(S).any(axis=1)
                if not seen.any():
                    continue
                Ss = S[seen]
                m = Ss.max(axis=1, keepdims=True)
                E = np.exp(Ss - m)
                l = E.sum(axis=1, keepdims=True)
                idx = np.arange(r0, r1)[seen]
                O[b, h, idx] = (E / l) @ v[b, h]
                LSE[b, h, idx] = (m + np.log(l))[:, 0]
    return O, LSE


def causal_kv_tiles(q_start, Br, N, Bc, causal):
    """Key-tile range of one query tile: (kv_limit, Tc).

    [FA2-v2 blog] section 3.4, block-level skip: the largest row of the tile
    is q_start+Br-1 and it sees keys up to that index, so with the causal mask
    the tile loop stops at kv_limit = min(q_start+Br, N); otherwise it covers
    all N keys.  Tc = ceil(kv_limit / Bc) tiles are visited; the rest are
    never loaded.
    """
    kv_limit = min(q_start + Br, N) if causal else N
    return kv_limit, -(-kv_limit // Bc)


def is_diagonal_tile(kv_start, Bc, q_start, causal):
    """Whether a visited key tile straddles the diagonal and needs the
    per-element mask ([FA2-v2 blog] section 3.4): its last key index
    kv_start+Bc-1 exceeds the first row q_start of the query tile."""
    return bool(causal) and (kv_start + Bc - 1 > q_start)


def online_attn_ref(q, k, v, scale, causal, Br, Bc, guard=True):
    """The tiled online-softmax forward, step by step, in float64.

    Follows [FA2-v2 blog] sections 1.2, 1.3, 3.3, 3.4 and 3.5, in that order
    of steps for each query tile of Br rows:
      running m = -inf, l = 0, unnormalised accumulator Oacc = 0;
      for each key tile j < Tc (block skip of section 3.4):
        S = scale * Q_tile K_j^T; keys >= N -> -inf (section 3.2, zero-filled
        tail rows); on a diagonal tile keys > row -> -inf (section 3.4);
        m~ = row max of S; P~ = exp(S - m~); l~ = row sum of P~;
        m_new = max(m, m~); alpha = exp(m - m_new); beta = exp(m~ - m_new);
        l = alpha l + beta l~; Oacc = alpha Oacc + beta (P~ V_j); m = m_new;
      O = Oacc / l (section 3.5).
    Returns (O, LSE) like ``attn_ref``.

    guard=True applies this library's reading for a row whose every score in
    a tile is masked (m~ = -inf): the tile contributes nothing to that row.
    guard=False keeps the recurrence exactly as printed, where
    exp(-inf - (-inf)) yields NaN for such rows; it exists so a test can show
    the trap is real (it arises when Br > Bc on diagonal tiles).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, _ = q.shape
    Dv = v.shape[3]
    O = np.zeros((B, H, N, Dv))
    LSE = np.zeros((B, H, N))
    with np.errstate(invalid="ignore"):
        for b in range(B):
            for h in range(H):
                for q_start in range(0, N, Br):
                    rows = np.arange(q_start, min(q_start + Br, N))
                    Qt = q[b, h, rows]
                    m = np.full(len(rows), -np.inf)
                    l = np.zeros(len(rows))
                    Oacc = np.zeros((len(rows), Dv))
                    _, Tc = causal_kv_tiles(q_start, Br, N, Bc, causal)
                    for j in range(Tc):
                        kv_start = j * Bc
                        keys = np.arange(kv_start, kv_start + Bc)
                        inb = keys < N
                        Kt = np.zeros((Bc, q.shape[3]))
                        Vt = np.zeros((Bc, Dv))
                        Kt[inb] = k[b, h, keys[inb]]
                        Vt[inb] = v[b, h, keys[inb]]
                        S = scale * (Qt @ Kt.T)
                        S[:, ~inb] = -np.inf
                        if is_diagonal_tile(kv_start, Bc, q_start, causal):
                            S = np.where(keys[None, :] > rows[:, None], -np.inf, S)
                        m_t = S.max(axis=1)
                        P_t = np.exp(S - m_t[:, None])
                        l_t = P_t.sum(axis=1)
                        m_new = np.maximum(m, m_t)
                        alpha = np.exp(m - m_new)
                        beta = np.exp(m_t - m_new)
                        if guard:
                            dead = np.isneginf(m_t)
                            P_t[dead] = 0.0
                            l_t[dead] = 0.0
                            beta[dead] = 0.0
                            alpha[dead] = 1.0
                            m_new[dead] = m[dead]
                        l = alpha * l + beta * l_t
                        Oacc = alpha[:, None] * Oacc + beta[:, None] * (P_t @ Vt)
                        m = m_new
                    O[b, h, rows] = Oacc / l[:, None]
                    LSE[b, h, rows] = m + np.log(l)
    return O, LSE


def v2_shared_bytes(Br, Bc, D):
    """Shared-memory footprint of the blog's v2 layout, in bytes.

    [FA2-v2 blog] section 3.1: K and V tiles double-buffered unpadded,
    [2][Bc][D] floats each; Qs and Oacc padded to a row stride of D+1 floats,
    [Br][D+1] each.  Returns (total, Qs + Oacc).  Section 4.2 quotes the
    total (97 KB at Br=128, Bc=32, D=64) and the Qs+Oacc share (66 KB).
    This is the page's design, recorded as a pinned fact; the MI355X kernels
    keep Q and the accumulator in registers instead.
    """
    kv = 2 * 2 * Bc * D * 4
    qo = 2 * Br * (D + 1) * 4
    return kv + qo, qo


def v2_launch_shape(B, H, N, D, Br, Bc):
    """The blog's v2 launch arithmetic: grid (ceil(N/Br), B*H), Br threads
    per block, and NVEC = Bc*D/4 16-byte chunks per K (or V) tile
    ([FA2-v2 blog] sections 1.1, 2 and 3.2)."""
    gx = -(-N // Br)
    return {"grid": (gx, B * H), "blocks": gx * B * H, "threads": Br, "nvec": Bc * D // 4}
