"""Seeded synthetic inputs for the five workloads and for test cases.

This module only draws random numbers: it holds none of the attention or
decode arithmetic, so both the HIP path and the CPU oracle can consume what
it produces.  Every tensor comes from one CPU ``torch.Generator`` seeded per
workload, drawn in float32 with ``torch.randn`` in the order listed, then
rounded to bfloat16 (round-to-nearest-even) where the workload is bf16.
No public dataset or trained weight is involved: the pages benchmark on
random inputs of these shapes, and the 67B-model numbers of the MLA article
need weights that are not reproduced here.

Workloads (sizes as used by the tests and the benchmark):
  attn_small   fp32  B=1  H=2  N=256  D=64    scale 1/8, causal and not (seed 1001)
  attn_fp32    fp32  B=4  H=8  N=8192 D=64    scale 1/8, causal and not (seed 1002)
  attn_bf16    bf16  B=4  H=16 N=4096 D=128   scale 1/sqrt(128), causal  (seed 1003)
  mla_fixed    bf16  B=16 H=128, 4096 cached tokens each, q [16,128,576] (seed 1004)
  mla_varlen   bf16  B=256 H=128, lengths uniform in [256, 8192], absorption
               prologue q_nope [256,128,128] @ W_UK [128,128,512] (std 0.02)
               (seed 1005)
"""

import math

import torch

LATENT = 512
ROPE = 64
ROW = LATENT + ROPE

ATTN_SHAPES = {
    "attn_small": dict(B=1, H=2, N=256, D=64, dtype=torch.float32, seed=1001),
    "attn_fp32": dict(B=4, H=8, N=8192, D=64, dtype=torch.float32, seed=1002),
    "attn_bf16": dict(B=4, H=16, N=4096, D=128, dtype=torch.bfloat16, seed=1003),
}


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def attn_inputs(B, H, N, D, dtype=torch.float32, seed=0):
    """q, k, v: [B, H, N, D] iid N(0, 1), drawn q then k then v."""
    g = _gen(seed)
    q = torch.randn((B, H, N, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, N, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, N, D), generator=g, dtype=torch.float32)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def attn_workload(name):
    s = ATTN_SHAPES[name]
    q, k, v = attn_inputs(s["B"], s["H"], s["N"], s["D"], s["dtype"], s["seed"])
    return dict(q=q, k=k, v=v, scale=1.0 / math.sqrt(s["D"]), **s)


def decode_inputs(B, H, seqlens, S_max=None, seed=0, pad_value=float("nan")):
    """Decode inputs with the query drawn as one 576-wide vector per head.

    Draw order: q [B, H, 576], then the cache of each sequence b in turn as
    [len_b, 576].  The cache is padded to [B, S_max, 576]; padding rows hold
    ``pad_value`` (NaN by default, so any read of them shows up).
    Returns dict(q_lat [B,H,512], q_rope [B,H,64], cache, seqlens int32).
    """
    seqlens = torch.as_tensor(seqlens, dtype=torch.int32)
    if S_max is None:
        S_max = int(seqlens.max().item()) if B > 0 else 0
    g = _gen(seed)
    q = torch.randn((B, H, ROW), generator=g, dtype=torch.float32).to(torch.bfloat16)
    cache = torch.full((B, S_max, ROW), pad_value, dtype=torch.bfloat16)
    for b in range(B):
        L = int(seqlens[b])
        if L:
            cache[b, :L] = torch.randn((L, ROW), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return dict(q_lat=q[..., :LATENT].contiguous(), q_rope=q[..., LATENT:].contiguous(),
                cache=cache, seqlens=seqlens, S_max=S_max)


def mla_fixed_workload(seed=1004, B=16, H=128, L=4096):
    """Batch 16, 128 heads, every sequence 4096 cached tokens."""
    d = decode_inputs(B, H, [L] * B, S_max=L, seed=seed)
    d.update(B=B, H=H, scale=1.0 / math.sqrt(ROW), seed=seed)
    return d


def mla_varlen_workload(seed=1005, B=256, H=128, Dn=128, lo=256, hi=8192, S_max=8192):
    """Variable-length decode with the absorption prologue's inputs.

    Draw order: seqlens = randint(lo, hi + 1) [B]; q_nope [B, H, Dn];
    W_UK [H, Dn, 512] scaled by 0.02 (std 0.02); q_rope [B, H, 64]; then the
    cache of each sequence b in turn as [len_b, 576] into the padded
    [B, S_max, 576] tensor (padding NaN).
    """
    g = _gen(seed)
    seqlens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    q_nope = torch.randn((B, H, Dn), generator=g, dtype=torch.float32).to(torch.bfloat16)
    w_uk = (torch.randn((H, Dn, LATENT), generator=g, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    q_rope = torch.randn((B, H, ROPE), generator=g, dtype=torch.float32).to(torch.bfloat16)
    cache = torch.full((B, S_max, ROW), float("nan"), dtype=torch.bfloat16)
    for b in range(B):
        L = int(seqlens[b])
        cache[b, :L] = torch.randn((L, ROW), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return dict(seqlens=seqlens, q_nope=q_nope, w_uk=w_uk, q_rope=q_rope, cache=cache,
                B=B, H=H, Dn=Dn, S_max=S_max, scale=1.0 / math.sqrt(ROW), seed=seed)


def w_uv_weights(H=128, Dl=LATENT, Dv=128, seed=1006):
    """Value up-projection weights W_UV [H, Dl, Dv], N(0, 0.02^2), bf16, from a
    stream of their own (so the decode workload's draws are unchanged)."""
    g = _gen(seed)
    return (torch.randn((H, Dl, Dv), generator=g, dtype=torch.float32) * 0.02).to(torch.bfloat16)


def random_seqlens(B, lo, hi, seed):
    """Integer lengths uniform in [lo, hi] (inclusive) from their own stream."""
    g = _gen(seed)
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
