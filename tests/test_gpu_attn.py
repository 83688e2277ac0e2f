"""GPU parity of attn_fwd (fp32 vector-ALU path and bf16 MFMA path) against
the fp64 oracle, called through the C ABI."""

import math

import numpy as np
import pytest
import torch

from mla_latent_kv_attn_amd import binding, workloads
from oracle import attention as OA
from tests.gpu_util import (attn_rows_ref, check_bf16, check_f32, check_lse, np64, pick_rows, say, sync)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(q, k, v, scale, causal):
    o, l = binding.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal)
    sync()
    return o, l


# ----------------------------------------------------------------- fp32 ----
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_small_workload(causal):
    w = workloads.attn_workload("attn_small")
    say(f"fp32 attn_small causal={causal}")
    o, l = run(w["q"], w["k"], w["v"], w["scale"], causal)
    Or, Lr = OA.attn_ref(np64(w["q"]), np64(w["k"]), np64(w["v"]), w["scale"], causal)
    check_f32(o, Or, "O")
    check_lse(l, Lr, "LSE")


@pytest.mark.parametrize("N", [1, 2, 31, 33, 127, 129, 200, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_ragged(N, causal):
    say(f"fp32 ragged N={N} causal={causal}")
    q, k, v = workloads.attn_inputs(2, 3, N, 64, torch.float32, seed=500 + N)
    o, l = run(q, k, v, 0.125, causal)
    Or, Lr = OA.attn_ref(np64(q), np64(k), np64(v), 0.125, causal)
    check_f32(o, Or, "O")
    check_lse(l, Lr, "LSE")


def test_fp32_causal_row0_is_v0_bitwise():
    q, k, v = workloads.attn_inputs(2, 2, 300, 64, torch.float32, seed=77)
    o, _ = run(q, k, v, 0.125, True)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


def test_fp32_identical_keys_give_mean_of_v():
    q, k, v = workloads.attn_inputs(1, 2, 300, 64, torch.float32, seed=81)
    k = k[:, :, :1].expand(-1, -1, 300, -1).contiguous()
    o, l = run(q, k, v, 0.125, False)
    ref = np64(v).mean(axis=2, keepdims=True).repeat(300, axis=2)
    check_f32(o, ref, "O=mean(V)")
    s = 0.125 * np.einsum("bhnd,bhd->bhn", np64(q), np64(k[:, :, 0]))
    check_lse(l, s + math.log(300), "LSE=s+ln N")
    oc, lc = run(q, k, v, 0.125, True)
    refc = np.cumsum(np64(v), axis=2) / np.arange(1, 301)[None, None, :, None]
    check_f32(oc, refc, "causal O=prefix mean(V)")
    check_lse(lc, s + np.log(np.arange(1, 301))[None, None, :], "causal LSE=s+ln(i+1)")


def whole_slices_ref(q, k, v, scale, causal, slices):
    """Oracle O and LSE of whole (b, h) slices, every query row."""
    O, L = [], []
    for b, h in slices:
        o, l = OA.attn_ref(np64(q[b:b + 1, h:h + 1]), np64(k[b:b + 1, h:h + 1]), np64(v[b:b + 1, h:h + 1]),
                           scale, causal)
        O.append(o[0, 0])
        L.append(l[0, 0])
    return np.stack(O), np.stack(L)


@pytest.mark.parametrize("causal", [False, True])
def test_fp32_full_size_sampled(causal):
    w = workloads.attn_workload("attn_fp32")
    say(f"fp32 attn_fp32 (B=4 H=8 N=8192 D=64) causal={causal}")
    o, l = run(w["q"], w["k"], w["v"], w["scale"], causal)
    picks = pick_rows(4, 8, 8192, 24, seed=3)
    Or, Lr = attn_rows_ref(w["q"], w["k"], w["v"], w["scale"], causal, picks)
    og = torch.stack([o[b, h, i] for b, h, i in picks])
    lg = torch.stack([l[b, h, i] for b, h, i in picks])
    check_f32(og, Or, "O(sampled)")
    check_lse(lg, Lr, "LSE(sampled)")
    assert torch.isfinite(o).all()
    # two whole (b, h) slices: every query tile, and under the causal mask
    # every rank of the heaviest-first order
    sl = [(0, 0), (3, 7)]
    Or, Lr = whole_slices_ref(w["q"], w["k"], w["v"], w["scale"], causal, sl)
    check_f32(torch.stack([o[b, h] for b, h in sl]), Or, "O(whole slices)")
    check_lse(torch.stack([l[b, h] for b, h in sl]), Lr, "LSE(whole slices)")


# ----------------------------------------------------------------- bf16 ----
@pytest.mark.parametrize("N", [1, 5, 64, 65, 128, 129, 255, 300, 512])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_ragged(N, causal):
    say(f"bf16 ragged N={N} causal={causal}")
    q, k, v = workloads.attn_inputs(1, 3, N, 128, torch.bfloat16, seed=900 + N)
    sc = 1 / math.sqrt(128)
    o, l = run(q, k, v, sc, causal)
    Or, Lr = OA.attn_ref(np64(q), np64(k), np64(v), sc, causal)
    check_bf16(o, Or, "O")
    check_lse(l, Lr, "LSE")


def test_bf16_causal_row0_is_v0_bitwise():
    q, k, v = workloads.attn_inputs(2, 2, 200, 128, torch.bfloat16, seed=78)
    o, _ = run(q, k, v, 1 / math.sqrt(128), True)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


def test_bf16_identical_keys_give_mean_of_v():
    q, k, v = workloads.attn_inputs(1, 2, 256, 128, torch.bfloat16, seed=79)
    k = k[:, :, :1].expand(-1, -1, 256, -1).contiguous()
    o, l = run(q, k, v, 1 / math.sqrt(128), False)
    ref = np64(v).mean(axis=2, keepdims=True).repeat(256, axis=2)
    check_bf16(o, ref, "O=mean(V)")


def test_bf16_full_size_sampled_and_deterministic():
    w = workloads.attn_workload("attn_bf16")
    say("bf16 attn_bf16 (B=4 H=16 N=4096 D=128) causal")
    q, k, v = w["q"].to(DEV), w["k"].to(DEV), w["v"].to(DEV)
    o1, l1 = binding.attn_fwd(q, k, v, w["scale"], True)
    o2, l2 = binding.attn_fwd(q, k, v, w["scale"], True)
    sync()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "run-to-run results differ"
    picks = pick_rows(4, 16, 4096, 24, seed=4)
    Or, Lr = attn_rows_ref(w["q"], w["k"], w["v"], w["scale"], True, picks)
    og = torch.stack([o1[b, h, i] for b, h, i in picks])
    lg = torch.stack([l1[b, h, i] for b, h, i in picks])
    check_bf16(og, Or, "O(sampled)")
    check_lse(lg, Lr, "LSE(sampled)")
    assert torch.isfinite(o1.float()).all()
    sl = [(0, 0), (1, 9), (3, 15)]
    Or, Lr = whole_slices_ref(w["q"], w["k"], w["v"], w["scale"], True, sl)
    check_bf16(torch.stack([o1[b, h] for b, h in sl]), Or, "O(whole slices)")
    check_lse(torch.stack([l1[b, h] for b, h in sl]), Lr, "LSE(whole slices)")


def test_bf16_noncausal_full_size_sampled():
    w = workloads.attn_workload("attn_bf16")
    say("bf16 attn_bf16 non-causal")
    o, l = run(w["q"], w["k"], w["v"], w["scale"], False)
    picks = pick_rows(4, 16, 4096, 12, seed=5)
    Or, Lr = attn_rows_ref(w["q"], w["k"], w["v"], w["scale"], False, picks)
    check_bf16(torch.stack([o[b, h, i] for b, h, i in picks]), Or, "O(sampled)")
    check_lse(torch.stack([l[b, h, i] for b, h, i in picks]), Lr, "LSE(sampled)")
    sl = [(2, 3), (3, 12)]
    Or, Lr = whole_slices_ref(w["q"], w["k"], w["v"], w["scale"], False, sl)
    check_bf16(torch.stack([o[b, h] for b, h in sl]), Or, "O(whole slices)")
    check_lse(torch.stack([l[b, h] for b, h in sl]), Lr, "LSE(whole slices)")


def test_lse_optional_and_outputs_untouched_on_error():
    q, k, v = workloads.attn_inputs(1, 1, 64, 64, torch.float32, seed=80)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    o, l = binding.attn_fwd(q, k, v, 0.125, False, want_lse=False)
    assert l is None
    o_ref, _ = binding.attn_fwd(q, k, v, 0.125, False)
    sync()
    assert torch.equal(o, o_ref)
    canary = torch.full_like(q, 7.0)
    with pytest.raises(binding.MlaError):
        binding.attn_fwd(q, k, v, -1.0, False, o=canary)
    sync()
    assert torch.all(canary == 7.0)


# ------------------------------------------------- chunk (Nq != Nk) ----
CHUNKS = [(64, 256), (33, 300), (200, 1000), (128, 128), (300, 100), (1, 513), (5, 0)]


def chunk_inputs(B, H, Nq, Nk, D, dtype, seed):
    q = workloads.attn_inputs(B, H, Nq, D, dtype, seed=seed)[0]
    _, k, v = workloads.attn_inputs(B, H, Nk, D, dtype, seed=seed + 1)
    return q, k, v


@pytest.mark.parametrize("Nq,Nk", CHUNKS)
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_chunk(Nq, Nk, causal):
    say(f"fp32 chunk Nq={Nq} Nk={Nk} causal={causal}")
    q, k, v = chunk_inputs(2, 3, Nq, Nk, 64, torch.float32, 1300 + Nq + Nk)
    o, l = binding.attn_fwd_chunk(q.to(DEV), k.to(DEV), v.to(DEV), 0.125, causal)
    sync()
    Or, Lr = OA.attn_ref(np64(q), np64(k), np64(v), 0.125, causal)
    check_f32(o, Or, "O")
    check_lse(l, Lr, "LSE")


@pytest.mark.parametrize("Nq,Nk", CHUNKS)
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_chunk(Nq, Nk, causal):
    say(f"bf16 chunk Nq={Nq} Nk={Nk} causal={causal}")
    q, k, v = chunk_inputs(1, 3, Nq, Nk, 128, torch.bfloat16, 1700 + Nq + Nk)
    sc = 1 / math.sqrt(128)
    o, l = binding.attn_fwd_chunk(q.to(DEV), k.to(DEV), v.to(DEV), sc, causal)
    sync()
    Or, Lr = OA.attn_ref(np64(q), np64(k), np64(v), sc, causal)
    check_bf16(o, Or, "O")
    check_lse(l, Lr, "LSE")


def test_bf16_chunk_at_benchmark_shape():
    # The chunk shape the benchmark times: B=4 H=16, 1024 queries over 4096
    # keys, causal bottom-right; whole (b, h) slices (every query tile).
    B, H, Nq, Nk, D = 4, 16, 1024, 4096, 128
    say(f"bf16 chunk at the benchmark shape B={B} H={H} Nq={Nq} Nk={Nk}")
    q, k, v = chunk_inputs(B, H, Nq, Nk, D, torch.bfloat16, 1007)
    sc = 1 / math.sqrt(D)
    o, l = binding.attn_fwd_chunk(q.to(DEV), k.to(DEV), v.to(DEV), sc, True)
    sync()
    sl = [(0, 0), (1, 5), (2, 10), (3, 15)]
    Or, Lr = whole_slices_ref(q, k, v, sc, True, sl)
    check_bf16(torch.stack([o[b, h] for b, h in sl]), Or, "O(whole slices)")
    check_lse(torch.stack([l[b, h] for b, h in sl]), Lr, "LSE(whole slices)")
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_rising_scores_rescale_every_tile(causal):
    # Scores rise by about 12 (log2 units) per 64-key tile for every query:
    # all queries share a direction u and key j carries u times a ramp in j,
    # so the exponent base moves on every tile and the accumulators are
    # rescaled.  Values stay N(0,1).
    B, H, N, D = 1, 2, 512, 128
    q, k, v = workloads.attn_inputs(B, H, N, D, torch.float32, seed=2201)
    g = torch.Generator().manual_seed(2202)
    u = torch.randn(D, generator=g) / math.sqrt(D)
    scale = 1 / math.sqrt(D)
    kappa = 12.0 / (scale * 3.0 * float(u @ u) * 1.4426950408889634)
    q = 3.0 * u + 0.3 * q
    k = k + (torch.arange(N, dtype=torch.float32)[:, None] / 64.0) * kappa * u
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    say(f"bf16 rising scores causal={causal}")
    o, l = run(q, k, v, scale, causal)
    Or, Lr = OA.attn_ref(np64(q), np64(k), np64(v), scale, causal)
    check_bf16(o, Or, "O")
    check_lse(l, Lr, "LSE")
