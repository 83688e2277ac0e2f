"""GPU parity of the MLA decode path (plan + split + combine), the standalone
LSE combine and the absorption prologue, against the fp64 oracle, through
the C ABI."""

import math

import numpy as np
import pytest
import torch

from mla_latent_kv_attn_amd import binding, workloads
from oracle import mla as OM
from oracle.plan import plan_pieces_ref, plan_ref
from tests.gpu_util import check_bf16, check_lse, np64, say, sync

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCALE = 1 / math.sqrt(576)


def decode(d, num_splits):
    ql, qr, c = d["q_lat"].to(DEV), d["q_rope"].to(DEV), d["cache"].to(DEV)
    sl = d["seqlens"].to(DEV)
    B, H, _ = ql.shape
    ws = binding.alloc_decode_workspace(B, H, num_splits, DEV)
    o, l = binding.mla_decode_fwd(ql, qr, c, sl, SCALE, num_splits, workspace=ws)
    sync()
    return o, l, ws


def oracle_decode(d, idx=None):
    lens = d["seqlens"].tolist()
    if idx is None:
        idx = list(range(len(lens)))
    ql = np64(d["q_lat"][idx])
    qr = np64(d["q_rope"][idx])
    Lmax = max(1, max(lens[i] for i in idx))
    c = np64(d["cache"][idx, :Lmax])
    return OM.mla_decode_ref(ql, qr, c, [lens[i] for i in idx], SCALE)


def check_plan(ws, d, num_splits):
    B = len(d["seqlens"])
    got = binding.read_plan(ws, B)
    ref = plan_ref(d["seqlens"].tolist(), got["tile"], got["parts"] if got["mode"] == "line" else B,
                   num_splits, got["c0"], got["t_min"])
    for key in ("t", "C", "parts_used", "max_n"):
        assert got[key] == ref[key], (key, got[key], ref[key])
    assert got["n"] == ref["n"]
    assert got["first"] == ref["first"]
    assert got["nsplit"] == ref["nsplit"]
    if got["mode"] == "line":
        assert got["start"] == ref["start"]
    assert got["part_first_seq"] == ref["part_first_seq"]
    assert max(got["nsplit"]) <= num_splits
    assert got["clamped"] == 0
    return got


CASES = [
    # (B, H, lens, S_max)
    (3, 16, [1, 64, 300], 320),
    (4, 128, [0, 65, 129, 1000], 1024),
    (2, 32, [511, 37], 512),
    (2, 144, [200, 77], 256),
    (5, 128, [63, 64, 65, 128, 2], 128),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("num_splits", [1, 2, 7, 32])
def test_decode_small(case, num_splits):
    B, H, lens, S = CASES[case]
    say(f"decode B={B} H={H} lens={lens} S_max={S} num_splits={num_splits}")
    d = workloads.decode_inputs(B, H, lens, S_max=S, seed=2000 + case)
    o, l, ws = decode(d, num_splits)
    check_plan(ws, d, num_splits)
    Or, Lr = oracle_decode(d)
    check_bf16(o, Or, "O")
    check_lse(l, Lr, "LSE")
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.all(o[b] == 0) and torch.all(torch.isneginf(l[b]))


@pytest.mark.parametrize("num_splits", [1, 8])
def test_decode_many_short_sequences(num_splits):
    # More sequences than the planner handles in one pass (1024 per chunk),
    # many of them empty: the plan is checked whole, outputs on a sample.
    B, H, S = 2500, 16, 100
    lens = workloads.random_seqlens(B, 0, S, 2200).tolist()
    say(f"decode B={B} H={H} lengths 0..{S} num_splits={num_splits}")
    d = workloads.decode_inputs(B, H, lens, S_max=S, seed=2201)
    o, l, ws = decode(d, num_splits)
    check_plan(ws, d, num_splits)
    empty = [b for b, L in enumerate(lens) if L == 0]
    assert empty, "the sample should hold empty sequences"
    assert torch.all(o[empty] == 0) and torch.all(torch.isneginf(l[empty]))
    rng = np.random.default_rng(2202)
    idx = sorted(set(rng.choice(B, 96, replace=False).tolist()) | {0, 1023, 1024, B - 1, empty[0]})
    Or, Lr = oracle_decode(d, idx)
    check_bf16(o[idx], Or, "O(sampled)")
    check_lse(l[idx], Lr, "LSE(sampled)")


@pytest.mark.parametrize("num_splits", [8, 32])
def test_decode_one_long_sequence(num_splits):
    # One 32768-token sequence: it is split over up to num_splits parts and
    # the combine merges that many partials.
    L = 32768
    say(f"decode B=1 H=128 len={L} num_splits={num_splits}")
    d = workloads.decode_inputs(1, 128, [L], S_max=L, seed=2300)
    o, l, ws = decode(d, num_splits)
    plan = check_plan(ws, d, num_splits)
    assert plan["nsplit"][0] == min(num_splits, plan["parts_used"])
    Or, Lr = oracle_decode(d)
    check_bf16(o, Or, "O")
    check_lse(l, Lr, "LSE")


def test_decode_concurrent_streams_match_serial():
    # The library keeps no state between calls: two decodes in flight at once
    # on two streams (each with its own workspace) give the serial results.
    H = 128
    d1 = workloads.decode_inputs(6, H, [700, 64, 1500, 33, 0, 900], S_max=1500, seed=2400)
    d2 = workloads.decode_inputs(4, H, [2000, 128, 1, 640], S_max=2000, seed=2401)
    o1, l1, _ = decode(d1, 7)
    o2, l2, _ = decode(d2, 32)
    ins = []
    for d, ns in ((d1, 7), (d2, 32)):
        B = d["q_lat"].shape[0]
        ins.append((d["q_lat"].to(DEV), d["q_rope"].to(DEV), d["cache"].to(DEV), d["seqlens"].to(DEV), ns,
                    binding.alloc_decode_workspace(B, H, ns, DEV)))
    sync()
    streams = [torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)]  # default priority
    outs = [None, None]
    for rep in range(3):
        for i, (ql, qr, c, sl, ns, ws) in enumerate(ins):
            with torch.cuda.stream(streams[i]):
                outs[i] = binding.mla_decode_fwd(ql, qr, c, sl, SCALE, ns, workspace=ws)
        sync()
        assert torch.equal(outs[0][0], o1) and torch.equal(outs[0][1], l1), rep
        assert torch.equal(outs[1][0], o2) and torch.equal(outs[1][1], l2), rep


def test_decode_in_hip_graph_replays_match_eager():
    # Nothing in the call allocates, frees, synchronises or sets memory, so
    # absorption + decode can be captured in a HIP graph; every replay (with
    # eager work and synchronisations between them) gives the eager result.
    B, H, ns = 5, 128, 7
    d = workloads.decode_inputs(B, H, [900, 1, 0, 2100, 333], S_max=2100, seed=2500)
    g = torch.Generator().manual_seed(2501)
    q_nope = torch.randn((B, H, 128), generator=g).to(torch.bfloat16).to(DEV)
    w_uk = (torch.randn((H, 128, 512), generator=g) * 0.02).to(torch.bfloat16).to(DEV)
    qr, c, sl = d["q_rope"].to(DEV), d["cache"].to(DEV), d["seqlens"].to(DEV)
    ws = binding.alloc_decode_workspace(B, H, ns, DEV)
    q_lat = torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV)
    o = torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)

    def step():
        binding.mla_absorb_q(q_nope, w_uk, q_lat=q_lat)
        binding.mla_decode_fwd(q_lat, qr, c, sl, SCALE, ns, workspace=ws, o=o, lse=lse)

    step()
    sync()
    o_ref, l_ref = o.clone(), lse.clone()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    sync()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        o.zero_()
        lse.zero_()
        q_lat.zero_()
        sync()
        graph.replay()
        sync()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), rep


def test_decode_identical_rows_and_single_token():
    H = 128
    d = workloads.decode_inputs(3, H, [300, 1, 64], S_max=300, seed=2100)
    d["cache"][0, :300] = d["cache"][0, 7]
    o, l, _ = decode(d, 4)
    ref_row = np64(d["cache"][0, 7, :512])
    check_bf16(o[0], np.broadcast_to(ref_row, (H, 512)), "identical rows -> row")
    assert torch.equal(o[1].cpu(), d["cache"][1, 0, :512].expand(H, -1))   # one token: P = 1 exactly
    Or, Lr = oracle_decode(d)
    check_lse(l, Lr, "LSE")


def test_decode_fixed_length_workload_full():
    d = workloads.mla_fixed_workload()
    say("decode mla_fixed (B=16 H=128, 4096 tokens each) full compare")
    o, l, ws = decode(d, 32)
    check_plan(ws, d, 32)
    Or, Lr = oracle_decode(d)
    check_bf16(o, Or, "O")
    check_lse(l, Lr, "LSE")


@pytest.fixture(scope="module")
def varlen():
    return workloads.mla_varlen_workload()


def test_decode_varlen_workload_end_to_end_all_sequences(varlen):
    # The variable-length workload end to end: GPU absorption -> GPU decode,
    # against the oracle's own absorption (float64), its own rounding of
    # q_lat to bf16 and its decode, for all 256 sequences at the stated
    # tolerances.  Nothing the GPU computed feeds the oracle.
    d = varlen
    say("absorb + decode mla_varlen (B=256 H=128, lengths 256..8192), all sequences")
    ql = binding.mla_absorb_q(d["q_nope"].to(DEV), d["w_uk"].to(DEV))
    qr, c, sl = d["q_rope"].to(DEV), d["cache"].to(DEV), d["seqlens"].to(DEV)
    ws = binding.alloc_decode_workspace(256, 128, 32, DEV)
    o1, l1 = binding.mla_decode_fwd(ql, qr, c, sl, SCALE, 32, workspace=ws)
    o2, l2 = binding.mla_decode_fwd(ql, qr, c, sl, SCALE, 32, workspace=ws)
    sync()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "run-to-run results differ"
    check_plan(ws, d, 32)
    del c
    lens = d["seqlens"].tolist()
    w_uk = np64(d["w_uk"])
    Or = np.empty((256, 128, 512))
    Lr = np.empty((256, 128))
    for b0 in range(0, 256, 16):
        idx = list(range(b0, b0 + 16))
        Lm = max(lens[i] for i in idx)
        Or[idx], Lr[idx] = OM.absorb_decode_ref(np64(d["q_nope"][idx]), w_uk, np64(d["q_rope"][idx]),
                                                np64(d["cache"][idx, :Lm]), [lens[i] for i in idx], SCALE)
    check_bf16(o1, Or, "O (256 sequences)")
    check_lse(l1, Lr, "LSE (256 sequences)")


def test_absorb_full_workload(varlen):
    d = varlen
    ql = binding.mla_absorb_q(d["q_nope"].to(DEV), d["w_uk"].to(DEV))
    sync()
    ref = OM.absorb_ref(np64(d["q_nope"]), np64(d["w_uk"]))
    mx, rel = check_bf16(ql, ref, "q_lat")
    assert rel <= 4e-3          # bf16 output rounding only (2^-9 relative)


@pytest.mark.parametrize("B,H,Dn,Dl", [(1, 1, 32, 128), (5, 3, 64, 256), (70, 2, 128, 512), (3, 4, 512, 128)])
def test_absorb_shapes(B, H, Dn, Dl):
    g = torch.Generator().manual_seed(B * 1000 + Dn)
    qn = torch.randn((B, H, Dn), generator=g).to(torch.bfloat16)
    w = (torch.randn((H, Dn, Dl), generator=g) * 0.05).to(torch.bfloat16)
    ql = binding.mla_absorb_q(qn.to(DEV), w.to(DEV))
    sync()
    ref = OM.absorb_ref(np64(qn), np64(w))
    mx, rel = check_bf16(ql, ref, f"q_lat {B}x{H}x{Dn}x{Dl}")
    assert rel <= 4e-3


def test_up_proj_full_shape():
    # The value up-projection at the decode shape: o_lat [256,128,512] @ W_UV [128,512,128].
    g = torch.Generator().manual_seed(2006)
    o_lat = torch.randn((256, 128, 512), generator=g).to(torch.bfloat16)
    w_uv = workloads.w_uv_weights()
    o_v = binding.mla_up_proj_v(o_lat.to(DEV), w_uv.to(DEV))
    sync()
    ref = OM.up_project_v_ref(np64(o_lat), np64(w_uv))
    mx, rel = check_bf16(o_v, ref, "o_v 256x128x512->128")
    assert rel <= 4e-3          # bf16 output rounding only


@pytest.mark.parametrize("B,H,Dl,Dv", [(1, 1, 32, 128), (7, 3, 512, 256), (65, 2, 256, 128)])
def test_up_proj_shapes(B, H, Dl, Dv):
    g = torch.Generator().manual_seed(B * 100 + Dl)
    o_lat = torch.randn((B, H, Dl), generator=g).to(torch.bfloat16)
    w = (torch.randn((H, Dl, Dv), generator=g) * 0.05).to(torch.bfloat16)
    o_v = binding.mla_up_proj_v(o_lat.to(DEV), w.to(DEV))
    sync()
    mx, rel = check_bf16(o_v, OM.up_project_v_ref(np64(o_lat), np64(w)), f"o_v {B}x{H}x{Dl}x{Dv}")
    assert rel <= 4e-3


def test_decode_then_up_proj_equals_attention_over_decompressed_values():
    # Latent decode, then W_UV, on the GPU, against the oracle's attention
    # over explicitly decompressed values c W_UV[h] (never formed on the GPU).
    B, H, lens, S_max = 3, 128, [300, 77, 1], 320
    d = workloads.decode_inputs(B, H, lens, S_max=S_max, seed=2007)
    w_uv = workloads.w_uv_weights(H=H, seed=2008)
    o, _, _ = decode(d, 4)
    o_v = binding.mla_up_proj_v(o, w_uv.to(DEV))
    sync()
    ref = OM.mla_decode_values_explicit_ref(np64(d["q_lat"]), np64(d["q_rope"]), np64(w_uv), np64(d["cache"]),
                                            lens, SCALE)
    check_bf16(o_v, ref, "decode + W_UV vs explicit values")


@pytest.mark.parametrize("S", [1, 2, 5, 32])
def test_combine_standalone(S):
    B, H = 3, 20
    rng = np.random.default_rng(S)
    o_part = rng.standard_normal((B, H, S, 512)).astype(np.float32)
    lse_part = (rng.standard_normal((B, H, S)) * 3).astype(np.float32)
    lse_part[rng.random((B, H, S)) < 0.3] = -np.inf
    lse_part[0, 0, :] = -np.inf                    # a fully empty row
    o, l = binding.mla_combine(torch.from_numpy(o_part).to(DEV), torch.from_numpy(lse_part).to(DEV))
    sync()
    Or, Lr = OM.combine_ref(o_part.astype(np.float64), lse_part.astype(np.float64))
    check_bf16(o, Or, "combined O")
    check_lse(l, Lr, "combined LSE")
    assert torch.all(o[0, 0] == 0) and torch.isneginf(l[0, 0])


def test_seqlens_out_of_range_are_clamped_and_flagged():
    d = workloads.decode_inputs(2, 16, [100, 50], S_max=100, seed=2200)
    d["seqlens"] = torch.tensor([150, -3], dtype=torch.int32)
    o, l, ws = decode(d, 4)
    got = binding.read_plan(ws, 2)
    assert got["clamped"] == 2 and got["len"] == [100, 0]
    d2 = dict(d, seqlens=torch.tensor([100, 0], dtype=torch.int32))
    Or, Lr = oracle_decode(d2)
    check_bf16(o, Or, "O")
    check_lse(l, Lr, "LSE")


def test_split_partials_cost_at_most_one_bf16_rounding():
    # Split sequences pass through bf16 partials (each normalised over its own
    # token range) before the log-sum-exp merge: one more bf16 rounding than
    # an unsplit sequence.  Its error against the oracle must stay within the
    # unsplit error plus one bf16 half-ulp (2^-9 relative), norm-wise and per
    # head row; and the LSE (merged in fp32 from fp32 partial LSEs) within the
    # stated tolerance.
    B, H = 3, 128
    lens = [8192, 5000, 2600]
    d = workloads.decode_inputs(B, H, lens, S_max=8192, seed=2600)
    o1, l1, ws1 = decode(d, 1)
    o32, l32, ws32 = decode(d, 32)
    p1, p32 = binding.read_plan(ws1, B), binding.read_plan(ws32, B)
    assert max(p1["nsplit"]) == 1 and min(p32["nsplit"]) >= 2, (p1["nsplit"], p32["nsplit"])
    Or, Lr = oracle_decode(d)
    e1 = np64(o1) - Or
    e32 = np64(o32) - Or
    half_ulp = 2.0 ** -9
    r1 = np.linalg.norm(e1) / np.linalg.norm(Or)
    r32 = np.linalg.norm(e32) / np.linalg.norm(Or)
    say(f"  rel error unsplit {r1:.3e}, split {r32:.3e} (splits {p32['nsplit']})")
    assert r32 <= r1 + half_ulp
    row_ref = np.linalg.norm(Or, axis=-1)
    row1 = np.linalg.norm(e1, axis=-1) / row_ref
    row32 = np.linalg.norm(e32, axis=-1) / row_ref
    assert np.all(row32 <= row1 + half_ulp), float((row32 - row1).max())
    check_bf16(o32, Or, "O split")
    check_lse(l32, Lr, "LSE split")
    check_lse(l1, Lr, "LSE unsplit")


# ------------------------------------------- decode + value up-projection ----
def decode_v(d, w_uv, num_splits):
    ql, qr, c, sl = (d[k].to(DEV) for k in ("q_lat", "q_rope", "cache", "seqlens"))
    B, H, _ = ql.shape
    ws = binding.alloc_decode_v_workspace(B, H, num_splits, DEV)
    o_v, l = binding.mla_decode_fwd_v(ql, qr, c, sl, w_uv.to(DEV), SCALE, num_splits, workspace=ws)
    sync()
    return o_v, l, ws


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("num_splits", [1, 2, 7, 32])
def test_decode_v_small(case, num_splits):
    # The fused merge + W_UV path against the oracle's attention over
    # explicitly decompressed values, and bitwise against the unfused path
    # (mla_decode_fwd, then mla_up_proj_v).
    B, H, lens, S = CASES[case]
    say(f"decode_v B={B} H={H} lens={lens} S_max={S} num_splits={num_splits}")
    d = workloads.decode_inputs(B, H, lens, S_max=S, seed=2700 + case)
    w_uv = workloads.w_uv_weights(H=H, seed=2710 + case)
    o_v, l, ws = decode_v(d, w_uv, num_splits)
    check_plan(ws, d, num_splits)
    ref = OM.mla_decode_values_explicit_ref(np64(d["q_lat"]), np64(d["q_rope"]), np64(w_uv), np64(d["cache"]),
                                            lens, SCALE)
    check_bf16(o_v, ref, "o_v")
    _, Lr = oracle_decode(d)
    check_lse(l, Lr, "LSE")
    o_lat, l2, _ = decode(d, num_splits)
    o_v2 = binding.mla_up_proj_v(o_lat, w_uv.to(DEV))
    sync()
    assert torch.equal(o_v, o_v2), "fused and unfused value paths differ"
    assert torch.equal(l, l2)
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.all(o_v[b] == 0) and torch.all(torch.isneginf(l[b]))


@pytest.mark.parametrize("num_splits", [1, 8])
def test_decode_v_many_short_sequences(num_splits):
    # B beyond the in-kernel plan (plan kernel path) and many empty sequences.
    B, H, S = 1500, 16, 80
    lens = workloads.random_seqlens(B, 0, S, 2720).tolist()
    d = workloads.decode_inputs(B, H, lens, S_max=S, seed=2721)
    w_uv = workloads.w_uv_weights(H=H, Dv=256, seed=2722)
    o_v, l, ws = decode_v(d, w_uv, num_splits)
    check_plan(ws, d, num_splits)
    o_lat, l2, _ = decode(d, num_splits)
    o_v2 = binding.mla_up_proj_v(o_lat, w_uv.to(DEV))
    sync()
    assert torch.equal(o_v, o_v2) and torch.equal(l, l2)
    idx = [0, 1, 2, 700, B - 1] + [b for b, L in enumerate(lens) if L == 0][:3]
    ref = OM.mla_decode_values_explicit_ref(np64(d["q_lat"][idx]), np64(d["q_rope"][idx]), np64(w_uv),
                                            np64(d["cache"][idx]), [lens[i] for i in idx], SCALE)
    check_bf16(o_v[idx], ref, "o_v(sampled)")


def test_decode_v_varlen_workload_end_to_end(varlen):
    # The full variable-length step with the value output: GPU absorption ->
    # fused decode + W_UV, against the oracle (own absorption, own bf16 q_lat,
    # decode, projection), all 256 sequences; and bitwise against the
    # unfused path.
    d = varlen
    say("absorb + decode_v mla_varlen (B=256 H=128 Dv=128), all sequences")
    w_uv = workloads.w_uv_weights(H=128)
    ql = binding.mla_absorb_q(d["q_nope"].to(DEV), d["w_uk"].to(DEV))
    qr, c, sl = d["q_rope"].to(DEV), d["cache"].to(DEV), d["seqlens"].to(DEV)
    ws = binding.alloc_decode_v_workspace(256, 128, 32, DEV)
    o_v, l = binding.mla_decode_fwd_v(ql, qr, c, sl, w_uv.to(DEV), SCALE, 32, workspace=ws)
    o_lat, l2 = binding.mla_decode_fwd(ql, qr, c, sl, SCALE, 32)
    o_v2 = binding.mla_up_proj_v(o_lat, w_uv.to(DEV))
    sync()
    assert torch.equal(o_v, o_v2) and torch.equal(l, l2), "fused and unfused value paths differ"
    del c
    lens = d["seqlens"].tolist()
    w_uk, w_uv64 = np64(d["w_uk"]), np64(w_uv)
    ref = np.empty((256, 128, 128))
    Lr = np.empty((256, 128))
    for b0 in range(0, 256, 16):
        idx = list(range(b0, b0 + 16))
        Lm = max(lens[i] for i in idx)
        Ob, Lr[idx] = OM.absorb_decode_ref(np64(d["q_nope"][idx]), w_uk, np64(d["q_rope"][idx]),
                                           np64(d["cache"][idx, :Lm]), [lens[i] for i in idx], SCALE)
        ref[idx] = OM.up_project_v_ref(Ob, w_uv64)
    check_bf16(o_v, ref, "o_v (256 sequences)")
    check_lse(l, Lr, "LSE (256 sequences)")


# ----------------------------------- workspace reuse between calls ----
def _fill(dst, src):
    dst.copy_(src.to(DEV))


def test_decode_graph_replays_with_new_inputs():
    # A captured decode replayed with new inputs copied into the captured
    # buffers must equal an eager call on those inputs: nothing of an earlier
    # replay (plan, partials) may leak into the next.
    B, H, ns, S = 5, 128, 7, 2100
    lens = [900, 1, 0, 2100, 333]
    sets = [workloads.decode_inputs(B, H, lens, S_max=S, seed=2800 + i) for i in range(4)]
    ql = torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV)
    qr = torch.empty((B, H, 64), dtype=torch.bfloat16, device=DEV)
    c = torch.empty((B, S, 576), dtype=torch.bfloat16, device=DEV)
    sl = torch.empty((B,), dtype=torch.int32, device=DEV)
    ws = binding.alloc_decode_workspace(B, H, ns, DEV)
    o = torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
    for t, k in ((ql, "q_lat"), (qr, "q_rope"), (c, "cache"), (sl, "seqlens")):
        _fill(t, sets[0][k])
    binding.mla_decode_fwd(ql, qr, c, sl, SCALE, ns, workspace=ws, o=o, lse=lse)
    sync()
    plan = binding.read_plan(ws, B)
    assert any(n == 1 for n in plan["nsplit"]) and max(plan["nsplit"]) > 2, plan["nsplit"]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        binding.mla_decode_fwd(ql, qr, c, sl, SCALE, ns, workspace=ws, o=o, lse=lse)
    for rep in range(6):
        d = sets[rep % 4]
        for t, k in ((ql, "q_lat"), (qr, "q_rope"), (c, "cache"), (sl, "seqlens")):
            _fill(t, d[k])
        sync()
        graph.replay()
        sync()
        o_ref, l_ref, _ = decode(d, ns)
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), rep


def test_decode_alternating_inputs_share_a_workspace():
    # Two input sets through one workspace, alternately: every call gives the
    # result of its own inputs (a stale partial from the other set would show).
    B, H, ns = 4, 128, 32
    lens = [3000, 700, 4100, 64]
    dA = workloads.decode_inputs(B, H, lens, S_max=4100, seed=2810)
    dB = workloads.decode_inputs(B, H, lens, S_max=4100, seed=2811)
    ins = [tuple(d[k].to(DEV) for k in ("q_lat", "q_rope", "cache", "seqlens")) for d in (dA, dB)]
    ws = binding.alloc_decode_workspace(B, H, ns, DEV)
    first = []
    for i in range(8):
        o, l = binding.mla_decode_fwd(*ins[i % 2], SCALE, ns, workspace=ws)
        sync()
        if i < 2:
            first.append((o.clone(), l.clone()))
        else:
            assert torch.equal(o, first[i % 2][0]) and torch.equal(l, first[i % 2][1]), i
    plan = binding.read_plan(ws, B)
    assert max(plan["nsplit"]) >= 2, plan["nsplit"]
    Or, Lr = oracle_decode(dB)
    check_bf16(first[1][0], Or, "O set B")
    check_lse(first[1][1], Lr, "LSE set B")


def _ramped_decode_inputs(B, H, lens, S_max, seed, per_tile_log2=12.0):
    """Decode inputs whose scores rise by about per_tile_log2 (log2 units)
    every 32 tokens, for every head, so that the exponent base moves on every
    tile and the accumulators are rescaled: the rope parts of all heads'
    queries share a direction u, and each cached row's rope part is u times
    a ramp in the token index.  The latent part (the values) stays N(0,1)."""
    d = workloads.decode_inputs(B, H, lens, S_max=S_max, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    u = torch.randn(64, generator=g) / 8.0                      # |u| about 1
    qr = 3.0 * u + 0.3 * torch.randn((B, H, 64), generator=g)
    d["q_rope"] = qr.to(torch.bfloat16)
    # score from the ramp: SCALE * 3 |u|^2 * kappa per tile, times log2(e)
    kappa = per_tile_log2 / (SCALE * 3.0 * float(u @ u) * 1.4426950408889634)
    for b, L in enumerate(lens):
        t = torch.arange(L, dtype=torch.float32)[:, None]
        d["cache"][b, :L, 512:] = (d["cache"][b, :L, 512:].float() + (t / 32.0) * kappa * u).to(torch.bfloat16)
    return d


@pytest.mark.parametrize("num_splits", [1, 2, 32])
def test_decode_rising_scores_rescale_every_tile(num_splits):
    # Every tile's max exceeds the exponent base by more than the lazy-rescale
    # slack, so each step runs the accumulator rescale (alpha < 1), in every
    # piece of a split sequence too.
    lens = [300, 1000, 33]
    say(f"decode rising scores lens={lens} num_splits={num_splits}")
    d = _ramped_decode_inputs(3, 128, lens, 1024, seed=2101)
    o, l, ws = decode(d, num_splits)
    check_plan(ws, d, num_splits)
    Or, Lr = oracle_decode(d)
    assert float(np.abs(Lr - Lr.mean()).max()) > 50, "the ramp reaches far above the first tile"
    check_bf16(o, Or, "O")
    check_lse(l, Lr, "LSE")
