"""mla_decode_fwd_noalloc (the library's fixed scratch as workspace) against
mla_decode_fwd (caller's workspace): same kernels, so the outputs must be
bitwise equal, on two calls in a row with the second one smaller, and at the
largest shape the benchmark runs (256 split-kernel parts at H = 128)."""

import math

import pytest
import torch

from mla_latent_kv_attn_amd import binding, workloads
from tests.gpu_util import say, sync

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCALE = 1 / math.sqrt(576)


def both(d, ns):
    ql, qr, c, sl = (d[k].to(DEV) for k in ("q_lat", "q_rope", "cache", "seqlens"))
    B, H, _ = ql.shape
    ws = binding.alloc_decode_workspace(B, H, ns, DEV)
    o_ref, l_ref = binding.mla_decode_fwd(ql, qr, c, sl, SCALE, ns, workspace=ws)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    binding.mla_decode_fwd_noalloc(ql, qr, c, sl, SCALE, ns, o=o, lse=lse)
    sync()
    return o, lse, o_ref, l_ref


def test_noalloc_matches_workspace_call_twice_second_smaller():
    cases = [(workloads.decode_inputs(64, 128, workloads.random_seqlens(64, 1, 4096, 3100).tolist(),
                                      S_max=4096, seed=3101), 32),
             (workloads.decode_inputs(3, 32, [700, 0, 65], S_max=700, seed=3102), 7)]
    for d, ns in cases:
        B, H = d["q_lat"].shape[:2]
        say(f"noalloc decode B={B} H={H} num_splits={ns}")
        o, lse, o_ref, l_ref = both(d, ns)
        assert torch.equal(o, o_ref), "O differs from mla_decode_fwd"
        assert torch.equal(lse, l_ref), "LSE differs from mla_decode_fwd"


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    B, H, S = 256, 256, 16
    need = binding.mla_decode_workspace_size(B, H, 32)
    assert need > (72 << 20)
    ql = torch.zeros((B, H, 512), dtype=torch.bfloat16, device=DEV)
    qr = torch.zeros((B, H, 64), dtype=torch.bfloat16, device=DEV)
    c = torch.zeros((B, S, 576), dtype=torch.bfloat16, device=DEV)
    sl = torch.full((B,), S, dtype=torch.int32, device=DEV)
    o = torch.full((B, H, 512), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(binding.MlaError) as e:
        binding.mla_decode_fwd_noalloc(ql, qr, c, sl, SCALE, 32, o=o)
    assert e.value.status == binding.MLA_ERR_SCRATCH
    sync()
    assert torch.all(o == 3.0)
