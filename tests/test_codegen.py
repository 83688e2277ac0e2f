"""Generated-code checks for the decode split kernel (CPU only: hipcc
cross-compiles gfx950 here).

The kernel keeps its value accumulators in fixed AGPRs named by inline asm
(a[4k .. 4k+3] for block k), which the compiler does not track.  That is only
sound while the compiler itself allocates no AGPR and spills nothing: a
compiler-chosen AGPR (an accumulator of a compiler MFMA, or a VGPR spilled to
an AGPR) would silently overwrite accumulator state.  The inline asm always
writes AGPRs in bracket form (a[N] or a[N:M]); the compiler prints single
AGPRs bare (aN), so any bare AGPR operand in the kernel body is a
compiler-allocated one.
"""

import os
import re
import subprocess

import pytest

from mla_latent_kv_attn_amd import build as B

SRC = os.path.join(B.CSRC, "mla_decode.hip")
KERNEL = "_ZN3mla16mla_split_kernelENS_9DecodeCtxE"


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "mla_decode.s"
    cmd = [B.HIPCC, *B.COMMON_FLAGS, "--cuda-device-only", "-S", SRC, "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return out.read_text()


def kernel_body(text):
    lines = text.splitlines()
    start = next(i for i, l in enumerate(lines) if l.startswith(KERNEL + ":"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return [l.split(";")[0].strip() for l in lines[start:end]]


def kernel_meta(text, key):
    # per-kernel metadata entries start with "- .agpr_count"; pick the split kernel's
    blocks = [b for b in re.split(r"\n\s+- \.agpr_count", text) if re.search(r"\.name:\s+" + re.escape(KERNEL) + r"\b", b)]
    assert len(blocks) == 1, "kernel metadata missing"
    v = re.findall(r"\." + key + r":\s+(\d+)", blocks[0])
    assert v, key
    return int(v[0])


def test_no_compiler_allocated_agprs(asm):
    bare = re.compile(r"(?<![\w\[:])a\d+\b")
    offenders = []
    for line in kernel_body(asm):
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        op, _, operands = line.partition(" ")
        if bare.search(operands):
            offenders.append(line)
    assert not offenders, offenders[:5]


def test_no_vgpr_spills_or_scratch(asm):
    # SGPR spills (in the per-piece set-up) go to lanes of a VGPR, which is
    # harmless; VGPR spills and any scratch memory are not allowed.
    assert kernel_meta(asm, "vgpr_spill_count") == 0
    m = re.search(KERNEL + r"\n(?:.*\n)*?\s+\.amdhsa_private_segment_fixed_size (\d+)", asm)
    assert m and int(m.group(1)) == 0
    assert not any(l.startswith("scratch_") for l in kernel_body(asm))


def test_one_step_of_each_kind(asm):
    # the piece body holds exactly one first step (72 MFMAs), one middle step
    # (136) and one last step (64): nothing is duplicated by the compiler
    body = kernel_body(asm)
    assert sum(1 for l in body if l.startswith("v_mfma")) == 72 + 136 + 64


def _vregs(operand):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", operand)
    return {int(m.group(1))} if m else set()


def test_valu_writes_reach_mfma_sources_two_wait_states_early(asm):
    # The MFMAs are inline asm, so the compiler inserts no wait states for
    # them.  A VGPR that a VALU instruction writes (for instance a move that
    # joins the two halves of a value fragment) may be read as an MFMA
    # source only two wait states later (s_nop N counts N + 1, any other
    # instruction 1): the rule the compiler itself applies on gfx950.
    body = [l for l in kernel_body(asm) if l and not l.startswith(".") and not l.endswith(":")]
    bad = []
    for i, line in enumerate(body):
        if not line.startswith("v_mfma"):
            continue
        args = [a.strip() for a in line.partition(" ")[2].split(",")]
        src = set().union(*(_vregs(a) for a in args[1:4]))
        ws = 0
        for j in range(i - 1, max(-1, i - 16), -1):
            op, _, rest = body[j].partition(" ")
            dst = rest.split(",")[0].strip() if rest else ""
            if op.startswith("v_") and not op.startswith("v_mfma") and _vregs(dst) & src:
                if ws < 2:
                    bad.append((body[j], line))
                break
            ws += int(rest) + 1 if op == "s_nop" else 1
            if ws >= 2:
                break
    assert not bad, bad[:4]
