"""ctypes binding of libmla_attn.so (C ABI in include/mla_attn.h).

Argument marshalling only: torch tensors are checked for device, dtype,
shape and contiguity, then passed as raw device pointers together with the
current HIP stream.  Every computation happens in the library's kernels.
The library is loaded on first use; if it is missing, or if a tensor is not
on a GPU, the call raises -- there is no CPU fallback.
"""

import ctypes
import os

import torch

# MLA_ATTN_LIB names another build of the same library (the host-only
# sanitizer build); by default the in-tree libmla_attn.so is loaded.
_LIB_PATH = os.environ.get("MLA_ATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "libmla_attn.so")
_lib = None

(MLA_OK, MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED, MLA_ERR_ALIGN, MLA_ERR_WORKSPACE, MLA_ERR_HIP,
 MLA_ERR_SCRATCH) = range(8)
MLA_F32, MLA_BF16 = 0, 1

EXPORTED = ("attn_fwd", "attn_fwd_chunk", "mla_decode_workspace_size", "mla_decode_fwd", "mla_decode_fwd_noalloc",
            "mla_decode_v_workspace_size", "mla_decode_fwd_v", "mla_combine", "mla_absorb_q", "mla_up_proj_v",
            "mla_status_string")


class MlaError(RuntimeError):
    """A non-zero mla_status_t returned by the library."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {_string(status)} (status {status})")


def load(path=None):
    """Load (once) and return the library handle with argument types set."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libmla_attn.so not built at {p}; run __graft_entry__.build() "
                           "or python -m mla_latent_kv_attn_amd.build")
    lib = ctypes.CDLL(p)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.attn_fwd.restype = i
    lib.attn_fwd_chunk.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.attn_fwd_chunk.restype = i
    lib.mla_decode_workspace_size.argtypes = [i, i, i]
    lib.mla_decode_workspace_size.restype = sz
    lib.mla_decode_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, f, i, vp, sz, vp]
    lib.mla_decode_fwd.restype = i
    lib.mla_decode_v_workspace_size.argtypes = [i, i, i]
    lib.mla_decode_v_workspace_size.restype = sz
    lib.mla_decode_fwd_v.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.mla_decode_fwd_v.restype = i
    lib.mla_decode_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, f, i, vp]
    lib.mla_decode_fwd_noalloc.restype = i
    lib.mla_combine.argtypes = [vp, vp, vp, vp, i, i, i, vp]
    lib.mla_combine.restype = i
    lib.mla_absorb_q.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib.mla_absorb_q.restype = i
    lib.mla_up_proj_v.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib.mla_up_proj_v.restype = i
    lib.mla_status_string.argtypes = [i]
    lib.mla_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _string(status):
    return load().mla_status_string(int(status)).decode()


def mla_status_string(status):
    return _string(status)


def _check(fn, status):
    if status != MLA_OK:
        raise MlaError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def attn_fwd(q, k, v, scale, causal, o=None, lse=None, want_lse=True):
    """Fused attention forward. q, k, v: [B, H, N, D] fp32 (D=64) or bf16 (D=128).
    Returns (o, lse) with lse [B, H, N] fp32 (None if want_lse is False)."""
    B, H, N, D = q.shape
    dt = {torch.float32: MLA_F32, torch.bfloat16: MLA_BF16}.get(q.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, q.dtype, (B, H, N, D))
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", q.dtype, (B, H, N, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H, N))
    st = load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, D, float(scale),
                         int(bool(causal)), dt, _stream(q.device))
    _check("attn_fwd", st)
    return o, lse


def attn_fwd_chunk(q, k, v, scale, causal, o=None, lse=None, want_lse=True):
    """Attention of Nq queries against Nk keys, causal mask aligned bottom
    right (row i sees keys <= i + Nk - Nq). q [B,H,Nq,D]; k, v [B,H,Nk,D].
    Returns (o [B,H,Nq,D], lse [B,H,Nq] or None)."""
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    dt = {torch.float32: MLA_F32, torch.bfloat16: MLA_BF16}.get(q.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {q.dtype}")
    _need(q, "q", q.dtype, (B, H, Nq, D))
    _need(k, "k", q.dtype, (B, H, Nk, D))
    _need(v, "v", q.dtype, (B, H, Nk, D))
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", q.dtype, (B, H, Nq, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H, Nq))
    st = load().attn_fwd_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, D, float(scale),
                               int(bool(causal)), dt, _stream(q.device))
    _check("attn_fwd_chunk", st)
    return o, lse


def mla_decode_workspace_size(B, H, num_splits):
    return int(load().mla_decode_workspace_size(int(B), int(H), int(num_splits)))


def mla_decode_fwd(q_lat, q_rope, kv_cache, seqlens, scale, num_splits, workspace=None, o=None, lse=None):
    """Absorbed MLA decode. q_lat [B,H,512] bf16, q_rope [B,H,64] bf16,
    kv_cache [B,S_max,576] bf16, seqlens [B] int32 (device).
    Returns (o [B,H,512] bf16, lse [B,H] fp32)."""
    B, H, _ = q_lat.shape
    S_max = kv_cache.shape[1]
    _need(q_lat, "q_lat", torch.bfloat16, (B, H, 512))
    _need(q_rope, "q_rope", torch.bfloat16, (B, H, 64))
    _need(kv_cache, "kv_cache", torch.bfloat16, (B, S_max, 576))
    _need(seqlens, "seqlens", torch.int32, (B,))
    if workspace is None:
        workspace = alloc_decode_workspace(B, H, num_splits, q_lat.device)
    _need(workspace, "workspace", torch.uint8)
    if o is None:
        o = torch.empty((B, H, 512), dtype=torch.bfloat16, device=q_lat.device)
    _need(o, "o", torch.bfloat16, (B, H, 512))
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_lat.device)
    _need(lse, "lse", torch.float32, (B, H))
    st = load().mla_decode_fwd(_ptr(q_lat), _ptr(q_rope), _ptr(kv_cache), _ptr(seqlens), _ptr(o), _ptr(lse),
                               B, H, S_max, float(scale), int(num_splits), _ptr(workspace),
                               workspace.numel(), _stream(q_lat.device))
    _check("mla_decode_fwd", st)
    return o, lse


def mla_decode_v_workspace_size(B, H, num_splits):
    return int(load().mla_decode_v_workspace_size(int(B), int(H), int(num_splits)))


def alloc_decode_v_workspace(B, H, num_splits, device):
    n = mla_decode_v_workspace_size(B, H, num_splits)
    if n == 0:
        raise MlaError("mla_decode_v_workspace_size", MLA_ERR_SHAPE)
    return torch.empty(n, dtype=torch.uint8, device=device)


def mla_decode_fwd_v(q_lat, q_rope, kv_cache, seqlens, w_uv, scale, num_splits, workspace=None, o_v=None, lse=None):
    """Decode + value up-projection. w_uv [H,512,Dv] bf16.
    Returns (o_v [B,H,Dv] bf16, lse [B,H] fp32)."""
    B, H, _ = q_lat.shape
    S_max = kv_cache.shape[1]
    Dv = w_uv.shape[2]
    _need(q_lat, "q_lat", torch.bfloat16, (B, H, 512))
    _need(q_rope, "q_rope", torch.bfloat16, (B, H, 64))
    _need(kv_cache, "kv_cache", torch.bfloat16, (B, S_max, 576))
    _need(seqlens, "seqlens", torch.int32, (B,))
    _need(w_uv, "w_uv", torch.bfloat16, (H, 512, Dv))
    if workspace is None:
        workspace = alloc_decode_v_workspace(B, H, num_splits, q_lat.device)
    _need(workspace, "workspace", torch.uint8)
    if o_v is None:
        o_v = torch.empty((B, H, Dv), dtype=torch.bfloat16, device=q_lat.device)
    _need(o_v, "o_v", torch.bfloat16, (B, H, Dv))
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_lat.device)
    _need(lse, "lse", torch.float32, (B, H))
    st = load().mla_decode_fwd_v(_ptr(q_lat), _ptr(q_rope), _ptr(kv_cache), _ptr(seqlens), _ptr(w_uv), _ptr(o_v),
                                 _ptr(lse), B, H, S_max, Dv, float(scale), int(num_splits), _ptr(workspace),
                                 workspace.numel(), _stream(q_lat.device))
    _check("mla_decode_fwd_v", st)
    return o_v, lse


def mla_decode_fwd_noalloc(q_lat, q_rope, kv_cache, seqlens, scale, num_splits, o=None, lse=None):
    """mla_decode_fwd with the library's fixed device scratch as workspace
    (no workspace argument; calls on one device must not overlap)."""
    B, H, _ = q_lat.shape
    S_max = kv_cache.shape[1]
    _need(q_lat, "q_lat", torch.bfloat16, (B, H, 512))
    _need(q_rope, "q_rope", torch.bfloat16, (B, H, 64))
    _need(kv_cache, "kv_cache", torch.bfloat16, (B, S_max, 576))
    _need(seqlens, "seqlens", torch.int32, (B,))
    if o is None:
        o = torch.empty((B, H, 512), dtype=torch.bfloat16, device=q_lat.device)
    _need(o, "o", torch.bfloat16, (B, H, 512))
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_lat.device)
    _need(lse, "lse", torch.float32, (B, H))
    st = load().mla_decode_fwd_noalloc(_ptr(q_lat), _ptr(q_rope), _ptr(kv_cache), _ptr(seqlens), _ptr(o), _ptr(lse),
                                       B, H, S_max, float(scale), int(num_splits), _stream(q_lat.device))
    _check("mla_decode_fwd_noalloc", st)
    return o, lse


def alloc_decode_workspace(B, H, num_splits, device):
    n = mla_decode_workspace_size(B, H, num_splits)
    if n == 0:
        raise MlaError("mla_decode_workspace_size", MLA_ERR_SHAPE)
    return torch.empty(n, dtype=torch.uint8, device=device)


def mla_combine(o_part, lse_part, o=None, lse=None):
    """LSE merge of split partials. o_part [B,H,S,512] fp32, lse_part [B,H,S] fp32."""
    B, H, S, Dv = o_part.shape
    _need(o_part, "o_part", torch.float32, (B, H, S, 512))
    _need(lse_part, "lse_part", torch.float32, (B, H, S))
    if o is None:
        o = torch.empty((B, H, 512), dtype=torch.bfloat16, device=o_part.device)
    _need(o, "o", torch.bfloat16, (B, H, 512))
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=o_part.device)
    _need(lse, "lse", torch.float32, (B, H))
    st = load().mla_combine(_ptr(o_part), _ptr(lse_part), _ptr(o), _ptr(lse), B, H, S, _stream(o_part.device))
    _check("mla_combine", st)
    return o, lse


def mla_absorb_q(q_nope, w_uk, q_lat=None):
    """q_lat[b,h,:] = q_nope[b,h,:] @ w_uk[h]. q_nope [B,H,Dn] bf16, w_uk [H,Dn,Dl] bf16."""
    B, H, Dn = q_nope.shape
    Dl = w_uk.shape[2]
    _need(q_nope, "q_nope", torch.bfloat16, (B, H, Dn))
    _need(w_uk, "w_uk", torch.bfloat16, (H, Dn, Dl))
    if q_lat is None:
        q_lat = torch.empty((B, H, Dl), dtype=torch.bfloat16, device=q_nope.device)
    _need(q_lat, "q_lat", torch.bfloat16, (B, H, Dl))
    st = load().mla_absorb_q(_ptr(q_nope), _ptr(w_uk), _ptr(q_lat), B, H, Dn, Dl, _stream(q_nope.device))
    _check("mla_absorb_q", st)
    return q_lat


def mla_up_proj_v(o_lat, w_uv, o_v=None):
    """o_v[b,h,:] = o_lat[b,h,:] @ w_uv[h]. o_lat [B,H,Dl] bf16, w_uv [H,Dl,Dv] bf16."""
    B, H, Dl = o_lat.shape
    Dv = w_uv.shape[2]
    _need(o_lat, "o_lat", torch.bfloat16, (B, H, Dl))
    _need(w_uv, "w_uv", torch.bfloat16, (H, Dl, Dv))
    if o_v is None:
        o_v = torch.empty((B, H, Dv), dtype=torch.bfloat16, device=o_lat.device)
    _need(o_v, "o_v", torch.bfloat16, (B, H, Dv))
    st = load().mla_up_proj_v(_ptr(o_lat), _ptr(w_uv), _ptr(o_v), B, H, Dl, Dv, _stream(o_lat.device))
    _check("mla_up_proj_v", st)
    return o_v


def read_plan(workspace, B):
    """Decode the planner's integer output from a workspace after a call
    (for tests): header words and the per-sequence / per-part arrays."""
    hdr = workspace[:256].view(torch.int32).cpu().tolist()
    parts = hdr[6]
    n_ints = 64 + 5 * B + parts
    ws = workspace[: 4 * n_ints].view(torch.int32).cpu().tolist()
    out = {"parts_used": hdr[0], "t": hdr[1], "C": hdr[2], "tile": hdr[3], "c0": hdr[4],
           "mode": "whole" if hdr[5] == 1 else "line", "parts": parts, "clamped": hdr[7],
           "max_n": hdr[8], "B": hdr[9], "t_min": hdr[10], "num_splits": hdr[11]}
    off = 64
    for nm in ("len", "n", "start", "first", "nsplit"):
        out[nm] = ws[off:off + B]
        off += B
    out["part_first_seq"] = ws[off:off + parts]
    return out
