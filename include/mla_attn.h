/*
 * mla_attn.h - C ABI of libmla_attn.so: fused attention forward and the
 * weight-absorbed MLA decode over a latent KV cache, for AMD Instinct MI355X
 * (gfx950).
 *
 * Sources of the operations (web pages, cited by title and section):
 *   [FA2-v2 blog]     blog post implementing a FlashAttention-2 style "v2"
 *                     fp32 forward on CUDA cores (RTX 5080), sections 1-3.
 *   [MLA-FA3 article] article on fusing Multi-head Latent Attention with
 *                     FlashAttention-3 on Hopper: fused dataflow figure,
 *                     section 1 (cache row layout), section 2 (absorption
 *                     equation).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees, or synchronises.  Work is enqueued on
 *     `stream` (a hipStream_t; NULL = the device's null stream) and results
 *     are valid once that stream has been synchronised.
 *   - Tensors are dense, row-major, contiguous, in the layouts stated per
 *     function.  "bf16" is bfloat16 (1-8-7), "f32" is IEEE binary32.
 *   - Every pointer must be 16-byte aligned.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     validation failure the function returns the error code, enqueues
 *     nothing and leaves every output untouched.
 *   - MLA_ERR_HIP is returned when the HIP runtime reports an error while
 *     enqueueing (for example when no GPU is present).
 *   - Nothing throws across this interface.  The library keeps no state
 *     except a per-device cache of the compute-unit count and, for
 *     mla_decode_fwd_noalloc only, a fixed per-device scratch array.
 */
#ifndef MLA_ATTN_H
#define MLA_ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes and data types are plain ints with named values, so that any
 * int a caller passes (say 99 to mla_status_string, or 7 as a dtype) is a
 * valid argument that the library can reject; an enum type would make such
 * values undefined on the C++ side. */
typedef int mla_status_t;
enum {
    MLA_OK = 0,
    MLA_ERR_NULL = 1,        /* a required pointer is NULL                     */
    MLA_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be,
                                or out of range                                */
    MLA_ERR_UNSUPPORTED = 3, /* valid but not compiled (see per-function list) */
    MLA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned               */
    MLA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required        */
    MLA_ERR_HIP = 6,         /* the HIP runtime reported an error              */
    MLA_ERR_SCRATCH = 7      /* mla_decode_fwd_noalloc: the call needs more
                                than the fixed scratch                         */
};

typedef int mla_dtype_t;
enum { MLA_F32 = 0, MLA_BF16 = 1 };

/*
 * attn_fwd - fused attention forward (prefill), [FA2-v2 blog] sections 1.1-3.5.
 *
 * For every batch b < B and head h < H, with S = scale * Q K^T:
 *   causal = 0: O = softmax_row(S) V
 *   causal = 1: row i only sees keys j <= i (top-left aligned, N_q == N_k)
 *   lse[b,h,i] = natural log of sum_j exp(S_ij) over the visible keys.
 * Query tiles stay on chip while key/value tiles stream past them; the
 * softmax is computed online and the output is divided by the row sum once.
 *
 * q, k, v, o : [B, H, N, D] of `dtype` (o has the same dtype as q).
 * lse        : [B, H, N] f32, or NULL to skip it.
 * dtype      : MLA_F32 -> fp32 vector-ALU path (D = 64);
 *              MLA_BF16 -> bf16 inputs, MFMA products with fp32
 *              accumulation, bf16 output rounded to nearest even (D = 128).
 * Sizes      : B, H >= 1; N >= 0 (N = 0 enqueues nothing); B*H <= 2^31-1,
 *              N <= 2^20.  Other D values -> MLA_ERR_UNSUPPORTED.
 */
mla_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int D, float scale, int causal,
                      mla_dtype_t dtype, hipStream_t stream);

/*
 * attn_fwd_chunk - attn_fwd for a chunk of Nq queries against Nk keys
 * (prefill of a chunk over an existing cache).  The queries are the last Nq
 * positions of the key sequence, so the causal mask ([FA2-v2 blog] section
 * 3.4, generalised) is aligned at the bottom right: query row i sees keys
 * 0 .. i + (Nk - Nq).  With Nq = Nk this is attn_fwd.  A row that sees no
 * key (only when Nq > Nk) gets O = 0 and LSE = -inf.
 *
 * q, o : [B, H, Nq, D]     k, v : [B, H, Nk, D]     lse : [B, H, Nq] f32
 * Other arguments, dtypes, sizes (Nq, Nk each 0 .. 2^20), alignment and
 * errors as attn_fwd; Nq = 0 enqueues nothing, Nk = 0 gives every row
 * O = 0 and LSE = -inf.  q and o may be NULL when Nq = 0, k and v when
 * Nk = 0 (empty tensors); otherwise NULL gives MLA_ERR_NULL.
 */
mla_status_t attn_fwd_chunk(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Nq, int Nk, int D, float scale, int causal,
                            mla_dtype_t dtype, hipStream_t stream);

/*
 * mla_decode_workspace_size - bytes of device workspace mla_decode_fwd needs
 * for (B, H, num_splits) on the CURRENT device (the size depends on its
 * compute-unit count).  Returns 0 if the arguments are invalid or the device
 * cannot be queried.
 */
size_t mla_decode_workspace_size(int B, int H, int num_splits);

/*
 * mla_decode_fwd - absorbed MLA decode against the latent cache, one query
 * token per sequence, [MLA-FA3 article] fused dataflow figure and section 2.
 *
 * Each cache row is 576 bf16: dims 0..511 are the compressed latent c^KV,
 * dims 512..575 the decoupled RoPE key k^R (already rotated).  With W_UK
 * absorbed into the query (q_lat = q_nope W_UK, see mla_absorb_q):
 *   s_t = scale * ([q_lat || q_rope] . cache_row_t)
 *   o   = sum_t softmax(s)_t * cache_row_t[0:512]   (output in latent space)
 *   lse = natural log of sum_t exp(s_t)
 * No decompressed key or value is ever written.  The token range of each
 * sequence is split across compute units (at most num_splits pieces per
 * sequence) by an on-device planner; pieces write partials (bf16 outputs
 * normalised by their own weight sum, fp32 LSE) to the workspace and a
 * log-sum-exp combine merges them.  Two or three kernels are enqueued: the
 * split kernel (which computes the plan itself when num_splits >= 2 and
 * B <= 1024; otherwise a one-workgroup plan kernel runs first) and the
 * combine.  None waits on the host.
 *
 * q_lat    : [B, H, 512] bf16      q_rope : [B, H, 64] bf16
 * kv_cache : [B, S_max, 576] bf16; token t of sequence b is row b*S_max + t.
 *            Rows t >= seqlens[b] are never read.
 * seqlens  : [B] int32 on the device, 0 <= seqlens[b] <= S_max.  A value
 *            outside that range is clamped into it (and the planner records
 *            it in workspace word 7); a length of 0 gives o = 0, lse = -inf.
 * o        : [B, H, 512] bf16 (round to nearest even)
 * lse      : [B, H] f32 (may be NULL to skip it)
 * num_splits : 1..32.  1 = every sequence handled whole by one workgroup.
 * workspace: at least mla_decode_workspace_size(B, H, num_splits) bytes of
 *            device memory; contents on entry are ignored.  Calls that share
 *            one workspace must be ordered on one stream.
 * Sizes    : B >= 1, H >= 16 with H % 16 == 0, H <= 1024, S_max >= 1,
 *            B * S_max <= 2^31 / 576.
 */
mla_status_t mla_decode_fwd(const void* q_lat, const void* q_rope, const void* kv_cache,
                            const int* seqlens, void* o, float* lse,
                            int B, int H, int S_max, float scale, int num_splits,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mla_decode_v_workspace_size - bytes of device workspace mla_decode_fwd_v
 * needs for (B, H, num_splits) on the CURRENT device; 0 if the arguments are
 * invalid or the device cannot be queried.  At least
 * mla_decode_workspace_size(B, H, num_splits): every sequence keeps its
 * latent partials (B * H * 1 KiB and up).
 */
size_t mla_decode_v_workspace_size(int B, int H, int num_splits);

/*
 * mla_decode_fwd_v - the absorbed MLA decode followed by the value
 * up-projection, with the split merge fused into the projection
 * ([MLA-FA3 article] fused dataflow figure: W_UK and W_UV belong to the
 * in-place absorption stage; the online-softmax partial reduction precedes
 * the output).
 *   o_lat[b, h] = the latent output of mla_decode_fwd (merged in fp32,
 *                 rounded to bf16, never written to memory)
 *   o_v[b, h, :] = o_lat[b, h, :] @ W_UV[h]    (fp32 accumulation)
 *   lse[b, h]   = as mla_decode_fwd
 * Attention is linear in its values, so o_v equals attention over the
 * explicitly decompressed values c^KV W_UV[h] without forming them.  The
 * results are bitwise those of mla_decode_fwd followed by mla_up_proj_v.
 * Two kernels are enqueued (the split kernel, with the plan inside it or a
 * plan kernel before it, then the merge + up-projection).
 *
 * q_lat, q_rope, kv_cache, seqlens, B, H, S_max, scale, num_splits: as
 *            mla_decode_fwd.
 * w_uv     : [H, 512, Dv] bf16 (per head: latent dim x value dim)
 * o_v      : [B, H, Dv] bf16 (round to nearest even); a length of 0 gives 0.
 * lse      : [B, H] f32 (may be NULL to skip it)
 * Dv       : multiple of 128, at most 4096 (else MLA_ERR_UNSUPPORTED).
 * workspace: at least mla_decode_v_workspace_size(B, H, num_splits) bytes.
 */
mla_status_t mla_decode_fwd_v(const void* q_lat, const void* q_rope, const void* kv_cache,
                              const int* seqlens, const void* w_uv, void* o_v, float* lse,
                              int B, int H, int S_max, int Dv, float scale, int num_splits,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mla_decode_fwd_noalloc - mla_decode_fwd without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same inputs, outputs, layouts, results (bitwise) and errors as
 * mla_decode_fwd, whose kernels it runs.  The workspace is a fixed device
 * array inside the library, MLA_DECODE_NOALLOC_SCRATCH_BYTES (72 MiB) per
 * device, allocated when the library's code is loaded on that device and
 * held until the process ends; this call allocates and frees nothing
 * itself.  A shape whose workspace (mla_decode_workspace_size) exceeds it
 * returns MLA_ERR_SCRATCH and enqueues nothing; H = 128 fits up to 256
 * split-kernel parts (any B on a 256-CU device with num_splits >= 2, and
 * every B with num_splits = 1).  Nothing in the scratch needs to start at
 * zero: every call writes what it reads.
 * Every call on one device shares that device's scratch: calls that may
 * overlap in time on one device (several streams, several host threads)
 * race and give undefined results; order them on one stream.
 */
#define MLA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)
mla_status_t mla_decode_fwd_noalloc(const void* q_lat, const void* q_rope, const void* kv_cache,
                                    const int* seqlens, void* o, float* lse,
                                    int B, int H, int S_max, float scale, int num_splits,
                                    hipStream_t stream);

/*
 * mla_combine - log-sum-exp merge of split-KV partials ([MLA-FA3 article],
 * "online softmax scaling and partial reduction" stage of the dataflow).
 *
 * o_part   : [B, H, num_splits, 512] f32, each split normalised over its own
 *            token range (o_s = sum over the range of softmax weights times
 *            rows, divided by the range's weight sum).
 * lse_part : [B, H, num_splits] f32; -inf marks an empty split.
 *   lse = log sum_s exp(lse_s)   (-inf when every split is empty)
 *   o   = sum_s exp(lse_s - lse) o_s   (0 when every split is empty)
 * o        : [B, H, 512] bf16 (round to nearest even)
 * lse      : [B, H] f32 (may be NULL)
 * Sizes    : B, H >= 1, 1 <= num_splits <= 32.
 */
mla_status_t mla_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                         int B, int H, int num_splits, hipStream_t stream);

/*
 * mla_absorb_q - weight absorption prologue, [MLA-FA3 article] section 2:
 *   q_lat[b, h, :] = q_nope[b, h, :] @ W_UK[h]     (fp32 accumulation)
 * q_nope : [B, H, Dn] bf16     w_uk : [H, Dn, Dl] bf16
 * q_lat  : [B, H, Dl] bf16 (round to nearest even)
 * Sizes  : B, H >= 1; Dn % 32 == 0, 32 <= Dn <= 512; Dl % 128 == 0,
 *          128 <= Dl <= 4096; otherwise MLA_ERR_UNSUPPORTED / MLA_ERR_SHAPE.
 */
mla_status_t mla_absorb_q(const void* q_nope, const void* w_uk, void* q_lat,
                          int B, int H, int Dn, int Dl, hipStream_t stream);

/*
 * mla_up_proj_v - value up-projection of the latent decode output,
 * [MLA-FA3 article] fused dataflow figure (the W_UK / W_UV projections of
 * the in-place absorption stage):
 *   o_v[b, h, :] = o_lat[b, h, :] @ W_UV[h]     (fp32 accumulation)
 * Attention is linear in its values, so this equals attending over the
 * explicitly decompressed values c^KV W_UV[h], without forming them.
 * o_lat : [B, H, Dl] bf16 (e.g. the o of mla_decode_fwd, Dl = 512)
 * w_uv  : [H, Dl, Dv] bf16 (per head: latent dim x value dim)
 * o_v   : [B, H, Dv] bf16 (round to nearest even); written, never read.
 * All buffers are device memory owned by the caller, 16-byte aligned.
 * Sizes : B, H >= 1; Dl % 32 == 0, 32 <= Dl <= 512; Dv % 128 == 0,
 *         128 <= Dv <= 4096; otherwise MLA_ERR_UNSUPPORTED / MLA_ERR_SHAPE,
 *         and nothing is enqueued.
 */
mla_status_t mla_up_proj_v(const void* o_lat, const void* w_uv, void* o_v,
                           int B, int H, int Dl, int Dv, hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* mla_status_string(mla_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ATTN_H */
