// api.hip - host side of the C ABI declared in include/mla_attn.h:
// argument validation, launch-configuration choice and dispatch.
//
// Validation runs before any HIP call, so a rejected call touches no device
// state and enqueues nothing.  The only library state is a per-device cache
// of the compute-unit count (filled once, lock-free, idempotent).
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>

#include "mla_attn.h"
#include "mla_plan.h"

#define MLA_EXPORT extern "C" __attribute__((visibility("default")))

namespace mla {
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                               int Nq, int Nk, float scale, bool causal, hipStream_t stream);
hipError_t launch_attn_fwd_bf16(const __bf16* q, const __bf16* k, const __bf16* v, __bf16* o, float* lse, int B,
                                int H, int Nq, int Nk, float scale, bool causal, hipStream_t stream);
hipError_t launch_mla_decode(const __bf16* q_lat, const __bf16* q_rope, const __bf16* cache, const int* seqlens,
                             __bf16* o, float* lse, int B, int H, int S_max, float scale, int num_splits,
                             const PlanLayout& L, int c0, int t_min, void* workspace, hipStream_t stream,
                             const __bf16* w_uv, int Dv);
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_mla_combine(const float* o_part, const float* lse_part, __bf16* o, float* lse, int B, int H,
                              int S, hipStream_t stream);
hipError_t launch_mla_absorb(const __bf16* q_nope, const __bf16* w_uk, __bf16* q_lat, int B, int H, int Dn, int Dl,
                             hipStream_t stream);
}  // namespace mla

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not yet queried

// Compute units of the current device, or -1 if it cannot be queried.
int current_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return -1;
    g_cu_count[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool good_scale(float s) { return std::isfinite(s) && s > 0.f; }

// Launch configuration of the split-KV decode.  Parts = one workgroup per
// compute unit on the cost line (at most B * num_splits); one per sequence
// when num_splits == 1.  c0 charges each sequence the fixed cost of a piece
// (loading its query block, filling and draining the tile pipeline, writing
// its output), in 32-token plan tiles.  Timestamps per workgroup on MI355X
// (256 sequences of 256..8192 tokens) put that cost at about 15 us, against
// about 1.9 us per 32-token step; c0 = 8 (256 tokens) measured fastest
// among 6, 8, 10 and 12 (321.9 us per call on one box, against 322.8, 323.9
// and 325.9 us; the 16 x 4096 batch is within 0.3 us for all four).  t_min
// keeps parts from becoming so short that the fixed cost dominates.
struct DecodeConfig {
    int parts, slots, c0, t_min;
};

// vmode (mla_decode_fwd_v): every piece keeps a partial slot, b + p.
DecodeConfig decode_config(int B, int num_splits, int cus, bool vmode = false) {
    DecodeConfig c;
    c.c0 = 8;
    c.t_min = 8;
    if (num_splits == 1) {
        c.parts = B;
        c.slots = 0;
    } else {
        long long p = (long long)B * num_splits;
        if (p > cus) p = cus;
        if (p > mla::kPlanMaxParts) p = mla::kPlanMaxParts;
        c.parts = (int)p;
        c.slots = 2 * c.parts;
    }
    if (vmode) c.slots = B + c.parts;
    return c;
}

bool decode_shape_ok(int B, int H, int num_splits) {
    return B >= 1 && B <= mla::kMaxBatch && H >= 16 && H % 16 == 0 && H <= 1024 && num_splits >= 1 &&
           num_splits <= mla::kMaxSplits;
}

mla_status_t hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

}  // namespace

MLA_EXPORT const char* mla_status_string(mla_status_t s) {
    switch (s) {
        case MLA_OK: return "MLA_OK";
        case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
        case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: a size or scalar argument is out of range";
        case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: combination not compiled";
        case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: a pointer is not 16-byte aligned";
        case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
        case MLA_ERR_HIP: return "MLA_ERR_HIP: the HIP runtime reported an error";
        case MLA_ERR_SCRATCH:
            return "MLA_ERR_SCRATCH: the call needs more workspace than the library's fixed 72 MiB scratch";
    }
    return "unknown mla_status_t";
}

namespace {
// Shared by attn_fwd (Nq = Nk) and attn_fwd_chunk.
mla_status_t attn_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                         int Nk, int D, float scale, int causal, mla_dtype_t dtype, hipStream_t stream) {
    // Empty tensors may come as NULL: q, o are needed only for Nq > 0, k, v for Nk > 0.
    if ((Nq != 0 && (!q || !o)) || (Nk != 0 && (!k || !v))) return MLA_ERR_NULL;
    if (B < 1 || H < 1 || Nq < 0 || Nk < 0 || D < 1 || Nq > (1 << 20) || Nk > (1 << 20) ||
        (long long)B * H > INT_MAX)
        return MLA_ERR_SHAPE;
    if ((causal != 0 && causal != 1) || !good_scale(scale)) return MLA_ERR_SHAPE;
    if (dtype == MLA_F32) {
        if (D != 64) return MLA_ERR_UNSUPPORTED;
    } else if (dtype == MLA_BF16) {
        if (D != 128) return MLA_ERR_UNSUPPORTED;
    } else {
        return MLA_ERR_UNSUPPORTED;
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
        return MLA_ERR_ALIGN;
    if (Nq == 0) return MLA_OK;
    hipError_t e;
    if (dtype == MLA_F32)
        e = mla::launch_attn_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                     static_cast<const float*>(v), static_cast<float*>(o), lse, B, H, Nq, Nk, scale,
                                     causal == 1, stream);
    else
        e = mla::launch_attn_fwd_bf16(static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                                      static_cast<const __bf16*>(v), static_cast<__bf16*>(o), lse, B, H, Nq, Nk, scale,
                                      causal == 1, stream);
    return hip_status(e);
}
}  // namespace

MLA_EXPORT mla_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                 int N, int D, float scale, int causal, mla_dtype_t dtype, hipStream_t stream) {
    return attn_common(q, k, v, o, lse, B, H, N, N, D, scale, causal, dtype, stream);
}

MLA_EXPORT mla_status_t attn_fwd_chunk(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                       int H, int Nq, int Nk, int D, float scale, int causal, mla_dtype_t dtype,
                                       hipStream_t stream) {
    return attn_common(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, dtype, stream);
}

MLA_EXPORT size_t mla_decode_workspace_size(int B, int H, int num_splits) {
    if (!decode_shape_ok(B, H, num_splits)) return 0;
    const int cus = current_cu_count();
    if (cus <= 0) return 0;
    const DecodeConfig c = decode_config(B, num_splits, cus);
    return mla::plan_layout(B, H, c.parts, c.slots).total_bytes;
}

MLA_EXPORT mla_status_t mla_decode_fwd(const void* q_lat, const void* q_rope, const void* kv_cache,
                                       const int* seqlens, void* o, float* lse, int B, int H, int S_max, float scale,
                                       int num_splits, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    if (!q_lat || !q_rope || !kv_cache || !seqlens || !o) return MLA_ERR_NULL;
    if (!decode_shape_ok(B, H, num_splits) || S_max < 1 || !good_scale(scale)) return MLA_ERR_SHAPE;
    if ((long long)B * S_max > (long long)INT_MAX / mla::kRow) return MLA_ERR_SHAPE;
    if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(kv_cache) || !aligned16(seqlens) || !aligned16(o) ||
        (lse && !aligned16(lse)) || (workspace && !aligned16(workspace)))
        return MLA_ERR_ALIGN;
    if (!workspace) return MLA_ERR_WORKSPACE;
    const int cus = current_cu_count();
    if (cus <= 0) return MLA_ERR_HIP;
    const DecodeConfig c = decode_config(B, num_splits, cus);
    const mla::PlanLayout L = mla::plan_layout(B, H, c.parts, c.slots);
    if (workspace_bytes < L.total_bytes) return MLA_ERR_WORKSPACE;
    return hip_status(mla::launch_mla_decode(
        static_cast<const __bf16*>(q_lat), static_cast<const __bf16*>(q_rope), static_cast<const __bf16*>(kv_cache),
        seqlens, static_cast<__bf16*>(o), lse, B, H, S_max, scale, num_splits, L, c.c0, c.t_min, workspace, stream, nullptr, 0));
}

MLA_EXPORT mla_status_t mla_decode_fwd_noalloc(const void* q_lat, const void* q_rope, const void* kv_cache,
                                               const int* seqlens, void* o, float* lse, int B, int H, int S_max,
                                               float scale, int num_splits, hipStream_t stream) {
    if (!q_lat || !q_rope || !kv_cache || !seqlens || !o) return MLA_ERR_NULL;
    if (!decode_shape_ok(B, H, num_splits) || S_max < 1 || !good_scale(scale)) return MLA_ERR_SHAPE;
    if ((long long)B * S_max > (long long)INT_MAX / mla::kRow) return MLA_ERR_SHAPE;
    if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(kv_cache) || !aligned16(seqlens) || !aligned16(o) ||
        (lse && !aligned16(lse)))
        return MLA_ERR_ALIGN;
    const int cus = current_cu_count();
    if (cus <= 0) return MLA_ERR_HIP;
    const DecodeConfig c = decode_config(B, num_splits, cus);
    const mla::PlanLayout L = mla::plan_layout(B, H, c.parts, c.slots);
    if (L.total_bytes > mla::kNoAllocScratchBytes) return MLA_ERR_SCRATCH;
    void* ws = nullptr;
    if (mla::noalloc_scratch(&ws) != hipSuccess) return MLA_ERR_HIP;
    return hip_status(mla::launch_mla_decode(
        static_cast<const __bf16*>(q_lat), static_cast<const __bf16*>(q_rope), static_cast<const __bf16*>(kv_cache),
        seqlens, static_cast<__bf16*>(o), lse, B, H, S_max, scale, num_splits, L, c.c0, c.t_min, ws, stream, nullptr, 0));
}

MLA_EXPORT size_t mla_decode_v_workspace_size(int B, int H, int num_splits) {
    if (!decode_shape_ok(B, H, num_splits)) return 0;
    const int cus = current_cu_count();
    if (cus <= 0) return 0;
    const DecodeConfig c = decode_config(B, num_splits, cus, true);
    return mla::plan_layout(B, H, c.parts, c.slots).total_bytes;
}

MLA_EXPORT mla_status_t mla_decode_fwd_v(const void* q_lat, const void* q_rope, const void* kv_cache,
                                         const int* seqlens, const void* w_uv, void* o_v, float* lse, int B, int H,
                                         int S_max, int Dv, float scale, int num_splits, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
    if (!q_lat || !q_rope || !kv_cache || !seqlens || !w_uv || !o_v) return MLA_ERR_NULL;
    if (!decode_shape_ok(B, H, num_splits) || S_max < 1 || Dv < 1 || !good_scale(scale)) return MLA_ERR_SHAPE;
    if ((long long)B * S_max > (long long)INT_MAX / mla::kRow) return MLA_ERR_SHAPE;
    if (Dv % 128 != 0 || Dv > 4096) return MLA_ERR_UNSUPPORTED;
    if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(kv_cache) || !aligned16(seqlens) || !aligned16(w_uv) ||
        !aligned16(o_v) || (lse && !aligned16(lse)) || (workspace && !aligned16(workspace)))
        return MLA_ERR_ALIGN;
    if (!workspace) return MLA_ERR_WORKSPACE;
    const int cus = current_cu_count();
    if (cus <= 0) return MLA_ERR_HIP;
    const DecodeConfig c = decode_config(B, num_splits, cus, true);
    const mla::PlanLayout L = mla::plan_layout(B, H, c.parts, c.slots);
    if (workspace_bytes < L.total_bytes) return MLA_ERR_WORKSPACE;
    return hip_status(mla::launch_mla_decode(
        static_cast<const __bf16*>(q_lat), static_cast<const __bf16*>(q_rope), static_cast<const __bf16*>(kv_cache),
        seqlens, static_cast<__bf16*>(o_v), lse, B, H, S_max, scale, num_splits, L, c.c0, c.t_min, workspace, stream,
        static_cast<const __bf16*>(w_uv), Dv));
}

MLA_EXPORT mla_status_t mla_combine(const float* o_part, const float* lse_part, void* o, float* lse, int B, int H,
                                    int num_splits, hipStream_t stream) {
    if (!o_part || !lse_part || !o) return MLA_ERR_NULL;
    if (B < 1 || H < 1 || num_splits < 1 || num_splits > mla::kMaxSplits || (long long)B * H > INT_MAX)
        return MLA_ERR_SHAPE;
    if (!aligned16(o_part) || !aligned16(lse_part) || !aligned16(o) || (lse && !aligned16(lse))) return MLA_ERR_ALIGN;
    return hip_status(mla::launch_mla_combine(o_part, lse_part, static_cast<__bf16*>(o), lse, B, H, num_splits,
                                              stream));
}

// The value up-projection is the same per-head product as the absorption
// (M = B, K = Dl, N = Dv) and runs on the same kernel.
MLA_EXPORT mla_status_t mla_up_proj_v(const void* o_lat, const void* w_uv, void* o_v, int B, int H, int Dl, int Dv,
                                      hipStream_t stream) {
    if (!o_lat || !w_uv || !o_v) return MLA_ERR_NULL;
    if (B < 1 || H < 1 || Dl < 1 || Dv < 1 || (long long)B * H > INT_MAX) return MLA_ERR_SHAPE;
    if (Dl % 32 != 0 || Dl > 512 || Dv % 128 != 0 || Dv > 4096 || H > 65535) return MLA_ERR_UNSUPPORTED;
    if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(o_v)) return MLA_ERR_ALIGN;
    return hip_status(mla::launch_mla_absorb(static_cast<const __bf16*>(o_lat), static_cast<const __bf16*>(w_uv),
                                             static_cast<__bf16*>(o_v), B, H, Dl, Dv, stream));
}

MLA_EXPORT mla_status_t mla_absorb_q(const void* q_nope, const void* w_uk, void* q_lat, int B, int H, int Dn, int Dl,
                                     hipStream_t stream) {
    if (!q_nope || !w_uk || !q_lat) return MLA_ERR_NULL;
    if (B < 1 || H < 1 || Dn < 1 || Dl < 1 || (long long)B * H > INT_MAX) return MLA_ERR_SHAPE;
    if (Dn % 32 != 0 || Dn > 512 || Dl % 128 != 0 || Dl > 4096 || H > 65535) return MLA_ERR_UNSUPPORTED;
    if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_lat)) return MLA_ERR_ALIGN;
    return hip_status(mla::launch_mla_absorb(static_cast<const __bf16*>(q_nope), static_cast<const __bf16*>(w_uk),
                                             static_cast<__bf16*>(q_lat), B, H, Dn, Dl, stream));
}
