// mla_merge.h - log-sum-exp merge of split-KV partials (device code).
//
// [MLA-FA3 article], "online softmax scaling and partial reduction" stage of
// the fused dataflow: each split s of a (sequence, head) holds its output
// o_s normalised over its own token range and lse_s = log of its weight sum;
//   lse = log sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) o_s.
// Empty splits (lse_s = -inf) weigh 0; all empty -> o = 0, lse = -inf.
// Used by the combine kernels and by the fused value up-projection, so the
// merged latent row is the same, bit for bit, on every path.
#pragma once

#include "common.h"

namespace mla {

__device__ __forceinline__ void load8(const __bf16* p, float* v) {
    const bf16x8 t = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)t[i];
}
__device__ __forceinline__ void load8(const float* p, float* v) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}

// Merge of one (sequence, head) row in two passes over its splits.
// merge_row_init: M = max_s lse_s, then W = sum_s exp(lse_s - M) in split
// order, and lse = M + log W.  merge_dims8: dims 8 d8 .. 8 d8 + 7 of the
// merged row, acc = sum_s exp(lse_s - M) o_s (the same weights, same order,
// fused multiply-adds), times 1 / W, rounded to bf16.  rows(s) is the row
// index of split s in lse_part (and, times 512, in o_part).  A single split
// comes out exactly (weight exp(0) = 1).  The loads of four splits are
// issued together.
struct MergeRow {
    float M, inv_W, lse;
    bool empty;
};

template <typename RowFn>
__device__ __forceinline__ MergeRow merge_row_init(const float* lse_part, int nsplit, RowFn rows) {
    // Four loads per round trip; the sums run in split order.
    auto lse4 = [&](int s0, float (&ls)[4]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) ls[k] = s0 + k < nsplit ? lse_part[rows(s0 + k)] : -INFINITY;
    };
    float first4[4];
    lse4(0, first4);
    float M = fmaxf(-INFINITY, fmaxf(fmaxf(first4[0], first4[1]), fmaxf(first4[2], first4[3])));
    for (int s0 = 4; s0 < nsplit; s0 += 4) {
        float ls[4];
        lse4(s0, ls);
        M = fmaxf(M, fmaxf(fmaxf(ls[0], ls[1]), fmaxf(ls[2], ls[3])));
    }
    MergeRow r;
    r.M = M;
    r.empty = M == -INFINITY;
    if (r.empty) {
        r.inv_W = 0.f;
        r.lse = -INFINITY;
        return r;
    }
    float W = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)  // the first four are still in registers
        if (first4[k] != -INFINITY) W += __expf(first4[k] - M);
    for (int s0 = 4; s0 < nsplit; s0 += 4) {
        float ls[4];
        lse4(s0, ls);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (ls[k] != -INFINITY) W += __expf(ls[k] - M);
    }
    r.inv_W = 1.f / W;
    r.lse = M + __logf(W);
    return r;
}

template <typename PT, typename RowFn>
__device__ __forceinline__ bf16x8 merge_dims8(const PT* o_part, const float* lse_part, int nsplit, RowFn rows,
                                              int d8, const MergeRow& mr) {
    bf16x8 out;
    if (mr.empty) {
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = to_bf16(0.f);
        return out;
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsplit; s0 += 4) {
        float ls[4], v[4][8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            ls[k] = -INFINITY;
            if (s0 + k < nsplit) {
                const size_t r = rows(s0 + k);
                ls[k] = lse_part[r];
                load8(o_part + r * 512 + 8 * d8, v[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (ls[k] == -INFINITY) continue;  // empty split or past the end: weight 0
            const float wgt = __expf(ls[k] - mr.M);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wgt, v[k][i], acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = to_bf16(acc[i] * mr.inv_W);
    return out;
}

// The B operand of a per-head product over a merged row: cur[kk] = dims
// 32 kk + 8 g .. + 7 for kk < KS, each element exactly what merge_dims8
// returns for it (same weights, same split order, same fused multiply-adds).
// The split loop is outermost so that the KS loads of one split are issued
// together (one memory round trip per split instead of one per k-step).
template <int KS, typename RowFn>
__device__ __forceinline__ void merge_row_kk(const __bf16* o_part, const float* lse_part, int nsplit, RowFn rows,
                                             int g, const MergeRow& mr, bf16x8 (&cur)[KS]) {
    if (mr.empty) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int i = 0; i < 8; ++i) cur[kk][i] = to_bf16(0.f);
        return;
    }
    float acc[KS][8];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[kk][i] = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const size_t r = rows(s);
        const float ls = lse_part[r];
        const bf16x8* row = reinterpret_cast<const bf16x8*>(o_part + r * 512);
        bf16x8 v[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) v[kk] = row[4 * kk + g];
        if (ls == -INFINITY) continue;  // empty split: weight 0
        const float wgt = __expf(ls - mr.M);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[kk][i] = __builtin_fmaf(wgt, (float)v[kk][i], acc[kk][i]);
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) cur[kk][i] = to_bf16(acc[kk][i] * mr.inv_W);
}

}  // namespace mla
