// attn_fwd_f32.hip - fp32 fused attention forward on the vector ALUs (no MFMA).
//
// What it computes is the definition in [FA2-v2 blog] sections 1.3 and 3.3:
// O = softmax(scale Q K^T) V with an optional causal mask (section 3.4), plus
// the per-row log-sum-exp.  The structure follows the blog's v2 loop order
// (section 1.1: query tile outer, key/value tiles inner, one workgroup per
// (query tile, batch*head)) with these MI355X choices:
//   * lanes l and l + 32 of a wave share two query rows: lane l holds dims
//     0..31 and lane l + 32 dims 32..63 of both rows, for the query and for
//     the unnormalised accumulator (64 + 64 floats per lane, in VGPRs rather
//     than shared memory -- the blog's section 4.2 attributes its remaining
//     stall to the 66KB of Qs+Oacc in shared memory capping occupancy).
//     Every 16-byte K or V read from LDS then feeds 8 FMAs instead of 4: with
//     one row per lane the broadcast LDS reads, one per 4 FMAs, limited the
//     kernel as much as the FMA pipe did;
//   * one v_permlane32_swap and one add per key complete both rows' scores:
//     afterwards lane l holds the score of the first row and lane l + 32 that
//     of the second, so each lane runs the softmax of one row (one exp per
//     key and lane), and a second swap hands each lane both rows' P for the
//     value product;
//   * K/V tiles are copied global -> LDS with global_load_lds_dwordx4 (no
//     register staging) into a double buffer (the cp.async double buffer of
//     section 3.2); rows past N are clamped to row N-1 and masked to -inf;
//   * all lanes of a wave half read the same K/V address, so LDS reads are
//     broadcasts and need no padding (section 3.1 makes the same point);
//   * the score is kept in the log2 domain (scale * log2(e) folded into Q)
//     and exponentials use v_exp_f32;
//   * P is formed as exp2(s - m_new) directly, which equals the blog's
//     beta * exp(S - m~) and saves one multiply per output element;
//     a row whose scores in a tile are all masked then contributes exact
//     zeros (exp2(-inf) = 0), avoiding the NaN of exp(-inf - (-inf)).
#include "common.h"

namespace mla {

constexpr int F32_D = 64;
constexpr int F32_DH = F32_D / 2;  // dims per lane
// A workgroup is 4 waves (one per SIMD) and 256 query rows.  With 2-wave,
// 128-row workgroups the start stamps of the workgroups showed only about
// three of them resident per CU (6 of the 8 wave slots that the register
// count allows), and the non-causal kernel took 1.5x longer.
constexpr int F32_BR = 256;        // query rows per workgroup (64 per wave, two per lane pair)
constexpr int F32_BC = 32;         // keys per tile
constexpr int F32_THREADS = 256;
constexpr int F32_LOADS_PER_WAVE = (F32_BC * F32_D * 4) / (16 * 64) / (F32_THREADS / 64);  // per K (or V) tile

// v_permlane32_swap(x, y) swaps the upper 32 lanes of x with the lower 32
// lanes of y.  Afterwards lane l < 32 holds (its own x, x of lane l + 32) and
// lane l + 32 holds (y of lane l, its own y).
__device__ __forceinline__ void swap_halves(float& x, float& y) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}

template <bool CAUSAL>
__global__ __launch_bounds__(F32_THREADS, 2) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int Nq, int Nk, int BH, int num_q_tiles, float scale_log2) {
    __shared__ __attribute__((aligned(16))) float Ks[2][F32_BC * F32_D];
    __shared__ __attribute__((aligned(16))) float Vs[2][F32_BC * F32_D];

    // Work mapping: the id's low part is batch*head, so every (b,h) keeps one
    // XCD (ids are dealt round-robin over the 8 XCDs and BH is a multiple of
    // 8 in practice); causal tiles are dealt heaviest first.
    const int id = blockIdx.x;
    const int bh = id % BH;
    const int rank = id / BH;
    const int qt = CAUSAL ? (num_q_tiles - 1 - rank) : rank;
    const int q_start = qt * F32_BR;
    const size_t base = (size_t)bh * Nq * F32_D;     // Q, O
    const size_t kbase = (size_t)bh * Nk * F32_D;    // K, V
    // Causal mask aligned at the bottom right: row i sees keys <= i + off.
    const int off = Nk - Nq;

    const int w = wave_id();
    const int lane = lane_id();
    const int half = lane >> 5;  // which 32 dims this lane holds
    const int pr = lane & 31;    // lane pair
    // The pair's rows: r[0] = base row + pr, r[1] = r[0] + 32.  The lane's
    // own row (the one whose softmax it runs) is r[half].
    int rows[2], rows_c[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        rows[j] = q_start + 64 * w + 32 * j + pr;
        rows_c[j] = rows[j] < Nq ? rows[j] : (Nq - 1);
    }
    const int my_row = half ? rows[1] : rows[0];
    const int my_row_c = half ? rows_c[1] : rows_c[0];

    // Query rows into registers (this lane's 32 dims of both rows),
    // pre-scaled into the log2 domain.
    float qr[2][F32_DH];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float4* qp = reinterpret_cast<const float4*>(q + base + (size_t)rows_c[j] * F32_D + F32_DH * half);
#pragma unroll
        for (int i = 0; i < F32_DH / 4; ++i) {
            float4 t = qp[i];
            qr[j][4 * i + 0] = t.x * scale_log2;
            qr[j][4 * i + 1] = t.y * scale_log2;
            qr[j][4 * i + 2] = t.z * scale_log2;
            qr[j][4 * i + 3] = t.w * scale_log2;
        }
    }

    const int kv_limit = max(CAUSAL ? min(q_start + F32_BR + off, Nk) : Nk, 0);
    const int Tc = (kv_limit + F32_BC - 1) / F32_BC;  // 0 when no row of the tile sees a key

    // Tile loader: wave w copies chunks [w*L*64, (w+1)*L*64) of 16 bytes of
    // the K tile and of the V tile (L = loads per wave per tile).
    auto issue_tile = [&](int j, int buf) {
        const int kv_start = j * F32_BC;
#pragma unroll
        for (int i = 0; i < F32_LOADS_PER_WAVE; ++i) {
            const int chunk0 = (w * F32_LOADS_PER_WAVE + i) * 64;
            const int chunk = chunk0 + lane;
            const int r = chunk / (F32_D / 4);
            const int c4 = chunk % (F32_D / 4);
            const int key = min(kv_start + r, Nk - 1);
            const size_t goff = kbase + (size_t)key * F32_D + c4 * 4;
            gload_lds16(k + goff, &Ks[buf][chunk0 * 4]);
            gload_lds16(v + goff, &Vs[buf][chunk0 * 4]);
        }
    };

    float oacc[2][F32_DH];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int d = 0; d < F32_DH; ++d) oacc[j][d] = 0.f;
    float m = -INFINITY, l = 0.f;  // of this lane's own row

    if (Tc > 0) issue_tile(0, 0);
    for (int jt = 0; jt < Tc; ++jt) {
        const int buf = jt & 1;
        if (jt + 1 < Tc) {
            issue_tile(jt + 1, buf ^ 1);
            wait_vmcnt<2 * F32_LOADS_PER_WAVE>();
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();

        const int kv_start = jt * F32_BC;
        // This lane's 32 dims of each K / V row start at float4 8 * half.
        const float4* Kt = reinterpret_cast<const float4*>(Ks[buf]) + (F32_DH / 4) * half;
        const float4* Vt = reinterpret_cast<const float4*>(Vs[buf]) + (F32_DH / 4) * half;

        // Scores: partial dot products over this lane's dims for both rows,
        // completed by one swap and one add per key.  Afterwards s[c] is the
        // score of this lane's own row.
        float s[F32_BC];
#pragma unroll
        for (int c = 0; c < F32_BC; ++c) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int i = 0; i < F32_DH / 4; ++i) {
                const float4 kk = Kt[c * (F32_D / 4) + i];
                a0 = __builtin_fmaf(qr[0][4 * i + 0], kk.x, a0);
                a1 = __builtin_fmaf(qr[1][4 * i + 0], kk.x, a1);
                a0 = __builtin_fmaf(qr[0][4 * i + 1], kk.y, a0);
                a1 = __builtin_fmaf(qr[1][4 * i + 1], kk.y, a1);
                a0 = __builtin_fmaf(qr[0][4 * i + 2], kk.z, a0);
                a1 = __builtin_fmaf(qr[1][4 * i + 2], kk.z, a1);
                a0 = __builtin_fmaf(qr[0][4 * i + 3], kk.w, a0);
                a1 = __builtin_fmaf(qr[1][4 * i + 3], kk.w, a1);
            }
            // Lower lane: (own row-0 partial, upper's row-0 partial);
            // upper lane: (lower's row-1 partial, own row-1 partial).
            swap_halves(a0, a1);
            s[c] = a0 + a1;
        }
        // Masks: keys past N only on the last tile; causal element mask only
        // on tiles that straddle the diagonal (section 3.4).
        const bool tail = kv_start + F32_BC > Nk;
        const bool diag = CAUSAL && (kv_start + F32_BC - 1 > q_start + off);
        if (tail || diag) {
            const int lim = diag ? min(my_row_c + off + 1, Nk) : Nk;
#pragma unroll
            for (int c = 0; c < F32_BC; ++c)
                if (kv_start + c >= lim) s[c] = -INFINITY;
        }
        float mt = s[0];
#pragma unroll
        for (int c = 1; c < F32_BC; ++c) mt = fmaxf(mt, s[c]);
        const float m_new = fmaxf(m, mt);
        const float mb = (m_new == -INFINITY) ? 0.f : m_new;
        float alpha0 = fast_exp2(m - mb), alpha1 = alpha0;
        float ls = 0.f;
#pragma unroll
        for (int c = 0; c < F32_BC; ++c) {
            s[c] = fast_exp2(s[c] - mb);
            ls += s[c];
        }
        l = l * alpha0 + ls;
        m = m_new;
        // Both rows' rescale factors in every lane: (row 0, row 1).
        swap_halves(alpha0, alpha1);
#pragma unroll
        for (int d = 0; d < F32_DH; ++d) {
            oacc[0][d] *= alpha0;
            oacc[1][d] *= alpha1;
        }
#pragma unroll
        for (int c = 0; c < F32_BC; ++c) {
            float p0 = s[c], p1 = s[c];
            swap_halves(p0, p1);  // (row 0, row 1) in every lane
#pragma unroll
            for (int i = 0; i < F32_DH / 4; ++i) {
                const float4 vv = Vt[c * (F32_D / 4) + i];
                oacc[0][4 * i + 0] = __builtin_fmaf(p0, vv.x, oacc[0][4 * i + 0]);
                oacc[1][4 * i + 0] = __builtin_fmaf(p1, vv.x, oacc[1][4 * i + 0]);
                oacc[0][4 * i + 1] = __builtin_fmaf(p0, vv.y, oacc[0][4 * i + 1]);
                oacc[1][4 * i + 1] = __builtin_fmaf(p1, vv.y, oacc[1][4 * i + 1]);
                oacc[0][4 * i + 2] = __builtin_fmaf(p0, vv.z, oacc[0][4 * i + 2]);
                oacc[1][4 * i + 2] = __builtin_fmaf(p1, vv.z, oacc[1][4 * i + 2]);
                oacc[0][4 * i + 3] = __builtin_fmaf(p0, vv.w, oacc[0][4 * i + 3]);
                oacc[1][4 * i + 3] = __builtin_fmaf(p1, vv.w, oacc[1][4 * i + 3]);
            }
        }
        lds_barrier();
    }

    // A row that saw no key (l = 0, only with Nq > Nk) gets O = 0, LSE = -inf.
    const float inv_own = l > 0.f ? 1.f / l : 0.f;
    float inv0 = inv_own, inv1 = inv_own;
    swap_halves(inv0, inv1);  // (row 0, row 1) in every lane
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (rows[j] < Nq) {
            const float inv = j ? inv1 : inv0;
            float4* op = reinterpret_cast<float4*>(o + base + (size_t)rows[j] * F32_D + F32_DH * half);
#pragma unroll
            for (int i = 0; i < F32_DH / 4; ++i)
                op[i] = make_float4(oacc[j][4 * i] * inv, oacc[j][4 * i + 1] * inv, oacc[j][4 * i + 2] * inv,
                                    oacc[j][4 * i + 3] * inv);
        }
    }
    if (lse && my_row < Nq) lse[(size_t)bh * Nq + my_row] = l > 0.f ? (m + __builtin_log2f(l)) * kLn2 : -INFINITY;
}

// Host-side launcher (called by the C ABI after validation).
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                               int B, int H, int Nq, int Nk, float scale, bool causal, hipStream_t stream) {
    const int BH = B * H;
    const int nqt = (Nq + F32_BR - 1) / F32_BR;
    const long long grid = (long long)nqt * BH;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float sl2 = scale * kLog2e;
    if (causal)
        hipLaunchKernelGGL(attn_fwd_f32_kernel<true>, dim3((unsigned)grid), dim3(F32_THREADS), 0, stream,
                           q, k, v, o, lse, Nq, Nk, BH, nqt, sl2);
    else
        hipLaunchKernelGGL(attn_fwd_f32_kernel<false>, dim3((unsigned)grid), dim3(F32_THREADS), 0, stream,
                           q, k, v, o, lse, Nq, Nk, BH, nqt, sl2);
    return hipGetLastError();
}

}  // namespace mla
