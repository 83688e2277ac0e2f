// attn_fwd_bf16.hip - bf16 fused attention forward on the matrix cores.
//
// Computes O = softmax(scale Q K^T) V (optional causal mask) and the per-row
// log-sum-exp, [FA2-v2 blog] sections 1.1-3.5, with bf16 inputs, fp32
// accumulation and a bf16 output.  The blog stops at CUDA cores and names
// tensor-core MMA as its next step (sections 1.3 and 5); this is that step
// written for CDNA4 matrix cores.
//
// Tiling (D = 128): a workgroup owns Br = 128 query rows of one (b, h);
// wave w owns rows 32w..32w+31.  Key/value tiles of Bc = 64 rows are copied
// global -> LDS (buffer_load_dwordx4 ... lds) into a double buffer, with the
// 16-byte chunks of each row permuted so that every LDS read is free of
// bank conflicts.  Each
// wave's per-lane source offsets within a tile are fixed; a tile only moves
// the buffer base, and the buffer ends at key N - 1, so keys past N read as
// zeros (and are masked).  LDS fragments are read with inline asm and waited
// for with counted waits, so the next tile's copies stay in flight while the
// current tile is computed.
//
// Products per wave and 64-key tile (v_mfma_f32_32x32x16_bf16):
//   S^T = K Q^T  : A = K rows from LDS, B = Q held in VGPRs.  The result
//                  puts one query per lane column, so a query's row max and
//                  sum need one exchange (lanes l and l^32).
//   O^T += V^T P^T: A = V^T read with ds_read_b64_tr_b16 straight from the
//                  row-major V tile; B = P^T, which is the S^T accumulator
//                  rounded to bf16 with no data movement (see the key
//                  permutation below).
// Softmax runs in the log2 domain: p = exp2(s*c - m) with c = scale*log2(e).
// The accumulator is rescaled only when some row max of the wave exceeds the
// current exponent base by more than kRescaleSlack.
// Masks follow section 3.4: tiles past the causal limit are never loaded;
// the element mask is applied only on tiles that straddle the diagonal; keys
// past N read as zeros and are masked.
#include "common.h"

namespace mla {

constexpr int B16_D = 128;
constexpr int B16_BR = 128;
constexpr int B16_BC = 64;
constexpr int B16_WAVES = 4;
constexpr int B16_THREADS = 64 * B16_WAVES;
constexpr int B16_ROW_CHUNKS = B16_D * 2 / 16;                       // 16 chunks of 16 B per row
constexpr int B16_STRIDE = B16_ROW_CHUNKS * 16;                      // 256 B per LDS row, chunks swizzled
constexpr int B16_TILE_BYTES = B16_BC * B16_STRIDE;                  // 16384
constexpr int B16_TILE_INSTR = B16_BC * B16_ROW_CHUNKS / 64;         // 16 wave-wide 1 KiB copies per tile
static_assert(B16_TILE_INSTR % B16_WAVES == 0, "copies split evenly over the waves");
constexpr int B16_COPIES = B16_TILE_INSTR / B16_WAVES;  // copies per tile and wave, K and V each
constexpr int B16_LOADS = 2 * B16_COPIES;               // K + V copies per tile and wave
// LDS fragment prefetch distances (MFMA steps) of the score and PV loops.
#ifndef MLA_B16_PF
#define MLA_B16_PF 2
#endif
#ifndef MLA_B16_PFV
#define MLA_B16_PFV 3
#endif
constexpr int B16_PF = MLA_B16_PF;
constexpr int B16_PFV = MLA_B16_PFV;

// Inside each 32-key block MFMA row rho = 16a + 8b + 4g + c is fed key
// 16a + 8b + g + 2c, so that register e of lane group g of S^T holds key
// 16(e/8) + 8((e/4)%2) + g + 2(e%4), i.e. the eight registers of k-step e/8
// are P^T with logical k index 8g + e%8 (no data movement between the two
// products).
__device__ __forceinline__ int b16_kappa32(int rho) { return (rho & ~7) + ((rho >> 2) & 1) + 2 * (rho & 3); }
__device__ __forceinline__ int b16_key_of_reg(int e, int g) {
    return 16 * (e >> 3) + 8 * ((e >> 2) & 1) + g + 2 * (e & 3);
}
// LDS tiles have 256-byte rows; 16-byte chunk c of row r is stored at chunk
// position c ^ swz(r).  With 64 four-byte banks, ds_read_b128 serves 16 lanes
// and ds_read_b64_tr_b16 32 lanes per pass.  The K swizzle puts the 16 rows
// one 16-lane group reads on 16 distinct chunk positions; the V swizzle moves
// rows 2jj, 2jj + 1 by 64 jj bytes, so the 32 lanes of one pass of a
// transposed read (rows 2jj + {0,1}, one 64-byte column group) hit 64
// distinct banks.  Both depend on r mod 16, so row offsets that are
// multiples of 16 (and 8, for V) stay immediates.
__device__ __forceinline__ int b16_kswz(int r) { return r & 15; }
__device__ __forceinline__ int b16_vswz(int r) { return 4 * ((r >> 1) & 3); }

template <bool CAUSAL>
__global__ __launch_bounds__(B16_THREADS, 2) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int Nq, int Nk, int BH, int num_q_tiles, float c_log2) {
    __shared__ __attribute__((aligned(1024))) char smem[2][2][B16_TILE_BYTES];  // [buf][K|V]

    // Work mapping: the id's low part is batch*head, so every (b,h) stays on
    // one XCD (ids are dealt round-robin over the XCDs); causal tiles are
    // dealt heaviest first.
    const int id = blockIdx.x;
    const int bh = id % BH;
    const int rank = id / BH;
    const int qt = CAUSAL ? (num_q_tiles - 1 - rank) : rank;
    const int q_start = qt * B16_BR;
    const size_t base = (size_t)bh * Nq * B16_D;     // Q, O
    const size_t kbase = (size_t)bh * Nk * B16_D;    // K, V
    // Causal mask aligned at the bottom right: row i sees keys <= i + off.
    const int off = Nk - Nq;

    const int w = wave_id();
    const int lane = lane_id();
    const int n = lane & 31;  // query column of the MFMA results
    const int g = lane >> 5;  // row group
    const int wrow0 = q_start + 32 * w;

    // Q as the B operand of S^T = K Q^T: lane holds row wrow0+n, dims 16kk+8g..+7.
    bf16x8 qf[B16_D / 16];
    {
        const int r = min(wrow0 + n, Nq - 1);
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(q + base + (size_t)r * B16_D);
#pragma unroll
        for (int kk = 0; kk < B16_D / 16; ++kk) qf[kk] = qp[2 * kk + g];
    }

    const int kv_limit = max(CAUSAL ? min(q_start + B16_BR + off, Nk) : Nk, 0);
    const int Tc = (kv_limit + B16_BC - 1) / B16_BC;
    if (Tc == 0) {  // no row of this tile sees a key (Nq > Nk): O = 0, LSE = -inf
        const int row = wrow0 + n;
        if (row < Nq) {
            __bf16* op = o + base + (size_t)row * B16_D;
            bf16x4 z;
#pragma unroll
            for (int r = 0; r < 4; ++r) z[r] = to_bf16(0.f);
#pragma unroll
            for (int c = 0; c < B16_D / 8; ++c) *reinterpret_cast<bf16x4*>(op + 8 * c + 4 * g) = z;
            if (lse && g == 0) lse[(size_t)bh * Nq + row] = -INFINITY;
        }
        return;
    }

    // Copy i (0..15) of 64 chunks of the K and of the V tile is issued by wave
    // i % 4.  LDS chunk position L is row L / 16, position L % 16, which holds
    // source chunk (L % 16) ^ swz(row); copy kc of this wave has the fixed
    // per-lane source offsets koff[kc] (K) and voff[kc] (V) within a tile.
    uint32_t koff[B16_COPIES], voff[B16_COPIES];
#pragma unroll
    for (int kc = 0; kc < B16_COPIES; ++kc) {
        const int L = (w + B16_WAVES * kc) * 64 + lane;  // LDS chunk position of this lane
        const int r = L / B16_ROW_CHUNKS, p = L % B16_ROW_CHUNKS;
        koff[kc] = (uint32_t)(r * B16_D * 2 + 16 * (p ^ b16_kswz(r)));
        voff[kc] = (uint32_t)(r * B16_D * 2 + 16 * (p ^ b16_vswz(r)));
    }
    // Buffers of tile j's K and V rows.  A tile past the last one gets empty
    // buffers: its copies write zeros into the free LDS slot and need no
    // branch.
    auto tile_rsrc = [&](int j, __amdgpu_buffer_rsrc_t& rk, __amdgpu_buffer_rsrc_t& rv) {
        const int kv_start = j < Tc ? j * B16_BC : 0;
        const uint32_t bytes = j < Tc ? (uint32_t)(Nk - kv_start) * (uint32_t)(B16_D * 2) : 0u;
        rk = make_rsrc(k + kbase + (size_t)kv_start * B16_D, bytes);
        rv = make_rsrc(v + kbase + (size_t)kv_start * B16_D, bytes);
    };
    // Copy c (0..B16_LOADS-1) of this wave for one tile: even c copy K chunk
    // block c/2, odd c the V block.
    auto issue_copy = [&](auto c_c, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int buf) {
        constexpr int c = decltype(c_c)::value, kc = c / 2;
        if constexpr (c % 2 == 0) bload_lds16(rk, &smem[buf][0][(w + B16_WAVES * kc) * 1024], koff[kc]);
        else bload_lds16(rv, &smem[buf][1][(w + B16_WAVES * kc) * 1024], voff[kc]);
    };

    f32x16 oacc[B16_D / 32];
#pragma unroll
    for (int db = 0; db < B16_D / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    float m = -INFINITY;  // running max, already scaled into the log2 domain
    float l = 0.f;        // this lane's share of the running sum

    // Per-lane LDS byte offsets (all other offsets are immediates).
    // K: row kappa(n), chunk 2kk + g (one base per score k-step kk).
    // V: row (G >> 1) + 2jj, chunk 4db + 2(G & 1) + qd / 2 (one base per dim block db).
    constexpr int KS = B16_D / 16;  // score k-steps
    const int G = lane >> 4, sl = lane & 15;  // ds_read_b64_tr_b16 source lane = 4*jj + qd
    const int jj = sl >> 2, qd = sl & 3;
    uint32_t k_off[KS], v_off[4];
    {
        const int kr = b16_kappa32(n), vr = (G >> 1) + 2 * jj;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) k_off[kk] = kr * B16_STRIDE + 16 * ((2 * kk + g) ^ b16_kswz(kr));
#pragma unroll
        for (int db = 0; db < 4; ++db)
            v_off[db] = vr * B16_STRIDE + 16 * ((4 * db + 2 * (G & 1) + (qd >> 1)) ^ b16_vswz(vr)) + 8 * (qd & 1);
    }
    const uint32_t smem_a = lds_addr(&smem[0][0][0]);
    constexpr int PS = 16;          // PV steps: (ks, db) = (step / 4, step % 4)

    {
        __amdgpu_buffer_rsrc_t rk, rv;
        tile_rsrc(0, rk, rv);
        static_for<B16_LOADS>([&](auto c) { issue_copy(c, rk, rv, 0); });
    }
    // Tile j + 1 is copied during the score products of tile j, one copy per
    // k-step, into the buffer that tile j - 1 used (free since the barrier
    // that ended step j - 1).  At the top of step j every copy of this wave
    // (tile j's, and the Q loads before the first) has landed.
    for (int j = 0; j < Tc; ++j) {
        const int buf = j & 1;
        wait_vmcnt<0>();
        lds_barrier();
        __amdgpu_buffer_rsrc_t nrk, nrv;
        tile_rsrc(j + 1, nrk, nrv);

        const int kv_start = j * B16_BC;
        // A tile entirely above this wave's rows (causal) is computed anyway:
        // its scores are all masked, so it adds nothing, and the uniform
        // control flow keeps the accumulators in place (a per-wave skip here
        // makes the compiler copy them on every tile).
        {
            const uint32_t Kt = smem_a + buf * 2 * B16_TILE_BYTES;
            const uint32_t Vt = smem_a + (buf * 2 + 1) * B16_TILE_BYTES;
            // Score fragments: ring of B16_PF + 1 pairs (keys 0..31 and 32..63).
            bf16x8 fa[B16_PF + 1], fb[B16_PF + 1];
            auto rd_k = [&](auto kk_c) {
                constexpr int kk = decltype(kk_c)::value;
                fa[kk % (B16_PF + 1)] = ds_read16<0>(Kt + k_off[kk]);
                fb[kk % (B16_PF + 1)] = ds_read16<32 * B16_STRIDE>(Kt + k_off[kk]);
            };
            f32x16 s0, s1;
#pragma unroll
            for (int e = 0; e < 16; ++e) { s0[e] = 0.f; s1[e] = 0.f; }
            static_for<B16_PF>([&](auto i) { rd_k(i); });
            // The two waves of a SIMD alternate between MFMA phases and the
            // softmax; the wave in an MFMA phase gets issue priority, so the
            // matrix pipe is fed first and the other wave's VALU work fills
            // the gaps.
            __builtin_amdgcn_s_setprio(2);
            static_assert(KS == B16_LOADS, "one tile copy per score k-step");
            static_for<KS>([&](auto kk_c) {
                constexpr int kk = decltype(kk_c)::value;
                if constexpr (kk + B16_PF < KS) rd_k(std::integral_constant<int, kk + B16_PF>{});
                constexpr int newer = 2 * ((KS - 1 - kk) < B16_PF ? (KS - 1 - kk) : B16_PF);
                wait_lgkm_for<newer>(fa[kk % (B16_PF + 1)], fb[kk % (B16_PF + 1)]);
                __builtin_amdgcn_sched_barrier(0);
                s0 = mfma32(fa[kk % (B16_PF + 1)], qf[kk], s0);
                issue_copy(kk_c, nrk, nrv, buf ^ 1);
                s1 = mfma32(fb[kk % (B16_PF + 1)], qf[kk], s1);
                __builtin_amdgcn_sched_barrier(0);
            });
            __builtin_amdgcn_s_setprio(0);
            // The first V^T fragments are requested before the softmax so that
            // its arithmetic covers their latency.
            bf16x8 fv[B16_PFV + 1];
            auto rd_v = [&](auto st_c) {
                constexpr int st = decltype(st_c)::value;
                constexpr int ks = st / 4, db = st % 4;
                fv[st % (B16_PFV + 1)] = join(ds_read_tr16<16 * ks * B16_STRIDE>(Vt + v_off[db]),
                                              ds_read_tr16<(16 * ks + 8) * B16_STRIDE>(Vt + v_off[db]));
            };
            static_for<B16_PFV>([&](auto i) { rd_v(i); });
            // Tile max on the raw MFMA results (in the same block as the MFMAs,
            // so the compiler knows them canonical and emits bare v_max3);
            // only masked tiles recompute it after masking.
            // (A sequential chain compiles to bare v_max3; nesting the pairwise
            // max makes the compiler canonicalize every input first.)
            float mt = s0[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) mt = fmaxf(mt, s0[e]);
#pragma unroll
            for (int e = 0; e < 16; ++e) mt = fmaxf(mt, s1[e]);
            const bool tail = kv_start + B16_BC > Nk;
            const bool diag = CAUSAL && (kv_start + B16_BC - 1 > wrow0 + off);
            if (tail || diag) {
                const int row = wrow0 + n;
                const int lim = diag ? min(row + off + 1, Nk) : Nk;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = kv_start + b16_key_of_reg(e, g);
                    if (key >= lim) s0[e] = -INFINITY;
                    if (key + 32 >= lim) s1[e] = -INFINITY;
                }
                float mm = s0[0];
#pragma unroll
                for (int e = 1; e < 16; ++e) mm = fmaxf(mm, s0[e]);
#pragma unroll
                for (int e = 0; e < 16; ++e) mm = fmaxf(mm, s1[e]);
                mt = fminf(mt, mm);  // == mm; keeps the raw max in the MFMA block
            }
            mt = max2_halves(mt) * c_log2;
            // P = exp2(s c - base) in bf16 and this lane's row-sum share, then
            // O^T += V^T P^T.  Written once per branch of the lazy rescale so
            // that the common (no-rescale) path keeps the accumulators in place.
            auto softmax_pv = [&]() {
                const float mb = (m == -INFINITY) ? 0.f : m;
                bf16x8 pb[4];  // k-step ks (keys 16ks..16ks+15 of the tile)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float p0 = fast_exp2(__builtin_fmaf(s0[e], c_log2, -mb));
                    const float p1 = fast_exp2(__builtin_fmaf(s1[e], c_log2, -mb));
                    l += p0 + p1;
                    pb[(e >> 3)][e & 7] = to_bf16(p0);
                    pb[2 + (e >> 3)][e & 7] = to_bf16(p1);
                }
                __builtin_amdgcn_s_setprio(2);
                static_for<PS>([&](auto st_c) {
                    constexpr int st = decltype(st_c)::value;
                    constexpr int ks = st / 4, db = st % 4;
                    if constexpr (st + B16_PFV < PS) rd_v(std::integral_constant<int, st + B16_PFV>{});
                    constexpr int newer = 2 * ((PS - 1 - st) < B16_PFV ? (PS - 1 - st) : B16_PFV);
                    wait_lgkm_for<newer>(fv[st % (B16_PFV + 1)]);
                    __builtin_amdgcn_sched_barrier(0);
                    oacc[db] = mfma32(fv[st % (B16_PFV + 1)], pb[ks], oacc[db]);
                    __builtin_amdgcn_sched_barrier(0);
                });
                __builtin_amdgcn_s_setprio(0);
            };
            // Lazy rescale (see kRescaleSlack): the base moves only when a
            // row max exceeds it by more than the slack.
            if (__builtin_amdgcn_ballot_w64(mt > m + kRescaleSlack) != 0) {
                const float m_new = fmaxf(m, mt);
                const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - m_new);
                l *= alpha;
                // In-place multiplies (each asm output tied to its input), so
                // the accumulators keep their registers across this rare branch
                // and the common path needs no copies.  The next reads of these
                // registers are the PV MFMAs after the whole softmax.
#pragma unroll
                for (int db = 0; db < B16_D / 32; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) asm("v_mul_f32_e32 %0, %1, %0" : "+v"(oacc[db][e]) : "v"(alpha));
                m = m_new;
            }
            softmax_pv();
        }
        lds_barrier();
    }
    // The last step's (empty) copies must land before the workgroup's LDS is
    // released.
    wait_vmcnt<0>();

    // Epilogue: O = Oacc / l; O^T register e of block db: dim 32db + 8(e/4) + 4g + e%4.
    // The rows go through LDS (the K/V buffers, free once every wave's last
    // copies have landed) so that each store writes four whole 256-byte rows.
    lds_barrier();
    l = sum2_halves(l);
    const int row = wrow0 + n;
    // A row that saw no key (l = 0, only with Nq > Nk) gets O = 0, LSE = -inf.
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    constexpr int STG = 272;  // staging row stride (bytes): 256 + 16 against bank conflicts
    char* stg = &smem[0][0][0] + w * 32 * STG;
#pragma unroll
    for (int db = 0; db < B16_D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x4 t;
#pragma unroll
            for (int r = 0; r < 4; ++r) t[r] = to_bf16(oacc[db][4 * i + r] * inv_l);
            *reinterpret_cast<bf16x4*>(stg + n * STG + 2 * (32 * db + 8 * i + 4 * g)) = t;
        }
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0): the wave's rows are in LDS
#pragma unroll
    for (int k8 = 0; k8 < 8; ++k8) {
        const int r = 4 * k8 + (lane >> 4), c = lane & 15;
        const bf16x8 vrow = *reinterpret_cast<const bf16x8*>(stg + r * STG + 16 * c);
        if (wrow0 + r < Nq) *reinterpret_cast<bf16x8*>(o + base + (size_t)(wrow0 + r) * B16_D + 8 * c) = vrow;
    }
    if (lse && g == 0 && row < Nq) lse[(size_t)bh * Nq + row] = l > 0.f ? (m + __builtin_log2f(l)) * kLn2 : -INFINITY;
}

hipError_t launch_attn_fwd_bf16(const __bf16* q, const __bf16* k, const __bf16* v, __bf16* o, float* lse,
                                int B, int H, int Nq, int Nk, float scale, bool causal, hipStream_t stream) {
    const int BH = B * H;
    const int nqt = (Nq + B16_BR - 1) / B16_BR;
    const long long grid = (long long)nqt * BH;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float c = scale * kLog2e;
    if (causal)
        hipLaunchKernelGGL(attn_fwd_bf16_kernel<true>, dim3((unsigned)grid), dim3(B16_THREADS), 0, stream,
                           q, k, v, o, lse, Nq, Nk, BH, nqt, c);
    else
        hipLaunchKernelGGL(attn_fwd_bf16_kernel<false>, dim3((unsigned)grid), dim3(B16_THREADS), 0, stream,
                           q, k, v, o, lse, Nq, Nk, BH, nqt, c);
    return hipGetLastError();
}

}  // namespace mla
