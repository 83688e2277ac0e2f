// mla_absorb.hip - weight-absorption prologue q_lat = q_nope W_UK (gfx950).
//
// [MLA-FA3 article] section 2: the key up-projection W_UK is absorbed into
// the query, so the score against the cache needs (q W_UK) once per query
// instead of W_UK c once per cached token.  This kernel forms
//   q_lat[b, h, :] = q_nope[b, h, :] @ W_UK[h]     (fp32 accumulation, bf16 out)
// for all b, h.  It is a per-head batched product (M = B, N = Dl, K = Dn);
// at the decode shapes it moves ~59 MB for ~4 GFLOP, so it is bound by
// memory, and the design only has to read W_UK once and stream q_nope.
//
// A workgroup owns (head h, 128 latent columns): it copies that
// [Dn x 128] slab of W_UK into LDS once, then walks all b in blocks of 64
// (16 per wave).  The product is taken transposed, q_lat^T = W^T q_nope^T
// (v_mfma_f32_16x16x32_bf16): A = W^T fragments read with ds_read_b64_tr_b16
// from the row-major slab, B = q_nope rows read straight from global memory
// (16 contiguous bytes per lane), so each lane ends with 4 consecutive
// latent columns of one row.  A wave's 16 x 128 output block goes through
// LDS so that each store instruction writes four whole 256-byte rows: the
// kernel is bound by its 34 MB of output writes, and 32-byte store segments
// (16 per instruction) cost ~13% more time than whole rows.
//
// The Dl / 128 workgroups of one head read the same q_nope rows.  Work is
// dealt to the 8 XCDs round-robin in dispatch order, so the block index is
// mapped such that a head's column blocks are dispatched to one XCD, one
// after another: the rows then come from that XCD's L2 after the first
// read.  When (head, column block) pairs alone would leave CUs idle (the
// value up-projection has one 128-column block per head), the rows are
// split into blocks as well.  For Dn = 128 and 512 the q_nope rows of the
// next 64-row block are loaded while the current block's MFMAs run.
#include "common.h"
#include "mla_merge.h"

namespace mla {

constexpr int ABS_THREADS = 256;
constexpr int ABS_COLS = 128;

__device__ __forceinline__ int abs_swz(int r) { return (r & 7) << 1; }

// Block index -> (head, column block, row block).  With H % 8 == 0, XCD x
// (= L % 8) receives heads x, x + 8, ..., each head's blocks consecutively.
__device__ __forceinline__ void abs_block(int L, int H, int nc, int nb, int& h, int& cb, int& rb) {
    const int units = nc * nb;
    int k;
    if ((H & 7) == 0) {
        const int x = L & 7;
        k = L >> 3;
        h = x + 8 * (k / units);
    } else {
        h = L / units;
        k = L;
    }
    const int rem = k - (k / units) * units;
    cb = rem % nc;
    rb = rem / nc;
}

// W_UK[h][:, col0:col0+128] -> LDS, chunk p of row r stored at p ^ abs_swz(r).
__device__ __forceinline__ void abs_load_w(const __bf16* w_uk, char* smem, int h, int col0, int Dn, int Dl, int w,
                                           int lane) {
    const __bf16* src = w_uk + (size_t)h * Dn * Dl + col0;
    const int chunks = Dn * 16;
    for (int c0 = w * 64; c0 < chunks; c0 += 4 * 64) {
        const int L = c0 + lane;
        const int r = L >> 4, p = L & 15;
        gload_lds16(src + (size_t)r * Dl + 8 * (p ^ abs_swz(r)), smem + c0 * 16);
    }
}

// acc[db] += W^T[cols 16db.., k-step kk] q^T for one k-step.
__device__ __forceinline__ void abs_kstep(const char* smem, int kk, int g, int jj, int qd, const bf16x8& bq,
                                          f32x4 (&acc)[ABS_COLS / 16]) {
    const int r_lo = 32 * kk + 8 * g + jj, r_hi = r_lo + 4;
#pragma unroll
    for (int db = 0; db < ABS_COLS / 16; ++db) {
        const int ch = 2 * db + (qd >> 1), half = (qd & 1) * 8;
        bf16x4 lo = lds_read_tr16(smem, r_lo * 256 + ((ch ^ abs_swz(r_lo)) << 4) + half);
        bf16x4 hi = lds_read_tr16(smem, r_hi * 256 + ((ch ^ abs_swz(r_hi)) << 4) + half);
        acc[db] = mfma16(join(lo, hi), bq, acc[db]);
    }
}

__device__ __forceinline__ void abs_store(__bf16* q_lat, const f32x4 (&acc)[ABS_COLS / 16], int b, int B, int H,
                                          int h, int Dl, int col0, int g) {
    if (b < B) {
        __bf16* out = q_lat + ((size_t)b * H + h) * Dl + col0;
#pragma unroll
        for (int db = 0; db < ABS_COLS / 16; ++db) {
            bf16x4 t;
#pragma unroll
            for (int r = 0; r < 4; ++r) t[r] = to_bf16(acc[db][r]);
            *reinterpret_cast<bf16x4*>(out + 16 * db + 4 * g) = t;
        }
    }
}

// Stores a wave's 16 rows x 128 columns through LDS (272-byte rows), so that
// each global store instruction writes four whole 256-byte rows.
constexpr int ABS_STG_STRIDE = 272;
constexpr int ABS_STG_BYTES = 16 * ABS_STG_STRIDE;  // per wave
__device__ __forceinline__ void abs_store_staged(__bf16* q_lat, const f32x4 (&acc)[ABS_COLS / 16], int b0, int B,
                                                 int H, int h, int Dl, int col0, char* stg, int n, int g, int lane) {
#pragma unroll
    for (int db = 0; db < ABS_COLS / 16; ++db) {
        bf16x4 t;
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = to_bf16(acc[db][r]);
        *reinterpret_cast<bf16x4*>(stg + n * ABS_STG_STRIDE + 32 * db + 8 * g) = t;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0): the wave's LDS writes landed
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = 4 * k + (lane >> 4), c = lane & 15;
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(stg + r * ABS_STG_STRIDE + 16 * c);
        const int b = b0 + r;
        if (b < B) *reinterpret_cast<bf16x8*>(q_lat + ((size_t)b * H + h) * Dl + col0 + 8 * c) = v;
    }
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // reads done before the next block's writes
    __builtin_amdgcn_wave_barrier();
}

// KS > 0: Dn = 32 KS, and each row block's q_nope rows are loaded while the
// previous block's MFMAs run.  KS == 0: any Dn, rows loaded per k-step.
// (A 512-row slab fills 128 KiB of LDS: one workgroup per CU, so that
// instance may use the whole register file.)
template <int KS>
__global__ __launch_bounds__(ABS_THREADS, KS == 16 ? 1 : 2) void mla_absorb_kernel(const __bf16* __restrict__ q_nope,
                                                                   const __bf16* __restrict__ w_uk,
                                                                   __bf16* __restrict__ q_lat, int B, int H,
                                                                   int Dn, int Dl, int rows) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];  // [Dn][128] bf16, 256-byte rows
    const int nb = (B + rows - 1) / rows;
    int h, cb, rb;
    abs_block(blockIdx.x, H, Dl / ABS_COLS, nb, h, cb, rb);
    const int col0 = cb * ABS_COLS;
    const int b_lo = rb * rows, b_hi = min(B, b_lo + rows);
    const int w = wave_id();
    const int lane = lane_id();
    const int n = lane & 15, g = lane >> 4;
    const int jj = n >> 2, qd = n & 3;
    auto qrow = [&](int bb) {
        const int bl = min(bb + 16 * w + n, B - 1);
        return reinterpret_cast<const bf16x8*>(q_nope + ((size_t)bl * H + h) * Dn);
    };

    abs_load_w(w_uk, smem, h, col0, Dn, Dl, w, lane);
    if constexpr (KS > 0) {
        bf16x8 cur[KS];
        {
            const bf16x8* q = qrow(b_lo);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) cur[kk] = q[4 * kk + g];
        }
        wait_vmcnt<0>();
        __syncthreads();
        for (int bb = b_lo; bb < b_hi; bb += 64) {
            bf16x8 nxt[KS];
            if (bb + 64 < b_hi) {
                const bf16x8* q = qrow(bb + 64);
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) nxt[kk] = q[4 * kk + g];
            }
            f32x4 acc[ABS_COLS / 16];
#pragma unroll
            for (int db = 0; db < ABS_COLS / 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) abs_kstep(smem, kk, g, jj, qd, cur[kk], acc);
            abs_store_staged(q_lat, acc, bb + 16 * w, b_hi, H, h, Dl, col0, smem + Dn * 256 + w * ABS_STG_BYTES, n, g,
                             lane);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) cur[kk] = nxt[kk];
        }
    } else {
        wait_vmcnt<0>();
        __syncthreads();
        for (int bb = b_lo; bb < b_hi; bb += 64) {
            const bf16x8* q = qrow(bb);
            f32x4 acc[ABS_COLS / 16];
#pragma unroll
            for (int db = 0; db < ABS_COLS / 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int kk = 0; kk < Dn / 32; ++kk) abs_kstep(smem, kk, g, jj, qd, q[4 * kk + g], acc);
            abs_store(q_lat, acc, bb + 16 * w + n, b_hi, H, h, Dl, col0, g);
        }
    }
}

// ---------------------------------------------------------------------------
// Merge of the split decode fused with the value up-projection.
//
// [MLA-FA3 article] fused dataflow figure: the value up-projection W_UV
// belongs to the same in-place stage as W_UK, after the online-softmax
// partial reduction.  Attention is linear in its values, so
//   o_v[b, h, :] = o[b, h, :] W_UV[h],  o = the merged latent output.
// The split kernel (value mode) leaves every piece of sequence b -- one for
// an unsplit sequence -- as a bf16 partial in slot b + p (p = its part).
// This kernel is the absorption kernel's per-head product with its B operand
// built on the fly: each lane merges its row's partials in fp32 for the 8
// latent dims it feeds (merge_row_init / merge_dims8, the same arithmetic as
// the combine kernel), rounds them to bf16, and multiplies by the W_UV slab
// held in LDS.  The merged latent row never goes to memory; the merged LSE
// is written once per (b, h).
// ---------------------------------------------------------------------------
template <int KS>
__global__ __launch_bounds__(ABS_THREADS, 1) void mla_merge_up_kernel(
    const int* __restrict__ ws, int seq_first, int seq_nsplit, const __bf16* __restrict__ o_part,
    const float* __restrict__ lse_part, const __bf16* __restrict__ w_uv, __bf16* __restrict__ o_v,
    float* __restrict__ lse, int B, int H, int Dv, int rows) {
    constexpr int Dl = 32 * KS;
    extern __shared__ __attribute__((aligned(1024))) char smem[];  // [Dl][128] bf16, 256-byte rows, then staging
    const int nb = (B + rows - 1) / rows;
    int h, cb, rb;
    abs_block(blockIdx.x, H, Dv / ABS_COLS, nb, h, cb, rb);
    const int col0 = cb * ABS_COLS;
    const int b_lo = rb * rows, b_hi = min(B, b_lo + rows);
    const int w = wave_id();
    const int lane = lane_id();
    const int n = lane & 15, g = lane >> 4;
    const int jj = n >> 2, qd = n & 3;

    // The slab's copies are issued first and land while the first row block
    // is merged; the next block's plan entries are read one block ahead.
    abs_load_w(w_uv, smem, h, col0, Dl, Dv, w, lane);
    auto entries = [&](int bb, int& b, int& first, int& ns) {
        b = min(bb + 16 * w + n, B - 1);
        first = ws[seq_first + b];
        ns = ws[seq_nsplit + b];
    };
    int nb_b, nb_first, nb_ns;
    entries(b_lo, nb_b, nb_first, nb_ns);
    bool slab_ready = false;
    for (int bb = b_lo; bb < b_hi; bb += 64) {
        const int row = bb + 16 * w + n;
        const int b = nb_b, first = nb_first, ns = nb_ns;
        if (bb + 64 < b_hi) entries(bb + 64, nb_b, nb_first, nb_ns);
        auto rows_fn = [&](int s) -> size_t { return (size_t)(b + first + s) * H + h; };
        const MergeRow mr = merge_row_init(lse_part, ns, rows_fn);
        bf16x8 cur[KS];
        merge_row_kk<KS>(o_part, lse_part, ns, rows_fn, g, mr, cur);
        if (!slab_ready) {  // the merge's loads were waited for, and with them the earlier slab copies
            wait_vmcnt<0>();
            __syncthreads();
            slab_ready = true;
        }
        if (lse && cb == 0 && g == 0 && row < b_hi) lse[(size_t)b * H + h] = mr.lse;
        f32x4 acc[ABS_COLS / 16];
#pragma unroll
        for (int db = 0; db < ABS_COLS / 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) abs_kstep(smem, kk, g, jj, qd, cur[kk], acc);
        abs_store_staged(o_v, acc, bb + 16 * w, b_hi, H, h, Dv, col0, smem + Dl * 256 + w * ABS_STG_BYTES, n, g,
                         lane);
    }
}

hipError_t ensure_smem_attr(const void* fn, int bytes);

// Rows of q_nope per workgroup: all of them when the (head, column block)
// grid alone fills the chip; otherwise split into row blocks (multiples of
// 64) until about 256 workgroups run.
static int abs_rows(int B, int H, int nc) {
    const int blocks64 = (B + 63) / 64;
    const long long units = (long long)H * nc;
    int nb = units >= 256 ? 1 : (int)((256 + units - 1) / units);
    nb = nb < 1 ? 1 : (nb > blocks64 ? blocks64 : nb);
    return 64 * ((blocks64 + nb - 1) / nb);
}

template <int KS>
static hipError_t launch_abs(const __bf16* q_nope, const __bf16* w_uk, __bf16* q_lat, int B, int H, int Dn, int Dl,
                             hipStream_t stream) {
    const int smem = Dn * ABS_COLS * 2 + 4 * ABS_STG_BYTES;
    if (smem > 64 * 1024) {
        hipError_t e = ensure_smem_attr((const void*)mla_absorb_kernel<KS>, smem);
        if (e != hipSuccess) return e;
    }
    const int nc = Dl / ABS_COLS;
    const int rows = abs_rows(B, H, nc);
    const long long grid = (long long)nc * H * ((B + rows - 1) / rows);
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(mla_absorb_kernel<KS>, dim3((unsigned)grid), dim3(ABS_THREADS), smem, stream, q_nope, w_uk,
                       q_lat, B, H, Dn, Dl, rows);
    return hipGetLastError();
}

hipError_t launch_mla_merge_up(const int* ws, int seq_first, int seq_nsplit, const __bf16* o_part,
                               const float* lse_part, const __bf16* w_uv, __bf16* o_v, float* lse, int B, int H,
                               int Dv, hipStream_t stream) {
    constexpr int KS = 16;  // Dl = 512
    const int smem = 32 * KS * ABS_COLS * 2 + 4 * ABS_STG_BYTES;
    hipError_t e = ensure_smem_attr((const void*)mla_merge_up_kernel<KS>, smem);
    if (e != hipSuccess) return e;
    const int nc = Dv / ABS_COLS;
    const int rows = abs_rows(B, H, nc);
    const long long grid = (long long)nc * H * ((B + rows - 1) / rows);
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(mla_merge_up_kernel<KS>, dim3((unsigned)grid), dim3(ABS_THREADS), smem, stream, ws, seq_first,
                       seq_nsplit, o_part, lse_part, w_uv, o_v, lse, B, H, Dv, rows);
    return hipGetLastError();
}

hipError_t launch_mla_absorb(const __bf16* q_nope, const __bf16* w_uk, __bf16* q_lat, int B, int H, int Dn, int Dl,
                             hipStream_t stream) {
    if (Dn == 128) return launch_abs<4>(q_nope, w_uk, q_lat, B, H, Dn, Dl, stream);
    if (Dn == 512) return launch_abs<16>(q_nope, w_uk, q_lat, B, H, Dn, Dl, stream);
    return launch_abs<0>(q_nope, w_uk, q_lat, B, H, Dn, Dl, stream);
}

}  // namespace mla
