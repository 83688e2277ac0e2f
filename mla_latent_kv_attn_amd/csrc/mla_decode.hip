// mla_decode.hip - absorbed MLA decode over the latent KV cache (gfx950).
//
// [MLA-FA3 article]: each cached token is one 576-wide bf16 row, the 512-dim
// compressed latent c^KV followed by the 64-dim decoupled RoPE key k^R
// (section 1 packs both into one descriptor row of latent_dim = 576).  With
// W_UK absorbed into the query (section 2, absorption equation) a head's
// score is one 576-wide dot product [q_lat || q_rope] . row, and the output
// is the softmax-weighted sum of the rows' first 512 dims.  The article's
// fused dataflow streams cache tiles on chip, takes both dot products there,
// applies online-softmax scaling with a partial reduction, accumulates in
// fp32 registers, and never writes a decompressed key or value.
//
// Three kernels run in stream order:
//   1. mla_plan_kernel   (one workgroup): split plan from seqlens.
//   2. mla_split_kernel  (one workgroup per part x 128-head block): streams
//      the part's cache tiles through LDS and writes either the final output
//      (sequence handled by one part) or a partial (o_s in bf16, lse_s fp32).
//   3. mla_combine_slots_kernel: log-sum-exp merge of the partials of every
//      split sequence; also writes o = 0, lse = -inf for empty sequences.
//
// Split-kernel design.  A workgroup has 8 waves (two per SIMD); wave w owns
// 16 heads, so one workgroup serves 128 heads and every cache byte crosses
// HBM -> LDS once for all of them.  Per wave the q fragments (16 heads x
// 576 bf16 = 72 VGPRs) and the fp32 output accumulator (16 x 512 = 128
// VGPRs) stay in registers.  The cache streams through a ring of four
// 32-token LDS tiles (4 x 37,888 B) filled by global_load_lds_dwordx4, so
// three tiles (~111 KiB per CU) are in flight while one is computed: with a
// single tile in flight the kernel is bound by memory latency, not by
// bandwidth.  Per tile and wave (v_mfma_f32_16x16x32_bf16):
//   S^T = C q^T   A = cache rows from LDS (K = 576 = 18 steps, two products
//                 of 16 tokens), B = the wave's q fragments.  Tokens are fed
//                 in a permuted order so that the S^T registers already form
//                 the P^T operand of the PV product.
//   O^T += C^T P^T  A = latent columns read transposed with
//                 ds_read_b64_tr_b16 from the same LDS tile, B = P in bf16.
// The same LDS bytes serve as key (576 dims) and value (first 512 dims).
#include <atomic>

#include "common.h"
#include "mla_plan.h"

namespace mla {

constexpr int DEC_WAVES = 8;
constexpr int DEC_HEADS = 16;  // heads per wave
constexpr int DEC_THREADS = DEC_WAVES * 64;
static_assert(DEC_WAVES * DEC_HEADS == kDecodeHeadsPerWG, "head split");
constexpr int DEC_ROW_CHUNKS = kRow * 2 / 16;                     // 72 chunks of 16 B per token
constexpr int DEC_STRIDE_CHUNKS = DEC_ROW_CHUNKS + 2;             // +2 pad chunks per row in LDS
constexpr int DEC_ROW_STRIDE = DEC_STRIDE_CHUNKS * 16;            // 1184 B (== 32 mod 128)
constexpr int DEC_TILE = 32;                                      // tokens per LDS tile (one MFMA k-step of PV)
constexpr int DEC_NBUF = 4;                                       // tiles in the LDS ring
constexpr int DEC_AHEAD = DEC_NBUF - 2;                           // tiles in flight (one tile is computed, one
                                                                  // kept for the lagging wave group's PV)
constexpr int DEC_TILE_BYTES = DEC_TILE * DEC_ROW_STRIDE;         // 37888
constexpr int DEC_TILE_INSTR = DEC_TILE * DEC_STRIDE_CHUNKS / 64; // 37 wave-wide 1 KiB copies per tile
constexpr int DEC_SMEM = DEC_NBUF * DEC_TILE_BYTES;               // 151552
static_assert(DEC_TILE * DEC_STRIDE_CHUNKS % 64 == 0, "whole copies");
static_assert(DEC_SMEM <= 160 * 1024, "LDS");
static_assert(kDecodeTile % DEC_TILE == 0, "plan tiles are whole LDS tiles");
constexpr int DEC_LOADS_HI = (DEC_TILE_INSTR + DEC_WAVES - 1) / DEC_WAVES;  // copies of waves < EXTRA
constexpr int DEC_LOADS_LO = DEC_TILE_INSTR / DEC_WAVES;                    // copies of the other waves
constexpr int DEC_LOADS_EXTRA = DEC_TILE_INSTR % DEC_WAVES;                 // waves issuing one more copy

// LDS fragment prefetch distances, in MFMA steps, for the S^T and PV loops.
#ifndef MLA_DEC_PF_QK
#define MLA_DEC_PF_QK 2
#endif
#ifndef MLA_DEC_PF_PV
#define MLA_DEC_PF_PV 4
#endif
constexpr int DEC_PF = MLA_DEC_PF_QK;
constexpr int DEC_PFV = MLA_DEC_PF_PV;
static_assert(DEC_PF <= DEC_PFV, "PV ring slots 0..DEC_PF-1 are filled during the S^T tail");
static_assert(2 * DEC_PF < 16 && 2 * DEC_PFV < 16, "lgkmcnt range");

struct PlanArgs {
    int seq_len, seq_n, seq_start, seq_first, seq_nsplit, part_first_seq;  // int32 offsets
    long long o_part_off, lse_part_off;                                    // byte offsets
};

// LDS layout of a tile: token row r at byte r * 1184 (72 data chunks + 2
// pad chunks).  A row stride of 32 (mod 128) bytes is what measured free of
// bank conflicts for the 16-row fragment reads of S^T (1152 runs 4x and
// 1168 or 1216 2x slower on gfx950); the transposed reads run at the same
// rate for every stride tried.

// ---------------------------------------------------------------------------
// 1. Plan.  Cost line: sequence b occupies n_b + c0 positions (n_b tiles
//    after c0 positions of fixed cost), empty sequences occupy none; part p
//    owns positions [p t, (p+1) t) with
//      t = max(ceil(C / parts), ceil(max_n / (num_splits - 1)), t_min, 1),
//    which bounds every sequence to at most num_splits parts.  With
//    num_splits == 1 each sequence gets its own part (t = max_n + c0).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void mla_plan_kernel(const int* __restrict__ seqlens, int* __restrict__ ws,
                                                       int B, int S_max, int parts, int c0, int t_min,
                                                       int num_splits, PlanArgs a) {
    __shared__ int scan[1024];
    __shared__ int s_max, s_clamp, s_carry;
    const int tid = threadIdx.x;
    if (tid == 0) { s_max = 0; s_clamp = 0; s_carry = 0; }
    __syncthreads();
    for (int base = 0; base < B; base += 1024) {
        const int b = base + tid;
        int cost = 0;
        if (b < B) {
            const int raw = seqlens[b];
            const int len = min(max(raw, 0), S_max);
            if (len != raw) atomicAdd(&s_clamp, 1);
            const int n = (len + kDecodeTile - 1) / kDecodeTile;
            cost = n > 0 ? n + c0 : 0;
            ws[a.seq_len + b] = len;
            ws[a.seq_n + b] = n;
            atomicMax(&s_max, n);
        }
        scan[tid] = cost;
        __syncthreads();
        for (int d = 1; d < 1024; d <<= 1) {
            const int add = tid >= d ? scan[tid - d] : 0;
            __syncthreads();
            scan[tid] += add;
            __syncthreads();
        }
        if (b < B) ws[a.seq_start + b] = s_carry + scan[tid] - cost + c0;
        __syncthreads();
        if (tid == 0) s_carry += scan[1023];
        __syncthreads();
    }
    const int max_n = s_max;
    const bool whole = num_splits == 1;
    int t, C, parts_used, nparts;
    if (whole) {
        t = max(max_n + c0, 1);
        C = B * t;
        parts_used = B;
        nparts = B;
    } else {
        C = s_carry;
        t = max(max((C + parts - 1) / parts, (max_n + num_splits - 2) / (num_splits - 1)), max(t_min, 1));
        parts_used = (C + t - 1) / t;
        nparts = parts;
    }
    for (int p = tid; p < nparts; p += 1024) ws[a.part_first_seq + p] = B;
    __syncthreads();
    for (int b = tid; b < B; b += 1024) {
        const int n = ws[a.seq_n + b];
        int start = ws[a.seq_start + b];
        if (whole) {
            start = b * t + c0;
            ws[a.seq_start + b] = start;
        }
        const int first = n > 0 ? start / t : 0;
        const int ns = n > 0 ? (start + n - 1) / t - first + 1 : 0;
        ws[a.seq_first + b] = first;
        ws[a.seq_nsplit + b] = ns;
        for (int p = first; p < first + ns; ++p) atomicMin(&ws[a.part_first_seq + p], b);
    }
    if (tid == 0) {
        ws[kHdrPartsUsed] = parts_used;
        ws[kHdrT] = t;
        ws[kHdrC] = C;
        ws[kHdrTile] = kDecodeTile;
        ws[kHdrC0] = c0;
        ws[kHdrMode] = whole ? 1 : 0;
        ws[kHdrParts] = nparts;
        ws[kHdrClamped] = s_clamp;
        ws[kHdrMaxN] = max_n;
        ws[kHdrB] = B;
        ws[kHdrTMin] = t_min;
        ws[kHdrNumSplits] = num_splits;
    }
}

// ---------------------------------------------------------------------------
// 2. Split kernel
// ---------------------------------------------------------------------------
struct DecodeCtx {
    const __bf16* q_lat;
    const __bf16* q_rope;
    const __bf16* cache;
    const int* ws;
    __bf16* o_part;
    float* lse_part;
    __bf16* o;
    float* lse;
    int H, S_max;
    float c_log2;
    PlanArgs a;
};

// Copy one 32-token tile to LDS: copy i (0..36) of 64 chunks is issued by
// wave i % 8.  Chunk L of the tile is row L / 74, chunk L % 74 of that row;
// the pad chunks (72, 73) receive second copies of chunks 0 and 1.  Each
// wave's per-lane source offsets within a tile are fixed (dec_copy_offsets);
// a tile only moves the buffer resource, whose size ends at the sequence's
// last token, so rows past the end read as zeros (their scores are masked).
__device__ __forceinline__ void dec_copy_offsets(uint32_t (&voff)[DEC_LOADS_HI], int w, int lane) {
#pragma unroll
    for (int k = 0; k < DEC_LOADS_HI; ++k) {
        const int L = (w + DEC_WAVES * k) * 64 + lane;
        const int r = L / DEC_STRIDE_CHUNKS;
        int c = L - r * DEC_STRIDE_CHUNKS;
        c = (c >= DEC_ROW_CHUNKS) ? c - DEC_ROW_CHUNKS : c;
        voff[k] = (uint32_t)(r * kRow * 2 + 16 * c);
    }
}

__device__ __forceinline__ void dec_issue_tile(const __bf16* seq, int len, int tok0, char* buf,
                                               const uint32_t (&voff)[DEC_LOADS_HI], int w) {
    const auto rsrc = make_rsrc(seq + (size_t)tok0 * kRow, (uint32_t)(len - tok0) * (uint32_t)(kRow * 2));
    static_for<DEC_LOADS_HI>([&](auto k_c) {
        constexpr int k = decltype(k_c)::value;
        if (k < DEC_LOADS_LO || w < DEC_LOADS_EXTRA)
            bload_lds16(rsrc, buf + (w + DEC_WAVES * k) * 1024, voff[k]);
    });
}

// Wait until this wave's copies of the oldest in-flight tile have landed,
// leaving `later` younger tiles in flight.
template <int LATER>
__device__ __forceinline__ void dec_wait_tile(int w) {
    if (w < DEC_LOADS_EXTRA) wait_vmcnt<LATER * DEC_LOADS_HI>();
    else wait_vmcnt<LATER * DEC_LOADS_LO>();
}

// Token permutation inside a 32-token block, for v_mfma_f32_16x16x32_bf16.
// The two S^T = C q^T products of a block (tokens 0..15 and 16..31) feed
// MFMA row i = 4g + j the token pi(i) = 2j + (g & 1) + 8(g >> 1) (+16 for the
// second).  Lane group g of the results then holds, in its eight registers
// (four per product), the tokens that the P^T operand of the PV product
// assigns to logical k = 8g + e, and:
//  * the rows an 8-lane group reads for S^T have distinct low 3 bits;
//  * the 4 rows a 16-lane ds_read_b64_tr_b16 touches are two apart.
__device__ __forceinline__ int dec_pi16(int i) { return 2 * (i & 3) + ((i >> 2) & 1) + 8 * (i >> 3); }
__device__ __forceinline__ int dec_token_of(int g, int e) {  // e = 0..7 of lane group g
    return 16 * (e >> 2) + 2 * (e & 3) + (g & 1) + 8 * (g >> 1);
}

__device__ void dec_piece(const DecodeCtx& x, char* smem, int p, int b, int tile_lo, int tile_hi, int len,
                          int nsplit, bool first_in_part) {
    const int w = wave_id();
    const int lane = lane_id();
    const int n = lane & 15;  // head column of the MFMA results / MFMA row of the A operand
    const int g = lane >> 4;  // row group (0..3)
    const int H = x.H;
    const int hbase = blockIdx.y * kDecodeHeadsPerWG + DEC_HEADS * w;
    const bool active = hbase < H;  // H % 16 == 0: a wave is fully in or out
    const int head = hbase + n;
    const int tok_end = min(tile_hi * kDecodeTile, len);

    f32x4 oacc[kLatent / 16];
#pragma unroll
    for (int db = 0; db < kLatent / 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    // Per-lane LDS byte offsets; everything else is a compile-time immediate.
    const int qk_off = dec_pi16(n) * DEC_ROW_STRIDE + 16 * g;
    const int jj = n >> 2, qd = n & 3;  // ds_read_b64_tr_b16 source lane = 4*jj + qd
    const int pv_off = dec_pi16(4 * g + jj) * DEC_ROW_STRIDE + 8 * qd;
    // The piece covers plan tiles [tile_lo, tile_hi); LDS tiles are 32 tokens.
    const int tok_lo = tile_lo * kDecodeTile;
    const int ntiles = (tok_end - tok_lo + DEC_TILE - 1) / DEC_TILE;

    // Ring of DEC_NBUF LDS tiles.  DEC_AHEAD tiles are in flight while tile j
    // is computed, enough outstanding HBM reads per CU to cover the memory
    // latency.  The two waves sharing a SIMD run half a tile apart: group A
    // (waves 0-3) does S^T, softmax and PV of tile j; group B (waves 4-7)
    // first finishes PV of tile j-1, then S^T and softmax of tile j, so one
    // wave's softmax overlaps the other's matrix work.  One barrier per tile
    // publishes tile j (every wave has waited for its own copies) and proves
    // tile j-2 fully consumed, so tile j+DEC_AHEAD can be copied into its
    // buffer right after it.
    const bool lag = w >= DEC_WAVES / 2;
    const __bf16* seq = x.cache + (size_t)b * x.S_max * kRow;
    uint32_t voff[DEC_LOADS_HI];
    dec_copy_offsets(voff, w, lane);
#pragma unroll
    for (int i = 0; i < DEC_AHEAD; ++i)
        if (i < ntiles) dec_issue_tile(seq, len, tok_lo + i * DEC_TILE, smem + i * DEC_TILE_BYTES, voff, w);

    // q fragments (loaded after the first tile copies are in flight) as the B
    // operand of S^T = C q^T: lane (head n, g) holds dims 32kk+8g..+7.
    bf16x8 qf[kRow / 32];
    if (active) {
        const bf16x8* ql = reinterpret_cast<const bf16x8*>(x.q_lat + ((size_t)b * H + head) * kLatent);
        const bf16x8* qr = reinterpret_cast<const bf16x8*>(x.q_rope + ((size_t)b * H + head) * kRope);
#pragma unroll
        for (int kk = 0; kk < kLatent / 32; ++kk) qf[kk] = ql[4 * kk + g];
#pragma unroll
        for (int kk = 0; kk < kRope / 32; ++kk) qf[kLatent / 32 + kk] = qr[4 * kk + g];
    }


    constexpr int KS = kRow / 32;      // S^T k-steps
    constexpr int NS = kLatent / 16;   // PV dim blocks
    bf16x8 fa[DEC_PF + 1], fb[DEC_PF + 1], fv[DEC_PFV + 1];
    bf16x8 pb_prev;                    // P of tile j-1 (lagging group)
    uint32_t pv_prev = 0;              // LDS address of tile j-1's PV fragments

    // Fragment rings: S^T fragments (fa, fb) run DEC_PF steps ahead of the
    // MFMAs that consume them, PV fragments (fv) DEC_PFV steps.  Every S^T
    // step issues one unit of two reads, so when step kk's pair is consumed
    // exactly 2*DEC_PF newer reads are outstanding; PV step db has
    // 2*min(DEC_PFV, NS-1-db).  Schedule barriers pin this order.
    auto pv_phase = [&](uint32_t pv_a, const bf16x8& p) {
        auto rd_pv = [&](auto db_c) {
            constexpr int db = decltype(db_c)::value;
            fv[db % (DEC_PFV + 1)] = join(ds_read_tr16<32 * db>(pv_a),
                                          ds_read_tr16<16 * DEC_ROW_STRIDE + 32 * db>(pv_a));
        };
        static_for<DEC_PFV>([&](auto i) { rd_pv(i); });
        static_for<NS>([&](auto db_c) {
            constexpr int db = decltype(db_c)::value;
            if constexpr (db + DEC_PFV < NS) rd_pv(std::integral_constant<int, db + DEC_PFV>{});
            constexpr int newer = 2 * ((NS - 1 - db) < DEC_PFV ? (NS - 1 - db) : DEC_PFV);
            wait_lgkm_for<newer>(fv[db % (DEC_PFV + 1)]);
            __builtin_amdgcn_sched_barrier(0);
            oacc[db] = mfma16(fv[db % (DEC_PFV + 1)], p, oacc[db]);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // S^T for the tile's 32 tokens (sa: first 16, sb: second 16), masks,
    // online softmax (log2 domain) and P in bf16.
    auto qk_softmax = [&](uint32_t qk_a, int valid) -> bf16x8 {
        auto rd_qk = [&](auto kk_c) {
            constexpr int kk = decltype(kk_c)::value;
            fa[kk % (DEC_PF + 1)] = ds_read16<64 * kk>(qk_a);
            fb[kk % (DEC_PF + 1)] = ds_read16<16 * DEC_ROW_STRIDE + 64 * kk>(qk_a);
        };
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
        static_for<DEC_PF>([&](auto i) { rd_qk(i); });
        static_for<KS>([&](auto kk_c) {
            constexpr int kk = decltype(kk_c)::value;
            if constexpr (kk + DEC_PF < KS) rd_qk(std::integral_constant<int, kk + DEC_PF>{});
            constexpr int newer = 2 * ((KS - 1 - kk) < DEC_PF ? (KS - 1 - kk) : DEC_PF);
            wait_lgkm_for<newer>(fa[kk % (DEC_PF + 1)], fb[kk % (DEC_PF + 1)]);
            __builtin_amdgcn_sched_barrier(0);
            sa = mfma16(fa[kk % (DEC_PF + 1)], qf[kk], sa);
            sb = mfma16(fb[kk % (DEC_PF + 1)], qf[kk], sb);
            __builtin_amdgcn_sched_barrier(0);
        });
        if (valid < DEC_TILE) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (dec_token_of(g, r) >= valid) sa[r] = -INFINITY;
                if (dec_token_of(g, 4 + r) >= valid) sb[r] = -INFINITY;
            }
        }
        float mt = fmaxf(fmaxf(fmaxf(sa[0], sa[1]), fmaxf(sa[2], sa[3])),
                         fmaxf(fmaxf(sb[0], sb[1]), fmaxf(sb[2], sb[3])));
        mt = max4_groups16(mt) * x.c_log2;
        // Lazy rescale: the exponent base m only moves when some head's max
        // exceeds it by more than kRescaleSlack (P stays below
        // 2^kRescaleSlack); l and the accumulator share the base, so the
        // final O = acc / l is unchanged.
        if (__builtin_amdgcn_ballot_w64(mt > m + kRescaleSlack) != 0) {
            const float m_new = fmaxf(m, mt);
            const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - m_new);
            l *= alpha;
#pragma unroll
            for (int db = 0; db < kLatent / 16; ++db) oacc[db] *= alpha;
            m = m_new;
        }
        const float mb = (m == -INFINITY) ? 0.f : m;
        bf16x8 pb;  // logical k = 8g + e
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float pa = fast_exp2(__builtin_fmaf(sa[r], x.c_log2, -mb));
            const float pq = fast_exp2(__builtin_fmaf(sb[r], x.c_log2, -mb));
            l += pa + pq;
            pb[r] = to_bf16(pa);
            pb[4 + r] = to_bf16(pq);
        }
        return pb;
    };

    for (int j = 0; j < ntiles; ++j) {
        char* cur = smem + (j % DEC_NBUF) * DEC_TILE_BYTES;
        if (j + 1 < ntiles) dec_wait_tile<1>(w);   // tile j+1 may still be in flight
        else wait_vmcnt<0>();
        lds_barrier();
        if (j + DEC_AHEAD < ntiles)
            dec_issue_tile(seq, len, tok_lo + (j + DEC_AHEAD) * DEC_TILE,
                           smem + ((j + DEC_AHEAD) % DEC_NBUF) * DEC_TILE_BYTES, voff, w);
        if (active) {
            const uint32_t base = lds_addr(cur);
            if (lag && j > 0) pv_phase(pv_prev, pb_prev);
            const bf16x8 pb = qk_softmax(base + qk_off, tok_end - (tok_lo + j * DEC_TILE));
            if (lag) {
                pb_prev = pb;
                pv_prev = base + pv_off;
            } else {
                pv_phase(base + pv_off, pb);
            }
        }
    }
    if (active && lag && ntiles > 0) pv_phase(pv_prev, pb_prev);
    lds_barrier();  // every wave is done with the ring before the next piece refills it

    if (!active) return;
    l = sum4_groups16(l);
    const float inv_l = 1.f / l;
    const float lse_v = (m + __builtin_log2f(l)) * kLn2;
    // O^T block db: lane (head n, g) holds dims 16db + 4g + 0..3.
    if (nsplit == 1) {
        __bf16* op = x.o + ((size_t)b * H + head) * kLatent + 4 * g;
#pragma unroll
        for (int db = 0; db < kLatent / 16; ++db) {
            bf16x4 t;
#pragma unroll
            for (int r = 0; r < 4; ++r) t[r] = to_bf16(oacc[db][r] * inv_l);
            *reinterpret_cast<bf16x4*>(op + 16 * db) = t;
        }
        if (x.lse && g == 0) x.lse[(size_t)b * H + head] = lse_v;
    } else {
        // Partial of a split sequence: normalised over this piece, stored in
        // bf16 (the merge weights sum to one, so its rounding stays at the
        // level of the final bf16 output's).
        const int slot = 2 * p + (first_in_part ? 0 : 1);
        __bf16* op = x.o_part + ((size_t)slot * H + head) * kLatent + 4 * g;
#pragma unroll
        for (int db = 0; db < kLatent / 16; ++db) {
            bf16x4 t;
#pragma unroll
            for (int r = 0; r < 4; ++r) t[r] = to_bf16(oacc[db][r] * inv_l);
            *reinterpret_cast<bf16x4*>(op + 16 * db) = t;
        }
        if (g == 0) x.lse_part[(size_t)slot * H + head] = lse_v;
    }
}

// Pieces of part p, found without a chain of dependent loads: lane i reads
// the plan entries of sequence b0 + i (b0 = the part's first sequence) in one
// round trip, and a ballot lists the lanes whose sequence has tiles in the
// part.  A part spans more than 64 sequences only when they are very short;
// then the next 64 are read the same way.
__global__ __launch_bounds__(DEC_THREADS, 2) void mla_split_kernel(DecodeCtx x) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int p = blockIdx.x;
    const int* ws = x.ws;
    const int parts_used = ws[kHdrPartsUsed];
    if (p >= parts_used) return;
    const int t = ws[kHdrT];
    const int whole = ws[kHdrMode];
    const int B = ws[kHdrB];
    const int pos_lo = p * t, pos_hi = pos_lo + t;
    const int lane = lane_id();
    const int b0 = ws[x.a.part_first_seq + p];
    for (int base = b0; base < B; base += 64) {
        const int b = base + lane;
        int nb = 0, sb = pos_hi, ln = 0, ns = 0;
        if (b < B && (!whole || b == b0)) {
            nb = ws[x.a.seq_n + b];
            sb = ws[x.a.seq_start + b];
            ln = ws[x.a.seq_len + b];
            ns = ws[x.a.seq_nsplit + b];
        }
        const int lo = max(sb, pos_lo) - sb;
        const int hi = min(sb + nb, pos_hi) - sb;
        uint64_t pieces = __builtin_amdgcn_ballot_w64(nb > 0 && lo < hi);
        const bool more = __builtin_amdgcn_ballot_w64(nb > 0 && sb >= pos_hi) == 0 && base + 64 < B && !whole;
        while (pieces) {
            const int i = __builtin_ctzll(pieces);
            pieces &= pieces - 1;
            dec_piece(x, smem, p, base + i, __builtin_amdgcn_readlane(lo, i), __builtin_amdgcn_readlane(hi, i),
                      __builtin_amdgcn_readlane(ln, i), __builtin_amdgcn_readlane(ns, i), base + i == b0);
        }
        if (!more) break;
    }
}

// ---------------------------------------------------------------------------
// 3. Combine: lse = log sum_s exp(lse_s); o = sum_s exp(lse_s - lse) o_s.
//    Empty splits (lse_s = -inf) weigh 0; all empty -> o = 0, lse = -inf.
//    A workgroup of 256 threads serves 4 heads of one sequence; a thread owns
//    8 consecutive output dims.  The per-split loads are independent, so
//    they are issued back to back.
// ---------------------------------------------------------------------------
constexpr int CMB_THREADS = 256;
constexpr int CMB_HEADS = CMB_THREADS / (kLatent / 8);  // 4

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

// rows(s) gives the row index of split s in lse_part (and, times 512, in o_part).
template <typename PT, typename RowFn>
__device__ __forceinline__ void combine_head(const PT* o_part, const float* lse_part, int nsplit, RowFn rows,
                                             __bf16* o_row, float* lse_out, int d8) {
    float M = -INFINITY;
#pragma unroll 4
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, lse_part[rows(s)]);
    bf16x8 out;
    if (M == -INFINITY) {
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = to_bf16(0.f);
        *reinterpret_cast<bf16x8*>(o_row + 8 * d8) = out;
        if (lse_out && d8 == 0) *lse_out = -INFINITY;
        return;
    }
    float W = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = 0; s < nsplit; ++s) {
        const size_t r = rows(s);
        const float ls = lse_part[r];
        const float wgt = (ls == -INFINITY) ? 0.f : __expf(ls - M);
        float v[8];
        load8(o_part + r * kLatent + 8 * d8, v);
        W += wgt;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = (wgt == 0.f) ? acc[i] : __builtin_fmaf(wgt, v[i], acc[i]);
    }
    const float inv = 1.f / W;
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = to_bf16(acc[i] * inv);
    *reinterpret_cast<bf16x8*>(o_row + 8 * d8) = out;
    if (lse_out && d8 == 0) *lse_out = M + __logf(W);
}

// Partials of the split kernel: slot-major [slots][H][512] bf16, lse [slots][H].
__global__ __launch_bounds__(CMB_THREADS) void mla_combine_slots_kernel(const int* __restrict__ ws,
                                                                       const __bf16* __restrict__ o_part,
                                                                       const float* __restrict__ lse_part,
                                                                       __bf16* __restrict__ o, float* lse, int H,
                                                                       PlanArgs a) {
    const int b = blockIdx.x;
    const int ns = ws[a.seq_nsplit + b];
    if (ns == 1) return;
    const int hh = blockIdx.y * CMB_HEADS + (threadIdx.x >> 6);
    if (hh >= H) return;
    const int d8 = threadIdx.x & 63;
    const int first = ws[a.seq_first + b];
    const int* pfs = ws + a.part_first_seq;
    auto rows = [&](int s) -> size_t {
        const int p = first + s;
        return (size_t)(2 * p + (pfs[p] == b ? 0 : 1)) * H + hh;
    };
    combine_head(o_part, lse_part, ns, rows, o + ((size_t)b * H + hh) * kLatent,
                 lse ? lse + (size_t)b * H + hh : nullptr, d8);
}

// Caller-supplied dense partials: o_part [B,H,S,512] fp32, lse_part [B,H,S].
__global__ __launch_bounds__(CMB_THREADS) void mla_combine_dense_kernel(const float* __restrict__ o_part,
                                                                       const float* __restrict__ lse_part,
                                                                       __bf16* __restrict__ o, float* lse, int H,
                                                                       int S) {
    const int b = blockIdx.x;
    const int hh = blockIdx.y * CMB_HEADS + (threadIdx.x >> 6);
    if (hh >= H) return;
    const int d8 = threadIdx.x & 63;
    const size_t row0 = ((size_t)b * H + hh) * S;
    auto rows = [&](int s) -> size_t { return row0 + s; };
    combine_head(o_part, lse_part, S, rows, o + ((size_t)b * H + hh) * kLatent,
                 lse ? lse + (size_t)b * H + hh : nullptr, d8);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
// Opt a kernel into more than 64 KiB of dynamic LDS, once per device.
hipError_t ensure_smem_attr(const void* fn, int bytes) {
    static std::atomic<int> done[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64 && done[dev].load(std::memory_order_acquire) >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && dev >= 0 && dev < 64) done[dev].store(bytes, std::memory_order_release);
    return e;
}

static PlanArgs plan_args(const PlanLayout& L) {
    PlanArgs a;
    a.seq_len = (int)L.seq_len;
    a.seq_n = (int)L.seq_n;
    a.seq_start = (int)L.seq_start;
    a.seq_first = (int)L.seq_first;
    a.seq_nsplit = (int)L.seq_nsplit;
    a.part_first_seq = (int)L.part_first_seq;
    a.o_part_off = (long long)L.o_part_bytes_off;
    a.lse_part_off = (long long)L.lse_part_bytes_off;
    return a;
}

hipError_t launch_mla_decode(const __bf16* q_lat, const __bf16* q_rope, const __bf16* cache, const int* seqlens,
                             __bf16* o, float* lse, int B, int H, int S_max, float scale, int num_splits,
                             const PlanLayout& L, int c0, int t_min, void* workspace, hipStream_t stream) {
    hipError_t e = ensure_smem_attr((const void*)mla_split_kernel, DEC_SMEM);
    if (e != hipSuccess) return e;
    int* ws = static_cast<int*>(workspace);
    const PlanArgs a = plan_args(L);
    hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(1024), 0, stream, seqlens, ws, B, S_max, L.parts, c0, t_min,
                       num_splits, a);
    DecodeCtx x;
    x.q_lat = q_lat;
    x.q_rope = q_rope;
    x.cache = cache;
    x.ws = ws;
    x.o_part = reinterpret_cast<__bf16*>(static_cast<char*>(workspace) + L.o_part_bytes_off);
    x.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.lse_part_bytes_off);
    x.o = o;
    x.lse = lse;
    x.H = H;
    x.S_max = S_max;
    x.c_log2 = scale * kLog2e;
    x.a = a;
    const int hblocks = (H + kDecodeHeadsPerWG - 1) / kDecodeHeadsPerWG;
    hipLaunchKernelGGL(mla_split_kernel, dim3(L.parts, hblocks), dim3(DEC_THREADS), DEC_SMEM, stream, x);
    hipLaunchKernelGGL(mla_combine_slots_kernel, dim3(B, (H + CMB_HEADS - 1) / CMB_HEADS), dim3(CMB_THREADS), 0,
                       stream, ws, x.o_part, x.lse_part, o, lse, H, a);
    return hipGetLastError();
}

hipError_t launch_mla_combine(const float* o_part, const float* lse_part, __bf16* o, float* lse, int B, int H,
                              int S, hipStream_t stream) {
    hipLaunchKernelGGL(mla_combine_dense_kernel, dim3(B, (H + CMB_HEADS - 1) / CMB_HEADS), dim3(CMB_THREADS), 0,
                       stream, o_part, lse_part, o, lse, H, S);
    return hipGetLastError();
}

}  // namespace mla
