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
// Split-kernel design.  A workgroup is 4 waves, one per SIMD, and serves 128
// heads, so every cache byte crosses HBM -> LDS once for all of them.  The
// cache streams through a ring of four 32-token LDS tiles (37,888 B each)
// filled by buffer_load ... lds (non-temporal: every cache row is read once).
// Wave w owns heads 32w..32w+31 for the whole
// computation:
//   * their q fragments stay in VGPRs (32 heads x 576 bf16 = 144 VGPRs);
//   * S^T = C q^T on v_mfma_f32_16x16x32_bf16, every cache fragment read from
//     LDS feeding the MFMAs of both 16-head blocks;
//   * online softmax (log2 domain, lazy rescale) in registers; P^T (bf16)
//     stays in the registers that the value product reads;
//   * O^T += C^T P^T with C^T read transposed (ds_read_b64_tr_b16) from the
//     same tile; the 32 x 512 fp32 accumulators fill the 256 AGPRs.
// Waves share nothing but the LDS tiles, so one barrier per tile suffices.
// With one wave per SIMD there is no second wave to hide latency behind:
// each tile step interleaves the value product of the previous tile with the
// scores of the current one, and fragment reads run several MFMA groups
// ahead, across the tile barrier where the tile is already resident.
// The MFMAs are inline asm so that the score accumulators stay in VGPRs and
// the value accumulators in fixed AGPRs.  The hardware interlocks
// MFMA-to-MFMA accumulator chains; the places where ordinary instructions
// read MFMA results carry explicit wait states (s_nop).
#include <atomic>
#include <mutex>

#include "common.h"
#include "mla_merge.h"
#include "mla_plan.h"

namespace mla {

constexpr int DEC_WAVES = 4;
constexpr int DEC_THREADS = DEC_WAVES * 64;
constexpr int DEC_HB = kDecodeHeadsPerWG / 16;                    // 8 head blocks of 16 per workgroup
constexpr int DEC_ROW_CHUNKS = kRow * 2 / 16;                     // 72 chunks of 16 B per token
constexpr int DEC_STRIDE_CHUNKS = DEC_ROW_CHUNKS + 2;             // +2 pad chunks per row in LDS
constexpr int DEC_ROW_STRIDE = DEC_STRIDE_CHUNKS * 16;            // 1184 B (== 32 mod 128)
constexpr int DEC_TILE = 32;                                      // tokens per LDS tile (one MFMA k-step of PV)
constexpr int DEC_NBUF = 4;                                       // tiles in the LDS ring
constexpr int DEC_AHEAD = 2;                                      // tiles in flight (one more is held for values)
constexpr int DEC_TILE_BYTES = DEC_TILE * DEC_ROW_STRIDE;         // 37888
constexpr int DEC_TILE_INSTR = DEC_TILE * DEC_STRIDE_CHUNKS / 64; // 37 wave-wide 1 KiB copies per tile
constexpr int DEC_SMEM = DEC_NBUF * DEC_TILE_BYTES;               // 151,552 B
static_assert(DEC_WAVES * 2 == DEC_HB, "two head blocks per wave");
static_assert(DEC_TILE * DEC_STRIDE_CHUNKS % 64 == 0, "whole copies");
static_assert(DEC_SMEM <= 160 * 1024, "LDS");
static_assert(kDecodeTile % DEC_TILE == 0, "plan tiles are whole LDS tiles");
static_assert(DEC_AHEAD + 2 <= DEC_NBUF, "ring: values tile, scores tile, tiles in flight");
constexpr int DEC_LOADS_HI = (DEC_TILE_INSTR + DEC_WAVES - 1) / DEC_WAVES;  // copies of waves < EXTRA
constexpr int DEC_LOADS_LO = DEC_TILE_INSTR / DEC_WAVES;                    // copies of the other waves
constexpr int DEC_LOADS_EXTRA = DEC_TILE_INSTR % DEC_WAVES;                 // waves issuing one more copy
static_assert(DEC_AHEAD * DEC_LOADS_HI < 64, "vmcnt range");

#define MLA_ALL_AGPRS "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15", "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31", "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47", "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63", "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79", "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95", "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111", "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127", "a128", "a129", "a130", "a131", "a132", "a133", "a134", "a135", "a136", "a137", "a138", "a139", "a140", "a141", "a142", "a143", "a144", "a145", "a146", "a147", "a148", "a149", "a150", "a151", "a152", "a153", "a154", "a155", "a156", "a157", "a158", "a159", "a160", "a161", "a162", "a163", "a164", "a165", "a166", "a167", "a168", "a169", "a170", "a171", "a172", "a173", "a174", "a175", "a176", "a177", "a178", "a179", "a180", "a181", "a182", "a183", "a184", "a185", "a186", "a187", "a188", "a189", "a190", "a191", "a192", "a193", "a194", "a195", "a196", "a197", "a198", "a199", "a200", "a201", "a202", "a203", "a204", "a205", "a206", "a207", "a208", "a209", "a210", "a211", "a212", "a213", "a214", "a215", "a216", "a217", "a218", "a219", "a220", "a221", "a222", "a223", "a224", "a225", "a226", "a227", "a228", "a229", "a230", "a231", "a232", "a233", "a234", "a235", "a236", "a237", "a238", "a239", "a240", "a241", "a242", "a243", "a244", "a245", "a246", "a247", "a248", "a249", "a250", "a251", "a252", "a253", "a254", "a255"

struct PlanArgs {
    int seq_len, seq_n, seq_start, seq_first, seq_nsplit, part_first_seq;  // int32 offsets
    long long o_part_off, lse_part_off;                                    // byte offsets
};

// LDS layout of a tile: token row r at byte r * 1184 (72 data chunks + 2
// pad chunks).  A row stride of 32 (mod 128) bytes is what measured free of
// bank conflicts for the 16-row fragment reads of S^T (1152 runs 4x and
// 1168 or 1216 2x slower on gfx950); the transposed reads run at the same
// rate for every stride tried.

// 1. Plan.  Cost line: sequence b occupies n_b + c0 positions (n_b tiles
//    after c0 positions of fixed cost), empty sequences occupy none; part p
//    owns positions [p t, (p+1) t) with
//      t = max(ceil(C / parts), ceil(max_n / (num_splits - 1)), t_min, 1),
//    which bounds every sequence to at most num_splits parts.  With
//    num_splits == 1 each sequence gets its own part (t = max_n + c0).
//    A block of 256 threads scans the lengths: each thread handles four
//    consecutive sequences of a 1024-sequence chunk, so the offsets need one
//    scan per chunk (within each wave by DPP lane shifts, then over the four
//    wave totals).  The first sequence of each part is found with LDS
//    atomics.
//    Where it runs: with num_splits >= 2 and B <= 1024 every split workgroup
//    computes the plan itself, in LDS, before its first tile (workgroup 0
//    also writes it to the workspace for the combine); otherwise a one-block
//    plan kernel writes it to the workspace first.  The separate launch cost
//    5.5-6.2 us per call on MI355X, the in-kernel scan about 1 us.
// ---------------------------------------------------------------------------
constexpr int PLAN_THREADS = 256;
constexpr int PLAN_PER = 4;
constexpr int PLAN_CHUNK = PLAN_THREADS * PLAN_PER;
static_assert(PLAN_THREADS == 256, "the split kernel's block runs the in-kernel plan");

// One chunk of the cost-line scan: thread tid handles sequences
// base + 4 tid + k (k < 4).  Returns their clamped lengths, tiles and
// cost-line starts (carry = cost of every sequence before the chunk), and
// the chunk's total cost, largest n and clamp count (block-uniform).
// s_red: 12 ints of LDS.
struct ChunkScan {
    int total, max_n, clamped;
};
__device__ ChunkScan plan_scan_chunk(const int* __restrict__ seqlens, int base, int B, int S_max, int c0, int carry,
                                     int (&n)[PLAN_PER], int (&len)[PLAN_PER], int (&start)[PLAN_PER], int* s_red) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    constexpr int NW = PLAN_THREADS / 64;
    int cost[PLAN_PER], sum = 0, mx = 0, ncl = 0;
#pragma unroll
    for (int k = 0; k < PLAN_PER; ++k) {
        const int b = base + PLAN_PER * tid + k;
        n[k] = 0;
        len[k] = 0;
        if (b < B) {
            const int raw = seqlens[b];
            len[k] = min(max(raw, 0), S_max);
            ncl += len[k] != raw;
            n[k] = (len[k] + kDecodeTile - 1) / kDecodeTile;
            mx = max(mx, n[k]);
        }
        cost[k] = n[k] > 0 ? n[k] + c0 : 0;
        sum += cost[k];
    }
    const int incl = dpp_incl_sum(sum);
    mx = dpp_wave_max(mx);
    ncl = __builtin_amdgcn_readlane(dpp_incl_sum(ncl), 63);
    if (lane == 63) s_red[wv] = incl;
    if (lane == 0) {
        s_red[NW + wv] = mx;
        s_red[2 * NW + wv] = ncl;
    }
    lds_barrier();  // LDS only: no wait for this block's global stores
    int woff = 0;
    ChunkScan r{0, 0, 0};
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        woff += i < wv ? s_red[i] : 0;
        r.total += s_red[i];
        r.max_n = max(r.max_n, s_red[NW + i]);
        r.clamped += s_red[2 * NW + i];
    }
    lds_barrier();  // s_red is rewritten by the next chunk
    int acc = carry + woff + incl - sum;  // cost of all sequences before this thread's first
#pragma unroll
    for (int k = 0; k < PLAN_PER; ++k) {
        start[k] = acc + c0;
        acc += cost[k];
    }
    return r;
}

__device__ __forceinline__ int plan_line_t(int C, int parts, int max_n, int num_splits, int t_min) {
    return max(max((C + parts - 1) / parts, (max_n + num_splits - 2) / (num_splits - 1)), max(t_min, 1));
}

__device__ __forceinline__ void plan_write_header(int* ws, int parts_used, int t, int C, int c0, bool whole,
                                                  int nparts, int clamped, int max_n, int B, int t_min,
                                                  int num_splits) {
    ws[kHdrPartsUsed] = parts_used;
    ws[kHdrT] = t;
    ws[kHdrC] = C;
    ws[kHdrTile] = kDecodeTile;
    ws[kHdrC0] = c0;
    ws[kHdrMode] = whole ? 1 : 0;
    ws[kHdrParts] = nparts;
    ws[kHdrClamped] = clamped;
    ws[kHdrMaxN] = max_n;
    ws[kHdrB] = B;
    ws[kHdrTMin] = t_min;
    ws[kHdrNumSplits] = num_splits;
}

__global__ __launch_bounds__(PLAN_THREADS) void mla_plan_kernel(const int* __restrict__ seqlens, int* __restrict__ ws,
                                                               int B, int S_max, int parts, int c0, int t_min,
                                                               int num_splits, PlanArgs a) {
    __shared__ int s_red[12];
    __shared__ int s_pfs[kPlanMaxParts];
    const int tid = threadIdx.x;
    int my_n[PLAN_PER], my_len[PLAN_PER], my_start[PLAN_PER];  // kept for the second pass when B <= PLAN_CHUNK
    int carry = 0, max_n = 0, clamped = 0;
    for (int base = 0; base < B; base += PLAN_CHUNK) {
        const ChunkScan cs = plan_scan_chunk(seqlens, base, B, S_max, c0, carry, my_n, my_len, my_start, s_red);
#pragma unroll
        for (int k = 0; k < PLAN_PER; ++k) {
            const int b = base + PLAN_PER * tid + k;
            if (b < B) {
                ws[a.seq_len + b] = my_len[k];
                ws[a.seq_n + b] = my_n[k];
                ws[a.seq_start + b] = my_start[k];
            }
        }
        carry += cs.total;
        max_n = max(max_n, cs.max_n);
        clamped += cs.clamped;
    }
    const bool whole = num_splits == 1;
    int t, C, parts_used, nparts;
    if (whole) {
        t = max(max_n + c0, 1);
        C = B * t;
        parts_used = B;
        nparts = B;
    } else {
        C = carry;
        t = plan_line_t(C, parts, max_n, num_splits, t_min);
        parts_used = (C + t - 1) / t;
        nparts = parts;  // <= kPlanMaxParts (checked by the host)
        for (int p = tid; p < nparts; p += PLAN_THREADS) s_pfs[p] = B;
    }
    __syncthreads();
    for (int base = 0; base < B; base += PLAN_CHUNK) {
#pragma unroll
        for (int k = 0; k < PLAN_PER; ++k) {
            const int b = base + PLAN_PER * tid + k;
            if (b >= B) continue;
            // With one chunk the entries are still in registers; otherwise
            // they are read back (this thread wrote them above).
            const int n = B <= PLAN_CHUNK ? my_n[k] : ws[a.seq_n + b];
            int start = B <= PLAN_CHUNK ? my_start[k] : ws[a.seq_start + b];
            if (whole) {
                // Part b holds sequence b alone (t >= max_n + c0 > c0 + n - 1).
                start = b * t + c0;
                ws[a.seq_start + b] = start;
                ws[a.part_first_seq + b] = n > 0 ? b : B;
            }
            const int first = n > 0 ? start / t : 0;
            const int ns = n > 0 ? (start + n - 1) / t - first + 1 : 0;
            ws[a.seq_first + b] = first;
            ws[a.seq_nsplit + b] = ns;
            if (!whole)
                for (int p = first; p < first + ns; ++p) atomicMin(&s_pfs[p], b);
        }
    }
    if (!whole) {
        __syncthreads();
        for (int p = tid; p < nparts; p += PLAN_THREADS) ws[a.part_first_seq + p] = s_pfs[p];
    }
    if (tid == 0) plan_write_header(ws, parts_used, t, C, c0, whole, nparts, clamped, max_n, B, t_min, num_splits);
}

// ---------------------------------------------------------------------------
// 2. Split kernel
// ---------------------------------------------------------------------------
template <int OFF>
__device__ __forceinline__ void ds_write8(uint32_t addr, const u32x2& v) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    asm volatile("ds_write_b64 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF));
}

struct DecodeCtx {
    const __bf16* q_lat;
    const __bf16* q_rope;
    const __bf16* cache;
    int* ws;
    const int* seqlens;
    __bf16* o_part;
    float* lse_part;
    __bf16* o;
    float* lse;
    int H, S_max;
    float c_log2;
    PlanArgs a;
    // In-kernel plan (fused = 1): the plan kernel's arguments.
    int fused, B, parts, c0, t_min, num_splits;
    // Value up-projection mode (vmode = 1): every piece, split or not, writes
    // its partial to slot b + p; the merge happens in the up-projection.
    int vmode;
};

// Copy one 32-token tile to LDS: copy i (0..36) of 64 chunks is issued by
// wave i % 4.  Chunk L of the tile is row L / 74, chunk L % 74 of that row;
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

// Wait until this wave's copies of the oldest in-flight tile have landed,
// leaving `later` younger tiles in flight.
template <int LATER>
__device__ __forceinline__ void dec_wait_tile(int w) {
    if (w < DEC_LOADS_EXTRA) wait_vmcnt<LATER * DEC_LOADS_HI>();
    else wait_vmcnt<LATER * DEC_LOADS_LO>();
}

// Tile barrier.  Every wave has waited for its own copies of the tile that
// becomes readable; LDS reads still in flight are fragment prefetches of the
// previous tile, which no copy overwrites before the next barrier, so they
// are not drained here.
__device__ __forceinline__ void dec_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
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

// Score MFMAs with VGPR accumulators.  mfma_v0: D = A B (C = 0); mfma_v:
// D += A B.  Early-clobber on the first keeps D from overlapping the sources.
__device__ __forceinline__ void mfma_v0(f32x4& d, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x4& d, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// The value accumulators live in fixed AGPRs: block k (= dim block * 2 +
// head block) in a[4k .. 4k+3].  The compiler does not manage them at all
// (it would keep VGPR copies of all 256 when any element is touched); every
// access below names the registers itself, and acc_zero_all(), run at the
// start of every piece, declares all 256 AGPRs clobbered so that the kernel
// reserves them.
__device__ __forceinline__ void acc_zero_all() {
    asm volatile(
        ".set .Lacc_i, 0\n\t"
        ".rept 256\n\t"
        "v_accvgpr_write_b32 a[.Lacc_i], 0\n\t"
        ".set .Lacc_i, .Lacc_i + 1\n\t"
        ".endr"
        :
        :
        : MLA_ALL_AGPRS);
}
template <int K>
__device__ __forceinline__ void acc_mfma(const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 a[%2:%3], %0, %1, a[%2:%3]" : : "v"(a), "v"(b), "i"(4 * K), "i"(4 * K + 3));
}
template <int K>
__device__ __forceinline__ void acc_scale(float s) {  // a[4K..4K+3] *= s
    float t0, t1, t2, t3;
    asm volatile(
        "v_accvgpr_read_b32 %0, a[%4]\n\tv_accvgpr_read_b32 %1, a[%5]\n\t"
        "v_accvgpr_read_b32 %2, a[%6]\n\tv_accvgpr_read_b32 %3, a[%7]\n\t"
        "v_mul_f32_e32 %0, %0, %8\n\tv_mul_f32_e32 %1, %1, %8\n\t"
        "v_mul_f32_e32 %2, %2, %8\n\tv_mul_f32_e32 %3, %3, %8\n\t"
        "v_accvgpr_write_b32 a[%4], %0\n\tv_accvgpr_write_b32 a[%5], %1\n\t"
        "v_accvgpr_write_b32 a[%6], %2\n\tv_accvgpr_write_b32 a[%7], %3"
        : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
        : "i"(4 * K), "i"(4 * K + 1), "i"(4 * K + 2), "i"(4 * K + 3), "v"(s));
}
template <int K>
__device__ __forceinline__ f32x4 acc_get() {
    float t0, t1, t2, t3;
    asm volatile(
        "v_accvgpr_read_b32 %0, a[%4]\n\tv_accvgpr_read_b32 %1, a[%5]\n\t"
        "v_accvgpr_read_b32 %2, a[%6]\n\tv_accvgpr_read_b32 %3, a[%7]"
        : "=v"(t0), "=v"(t1), "=v"(t2), "=v"(t3)
        : "i"(4 * K), "i"(4 * K + 1), "i"(4 * K + 2), "i"(4 * K + 3));
    return f32x4{t0, t1, t2, t3};
}
// Wait states before ordinary instructions read registers that an MFMA just
// wrote (more than the 16x16x32 bf16 MFMA's pass count needs).
__device__ __forceinline__ void mfma_result_wait() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }

// Max of a lane's eight scores of one head (two MFMA results), and the max
// over the four lanes that hold the same head.  Written out because the
// compiler canonicalises every operand of fmaxf that it did not produce
// itself (one extra v_max per score).
__device__ __forceinline__ float dec_max8(const f32x4& a, const f32x4& b) {
    float t;
    asm("v_max3_f32 %0, %1, %2, %3\n\t"
        "v_max3_f32 %0, %0, %4, %5\n\t"
        "v_max3_f32 %0, %0, %6, %7\n\t"
        "v_max_f32_e32 %0, %0, %8"
        : "=&v"(t)
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]));
    return t;
}
__device__ __forceinline__ float dec_max_heads(float x) {
    uint32_t u = __float_as_uint(x);
    auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    float y;
    asm("v_max_f32_e32 %0, %1, %2" : "=v"(y) : "v"(p[0]), "v"(p[1]));
    u = __float_as_uint(y);
    auto q = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    asm("v_max_f32_e32 %0, %1, %2" : "=v"(y) : "v"(q[0]), "v"(q[1]));
    return y;
}

// Schedule of one tile step.  A step runs the value product of the previous
// tile (32 dim blocks, "V" groups: two transposed reads and two MFMAs each)
// and the scores of the current tile (18 k-steps, "K" groups: two reads and
// four MFMAs each).  Group t's reads are issued DEC_D groups ahead, during
// the MFMAs of group t - DEC_D.  A step with both products runs DEC_LEAD V
// groups first (their reads are issued by the step before, across the tile
// barrier, where that tile is already resident), then the 18 K groups with
// DEC_NVK V groups spread evenly among them, then the remaining V groups,
// over which the softmax of the tile is spread, one slice on every second
// MFMA (those slots already carry a fragment read, and a wave issues only
// about two other instructions in the shadow of one MFMA).  Steps without scores (the
// last of a piece) or without values (the first) keep only the groups they
// have.  The constants were chosen by measurement on MI355X (B=256, H=128,
// varlen cache): prefetch 4 groups, 9 V groups among the K groups (6 and 12
// measured within 1%), softmax slices two MFMAs apart (2% faster than one).
constexpr int DEC_NK = kRow / 32;    // 18
constexpr int DEC_NV = kLatent / 16; // 32
constexpr int DEC_D = 4;
constexpr int DEC_LEAD = 4;
constexpr int DEC_NVK = 9;
constexpr int DEC_SMX_AT = 1;        // softmax starts at the first MFMA of group last_k + 1
constexpr int DEC_SMX_STRIDE = 2;    // MFMA slots from one softmax slice to the next
static_assert(DEC_LEAD >= DEC_D && 2 * (DEC_D - 1) < 16, "prefetch across the barrier; lgkmcnt range");
// The softmax reads the tile's scores, which are complete only after the
// MFMAs of the last K group: its first slice must come after that group
// (with DEC_SMX_AT = 0 it would read unfinished accumulators).
static_assert(DEC_SMX_AT >= 1, "softmax after the last score MFMA");
static_assert(DEC_LEAD + DEC_NVK <= DEC_NV, "V groups");
// Fragment registers are named per group (one name per group of a step):
// every read is a new value, so the names cost no registers, and the V
// groups that one step prefetches for the next keep the names the next
// step reads.
constexpr int DEC_RK = DEC_NK;
constexpr int DEC_RV = DEC_NV;

struct DecTab {
    int kind[DEC_NK + DEC_NV];
    int idx[DEC_NK + DEC_NV];
    int slot0[DEC_NK + DEC_NV];  // MFMA slots before group t
    int kpos[DEC_NK + DEC_NV];   // K groups before group t
    int n, last_k, nslots;
};
constexpr DecTab dec_make_tab(bool hk, bool hv) {
    DecTab t{};
    int n = 0, v = 0;
    auto put = [&](int kind, int i) { t.kind[n] = kind; t.idx[n] = i; ++n; };
    if (hk && hv) {
        for (; v < DEC_LEAD; ++v) put(1, v);
        for (int k = 0; k < DEC_NK; ++k) {
            put(0, k);
            t.last_k = n - 1;
            for (const int target = DEC_LEAD + (k + 1) * DEC_NVK / DEC_NK; v < target; ++v) put(1, v);
        }
        for (; v < DEC_NV; ++v) put(1, v);
    } else if (hk) {
        for (int k = 0; k < DEC_NK; ++k) put(0, k);
        t.last_k = n - 1;
    } else {
        for (; v < DEC_NV; ++v) put(1, v);
        t.last_k = -1;
    }
    t.n = n;
    int sl = 0, kp = 0;
    for (int i = 0; i < n; ++i) {
        t.slot0[i] = sl;
        t.kpos[i] = kp;
        sl += t.kind[i] == 0 ? 4 : 2;
        kp += t.kind[i] == 0 ? 1 : 0;
    }
    t.nslots = sl;
    return t;
}
template <bool HK, bool HV>
struct DecSched {
    static constexpr DecTab tab = dec_make_tab(HK, HV);
    static constexpr int NG = tab.n;
    static constexpr int kind(int t) { return tab.kind[t]; }
    static constexpr int index(int t) { return tab.idx[t]; }
    static constexpr int last_k() { return tab.last_k; }
    static constexpr int slot0(int t) { return tab.slot0[t]; }
    static constexpr int kpos(int t) { return tab.kpos[t]; }
    static constexpr int nslots = tab.nslots;
};

struct DecState {
    bf16x8 qf[2][DEC_NK];        // q fragments of the wave's two head blocks
    bf16x8 fk[DEC_RK][2];        // K-group fragments (tokens 0..15 and 16..31)
    bf16x4 fvl[DEC_RV], fvh[DEC_RV];  // V-group fragments (tokens 0..15 and 16..31)
    bf16x8 pb[2];                // P^T of the previous tile, per head block
    bf16x8 pnext[2];             // P^T of the current tile
    float m[2], l[2], alpha[2];  // exponent base, row-sum share, pending rescale
    bool resc;                   // a rescale is pending for the accumulators
};

// A workgroup whose head block is partial (H not a multiple of 128) computes
// all eight 16-head blocks: missing heads get q = 0 and are never stored, so
// the loops carry no head guards.
__device__ void dec_piece(const DecodeCtx& x, char* smem, int p, int b, int tile_lo, int tile_hi, int len,
                          int nsplit, bool first_in_part) {
    const int w = wave_id();
    // Redefined per piece so that lane-derived addresses are recomputed here
    // instead of being hoisted out of the piece loop.
    int lane = lane_id();
    asm volatile("" : "+v"(lane));
    const int n = lane & 15;  // head column of the MFMA results / MFMA row of the A operand
    const int g = lane >> 4;  // row group (0..3)
    const int H = x.H;
    const int hblk = blockIdx.y * kDecodeHeadsPerWG;
    const int nhb = min(DEC_HB, (H - hblk) >> 4);  // existing 16-head blocks (H % 16 == 0)
    const int tok_end = min(tile_hi * kDecodeTile, len);
    const int tok_lo = tile_lo * kDecodeTile;
    const int ntiles = (tok_end - tok_lo + DEC_TILE - 1) / DEC_TILE;

    DecState st;
    // q fragments (B operand of S^T = C q^T) of head blocks 2w and 2w+1: lane
    // (head n, g) holds dims 32kk+8g..+7.  Missing heads read as zeros.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const bool act = 2 * w + h < nhb;
        const size_t row = (size_t)b * H + hblk + 16 * (2 * w + h) + n;
        const bf16x8* ql = reinterpret_cast<const bf16x8*>(x.q_lat + row * kLatent);
        const bf16x8* qr = reinterpret_cast<const bf16x8*>(x.q_rope + row * kRope);
#pragma unroll
        for (int kk = 0; kk < kLatent / 32; ++kk) st.qf[h][kk] = act ? ql[4 * kk + g] : bf16x8{};
#pragma unroll
        for (int kk = 0; kk < kRope / 32; ++kk) st.qf[h][kLatent / 32 + kk] = act ? qr[4 * kk + g] : bf16x8{};
    }

    const __bf16* seq = x.cache + (size_t)b * x.S_max * kRow;
    uint32_t voff[DEC_LOADS_HI];
    dec_copy_offsets(voff, w, lane);
    // (the first DEC_AHEAD tiles are copied below, once tile_rsrc exists)

    acc_zero_all();  // value accumulators: block (i, h) = dims 16i.., heads 16(2w+h)..
#pragma unroll
    for (int h = 0; h < 2; ++h) { st.m[h] = -INFINITY; st.l[h] = 0.f; st.alpha[h] = 1.f; }
    st.resc = false;

    // Per-lane LDS addresses; everything else is a compile-time immediate.
    const uint32_t smem_a = lds_addr(smem);
    const uint32_t qk_off = dec_pi16(n) * DEC_ROW_STRIDE + 16 * g;
    const int jj = n >> 2, qd = n & 3;  // ds_read_b64_tr_b16 source lane = 4*jj + qd
    const uint32_t pv_off = dec_pi16(4 * g + jj) * DEC_ROW_STRIDE + 8 * qd;

    // One fragment read: half 0 / 1 of group u of a step (tokens 0..15 / 16..31).
    auto rd_k = [&](uint32_t qk_a, auto kk_c, auto half_c) {
        constexpr int kk = decltype(kk_c)::value, half = decltype(half_c)::value;
        st.fk[kk][half] = ds_read16<half * 16 * DEC_ROW_STRIDE + 64 * kk>(qk_a);
    };
    auto rd_v = [&](uint32_t pv_a, auto i_c, auto half_c) {
        constexpr int i = decltype(i_c)::value, half = decltype(half_c)::value;
        if constexpr (half == 0) st.fvl[i] = ds_read_tr16<32 * i>(pv_a);
        else st.fvh[i] = ds_read_tr16<16 * DEC_ROW_STRIDE + 32 * i>(pv_a);
    };

    // One step: value product of the tile at pv_a (if HV), scores and softmax
    // of the tile at qk_a (if HK), and (if HK and dma) the copies of a later
    // tile into dst.  Each MFMA is followed by at most one fragment read or
    // copy, and in the softmax region every second MFMA also by one slice of
    // the softmax, so that the work issues while the matrix pipe is busy: a
    // wave issues in order, and work bunched between two MFMAs holds the next
    // MFMA back.  Group t
    // issues the reads of group t + DEC_D after its first two MFMAs; on entry
    // the first DEC_D groups' reads are in flight (issued by the previous
    // step, or by the caller for the first), and a step with scores leaves
    // the next step's first DEC_D groups (V groups of the tile at nv_a) in
    // flight.
    constexpr int NPIECE = 18;  // softmax slices: two for the max/rescale, sixteen exponentials
    auto step = [&](auto hk_c, auto hv_c, uint32_t qk_a, uint32_t pv_a, uint32_t nv_a, int valid,
                    __amdgpu_buffer_rsrc_t rsrc, char* dst) {
        constexpr bool HK = decltype(hk_c)::value, HV = decltype(hv_c)::value;
        using Sch = DecSched<HK, HV>;
        constexpr int NG = Sch::NG;
        if constexpr (HV) {
            if (st.resc) {  // wave-uniform; the previous value product has finished
                mfma_result_wait();
                static_for<DEC_NV>([&](auto i_c) {
                    constexpr int i = decltype(i_c)::value;
                    acc_scale<2 * i>(st.alpha[0]);
                    acc_scale<2 * i + 1>(st.alpha[1]);
                });
                asm volatile("s_nop 4");  // accumulator writes before the next MFMA reads them
            }
        }
        f32x4 s[2][2];  // s[token half][head block]
        float lm[2];    // this lane's max of the tile's scores, per head block

        auto issue_read = [&](auto u_c, auto half_c) {
            constexpr int u = decltype(u_c)::value;
            if constexpr (u < NG) {
                if constexpr (Sch::kind(u) == 0) rd_k(qk_a, std::integral_constant<int, Sch::index(u)>{}, half_c);
                else rd_v(pv_a, std::integral_constant<int, Sch::index(u)>{}, half_c);
            } else if constexpr (HK) {
                rd_v(nv_a, std::integral_constant<int, u - NG>{}, half_c);
            }
        };
        auto piece = [&](auto p_c) {
            constexpr int p = decltype(p_c)::value;
            if constexpr (p == 0) {
                mfma_result_wait();
                if (valid < DEC_TILE) {  // the sequence's last tile; kept as a branch
                    asm volatile("");
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if (dec_token_of(g, r) >= valid) s[0][h][r] = -INFINITY;
                            if (dec_token_of(g, 4 + r) >= valid) s[1][h][r] = -INFINITY;
                        }
                }
                lm[0] = dec_max8(s[0][0], s[1][0]);
            } else if constexpr (p == 1) {
                lm[1] = dec_max8(s[0][1], s[1][1]);
                // The base only moves when some head's max exceeds it by more
                // than kRescaleSlack (always on the first tile, where m = -inf:
                // every tile has at least one valid token, so the new base is
                // finite and alpha = exp2(-inf) = 0); the accumulators are then
                // scaled by alpha before the next value product.  Each lane
                // tests its own max: x -> fl(x c_log2) is monotone (c_log2 > 0),
                // so some lane of a head passes exactly when the head's max
                // (over its four lanes) does, and the cross-lane max is only
                // taken when the base moves.
                const bool grow = (lm[0] * x.c_log2 > st.m[0] + kRescaleSlack) ||
                                  (lm[1] * x.c_log2 > st.m[1] + kRescaleSlack);
                st.resc = __builtin_amdgcn_ballot_w64(grow) != 0;
                st.alpha[0] = st.alpha[1] = 1.f;
                if (st.resc) {
                    asm volatile("");
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float mt = dec_max_heads(lm[h]) * x.c_log2;  // the head's max (log2 units)
                        const float m_new = fmaxf(st.m[h], mt);
                        st.alpha[h] = fast_exp2(st.m[h] - m_new);
                        st.l[h] *= st.alpha[h];
                        st.m[h] = m_new;
                    }
                }
            } else {
                constexpr int q = p - 2, h = q >> 3, r = (q >> 1) & 3, half = q & 1;
                const float e = fast_exp2(__builtin_fmaf(s[half][h][r], x.c_log2, -st.m[h]));
                st.l[h] += e;
                st.pnext[h][4 * half + r] = to_bf16(e);  // logical k = 8g + e
            }
        };
        // Slot of the first softmax slice: the first MFMA of group
        // last_k + DEC_SMX_AT (steps with values); steps without values run
        // the softmax after their last MFMA.
        constexpr int smx0 = HV && HK ? Sch::slot0(Sch::last_k() + DEC_SMX_AT) : 1 << 20;
        static_assert(!(HV && HK) || smx0 + DEC_SMX_STRIDE * (NPIECE - 1) < Sch::nslots, "softmax slices fit in the step");

        static_for<NG>([&](auto t_c) {
            constexpr int t = decltype(t_c)::value;
            constexpr int idx = Sch::index(t);
            constexpr int kind = Sch::kind(t);
            constexpr int nm = kind == 0 ? 4 : 2;
            constexpr int newer = HK ? 2 * (DEC_D - 1) : 2 * (NG - 1 - t < DEC_D - 1 ? NG - 1 - t : DEC_D - 1);
            if constexpr (kind == 0) wait_lgkm_for<newer>(st.fk[idx][0], st.fk[idx][1]);
            else wait_lgkm_for<newer>(st.fvl[idx], st.fvh[idx]);
            static_for<nm>([&](auto m_c) {
                constexpr int m = decltype(m_c)::value;
                if constexpr (kind == 0) {
                    const bf16x8& f = st.fk[idx][m >> 1];
                    const bf16x8& q = st.qf[m & 1][idx];
                    f32x4& acc = s[m >> 1][m & 1];
                    if constexpr (idx == 0) mfma_v0(acc, f, q);
                    else mfma_v(acc, f, q);
                } else {
                    acc_mfma<2 * idx + m>(join(st.fvl[idx], st.fvh[idx]), st.pb[m]);
                }
                if constexpr (m < 2) {
                    issue_read(std::integral_constant<int, t + DEC_D>{}, std::integral_constant<int, m>{});
                } else if constexpr (HK) {
                    constexpr int c = 2 * Sch::kpos(t) + (m - 2);  // copy number of this slot
                    static_assert(kind == 0 && m >= 2 && c >= 0, "copies sit in the last two slots of K groups");
                    if constexpr (c < DEC_LOADS_LO) {
                        bload_lds16_stream(rsrc, dst + (w + DEC_WAVES * c) * 1024, voff[c]);
                    } else if constexpr (c < DEC_LOADS_HI) {
                        if (w < DEC_LOADS_EXTRA) bload_lds16_stream(rsrc, dst + (w + DEC_WAVES * c) * 1024, voff[c]);
                    }
                }
                constexpr int d = Sch::slot0(t) + m - smx0;
                if constexpr (d >= 0 && d % DEC_SMX_STRIDE == 0 && d / DEC_SMX_STRIDE < NPIECE)
                    piece(std::integral_constant<int, d / DEC_SMX_STRIDE>{});
                __builtin_amdgcn_sched_barrier(0);  // keep each slot's work in its place
            });
        });
        if constexpr (HK && !HV) static_for<NPIECE>([&](auto p) { piece(p); });
        if constexpr (HK) {
            st.pb[0] = st.pnext[0];
            st.pb[1] = st.pnext[1];
        }
    };

    // Tile j is read as keys in step j and as values in step j + 1.  At the
    // top of step j (< ntiles) every wave waits for its copies of tile j and
    // passes the barrier; step j then copies tile j + 2 into the slot of tile
    // j - 2, whose value product finished in step j - 1.
    auto top = [&](int j) {
        dec_wait_tile<1>(w);  // tile j has landed; tile j + 1 (real or empty) may still be in flight
        dec_barrier();
    };
    auto tile_a = [&](int j) { return smem_a + (uint32_t)((j % DEC_NBUF) * DEC_TILE_BYTES); };
    // Buffer of tile j's rows; a tile past the piece's end gets an empty
    // buffer, whose copies write zeros into a slot that nothing reads, so the
    // copies need no branch and the per-tile copy counts stay fixed.
    auto tile_rsrc = [&](int j) {
        const int tok0 = tok_lo + j * DEC_TILE;
        const uint32_t bytes = j < ntiles ? (uint32_t)(len - tok0) * (uint32_t)(kRow * 2) : 0u;
        return make_rsrc(seq + (size_t)(j < ntiles ? tok0 : 0) * kRow, bytes);
    };

#pragma unroll
    for (int i = 0; i < DEC_AHEAD; ++i) {
        const auto r = tile_rsrc(i);
        static_for<DEC_LOADS_HI>([&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            if (k < DEC_LOADS_LO || w < DEC_LOADS_EXTRA) bload_lds16_stream(r, smem + i * DEC_TILE_BYTES + (w + DEC_WAVES * k) * 1024, voff[k]);
        });
    }
    top(0);
    {
        const uint32_t qa = tile_a(0) + qk_off;
        static_for<DEC_D>([&](auto i) {
            rd_k(qa, i, std::integral_constant<int, 0>{});
            rd_k(qa, i, std::integral_constant<int, 1>{});
        });
        step(std::true_type{}, std::false_type{}, qa, 0u, tile_a(0) + pv_off, tok_end - tok_lo, tile_rsrc(DEC_AHEAD),
             smem + (DEC_AHEAD % DEC_NBUF) * DEC_TILE_BYTES);
        // The first tile always moves the exponent base (from -inf), but the
        // accumulators are still zero: the rescale by alpha = 0 would leave
        // them unchanged, so it is skipped (256 AGPR reads, multiplies and
        // writes per wave and piece).
        st.resc = false;
    }
    for (int j = 1; j < ntiles; ++j) {
        top(j);
        step(std::true_type{}, std::true_type{}, tile_a(j) + qk_off, tile_a(j - 1) + pv_off, tile_a(j) + pv_off,
             tok_end - (tok_lo + j * DEC_TILE), tile_rsrc(j + DEC_AHEAD), smem + ((j + DEC_AHEAD) % DEC_NBUF) * DEC_TILE_BYTES);
    }
    step(std::false_type{}, std::true_type{}, 0u, tile_a(ntiles - 1) + pv_off, 0u, 0, tile_rsrc(0), smem);

    // Normalise and store.  O^T block (i, h) holds dims 16i + 4g + 0..3 of
    // head 16(2w+h) + n.  The rows go through LDS (the ring is free once
    // this piece's last copies have landed and every wave has finished its
    // last value product), so that each global store writes one whole 1 KB
    // head row.  Staging row stride 1040 B: the 8-byte writes of 32 lanes
    // (16 heads x 2 lane groups) then hit 64 distinct banks.
    wait_vmcnt<0>();
    lds_barrier();
    mfma_result_wait();  // the accumulators are read below
    constexpr int STG = 1040;
    static_assert(DEC_WAVES * 32 * STG <= DEC_SMEM, "staging fits in the ring");
    const uint32_t stg = smem_a + (uint32_t)(w * 32 * STG);
    static_for<2>([&](auto h_c) {
        constexpr int h = decltype(h_c)::value;
        const bool act = 2 * w + h < nhb;
        const float lsum = sum4_groups16(st.l[h]);
        const float il = 1.f / lsum;
        const int head = hblk + 16 * (2 * w + h) + n;
        if (act && g == 0) {
            const float lse_v = (st.m[h] + __builtin_log2f(lsum)) * kLn2;
            if (nsplit == 1 && !x.vmode) {
                if (x.lse) x.lse[(size_t)b * H + head] = lse_v;
            } else {
                const int slot = x.vmode ? b + p : 2 * p + (first_in_part ? 0 : 1);
                x.lse_part[(size_t)slot * H + head] = lse_v;
            }
        }
        uint32_t wa = stg + (uint32_t)((16 * h + n) * STG + 8 * g);
        static_for<DEC_NV>([&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            const f32x4 v = acc_get<2 * i + h>();
            bf16x4 t;
#pragma unroll
            for (int r = 0; r < 4; ++r) t[r] = to_bf16(v[r] * il);
            const u32x2 u = __builtin_bit_cast(u32x2, t);
            ds_write8<32 * i>(wa, u);
        });
    });
    wait_lgkm<0>();
    // Row r of the wave's staging area is head hblk + 32w + r.
    __bf16* obase;
    if (nsplit == 1 && !x.vmode) {
        obase = x.o + ((size_t)b * H + hblk + 32 * w) * kLatent;
    } else {
        const int slot = x.vmode ? b + p : 2 * p + (first_in_part ? 0 : 1);
        obase = x.o_part + ((size_t)slot * H + hblk + 32 * w) * kLatent;
    }
    const uint32_t ra = stg + (uint32_t)(16 * lane);
    static_for<2>([&](auto h_c) {
        constexpr int h = decltype(h_c)::value;
        if (2 * w + h < nhb) {
            u32x4 rowv[16];
            static_for<16>([&](auto r_c) {
                constexpr int r = decltype(r_c)::value;
                rowv[r] = ds_read_u32x4<(16 * h + r) * STG>(ra);
            });
            wait_lgkm<0>();
            static_for<16>([&](auto r_c) {
                constexpr int r = decltype(r_c)::value;
                *reinterpret_cast<u32x4*>(obase + (size_t)(16 * h + r) * kLatent + 8 * lane) = rowv[r];
            });
        }
    });
    // The next piece copies into the ring: every wave's staging reads first.
    lds_barrier();
}

// Workgroups are dealt to the eight XCDs round-robin by id, and each XCD has
// its own L2.  Part p of the plan runs on the workgroup whose id places
// consecutive parts on one XCD: XCD x takes the parts
// [x q + min(x, r), ...) with q = n / 8, r = n % 8, so the parts that share a
// sequence (and its query block) mostly share an L2.  Only the speed depends
// on the dealing order; any bijection gives the same results.
__host__ __device__ constexpr int xcd_part(int id, int n) {
    const int x = id & 7, k = id >> 3, q = n >> 3, r = n & 7;
    return x * q + (x < r ? x : r) + k;
}
constexpr bool xcd_part_is_bijection(int n) {
    bool seen[kPlanMaxParts] = {};
    for (int id = 0; id < n; ++id) {
        const int p = xcd_part(id, n);
        if (p < 0 || p >= n || seen[p]) return false;
        seen[p] = true;
    }
    return true;
}
static_assert(xcd_part_is_bijection(1) && xcd_part_is_bijection(7) && xcd_part_is_bijection(8) &&
                  xcd_part_is_bijection(10) && xcd_part_is_bijection(255) && xcd_part_is_bijection(256) &&
                  xcd_part_is_bijection(1000) && xcd_part_is_bijection(kPlanMaxParts),
              "part mapping");

// LDS after the tile ring: the in-kernel plan's per-sequence n, start and
// len (PLAN_CHUNK each); read by the piece loop for the whole kernel.
constexpr int DEC_PLAN_LDS = 3 * PLAN_CHUNK * 4;
constexpr int DEC_SMEM_TOTAL = DEC_SMEM + DEC_PLAN_LDS;
static_assert(DEC_SMEM_TOTAL <= 160 * 1024, "LDS");
static_assert(PLAN_THREADS == DEC_THREADS, "the split workgroup runs the plan scan");

// In-kernel plan (line mode, B <= PLAN_CHUNK): every workgroup scans the
// lengths into LDS.  Returns (block-uniform) t, parts_used and the first
// sequence of part p; workgroup (0, 0) also writes the whole plan to the
// workspace, as the plan kernel would, for the combine kernel.  Uses the
// start of the ring as scratch; a barrier ends it before any tile copy.
__device__ void dec_plan_in_kernel(const DecodeCtx& x, char* smem, int p, int& t, int& parts_used, int& b0) {
    int* l_n = reinterpret_cast<int*>(smem + DEC_SMEM);
    int* l_start = l_n + PLAN_CHUNK;
    int* l_len = l_start + PLAN_CHUNK;
    int* s_red = reinterpret_cast<int*>(smem);    // 12 ints
    int* s_b0 = s_red + 12;                       // 1 int
    int* s_pfs = s_red + 16;                      // parts ints (workgroup 0)
    const int tid = threadIdx.x, B = x.B, c0 = x.c0;
    int n[PLAN_PER], len[PLAN_PER], start[PLAN_PER];
    const ChunkScan cs = plan_scan_chunk(x.seqlens, 0, B, x.S_max, c0, 0, n, len, start, s_red);
    const int C = cs.total;
    t = plan_line_t(C, x.parts, cs.max_n, x.num_splits, x.t_min);
    parts_used = (C + t - 1) / t;
    const bool writer = blockIdx.x == 0 && blockIdx.y == 0;
    if (tid == 0) *s_b0 = B;
    if (writer)
        for (int q = tid; q < x.parts; q += PLAN_THREADS) s_pfs[q] = B;
    lds_barrier();
#pragma unroll
    for (int k = 0; k < PLAN_PER; ++k) {
        const int b = PLAN_PER * tid + k;
        if (b >= B) continue;
        l_n[b] = n[k];
        l_start[b] = start[k];
        l_len[b] = len[k];
        const int first = n[k] > 0 ? start[k] / t : 0;
        const int ns = n[k] > 0 ? (start[k] + n[k] - 1) / t - first + 1 : 0;
        if (ns > 0 && first <= p && p < first + ns) atomicMin(s_b0, b);
        if (writer) {
            int* ws = x.ws;
            ws[x.a.seq_len + b] = len[k];
            ws[x.a.seq_n + b] = n[k];
            ws[x.a.seq_start + b] = start[k];
            ws[x.a.seq_first + b] = first;
            ws[x.a.seq_nsplit + b] = ns;
            for (int q = first; q < first + ns; ++q) atomicMin(&s_pfs[q], b);
        }
    }
    lds_barrier();
    b0 = *s_b0;
    if (writer) {
        for (int q = tid; q < x.parts; q += PLAN_THREADS) x.ws[x.a.part_first_seq + q] = s_pfs[q];
        if (tid == 0)
            plan_write_header(x.ws, parts_used, t, C, c0, false, x.parts, cs.clamped, cs.max_n, B, x.t_min,
                              x.num_splits);
    }
    lds_barrier();  // the ring's scratch is free again (the plan record's stores need not have landed)
}

// Pieces of part p, found without a chain of dependent loads: lane i reads
// the plan entries of sequence b0 + i (b0 = the part's first sequence) in one
// round trip, and a ballot lists the lanes whose sequence has tiles in the
// part.  Only the ballot mask stays live across pieces; each piece re-reads
// its sequence's entries.  A part spans more than 64 sequences only when
// they are very short; then the next 64 are read the same way.  The plan
// entries come from LDS (in-kernel plan) or from the workspace.
__global__ __launch_bounds__(DEC_THREADS, 1) void mla_split_kernel(DecodeCtx x) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int p = xcd_part(blockIdx.x, gridDim.x);
    const int* pl_n;
    const int* pl_start;
    const int* pl_len;
    int t, parts_used, b0, B, whole;
    if (x.fused) {
        dec_plan_in_kernel(x, smem, p, t, parts_used, b0);
        B = x.B;
        whole = 0;
        pl_n = reinterpret_cast<const int*>(smem + DEC_SMEM);
        pl_start = pl_n + PLAN_CHUNK;
        pl_len = pl_start + PLAN_CHUNK;
    } else {
        const int* ws = x.ws;
        parts_used = ws[kHdrPartsUsed];
        t = ws[kHdrT];
        whole = ws[kHdrMode];
        B = ws[kHdrB];
        b0 = p < parts_used ? ws[x.a.part_first_seq + p] : B;
        pl_n = ws + x.a.seq_n;
        pl_start = ws + x.a.seq_start;
        pl_len = ws + x.a.seq_len;
    }
    if (p >= parts_used) return;
    const int pos_lo = p * t, pos_hi = pos_lo + t;
    const int lane = lane_id();
    for (int base = b0; base < B; base += 64) {
        uint64_t pieces, more;
        {
            const int b = base + lane;
            int nb = 0, sb = pos_hi;
            if (b < B && (!whole || b == b0)) {
                nb = pl_n[b];
                sb = pl_start[b];
            }
            pieces = __builtin_amdgcn_ballot_w64(nb > 0 && max(sb, pos_lo) < min(sb + nb, pos_hi));
            more = __builtin_amdgcn_ballot_w64(nb > 0 && sb >= pos_hi);
        }
        while (pieces) {
            const int i = __builtin_ctzll(pieces);
            pieces &= pieces - 1;
            const int b = __builtin_amdgcn_readfirstlane(base + i);
            const int nb = __builtin_amdgcn_readfirstlane(pl_n[b]);
            const int sb = __builtin_amdgcn_readfirstlane(pl_start[b]);
            const int ln = __builtin_amdgcn_readfirstlane(pl_len[b]);
            const int first = sb / t;
            const int ns = whole ? 1 : (sb + nb - 1) / t - first + 1;
            const int lo = max(sb, pos_lo) - sb, hi = min(sb + nb, pos_hi) - sb;
            dec_piece(x, smem, p, b, lo, hi, ln, ns, b == b0);
        }
        if (more != 0 || base + 64 >= B || whole) break;
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

// rows(s) gives the row index of split s in lse_part (and, times 512, in o_part).
template <typename PT, typename RowFn>
__device__ __forceinline__ void combine_head(const PT* o_part, const float* lse_part, int nsplit, RowFn rows,
                                             __bf16* o_row, float* lse_out, int d8) {
    const MergeRow mr = merge_row_init(lse_part, nsplit, rows);
    *reinterpret_cast<bf16x8*>(o_row + 8 * d8) = merge_dims8(o_part, lse_part, nsplit, rows, d8, mr);
    if (lse_out && d8 == 0) *lse_out = mr.lse;
}

// Partials of the split kernel: slot-major [slots][H][512] bf16, lse [slots][H].
__global__ __launch_bounds__(CMB_THREADS) void mla_combine_slots_kernel(const int* __restrict__ ws,
                                                                       const __bf16* __restrict__ o_part,
                                                                       const float* __restrict__ lse_part,
                                                                       __bf16* __restrict__ o, float* lse, int H,
                                                                       PlanArgs a) {
    const int b = blockIdx.x;
    // All plan words are loaded before any of them is used: one round trip.
    const int ns = ws[a.seq_nsplit + b];
    const int first = ws[a.seq_first + b];
    const int start = ws[a.seq_start + b];
    const int c0 = ws[kHdrC0], t = ws[kHdrT];
    if (ns == 1) return;
    const int hh = blockIdx.y * CMB_HEADS + (threadIdx.x >> 6);
    if (hh >= H) return;
    const int d8 = threadIdx.x & 63;
    // Part `first` may begin with an earlier sequence (then b's piece is in
    // its second slot); every later part of b begins inside b, so b's piece
    // there is in the part's first slot.  No earlier sequence has tiles in
    // part `first` exactly when b's range on the cost line, which begins c0
    // positions before its first tile, begins at or before the part does.
    const int slot0 = 2 * first + (start - c0 <= first * t ? 0 : 1);
    auto rows = [&](int s) -> size_t { return (size_t)(s == 0 ? slot0 : 2 * (first + s)) * H + hh; };
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

// Workspace of mla_decode_fwd_noalloc: one file-scope device array, so that
// that entry point needs no allocation.  Every device the library runs on
// holds its own copy until the process ends.  In host code `scratch` only
// names the symbol; its device address (per device) comes from
// hipGetSymbolAddress and is the only form passed to kernels.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
    static std::atomic<void*> addr[64];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
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

hipError_t launch_mla_merge_up(const int* ws, int seq_first, int seq_nsplit, const __bf16* o_part,
                               const float* lse_part, const __bf16* w_uv, __bf16* o_v, float* lse, int B, int H,
                               int Dv, hipStream_t stream);

// w_uv == nullptr: the latent decode (plan, split kernel, combine) writing
// o [B, H, 512].  w_uv != nullptr: the same split kernel in value mode, then
// the merge fused with the value up-projection, writing o_v [B, H, Dv].
hipError_t launch_mla_decode(const __bf16* q_lat, const __bf16* q_rope, const __bf16* cache, const int* seqlens,
                             __bf16* o, float* lse, int B, int H, int S_max, float scale, int num_splits,
                             const PlanLayout& L, int c0, int t_min, void* workspace, hipStream_t stream,
                             const __bf16* w_uv, int Dv) {
    hipError_t e = ensure_smem_attr((const void*)mla_split_kernel, DEC_SMEM_TOTAL);
    if (e != hipSuccess) return e;
    int* ws = static_cast<int*>(workspace);
    const PlanArgs a = plan_args(L);
    const bool fused = num_splits >= 2 && B <= PLAN_CHUNK;
    if (!fused)
        hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, seqlens, ws, B, S_max, L.parts,
                           c0, t_min, num_splits, a);
    DecodeCtx x;
    x.seqlens = seqlens;
    x.fused = fused ? 1 : 0;
    x.B = B;
    x.parts = L.parts;
    x.c0 = c0;
    x.t_min = t_min;
    x.num_splits = num_splits;
    x.vmode = w_uv ? 1 : 0;
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
    hipLaunchKernelGGL(mla_split_kernel, dim3(L.parts, hblocks), dim3(DEC_THREADS), DEC_SMEM_TOTAL, stream, x);
    if (w_uv) {
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_mla_merge_up(ws, a.seq_first, a.seq_nsplit, x.o_part, x.lse_part, w_uv, o, lse, B, H, Dv,
                                   stream);
    }
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

