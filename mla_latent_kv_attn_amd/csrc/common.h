// common.h - device primitives shared by the gfx950 kernels of libmla_attn.
//
// Everything here is CDNA4 (gfx950) specific: wave64, bf16 MFMA with eight
// bf16 per lane (v_mfma_f32_16x16x32_bf16 / v_mfma_f32_32x32x16_bf16), the
// transposing LDS read ds_read_b64_tr_b16, direct global->LDS loads
// (global_load_lds_dwordx4), and v_permlane16/32_swap for cross-row
// exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))
#define MLA_GLOBAL __attribute__((address_space(1)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Online softmax keeps an exponent base m (log2 domain) for each row and
// forms p = exp2(s - m).  The base is raised -- and the accumulator and the
// running sum rescaled by exp2(m_old - m_new) -- only when a row's new max
// exceeds the base by more than this slack, so p <= 2^8.  Because l and the
// accumulator always share the same base, O = acc / l and LSE = m + log2(l)
// are unchanged; rescales become rare after the first tiles.
constexpr float kRescaleSlack = 8.f;

// ---------------------------------------------------------------------------
// MFMA.  Operand layouts (verified on the device):
//  16x16x32: A lane l holds row l%16, k = 8*(l/16)+[0..7];
//            B lane l holds col l%16, k = 8*(l/16)+[0..7];
//            D lane l holds col l%16, rows 4*(l/16)+[0..3].
//  32x32x16: A lane l holds row l%32, k = 8*(l/32)+[0..7];
//            B lane l holds col l%32, k = 8*(l/32)+[0..7];
//            D register v of lane l: col l%32, row 8*(v/4)+4*(l/32)+v%4.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS helpers
// ---------------------------------------------------------------------------
// 16-byte LDS read at a byte offset from an LDS base.
__device__ __forceinline__ bf16x8 lds_read16(const char* base, uint32_t byte_off) {
    return *reinterpret_cast<const bf16x8*>(base + byte_off);
}

// ds_read_b64_tr_b16.  Within each group of 16 lanes, lane s supplies the
// address of four consecutive 16-bit elements; result lane i, element j is
// element i%4 of the chunk addressed by lane 4*j + i/4 of the same group.
// Used to fetch a B (or A) MFMA operand whose contraction index runs down
// the rows of a row-major tile: if lane s = 4*j + q of a group points at
// row (r0 + j), columns (c0 + 4q .. c0 + 4q + 3), lane i receives
// rows r0..r0+3 of column c0 + i.
__device__ __forceinline__ bf16x4 lds_read_tr16(const char* base, uint32_t byte_off) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 MLA_LDS*)((MLA_LDS char*)(base) + byte_off));
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 join(const bf16x4& lo, const bf16x4& hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Direct global -> LDS copy of 16 bytes per lane.  The wave's 64 chunks land
// contiguously at lds_wave_base + 16 * lane, whatever global address each
// lane supplies (lane order fixes the LDS position).
__device__ __forceinline__ void gload_lds16(const void* gsrc, void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds((const void MLA_GLOBAL*)gsrc,
                                     (void MLA_LDS*)lds_wave_base, 16, 0, 0);
}

// Raw buffer resource over `bytes` bytes at `base` (stride 0, so the record
// count is a byte count; the fourth descriptor word selects 32-bit data
// format as gfx9 raw buffers require).  Buffer reads at or past `bytes`
// return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer -> LDS copy of 16 bytes per lane from byte offset `voff` of the
// buffer; like gload_lds16, the wave's chunks land at lds_wave_base + 16*lane.
__device__ __forceinline__ void bload_lds16(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void MLA_LDS*)lds_wave_base, 16, (int)voff, 0, 0, 0);
}
// The same copy with the non-temporal cache policy bit (nt): for data read
// exactly once, such as the decode's cache rows, so that the caches keep the
// lines that are read again (queries, split partials) instead.
__device__ __forceinline__ void bload_lds16_stream(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t voff) {
    constexpr int kNonTemporal = 2;  // cache policy operand: nt
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void MLA_LDS*)lds_wave_base, 16, (int)voff, 0, 0, kNonTemporal);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
}

// ---------------------------------------------------------------------------
// Explicitly scheduled LDS fragment reads.
//
// The compiler treats every LDS read as possibly aliasing in-flight
// direct-to-LDS copies and waits for all of them (vmcnt(0)), and it also
// drains every outstanding LDS read (lgkmcnt(0)) before each use.  In the
// tile loops that would serialise the multi-tile copy pipeline and the
// fragment prefetch.  The loops therefore issue their fragment reads with
// these asm forms, which the compiler does not count, and wait for them with
// wait_lgkm<N>() where N is the exact number of reads issued after the one
// being consumed (the issue order is pinned with sched_barrier).  Only LDS
// reads count in lgkmcnt inside those loops: the copies count in vmcnt and
// the loops issue no scalar memory reads.
// ---------------------------------------------------------------------------
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
        (f(std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)((const MLA_LDS char*)(p));
}

template <int OFF>
__device__ __forceinline__ bf16x8 ds_read16(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    bf16x8 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

template <int OFF>
__device__ __forceinline__ bf16x4 ds_read_tr16(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return __builtin_bit_cast(bf16x4, r);
}

template <int OFF>
__device__ __forceinline__ u32x4 ds_read_u32x4(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

template <int OFF>
__device__ __forceinline__ float ds_read_f32(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    float r;
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

// LDS writes in the same explicitly counted form (they count in lgkmcnt).
template <int OFF>
__device__ __forceinline__ void ds_write16(uint32_t addr, const bf16x8& v) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF));
}

template <int OFF>
__device__ __forceinline__ void ds_write_f32(uint32_t addr, float v) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    asm volatile("ds_write_b32 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF));
}

template <int OFF>
__device__ __forceinline__ void ds_write_u32(uint32_t addr, uint32_t v) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    asm volatile("ds_write_b32 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF));
}

template <int N>
__device__ __forceinline__ void wait_lgkm() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (N << 8) | (3 << 14));
}

// The same wait, written so that the values it guards (results of earlier
// asm LDS reads) are operands of it: their consumers then depend on the wait
// and cannot be scheduled ahead of it.  A bare waitcnt gives the compiler no
// such dependency, and it does move arithmetic on asm results above it.
template <int N, typename A>
__device__ __forceinline__ void wait_lgkm_for(A& a) {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%[n])" : "+v"(a) : [n] "n"(N));
}
template <int N, typename A, typename B>
__device__ __forceinline__ void wait_lgkm_for(A& a, B& b) {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%[n])" : "+v"(a), "+v"(b) : [n] "n"(N));
}

// ---------------------------------------------------------------------------
// Cross-lane reductions
// ---------------------------------------------------------------------------
// Max / sum over the four lanes {l, l^16, l^32, l^48} (the four row groups
// of a 16x16 MFMA result).  v_permlane16_swap exchanges lanes l and l^16
// (within each 32-lane half), v_permlane32_swap exchanges l and l^32; each
// returns the pair (own, partner) in some order.
__device__ __forceinline__ float max4_groups16(float x) {
    uint32_t u = __float_as_uint(x);
    auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    u = __float_as_uint(x);
    auto q = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float sum4_groups16(float x) {
    uint32_t u = __float_as_uint(x);
    auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    u = __float_as_uint(x);
    auto q = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
// Max / sum over lanes {l, l^32} (the two row groups of a 32x32 result).
__device__ __forceinline__ float max2_halves(float x) {
    uint32_t u = __float_as_uint(x);
    auto q = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float sum2_halves(float x) {
    uint32_t u = __float_as_uint(x);
    auto q = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Inclusive prefix sum and maximum over the 64 lanes of a wave with DPP row
// shifts (within rows of 16 lanes) and row broadcasts (lane 15 into the next
// row, lane 31 into rows 2 and 3); verified against a host reference on the
// device.  dpp_wave_max returns the maximum in every lane.
__device__ __forceinline__ int dpp_incl_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}
__device__ __forceinline__ int dpp_wave_max(int x) {
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x111, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x112, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x114, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x118, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x142, 0xa, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x143, 0xc, 0xf, false));
    return __builtin_amdgcn_readlane(x, 63);
}

// Workgroup barrier for LDS hand-offs in the tile loops.  The wave's own
// direct-to-LDS copies are waited for explicitly (wait_vmcnt) before it, and
// its LDS reads are drained here (lgkmcnt 0), so no memory fence -- which
// would also drain the next tile's in-flight copies -- is needed.  The empty
// asm statements stop the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// float -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

}  // namespace mla
