// mla_plan.h - workspace layout of the split-KV decode (host and device).
//
// The planner turns per-sequence lengths into a partition of all cache
// tiles over the workgroups of the split kernel (see mla_decode.hip for the
// rule).  Everything the split and combine kernels need is written to the
// caller's workspace by the plan kernel; the host never reads it back.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kDecodeTile = 32;        // cache tokens per plan tile (one LDS tile of the split kernel)
constexpr int kDecodeHeadsPerWG = 128;  // heads one split workgroup serves
constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kRow = kLatent + kRope;  // 576 bf16 per cached token
constexpr int kMaxSplits = 32;
constexpr int kMaxBatch = 1 << 16;
constexpr int kPlanMaxParts = 1024;  // split-kernel parts in line mode (one per CU, capped)
// Fixed device scratch of mla_decode_fwd_noalloc (72 MiB per device).
constexpr size_t kNoAllocScratchBytes = (size_t)72 << 20;

// Header words (int32) at the start of the workspace.
enum PlanWord {
    kHdrPartsUsed = 0,  // parts that hold at least one position
    kHdrT = 1,          // part capacity t, in tiles
    kHdrC = 2,          // cost-line length C
    kHdrTile = 3,       // tokens per tile
    kHdrC0 = 4,         // fixed cost per sequence, in tiles
    kHdrMode = 5,       // 0 = cost line, 1 = one part per sequence
    kHdrParts = 6,      // parts in the grid
    kHdrClamped = 7,    // number of seqlens clamped into [0, S_max]
    kHdrMaxN = 8,       // max tiles of any sequence
    kHdrB = 9,
    kHdrTMin = 10,
    kHdrNumSplits = 11,
    kHdrWords = 64      // header is 256 bytes
};

struct PlanLayout {
    // int32 offsets (in elements) of each array from the workspace start
    size_t seq_len, seq_n, seq_start, seq_first, seq_nsplit, part_first_seq;
    // byte offsets of the partial results (bf16 outputs, fp32 LSE)
    size_t o_part_bytes_off, lse_part_bytes_off;
    size_t total_bytes;
    int parts;      // grid size of the split kernel
    int slots;      // partial slots (2 per part in line mode, 0 in whole mode)
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Layout for B sequences, H heads, `parts` workgroups and `slots` partial
// slots (slots = 2 * parts in line mode, 0 in whole mode).
inline PlanLayout plan_layout(int B, int H, int parts, int slots) {
    PlanLayout L;
    size_t off = kHdrWords;
    L.seq_len = off; off += (size_t)B;
    L.seq_n = off; off += (size_t)B;
    L.seq_start = off; off += (size_t)B;
    L.seq_first = off; off += (size_t)B;
    L.seq_nsplit = off; off += (size_t)B;
    L.part_first_seq = off; off += (size_t)parts;
    size_t bytes = align_up(off * 4, 256);
    L.o_part_bytes_off = bytes;
    bytes += (size_t)slots * H * kLatent * 2;  // bf16 partial outputs
    bytes = align_up(bytes, 256);
    L.lse_part_bytes_off = bytes;
    bytes += (size_t)slots * H * 4;
    L.total_bytes = align_up(bytes, 256);
    L.parts = parts;
    L.slots = slots;
    return L;
}

}  // namespace mla
