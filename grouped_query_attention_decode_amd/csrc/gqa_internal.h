// Internal interface between the host planner (gqa_api.cpp) and the kernel
// launchers (gqa_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

constexpr int kWave = 64;          // CDNA wavefront width; one wave per workgroup
constexpr int kSlotsPerLane = 4;   // cache rows one lane loads per tile (VALU)
constexpr int kMaxRowBlock = 16;   // query rows per VALU segment
constexpr int kMaxSegments = 1 << 18;  // (sequence, KV head, row block) triples per call
constexpr int kWavesPerCU = 3;     // one-wave workgroups per compute unit (measured best)
constexpr int kWavesPerCUOneBlock = 2;  // matrix-core waves carrying one 16-row block of a bf16 cache
constexpr int kMinRowsPerWaveOneBlock = 256;  // least cache rows per one-block matrix-core wave on small caches (measured)
constexpr int kMaxPiecesPerSegment = 32;  // planner bound on the split of one segment
constexpr int kMultiWaveWavesPerCU = 8;   // multi-wave matrix-core kernel: two waves per SIMD
constexpr int kMfxMinRowsPerGroup = 256;  // least cache rows per workgroup of the 32 x 32 kernel
// Row-split workgroups of the 16 x 16 kernel (measured): caches up to 128 MB,
// one workgroup per 128 KB of K/V, four waves up to 32 MB (or D = 64).
constexpr int64_t kRowSplitMaxBytes = (int64_t)128 << 20;
constexpr int64_t kRowSplitFourWaveBytes = (int64_t)32 << 20;
constexpr int64_t kRowSplitBytesPerGroup = (int64_t)128 << 10;
// Rows' worth of streaming that starting a piece costs a workgroup (loading
// its queries, filling the load pipeline, writing its result), charged in the
// work split: the 16 x 16 kernels ~3 us (measured); the 32 x 32 kernel's
// pieces are longer and start slower (measured per piece: ~15 K cycles to the
// first tile, ~10 K to write a 256-row partial).
constexpr int kPieceCost = 64;
constexpr int kMfxPieceCost = 256;
// Waves per workgroup of the 32 x 32 kernel for a segment of row_block rows
// (32 query rows per wave): 64 rows as 2 query groups x 2 splits, one wave
// per SIMD; 128 rows as 4 x 2 and 256 rows as 8 query groups, two per SIMD.
inline int mfx_waves(int row_block) { return row_block <= 64 ? 4 : 8; }   // 32 rows: 4 splits
constexpr int64_t kMergeBytesInKernel = 64 << 10;  // larger merges go to the combine kernel
// Partial slots are addressed by 32-bit byte offsets within one buffer
// resource: their area stays below 2 GiB (the planner caps the grid).
constexpr int64_t kMaxPartBytes = (int64_t)1 << 31;
// The workspace starts with one arrival counter per possible segment, at a
// fixed place whatever the shape, so counters never land on another call's
// partials; the partials follow.
constexpr size_t kCounterRegion = (size_t)kMaxSegments * sizeof(int32_t);

enum class Path : int { VALU = 1, MFMA = 2, MFMA_QK = 3 };

// Floats in one partial slot: rb rows of d values, then the rows'
// log2-sum-exp padded to a multiple of 16 (slots stay 64-byte aligned).
__host__ __device__ constexpr int slot_floats(int rb, int d) { return rb * d + (((rb > 16 ? rb : 16) + 15) & ~15); }

struct Plan {
    Path path;
    int kv_bf16;        // 1: bf16 q/k/v, 0: fp32
    int kv_fp8;         // 1: bf16 q, 8-bit k/v codes (fp8 E4M3 or int8) with per-KV-head scales
    int kv_i8;          // 1: the 8-bit codes are int8
    int kv_f16;         // 1: fp16 q/k/v
    int D;
    int R;              // (H/G)*sq query rows per KV head
    int row_block;      // query rows per segment: a power of two <= 16 (vector ALU), 16, 32, 64 or 128 (MFMA)
    int n_rb;           // row blocks per (b, g)
    int64_t grid;       // workgroups P (of wg_waves waves each)
    int deferred;       // 1: split segments are merged by a second, parallel kernel
    int slot_rows;      // matrix-core path: rows per partial slot, min(row_block, R)
    int src;            // matrix-core path: 0 cache, 1 cache + appended tokens, 2 paged cache
    int piece_cost;     // matrix-core path: cost units (rows) charged for starting a piece
    int wg_waves;       // waves per workgroup: 1, or 4 / 8 for the multi-wave matrix-core kernels
    int mfx;            // 1: the 32 x 32 matrix-core kernel (more than 32 query rows, bf16 cache)
    int rsplit;         // > 1: 16 x 16 kernel with rsplit waves per workgroup splitting each piece's rows
    size_t part_bytes;  // partials: P * 2 * slot_floats(row_block, D) floats
    size_t ws_bytes;    // kCounterRegion + part_bytes
};

struct Args {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* seq_lens;
    float* out;
    float* part;        // [P][2] slots: row_block rows of D values, then 16 lse floats
    int32_t* counters;  // [kMaxSegments], zero before and after every call
    int B, H, G, sq, T;
    float scale_log2;   // scale * log2(e): scores kept in base-2 exponent units
    int deferred;       // leave every split segment's partials for the combine kernel
    int slot_rows;      // matrix-core path: query rows per partial slot
    int piece_cost;     // matrix-core path: rows' worth of time a piece start costs (work split)
    // cache with appended tokens: the sq new rows of every (b, g), [B, G, sq, D]
    const void* k_new;
    const void* v_new;
    // paged cache: k / v are page pools [num_pages, G, 1 << page_shift, D];
    // block_table [B, max_pages] holds each sequence's pages in order
    const int32_t* block_table;
    int page_shift;
    int num_pages;
    int max_pages;
    // fp8 cache: per-KV-head scales [G] (NULL: 1)
    const float* k_scale;
    const float* v_scale;
};

// Queue the decode kernel on stream.
hipError_t launch_decode(const Plan& plan, const Args& args, hipStream_t stream);

// Fixed device scratch of the entry point that allocates nothing (counters,
// then partials), and its address on the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

// Zero counters[0 .. n) on stream (a kernel, so a graph may capture it).
hipError_t launch_clear_counters(int32_t* counters, int n, hipStream_t stream);

// Workgroups of the plan's kernel one compute unit can hold (0 if unknown).
int resident_groups_per_cu(const Plan& plan);

// Cache rows one wave covers per tile: 16 on the matrix-core paths; on the
// vector-ALU path kSlotsPerLane rows per lane times the cache rows one
// wave-wide 16-byte load covers.
inline int cache_rows_per_wave_tile(const Plan& p)
{
    if (p.path != Path::VALU) return 16;
    const int es = (p.kv_bf16 || p.kv_f16) ? 2 : 4;
    const int lpt = p.D * es / 16;
    return kSlotsPerLane * (kWave / lpt);
}

}  // namespace gqa
