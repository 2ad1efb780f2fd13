// Internal interface between the host planner (gqa_api.cpp) and the kernel
// launchers (gqa_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kSplitWaves = 4;     // waves per split workgroup
constexpr int kSlotsPerLane = 4;   // cache rows one lane loads per tile (VALU)
constexpr int kMaxRowBlock = 16;   // query rows per VALU workgroup
constexpr int kMfmaRows = 16;      // query rows per MFMA row tile
constexpr int kMfmaMaxRows = 64;   // query rows one MFMA workgroup holds
constexpr int kMfmaTile = 32;      // cache rows per MFMA wave tile
constexpr int kTargetSplitGroups = 2048;  // planner aims for this many workgroups

enum class Path : int { VALU = 1, MFMA = 2 };

struct Plan {
    Path path;
    int kv_bf16;        // 1: bf16 q/k/v, 0: fp32
    int D;
    int R;              // (H/G)*sq query rows per KV head
    int row_block;      // rows per workgroup (VALU: power of two <= 16; MFMA: 16/32/64)
    int n_rb;           // row blocks per (b, g)
    int chunk;          // cache rows per workgroup
    int max_chunks;     // ceil(T / chunk)
    int64_t split_grid; // B * G * n_rb * max_chunks
    int64_t combine_grid;
    size_t lds_bytes;   // dynamic LDS of the split kernel
    size_t ws_bytes;    // partial outputs + log-sum-exp
};

struct Args {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* seq_lens;
    float* out;
    float* part_o;      // [B*H*sq, max_chunks, D]
    float* part_lse;    // [B*H*sq, max_chunks]
    int B, H, G, sq, T;
    float scale_log2;   // scale * log2(e): scores kept in base-2 exponent units
};

// Queue the split kernel (and the merge kernel when chunks > 1).  When
// split_done is not null it is recorded on stream between the two.
hipError_t launch_decode(const Plan& plan, const Args& args, hipStream_t stream,
                         hipEvent_t split_done);

// Tile geometry the planner needs: cache rows a whole split workgroup
// covers per iteration, for the given path / dtype / head dim.
int split_tile_rows(Path path, int kv_bf16, int D);

}  // namespace gqa
