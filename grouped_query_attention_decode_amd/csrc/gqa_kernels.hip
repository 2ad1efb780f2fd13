// gqa_kernels.hip -- HIP kernels for grouped-query attention at decode time,
// written for CDNA4 (gfx950, MI355X): 64-wide wavefronts, DPP lane exchange,
// 160 KB LDS per compute unit, HBM3E.
//
// The operation ("GQA (Grouped-Query Attention) 분석", section "Grouped
// broadcast"): query head h reads KV head g = h / (H/G).  Following "Same GQA,
// Different Execution Cost Across Backends" (section 4, the prefill direction
// that expands a KV head into its query heads, and section 6, the query
// reshaped to [B, Hkv, group, D]), one workgroup owns one KV head of one
// sequence and serves every query row that reads it:
//     R = (H/G) * sq rows,  row r = (head within group) * sq + s,
// which are contiguous in q and in out (section 7 of the same page gives the
// same row order, r = g * q_len + s).  Each K/V byte is fetched from HBM once
// for all R rows; no repeated K/V exists anywhere.
//
// Work split (one persistent launch, no second kernel):
//   A "segment" is one (sequence b, KV head g, row block) with L_b cache rows.
//   All segments laid end to end form W = sum_b L_b * G * row_blocks units of
//   work; workgroup p of P takes the units [p*W/P, (p+1)*W/P), i.e. the same
//   number of cache rows for every workgroup however ragged seq_lens is.
//   Each workgroup reads seq_lens itself to find its pieces, so the host never
//   reads device memory.
// A workgroup is one wave.  Per piece (a run of cache rows of one segment)
// the wave streams tiles of 16-byte coalesced K and V loads, with the next
// two tiles' loads in flight while the current one is computed, and keeps an
// online softmax (running max and sum) per query row.  A segment held by one
// workgroup is written to out directly.
// A segment cut between workgroups leaves one (output, log2-sum-exp) partial
// per piece in the workspace; the workgroup that finishes last (per-segment
// arrival counter) merges the pieces in piece order -- deterministic -- with
// weights 2^(lse_k - max lse) and resets the counter to zero, so every call
// leaves the counters as it found them.
//
// Splitting the softmax into pieces and merging them by log-sum-exp is an
// exact rewrite of one softmax over all rows (the oracle pins check this in
// float64).

#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "gqa_chunkmap.h"
#include "gqa_internal.h"

namespace gqa {

// ---------------------------------------------------------------------------
// Lane exchange.  xchg<M>(x) returns x from lane (lane ^ M).
//   M = 1, 2      : DPP quad_perm
//   M = 7, 15     : DPP row_half_mirror / row_mirror (lane ^ 7, lane ^ 15 in a row of 16)
//   M = 8         : DPP row_ror:8 (lane ^ 8 in a row of 16)
//   M = 4, 16     : ds_swizzle bit mode (xor within 32 lanes, no LDS memory)
//   M = 32        : ds_bpermute
// ---------------------------------------------------------------------------
template <int M>
__device__ __forceinline__ float xchg(float x)
{
    const int xi = __builtin_bit_cast(int, x);
    int r;
    if constexpr (M == 1) {
        r = __builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, true);
    } else if constexpr (M == 2) {
        r = __builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, true);
    } else if constexpr (M == 7) {
        r = __builtin_amdgcn_mov_dpp(xi, 0x141, 0xF, 0xF, true);
    } else if constexpr (M == 15) {
        r = __builtin_amdgcn_mov_dpp(xi, 0x140, 0xF, 0xF, true);
    } else if constexpr (M == 8) {
        r = __builtin_amdgcn_mov_dpp(xi, 0x128, 0xF, 0xF, true);
    } else if constexpr (M == 4 || M == 16) {
        r = __builtin_amdgcn_ds_swizzle(xi, 0x1F | (M << 10));
    } else {
        static_assert(M == 32, "unsupported lane exchange");
        r = __shfl_xor(xi, 32);
    }
    return __builtin_bit_cast(float, r);
}

// Partner mask used to split on lane bit BIT when every lane of a cache row
// holds the same row (the K-pass dot products): any mask whose highest bit
// is BIT works, so the cheap DPP mirrors are used.
template <int BIT>
struct RowMask {
    static constexpr int value = BIT == 8 ? 15 : BIT == 4 ? 7 : BIT;
};

// One reduce-scatter stage on N values split on lane bit BIT: lanes with the
// bit clear keep the first half, the others the second half, each summed
// with the partner's copy.  N == 1: plain all-reduce step.
template <int N, int BIT, int MASK>
__device__ __forceinline__ void rs_stage(float* v, int lane)
{
    if constexpr (N == 1) {
        v[0] += xchg<MASK>(v[0]);
    } else {
        const bool low = (lane & BIT) == 0;
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            const float send = low ? v[N / 2 + k] : v[k];
            const float keep = low ? v[k] : v[N / 2 + k];
            v[k] = keep + xchg<MASK>(send);
        }
    }
}

// Reduce N values per lane over the lane bits BIT, BIT/2, ..., LO.  Each
// stage halves the values a lane keeps (down to one).  With ROW = true the
// partner masks may flip lower bits too (for lanes sharing one cache row).
// Afterwards a lane holds min(N, ...) values whose first index is
// (lane bits LO..BIT as an integer) * (values kept) -- see the callers.
template <int N, int BIT, int LO, bool ROW>
__device__ __forceinline__ void reduce_scatter(float* v, int lane)
{
    if constexpr (BIT >= LO) {
        constexpr int MASK = ROW ? RowMask<BIT>::value : BIT;
        rs_stage<N, BIT, MASK>(v, lane);
        reduce_scatter<(N > 1 ? N / 2 : 1), BIT / 2, LO, ROW>(v, lane);
    }
}

__device__ __forceinline__ float wave_max(float x)
{
    x = fmaxf(x, xchg<15>(x));
    x = fmaxf(x, xchg<7>(x));
    x = fmaxf(x, xchg<2>(x));
    x = fmaxf(x, xchg<1>(x));
    x = fmaxf(x, xchg<16>(x));
    x = fmaxf(x, xchg<32>(x));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
    x += xchg<15>(x);
    x += xchg<7>(x);
    x += xchg<2>(x);
    x += xchg<1>(x);
    x += xchg<16>(x);
    x += xchg<32>(x);
    return x;
}

// ---------------------------------------------------------------------------
// Element formats.  A lane always moves 16 bytes: 8 bf16 or 4 fp32 values.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct Bf16 {
    static constexpr int kBytes = 2;
    static constexpr int kPerLoad = 8;
    // <a, b> over 8 bf16 pairs, accumulated in fp32 (v_dot2_f32_bf16).
    static __device__ __forceinline__ float dot(const uint4& a, const uint4& b, float c)
    {
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                            __builtin_bit_cast(bf16x2_t, b.x), c, false);
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                            __builtin_bit_cast(bf16x2_t, b.y), c, false);
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                            __builtin_bit_cast(bf16x2_t, b.z), c, false);
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                            __builtin_bit_cast(bf16x2_t, b.w), c, false);
        return c;
    }
    static __device__ __forceinline__ void unpack(const uint4& a, float* f)
    {
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
};

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

struct F16 {
    static constexpr int kBytes = 2;
    static constexpr int kPerLoad = 8;
    // <a, b> over 8 fp16 pairs, accumulated in fp32 (v_dot2_f32_f16).
    static __device__ __forceinline__ float dot(const uint4& a, const uint4& b, float c)
    {
        c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.x), __builtin_bit_cast(f16x2_t, b.x), c, false);
        c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.y), __builtin_bit_cast(f16x2_t, b.y), c, false);
        c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.z), __builtin_bit_cast(f16x2_t, b.z), c, false);
        c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.w), __builtin_bit_cast(f16x2_t, b.w), c, false);
        return c;
    }
    static __device__ __forceinline__ void unpack(const uint4& a, float* f)
    {
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f16x2_t h = __builtin_bit_cast(f16x2_t, w[i]);
            f[2 * i] = (float)h[0];
            f[2 * i + 1] = (float)h[1];
        }
    }
};

struct F32 {
    static constexpr int kBytes = 4;
    static constexpr int kPerLoad = 4;
    static __device__ __forceinline__ float dot(const uint4& a, const uint4& b, float c)
    {
        c = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), c);
        c = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), c);
        c = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), c);
        c = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), c);
        return c;
    }
    static __device__ __forceinline__ void unpack(const uint4& a, float* f)
    {
        f[0] = __uint_as_float(a.x);
        f[1] = __uint_as_float(a.y);
        f[2] = __uint_as_float(a.z);
        f[3] = __uint_as_float(a.w);
    }
};

__device__ __forceinline__ uint4 load16(const char* p)
{
    return *reinterpret_cast<const uint4*>(p);
}

// Streaming (non-temporal) 16-byte load, for K/V rows read once per call:
// they are not kept in the caches at the expense of other lines.
__device__ __forceinline__ uint4 load16_stream(const char* p)
{
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ int clamp_len(const int32_t* seq_lens, int b, int T)
{
    int L = seq_lens ? seq_lens[b] : T;
    return L < 0 ? 0 : (L > T ? T : L);
}

// Max / sum over the lane bits LO..5 (exact xor partners): lanes that differ
// only in those bits end with the same result.
template <int LO>
__device__ __forceinline__ float lanes_max(float x)
{
    if constexpr (LO <= 0) x = fmaxf(x, xchg<1>(x));
    if constexpr (LO <= 1) x = fmaxf(x, xchg<2>(x));
    if constexpr (LO <= 2) x = fmaxf(x, xchg<4>(x));
    if constexpr (LO <= 3) x = fmaxf(x, xchg<8>(x));
    if constexpr (LO <= 4) x = fmaxf(x, xchg<16>(x));
    if constexpr (LO <= 5) x = fmaxf(x, xchg<32>(x));
    return x;
}

template <int LO>
__device__ __forceinline__ float lanes_sum(float x)
{
    if constexpr (LO <= 0) x += xchg<1>(x);
    if constexpr (LO <= 1) x += xchg<2>(x);
    if constexpr (LO <= 2) x += xchg<4>(x);
    if constexpr (LO <= 3) x += xchg<8>(x);
    if constexpr (LO <= 4) x += xchg<16>(x);
    if constexpr (LO <= 5) x += xchg<32>(x);
    return x;
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// Compiler-level fence for LDS traffic private to one wave: the hardware
// executes one wave's LDS operations in order; this keeps the compiler from
// moving them across each other.
__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Hand-over of a split segment's partials between workgroups.
//  1. Each partial store carries the SC1 cache policy: it is written through
//     to the device-coherent level (HBM side of every XCD's L2).
//  2. s_waitcnt vmcnt(0) returns only once every memory operation of the
//     wave is complete; for an SC1 store that is the device-coherent
//     level's acknowledgement.
//  3. Only then is the arrival counted: the device-scope atomic add is
//     issued after the wait, so any wave whose add returns the last count
//     was ordered after every earlier arrival's completed stores.
//  4. The merge's loads carry SC1 as well: they read the device-coherent
//     level, never a stale line of the reader's own L2; they are issued only
//     after the atomic's result has been compared (a branch on it).
// The hardware keeps this order for instructions in program order; the
// compiler-only fences below keep the compiler from moving the buffer stores
// below the wait, or the buffer loads above the atomic's result (HIP's
// memory model says nothing about the order of a relaxed atomic and plain
// buffer intrinsics, so the order is pinned here at both levels).
__device__ __forceinline__ void partials_stored_before_arrival()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ void arrival_before_partial_loads()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int M>
__device__ __forceinline__ uint32_t xchg_u(uint32_t x)
{
    return __builtin_bit_cast(uint32_t, xchg<M>(__builtin_bit_cast(float, x)));
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x)
{
    x += xchg_u<15>(x);
    x += xchg_u<7>(x);
    x += xchg_u<2>(x);
    x += xchg_u<1>(x);
    x += xchg_u<16>(x);
    x += xchg_u<32>(x);
    return x;
}

// Inclusive prefix sum over the wave, on DPP moves only (no LDS round
// trips): shifts by 1, 2, 4 and 8 lanes within each row of 16 (lanes with
// no source read 0), then row_bcast:15 adds the last lane of rows 0 and 2
// to rows 1 and 3, and row_bcast:31 the last lane of row 1 (the sum of rows
// 0 and 1) to rows 2 and 3.  Rows the row mask leaves out add 0.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x)
{
    int v = (int)x;
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);    // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);    // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);    // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);    // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return (uint32_t)v;
}

// x of lane l (l uniform across the wave), without an LDS round trip.
__device__ __forceinline__ uint32_t lane_u32(uint32_t x, int l)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}

// A value every lane of the wave holds, marked as such for the compiler
// (read from the first active lane), so that what is computed from it lives
// in scalar registers and branches on it are scalar branches.
__device__ __forceinline__ long long uniform_i64(long long x)
{
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)x);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)((unsigned long long)x >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ double uniform_f64(double x)
{
    return __builtin_bit_cast(double, uniform_i64(__builtin_bit_cast(long long, x)));
}

constexpr int kLensWindow = 256;   // seq_lens entries a wave keeps in LDS

// ---------------------------------------------------------------------------
// Work split, the same for every kernel.  Work is counted in cost units: a
// segment (sequence b, KV head g, row block rb) with L > 0 cache rows costs
// piece_cost + L -- its rows plus what starting a piece of it costs a
// workgroup (loading its queries, filling the load pipeline, writing its
// result).  All segments end to end span V cost units, cut into P chunks
// with fixed boundaries, chunk c = [c V / P, (c + 1) V / P), taken by
// workgroup c; with V < P only the first V workgroups take one unit each.
// A chunk that holds the start of a segment (so one more piece) thereby
// gets fewer rows.  A piece is a chunk's part of one segment's rows; its
// partial lives in a slot of the chunk, and merges go in chunk order.  A
// chunk may hold only start cost and no rows: it has no piece, and no
// segment counts it among its pieces (every chunk between a segment's first
// and last row holds rows of it).
//
// (A guided deal -- most of each share static, the rest in small chunks
// handed out by a global counter -- was measured slower on every workload:
// thousands of device-scope atomics on one address serialise.)
// ---------------------------------------------------------------------------
// Cost units of one segment of a sequence with L clamped rows; pc: the
// plan's charge for starting a piece (a.piece_cost).
__device__ __forceinline__ uint32_t seg_cost(int L, int pc)
{
    return L > 0 ? (uint32_t)(L + pc) : 0u;
}

// Partial slots: two per chunk (slot 0 for the segment holding the chunk's
// first unit, slot 1 for the one that starts inside it and runs past its
// end), each a.slot_rows rows of D values, then their log2-sum-exp.
struct MSlots {
    int stride;   // floats per slot
    int lse;      // offset of the log2-sum-exp values in a slot
    __device__ __forceinline__ int base(int c, int which) const { return (2 * c + which) * stride; }
};

template <int D>
__device__ __forceinline__ MSlots mslots(const Args& a)
{
    MSlots m;
    m.lse = a.slot_rows * D;
    m.stride = slot_floats(a.slot_rows, D);
    return m;
}

__device__ __forceinline__ int lens_at(const Args& a, const int* lens, int b)
{
    return b < kLensWindow ? lens[b] : clamp_len(a.seq_lens, b, a.T);
}

// Cost units of one segment of every sequence, summed (every lane gets it).
__device__ __forceinline__ long long total_cost(const Args& a, const int* lens)
{
    const int lane = threadIdx.x & (kWave - 1);
    long long tot = 0;
    for (int b0 = 0; b0 < a.B; b0 += kWave) {
        const int b = b0 + lane;
        tot += wave_sum_u32(b < a.B ? seg_cost(lens_at(a, lens, b), a.piece_cost) : 0u);
    }
    return tot;
}

// First sequence whose cost units reach past unit x, and the units before it.
__device__ __forceinline__ void locate(const Args& a, const int* lens, int units, long long x, int& first_b,
                                       long long& first_v)
{
    const int lane = threadIdx.x & (kWave - 1);
    long long carry = 0;
    for (int b0 = 0; b0 < a.B; b0 += kWave) {
        const int b = b0 + lane;
        const uint32_t c = b < a.B ? seg_cost(lens_at(a, lens, b), a.piece_cost) : 0u;
        const uint32_t incl = wave_incl_scan_u32(c);
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(b < a.B && (carry + incl) * units > x);
        if (hit) {
            const int f = __builtin_ctzll(hit);
            first_b = b0 + f;
            first_v = (carry + lane_u32(incl - c, f)) * units;
            return;
        }
        carry += lane_u32(incl, kWave - 1);
    }
    first_b = a.B;
    first_v = carry * units;
}

// This workgroup's chunk of the split: the chunk map, the chunk [vA, vE) in
// cost units, the first sequence whose units reach past vA and the units
// before it.
struct ChunkPlan {
    ChunkMap cm;
    long long vA, vE, fv;
    int fb;
};

// Plans chunk `chunk` of P; false when it holds no work (no cost units at
// all, or fewer units than workgroups and this chunk past them).  Up to 64
// sequences take one pass: the scan of the segment costs gives the total
// (its last lane) and, by a ballot, the first sequence past vA.
// SCALAR: mark the plan wave-uniform (readfirstlane), so that the piece walk
// built on it runs on scalar registers and branches.  Kernels short of
// scalar registers keep the per-lane form: with it the 32 x 32 kernel
// spilled scalars to vector lanes (64 new tokens 61.75 -> 64.43 us).
template <bool SCALAR>
__device__ __forceinline__ bool plan_chunk(const Args& a, const int* lens, int units, int P, int chunk,
                                           ChunkPlan& cp)
{
    const int lane = threadIdx.x & (kWave - 1);
    if (a.B <= kWave) {
        const uint32_t c = lane < a.B ? seg_cost(lens[lane], a.piece_cost) : 0u;
        const uint32_t incl = wave_incl_scan_u32(c);
        const long long V = (long long)lane_u32(incl, kWave - 1) * units;
        if (V == 0) return false;
        cp.cm = make_map(V, P);
        if (chunk >= cp.cm.P) return false;
        if constexpr (SCALAR) {
            cp.cm.rV = uniform_f64(cp.cm.rV);
            cp.cm.rP = uniform_f64(cp.cm.rP);
        }
        cp.vA = cp.cm.start(chunk);
        cp.vE = cp.cm.start(chunk + 1);
        if constexpr (SCALAR) {
            cp.vA = uniform_i64(cp.vA);
            cp.vE = uniform_i64(cp.vE);
        }
        // some lane below B reaches past vA < V
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < a.B && (long long)incl * units > cp.vA);
        const int f = __builtin_ctzll(hit);
        cp.fb = f;
        cp.fv = (long long)(lane_u32(incl, f) - lane_u32(c, f)) * units;
        return true;
    }
    long long V = total_cost(a, lens) * units;
    if constexpr (SCALAR) V = uniform_i64(V);
    if (V == 0) return false;
    cp.cm = make_map(V, P);
    if (chunk >= cp.cm.P) return false;
    cp.vA = cp.cm.start(chunk);
    cp.vE = cp.cm.start(chunk + 1);
    locate(a, lens, units, cp.vA, cp.fb, cp.fv);
    if constexpr (SCALAR) {
        cp.cm.rV = uniform_f64(cp.cm.rV);
        cp.cm.rP = uniform_f64(cp.cm.rP);
        cp.vA = uniform_i64(cp.vA);
        cp.vE = uniform_i64(cp.vE);
        cp.fb = __builtin_amdgcn_readfirstlane(cp.fb);
        cp.fv = uniform_i64(cp.fv);
    }
    return true;
}

// One piece: a run [ta, tb) of cache rows of segment (b, g, rb).
struct Piece {
    int b, g, rb, ta, tb, L;
    long long off;       // cost-unit position of the segment's first row
};

// Yields the pieces of the chunk [vA, vE) (cost units) in order; a piece's
// `off` is the cost-unit position of its segment's first row.
template <bool SCALAR>
struct CostPieceIter {
    long long vA, vE, Vb;   // the chunk; cost units before sequence b
    int b, k, units, n_rb;

    __device__ __forceinline__ void init(long long vA_, long long vE_, int fb, long long fv, int G, int n_rb_)
    {
        vA = vA_;
        vE = vE_;
        Vb = fv;
        b = fb;
        k = -1;
        n_rb = n_rb_;
        units = G * n_rb_;
    }

    __device__ __forceinline__ bool next(const Args& a, const int* lens, Piece& pc)
    {
        while (b < a.B && Vb < vE) {
            // every lane reads the same length; SCALAR: readfirstlane tells
            // the compiler so, and the walk runs on scalar registers and
            // branches (as a per-lane value, on the vector ALU under exec
            // masks: ~0.5 us per piece with one wave per SIMD)
            int Lb = lens_at(a, lens, b);
            if constexpr (SCALAR) Lb = __builtin_amdgcn_readfirstlane(Lb);
            if (Lb > 0) {
                const int pcost = a.piece_cost;
                const long long sc = (long long)Lb + pcost;
                // first piece of this sequence in the chunk (exact; no 64-bit division)
                if (k < 0) k = vA > Vb ? (int)div_floor(vA - Vb, sc, 1.0 / (double)sc) : 0;
                while (k < units) {
                    const long long vfirst = Vb + k * sc + pcost;
                    if (vfirst - pcost >= vE) return false;
                    const long long ta = vA > vfirst ? vA - vfirst : 0;
                    const long long tb = vE - vfirst < Lb ? vE - vfirst : Lb;
                    const int kk = k++;
                    if (tb > ta) {
                        pc.b = b;
                        pc.g = kk / n_rb;
                        pc.rb = kk % n_rb;
                        pc.ta = (int)ta;
                        pc.tb = (int)tb;
                        pc.L = Lb;
                        pc.off = vfirst;
                        return true;
                    }
                }
            }
            Vb += (long long)units * seg_cost(Lb, a.piece_cost);
            ++b;
            k = -1;
        }
        return false;
    }
};

// Partials cross workgroups that may run on different XCDs, whose L2 caches
// are not coherent with each other.  They are written and read through a
// buffer resource with the device-scope cache policy (SC1): stores write
// through to, and loads read from, the device-coherent level, so no fence
// has to write back or invalidate a whole L2 (which would also throw away
// the K/V lines other waves are streaming), and -- unlike atomic loads --
// the loads of a merge can all be in flight at once.
constexpr int kCoherent = 16;                // SC1 cache-policy bit

__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(float* base)
{
    // raw (untyped) buffer, no swizzle, 2 GiB - 1 byte range
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0x7FFFFFFF, 0x00020000);
}

__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, int index, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, index * 4, 0, kCoherent);
}

__device__ __forceinline__ float load_coherent(__amdgpu_buffer_rsrc_t r, int index)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, index * 4, 0, kCoherent));
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Four consecutive floats (index a multiple of 4): one 16-byte access, so a
// written-through line is not split into many small writes.
__device__ __forceinline__ void store4_coherent(__amdgpu_buffer_rsrc_t r, int index, const float* v)
{
    const u32x4_t x = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
    __builtin_amdgcn_raw_buffer_store_b128(x, r, index * 4, 0, kCoherent);
}

__device__ __forceinline__ void load4_coherent(__amdgpu_buffer_rsrc_t r, int index, float* v)
{
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, index * 4, 0, kCoherent);
    v[0] = __uint_as_float(x[0]);
    v[1] = __uint_as_float(x[1]);
    v[2] = __uint_as_float(x[2]);
    v[3] = __uint_as_float(x[3]);
}

// A segment for which this wave left a partial; merged once every piece has
// arrived.
struct Pending {
    int seg;          // arrival counter index
    int p_first;      // first workgroup holding a piece of the segment
    int npieces;
    long long off;    // position of the segment's first row in the work split
    int64_t qrow0;    // output row of the segment's first query row
    int row0;         // first query row of the segment within its KV head
};

// Partial slot of chunk q for the segment whose first row is cost unit off:
// slot 0 when the segment holds q's first unit, else slot 1 (the segment
// that runs past q's last unit).  A slot is RB rows of D values (16-byte
// aligned) and then RB log2-sum-exp values (at least 16 floats); offset in
// floats.
template <int D, int RB>
__device__ __forceinline__ int slot_base(int q, long long off, const ChunkMap& cm)
{
    return (q * 2 + (cm.start(q) >= off ? 0 : 1)) * slot_floats(RB, D);
}

// The same for the pieces of one segment, q = p_first + k: only the first
// chunk can hold the segment in its second slot (tail1: it starts before
// the segment's first row), so no division per piece.
template <int D, int RB>
__device__ __forceinline__ int piece_slot(int p_first, int k, bool tail1)
{
    return ((p_first + k) * 2 + (k == 0 && tail1 ? 1 : 0)) * slot_floats(RB, D);
}

// One step of the running log-sum-exp merge, branch-free (so that the
// compiler keeps every load of a batch ahead of the arithmetic): x is the
// piece's log2-sum-exp (-inf for an empty or absent piece); returns the
// factor for the old sums and sets *w to the piece's weight.
__device__ __forceinline__ float lse_step(float& M, float x, float* w)
{
    const float Mn = fmaxf(M, x);
    const float sc = (Mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(M - Mn);
    *w = (x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x - Mn);
    M = Mn;
    return sc;
}

// End of a piece, for one wave.  row_m / row_l (LDS) hold each row's max and
// sum over the piece; acc[m] is the weighted V sum of query row u / EPL,
// element doff + u % EPL, for u = ubase + m.  Writes out directly when the
// segment lies in this workgroup; else stores the partial (output / sum and
// log2-sum-exp) and fills *pd.  Returns whether a partial was left.  Issues
// stores only -- nothing waits here.
template <int D, int RB, int EPL, int NAK>
__device__ __forceinline__ bool piece_output(const Args& a, const float* row_m, const float* row_l,
                                             const float* acc, int ubase, int doff, int64_t qrow0,
                                             int row0, int R, int n_rb, int b, int g, int rb,
                                             long long off, int L, const ChunkMap& cm, int chunk,
                                             Pending* pd)
{
    const int p_first = cm.of(off);
    const int npieces = cm.of(off + L - 1) - p_first + 1;
    const __amdgpu_buffer_rsrc_t part = part_rsrc(a.part);
    const int mine = slot_base<D, RB>(chunk, off, cm);
    float val[NAK];
#pragma unroll
    for (int m = 0; m < NAK; ++m) {
        const int i = (ubase + m) / EPL;
        const float l = row_l[i];
        val[m] = l > 0.0f ? acc[m] / l : 0.0f;
    }
    if (npieces == 1) {
#pragma unroll
        for (int m = 0; m < NAK; ++m) {
            const int u = ubase + m;
            const int i = u / EPL;
            if (row0 + i < R) a.out[(qrow0 + i) * D + doff + u % EPL] = val[m];
        }
        return false;
    }
    // a lane's accumulators are runs of consecutive elements of one row
    if constexpr (NAK % 4 == 0 && EPL % 4 == 0) {
#pragma unroll
        for (int m = 0; m < NAK; m += 4) {
            const int u = ubase + m;
            store4_coherent(part, mine + (u / EPL) * D + doff + u % EPL, &val[m]);
        }
    } else {
#pragma unroll
        for (int m = 0; m < NAK; ++m) {
            const int u = ubase + m;
            store_coherent(part, mine + (u / EPL) * D + doff + u % EPL, val[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < NAK; ++m) {
        const int u = ubase + m;
        const int i = u / EPL;
        if (doff + u % EPL == 0) {
            const float l = row_l[i];
            store_coherent(part, mine + RB * D + i, l > 0.0f ? row_m[i] + log2f(l) : -INFINITY);
        }
    }
    pd->seg = (b * a.G + g) * n_rb + rb;
    pd->p_first = p_first;
    pd->npieces = npieces;
    pd->off = off;
    pd->qrow0 = qrow0;
    pd->row0 = row0;
    return true;
}

// Count this wave's arrival for a pending segment; the last arrival merges
// the pieces' partials in piece order (deterministic) and resets the
// counter.  The caller must have waited for its own partial stores
// (s_waitcnt 0), so that the last arrival sees every partial.
template <int D, int RB, int EPL, int NAK>
__device__ __forceinline__ void arrive_and_merge(const Args& a, const Pending& pd, int lane, int ubase,
                                                 int doff, int R, const ChunkMap& cm)
{
    constexpr int NR = NAK >= EPL ? NAK / EPL : 1;    // query rows among a lane's accumulators
    int old = 0;
    if (lane == 0)
        old = __hip_atomic_fetch_add(&a.counters[pd.seg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0);
    if (old != pd.npieces - 1) return;
    arrival_before_partial_loads();

    const __amdgpu_buffer_rsrc_t part = part_rsrc(a.part);
    const int i0 = ubase / EPL;
    float M[NR], den[NR], num[NAK];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        M[r] = -INFINITY;
        den[r] = 0.0f;
    }
#pragma unroll
    for (int m = 0; m < NAK; ++m) num[m] = 0.0f;
    const bool tail1 = cm.start(pd.p_first) < pd.off;
    for (int k0 = 0; k0 < pd.npieces; k0 += 4) {
        // the loads of four pieces are in flight together
        float lse[4][NR], ov[4][NAK];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int base = piece_slot<D, RB>(pd.p_first, min(k0 + kk, pd.npieces - 1), tail1);
#pragma unroll
            for (int r = 0; r < NR; ++r) lse[kk][r] = load_coherent(part, base + RB * D + i0 + r);
            if constexpr (NAK % 4 == 0 && EPL % 4 == 0) {
#pragma unroll
                for (int m = 0; m < NAK; m += 4) {
                    const int u = ubase + m;
                    load4_coherent(part, base + (u / EPL) * D + doff + u % EPL, &ov[kk][m]);
                }
            } else {
#pragma unroll
                for (int m = 0; m < NAK; ++m) {
                    const int u = ubase + m;
                    ov[kk][m] = load_coherent(part, base + (u / EPL) * D + doff + u % EPL);
                }
            }
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                // running log-sum-exp merge, in piece order
                float w;
                const float sc = lse_step(M[r], k0 + kk < pd.npieces ? lse[kk][r] : -INFINITY, &w);
                den[r] = fmaf(den[r], sc, w);
#pragma unroll
                for (int m = 0; m < NAK; ++m)
                    if ((ubase + m) / EPL == i0 + r) num[m] = fmaf(num[m], sc, w * ov[kk][m]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < NAK; ++m) {
        const int u = ubase + m;
        const int i = u / EPL;
        if (pd.row0 + i >= R) continue;
        const float dd = den[i - i0];
        a.out[(pd.qrow0 + i) * D + doff + u % EPL] = dd > 0.0f ? num[m] / dd : 0.0f;
    }
    if (lane == 0) __hip_atomic_store(&a.counters[pd.seg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Output of a piece, resolving a partial right away (vector-ALU kernel).
template <int D, int RB, int EPL, int NAK>
__device__ __forceinline__ void finish_piece(const Args& a, const float* row_m, const float* row_l,
                                             const float* acc, int lane, int ubase, int doff,
                                             int64_t qrow0, int row0, int R, int n_rb, int b, int g,
                                             int rb, long long off, int L, const ChunkMap& cm, int chunk)
{
    Pending pd;
    if (piece_output<D, RB, EPL, NAK>(a, row_m, row_l, acc, ubase, doff, qrow0, row0, R, n_rb, b, g, rb,
                                      off, L, cm, chunk, &pd)) {
        partials_stored_before_arrival();    // own partial stores complete at device scope
        arrive_and_merge<D, RB, EPL, NAK>(a, pd, lane, ubase, doff, R, cm);
    }
}

// ---------------------------------------------------------------------------
// Split pass, vector-ALU form.  One wave per workgroup: every wave is an
// independent worker with its own share of the work, so no barrier ever
// stalls a compute unit -- while one wave is at a piece boundary the others
// keep streaming.
//   FMT : Bf16 or F32 (q, k, v share it)
//   D   : head dim (64 or 128)
//   RB  : query rows per segment (1, 2, 4, 8, 16)
//
// Lane layout for one wave-wide 16-byte load: lane = lrow * LPT + dslot,
// cache row = tile + j * TPL + lrow (j = 0..NL-1 slots), elements
// dslot * EPL .. + EPL.  After the K dot products and the reduce-scatter a
// lane holds NSC whole scores; score index idx = j * RB + i (row i).
// ---------------------------------------------------------------------------
template <class FMT, int D, int RB>
struct ValuGeom {
    static constexpr int ES = FMT::kBytes;
    static constexpr int EPL = FMT::kPerLoad;        // elements per 16-byte load
    static constexpr int LPT = D * ES / 16;          // lanes covering one cache row
    static constexpr int TPL = kWave / LPT;          // cache rows per wave-wide load
    static constexpr int NL = kSlotsPerLane;         // rows per lane per tile
    static constexpr int TW = NL * TPL;              // cache rows per tile
    static constexpr int NV = NL * RB;               // partial dots per lane per tile
    static constexpr int NSC = NV >= LPT ? NV / LPT : 1;    // whole scores per lane
    static constexpr int REP = NV >= LPT ? 1 : LPT / NV;    // lanes holding the same score
    static constexpr int ROWLO = ilog2(LPT / NL);    // lane bits >= ROWLO never change a score's row
    static constexpr int NA = RB * EPL;              // accumulators per lane
    static constexpr int NAK = NA / TPL;             // accumulators kept after the row-group sum
    static constexpr int PB = RB * NL;               // p values of one load row group
    static_assert(LPT >= 1 && LPT <= 32 && (LPT & (LPT - 1)) == 0, "row lanes");
    static_assert(NA >= TPL, "accumulator scatter needs RB * D >= 64");
};

template <class FMT, int D, int RB>
struct ValuShared {
    using Gm = ValuGeom<FMT, D, RB>;
    uint32_t pbuf[Gm::TPL * Gm::PB];   // p of the current tile, [lrow][j][i]
    float alpha[RB];                   // per-row rescale factors
    float row_m[RB];                   // per-row max and sum at the end of a piece
    float row_l[RB];
    int lens[kLensWindow];             // clamped seq_lens[i]
};

// Rows of sequences with no valid cache rows are all zeros; workgroup p
// writes those of sequences b = p, p + P, ...
template <int D>
__device__ void zero_empty_sequences(const Args& a, int P, int p)
{
    const int rows = a.H * a.sq;
    for (int b = p; b < a.B; b += P) {
        if (clamp_len(a.seq_lens, b, a.T) != 0) continue;
        float* o = a.out + (int64_t)b * rows * D;
        for (int idx = threadIdx.x; idx < rows * D; idx += blockDim.x) o[idx] = 0.0f;
    }
}

// Stream cache rows [ta, tb) of segment (b, g, rb) -- one piece -- and
// finish it: write out directly when the segment lies in this chunk, else
// leave a partial and merge all partials if this piece arrives last.
template <class FMT, int D, int RB>
__device__ __forceinline__ void valu_piece(const Args& a, ValuShared<FMT, D, RB>& sm, int R, int n_rb,
                                           const Piece& pc, const ChunkMap& cm, int chunk)
{
    const int b = pc.b, g = pc.g, rb = pc.rb, ta = pc.ta, tb = pc.tb, L = pc.L;
    using Gm = ValuGeom<FMT, D, RB>;
    constexpr int ES = Gm::ES, EPL = Gm::EPL, LPT = Gm::LPT, TPL = Gm::TPL, NL = Gm::NL;
    constexpr int TW = Gm::TW, NV = Gm::NV, NSC = Gm::NSC, REP = Gm::REP;
    constexpr int ROWLO = Gm::ROWLO, NA = Gm::NA, NAK = Gm::NAK, PB = Gm::PB;

    const int lane = threadIdx.x & (kWave - 1);
    const int row0 = rb * RB;
    const int sq = a.sq;
    const int dslot = lane % LPT;
    const int doff = dslot * EPL;
    const int lrow = lane / LPT;

    // rows past R (padding of the last row block) re-read row R-1; their
    // scores are masked, so the values never matter
    const int64_t qrow0 = (int64_t)b * a.H * sq + (int64_t)g * R + row0;
    uint4 qv[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        const int64_t r = qrow0 + min(i, R - 1 - row0);
        qv[i] = load16(static_cast<const char*>(a.q) + (r * D + doff) * ES);
    }

    // rows (and their visibility limit) of the scores this lane holds
    int my_i[NSC], my_j[NSC], my_last[NSC];
#pragma unroll
    for (int m = 0; m < NSC; ++m) {
        const int idx = (NV >= LPT) ? dslot * NSC + m : dslot / REP;
        my_i[m] = idx % RB;
        my_j[m] = idx / RB;
        const int r = row0 + my_i[m];
        my_last[m] = (r < R) ? L - sq + (r % sq) : -1;
    }
    const bool p_writer = (NV >= LPT) || (dslot % REP == 0);
    uint32_t* pbuf = sm.pbuf;
    float* alpha = sm.alpha;

    const int64_t slab = ((int64_t)b * a.G + g) * a.T * D;
    const char* kbase = static_cast<const char*>(a.k) + slab * ES;
    const char* vbase = static_cast<const char*>(a.v) + slab * ES;

    float m_run[NSC], l_run[NSC];
#pragma unroll
    for (int m = 0; m < NSC; ++m) {
        m_run[m] = -INFINITY;
        l_run[m] = 0.0f;
    }
    float acc[NA];
#pragma unroll
    for (int u = 0; u < NA; ++u) acc[u] = 0.0f;

    // Rows past the piece's end re-read row tb - 1, which is valid: their
    // scores are masked to -inf and their weights are exactly 0, so no row
    // at or beyond tb is ever read and no branch guards the loads.
    auto load_tile = [&](int t0, uint4* kk, uint4* vv) {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int t = min(t0 + j * TPL + lrow, tb - 1);
            const int64_t o = ((int64_t)t * D + doff) * ES;
            kk[j] = load16_stream(kbase + o);
            vv[j] = load16_stream(vbase + o);
        }
    };

    auto compute_tile = [&](int t0, const uint4* kk, const uint4* vv) {
        // scores: partial dots, then reduce-scatter within each cache row's lanes
        float part[NV];
#pragma unroll
        for (int j = 0; j < NL; ++j)
#pragma unroll
            for (int i = 0; i < RB; ++i) part[j * RB + i] = FMT::dot(qv[i], kk[j], 0.0f);
        reduce_scatter<NV, LPT / 2, 1, true>(part, lane);

        float s[NSC], m_new[NSC];
        bool grew = false;
#pragma unroll
        for (int m = 0; m < NSC; ++m) {
            const int t = t0 + my_j[m] * TPL + lrow;
            const bool vis = (t < tb) && (t <= my_last[m]);
            s[m] = vis ? part[m] * a.scale_log2 : -INFINITY;
            const float tmax = lanes_max<ROWLO>(s[m]);
            m_new[m] = fmaxf(m_run[m], tmax);
            grew |= m_new[m] > m_run[m];
        }
        // a row's max grew: rescale that row's sums (rare after the first tiles)
        if (__builtin_amdgcn_ballot_w64(grew) != 0) {
#pragma unroll
            for (int m = 0; m < NSC; ++m) {
                const float al = (m_new[m] > m_run[m]) ? __builtin_amdgcn_exp2f(m_run[m] - m_new[m]) : 1.0f;
                l_run[m] *= al;
                m_run[m] = m_new[m];
                if (p_writer) alpha[my_i[m]] = al;
            }
            wave_lds_fence();
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const float al = alpha[i];
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[i * EPL + e] *= al;
            }
        }
        // p = 2^(s - m) in fp32, shared with the lanes of the same cache row group
#pragma unroll
        for (int m = 0; m < NSC; ++m) {
            const float pv = (s[m] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s[m] - m_run[m]);
            l_run[m] += pv;
            if (p_writer) pbuf[lrow * PB + my_j[m] * RB + my_i[m]] = __float_as_uint(pv);
        }
        wave_lds_fence();
        // weighted V sum, fp32 weights and fp32 accumulation
        {
            const float* src = reinterpret_cast<const float*>(pbuf) + lrow * PB;
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                float vf[EPL];
                FMT::unpack(vv[j], vf);
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    const float pv = src[j * RB + i];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[i * EPL + e] = fmaf(pv, vf[e], acc[i * EPL + e]);
                }
            }
        }
        wave_lds_fence();   // next tile's p writes stay behind these reads
    };

    // Three register buffers in rotation: the next two tiles are in flight
    // while the current one is computed.  The loads are issued
    // unconditionally (rows clamped into the piece): with the same number of
    // loads on every path the compiler waits for exactly the oldest tile
    // instead of draining the prefetches.
    {
        uint4 ka[NL], va[NL], kb[NL], vb[NL], kc[NL], vc[NL];
        int t0 = ta;
        const int ntile = (tb - ta + TW - 1) / TW;
        load_tile(t0, ka, va);
        load_tile(t0 + TW, kb, vb);
        for (int it = 0; it < ntile; it += 3) {
            load_tile(t0 + 2 * TW, kc, vc);
            compute_tile(t0, ka, va);
            t0 += TW;
            if (it + 1 >= ntile) break;
            load_tile(t0 + 2 * TW, ka, va);
            compute_tile(t0, kb, vb);
            t0 += TW;
            if (it + 2 >= ntile) break;
            load_tile(t0 + 2 * TW, kb, vb);
            compute_tile(t0, kc, vc);
            t0 += TW;
        }
    }

    // ---- end of the piece: sums over the lanes of the wave ------------------
#pragma unroll
    for (int m = 0; m < NSC; ++m) l_run[m] = lanes_sum<ROWLO>(l_run[m]);
    reduce_scatter<NA, kWave / 2, LPT, false>(acc, lane);
    if (lrow == 0 && p_writer) {
#pragma unroll
        for (int m = 0; m < NSC; ++m) {
            if (my_j[m] == 0) {
                sm.row_m[my_i[m]] = m_run[m];
                sm.row_l[my_i[m]] = l_run[m];
            }
        }
    }
    wave_lds_fence();

    finish_piece<D, RB, EPL, NAK>(a, sm.row_m, sm.row_l, acc, lane, lrow * NAK, doff, qrow0, row0, R,
                                  n_rb, b, g, rb, pc.off, L, cm, chunk);
    wave_lds_fence();   // row_m/row_l/pbuf are rewritten by the next piece
}

template <class FMT, int D, int RB>
__global__ void __launch_bounds__(kWave)
decode_valu(const int32_t* __restrict__ lens_in, const int nB, const int nT, const Args a, const int R, const int n_rb)
{
    __shared__ ValuShared<FMT, D, RB> sm;
    const int P = gridDim.x;
    const int p = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    for (int i = lane; i < kLensWindow && i < nB; i += kWave) sm.lens[i] = clamp_len(lens_in, i, nT);
    zero_empty_sequences<D>(a, P, p);
    wave_lds_fence();
    const int units = a.G * n_rb;
    const int chunk = p;
    ChunkPlan cp;
    if (!plan_chunk<false>(a, sm.lens, units, P, chunk, cp)) return;
    const ChunkMap& cm = cp.cm;
    CostPieceIter<false> it;
    it.init(cp.vA, cp.vE, cp.fb, cp.fv, a.G, n_rb);
    Piece pc;
    while (it.next(a, sm.lens, pc)) valu_piece<FMT, D, RB>(a, sm, R, n_rb, pc, cm, chunk);
}

// ---------------------------------------------------------------------------
// bf16, up to 16 query rows per segment: scores on the matrix cores.
// S[16 query rows x 16 cache rows] = Q . K^T with v_mfma_f32_16x16x32_bf16
// (D/32 instructions per tile, fp32 accumulation); the softmax and the
// weighted V sum stay on the vector ALU in fp32.
//   operand A (Q):   lane l holds query row l % 16, elements 8*(l/16) + 32*kk .. +8
//   operand B (K^T): lane l holds cache row tile + l % 16, the same elements
//   result:          lane l holds S[4*(l/16) + jj][l % 16], jj = 0..3
// A and B give every lane's k slots the same head-dim elements, so the
// products pair up correctly whatever order the unit sums them in.  Rows of
// the block past RB (or past R) repeat its first row in A and are masked in S.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));


struct MqkShared {
    float pbuf[16][16];      // p of the current tile: [cache row][query row]
    float row_m[16];         // per-row max and sum at the end of a piece
    float row_l[16];
    int lens[kLensWindow];   // clamped seq_lens[i]
};

template <int M>
__device__ __forceinline__ float row16_max(float x)
{
    x = fmaxf(x, xchg<15>(x));
    x = fmaxf(x, xchg<7>(x));
    x = fmaxf(x, xchg<2>(x));
    x = fmaxf(x, xchg<1>(x));
    return x;
}

__device__ __forceinline__ float row16_sum(float x)
{
    x += xchg<15>(x);
    x += xchg<7>(x);
    x += xchg<2>(x);
    x += xchg<1>(x);
    return x;
}

__device__ __forceinline__ float readlane_f(float x, int l)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// One piece of segment (b, g, rb): cache rows [ta, tb).  The wave streams
// 16-row tiles with the loads of the next two tiles in flight, then writes
// the piece out (or stores its partial, returned in *pd without waiting).
template <int D, int RB>
__device__ __forceinline__ bool mqk_piece(const Args& a, MqkShared& sm, int R, int n_rb, const Piece& pc,
                                          const ChunkMap& cm, int chunk, Pending* pd)
{
    constexpr int NK = D / 32;           // matrix-core k steps per tile
    constexpr int EPL = 8;               // bf16 per 16-byte load (V layout)
    constexpr int LPT = D / EPL;         // lanes per cache row in the V layout
    constexpr int TPL = kWave / LPT;     // cache rows per wave-wide V load
    constexpr int TW = 16;               // cache rows per tile
    constexpr int NLV = TW / TPL;        // V loads per lane per tile
    constexpr int NA = RB * EPL;         // V-sum accumulators per lane
    constexpr int NAK = NA / TPL;        // kept after the row-group sum
    static_assert(RB >= 4 && RB <= 16 && NA >= TPL, "row block");

    const int lane = threadIdx.x & (kWave - 1);
    const int col = lane & 15;           // MFMA column / A row of this lane
    const int kg = lane >> 4;            // MFMA k group
    const int lrow = lane / LPT;         // V layout
    const int doff = (lane % LPT) * EPL;
    const int ta = pc.ta, tb = pc.tb;
    const int row0 = pc.rb * RB;
    const int64_t qrow0 = (int64_t)pc.b * a.H * a.sq + (int64_t)pc.g * R + row0;

    // A operand: query row `col` of the block; rows past RB or R read the
    // block's first row (their scores are masked, and never stored)
    uint4 qa[NK];
    {
        const bool live = col < RB && row0 + col < R;
        const char* qp = static_cast<const char*>(a.q) + ((qrow0 + (live ? col : 0)) * D + 8 * kg) * 2;
#pragma unroll
        for (int s = 0; s < NK; ++s) qa[s] = load16(qp + 64 * s);
    }
    int last[4];
    float m_run[4], l_run[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int r = 4 * kg + jj;
        last[jj] = (r < RB && row0 + r < R) ? pc.L - a.sq + ((row0 + r) % a.sq) : -1;
        m_run[jj] = -INFINITY;
        l_run[jj] = 0.0f;
    }
    float acc[NA];
#pragma unroll
    for (int u = 0; u < NA; ++u) acc[u] = 0.0f;

    const int64_t slab = ((int64_t)pc.b * a.G + pc.g) * a.T * D;
    const char* kbase = static_cast<const char*>(a.k) + (slab + 8 * kg) * 2;
    const char* vbase = static_cast<const char*>(a.v) + (slab + doff) * 2;

    // rows past the piece's end re-read row tb - 1 (valid; masked / weight 0)
    auto load_tile = [&](int t0, uint4* kk, uint4* vv) {
        const int tk = min(t0 + col, tb - 1);
#pragma unroll
        for (int s = 0; s < NK; ++s) kk[s] = load16(kbase + ((int64_t)tk * D + 32 * s) * 2);
#pragma unroll
        for (int j = 0; j < NLV; ++j) {
            const int tv = min(t0 + j * TPL + lrow, tb - 1);
            vv[j] = load16(vbase + (int64_t)tv * D * 2);
        }
    };

    auto compute_tile = [&](int t0, const uint4* kk, const uint4* vv) {
        f32x4_t s4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < NK; ++s)
            s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[s]),
                                                         __builtin_bit_cast(bf16x8_t, kk[s]), s4, 0, 0, 0);
        const int t = t0 + col;
        float sc[4], m_new[4];
        bool grew = false;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            sc[jj] = (t < tb && t <= last[jj]) ? s4[jj] * a.scale_log2 : -INFINITY;
            m_new[jj] = fmaxf(m_run[jj], row16_max<0>(sc[jj]));
            grew |= m_new[jj] > m_run[jj];
        }
        if (__builtin_amdgcn_ballot_w64(grew) != 0) {
            float al[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                al[jj] = (m_new[jj] > m_run[jj]) ? __builtin_amdgcn_exp2f(m_run[jj] - m_new[jj]) : 1.0f;
                l_run[jj] *= al[jj];
                m_run[jj] = m_new[jj];
            }
            // row i's factor sits in the lanes of k group i / 4
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const float f = readlane_f(al[i % 4], 16 * (i / 4));
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[i * EPL + e] *= f;
            }
        }
        float pv[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            pv[jj] = (sc[jj] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[jj] - m_run[jj]);
            l_run[jj] += pv[jj];
        }
        if (4 * kg < RB)
            *reinterpret_cast<float4*>(&sm.pbuf[col][4 * kg]) = make_float4(pv[0], pv[1], pv[2], pv[3]);
        wave_lds_fence();
        // weighted V sum, fp32 weights and fp32 accumulation
#pragma unroll
        for (int j = 0; j < NLV; ++j) {
            const float* prow = sm.pbuf[j * TPL + lrow];
            float vf[EPL];
            Bf16::unpack(vv[j], vf);
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const float w = prow[i];
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[i * EPL + e] = fmaf(w, vf[e], acc[i * EPL + e]);
            }
        }
        wave_lds_fence();   // next tile's p writes stay behind these reads
    };

    // Three register buffers in rotation; the loads are unconditional (rows
    // clamped into the piece) so the compiler waits for exactly the oldest
    // tile instead of draining the prefetches.
    {
        uint4 ka[NK], va[NLV], kb[NK], vb[NLV], kc[NK], vc[NLV];
        int t0 = ta;
        const int ntile = (tb - ta + TW - 1) / TW;
        load_tile(t0, ka, va);
        load_tile(t0 + TW, kb, vb);
        for (int it = 0; it < ntile; it += 3) {
            load_tile(t0 + 2 * TW, kc, vc);
            compute_tile(t0, ka, va);
            t0 += TW;
            if (it + 1 >= ntile) break;
            load_tile(t0 + 2 * TW, ka, va);
            compute_tile(t0, kb, vb);
            t0 += TW;
            if (it + 2 >= ntile) break;
            load_tile(t0 + 2 * TW, kb, vb);
            compute_tile(t0, kc, vc);
            t0 += TW;
        }
    }

    // ---- end of the piece ------------------------------------------------------
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) l_run[jj] = row16_sum(l_run[jj]);
    reduce_scatter<NA, kWave / 2, LPT, false>(acc, lane);
    if (col == 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r = 4 * kg + jj;
            if (r < RB) {
                sm.row_m[r] = m_run[jj];
                sm.row_l[r] = l_run[jj];
            }
        }
    }
    wave_lds_fence();
    const bool left = piece_output<D, RB, EPL, NAK>(a, sm.row_m, sm.row_l, acc, lrow * NAK, doff, qrow0, row0,
                                                    R, n_rb, pc.b, pc.g, pc.rb, pc.off, pc.L, cm, chunk, pd);
    wave_lds_fence();   // row_m / row_l / pbuf are rewritten by the next piece
    return left;
}

// Pieces are streamed one after another.  A piece that left a partial is
// counted (and, by the last arrival, merged) right away: merging early
// spreads the merges over the run instead of piling them up at its end.
template <int D, int RB>
__global__ void __launch_bounds__(kWave)
decode_mqk(const int32_t* __restrict__ lens_in, const int nB, const int nT, const Args a, const int R, const int n_rb)
{
    constexpr int EPL = 8;
    constexpr int LPT = D / EPL;
    constexpr int NAK = RB * EPL / (kWave / LPT);
    __shared__ MqkShared sm;
    const int P = gridDim.x;
    const int p = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    for (int i = lane; i < kLensWindow && i < nB; i += kWave) sm.lens[i] = clamp_len(lens_in, i, nT);
    zero_empty_sequences<D>(a, P, p);
    wave_lds_fence();
    const int units = a.G * n_rb;
    const int chunk = p;
    ChunkPlan cp;
    if (!plan_chunk<false>(a, sm.lens, units, P, chunk, cp)) return;
    const ChunkMap& cm = cp.cm;
    CostPieceIter<false> it;
    it.init(cp.vA, cp.vE, cp.fb, cp.fv, a.G, n_rb);
    Piece pc;
    while (it.next(a, sm.lens, pc)) {
        Pending pd;
        if (mqk_piece<D, RB>(a, sm, R, n_rb, pc, cm, chunk, &pd)) {
            partials_stored_before_arrival();    // own partial stores complete at device scope
            arrive_and_merge<D, RB, EPL, NAK>(a, pd, lane, (lane / LPT) * NAK, (lane % LPT) * EPL, R, cm);
        }
    }
}

// ---------------------------------------------------------------------------
// Matrix-core pass: both products on the MFMA units (bf16 inputs).
//
// Per tile of cache rows t (32, as two 16-row halves h) and each block of
// (up to) 16 query rows r of a segment:
//   S^T_h[t][r] = K_h[t][:] . Q[r][:]         v_mfma_f32_16x16x32_bf16, A = K, B = Q^T
//   O^T[d][r]  += V^T[d][t] . P^T[t][r]       v_mfma_f32_16x16x32_bf16, A = V^T, B = P^T
// The score accumulator of half h gives lane l the scores of query row
// l % 16 at cache rows 16 h + 4 (l / 16) + 0..3, and the V product takes
// its k index 8 (l / 16) + i as tile row 16 (i / 4) + 4 (l / 16) + i % 4:
// the weights are already where its B operand wants them and never move
// between lanes.  V^T comes from the row-major LDS copy of the tile by the
// transpose read below.  Every output element of lane l belongs to query
// row l % 16, so a rescale multiplies a lane's accumulators by one factor.
// (With 16-row tiles the V product is v_mfma_f32_16x16x16_bf16, k index
// 4 (l / 16) + i as row 4 (l / 16) + i.)
//
// The weights p (fp32, in (0, 2^kSlack]) enter the V product as two bf16
// terms, p = hi + lo, which keeps about 16 bits of each weight; V is exact in
// bf16, and accumulation is fp32.
// ---------------------------------------------------------------------------
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Four bf16 of one column of a row-major bf16 block in LDS, four rows apart
// in the A-operand order of v_mfma_f32_16x16x16_bf16, by the gfx950 LDS
// transpose read (ds_read_b64_tr_b16).  Within each 16-lane group, lane i
// receives element i % 4 of the 8-byte pieces addressed by lanes i / 4,
// 4 + i / 4, 8 + i / 4 and 12 + i / 4 of its group, in that order.  So when
// lane (kg, s) of the wave addresses row 4 kg + s / 4, columns 4 (s % 4) ..
// 4 (s % 4) + 3 of a 16 x 16 block, lane (kg, col) receives column col of
// rows 4 kg .. 4 kg + 3.  p must be 8-byte aligned.
__device__ __forceinline__ s16x4_t lds_read_tr16(const uint16_t* p)
{
    typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p));
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// The running max is moved only when a tile's max exceeds it by more than
// kSlack (base-2 units); weights then stay below 2^kSlack.  The result is
// the same -- numerator and denominator share the reference -- and most
// tiles skip the rescale.
constexpr float kSlack = 8.0f;

// Cache rows per tile of the one-wave matrix-core pass: 32 (two 16-row
// halves sharing one softmax step and K = 32 weighted-sum products); 16 when
// four query blocks' accumulators and operands leave no room for 32-row
// tiles in flight.
template <int NB>
constexpr int mfa_tile_rows() { return NB >= 4 ? 16 : 32; }

// K/V tiles held in registers per wave: two 32-row tiles (one in flight
// while one is computed: 16 KB of a bf16 cache), or two 16-row tiles with
// four query blocks.  An fp8 tile is half the bytes, but its waves run four
// per compute unit: two tiles each keep the same ~64 KB per compute unit in
// flight as two bf16 waves do, and measured faster than three (batched
// GQA-8: 43.1 -> 41.9 us; four: 44.2).  Four 16-row fp8 blocks keep three.
template <int NB, bool KV8>
constexpr int mfa_buffers() { return (KV8 && NB >= 4) ? 3 : 2; }

// Head-dim element where the 8 elements of score-product step s start for
// k group kg (the order of the reduction over d is free as long as K and Q
// use the same one): bf16 rows are read as 16-byte pieces at 8 kg + 32 s;
// fp8 rows as 16-code pieces at 16 kg + 64 h, each splitting into steps 2h
// and 2h + 1.
template <int D, bool KV8>
__device__ __forceinline__ int kdim0(int kg, int s)
{
    return KV8 ? 16 * kg + 64 * (s >> 1) + 8 * (s & 1) : 8 * kg + 32 * s;
}

// 16 fp8 E4M3 codes (one 16-byte load, code i in byte i) to 16 bf16 values
// in order: lo holds codes 0..7, hi codes 8..15.  Every E4M3 value is a bf16
// number, so the conversion (scale 1) is exact.
__device__ __forceinline__ void fp8x16_to_bf16(const uint4& c, uint4& lo, uint4& hi)
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
        o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
    }
    lo = make_uint4(o[0], o[1], o[2], o[3]);
    hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// 16 int8 codes -> two 8-element bf16 operands, each code c stored as the
// unsigned u = c + 128 (exact: u has at most 8 significant bits, so its fp32
// value truncates to bf16 without loss).  The offset of 128 is undone where
// it lands: in the scores it adds the same amount to every score of a query
// row (128 scale <q, 1>), which the softmax does not see; in the weighted V
// sum it adds 128 to every output, subtracted when the rows are finished.
__device__ __forceinline__ void i8x16_to_bf16(const uint4& c, uint4& lo, uint4& hi)
{
    const uint32_t w[4] = {c.x ^ 0x80808080u, c.y ^ 0x80808080u, c.z ^ 0x80808080u, c.w ^ 0x80808080u};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t f0 = __float_as_uint((float)(w[i] & 0xFFu));
        const uint32_t f1 = __float_as_uint((float)((w[i] >> 8) & 0xFFu));
        const uint32_t f2 = __float_as_uint((float)((w[i] >> 16) & 0xFFu));
        const uint32_t f3 = __float_as_uint((float)(w[i] >> 24));
        // high halves of (f0, f1) and of (f2, f3): element 0 in the low half
        o[2 * i] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
        o[2 * i + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
    }
    lo = make_uint4(o[0], o[1], o[2], o[3]);
    hi = make_uint4(o[4], o[5], o[6], o[7]);
}

constexpr int kPageWindow = 1024;        // block-table entries a wave keeps in LDS (paged cache)

// Where the matrix-core pass reads K/V rows from.
constexpr int kSrcCache = 0;    // contiguous [B, G, T, D] cache
constexpr int kSrcAppend = 1;   // the cache, the last sq rows taken from (and written with) new tokens
constexpr int kSrcPaged = 2;    // page pool [num_pages, G, page_size, D] and a block table

template <int D>
struct MfaShared {
    static constexpr int SE = D + 16;   // LDS row stride (bf16): the 32-byte pieces of eight consecutive rows cover all 64 banks
    alignas(16) uint16_t vt[32 * SE];   // V tile (up to 32 rows), row-major
    int lens[kLensWindow];              // clamped seq_lens[i]
    int pages[kPageWindow];             // paged cache: physical pages of the current row window
};

// Workgroup of NW waves that split each piece's cache rows (NB 16-row query
// blocks): one V tile per wave, and the exchange area through which waves
// 1 .. NW - 1 hand their running max, partial sums and accumulators to wave 0.
template <int D, int NB, int NW>
struct MfsShared {
    static constexpr int SE = MfaShared<D>::SE;
    static constexpr int NV = NB * (2 + 4 * (D / 16));   // floats per lane handed over
    alignas(16) uint16_t vt[NW][32 * SE];
    float xch[NW - 1][NV][kWave];
    int lens[kLensWindow];              // clamped seq_lens[i]
};

template <int D>
__device__ __forceinline__ uint16_t* wave_vt(MfaShared<D>& sm) { return sm.vt; }

template <int D, int NB, int NW>
__device__ __forceinline__ uint16_t* wave_vt(MfsShared<D, NB, NW>& sm) { return sm.vt[threadIdx.x / kWave]; }

// Two floats to packed bf16 (round to nearest even), element 0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float x0, float x1)
{
    const f32x2_t v = {x0, x1};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

// The 16-bit operands of the matrix-core products: bf16 (a bf16 cache, and
// the fp8 cache decoded to bf16) or fp16.  pack2 rounds two floats to nearest
// even (element 0 in the low half), lo / hi give the value of element 0 / 1
// of a packed pair; the products accumulate in fp32.
//   mma16x32: v_mfma_f32_16x16x32_{bf16,f16}   (8 elements per lane)
//   mma16x16: v_mfma_f32_16x16x16_{bf16,f16}   (4 elements per lane)
//   mma32x16: v_mfma_f32_32x32x16_{bf16,f16}   (8 elements per lane)
template <bool F16>
struct Mx {
    static __device__ __forceinline__ uint32_t pack2(float x0, float x1) { return pack_bf16x2(x0, x1); }
    static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
    // the rounding residuals x0 - lo(w), x1 - hi(w), packed
    static __device__ __forceinline__ uint32_t resid2(float x0, float x1, uint32_t w)
    {
        return pack2(x0 - lo(w), x1 - hi(w));
    }
    static __device__ __forceinline__ f32x4_t mma16x32(const uint4& a, const uint4& b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t mma16x16(const uint2& a, const uint2& b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                         c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x16_t mma32x16(const uint4& a, const uint4& b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       c, 0, 0, 0);
    }
};

template <>
struct Mx<true> {
    static __device__ __forceinline__ uint32_t pack2(float x0, float x1)
    {
        const f32x2_t v = {x0, x1};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
    }
    static __device__ __forceinline__ float lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[0]; }
    static __device__ __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[1]; }
    static __device__ __forceinline__ uint32_t resid2(float x0, float x1, uint32_t w)
    {
        return pack2(x0 - lo(w), x1 - hi(w));
    }
    static __device__ __forceinline__ f32x4_t mma16x32(const uint4& a, const uint4& b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                      0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t mma16x16(const uint2& a, const uint2& b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c, 0,
                                                     0, 0);
    }
    static __device__ __forceinline__ f32x16_t mma32x16(const uint4& a, const uint4& b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                      0, 0, 0);
    }
};

// Reductions over lane pairs (l, l ^ 16) and (l, l ^ 32) with the gfx950
// row-swap permutes (VALU only).  The two results of a swap of x with itself
// hold, in every lane, its own value and its partner's, so combining them
// gives the pair's result in both lanes, in the same order.
__device__ __forceinline__ float max_x16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float max_x32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_x16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float sum_x32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One piece of segment (b, g, rb) -- cache rows [ta, tb) for the RB = 16 NB
// query rows RB rb .. RB rb + RB - 1 -- streamed in 32-row tiles with the
// next tiles' loads in flight; then written out, or left as a partial
// (returned in *pd, stores issued, nothing waited for).  The NB 16-row
// blocks share every K/V tile: it is read once for all of them.
template <int D, int NB, int SRC, bool KV8, int NW = 1, class SM = MfaShared<D>, bool F16 = false,
          bool I8 = false>
__device__ __forceinline__ bool mfa_piece(const Args& a, SM& sm, int R, int n_rb, const Piece& pc,
                                          const ChunkMap& cm, int chunk, Pending* pd)
{
    static_assert(NW == 1 || (SRC == kSrcCache && !KV8), "row-split workgroups read a plain 16-bit cache");
    static_assert(!F16 || !KV8, "an 8-bit cache takes bf16 queries");
    static_assert(!I8 || KV8, "int8 codes are an 8-bit cache");
    using MX = Mx<F16>;
    constexpr int NK = D / 32;           // k steps of the score product
    constexpr int NC = D / 16;           // column blocks of the V product
    constexpr int SE = MfaShared<D>::SE;
    constexpr int ES = KV8 ? 1 : 2;      // bytes per cache element (fp8 codes or bf16)
    constexpr int EPC = 16 / ES;         // cache elements per 16-byte chunk
    constexpr int CPR = D / EPC;         // 16-byte chunks per cache row
    constexpr int TR = mfa_tile_rows<NB>();  // cache rows per tile
    constexpr int NH = TR / 16;              // 16-row halves of a tile
    constexpr int NLV = TR * CPR / kWave;   // V loads per lane per tile
    constexpr int NLK = KV8 ? D / 64 : NK;  // K loads per lane per half tile
    constexpr int RB = 16 * NB;

    const int lane = threadIdx.x & (kWave - 1);
    const int col = lane & 15;           // query row of this lane within a block
    const int kg = lane >> 4;            // k group: cache rows 4 kg .. 4 kg + 3 of a tile
    // NW > 1: wave w streams tiles [n w / NW, n (w + 1) / NW) of the piece's
    // n tiles (rows past the piece's end read as its last row, weight 0)
    int ta = pc.ta, tb = pc.tb;
    if constexpr (NW > 1) {
        const int n = (pc.tb - pc.ta + TR - 1) / TR;
        const int w = threadIdx.x / kWave;
        ta = min(pc.tb, pc.ta + TR * (n * w / NW));
        tb = min(pc.tb, pc.ta + TR * (n * (w + 1) / NW));
    }
    uint16_t* const vt = wave_vt(sm);
    const int row0 = pc.rb * RB;
    const int64_t qrow0 = (int64_t)pc.b * a.H * a.sq + (int64_t)pc.g * R + row0;

    // B operands of the score product: query row 16 nb + col.  Rows past R
    // read the block's first row: their scores are masked (last = -1) or, in a
    // full tile, feed only their own rows, which are never stored; no select
    // on the loaded values, so nothing waits for these loads before the first
    // tile's compute.
    uint4 qb[NB][NK];
    bool live[NB];
    int last[NB];
    float m_run[NB], l_run[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int r = row0 + 16 * nb + col;
        live[nb] = r < R;
        last[nb] = live[nb] ? pc.L - a.sq + (r % a.sq) : -1;
        m_run[nb] = -INFINITY;
        l_run[nb] = 0.0f;
        const char* qp = static_cast<const char*>(a.q) + (qrow0 + (live[nb] ? 16 * nb + col : 0)) * D * 2;
#pragma unroll
        for (int s = 0; s < NK; ++s) qb[nb][s] = load16(qp + 2 * kdim0<D, KV8>(kg, s));
    }
    f32x4_t acc[NB][NC];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[nb][c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // fp8 cache: the value of a code is decode(code) * scale of its KV head;
    // K's scale joins the score scale, V's multiplies the output
    float score_scale = a.scale_log2, out_scale = 1.0f;
    if constexpr (KV8) {
        if (a.k_scale) score_scale *= a.k_scale[pc.g];
        if (a.v_scale) out_scale = a.v_scale[pc.g];
    }

    // Where cache row t of (b, g) lives (byte address of its element 0):
    //   kSrcCache  : the [B, G, T, D] cache;
    //   kSrcAppend : rows t >= L - sq are the new tokens, read from
    //                k_new / v_new [B, G, sq, D] (and written into the cache);
    //   kSrcPaged  : page block_table[b][t >> page_shift] of the page pool
    //                [num_pages, G, page_size, D], row t & (page_size - 1).
    const int64_t slab = ((int64_t)pc.b * a.G + pc.g) * a.T * D;
    const int la = pc.L - a.sq;
    const int64_t nslab = ((int64_t)pc.b * a.G + pc.g) * a.sq * D;
    int wpage0 = 0;                      // paged: first page of the LDS window
    int tend = tb;                       // end of the current row window
    // paged: pages of the rows the next load_tile reads (the K rows of both
    // halves, the V rows), looked up one tile ahead so the LDS latency hides
    // behind a compute_tile
    int pgk[NH], pgv[NLV];
#pragma unroll
    for (int h = 0; h < NH; ++h) pgk[h] = 0;
    auto lookup = [&](int t0) {
        if constexpr (SRC == kSrcPaged) {
#pragma unroll
            for (int h = 0; h < NH; ++h)
                pgk[h] = sm.pages[(min(t0 + 16 * h + col, tend - 1) >> a.page_shift) - wpage0];
#pragma unroll
            for (int j = 0; j < NLV; ++j)
                pgv[j] = sm.pages[(min(t0 + (lane + kWave * j) / CPR, tend - 1) >> a.page_shift) - wpage0];
        } else {
            (void)t0;
        }
    };
    auto row_addr = [&](const void* base, const void* fresh, int pg, int t) -> const char* {
        if constexpr (SRC == kSrcPaged) {
            (void)fresh;
            pg = min(max(pg, 0), a.num_pages - 1);
            const int64_t r = (((int64_t)pg * a.G + pc.g) << a.page_shift) + (t & ((1 << a.page_shift) - 1));
            return static_cast<const char*>(base) + r * D * ES;
        } else if constexpr (SRC == kSrcAppend) {
            (void)pg;
            return t >= la ? static_cast<const char*>(fresh) + (nslab + (int64_t)(t - la) * D) * ES
                           : static_cast<const char*>(base) + (slab + (int64_t)t * D) * ES;
        } else {
            (void)fresh;
            (void)pg;
            return static_cast<const char*>(base) + (slab + (int64_t)t * D) * ES;
        }
    };

    // A tile is TR cache rows, NH halves h of 16.  Rows past the window's
    // end re-read its last row (valid): their weights are exactly 0, so no
    // row at or beyond the end is read and no branch guards the loads.
    // K: lane (kg, col) loads row 16 h + col of each half, elements
    // 8 kg + 32 s ..; V: chunk c = lane + 64 j is row c / CPR, elements
    // EPC (c % CPR) ..
    auto load_tile = [&](int t0, uint4* kk, uint4* vv) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const char* kr = row_addr(a.k, a.k_new, pgk[h], min(t0 + 16 * h + col, tend - 1));
            // bf16: elements kdim0(kg, s) .. + 7 for step s; fp8: 16 codes from
            // element 16 kg + 64 s (steps 2s and 2s + 1)
#pragma unroll
            for (int s = 0; s < NLK; ++s)
                kk[h * NLK + s] = load16_stream(kr + (KV8 ? 16 * kg + 64 * s : 2 * kdim0<D, KV8>(kg, s)));
        }
#pragma unroll
        for (int j = 0; j < NLV; ++j) {
            const int c = lane + kWave * j;
            vv[j] = load16_stream(row_addr(a.v, a.v_new, pgv[j], min(t0 + c / CPR, tend - 1)) + (c % CPR) * 16);
        }
        lookup(t0 + TR);
    };

    // Scores per half, S^T_h = K_h Q^T on v_mfma_f32_16x16x32_bf16 (lane
    // (kg, col) gets rows 4 kg .. 4 kg + 3 of half h for query row col), one
    // online-softmax step over the tile's rows, then O^T += V^T P^T: for a
    // 32-row tile on v_mfma_f32_16x16x32_bf16 whose k index 8 kg + i stands
    // for tile row 16 (i / 4) + 4 kg + i % 4 -- the rows whose weights lane
    // (kg, col) holds, and the rows the two LDS transpose reads of V deliver
    // to it; for a 16-row tile on v_mfma_f32_16x16x16_bf16 (k index 4 kg + i
    // is row 4 kg + i).
    auto compute_tile = [&](int t0, const uint4* kin, const uint4* vv) {
        uint4 kk[NH][NK];
        if constexpr (KV8) {
            // 16 fp8 codes -> two 8-element bf16 operands (exact)
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int s = 0; s < NLK; ++s) {
                    if constexpr (I8)
                        i8x16_to_bf16(kin[h * NLK + s], kk[h][2 * s], kk[h][2 * s + 1]);
                    else
                        fp8x16_to_bf16(kin[h * NLK + s], kk[h][2 * s], kk[h][2 * s + 1]);
                }
#pragma unroll
            for (int j = 0; j < NLV; ++j) {
                const int c = lane + kWave * j;
                uint4 lo, hi;
                if constexpr (I8)
                    i8x16_to_bf16(vv[j], lo, hi);
                else
                    fp8x16_to_bf16(vv[j], lo, hi);
                uint16_t* dst = &vt[(c / CPR) * SE + (c % CPR) * 16];
                *reinterpret_cast<uint4*>(dst) = lo;
                *reinterpret_cast<uint4*>(dst + 8) = hi;
            }
        } else {
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int s = 0; s < NK; ++s) kk[h][s] = kin[h * NLK + s];
#pragma unroll
            for (int j = 0; j < NLV; ++j) {
                const int c = lane + kWave * j;
                *reinterpret_cast<uint4*>(&vt[(c / CPR) * SE + (c % CPR) * 8]) = vv[j];
            }
        }
        if constexpr (SRC == kSrcAppend) {
            // the first row block's pieces store the new tokens' rows into the cache
            if (pc.rb == 0 && t0 + TR > la) {
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    const int tk = t0 + 16 * h + col;
                    if (tk >= la && tk < tend) {
                        char* kr = static_cast<char*>(const_cast<void*>(a.k)) + (slab + (int64_t)tk * D) * 2 + 16 * kg;
#pragma unroll
                        for (int s = 0; s < NK; ++s) *reinterpret_cast<uint4*>(kr + 64 * s) = kk[h][s];
                    }
                }
#pragma unroll
                for (int j = 0; j < NLV; ++j) {
                    const int c = lane + kWave * j;
                    const int tv = t0 + c / CPR;
                    if (tv >= la && tv < tend)
                        *reinterpret_cast<uint4*>(static_cast<char*>(const_cast<void*>(a.v)) +
                                                  (slab + (int64_t)tv * D) * 2 + (c % CPR) * 16) = vv[j];
                }
            }
        }
        uint32_t hw[NB][2 * NH], lw[NB][2 * NH];   // weights p = hi + lo, bf16 pairs
        // no row of the tile is past the window or after the first new token
        const bool full = t0 + TR <= tend && t0 + TR - 1 <= pc.L - a.sq;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            f32x4_t s4[NH];
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                s4[h] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < NK; ++s)
                    s4[h] = MX::mma16x32(kk[h][s], qb[nb][s], s4[h]);
            }
            float sc[4 * NH];
            float mx = -INFINITY;
            if (full) {
                // every row of the tile is visible to every new token (rows of
                // padding query rows are not masked either: their results are
                // never stored)
#pragma unroll
                for (int i = 0; i < 4 * NH; ++i) {
                    sc[i] = s4[i >> 2][i & 3] * score_scale;
                    mx = fmaxf(mx, sc[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4 * NH; ++i) {
                    const int t = t0 + 16 * (i >> 2) + 4 * kg + (i & 3);
                    sc[i] = (t < tend && t <= last[nb]) ? s4[i >> 2][i & 3] * score_scale : -INFINITY;
                    mx = fmaxf(mx, sc[i]);
                }
            }
            mx = max_x32(max_x16(mx));
            // the four lanes of a query row take the same decision
            const bool need = mx > m_run[nb] + kSlack;
            if (__builtin_amdgcn_ballot_w64(need) != 0) {
                const float al = need ? __builtin_amdgcn_exp2f(m_run[nb] - mx) : 1.0f;
                m_run[nb] = need ? mx : m_run[nb];
                l_run[nb] *= al;
#pragma unroll
                for (int c = 0; c < NC; ++c) acc[nb][c] *= al;
            }
            float pv[4 * NH];
#pragma unroll
            for (int i = 0; i < 4 * NH; ++i) {
                // in a full tile every score is finite and so is m_run
                pv[i] = (!full && sc[i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[i] - m_run[nb]);
                l_run[nb] += pv[i];
            }
#pragma unroll
            for (int q = 0; q < 2 * NH; ++q) {
                hw[nb][q] = MX::pack2(pv[2 * q], pv[2 * q + 1]);
                lw[nb][q] = MX::resid2(pv[2 * q], pv[2 * q + 1], hw[nb][q]);
            }
        }
        // lane (kg, col) addresses row 4 kg + col / 4 (of each half), columns
        // 4 (col % 4) .. of each 16-column block and receives
        // V^T[col][4 kg .. 4 kg + 3] of the half
        const uint16_t* vr = vt + (4 * kg + (col >> 2)) * SE + 4 * (col & 3);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const uint2 v0 = __builtin_bit_cast(uint2, lds_read_tr16(vr + 16 * c));
            if constexpr (NH == 2) {
                const uint2 v1 = __builtin_bit_cast(uint2, lds_read_tr16(vr + 16 * SE + 16 * c));
                const uint4 va = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    acc[nb][c] = MX::mma16x32(va, make_uint4(hw[nb][0], hw[nb][1], hw[nb][2], hw[nb][3]), acc[nb][c]);
                    acc[nb][c] = MX::mma16x32(va, make_uint4(lw[nb][0], lw[nb][1], lw[nb][2], lw[nb][3]), acc[nb][c]);
                }
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    acc[nb][c] = MX::mma16x16(v0, make_uint2(hw[nb][0], hw[nb][1]), acc[nb][c]);
                    acc[nb][c] = MX::mma16x16(v0, make_uint2(lw[nb][0], lw[nb][1]), acc[nb][c]);
                }
            }
        }
    };

    // NBUF register buffers in rotation, NBUF - 1 tiles' loads in flight
    // while one is computed.  The loads are unconditional (rows clamped into
    // the window), so the compiler waits for exactly the oldest tile.  A
    // paged cache walks the piece in row windows whose pages fit the LDS
    // copy of the block table (one window unless the piece spans more than
    // kPageWindow pages).  An append reads each row from the cache or, for
    // the new tokens' rows, from k_new / v_new, in one window.
    for (int w0 = ta; w0 < tb; w0 = tend) {
        if constexpr (SRC == kSrcPaged) {
            wpage0 = w0 >> a.page_shift;
            tend = (int)min((long long)tb, (long long)(wpage0 + kPageWindow) << a.page_shift);
            const int np = ((tend - 1) >> a.page_shift) - wpage0 + 1;
            const int32_t* bt = a.block_table + (int64_t)pc.b * a.max_pages + wpage0;
            wave_lds_fence();            // the previous window's page reads are done
            for (int i = lane; i < np; i += kWave) sm.pages[i] = bt[i];
            wave_lds_fence();
        }
        lookup(w0);
        constexpr int NBUF = mfa_buffers<NB, KV8>();
        uint4 kb[NBUF][NH * NLK], vb[NBUF][NLV];
        int t0 = w0;
        const int ntile = (tend - w0 + TR - 1) / TR;
#pragma unroll
        for (int u = 0; u < NBUF - 1; ++u) load_tile(t0 + TR * u, kb[u], vb[u]);
        for (int it = 0; it < ntile; it += NBUF) {
#pragma unroll
            for (int u = 0; u < NBUF; ++u) {
                if (it + u >= ntile) break;
                const int nxt = (u + NBUF - 1) % NBUF;
                load_tile(t0 + TR * (NBUF - 1), kb[nxt], vb[nxt]);
                compute_tile(t0, kb[u], vb[u]);
                t0 += TR;
            }
        }
    }

    if constexpr (NW > 1) {
        // waves 1 .. NW - 1 hand (m, per-lane sum, accumulators) to wave 0,
        // which rescales each to the common max and adds them up (a wave
        // with no visible row has m = -inf and weight 0)
        constexpr int NV = NB * (2 + 4 * NC);
        static_assert(NV == SM::NV, "exchange layout");
        const int w = threadIdx.x / kWave;
        if (w > 0) {
            float (*x)[kWave] = sm.xch[w - 1];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                x[nb * (2 + 4 * NC)][lane] = m_run[nb];
                x[nb * (2 + 4 * NC) + 1][lane] = l_run[nb];
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int q = 0; q < 4; ++q) x[nb * (2 + 4 * NC) + 2 + 4 * c + q][lane] = acc[nb][c][q];
            }
        }
        __syncthreads();
        if (w == 0) {
#pragma unroll
            for (int u = 0; u < NW - 1; ++u) {
                const float (*x)[kWave] = sm.xch[u];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const float mw = x[nb * (2 + 4 * NC)][lane];
                    const float M = fmaxf(m_run[nb], mw);
                    const float fa = m_run[nb] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[nb] - M);
                    const float fb = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
                    m_run[nb] = M;
                    l_run[nb] = l_run[nb] * fa + x[nb * (2 + 4 * NC) + 1][lane] * fb;
#pragma unroll
                    for (int c = 0; c < NC; ++c)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[nb][c][q] = acc[nb][c][q] * fa + x[nb * (2 + 4 * NC) + 2 + 4 * c + q][lane] * fb;
                }
            }
        }
        __syncthreads();                 // the exchange area is free again
        if (w > 0) return false;
    }

    // ---- end of the piece ------------------------------------------------------
    // int8 codes: the weighted sum ran over c + 128, so 128 v_scale comes off
    // every finished row (rows that see nothing stay 0)
    float inv[NB], lse[NB], sub[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float l = sum_x32(sum_x16(l_run[nb]));
        inv[nb] = l > 0.0f ? out_scale / l : 0.0f;
        lse[nb] = l > 0.0f ? m_run[nb] + __log2f(l) : -INFINITY;
        sub[nb] = (I8 && l > 0.0f) ? 128.0f * out_scale : 0.0f;
    }
    const int c_first = cm.of(pc.off);
    const int npieces = cm.of(pc.off + pc.L - 1) - c_first + 1;
    if (npieces == 1) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if (!live[nb]) continue;
            float* o = a.out + (qrow0 + 16 * nb + col) * D + 4 * kg;
#pragma unroll
            for (int c = 0; c < NC; ++c) *reinterpret_cast<f32x4_t*>(o + 16 * c) = acc[nb][c] * inv[nb] - sub[nb];
        }
        return false;
    }
    const __amdgpu_buffer_rsrc_t part = part_rsrc(a.part);
    const MSlots ms = mslots<D>(a);
    const int mine = ms.base(chunk, cm.start(chunk) >= pc.off ? 0 : 1);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        if (!live[nb]) continue;
        const int r = 16 * nb + col;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const f32x4_t o = acc[nb][c] * inv[nb] - sub[nb];
            const float ov[4] = {o[0], o[1], o[2], o[3]};
            store4_coherent(part, mine + r * D + 16 * c + 4 * kg, ov);
        }
        if (kg == 0) store_coherent(part, mine + ms.lse + r, lse[nb]);
    }
    pd->seg = (pc.b * a.G + pc.g) * n_rb + pc.rb;
    pd->p_first = c_first;
    pd->npieces = npieces;
    pd->off = pc.off;
    pd->qrow0 = qrow0;
    pd->row0 = row0;
    return true;
}

// Merge of a segment's partials by its last arrival (slots of RB rows of D
// values, then the rows' log2-sum-exp), in piece order.  The live rows are
// spread over the wave, LPR lanes per row, NF float4 of the row per lane;
// KB pieces are loaded at a time, all their loads in flight together.
template <int D, int NF, int KB>
__device__ __forceinline__ void merge_pieces(const Args& a, const Pending& pd, int lane, int r0, int rows,
                                             const ChunkMap& cm)
{
    constexpr int LPR = D / (4 * NF);
    const __amdgpu_buffer_rsrc_t part = part_rsrc(a.part);
    const MSlots ms = mslots<D>(a);
    const int i = lane / LPR;
    const int ic = r0 + min(i, rows - 1);
    const int e0 = (lane % LPR) * 4 * NF;
    float M = -INFINITY, den = 0.0f;
    float num[NF][4];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) num[f][q] = 0.0f;
    const bool tail1 = cm.start(pd.p_first) < pd.off;
    for (int k0 = 0; k0 < pd.npieces; k0 += KB) {
        float lse[KB], ov[KB][NF][4];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            const int k = min(k0 + kk, pd.npieces - 1);
            const int base = ms.base(pd.p_first + k, k == 0 && tail1 ? 1 : 0);
            lse[kk] = load_coherent(part, base + ms.lse + ic);
#pragma unroll
            for (int f = 0; f < NF; ++f) load4_coherent(part, base + ic * D + e0 + 4 * f, ov[kk][f]);
        }
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            float w;
            const float sc = lse_step(M, k0 + kk < pd.npieces ? lse[kk] : -INFINITY, &w);
            den = fmaf(den, sc, w);
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int q = 0; q < 4; ++q) num[f][q] = fmaf(num[f][q], sc, w * ov[kk][f][q]);
        }
    }
    if (i < rows) {
        const float inv = den > 0.0f ? 1.0f / den : 0.0f;
        float* o = a.out + (pd.qrow0 + r0 + i) * D + e0;
#pragma unroll
        for (int f = 0; f < NF; ++f)
            *reinterpret_cast<float4*>(o + 4 * f) =
                make_float4(num[f][0] * inv, num[f][1] * inv, num[f][2] * inv, num[f][3] * inv);
    }
}

// merge_pieces with its load batch cut to the piece count: a segment split in
// 2-4 pieces (the common case when the workgroups outnumber the segments a
// few times) loads 4 pieces per batch instead of re-loading its last piece up
// to 16 times (the merge on the step's critical path: batched GQA-8
// 63.6 -> 62.8 us, fp8 40.9 -> 39.8, append 64.3 -> 63.2).
template <int D, int NF, int KBMAX>
__device__ __forceinline__ void merge_pieces_n(const Args& a, const Pending& pd, int lane, int r0, int rows,
                                               const ChunkMap& cm)
{
    if (pd.npieces <= 4)
        merge_pieces<D, NF, (KBMAX < 4 ? KBMAX : 4)>(a, pd, lane, r0, rows, cm);
    else if (pd.npieces <= 8)
        merge_pieces<D, NF, (KBMAX < 8 ? KBMAX : 8)>(a, pd, lane, r0, rows, cm);
    else
        merge_pieces<D, NF, KBMAX>(a, pd, lane, r0, rows, cm);
}

// Count this wave's arrival for a pending segment of RB rows; the last
// arrival merges, 16 rows at a time (choosing the lane layout by the number
// of live rows), and resets the counter.  The caller has waited for its own
// partial stores.
template <int D, int RB>
__device__ __forceinline__ void arrive_and_merge_mfa(const Args& a, const Pending& pd, int lane, int R,
                                                     const ChunkMap& cm)
{
    int old = 0;
    if (lane == 0)
        old = __hip_atomic_fetch_add(&a.counters[pd.seg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0);
    if (old != pd.npieces - 1) return;
    arrival_before_partial_loads();
    const int live_rows = min(RB, R - pd.row0);
    for (int r0 = 0; r0 < live_rows; r0 += 16) {
        const int rows = min(16, live_rows - r0);
        // lanes per row: 64 / (rows rounded up to a power of two), at most D / 4;
        // about 32 to 48 loads of a batch in flight per lane
        if (rows > 8)
            merge_pieces_n<D, D / 16, (D == 128 ? 4 : 8)>(a, pd, lane, r0, rows, cm);
        else if (rows > 4)
            merge_pieces_n<D, D / 32, (D == 128 ? 8 : 16)>(a, pd, lane, r0, rows, cm);
        else if (rows > 2 || D == 64)
            merge_pieces_n<D, (D == 128 ? 2 : 1), 16>(a, pd, lane, r0, rows, cm);
        else
            merge_pieces_n<D, 1, 16>(a, pd, lane, r0, rows, cm);
    }
    if (lane == 0) __hip_atomic_store(&a.counters[pd.seg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int NB, int SRC, bool KV8, bool F16 = false, bool I8 = false>
__global__ void __launch_bounds__(kWave)
decode_mfa(const int32_t* __restrict__ lens_in, const int nB, const int nT, const Args a, const int R, const int n_rb)
{
    // the piece walk on scalar registers for the plain bf16 cache with one
    // query block (batched GQA-8 decode 61.75 -> 60.79 us, the sq = 2 sweep
    // at G = 8 158.7 -> 157.5); the other variants run out of scalar
    // registers with it (spills to vector lanes; appended tokens 60.9 -> 61.8)
    constexpr bool kScalarWalk = SRC == kSrcCache && !KV8 && NB == 1;
    __shared__ MfaShared<D> sm;
    const int P = gridDim.x;
    const int p = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    for (int i = lane; i < kLensWindow && i < nB; i += kWave) sm.lens[i] = clamp_len(lens_in, i, nT);
    zero_empty_sequences<D>(a, P, p);
    wave_lds_fence();
    const int units = a.G * n_rb;
    const int chunk = p;
    ChunkPlan cp;
    if (!plan_chunk<kScalarWalk>(a, sm.lens, units, P, chunk, cp)) return;
    const ChunkMap& cm = cp.cm;
    CostPieceIter<kScalarWalk> it;
    it.init(cp.vA, cp.vE, cp.fb, cp.fv, a.G, n_rb);
    Piece pc;
    while (it.next(a, sm.lens, pc)) {
        Pending pd;
        if (mfa_piece<D, NB, SRC, KV8, 1, MfaShared<D>, F16, I8>(a, sm, R, n_rb, pc, cm, chunk, &pd) &&
            !a.deferred) {
            partials_stored_before_arrival();    // own partial stores complete at device scope
            arrive_and_merge_mfa<D, 16 * NB>(a, pd, lane, R, cm);
        }
    }
}

// The same pass with NW waves per workgroup, one per SIMD, splitting every
// piece's cache rows among them (contiguous runs of whole tiles); wave 0
// combines the waves' results in LDS and finishes the piece.  For small
// caches, where a one-wave workgroup's stream is bound by its own load
// latency and per-tile chain rather than by HBM, this puts NW waves' loads in
// flight per workgroup without adding pieces, partials or merges.
template <int D, int NB, int NW, bool F16 = false>
__global__ void __launch_bounds__(kWave * NW)
decode_mfs(const int32_t* __restrict__ lens_in, const int nB, const int nT, const Args a, const int R, const int n_rb)
{
    __shared__ MfsShared<D, NB, NW> sm;
    const int P = gridDim.x;
    const int p = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    for (int i = threadIdx.x; i < kLensWindow && i < nB; i += kWave * NW) sm.lens[i] = clamp_len(lens_in, i, nT);
    zero_empty_sequences<D>(a, P, p);
    __syncthreads();
    const int units = a.G * n_rb;
    const int chunk = p;
    ChunkPlan cp;
    if (!plan_chunk<false>(a, sm.lens, units, P, chunk, cp)) return;
    const ChunkMap& cm = cp.cm;
    CostPieceIter<false> it;
    it.init(cp.vA, cp.vE, cp.fb, cp.fv, a.G, n_rb);
    Piece pc;
    while (it.next(a, sm.lens, pc)) {
        Pending pd;
        if (mfa_piece<D, NB, kSrcCache, false, NW, MfsShared<D, NB, NW>, F16>(a, sm, R, n_rb, pc, cm, chunk, &pd) &&
            !a.deferred) {
            partials_stored_before_arrival();    // own partial stores complete at device scope
            arrive_and_merge_mfa<D, 16 * NB>(a, pd, lane, R, cm);
        }
    }
}

// ---------------------------------------------------------------------------
// Matrix-core pass for groups of more than 32 query rows.  A workgroup of NW
// waves (NW = 4 or 8) owns segments of 16 NW query rows; wave w computes rows
// 16 w .. 16 w + 15, and the NW waves share every K/V tile of 32 cache rows:
// the workgroup loads it once (each thread a share of its 16-byte chunks,
// one tile ahead in registers) and stages it in LDS, double-buffered, one
// barrier per tile.  Compared with one wave carrying all the blocks, the
// blocks' arithmetic runs on NW SIMDs at once, and a split segment's merge
// is shared by the NW waves too.
// ---------------------------------------------------------------------------
template <int D, int NW>
struct MfwShared {
    static constexpr int TR = 32;       // cache rows per tile
    static constexpr int SK = D + 8;    // K row stride (bf16): the 16 rows of an A-operand read hit distinct banks
    static constexpr int SE = D + 16;   // V row stride, as in MfaShared
    alignas(16) uint16_t kt[2][TR * SK];
    alignas(16) uint16_t vt[2][TR * SE];
    int lens[kLensWindow];              // clamped seq_lens[i]
    int merge;                          // 1 when this workgroup arrived last for the current piece
};

template <int D, int NW>
__device__ __forceinline__ bool mfw_piece(const Args& a, MfwShared<D, NW>& sm, int R, const Piece& pc,
                                          const ChunkMap& cm, int chunk, int n_rb, Pending* pd)
{
    constexpr int NK = D / 32;
    constexpr int NC = D / 16;
    constexpr int SK = MfwShared<D, NW>::SK;
    constexpr int SE = MfwShared<D, NW>::SE;
    constexpr int TR = MfwShared<D, NW>::TR;
    constexpr int CPR = D / 8;           // 16-byte chunks per cache row
    constexpr int NT = kWave * NW;       // threads of the workgroup
    constexpr int NCH = (TR * CPR + NT - 1) / NT;   // K chunks (and V chunks) per thread per tile
    constexpr int RB = 16 * NW;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int col = lane & 15;
    const int kg = lane >> 4;
    const int ta = pc.ta, tb = pc.tb;
    const int row0 = pc.rb * RB;
    const int64_t qrow0 = (int64_t)pc.b * a.H * a.sq + (int64_t)pc.g * R + row0;
    const int r = row0 + 16 * w + col;   // this lane's query row (score / output column)
    const bool live = r < R;
    const int last = live ? pc.L - a.sq + (r % a.sq) : -1;
    // with D = 64 and four waves half of the threads have no chunk
    auto has = [&](int j) { return (TR * CPR) % NT == 0 || tid + NT * j < TR * CPR; };

    uint4 qb[NK];
    {
        const char* qp = static_cast<const char*>(a.q) + (qrow0 + (live ? 16 * w + col : 0)) * D * 2;
#pragma unroll
        for (int s = 0; s < NK; ++s) qb[s] = load16(qp + 2 * kdim0<D, false>(kg, s));
    }
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4_t acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t slab = ((int64_t)pc.b * a.G + pc.g) * a.T * D;
    const char* kbase = static_cast<const char*>(a.k) + slab * 2;
    const char* vbase = static_cast<const char*>(a.v) + slab * 2;

    // chunk c = tid + NT j of a tile: row c / CPR, elements 8 (c % CPR) ..;
    // rows past the piece's end re-read its last row (weight 0)
    auto load_tile = [&](int t0, uint4* kk, uint4* vv) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int c = min(tid + NT * j, TR * CPR - 1);
            const int64_t off = ((int64_t)min(t0 + c / CPR, tb - 1) * D + (c % CPR) * 8) * 2;
            kk[j] = load16_stream(kbase + off);
            vv[j] = load16_stream(vbase + off);
        }
    };
    auto stage = [&](int buf, const uint4* kk, const uint4* vv) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int c = tid + NT * j;
            if (!has(j)) continue;
            *reinterpret_cast<uint4*>(&sm.kt[buf][(c / CPR) * SK + (c % CPR) * 8]) = kk[j];
            *reinterpret_cast<uint4*>(&sm.vt[buf][(c / CPR) * SE + (c % CPR) * 8]) = vv[j];
        }
    };
    // A tile is two 16-row halves h: scores S^T_h = K_h Q^T on
    // v_mfma_f32_16x16x32_bf16 (lane (kg, col) gets rows 4 kg .. 4 kg + 3 of
    // half h for query row col), then one online-softmax step over the 32
    // rows, and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 with its k index
    // 8 kg + i standing for tile row 16 (i / 4) + 4 kg + i % 4 -- the rows
    // lane (kg, col) already holds the weights of, and the rows the two
    // transpose reads of V deliver.
    auto compute = [&](int buf, int t0) {
        f32x4_t s4[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint4 kk[NK];
#pragma unroll
            for (int s = 0; s < NK; ++s)
                kk[s] = *reinterpret_cast<const uint4*>(&sm.kt[buf][(16 * h + col) * SK + kdim0<D, false>(kg, s)]);
            s4[h] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < NK; ++s)
                s4[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kk[s]),
                                                                __builtin_bit_cast(bf16x8_t, qb[s]), s4[h], 0, 0, 0);
        }
        const bool full = t0 + TR <= tb && t0 + TR - 1 <= pc.L - a.sq;
        float sc[8];
        float mx = -INFINITY;
        if (full) {
            // one uniform branch: every row of the tile is visible to every query row
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sc[i] = s4[i >> 2][i & 3] * a.scale_log2;
                mx = fmaxf(mx, sc[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = t0 + 16 * (i >> 2) + 4 * kg + (i & 3);
                sc[i] = (t < tb && t <= last) ? s4[i >> 2][i & 3] * a.scale_log2 : -INFINITY;
                mx = fmaxf(mx, sc[i]);
            }
        }
        mx = max_x32(max_x16(mx));
        const bool need = mx > m_run + kSlack;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float al = need ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;
            m_run = need ? mx : m_run;
            l_run *= al;
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[c] *= al;
        }
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pv[i] = (!full && sc[i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[i] - m_run);
            l_run += pv[i];
        }
        // p = hi + lo, both bf16
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            hw[q] = pack_bf16x2(pv[2 * q], pv[2 * q + 1]);
            lw[q] = pack_bf16x2(pv[2 * q] - __uint_as_float(hw[q] << 16),
                                pv[2 * q + 1] - __uint_as_float(hw[q] & 0xFFFF0000u));
        }
        const bf16x8_t ph = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
        const uint16_t* vr = sm.vt[buf] + (4 * kg + (col >> 2)) * SE + 4 * (col & 3);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const uint2 v0 = __builtin_bit_cast(uint2, lds_read_tr16(vr + 16 * c));
            const uint2 v1 = __builtin_bit_cast(uint2, lds_read_tr16(vr + 16 * SE + 16 * c));
            const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y));
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph, acc[c], 0, 0, 0);
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl, acc[c], 0, 0, 0);
        }
    };

    // Iteration i stages tile i + 1 (loaded during iteration i - 1) into
    // LDS buffer (i + 1) & 1, issues the loads of tile i + 2 into the
    // registers just freed, and computes tile i from buffer i & 1; the
    // barrier after each tile orders the staging for the next.
    {
        uint4 kr[2][NCH], vr[2][NCH];
        const int ntile = (tb - ta + TR - 1) / TR;
        load_tile(ta, kr[0], vr[0]);
        load_tile(ta + TR, kr[1], vr[1]);
        stage(0, kr[0], vr[0]);
        __syncthreads();
        for (int it = 0; it < ntile; it += 2) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int i = it + u;
                if (i >= ntile) break;
                if (i + 1 < ntile) stage((i + 1) & 1, kr[1 - u], vr[1 - u]);
                load_tile(ta + TR * (i + 2), kr[u], vr[u]);
                compute(i & 1, ta + TR * i);
                __syncthreads();
            }
        }
    }

    // ---- end of the piece ------------------------------------------------------
    const float l = sum_x32(sum_x16(l_run));
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float lse = l > 0.0f ? m_run + __log2f(l) : -INFINITY;
    const int c_first = cm.of(pc.off);
    const int npieces = cm.of(pc.off + pc.L - 1) - c_first + 1;
    if (npieces == 1) {
        if (live) {
            float* o = a.out + (qrow0 + 16 * w + col) * D + 4 * kg;
#pragma unroll
            for (int c = 0; c < NC; ++c) *reinterpret_cast<f32x4_t*>(o + 16 * c) = acc[c] * inv;
        }
        return false;
    }
    const __amdgpu_buffer_rsrc_t part = part_rsrc(a.part);
    const MSlots ms = mslots<D>(a);
    const int mine = ms.base(chunk, cm.start(chunk) >= pc.off ? 0 : 1);
    if (live) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const f32x4_t o = acc[c] * inv;
            const float ov[4] = {o[0], o[1], o[2], o[3]};
            store4_coherent(part, mine + (16 * w + col) * D + 16 * c + 4 * kg, ov);
        }
        if (kg == 0) store_coherent(part, mine + ms.lse + 16 * w + col, lse);
    }
    pd->seg = (pc.b * a.G + pc.g) * n_rb + pc.rb;
    pd->p_first = c_first;
    pd->npieces = npieces;
    pd->off = pc.off;
    pd->qrow0 = qrow0;
    pd->row0 = row0;
    return true;
}

// Merge of this wave's 16 rows of a segment (rows r0 .. r0 + rows - 1 of
// its slots), choosing the lane layout by the number of live rows.
template <int D>
__device__ __forceinline__ void merge_block16(const Args& a, const Pending& pd, int lane, int r0, int rows,
                                              const ChunkMap& cm)
{
    if (rows > 8)
        merge_pieces<D, D / 16, (D == 128 ? 4 : 8)>(a, pd, lane, r0, rows, cm);
    else if (rows > 4)
        merge_pieces<D, D / 32, (D == 128 ? 8 : 16)>(a, pd, lane, r0, rows, cm);
    else if (rows > 2 || D == 64)
        merge_pieces<D, (D == 128 ? 2 : 1), 16>(a, pd, lane, r0, rows, cm);
    else
        merge_pieces<D, 1, 16>(a, pd, lane, r0, rows, cm);
}

template <int D, int NW>
__global__ void __launch_bounds__(kWave * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_mfw(const int32_t* __restrict__ lens_in, const int nB, const int nT, const Args a, const int R, const int n_rb)
{
    __shared__ MfwShared<D, NW> sm;
    const int P = gridDim.x;
    const int p = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    for (int i = tid; i < kLensWindow && i < nB; i += kWave * NW) sm.lens[i] = clamp_len(lens_in, i, nT);
    zero_empty_sequences<D>(a, P, p);
    __syncthreads();
    const int units = a.G * n_rb;
    const int chunk = p;
    ChunkPlan cp;
    if (!plan_chunk<false>(a, sm.lens, units, P, chunk, cp)) return;
    const ChunkMap& cm = cp.cm;
    CostPieceIter<false> it;
    it.init(cp.vA, cp.vE, cp.fb, cp.fv, a.G, n_rb);
    Piece pc;
    while (it.next(a, sm.lens, pc)) {
        Pending pd;
        if (mfw_piece<D, NW>(a, sm, R, pc, cm, chunk, n_rb, &pd) && !a.deferred) {
            partials_stored_before_arrival();    // this wave's partial stores complete at device scope
            __syncthreads();                 // ... and every other wave's
            if (tid == 0) {
                const int old = __hip_atomic_fetch_add(&a.counters[pd.seg], 1, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
                sm.merge = old == pd.npieces - 1;
                if (sm.merge) __hip_atomic_store(&a.counters[pd.seg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            arrival_before_partial_loads();
            if (sm.merge) {
                const int rows = min(16, min(16 * NW, R - pd.row0) - 16 * w);
                if (rows > 0) merge_block16<D>(a, pd, lane, 16 * w, rows, cm);
            }
            __syncthreads();                 // sm.merge is rewritten by the next piece
        }
    }
}

// ---------------------------------------------------------------------------
// Matrix-core pass on 32 x 32 tiles (v_mfma_f32_32x32x16_bf16), for groups
// of more than 32 query rows of a bf16 cache.
//
// A workgroup has four waves, one per SIMD, and owns segments of
// RB = 32 QB NQ query rows; it streams its chunk's pieces in 32-row K/V
// tiles.  Its waves are NQ query groups x NS splits (NQ NS = 4):
//   * a wave computes QB blocks of 32 query rows (all rows of its query
//     group) against the tiles of its split;
//   * the NQ waves of a split share each of its tiles: they load it once
//     (coalesced 16-byte loads, every thread a share) into LDS;
//   * split s takes tiles s, s + NS, s + 2 NS, ... of a piece, and at the
//     piece's end the splits' running (max, sum, weighted V sum) merge
//     through LDS -- so a piece spans NS times the rows a single wave would
//     stream, and a segment is cut into NS times fewer pieces (fewer
//     partials to write and merge).
// NQ = 1 (up to 64 rows): every wave streams its own tiles, no barrier per
// tile; NS = 1 (more than 128 rows): one K/V read serves 256 query rows.
//
// Per tile and 32-row query block (lane l: query row l % 32, k half
// h = l / 32):
//   S^T[t][r] = K[t][:] . Q[r][:]      A = K (row l % 32, elements
//                                      16 s + 8 h .. + 7 at step s),
//                                      B = Q^T (same elements of row l % 32)
//   the accumulator gives lane l the scores of query row l % 32 at tile rows
//   8 i + 4 h + j (index 4 i + j), so a row's max and sum need only the lane
//   pair (l, l ^ 32);
//   O^T[d][r] += V^T[d][t] P^T[t][r]   k step u covers tile rows 16 u ..:
//                                      k index 8 h + e stands for tile row
//                                      16 u + 8 (e / 4) + 4 h + e % 4 -- the
//                                      rows whose weights lane l already
//                                      holds (scores 8 u + e), and the rows
//                                      two LDS transpose reads of V deliver.
// Weights enter as bf16 hi + lo (about 16 bits), V is exact, accumulation
// fp32 -- as in the 16 x 16 pass.
//
// LDS tiles are padded so that every access is free of bank conflicts and
// every lane's addresses differ by compile-time constants: K rows are 2 D + 16
// bytes apart (the 16 rows of an A-operand read start 4 banks apart), V rows
// 2 D + 64 bytes apart (the 4 rows x 64 bytes a transpose read covers per 32
// lanes start 16 banks apart); the row-contiguous stores of 16 lanes cover
// one row.
// ---------------------------------------------------------------------------
template <int D>
struct MfxGeom {
    static constexpr int TR = 32;               // cache rows per tile
    static constexpr int CPR = D / 8;           // 16-byte chunks per cache row
    static constexpr int TILE_CH = TR * CPR;    // chunks of K (and of V) per tile
    static constexpr int NKS = D / 16;          // k steps of the score product
    static constexpr int NDB = D / 32;          // 32-column blocks of the weighted sum
    static constexpr int SK = 2 * D + 16;       // K row stride in LDS (bytes)
    static constexpr int SV = 2 * D + 64;       // V row stride in LDS (bytes)
};

template <int D>
struct MfxTile {
    alignas(16) char k[32 * MfxGeom<D>::SK];
    alignas(16) char v[32 * MfxGeom<D>::SV];
};

// A wave that streams its own tiles (NQ = 1) needs one LDS buffer (its
// accesses run in order); waves sharing tiles need two.
template <int D, int QB, int NQ, int NS>
struct MfxShared {
    static constexpr int NBUF = NQ > 1 ? 2 : 1;
    static constexpr int OS = D + 4;      // row stride (floats) of a wave's staged output rows
    union {
        MfxTile<D> t[NS][NBUF];
        float out[NQ][QB * 32 * OS];      // piece end: the results, staged for coalesced stores
    };
    float ml[2][NS][NQ * QB * 32];        // piece merge: each row's max and sum per split
    int lens[kLensWindow];                // clamped seq_lens[i]
    int merge;                            // 1 when this workgroup arrived last for the current piece
};


// Tiles of loads in flight per thread: one per wave when each wave streams
// its own tiles (64 registers each); two when waves share a tile (four, with
// two waves per tile, measured slower: G = 1 sweep 42.2 -> 47.2 us, the AGPR
// copies of the extra registers slowing every phase).
template <int NQ>
constexpr int mfx_reg_tiles() { return NQ == 1 ? 1 : 2; }

template <int D, int QB, int NQ, int NS, bool F16 = false>
__device__ __forceinline__ bool mfx_piece(const Args& a, MfxShared<D, QB, NQ, NS>& sm, int R, const Piece& pc,
                                          const ChunkMap& cm, int chunk, int n_rb, Pending* pd)
{
    using Gm = MfxGeom<D>;
    constexpr int TR = Gm::TR, CPR = Gm::CPR, NKS = Gm::NKS, NDB = Gm::NDB, SK = Gm::SK, SV = Gm::SV;
    constexpr int NBUF = MfxShared<D, QB, NQ, NS>::NBUF;
    constexpr int RB = 32 * QB * NQ;
    constexpr int NTG = kWave * NQ;                 // threads sharing a split's tiles
    constexpr int NCH = (Gm::TILE_CH + NTG - 1) / NTG;   // K (and V) chunks per thread per tile
    constexpr int NREG = mfx_reg_tiles<NQ>();

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int qs = w % NQ;                          // query group of this wave
    const int sp = w / NQ;                          // split of this wave
    const int gtid = qs * kWave + lane;             // thread within the split's group
    // with D = 64 and eight query groups half of the threads have no chunk
    auto has = [&](int j) { return Gm::TILE_CH % NTG == 0 || gtid + NTG * j < Gm::TILE_CH; };
    const int col = lane & 31;                      // query row within a block; A-operand row
    const int hf = lane >> 5;                       // k half
    const int ta = pc.ta, tb = pc.tb;
    const int row0 = pc.rb * RB;
    const int wrow0 = qs * 32 * QB;                 // this wave's first row within the segment
    const int64_t qrow0 = (int64_t)pc.b * a.H * a.sq + (int64_t)pc.g * R + row0;

    // B operands of the score product: query row wrow0 + 32 qb + col; a row
    // past R reads the segment's first row instead (its results are never
    // stored, and no select waits on the loaded values before the first
    // tile's loads are issued)
    uint4 qop[QB][NKS];
    bool live[QB];
    int last[QB];
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int r = row0 + wrow0 + 32 * qb + col;
        live[qb] = r < R;
        last[qb] = live[qb] ? pc.L - a.sq + (r % a.sq) : -1;
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.0f;
        const char* qp = static_cast<const char*>(a.q) + (qrow0 + (live[qb] ? wrow0 + 32 * qb + col : 0)) * D * 2;
#pragma unroll
        for (int s = 0; s < NKS; ++s) qop[qb][s] = load16(qp + 2 * (16 * s + 8 * hf));
    }
    f32x16_t acc[QB][NDB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x16_t{};

    const int64_t slab = ((int64_t)pc.b * a.G + pc.g) * a.T * D;
    const char* kbase = static_cast<const char*>(a.k) + slab * 2;
    const char* vbase = static_cast<const char*>(a.v) + slab * 2;
    const int ntile_all = (tb - ta + TR - 1) / TR;
    const int ntile = ntile_all > sp ? (ntile_all - sp + NS - 1) / NS : 0;   // tiles of this split
    MfxTile<D>* bufs = sm.t[sp];

    // tile i of this split: cache rows ta + TR (sp + NS i) ..; chunk c =
    // gtid + NTG j is row c / CPR, elements 8 (c % CPR) ..; rows past the
    // piece's end re-read its last row (weight 0)
    auto load = [&](int i, uint4* kk, uint4* vv) {
        const int t0 = ta + TR * (sp + NS * i);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int c = min(gtid + NTG * j, Gm::TILE_CH - 1);
            const int64_t off = ((int64_t)min(t0 + c / CPR, tb - 1) * D + (c % CPR) * 8) * 2;
            kk[j] = load16_stream(kbase + off);
            vv[j] = load16_stream(vbase + off);
        }
    };
    auto stage = [&](int buf, const uint4* kk, const uint4* vv) {
        char* kt = bufs[buf % NBUF].k;
        char* vt = bufs[buf % NBUF].v;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            if (!has(j)) continue;
            const int c = gtid + NTG * j;
            const int r = c / CPR, cc = c % CPR;
            *reinterpret_cast<uint4*>(kt + r * SK + cc * 16) = kk[j];
            *reinterpret_cast<uint4*>(vt + r * SV + cc * 16) = vv[j];
        }
    };
    // Scores are scaled inside the exponent: p = 2^(c s - m) with
    // c = |scale * log2 e|, one FMA per score, and a row's maximum of c s is
    // c times its raw maximum; a negative scale flips the sign of every query
    // element instead (exact in bf16; applied once the first tile is in).
    const float csc = fabsf(a.scale_log2);
    const uint32_t qsign = a.scale_log2 < 0.0f ? 0x80008000u : 0u;

    // One tile: scores of every query block, one K step (A operand) at a
    // time; then per block one online-softmax step and the weighted V sum.
    // FULL: no row of the tile is past the piece or after the first new
    // token, so nothing is masked (a uniform branch selects the variant: the
    // masking costs a third of the softmax's instructions).
    auto compute = [&](int buf, int t0, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const char* kt = bufs[buf % NBUF].k;
        const char* vt = bufs[buf % NBUF].v;
        f32x16_t s16q[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s16q[qb] = f32x16_t{};
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const uint4 kop = *reinterpret_cast<const uint4*>(kt + col * SK + (2 * s + hf) * 16);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s16q[qb] = Mx<F16>::mma32x16(kop, qop[qb][s], s16q[qb]);
        }
        uint32_t ph[QB][8], pl[QB][8];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float sc[16];
            float mx;
            if constexpr (FULL) {
#pragma unroll
                for (int v = 0; v < 16; ++v) sc[v] = s16q[qb][v];
                float m4[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    m4[k] = fmaxf(fmaxf(sc[4 * k], sc[4 * k + 1]), fmaxf(sc[4 * k + 2], sc[4 * k + 3]));
                mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
                mx = max_x32(mx) * csc;
            } else {
                mx = -INFINITY;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int t = t0 + 8 * (v >> 2) + 4 * hf + (v & 3);
                    sc[v] = (t < tb && t <= last[qb]) ? s16q[qb][v] : -INFINITY;
                    mx = fmaxf(mx, sc[v]);
                }
                mx = max_x32(mx);
                mx = mx == -INFINITY ? -INFINITY : mx * csc;
            }
            const bool need = mx > m_run[qb] + kSlack;
            if (__builtin_amdgcn_ballot_w64(need) != 0) {
                const float al = need ? __builtin_amdgcn_exp2f(m_run[qb] - mx) : 1.0f;
                m_run[qb] = need ? mx : m_run[qb];
                l_run[qb] *= al;
#pragma unroll
                for (int db = 0; db < NDB; ++db) acc[qb][db] *= al;
            }
            float p[16];
            const float nm = -m_run[qb];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                // in a full tile every score and m_run are finite
                if constexpr (FULL)
                    p[v] = __builtin_amdgcn_exp2f(fmaf(sc[v], csc, nm));
                else
                    p[v] = sc[v] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(fmaf(sc[v], csc, nm));
            }
            // row sum as a tree (no 16-long chain of dependent adds)
            float s8[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) s8[k] = p[2 * k] + p[2 * k + 1];
            l_run[qb] += ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                ph[qb][q] = Mx<F16>::pack2(p[2 * q], p[2 * q + 1]);
                pl[qb][q] = Mx<F16>::resid2(p[2 * q], p[2 * q + 1], ph[qb][q]);
            }
        }
        // V^T: in each 16-lane group (h, cb) lane j addresses tile row
        // 16 u + 4 h + j / 4 (and 8 rows on for the second read), columns
        // 32 db + 16 cb + 4 (j % 4) ..; lane (h, cb, i) receives column
        // 32 db + 16 cb + i of the group's four rows
        const int j16 = lane & 15, cb = (lane >> 4) & 1;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ra = 16 * u + 4 * hf + (j16 >> 2);
            const int rb2 = ra + 8;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int cl = 32 * db + 16 * cb + 4 * (j16 & 3);   // first bf16 column
                const uint2 v0 = __builtin_bit_cast(
                    uint2, lds_read_tr16(reinterpret_cast<const uint16_t*>(vt + ra * SV + 2 * cl)));
                const uint2 v1 = __builtin_bit_cast(
                    uint2, lds_read_tr16(reinterpret_cast<const uint16_t*>(vt + rb2 * SV + 2 * cl)));
                const uint4 va = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    acc[qb][db] = Mx<F16>::mma32x16(va, make_uint4(ph[qb][4 * u], ph[qb][4 * u + 1], ph[qb][4 * u + 2],
                                                        ph[qb][4 * u + 3]), acc[qb][db]);
                    acc[qb][db] = Mx<F16>::mma32x16(va, make_uint4(pl[qb][4 * u], pl[qb][4 * u + 1], pl[qb][4 * u + 2],
                                                        pl[qb][4 * u + 3]), acc[qb][db]);
                }
            }
        }
    };

    // Iteration i computes tile i from LDS buffer i % NBUF, then stages tile
    // i + 1 (loaded NREG iterations earlier) into buffer (i + 1) % NBUF and
    // issues the loads of tile i + 1 + NREG into the registers it freed.
    // With NQ > 1 one barrier per tile orders each buffer's stores before
    // its reads by the split's other waves, and its reads before the next
    // stores into it (a wave alone needs no barrier and one buffer: its LDS
    // accesses run in order).
    // With NQ > 1 every wave runs the same number of iterations (the most
    // any split has), so that all meet the same barriers; a split past its
    // last tile stages clamped rows it never computes.
    const int nloop = NQ > 1 ? (ntile_all + NS - 1) / NS : ntile;
    if (nloop > 0) {
        uint4 kr[NREG][NCH], vr[NREG][NCH];
#pragma unroll
        for (int u = 0; u < NREG; ++u) load(u, kr[u], vr[u]);
        stage(0, kr[0], vr[0]);
        load(NREG, kr[0], vr[0]);
        // the query rows arrived before the first tile did
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                qop[qb][s] = make_uint4(qop[qb][s].x ^ qsign, qop[qb][s].y ^ qsign, qop[qb][s].z ^ qsign,
                                        qop[qb][s].w ^ qsign);
        if constexpr (NQ > 1) __syncthreads();
        else wave_lds_fence();
        for (int it = 0; it < nloop; it += 2 * NREG) {
#pragma unroll
            for (int u = 0; u < 2 * NREG; ++u) {
                const int i = it + u;
                if (i >= nloop) break;
                if (NQ == 1 || i < ntile) {
                    const int t0 = ta + TR * (sp + NS * i);
                    if (t0 + TR <= tb && t0 + TR - 1 <= pc.L - a.sq)
                        compute(i & 1, t0, std::true_type{});
                    else
                        compute(i & 1, t0, std::false_type{});
                }
                // the loads are issued on every path (rows past the piece
                // clamp to its last row): with the same loads in flight on
                // every path the compiler waits for exactly the oldest tile
                // instead of draining the prefetches
                const int nr = (u + 1) % NREG;
                if (i + 1 < nloop) {
                    if constexpr (NQ == 1) wave_lds_fence();   // this tile's reads stay before the next stores
                    stage((i + 1) & 1, kr[nr], vr[nr]);
                }
                load(i + 1 + NREG, kr[nr], vr[nr]);
                if constexpr (NQ > 1) __syncthreads();
                else wave_lds_fence();
            }
        }
    }

    // ---- end of the piece ------------------------------------------------------
    float l_full[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_full[qb] = sum_x32(l_run[qb]);
    if constexpr (NS > 1) {
        // merge the splits' running sums: every wave is past its tiles, so
        // the tile buffers hold the merge
        __syncthreads();
        if (hf == 0) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                sm.ml[0][sp][(qs * QB + qb) * 32 + col] = m_run[qb];
                sm.ml[1][sp][(qs * QB + qb) * 32 + col] = l_full[qb];
            }
        }
        __syncthreads();
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int ix = (qs * QB + qb) * 32 + col;
            float M = -INFINITY;
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2) M = fmaxf(M, sm.ml[0][s2][ix]);
            float Lt = 0.0f;
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2) {
                const float ms = sm.ml[0][s2][ix];
                Lt += ms == -INFINITY ? 0.0f : sm.ml[1][s2][ix] * __builtin_amdgcn_exp2f(ms - M);
            }
            const float f = m_run[qb] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[qb] - M);
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[qb][db] *= f;
            m_run[qb] = M;
            l_full[qb] = Lt;
        }
        // sum the scaled accumulators over the splits, pairwise: at step st
        // split sp (sp % 2 st == st) hands its sums to split sp - st through
        // slot sp / (2 st) of the tile buffers
        constexpr int SLOT = NQ * QB * NDB * 4 * kWave;   // float4 per split's accumulators
        static_assert(((NS + 1) / 2) * SLOT * sizeof(float4) <= sizeof(sm.t), "split merge fits the tile buffers");
        float4* mg = reinterpret_cast<float4*>(&sm.t[0][0]);
#pragma unroll
        for (int st = 1; st < NS; st *= 2) {
            if (sp % (2 * st) == st) {
                float4* dst = mg + (sp / (2 * st)) * SLOT;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            dst[(((qs * QB + qb) * NDB + db) * 4 + i) * kWave + lane] =
                                make_float4(acc[qb][db][4 * i], acc[qb][db][4 * i + 1], acc[qb][db][4 * i + 2],
                                            acc[qb][db][4 * i + 3]);
            }
            __syncthreads();
            if (sp % (2 * st) == 0 && sp + st < NS) {
                const float4* src = mg + (sp / (2 * st)) * SLOT;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float4 x = src[(((qs * QB + qb) * NDB + db) * 4 + i) * kWave + lane];
                            acc[qb][db][4 * i] += x.x;
                            acc[qb][db][4 * i + 1] += x.y;
                            acc[qb][db][4 * i + 2] += x.z;
                            acc[qb][db][4 * i + 3] += x.w;
                        }
            }
            __syncthreads();
        }
    }

    const int c_first = cm.of(pc.off);
    const int npieces = cm.of(pc.off + pc.L - 1) - c_first + 1;
    // The results of the split-0 waves: a segment held by this chunk goes to
    // out, else the piece's partial (rows divided by their sums, and their
    // log2-sum-exp) to its slot -- device-scope stores when this launch
    // merges it, plain ones for the combine kernel.  Each wave stages its
    // rows in LDS (lane (col, h) holds row col, columns 32 db + 8 i + 4 h ..)
    // and stores two whole rows per instruction.
    if (sp == 0) {
        constexpr int OS = MfxShared<D, QB, NQ, NS>::OS;
        float* ob = sm.out[qs];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float inv = l_full[qb] > 0.0f ? 1.0f / l_full[qb] : 0.0f;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<float4*>(ob + (32 * qb + col) * OS + 32 * db + 8 * i + 4 * hf) =
                        make_float4(acc[qb][db][4 * i] * inv, acc[qb][db][4 * i + 1] * inv,
                                    acc[qb][db][4 * i + 2] * inv, acc[qb][db][4 * i + 3] * inv);
        }
        wave_lds_fence();
        constexpr int LPR = D / 4;                      // lanes per row (one float4 each)
        constexpr int RPI = kWave / LPR;                // rows per store instruction
        const int rsub = lane / LPR, c4 = 4 * (lane % LPR);
        const int live_rows = R - row0 - wrow0;         // rows of this wave below R
        const __amdgpu_buffer_rsrc_t part = part_rsrc(a.part);
        const MSlots ms = mslots<D>(a);
        const int mine = ms.base(chunk, cm.start(chunk) >= pc.off ? 0 : 1);
        const int nrow = min(32 * QB, live_rows);
        if (npieces == 1 || a.deferred) {
            float* dst = npieces == 1 ? a.out + (qrow0 + wrow0) * D : a.part + mine + wrow0 * D;
#pragma unroll 2
            for (int r = rsub; r < nrow; r += RPI)
                *reinterpret_cast<float4*>(dst + r * D + c4) = *reinterpret_cast<const float4*>(ob + r * OS + c4);
        } else {
#pragma unroll 2
            for (int r = rsub; r < nrow; r += RPI) {
                const float4 x = *reinterpret_cast<const float4*>(ob + r * OS + c4);
                const float v4[4] = {x.x, x.y, x.z, x.w};
                store4_coherent(part, mine + (wrow0 + r) * D + c4, v4);
            }
        }
        if (npieces > 1 && hf == 0) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                if (!live[qb]) continue;
                const float lse = l_full[qb] > 0.0f ? m_run[qb] + __log2f(l_full[qb]) : -INFINITY;
                const int rr = wrow0 + 32 * qb + col;
                if (a.deferred)
                    a.part[mine + ms.lse + rr] = lse;
                else
                    store_coherent(part, mine + ms.lse + rr, lse);
            }
        }
        wave_lds_fence();
    }
    // the staging area is the next piece's tile buffers
    if constexpr (NQ > 1) __syncthreads();
    if (npieces == 1) return false;
    pd->seg = (pc.b * a.G + pc.g) * n_rb + pc.rb;
    pd->p_first = c_first;
    pd->npieces = npieces;
    pd->off = pc.off;
    pd->qrow0 = qrow0;
    pd->row0 = row0;
    return true;
}

template <int D, int QB, int NQ, int NS, bool F16 = false>
__global__ void __launch_bounds__(kWave * NQ * NS) __attribute__((amdgpu_waves_per_eu(NQ * NS / 4, NQ * NS / 4)))
decode_mfx(const int32_t* __restrict__ lens_in, const int nB, const int nT, const Args a, const int R, const int n_rb)
{
    constexpr int NW = NQ * NS;
    __shared__ MfxShared<D, QB, NQ, NS> sm;
    const int P = gridDim.x;
    const int p = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    for (int i = tid; i < kLensWindow && i < nB; i += kWave * NW) sm.lens[i] = clamp_len(lens_in, i, nT);
    zero_empty_sequences<D>(a, P, p);
    __syncthreads();
    const int units = a.G * n_rb;
    const int chunk = p;
    ChunkPlan cp;
    if (!plan_chunk<false>(a, sm.lens, units, P, chunk, cp)) return;
    const ChunkMap& cm = cp.cm;
    CostPieceIter<false> it;
    it.init(cp.vA, cp.vE, cp.fb, cp.fv, a.G, n_rb);
    Piece pc;
    while (it.next(a, sm.lens, pc)) {
        Pending pd;
        if (mfx_piece<D, QB, NQ, NS, F16>(a, sm, R, pc, cm, chunk, n_rb, &pd) && !a.deferred) {
            partials_stored_before_arrival();    // this wave's partial stores complete at device scope
            __syncthreads();                     // ... and every other wave's
            if (tid == 0) {
                const int old = __hip_atomic_fetch_add(&a.counters[pd.seg], 1, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
                sm.merge = old == pd.npieces - 1;
                if (sm.merge) __hip_atomic_store(&a.counters[pd.seg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            arrival_before_partial_loads();
            if (sm.merge) {
                const int live_rows = min(32 * QB * NQ, R - pd.row0);
                for (int r0 = 16 * w; r0 < live_rows; r0 += 16 * NW)
                    merge_block16<D>(a, pd, lane, r0, min(16, live_rows - r0), cm);
            }
            __syncthreads();                     // sm.merge is rewritten by the next piece
        }
    }
}

// Combine pass for a deferred plan: one wave per (segment, RW query rows)
// of a split segment merges the rows' partials, in chunk order (the same
// log2-sum-exp merge as the in-kernel one).  D / 4 lanes per row: a lane
// holds elements 4 (l % (D / 4)) .. + 3 of row l / (D / 4) of each of the
// wave's NG groups of RPW rows.  With few pieces per segment (NG = 2 or 4)
// one schedule walk serves RW = RPW * NG rows and the loads of several rows'
// pieces are in flight together; with many (NG = 1) each wave keeps up to 16
// pieces of its RPW rows in flight.
template <int D>
constexpr int combine_rows_per_group() { return kWave / (D / 4); }

// Merge the pieces of row groups G0 .. G0 + NG - 1 (row rl[g] of the slots),
// KB pieces' loads in flight per group at a time.  Pieces past the last are
// clamped to it and weighted 0, so the per-row arithmetic does not depend on
// KB or on the grouping.
template <int D, int KB, int G0, int NG>
__device__ __forceinline__ void combine_groups(__amdgpu_buffer_rsrc_t part, const MSlots& ms, int c_first,
                                               int npieces, bool tail1, const int* rl, int e, float* M, float* den,
                                               float (*num)[4])
{
    for (int k0 = 0; k0 < npieces; k0 += KB) {
        float lse[NG][KB], ov[NG][KB][4];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            const int k = min(k0 + kk, npieces - 1);
            const int base = ms.base(c_first + k, k == 0 && tail1 ? 1 : 0);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                lse[g][kk] = load_coherent(part, base + ms.lse + rl[G0 + g]);
                load4_coherent(part, base + rl[G0 + g] * D + e, ov[g][kk]);
            }
        }
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                float w;
                const float sc = lse_step(M[G0 + g], k0 + kk < npieces ? lse[g][kk] : -INFINITY, &w);
                den[G0 + g] = fmaf(den[G0 + g], sc, w);
#pragma unroll
                for (int q = 0; q < 4; ++q) num[G0 + g][q] = fmaf(num[G0 + g][q], sc, w * ov[g][kk][q]);
            }
    }
}

template <int D, int RB, int NG>
__global__ void __launch_bounds__(kWave)
combine_rows(const Args a, const int R, const int n_rb, const int P)
{
    constexpr int RPW = combine_rows_per_group<D>();
    constexpr int RW = RPW * NG;
    static_assert(RB % RW == 0, "rows of a block split evenly over the waves");
    static_assert(NG == 1 || NG == 2 || NG == 4, "groups per wave");
    const int lane = threadIdx.x & (kWave - 1);
    const int rw0 = (int)(blockIdx.x % (RB / RW)) * RW;   // first row of this wave within the segment
    const long long seg = blockIdx.x / (RB / RW);
    const int rb = (int)(seg % n_rb);
    const int g = (int)((seg / n_rb) % a.G);
    const int b = (int)(seg / ((long long)n_rb * a.G));
    if (rb * RB + rw0 >= R) return;            // every row of this wave is past R
    const int L = clamp_len(a.seq_lens, b, a.T);
    if (L == 0) return;
    // cost units before sequence b, and in total (every wave of the grid agrees)
    long long before = 0, tot = 0;
    for (int b0 = 0; b0 < a.B; b0 += kWave) {
        const int bb = b0 + lane;
        const uint32_t c = bb < a.B ? seg_cost(clamp_len(a.seq_lens, bb, a.T), a.piece_cost) : 0u;
        tot += wave_sum_u32(c);
        before += wave_sum_u32(bb < b ? c : 0u);
    }
    const long long units = (long long)a.G * n_rb;
    const ChunkMap cm = make_map(tot * units, P);
    // the cost-unit position of the segment's first row
    const long long off = before * units + ((long long)g * n_rb + rb) * ((long long)L + a.piece_cost) + a.piece_cost;
    const int c_first = cm.of(off);
    const int npieces = cm.of(off + L - 1) - c_first + 1;
    if (npieces == 1) return;                 // written by its piece
    const bool tail1 = cm.start(c_first) < off;
    const __amdgpu_buffer_rsrc_t part = part_rsrc(a.part);
    const MSlots ms = mslots<D>(a);
    const int e = 4 * (lane % (D / 4));
    int rl[NG];
    float M[NG], den[NG], num[NG][4];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int r = rw0 + gi * RPW + lane / (D / 4);
        rl[gi] = min(r, R - 1 - rb * RB);      // a lane past R reads the last live row (its result is dropped)
        M[gi] = -INFINITY;
        den[gi] = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) num[gi][q] = 0.0f;
    }
    // at most 16 (group, piece) loads in flight; the batch fits the piece count
    if (npieces <= 4) {
        combine_groups<D, 4, 0, NG>(part, ms, c_first, npieces, tail1, rl, e, M, den, num);
    } else if (npieces <= 8) {
        if constexpr (NG == 1) {
            combine_groups<D, 8, 0, 1>(part, ms, c_first, npieces, tail1, rl, e, M, den, num);
        } else {
            combine_groups<D, 8, 0, NG / 2>(part, ms, c_first, npieces, tail1, rl, e, M, den, num);
            combine_groups<D, 8, NG / 2, NG / 2>(part, ms, c_first, npieces, tail1, rl, e, M, den, num);
        }
    } else {
        combine_groups<D, 16, 0, 1>(part, ms, c_first, npieces, tail1, rl, e, M, den, num);
        if constexpr (NG >= 2) combine_groups<D, 16, 1, 1>(part, ms, c_first, npieces, tail1, rl, e, M, den, num);
        if constexpr (NG >= 4) {
            combine_groups<D, 16, 2, 1>(part, ms, c_first, npieces, tail1, rl, e, M, den, num);
            combine_groups<D, 16, 3, 1>(part, ms, c_first, npieces, tail1, rl, e, M, den, num);
        }
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int row = rw0 + gi * RPW + lane / (D / 4);
        if (rb * RB + row < R) {
            const float inv = den[gi] > 0.0f ? 1.0f / den[gi] : 0.0f;
            const int64_t qrow = (int64_t)b * a.H * a.sq + (int64_t)g * R + rb * RB + row;
            *reinterpret_cast<float4*>(a.out + qrow * D + e) =
                make_float4(num[gi][0] * inv, num[gi][1] * inv, num[gi][2] * inv, num[gi][3] * inv);
        }
    }
}

// ---------------------------------------------------------------------------
// Host-side launch
// ---------------------------------------------------------------------------
// Every decode kernel takes (seq_lens, B, T) ahead of the argument block: the
// build preloads the first arguments into scalar registers, so the first
// global load (the lengths) need not wait for the argument block.
typedef void (*DecodeFn)(const int32_t*, int, int, const Args, int, int);

template <class FMT, int D>
static DecodeFn pick_valu(int rb)
{
    switch (rb) {
    case 1: return decode_valu<FMT, D, 1>;
    case 2: return decode_valu<FMT, D, 2>;
    case 4: return decode_valu<FMT, D, 4>;
    case 8: return decode_valu<FMT, D, 8>;
    case 16: return decode_valu<FMT, D, 16>;
    default: return nullptr;
    }
}

template <int D>
static DecodeFn pick_mqk(int rb)
{
    switch (rb) {
    case 4: return decode_mqk<D, 4>;
    case 8: return decode_mqk<D, 8>;
    case 16: return decode_mqk<D, 16>;
    default: return nullptr;
    }
}

template <int SRC, bool KV8, bool F16 = false, bool I8 = false>
static DecodeFn pick_mfa(const Plan& p)
{
    switch (p.row_block) {
    case 16: return p.D == 64 ? decode_mfa<64, 1, SRC, KV8, F16, I8> : decode_mfa<128, 1, SRC, KV8, F16, I8>;
    case 32: return p.D == 64 ? decode_mfa<64, 2, SRC, KV8, F16, I8> : decode_mfa<128, 2, SRC, KV8, F16, I8>;
    case 64: return p.D == 64 ? decode_mfa<64, 4, SRC, KV8, F16, I8> : decode_mfa<128, 4, SRC, KV8, F16, I8>;
    default: return nullptr;
    }
}

template <int D, bool F16>
static DecodeFn pick_mfx(int row_block)
{
    switch (row_block) {
    case 32: return decode_mfx<D, 1, 1, 4, F16>;
    case 64: return decode_mfx<D, 1, 2, 2, F16>;
    case 128: return decode_mfx<D, 1, 4, 2, F16>;
    case 256: return decode_mfx<D, 1, 8, 1, F16>;
    default: return nullptr;
    }
}

template <bool F16>
static DecodeFn pick_mfs(const Plan& p)
{
    if (p.rsplit == 2) return p.D == 64 ? decode_mfs<64, 1, 2, F16> : decode_mfs<128, 1, 2, F16>;
    if (p.rsplit == 4) return p.D == 64 ? decode_mfs<64, 1, 4, F16> : decode_mfs<128, 1, 4, F16>;
    return nullptr;
}

static DecodeFn pick(const Plan& p)
{
    // an fp16 cache: on the 32 x 32, row-split and one-block matrix-core
    // kernels (appended tokens and paged caches on the one-block kernel) or
    // the vector-ALU kernel
    if (p.kv_f16 && p.path == Path::MFMA_QK) return nullptr;
    if (p.path == Path::MFMA && p.mfx) {
        if (!(p.kv_bf16 || p.kv_f16) || p.src != kSrcCache) return nullptr;
        if (p.kv_f16) return p.D == 64 ? pick_mfx<64, true>(p.row_block) : pick_mfx<128, true>(p.row_block);
        return p.D == 64 ? pick_mfx<64, false>(p.row_block) : pick_mfx<128, false>(p.row_block);
    }
    if (p.path == Path::MFMA && p.rsplit > 1) {
        if (!(p.kv_bf16 || p.kv_f16) || p.src != kSrcCache || p.row_block != 16 || p.wg_waves != p.rsplit)
            return nullptr;
        return p.kv_f16 ? pick_mfs<true>(p) : pick_mfs<false>(p);
    }
    if (p.path == Path::MFMA && p.wg_waves > 1) {
        if (!p.kv_bf16 || p.src != kSrcCache) return nullptr;
        if (p.wg_waves == 4) return p.D == 64 ? decode_mfw<64, 4> : decode_mfw<128, 4>;
        if (p.wg_waves == 8) return p.D == 64 ? decode_mfw<64, 8> : decode_mfw<128, 8>;
        return nullptr;
    }
    if (p.path == Path::MFMA) {
        if (p.kv_fp8) {
            if (p.src == kSrcCache)
                return p.kv_i8 ? pick_mfa<kSrcCache, true, false, true>(p) : pick_mfa<kSrcCache, true>(p);
            if (p.src == kSrcPaged)
                return p.kv_i8 ? pick_mfa<kSrcPaged, true, false, true>(p) : pick_mfa<kSrcPaged, true>(p);
            return nullptr;
        }
        if (p.kv_f16) {
            switch (p.src) {
            case kSrcCache: return pick_mfa<kSrcCache, false, true>(p);
            case kSrcAppend: return pick_mfa<kSrcAppend, false, true>(p);
            case kSrcPaged: return pick_mfa<kSrcPaged, false, true>(p);
            default: return nullptr;
            }
        }
        if (!p.kv_bf16) return nullptr;
        switch (p.src) {
        case kSrcCache: return pick_mfa<kSrcCache, false>(p);
        case kSrcAppend: return pick_mfa<kSrcAppend, false>(p);
        case kSrcPaged: return pick_mfa<kSrcPaged, false>(p);
        default: return nullptr;
        }
    }
    if (p.path == Path::MFMA_QK) {
        if (!p.kv_bf16) return nullptr;
        return p.D == 64 ? pick_mqk<64>(p.row_block) : pick_mqk<128>(p.row_block);
    }
    if (p.kv_bf16)
        return p.D == 64 ? pick_valu<Bf16, 64>(p.row_block) : pick_valu<Bf16, 128>(p.row_block);
    if (p.kv_f16)
        return p.D == 64 ? pick_valu<F16, 64>(p.row_block) : pick_valu<F16, 128>(p.row_block);
    return p.D == 64 ? pick_valu<F32, 64>(p.row_block) : pick_valu<F32, 128>(p.row_block);
}

int resident_groups_per_cu(const Plan& p)
{
    DecodeFn fn = pick(p);
    if (!fn) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(fn), kWave * p.wg_waves, 0) !=
        hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return n;
}

typedef void (*CombineFn)(const Args, int, int, int);

template <int NG>
static CombineFn pick_combine_ng(const Plan& p)
{
    switch (p.row_block) {
    case 16: return p.D == 64 ? combine_rows<64, 16, NG> : combine_rows<128, 16, NG>;
    case 32: return p.D == 64 ? combine_rows<64, 32, NG> : combine_rows<128, 32, NG>;
    case 64: return p.D == 64 ? combine_rows<64, 64, NG> : combine_rows<128, 64, NG>;
    case 128: return p.D == 64 ? combine_rows<64, 128, NG> : combine_rows<128, 128, NG>;
    case 256: return p.D == 64 ? combine_rows<64, 256, NG> : combine_rows<128, 256, NG>;
    default: return nullptr;
    }
}

// Row groups per combine wave from the expected pieces per segment (the
// planner's estimate: workgroups per segment, plus the two partial ends):
// up to 4 pieces, four groups share one schedule walk and one load batch;
// up to 8, two; more, one group per wave with 16 pieces in flight
// (measured: multi-token ~4 pieces 78.6 -> 73.8 us per step; MQA ~14 and the
// sq = 2 sweep at G = 1 ~34 pieces lose 3-5 us with four groups).
static int combine_groups_for(const Plan& p, const Args& a)
{
    const int64_t segs = (int64_t)a.B * a.G * p.n_rb;
    const int64_t pieces = segs > 0 ? p.grid / segs + 2 : 1;
    const int rpg = p.D == 64 ? combine_rows_per_group<64>() : combine_rows_per_group<128>();
    int ng = pieces <= 4 ? 4 : pieces <= 8 ? 2 : 1;
    while (ng > 1 && p.row_block % (rpg * ng) != 0) ng /= 2;   // a wave's rows within one segment
    return ng;
}

static CombineFn pick_combine(const Plan& p, int ng)
{
    if (p.path != Path::MFMA) return nullptr;
    switch (ng) {
    case 1: return pick_combine_ng<1>(p);
    case 2: return pick_combine_ng<2>(p);
    case 4: return pick_combine_ng<4>(p);
    default: return nullptr;
    }
}

// ---------------------------------------------------------------------------
// Scratch of the entry point that allocates nothing: the arrival counters and
// partials of one call at a time per device, in a fixed device array (zero
// when the code object loads).  Host code reaches it only through the
// per-device address hipGetSymbolAddress returns, taken once per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr)
{
    static std::mutex mu;
    static std::vector<void*> addr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

__global__ void __launch_bounds__(256) clear_ints(int32_t* c, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) c[i] = 0;
}

hipError_t launch_clear_counters(int32_t* counters, int n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    (void)hipGetLastError();
    const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
    hipLaunchKernelGGL(clear_ints, dim3(blocks), dim3(256), 0, stream, counters, n);
    return hipGetLastError();
}

hipError_t launch_decode(const Plan& p, const Args& a, hipStream_t stream)
{
    if (p.grid <= 0) return hipSuccess;
    DecodeFn fn = pick(p);
    if (!fn) return hipErrorInvalidValue;
    CombineFn comb = nullptr;
    const int ng = combine_groups_for(p, a);
    if (p.deferred) {
        comb = pick_combine(p, ng);
        if (!comb || a.deferred != 1) return hipErrorInvalidValue;
    }
    // an error left by unrelated earlier work would otherwise be reported
    // as this launch's
    (void)hipGetLastError();
    hipLaunchKernelGGL(fn, dim3((unsigned)p.grid), dim3(kWave * p.wg_waves), 0, stream, a.seq_lens, a.B, a.T, a,
                       p.R, p.n_rb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !comb) return e;
    const int rpw = (p.D == 64 ? combine_rows_per_group<64>() : combine_rows_per_group<128>()) * ng;
    const int64_t waves = (int64_t)a.B * a.G * p.n_rb * (p.row_block / rpw);
    hipLaunchKernelGGL(comb, dim3((unsigned)waves), dim3(kWave), 0, stream, a, p.R, p.n_rb, (int)p.grid);
    return hipGetLastError();
}

}  // namespace gqa
