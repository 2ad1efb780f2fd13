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
// Split pass, one workgroup per (b, g, row block, chunk of cache rows):
//   1. K pass: 16-byte coalesced loads of the chunk's K rows; dot products
//      with the R query rows; lane-exchange reduce-scatter (DPP) so that each
//      lane ends with whole scores; scores (in base-2 exponent units) to LDS.
//   2. Softmax over the chunk in LDS: per-row max, p = 2^(s - max), sum.
//   3. V pass: 16-byte coalesced loads of the chunk's V rows; acc += p * v.
//   4. Cross-lane / cross-wave sum; chunk output normalised by its own sum.
//      A sequence with one chunk writes out directly; otherwise the chunk's
//      (output, log2-sum-exp) goes to the workspace.
// Merge pass, one wave per output row: weights 2^(lse_c - max_c lse) in chunk
// order (deterministic), out = sum_c w_c o_c / sum_c w_c.
//
// Split-then-merge is an exact rewrite of one softmax over all rows (the
// log-sum-exp identity; the oracle pins check it in float64).

#include <math.h>
#include <stdint.h>

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
        r = __builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xF, 0xF, false);
    } else if constexpr (M == 2) {
        r = __builtin_amdgcn_update_dpp(0, xi, 0x4E, 0xF, 0xF, false);
    } else if constexpr (M == 7) {
        r = __builtin_amdgcn_update_dpp(0, xi, 0x141, 0xF, 0xF, false);
    } else if constexpr (M == 15) {
        r = __builtin_amdgcn_update_dpp(0, xi, 0x140, 0xF, 0xF, false);
    } else if constexpr (M == 8) {
        r = __builtin_amdgcn_update_dpp(0, xi, 0x128, 0xF, 0xF, false);
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

__device__ __forceinline__ int clamp_len(const int32_t* seq_lens, int b, int T)
{
    int L = seq_lens ? seq_lens[b] : T;
    return L < 0 ? 0 : (L > T ? T : L);
}

// ---------------------------------------------------------------------------
// Split pass, vector-ALU form.
//   FMT : Bf16 or F32 (q, k, v share it)
//   D   : head dim (64 or 128)
//   RB  : query rows per workgroup (1, 2, 4, 8, 16)
// Grid: B * G * n_rb * max_chunks workgroups of kSplitWaves waves.
// Dynamic LDS: max(chunk * RB, kSplitWaves * RB * D) floats + 2 * RB floats.
// ---------------------------------------------------------------------------
template <class FMT, int D, int RB>
__global__ void __launch_bounds__(kSplitWaves * kWave)
split_valu(const Args a, const int R, const int n_rb, const int chunk, const int max_chunks)
{
    constexpr int ES = FMT::kBytes;
    constexpr int EPL = FMT::kPerLoad;        // elements per 16-byte load
    constexpr int LPT = D * ES / 16;          // lanes covering one cache row
    constexpr int TPL = kWave / LPT;          // cache rows per wave-wide load
    constexpr int NL = kSlotsPerLane;         // rows per lane per tile
    constexpr int TW = NL * TPL;              // cache rows per wave tile
    constexpr int NW = kSplitWaves;
    constexpr int NV = NL * RB;               // partial dots per lane per tile
    constexpr int NSC = NV >= LPT ? NV / LPT : 1;   // whole scores per lane
    constexpr int NA = RB * EPL;              // accumulators per lane
    constexpr int NAK = NA / TPL;             // accumulators kept after the lane-group sum
    static_assert(LPT >= 1 && LPT <= 32 && (LPT & (LPT - 1)) == 0, "row lanes");
    static_assert(NA >= TPL, "accumulator scatter needs RB * D >= 64");

    extern __shared__ float smem[];
    float* s_lds = smem;                      // [chunk][RB] scores, then p
    const int lds_main = (chunk * RB > NW * RB * D) ? chunk * RB : NW * RB * D;
    float* row_m = smem + lds_main;           // [RB] chunk max (base-2 units)
    float* row_l = row_m + RB;                // [RB] chunk sum of p
    float* red = smem;                        // [NW][RB][D], reuses s_lds at the end

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    int bid = blockIdx.x;
    const int c = bid % max_chunks;
    bid /= max_chunks;
    const int rb = bid % n_rb;
    bid /= n_rb;
    const int g = bid % a.G;
    const int b = bid / a.G;

    const int L = clamp_len(a.seq_lens, b, a.T);
    const int nc = (L + chunk - 1) / chunk;
    if (c > 0 && c >= nc) return;             // empty chunk (chunk 0 always runs)
    const int t0 = c * chunk;
    const int t1 = min(t0 + chunk, L);        // may be <= t0 when L == 0
    const int row0 = rb * RB;
    const int sq = a.sq;

    // Query rows of this block (contiguous in q); lane holds its 16-byte slice.
    const int dslot = lane % LPT;
    const int doff = dslot * EPL;
    const int64_t qrow0 = (int64_t)b * a.H * sq + (int64_t)g * R + row0;
    uint4 qv[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        if (row0 + i < R)
            qv[i] = load16(static_cast<const char*>(a.q) + ((qrow0 + i) * D + doff) * ES);
        else
            qv[i] = make_uint4(0, 0, 0, 0);
    }

    const int64_t slab = ((int64_t)b * a.G + g) * a.T * D;
    const char* kbase = static_cast<const char*>(a.k) + slab * ES;
    const char* vbase = static_cast<const char*>(a.v) + slab * ES;
    const int lrow = lane / LPT;              // which of the TPL rows of a load

    // ---- 1. K pass --------------------------------------------------------
    for (int tb = t0 + wave * TW; tb < t1; tb += NW * TW) {
        uint4 kv[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int t = tb + j * TPL + lrow;
            kv[j] = (t < t1) ? load16(kbase + ((int64_t)t * D + doff) * ES) : make_uint4(0, 0, 0, 0);
        }
        float part[NV];
#pragma unroll
        for (int j = 0; j < NL; ++j)
#pragma unroll
            for (int i = 0; i < RB; ++i) part[j * RB + i] = FMT::dot(qv[i], kv[j], 0.0f);
        reduce_scatter<NV, LPT / 2, 1, true>(part, lane);
        const bool writer = (NV >= LPT) || (dslot % (LPT / (NV < LPT ? NV : LPT)) == 0);
        if (writer) {
            const int base = (NV >= LPT) ? dslot * NSC : dslot / (LPT / (NV < LPT ? NV : LPT));
#pragma unroll
            for (int m = 0; m < NSC; ++m) {
                const int idx = base + m;
                const int j = idx / RB;
                const int i = idx % RB;
                const int t = tb + j * TPL + lrow;
                const int r = row0 + i;
                const bool vis = (t < t1) && (r < R) && (t <= L - sq + (r % sq));
                s_lds[(t - t0) * RB + i] = vis ? part[m] * a.scale_log2 : -INFINITY;
            }
        }
    }
    __syncthreads();

    // ---- 2. softmax over this chunk, one wave per row ----------------------
    const int nt = t1 > t0 ? t1 - t0 : 0;
    for (int i = wave; i < RB; i += NW) {
        float mx = -INFINITY;
        for (int t = lane; t < nt; t += kWave) mx = fmaxf(mx, s_lds[t * RB + i]);
        mx = wave_max(mx);
        float sum = 0.0f;
        for (int t = lane; t < nt; t += kWave) {
            const float p = (mx == -INFINITY) ? 0.0f : exp2f(s_lds[t * RB + i] - mx);
            s_lds[t * RB + i] = p;
            sum += p;
        }
        sum = wave_sum(sum);
        if (lane == 0) {
            row_m[i] = mx;
            row_l[i] = sum;
        }
    }
    __syncthreads();

    // ---- 3. V pass ------------------------------------------------------------
    float acc[NA];
#pragma unroll
    for (int u = 0; u < NA; ++u) acc[u] = 0.0f;
    for (int tb = t0 + wave * TW; tb < t1; tb += NW * TW) {
        uint4 vv[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int t = tb + j * TPL + lrow;
            vv[j] = (t < t1) ? load16(vbase + ((int64_t)t * D + doff) * ES) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int t = tb + j * TPL + lrow;
            float pr[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) pr[i] = (t < t1) ? s_lds[(t - t0) * RB + i] : 0.0f;
            float vf[EPL];
            FMT::unpack(vv[j], vf);
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[i * EPL + e] = fmaf(pr[i], vf[e], acc[i * EPL + e]);
        }
    }

    // ---- 4. sum over the TPL row groups of the wave, then over waves ---------
    reduce_scatter<NA, kWave / 2, LPT, false>(acc, lane);
    __syncthreads();                          // s_lds is reused as red[] below
    {
        const int ubase = lrow * NAK;
#pragma unroll
        for (int m = 0; m < NAK; ++m) {
            const int u = ubase + m;
            const int i = u / EPL;
            const int e = u % EPL;
            red[(wave * RB + i) * D + doff + e] = acc[m];
        }
    }
    __syncthreads();

    const bool direct = nc <= 1;
    for (int idx = threadIdx.x; idx < RB * D; idx += NW * kWave) {
        const int i = idx / D;
        const int d = idx % D;
        const int r = row0 + i;
        if (r >= R) continue;
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) o += red[(w * RB + i) * D + d];
        const float l = row_l[i];
        const float val = l > 0.0f ? o / l : 0.0f;
        const int64_t orow = qrow0 + i;
        if (direct) {
            a.out[orow * D + d] = val;
        } else {
            a.part_o[(orow * max_chunks + c) * D + d] = val;
            if (d == 0) a.part_lse[orow * max_chunks + c] = l > 0.0f ? row_m[i] + log2f(l) : -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// Merge pass: one wave per output row (b, h, s), 4 rows per workgroup.
// Rows of sequences with at most one chunk were written by the split pass.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
merge_chunks(const Args a, const int chunk, const int max_chunks)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int64_t rows_per_b = (int64_t)a.H * a.sq;
    if (row >= (int64_t)a.B * rows_per_b) return;
    const int b = (int)(row / rows_per_b);
    const int L = clamp_len(a.seq_lens, b, a.T);
    const int nc = (L + chunk - 1) / chunk;
    if (nc <= 1) return;

    const float* lse = a.part_lse + row * max_chunks;
    float M = -INFINITY;
    for (int c = lane; c < nc; c += kWave) M = fmaxf(M, lse[c]);
    M = wave_max(M);
    const float* po = a.part_o + row * max_chunks * D;
    for (int d = lane; d < D; d += kWave) {
        float num = 0.0f, den = 0.0f;
        if (M != -INFINITY) {
            for (int c = 0; c < nc; ++c) {
                const float w = exp2f(lse[c] - M);
                num = fmaf(w, po[(int64_t)c * D + d], num);
                den += w;
            }
        }
        a.out[row * D + d] = den > 0.0f ? num / den : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
int split_tile_rows(Path path, int kv_bf16, int D)
{
    if (path == Path::MFMA) return kSplitWaves * kMfmaTile;
    const int es = kv_bf16 ? 2 : 4;
    const int lpt = D * es / 16;
    return kSplitWaves * kSlotsPerLane * (kWave / lpt);
}

typedef void (*SplitFn)(const Args, int, int, int, int);

template <class FMT, int D>
static SplitFn pick_valu(int rb)
{
    switch (rb) {
    case 1: return split_valu<FMT, D, 1>;
    case 2: return split_valu<FMT, D, 2>;
    case 4: return split_valu<FMT, D, 4>;
    case 8: return split_valu<FMT, D, 8>;
    case 16: return split_valu<FMT, D, 16>;
    default: return nullptr;
    }
}

hipError_t launch_decode(const Plan& p, const Args& a, hipStream_t stream, hipEvent_t split_done)
{
    if (p.split_grid <= 0) return hipSuccess;
    SplitFn fn = nullptr;
    if (p.path == Path::VALU) {
        if (p.kv_bf16)
            fn = p.D == 64 ? pick_valu<Bf16, 64>(p.row_block) : pick_valu<Bf16, 128>(p.row_block);
        else
            fn = p.D == 64 ? pick_valu<F32, 64>(p.row_block) : pick_valu<F32, 128>(p.row_block);
    }
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3((unsigned)p.split_grid), dim3(kSplitWaves * kWave),
                       p.lds_bytes, stream, a, p.R, p.n_rb, p.chunk, p.max_chunks);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (split_done) {
        err = hipEventRecord(split_done, stream);
        if (err != hipSuccess) return err;
    }
    if (p.combine_grid > 0) {
        if (p.D == 64)
            hipLaunchKernelGGL(merge_chunks<64>, dim3((unsigned)p.combine_grid), dim3(256), 0,
                               stream, a, p.chunk, p.max_chunks);
        else
            hipLaunchKernelGGL(merge_chunks<128>, dim3((unsigned)p.combine_grid), dim3(256), 0,
                               stream, a, p.chunk, p.max_chunks);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace gqa
