// gqa_chunkmap.h -- the integer map from cost units to chunks (workgroups)
// of the matrix-core pass.  Host and device share this code: the device uses
// it in every piece's epilogue, the host-side checker compares it with exact
// integer division over the whole admitted range.
#pragma once

#include <hip/hip_runtime.h>

namespace gqa {

// floor(n / d) for 0 <= n < 2^60 and 0 < d, given r ~ 1 / d in double.
// With the sizes the planner admits (P <= 2^16 chunks, V < 2^44 cost units)
// the quotient stays below 2^44, so the double estimate is within 2^-7 of
// it and off by at most one, which one integer step corrects.  (A 64-bit
// integer division is a long software loop on the GPU, and this runs in
// every piece's epilogue.)
__host__ __device__ __forceinline__ long long div_floor(long long n, long long d, double r)
{
    long long q = (long long)((double)n * r);
    const long long rem = n - q * d;
    q += rem < 0 ? -1 : (rem >= d ? 1 : 0);
    return q;
}

// V cost units cut into P chunks with fixed boundaries: chunk c is
// [floor(c V / P), floor((c + 1) V / P)).
struct ChunkMap {
    long long V;
    int P;
    double rV, rP;   // 1 / V, 1 / P

    __host__ __device__ __forceinline__ long long start(int c) const { return div_floor((long long)c * V, P, rP); }
    // the chunk holding cost unit x, 0 <= x < V
    __host__ __device__ __forceinline__ int of(long long x) const { return (int)div_floor((x + 1) * P - 1, V, rV); }
};

// With fewer cost units than workgroups only the first V take one unit each.
__host__ __device__ __forceinline__ ChunkMap make_map(long long V, int P)
{
    ChunkMap m;
    m.V = V;
    m.P = V < P ? (int)V : P;
    m.rV = 1.0 / (double)V;
    m.rP = 1.0 / (double)m.P;
    return m;
}

}  // namespace gqa
