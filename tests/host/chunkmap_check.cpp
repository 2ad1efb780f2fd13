// Host-side check of the chunk map the matrix-core pass runs on the device
// (csrc/gqa_chunkmap.h, compiled here for the host from the same source):
// every start() and of() is compared with exact 128-bit integer division,
// at the edges of the range the planner admits and at random points.
// Prints "checked N" and exits 0, or prints the first mismatches and exits 1.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "gqa_chunkmap.h"

typedef __int128 i128;

static long long exact_start(long long V, int P, int c) { return (long long)((i128)c * V / P); }
static int exact_of(long long V, int P, long long x) { return (int)(((i128)(x + 1) * P - 1) / V); }

int main()
{
    // The planner admits at most 2^18 (sequence, KV head, row block)
    // segments, T * D < 2^31 with D >= 64 (T < 2^25), and a segment costs
    // its rows plus a piece charge of at most 4096: V <= 2^18 * (2^25 - 1 +
    // 4096).  Grids: 1 .. 2^16.
    const long long vmax = (1LL << 18) * ((1LL << 25) - 1 + 4096);
    std::vector<long long> Vs = {1, 2, 3, 7, 63, 64, 65, 255, 256, 257, 511, 512, 513, 65535, 65536, 65537,
                                 80681LL * 8 + 64 * 256, 1LL << 20, (1LL << 20) + 7, (1LL << 31) - 1, 1LL << 31,
                                 (1LL << 32) + 5, (1LL << 40) - 3, (1LL << 43) - 1, 1LL << 43, vmax - 1, vmax};
    std::vector<int> Ps = {1, 2, 3, 64, 255, 256, 511, 512, 768, 1000, 1024, 4096, 16255, 16256, 65535, 65536};
    std::mt19937_64 rng(20261203);
    for (int i = 0; i < 200; ++i) Vs.push_back(1 + (long long)(rng() % (unsigned long long)vmax));
    for (int i = 0; i < 40; ++i) Ps.push_back(1 + (int)(rng() % 65536));

    long long checks = 0, bad = 0;
    auto report = [&](const char* what, long long V, int P, long long arg, long long got, long long want) {
        if (bad++ < 10)
            std::printf("MISMATCH %s V=%lld P=%d arg=%lld got=%lld want=%lld\n", what, V, P, arg, got, want);
    };
    for (long long V : Vs) {
        for (int P0 : Ps) {
            const gqa::ChunkMap m = gqa::make_map(V, P0);
            const int P = m.P;
            if (P != (V < P0 ? (int)V : P0)) report("P", V, P0, 0, P, V < P0 ? V : P0);
            std::vector<int> cs = {0, 1, 2, P / 2, P - 2, P - 1, P};
            for (int i = 0; i < 24; ++i) cs.push_back((int)(rng() % (unsigned long long)(P + 1)));
            for (int c : cs) {
                if (c < 0 || c > P) continue;
                const long long got = m.start(c), want = exact_start(V, P, c);
                ++checks;
                if (got != want) report("start", V, P, c, got, want);
            }
            std::vector<long long> xs = {0, 1, V - 1, V - 2, V / 2};
            for (int c : cs) {
                if (c < 0 || c > P) continue;
                const long long s = exact_start(V, P, c);
                xs.push_back(s - 1);
                xs.push_back(s);
                xs.push_back(s + 1);
            }
            for (int i = 0; i < 24; ++i) xs.push_back((long long)(rng() % (unsigned long long)V));
            for (long long x : xs) {
                if (x < 0 || x >= V) continue;
                const int got = m.of(x), want = exact_of(V, P, x);
                ++checks;
                if (got != want) report("of", V, P, x, got, want);
                // the chunk found holds x
                if (!(exact_start(V, P, got) <= x && x < exact_start(V, P, got + 1)))
                    report("holds", V, P, x, got, want);
            }
        }
    }
    std::printf("checked %lld, mismatches %lld\n", checks, bad);
    return bad == 0 ? 0 : 1;
}
