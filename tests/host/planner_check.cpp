// Drives libgqa's host planner and argument checks (gqa_api.cpp, linked with
// kernel_stub.cpp) over a sweep of shapes and bad arguments.  Built with
// AddressSanitizer and UndefinedBehaviorSanitizer by the test that runs it;
// any report aborts the run.  Exits 0 when every expectation holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "gqa.h"

static int failures = 0;
#define EXPECT(c)                                                              \
    do {                                                                       \
        if (!(c)) {                                                            \
            std::printf("FAILED line %d: %s\n", __LINE__, #c);                 \
            ++failures;                                                        \
        }                                                                      \
    } while (0)

static gqa_shape_t shape(int B, int H, int G, int sq, int T, int D, int qd = GQA_BF16, int kvd = GQA_BF16,
                         int od = GQA_F32)
{
    gqa_shape_t s;
    s.B = B; s.H = H; s.G = G; s.sq = sq; s.T = T; s.D = D;
    s.q_dtype = qd; s.kv_dtype = kvd; s.out_dtype = od;
    return s;
}

int main()
{
    long planned = 0;
    const int Bs[] = {0, 1, 2, 7, 32, 64, 1000, 1 << 15};
    const int HGs[][2] = {{32, 8}, {32, 32}, {32, 1}, {6, 1}, {12, 4}, {64, 8}, {1, 1}};
    const int sqs[] = {1, 2, 3, 5, 64, 65, 200};
    const int Ts[] = {1, 15, 16, 100, 4096, 16384, (1 << 24) - 1};
    const int Ds[] = {64, 128};
    const int wgs[] = {0, 1, 100, 65536, 1 << 20};
    const int paths[] = {GQA_PATH_AUTO, GQA_PATH_VALU, GQA_PATH_MFMA, GQA_PATH_MFMA_QK};
    const int dts[][3] = {{GQA_BF16, GQA_BF16, GQA_F32}, {GQA_F32, GQA_F32, GQA_F32},
                          {GQA_BF16, GQA_FP8_E4M3, GQA_F32}};
    for (int B : Bs)
        for (auto& hg : HGs)
            for (int sq : sqs)
                for (int T : Ts)
                    for (int D : Ds)
                        for (auto& dt : dts)
                            for (int path : paths)
                                for (int wg : wgs) {
                                    gqa_shape_t s = shape(B, hg[0], hg[1], sq, T, D, dt[0], dt[1], dt[2]);
                                    gqa_options_t o;
                                    std::memset(&o, 0, sizeof(o));
                                    o.path = path;
                                    o.workgroups = wg;
                                    o.merge = (wg / 100) % 3;
                                    gqa_plan_t p;
                                    const gqa_status_t st = gqa_plan(&s, &o, &p);
                                    ++planned;
                                    if (st != GQA_OK) {
                                        EXPECT(std::strlen(gqa_last_error()) > 0);
                                        continue;
                                    }
                                    EXPECT(p.workgroups >= (B > 0 ? 1 : 0) && p.workgroups <= 65536);
                                    EXPECT(p.rows_per_group == hg[0] / hg[1] * sq);
                                    EXPECT((int64_t)p.row_blocks * p.row_block >= p.rows_per_group);
                                    // partial slots stay addressable with 32-bit byte offsets
                                    EXPECT(p.workspace_bytes < ((uint64_t)1 << 20) + ((uint64_t)1 << 31));
                                }
    // bad arguments
    gqa_shape_t s = shape(2, 30, 8, 1, 16, 128);
    EXPECT(gqa_decode(&s, (void*)16, (void*)16, (void*)16, nullptr, 0.1f, (void*)16, nullptr) ==
           GQA_ERR_INVALID_ARG);
    s = shape(2, 32, 8, 1, 16, 96);
    EXPECT(gqa_decode(&s, (void*)16, (void*)16, (void*)16, nullptr, 0.1f, (void*)16, nullptr) ==
           GQA_ERR_UNSUPPORTED);
    s = shape(2, 32, 8, 1, 16, 128);
    EXPECT(gqa_decode(nullptr, (void*)16, (void*)16, (void*)16, nullptr, 0.1f, (void*)16, nullptr) ==
           GQA_ERR_INVALID_ARG);
    EXPECT(gqa_decode(&s, nullptr, (void*)16, (void*)16, nullptr, 0.1f, (void*)16, nullptr) ==
           GQA_ERR_INVALID_ARG);
    EXPECT(gqa_decode(&s, (void*)18, (void*)16, (void*)16, nullptr, 0.1f, (void*)16, nullptr) ==
           GQA_ERR_INVALID_ARG);
    EXPECT(gqa_decode_ws(&s, (void*)16, (void*)16, (void*)16, nullptr, 0.1f, (void*)16, (void*)16, 8, nullptr) ==
           GQA_ERR_ALLOC);
    s = shape(0, 32, 8, 1, 16, 128);
    EXPECT(gqa_decode(&s, nullptr, nullptr, nullptr, nullptr, 0.1f, nullptr, nullptr) == GQA_OK);
    // the allocation-failure hook
    s = shape(2, 32, 8, 1, 16, 128);
    setenv("GQA_TEST_FAIL_ALLOC", "1", 1);
    EXPECT(gqa_decode(&s, (void*)16, (void*)16, (void*)16, nullptr, 0.1f, (void*)16, nullptr) == GQA_ERR_ALLOC);
    unsetenv("GQA_TEST_FAIL_ALLOC");
    // the entry point that allocates nothing refuses a workspace beyond its
    // fixed scratch before touching a device
    {
        gqa_shape_t big = shape(64, 32, 8, 64, 4096, 128);
        gqa_options_t o;
        std::memset(&o, 0, sizeof(o));
        o.workgroups = 65536;
        EXPECT(gqa_decode_noalloc(&big, (void*)16, (void*)16, (void*)16, nullptr, 0.1f, (void*)16, &o, nullptr) ==
               GQA_ERR_ALLOC);
        EXPECT(gqa_decode_noalloc(nullptr, (void*)16, (void*)16, (void*)16, nullptr, 0.1f, (void*)16, &o, nullptr) ==
               GQA_ERR_INVALID_ARG);
    }
    // paged shapes
    gqa_paged_shape_t ps;
    std::memset(&ps, 0, sizeof(ps));
    ps.B = 4; ps.H = 32; ps.G = 8; ps.sq = 1; ps.D = 128; ps.page_size = 16; ps.num_pages = 1024;
    ps.max_pages = 256; ps.q_dtype = GQA_BF16; ps.kv_dtype = GQA_BF16; ps.out_dtype = GQA_F32;
    EXPECT(gqa_paged_workspace_bytes(&ps) > 0);
    ps.page_size = 24;
    EXPECT(gqa_paged_workspace_bytes(&ps) == 0);
    ps.page_size = 1 << 16;
    ps.max_pages = 1 << 20;
    EXPECT(gqa_paged_workspace_bytes(&ps) == 0);
    EXPECT(std::strstr(gqa_version(), "gfx950") != nullptr);
    std::printf("planned %ld shapes, %d failures\n", planned, failures);
    return failures == 0 ? 0 : 1;
}
