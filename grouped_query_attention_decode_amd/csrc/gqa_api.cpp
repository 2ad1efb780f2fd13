// gqa_api.cpp -- the C ABI of libgqa (include/gqa.h): argument checks, the
// work planner, the library-owned workspace and the launch.
//
// The checks follow the shape rules of "GQA (Grouped-Query Attention) 분석",
// section "Tensor parallelism과 kernel 제약" (head dims must agree and H must
// be a multiple of G; the cache is [batch, kv_heads, sequence, head_dim]).

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/gqa.h"
#include "gqa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

gqa_status_t fail(gqa_status_t st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

gqa_status_t ok()
{
    g_last_error[0] = '\0';
    return GQA_OK;
}

int pow2_ceil(int x)
{
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

int device_compute_units()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return 256;                          // MI355X
    }
    return n;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Validate the shape and options and build the launch plan.
gqa_status_t make_plan(const gqa_shape_t* s, const gqa_options_t* o, gqa::Plan* p, int src = 0)
{
    if (!s) return fail(GQA_ERR_INVALID_ARG, "shape is NULL");
    if (s->B < 0 || s->H <= 0 || s->G <= 0 || s->sq <= 0 || s->T <= 0 || s->D <= 0)
        return fail(GQA_ERR_INVALID_ARG, "sizes must be positive (B >= 0): B=%d H=%d G=%d sq=%d T=%d D=%d",
                    s->B, s->H, s->G, s->sq, s->T, s->D);
    if (s->H % s->G != 0)
        return fail(GQA_ERR_INVALID_ARG, "H (%d) must be a multiple of G (%d)", s->H, s->G);
    if (s->D != 64 && s->D != 128) return fail(GQA_ERR_UNSUPPORTED, "head dim %d not supported (64, 128)", s->D);
    const bool f32 = s->q_dtype == GQA_F32 && s->kv_dtype == GQA_F32 && s->out_dtype == GQA_F32;
    // an 8-bit cache: fp8 E4M3 or int8 codes (the planner treats both alike)
    const bool i8 = s->q_dtype == GQA_BF16 && s->kv_dtype == GQA_INT8 && s->out_dtype == GQA_F32;
    const bool fp8 = (s->q_dtype == GQA_BF16 && s->kv_dtype == GQA_FP8_E4M3 && s->out_dtype == GQA_F32) || i8;
    const bool bf16 = (s->q_dtype == GQA_BF16 && s->kv_dtype == GQA_BF16 && s->out_dtype == GQA_F32) || fp8;
    const bool f16 = s->q_dtype == GQA_F16 && s->kv_dtype == GQA_F16 && s->out_dtype == GQA_F32;
    if (!f32 && !bf16 && !f16)
        return fail(GQA_ERR_UNSUPPORTED,
                    "dtypes (q=%d, kv=%d, out=%d) not supported; use (F32,F32,F32), (BF16,BF16,F32), "
                    "(F16,F16,F32), (BF16,FP8_E4M3,F32) or (BF16,INT8,F32)", s->q_dtype, s->kv_dtype, s->out_dtype);
    if ((int64_t)s->T * s->D >= (int64_t)1 << 31)
        return fail(GQA_ERR_INVALID_ARG, "T * D must be below 2^31");
    if ((int64_t)s->B * s->H * s->sq * s->D >= (int64_t)1 << 40)
        return fail(GQA_ERR_INVALID_ARG, "B * H * sq * D too large");
    const int64_t R64 = (int64_t)(s->H / s->G) * s->sq;
    if (R64 > (1 << 20)) return fail(GQA_ERR_INVALID_ARG, "(H/G)*sq too large");
    int path_req = GQA_PATH_AUTO, wg_req = 0, merge_req = GQA_MERGE_AUTO;
    if (o) {
        path_req = o->path;
        wg_req = o->workgroups;
        merge_req = o->merge;
        for (int i = 0; i < 5; ++i)
            if (o->reserved[i] != 0) return fail(GQA_ERR_INVALID_ARG, "options.reserved must be zero");
        if (merge_req < GQA_MERGE_AUTO || merge_req > GQA_MERGE_COMBINE)
            return fail(GQA_ERR_INVALID_ARG, "unknown merge mode %d", merge_req);
        if (path_req < GQA_PATH_AUTO || path_req > GQA_PATH_MFMA_QK)
            return fail(GQA_ERR_INVALID_ARG, "unknown path %d", path_req);
        if (wg_req < 0) return fail(GQA_ERR_INVALID_ARG, "workgroups must be >= 0");
    }
    if ((path_req == GQA_PATH_MFMA || path_req == GQA_PATH_MFMA_QK) && !bf16 && !f16)
        return fail(GQA_ERR_UNSUPPORTED, "the matrix-core paths need bf16 or fp16 q/k/v");
    if (path_req == GQA_PATH_MFMA_QK && f16)
        return fail(GQA_ERR_UNSUPPORTED, "GQA_PATH_MFMA_QK reads bf16 only");
    if (fp8 && (path_req == GQA_PATH_VALU || path_req == GQA_PATH_MFMA_QK))
        return fail(GQA_ERR_UNSUPPORTED, "an 8-bit cache runs on GQA_PATH_MFMA only");

    const int R = (int)R64;
    // bf16 and fp16 go to the matrix cores (both products unless asked otherwise);
    // fp32, or a forced VALU path, stays on the vector ALU
    const bool mfma = (bf16 || f16) && path_req != GQA_PATH_VALU;
    if (!mfma)
        p->path = gqa::Path::VALU;
    else if (path_req == GQA_PATH_MFMA_QK)
        p->path = gqa::Path::MFMA_QK;
    else
        p->path = gqa::Path::MFMA;
    p->kv_bf16 = bf16 && !fp8 ? 1 : 0;
    p->kv_fp8 = fp8 ? 1 : 0;
    p->kv_i8 = i8 ? 1 : 0;
    p->kv_f16 = f16 ? 1 : 0;
    p->src = src;
    p->D = s->D;
    p->R = R;
    p->row_block = pow2_ceil(R < gqa::kMaxRowBlock ? R : gqa::kMaxRowBlock);
    if (p->path == gqa::Path::MFMA_QK && p->row_block < 4) p->row_block = 4;   // one k group of the 16x16 tile
    // matrix-core path: 16, 32 or 64 query rows (one to four 16-row MFMA
    // blocks) share each K/V tile a wave reads; a plain bf16 cache with more
    // than 64 rows uses 128-row segments (eight waves of a workgroup)
    if (p->path == gqa::Path::MFMA) p->row_block = R <= 16 ? 16 : R <= 32 ? 32 : (R <= 64 || src != 0 || fp8) ? 64 : 128;
    // More than 16 rows of a plain bf16 cache: the 32 x 32 matrix-core kernel,
    // segments of 32, 64, 128 or 256 rows (workgroups of four or eight
    // waves).  Measured against the 16 x 16 kernels on one machine: MQA
    // (32 rows) 57.7 -> 54.3 us, the sq = 2 sweep at G = 1 (64 rows)
    // 43.9 -> 42.2 us, 64 new tokens (256 rows) 73.0 -> 63.4 us.  At 16 rows
    // or fewer the one-wave 16 x 16 kernel stays faster (batched GQA-8
    // decode 59.3 vs 62.9 us, the sq = 2 sweep at G = 8 157 vs 171, G = 4
    // 87.3 vs 89.6).
    // GQA_MFX=0 selects the 16 x 16 kernels instead (for same-machine
    // comparisons).
    {
        const char* mfx_env = getenv("GQA_MFX");
        // (an fp16 cache has no 16 x 16 multi-wave kernel: it always takes the 32 x 32 one)
        p->mfx = (p->path == gqa::Path::MFMA && !fp8 && src == 0 && R > 16 &&
                  (f16 || !(mfx_env && mfx_env[0] == '0'))) ? 1 : 0;
    }
    if (p->mfx) p->row_block = R <= 32 ? 32 : R <= 64 ? 64 : R <= 128 ? 128 : 256;
    // Up to 16 query rows of a plain bf16 / fp16 cache of at most 128 MB: workgroups
    // of 2 or 4 waves that split each piece's rows (one workgroup per 128 KB
    // of K/V, between half the compute units and all of them).  On such
    // caches a one-wave workgroup's stream is bound by its own load latency
    // and per-tile chain, not by HBM.  Measured per isolated call (one-wave
    // grid -> split): B = 1, D = 64, T = 4096 (Exaone layer, 8 MB) 17.0 ->
    // 14.6 us; B = 2 15.7 vs 18.3; B = 4 16.5 vs 18.7; B = 8 20.7 vs 23.0;
    // B = 16 30.1 vs 32.5; D = 128: B = 1 19.1 vs 20.4, B = 2 20.9 vs 21.9,
    // B = 4 22.7 vs 24.0 (two waves; four: 24.6), B = 8 34.0 vs 33.9, and
    // the batched B = 32 decode (338 MB) 62.7 vs 62.5 -- so larger caches
    // keep one-wave workgroups.  Four waves carry a 64-dim cache or up to
    // 32 MB; two otherwise (four waves' loads in flight, 128 KB per compute
    // unit, slowed larger 128-dim caches).  GQA_RSPLIT=0 / 2 / 4 forces the
    // choice (same-machine comparisons).
    p->rsplit = 0;
    const int64_t kv_bytes = (int64_t)s->B * s->G * s->T * s->D * 2 * 2;
    {
        const bool eligible = p->path == gqa::Path::MFMA && !fp8 && src == 0 && p->row_block == 16;
        const char* rs_env = getenv("GQA_RSPLIT");
        if (eligible && rs_env && rs_env[0] != '\0') {
            const int rs = atoi(rs_env);
            if (rs == 2 || rs == 4) p->rsplit = rs;
        } else if (eligible && kv_bytes <= gqa::kRowSplitMaxBytes) {
            p->rsplit = (s->D == 64 || kv_bytes <= gqa::kRowSplitFourWaveBytes) ? 4 : 2;
        }
    }
    p->n_rb = (R + p->row_block - 1) / p->row_block;
    if ((int64_t)s->B * s->G * p->n_rb > gqa::kMaxSegments)
        return fail(GQA_ERR_INVALID_ARG, "B * G * ceil(R / %d) = %lld exceeds %d (sequence, KV head) segments",
                    p->row_block, (long long)s->B * s->G * p->n_rb, gqa::kMaxSegments);

    // Persistent grid of one-wave workgroups: as many as the GPU holds at
    // once, each taking an equal share of the cache rows; fewer when the
    // cache is so small that a share would drop below two tiles.
    const int64_t max_units = (int64_t)s->B * s->G * p->n_rb * s->T;
    int64_t min_share = 2 * (int64_t)gqa::cache_rows_per_wave_tile(*p);
    // A matrix-core wave with one 16-row query block pays a fixed cost per
    // piece (its start, the partial, the merge) worth about 64 streamed rows,
    // so on small caches fewer, longer waves win: from 8 to 32 MB of bf16
    // K/V, waves of 170-340 rows were fastest (B = 1, D = 128, T = 4096: 512
    // waves and the combine kernel 24.2 us -> 128 waves 21.2 us; B = 2,
    // D = 64: 512 -> 256 waves 21.0 -> 18.9 us; B = 1, D = 64: 256 -> 128
    // waves 14.0 -> 13.4 us by kernel trace); an fp8 cache likewise (B = 1,
    // D = 128: 512 waves 22.8 us, 128 waves 20.2 us; D = 64: 18.0 -> 17.7 us);
    // appended tokens and the paged cache were flat from 128 to 256 waves.
    if (p->path == gqa::Path::MFMA && p->row_block == 16)
        min_share = std::max<int64_t>(min_share, gqa::kMinRowsPerWaveOneBlock);
    if (p->mfx) min_share = gqa::kMfxMinRowsPerGroup;
    // One-wave workgroups: kWavesPerCU per compute unit (fewer if they do not
    // fit) -- enough loads in flight to saturate HBM; more waves only add
    // pieces, and so partials and merges.  A matrix-core wave with one 16-row
    // query block of a bf16 cache keeps two 32-row tiles (32 KB) in flight:
    // two such waves per compute unit stream faster than three (batched
    // GQA-8 decode 64.5 -> 63.5 us, the sq = 2 sweep at G = 32 / 4 4.5% / 2%
    // faster, measured on two machines), while two query blocks per wave (MQA)
    // still want three.
    // Four 16-row blocks per wave make the matrix-core kernel compute-bound:
    // then one wave on each of the four SIMDs of a compute unit.  So does an
    // fp8 cache (half the bytes per tile for the same arithmetic).
    // More than 32 query rows of a plain bf16 cache: workgroups of four (64
    // rows) or eight (128 rows) waves sharing each K/V tile through LDS, two
    // waves per SIMD (up to 32 rows one wave carrying two blocks measured
    // faster).
    p->wg_waves = (p->path == gqa::Path::MFMA && !p->kv_fp8 && src == 0 && p->row_block >= 64)
                      ? p->row_block / 16 : 1;
    int want = (p->path == gqa::Path::MFMA && (p->row_block >= 64 || p->kv_fp8)) ? 4
               : (p->path == gqa::Path::MFMA && p->row_block == 16) ? gqa::kWavesPerCUOneBlock
                                                                      : gqa::kWavesPerCU;
    if (p->wg_waves > 1) want = gqa::kMultiWaveWavesPerCU / p->wg_waves;
    // the 32 x 32 kernel: one workgroup per compute unit
    if (p->mfx) {
        p->wg_waves = gqa::mfx_waves(p->row_block);
        want = 1;
    }
    if (p->rsplit > 1) {
        p->wg_waves = p->rsplit;
        want = 1;
    }
    int occ = gqa::resident_groups_per_cu(*p);
    if (occ <= 0 || occ > want) occ = want;
    int64_t P = (int64_t)device_compute_units() * occ;
    const int64_t by_size = (max_units + min_share - 1) / min_share;
    if (P > by_size) P = by_size;
    if (p->rsplit > 1) {
        // one workgroup per kRowSplitBytesPerGroup of K/V, between half the
        // compute units and all of them, and at least a tile per wave
        const int64_t cus = device_compute_units();
        P = kv_bytes / gqa::kRowSplitBytesPerGroup;
        if (P < cus / 2) P = cus / 2;
        if (P > cus) P = cus;
        const int64_t by_tiles = (max_units + 32 * p->rsplit - 1) / (32 * p->rsplit);
        if (P > by_tiles) P = by_tiles;
    }
    // A split segment merged in-kernel is merged by one wave reading every
    // piece's partial: keep the pieces per segment (at full length) bounded
    // unless the combine kernel (one wave per query row) does the merging.
    const int64_t by_merge = (int64_t)s->B * s->G * p->n_rb * gqa::kMaxPiecesPerSegment;
    const int64_t live = R < p->row_block ? R : p->row_block;
    const bool big_merges = p->path == gqa::Path::MFMA &&
                            (std::min(P, by_merge) / std::max<int64_t>(1, (int64_t)s->B * s->G * p->n_rb) + 2) *
                                    live * s->D * 4 > gqa::kMergeBytesInKernel;
    if (P > by_merge && !(big_merges && merge_req != GQA_MERGE_IN_KERNEL)) P = by_merge;
    if (wg_req > 0) P = wg_req;
    if (P > (1 << 16)) P = 1 << 16;
    // matrix-core path: a slot holds only the live rows, min(row_block, R)
    p->slot_rows = (p->path == gqa::Path::MFMA && R < p->row_block) ? R : p->row_block;
    p->piece_cost = p->mfx ? gqa::kMfxPieceCost : gqa::kPieceCost;
    {
        // development override of the piece charge (tuning runs)
        const char* pc_env = getenv("GQA_PIECE_COST");
        if (pc_env && atoi(pc_env) >= 0 && atoi(pc_env) <= 4096) p->piece_cost = atoi(pc_env);
    }
    // The kernels address the partial slots with 32-bit byte offsets through
    // a buffer resource of 2^31 - 1 bytes: cap the grid so that all of its
    // slots fit (a larger grid would drop stores silently).  Any grid gives
    // the same result to rounding.
    {
        const int64_t slot_bytes = 2 * (int64_t)gqa::slot_floats(p->slot_rows, s->D) * (int64_t)sizeof(float);
        const int64_t max_p = (gqa::kMaxPartBytes - 256) / slot_bytes;
        if (P > max_p) P = max_p;
    }
    if (P < 1) P = 1;
    p->grid = s->B > 0 ? P : 0;
    // Merges by the last arriving wave read every piece's partial alone; when
    // a segment's partials are large (many pieces of many live rows) a
    // second kernel merges them, one wave per query row, instead.
    {
        const int64_t segs = (int64_t)s->B * s->G * p->n_rb;
        const int64_t pieces = segs > 0 ? P / segs + 2 : 1;
        p->deferred = (p->path == gqa::Path::MFMA && pieces * live * s->D * 4 > gqa::kMergeBytesInKernel) ? 1 : 0;
    }
    if (merge_req == GQA_MERGE_IN_KERNEL) p->deferred = 0;
    if (merge_req == GQA_MERGE_COMBINE) {
        if (p->path != gqa::Path::MFMA)
            return fail(GQA_ERR_UNSUPPORTED, "the combine kernel serves the MFMA path only");
        p->deferred = 1;
    }
    p->part_bytes = round_up((size_t)P * 2 * gqa::slot_floats(p->slot_rows, s->D) * sizeof(float), 256);
    p->ws_bytes = gqa::kCounterRegion + p->part_bytes;
    return GQA_OK;
}

struct DeviceWorkspace {
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::vector<DeviceWorkspace> g_ws;

gqa_status_t library_workspace(size_t need, void** out)
{
    *out = nullptr;
    if (need == 0) return GQA_OK;
    // test hook: report the allocation failure the next growth would meet
    // (checked before any device call, so the path runs without a GPU too)
    const char* inject = getenv("GQA_TEST_FAIL_ALLOC");
    const bool fail_alloc = inject && inject[0] == '1';
    int dev = 0;
    if (fail_alloc) return fail(GQA_ERR_ALLOC, "workspace allocation failed (injected by GQA_TEST_FAIL_ALLOC)");
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
    DeviceWorkspace& w = g_ws[dev];
    if (w.bytes < need) {
        if (w.ptr) {
            // earlier calls on any stream may still use the old buffer
            e = hipDeviceSynchronize();
            if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipDeviceSynchronize: %s", hipGetErrorString(e));
            (void)hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
        }
        size_t grow = need + need / 4;
        e = hipMalloc(&w.ptr, grow);
        if (e != hipSuccess) {
            w.ptr = nullptr;
            (void)hipGetLastError();
            return fail(GQA_ERR_ALLOC, "hipMalloc(%zu) for the workspace: %s", grow, hipGetErrorString(e));
        }
        // the arrival counters must start at zero; every call leaves them zero
        e = hipMemset(w.ptr, 0, grow);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) return fail(GQA_ERR_HIP, "zeroing the workspace: %s", hipGetErrorString(e));
        w.bytes = grow;
    }
    *out = w.ptr;
    return GQA_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Where the K/V rows come from, beyond the plain [B, G, T, D] caches.
struct Source {
    int src = 0;                       // gqa kernel source kind (0 cache, 1 append, 2 paged)
    const float* k_scale = nullptr;    // fp8 cache: per-KV-head scales [G]
    const float* v_scale = nullptr;
    const void* k_new = nullptr;       // append: [B, G, sq, D]
    const void* v_new = nullptr;
    const int32_t* block_table = nullptr;  // paged: [B, max_pages]
    int page_shift = 0, num_pages = 0, max_pages = 0;
};

gqa_status_t run(const gqa_shape_t* shape, const void* q, const void* k, const void* v,
                 const int32_t* seq_lens, float scale, void* out, void* workspace, size_t ws_bytes,
                 bool library_ws, const gqa_options_t* opts, void* stream, const Source& srcx = Source(),
                 bool fixed_scratch = false)
{
    gqa::Plan plan;
    gqa_status_t st = make_plan(shape, opts, &plan, srcx.src);
    if (st != GQA_OK) return st;
    if (srcx.src != 0 && plan.path != gqa::Path::MFMA)
        return fail(GQA_ERR_UNSUPPORTED, "appended tokens and paged caches need the matrix-core path");
    if (srcx.src == 1 && plan.kv_fp8)
        return fail(GQA_ERR_UNSUPPORTED, "appended tokens need a bf16 / fp16 cache");
    if ((srcx.k_scale || srcx.v_scale) && !plan.kv_fp8)
        return fail(GQA_ERR_INVALID_ARG, "k_scale / v_scale apply to an 8-bit cache only");
    plan.src = srcx.src;
    if (!std::isfinite(scale)) return fail(GQA_ERR_INVALID_ARG, "scale must be finite");
    if (shape->B == 0) return ok();
    if (!q || !k || !v || !out) return fail(GQA_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be non-NULL");
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out))
        return fail(GQA_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
    if (srcx.src == 1 && (!srcx.k_new || !srcx.v_new || misaligned(srcx.k_new) || misaligned(srcx.v_new)))
        return fail(GQA_ERR_INVALID_ARG, "k_new and v_new must be non-NULL and 16-byte aligned");
    if (srcx.src == 2 && !srcx.block_table) return fail(GQA_ERR_INVALID_ARG, "block_table must be non-NULL");
    if (fixed_scratch) {
        // the fixed device array: no allocation of any kind
        if (plan.ws_bytes > gqa::kNoAllocScratchBytes)
            return fail(GQA_ERR_ALLOC,
                        "this shape needs a %zu-byte workspace, above the fixed %zu-byte scratch of "
                        "gqa_decode_noalloc; lower options->workgroups (gqa_plan reports the size)",
                        plan.ws_bytes, gqa::kNoAllocScratchBytes);
        hipError_t e = gqa::noalloc_scratch(&workspace);
        if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        ws_bytes = gqa::kNoAllocScratchBytes;
    } else if (library_ws) {
        st = library_workspace(plan.ws_bytes, &workspace);
        if (st != GQA_OK) return st;
    } else if (plan.ws_bytes > 0) {
        if (!workspace || ws_bytes < plan.ws_bytes)
            return fail(GQA_ERR_ALLOC, "workspace of %zu bytes needed, %zu given", plan.ws_bytes,
                        workspace ? ws_bytes : (size_t)0);
        if (misaligned(workspace)) return fail(GQA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    }

    gqa::Args a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.seq_lens = seq_lens;
    a.out = static_cast<float*>(out);
    a.counters = static_cast<int32_t*>(workspace);
    a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + gqa::kCounterRegion);
    a.B = shape->B;
    a.H = shape->H;
    a.G = shape->G;
    a.sq = shape->sq;
    a.T = shape->T;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.deferred = plan.deferred;
    a.slot_rows = plan.slot_rows;
    a.piece_cost = plan.piece_cost;
    a.k_new = srcx.k_new;
    a.v_new = srcx.v_new;
    a.block_table = srcx.block_table;
    a.page_shift = srcx.page_shift;
    a.num_pages = srcx.num_pages;
    a.max_pages = srcx.max_pages;
    a.k_scale = srcx.k_scale;
    a.v_scale = srcx.v_scale;

    if (fixed_scratch) {
        // the shared array keeps the last call's contents: clear the arrival
        // counters this call uses (the partials need no clearing)
        const int64_t nseg = (int64_t)shape->B * shape->G * plan.n_rb;
        hipError_t e = gqa::launch_clear_counters(a.counters, (int)nseg, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(GQA_ERR_HIP, "clearing the counters: %s", hipGetErrorString(e));
    }
    hipError_t e = gqa::launch_decode(plan, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GQA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

gqa_status_t gqa_decode(const gqa_shape_t* shape, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* seq_lens, float scale, void* out,
                        void* stream)
{
    return run(shape, q, k_cache, v_cache, seq_lens, scale, out, nullptr, 0, true, nullptr, stream);
}

size_t gqa_workspace_bytes(const gqa_shape_t* shape)
{
    gqa::Plan plan;
    if (make_plan(shape, nullptr, &plan) != GQA_OK) return 0;
    return plan.ws_bytes;
}

size_t gqa_append_workspace_bytes(const gqa_shape_t* shape)
{
    gqa::Plan plan;
    if (make_plan(shape, nullptr, &plan, 1) != GQA_OK) return 0;
    return plan.ws_bytes;
}

gqa_status_t gqa_decode_ws(const gqa_shape_t* shape, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* seq_lens, float scale, void* out,
                           void* workspace, size_t ws_bytes, void* stream)
{
    return run(shape, q, k_cache, v_cache, seq_lens, scale, out, workspace, ws_bytes, false, nullptr,
               stream);
}

gqa_status_t gqa_workspace_clear(void* workspace, size_t ws_bytes, void* stream)
{
    if (!workspace) return fail(GQA_ERR_INVALID_ARG, "workspace is NULL");
    if (ws_bytes < gqa::kCounterRegion)
        return fail(GQA_ERR_INVALID_ARG, "ws_bytes (%zu) is below the %zu-byte counter region of every workspace",
                    ws_bytes, (size_t)gqa::kCounterRegion);
    const hipError_t e = gqa::launch_clear_counters(static_cast<int32_t*>(workspace),
                                                    (int)(gqa::kCounterRegion / sizeof(int32_t)),
                                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GQA_ERR_HIP, "clearing the workspace counters: %s", hipGetErrorString(e));
    return ok();
}

gqa_status_t gqa_decode_ex(const gqa_shape_t* shape, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* seq_lens, float scale, void* out,
                           void* workspace, size_t ws_bytes, const gqa_options_t* opts, void* stream)
{
    const bool lib_ws = workspace == nullptr && ws_bytes == 0;
    return run(shape, q, k_cache, v_cache, seq_lens, scale, out, workspace, ws_bytes, lib_ws, opts,
               stream);
}

gqa_status_t gqa_decode_noalloc(const gqa_shape_t* shape, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* seq_lens, float scale, void* out,
                                const gqa_options_t* opts, void* stream)
{
    return run(shape, q, k_cache, v_cache, seq_lens, scale, out, nullptr, 0, false, opts, stream, Source(), true);
}

gqa_status_t gqa_decode_append(const gqa_shape_t* shape, const void* q, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, const int32_t* seq_lens, float scale, void* out,
                               void* workspace, size_t ws_bytes, const gqa_options_t* opts, void* stream)
{
    Source sx;
    sx.src = 1;
    sx.k_new = k_new;
    sx.v_new = v_new;
    const bool lib_ws = workspace == nullptr && ws_bytes == 0;
    return run(shape, q, k_cache, v_cache, seq_lens, scale, out, workspace, ws_bytes, lib_ws, opts, stream, sx);
}

static gqa_status_t decode_codes(const gqa_shape_t* shape, const void* q, const void* k_cache, const void* v_cache,
                                 const float* k_scale, const float* v_scale, const int32_t* seq_lens, float scale,
                                 void* out, void* workspace, size_t ws_bytes, const gqa_options_t* opts, void* stream)
{
    Source sx;
    sx.k_scale = k_scale;
    sx.v_scale = v_scale;
    const bool lib_ws = workspace == nullptr && ws_bytes == 0;
    return run(shape, q, k_cache, v_cache, seq_lens, scale, out, workspace, ws_bytes, lib_ws, opts, stream, sx);
}

gqa_status_t gqa_decode_fp8(const gqa_shape_t* shape, const void* q, const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale, const int32_t* seq_lens, float scale,
                            void* out, void* workspace, size_t ws_bytes, const gqa_options_t* opts, void* stream)
{
    if (shape && shape->kv_dtype != GQA_FP8_E4M3)
        return fail(GQA_ERR_INVALID_ARG, "gqa_decode_fp8 needs kv_dtype GQA_FP8_E4M3");
    return decode_codes(shape, q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale, out, workspace, ws_bytes, opts,
                        stream);
}

gqa_status_t gqa_decode_int8(const gqa_shape_t* shape, const void* q, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, const int32_t* seq_lens, float scale,
                             void* out, void* workspace, size_t ws_bytes, const gqa_options_t* opts, void* stream)
{
    if (shape && shape->kv_dtype != GQA_INT8)
        return fail(GQA_ERR_INVALID_ARG, "gqa_decode_int8 needs kv_dtype GQA_INT8");
    return decode_codes(shape, q, k_cache, v_cache, k_scale, v_scale, seq_lens, scale, out, workspace, ws_bytes, opts,
                        stream);
}

// The contiguous shape a paged one plans as: T = page_size * max_pages.
static gqa_status_t paged_as_shape(const gqa_paged_shape_t* ps, gqa_shape_t* s, int* shift)
{
    if (!ps) return fail(GQA_ERR_INVALID_ARG, "shape is NULL");
    if (ps->page_size < 16 || ps->page_size > (1 << 16) || (ps->page_size & (ps->page_size - 1)))
        return fail(GQA_ERR_INVALID_ARG, "page_size (%d) must be a power of two in [16, 65536]", ps->page_size);
    if (ps->num_pages <= 0 || ps->max_pages <= 0)
        return fail(GQA_ERR_INVALID_ARG, "num_pages (%d) and max_pages (%d) must be positive", ps->num_pages,
                    ps->max_pages);
    const int64_t T = (int64_t)ps->page_size * ps->max_pages;
    if (T >= ((int64_t)1 << 30)) return fail(GQA_ERR_INVALID_ARG, "page_size * max_pages too large");
    if ((int64_t)ps->num_pages * ps->G * ps->page_size * (ps->D > 0 ? ps->D : 1) >= ((int64_t)1 << 40))
        return fail(GQA_ERR_INVALID_ARG, "page pool too large");
    s->B = ps->B;
    s->H = ps->H;
    s->G = ps->G;
    s->sq = ps->sq;
    s->T = (int32_t)T;
    s->D = ps->D;
    s->q_dtype = ps->q_dtype;
    s->kv_dtype = ps->kv_dtype;
    s->out_dtype = ps->out_dtype;
    int sh = 0;
    while ((1 << sh) < ps->page_size) ++sh;
    *shift = sh;
    return GQA_OK;
}

size_t gqa_paged_workspace_bytes(const gqa_paged_shape_t* shape)
{
    gqa_shape_t s;
    int sh = 0;
    if (paged_as_shape(shape, &s, &sh) != GQA_OK) return 0;
    gqa::Plan plan;
    if (make_plan(&s, nullptr, &plan, 2) != GQA_OK) return 0;
    return plan.ws_bytes;
}

gqa_status_t gqa_decode_paged(const gqa_paged_shape_t* shape, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                              float scale, void* out, void* workspace, size_t ws_bytes,
                              const gqa_options_t* opts, void* stream)
{
    gqa_shape_t s;
    Source sx;
    gqa_status_t st = paged_as_shape(shape, &s, &sx.page_shift);
    if (st != GQA_OK) return st;
    sx.src = 2;
    sx.block_table = block_table;
    sx.num_pages = shape->num_pages;
    sx.max_pages = shape->max_pages;
    const bool lib_ws = workspace == nullptr && ws_bytes == 0;
    return run(&s, q, k_pages, v_pages, seq_lens, scale, out, workspace, ws_bytes, lib_ws, opts, stream, sx);
}

gqa_status_t gqa_plan(const gqa_shape_t* shape, const gqa_options_t* opts, gqa_plan_t* plan)
{
    if (!plan) return fail(GQA_ERR_INVALID_ARG, "plan is NULL");
    gqa::Plan p;
    gqa_status_t st = make_plan(shape, opts, &p);
    if (st != GQA_OK) return st;
    std::memset(plan, 0, sizeof(*plan));
    plan->path = p.path == gqa::Path::MFMA ? GQA_PATH_MFMA
                 : p.path == gqa::Path::MFMA_QK ? GQA_PATH_MFMA_QK : GQA_PATH_VALU;
    plan->workgroups = (int32_t)p.grid;
    plan->rows_per_group = p.R;
    plan->row_blocks = p.n_rb;
    plan->row_block = p.row_block;
    plan->combine = p.deferred;
    plan->waves_per_group = p.wg_waves;
    plan->workspace_bytes = p.ws_bytes;
    return ok();
}

const char* gqa_last_error(void) { return g_last_error; }

const char* gqa_version(void) { return "libgqa 0.1.0 (gfx950)"; }

}  // extern "C"
