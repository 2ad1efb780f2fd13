/*
 * gqa.h -- C ABI of libgqa: grouped-query attention at decode time on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation ("GQA (Grouped-Query Attention) 분석", sections "Grouped
 * broadcast" and "동작 원리 / 3. Incremental decode"; "Same GQA, Different
 * Execution Cost Across Backends", section 1):
 *
 *   for every batch row b, query head h, new-token index s:
 *     g       = h / (H / G)                 (KV head shared by H/G query heads)
 *     L       = clamp(seq_lens[b], 0, T)    (valid cache rows; T if seq_lens is NULL)
 *     last    = L - sq + s                  (query s sees cache rows 0..last)
 *     p       = softmax_j( scale * <q[b,h,s,:], k_cache[b,g,j,:]> ),  j = 0..last
 *     out[b,h,s,:] = sum_j p_j * v_cache[b,g,j,:]      (zeros when last < 0)
 *
 * The sq new tokens are taken to be already appended to the cache, as the
 * last sq of its L valid rows (the incremental-decode loop on the same
 * page appends the new K/V before attending).  Each K/V head is read from
 * device memory once for all H/G query heads that share it; no repeated
 * copy of K/V is ever made (the cost that "Same GQA, Different Execution
 * Cost Across Backends", section 2, measures for the repeat_kv path).
 *
 * Conventions for every entry point below:
 *   - Tensor pointers are DEVICE pointers (memory from hipMalloc or any
 *     allocator of the same device), row-major and contiguous:
 *       q        [B, H, sq, D]   dtype q_dtype
 *       k_cache  [B, G, T, D]    dtype kv_dtype
 *       v_cache  [B, G, T, D]    dtype kv_dtype
 *       seq_lens [B]             int32, or NULL (every sequence holds T rows)
 *       out      [B, H, sq, D]   dtype out_dtype
 *     All must be 16-byte aligned.  out must not overlap the inputs.
 *   - The caller owns every tensor; the library neither frees nor keeps
 *     them after the call returns.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls are asynchronous: the work is queued on stream and the call
 *     returns without waiting; the host never reads seq_lens.
 *   - Status codes, never an abort.  On a non-OK status nothing was queued
 *     (GQA_ERR_HIP: a launch failed, and out may be partly written) and
 *     gqa_last_error() describes the reason.
 *   - seq_lens values outside [0, T] are clamped on the device.
 *
 * Supported in this version: D in {64, 128}; dtypes (q, kv, out) =
 * (F32, F32, F32), (BF16, BF16, F32), (F16, F16, F32),
 * (BF16, FP8_E4M3, F32) or (BF16, INT8, F32) (the 8-bit caches through
 * gqa_decode_fp8 / gqa_decode_int8, or gqa_decode with unit scales;
 * appended tokens bf16 or fp16; paged caches also 8-bit, with unit scales);
 * H % G == 0;
 * any B >= 0, sq >= 1, T >= 1 with T * D < 2^31, B * H * sq * D < 2^40,
 * (H/G) * sq <= 2^20 and B * G * (row blocks per KV head) <= 2^18, where a
 * row block is 16 query rows on the vector-ALU path and 16, 32, 64 or 128
 * on the matrix-core path (gqa_plan_t.row_block).
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARG = 1, /* null pointer, bad sizes, H % G != 0, bad scale   */
    GQA_ERR_UNSUPPORTED = 2, /* head dim or dtype combination not built          */
    GQA_ERR_ALLOC = 3,       /* workspace allocation failed or is too small      */
    GQA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed        */
} gqa_status_t;

/* GQA_FP8_E4M3: OCP FP8 E4M3 ("E4M3FN") codes -- sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, subnormals, no infinities; codes S.1111.111 are
 * NaN and must not appear in the rows read.  A cache only.
 * GQA_F16: IEEE binary16, for q, k and v together (the 4 MB K cache of
 * [1, 8, 4096, 64] in the repeat_kv example of "Same GQA, Different
 * Execution Cost Across Backends", section 2, holds 2-byte values of a type
 * the page does not name); both products on the matrix cores in fp16 with
 * fp32 accumulation, the softmax weights as an fp16 pair hi + lo.
 * GQA_INT8: two's-complement 8-bit integer codes, a cache only. */
typedef enum { GQA_F32 = 0, GQA_BF16 = 1, GQA_FP8_E4M3 = 2, GQA_F16 = 3, GQA_INT8 = 4 } gqa_dtype_t;

/* Problem shape.  H: query heads, G: KV heads ("num_key_value_heads"),
 * sq: new query tokens per sequence, T: cache capacity in rows, D: head dim. */
typedef struct {
    int32_t B, H, G, sq, T, D;
    int32_t q_dtype, kv_dtype, out_dtype; /* gqa_dtype_t values */
} gqa_shape_t;

/* Kernel choice for the split pass. */
typedef enum {
    GQA_PATH_AUTO = 0,    /* bf16 inputs: a matrix-core path; fp32: VALU              */
    GQA_PATH_VALU = 1,    /* vector ALU dot products, any supported shape             */
    GQA_PATH_MFMA = 2,    /* bf16 matrix cores for both products (scores, V sum);
                             bf16 inputs only                                         */
    GQA_PATH_MFMA_QK = 3  /* bf16 matrix cores for the scores, vector ALU for the
                             V sum; bf16 inputs only                                  */
} gqa_path_t;

/* Merge of the pieces of a (sequence, KV head) segment split over several
 * workgroups (GQA_PATH_MFMA only; the other paths always merge in-kernel). */
typedef enum {
    GQA_MERGE_AUTO = 0,      /* in-kernel while a segment's partials are small       */
    GQA_MERGE_IN_KERNEL = 1, /* the last arriving wave merges all pieces              */
    GQA_MERGE_COMBINE = 2    /* a second kernel merges, one wave per query row        */
} gqa_merge_t;

/* Optional knobs; zero-initialise for defaults. */
typedef struct {
    int32_t path;        /* gqa_path_t                                                 */
    int32_t workgroups;  /* workgroups of the (single, persistent) kernel; 0 = as many
                            as the GPU holds at once.  Each takes an equal share of the
                            cache rows, so any value gives the same result to rounding.
                            Capped at 65536, and where the partial results of that many
                            workgroups would pass 2 GiB (gqa_plan reports the grid). */
    int32_t merge;       /* gqa_merge_t: who merges a segment split over workgroups  */
    int32_t reserved[5]; /* must be zero                                               */
} gqa_options_t;

/* What the planner decided for a shape (filled by gqa_plan). */
typedef struct {
    int32_t path;           /* GQA_PATH_VALU, GQA_PATH_MFMA or GQA_PATH_MFMA_QK        */
    int32_t workgroups;     /* workgroups of the kernel                                */
    int32_t rows_per_group; /* (H/G)*sq: query rows sharing one KV head                */
    int32_t row_blocks;     /* segments per (b, KV head) along those rows              */
    int32_t row_block;      /* query rows per segment                                  */
    int32_t combine;        /* 1: split segments are merged by a second kernel (one
                               wave per query row); 0: by the last arriving wave      */
    int32_t waves_per_group;/* waves (64 lanes) per workgroup of the kernel            */
    int32_t reserved[1];
    uint64_t workspace_bytes; /* device scratch the call needs                        */
} gqa_plan_t;

/*
 * gqa_decode -- out = grouped-query attention (see top of file).
 * One kernel launch (two when the plan merges split segments in a combine
 * kernel, gqa_plan_t.combine).  Uses a workspace owned by the library: one buffer per
 * device, grown on demand (hipMalloc and a zero fill, after waiting for the
 * device) and kept until process exit.  Calls that run concurrently on
 * different streams of one device must use gqa_decode_ws with their own
 * workspaces instead.
 * scale: any finite float (the pages use 1/sqrt(D)).
 */
gqa_status_t gqa_decode(const gqa_shape_t *shape, const void *q,
                        const void *k_cache, const void *v_cache,
                        const int32_t *seq_lens, float scale, void *out,
                        void *stream);

/* Device scratch bytes gqa_decode_ws needs for this shape (0 on bad shape). */
size_t gqa_workspace_bytes(const gqa_shape_t *shape);

/* Device scratch bytes gqa_decode_append needs for this shape (0 on bad
 * shape); it can differ from gqa_workspace_bytes, because appended tokens are
 * planned with other row blocks and workgroups above 32 query rows per KV
 * head.  Default options; a caller that sets workgroups in gqa_options_t
 * needs the workspace of that grid (gqa_plan reports the plain decode's). */
size_t gqa_append_workspace_bytes(const gqa_shape_t *shape);

/*
 * gqa_decode_ws -- as gqa_decode, with a caller-owned device workspace of
 * ws_bytes >= gqa_workspace_bytes(shape) bytes.  The workspace starts with
 * a fixed 1 MiB region of arrival counters (one per sequence, KV head and
 * row block) followed by per-workgroup partial results.  It must be
 * zero-filled once before its first use (for example with hipMemset); every
 * call leaves the counter region zero again, so the buffer can be reused for
 * any shape without clearing.  It must not be touched, and must not be
 * shared with another call, until the queued work finishes.
 */
gqa_status_t gqa_decode_ws(const gqa_shape_t *shape, const void *q,
                           const void *k_cache, const void *v_cache,
                           const int32_t *seq_lens, float scale, void *out,
                           void *workspace, size_t ws_bytes, void *stream);

/*
 * gqa_workspace_clear -- zero the arrival-counter region (the first 1 MiB)
 * of a caller-owned workspace, asynchronously on stream, with a fill kernel
 * (no allocation, no memset node: a graph may capture it).  Use it in place
 * of the one-time zero fill before a workspace's first use, or to make a
 * workspace usable again after queued work on it did not run to completion
 * (a failed or abandoned launch can leave counters non-zero, and a later
 * merge would then be wrong).  The partial-result region needs no clearing.
 * workspace: device pointer; ws_bytes: its size, at least the 1 MiB counter
 * region (gqa_workspace_bytes is always larger).  Errors: INVALID_ARG for a
 * NULL workspace or ws_bytes below the counter region; HIP if the launch
 * fails.  Ordering and sharing rules are those of gqa_decode_ws.
 */
gqa_status_t gqa_workspace_clear(void *workspace, size_t ws_bytes, void *stream);

/*
 * gqa_decode_ex -- as gqa_decode_ws with tuning options (may be NULL).
 * Results for a given input are deterministic for a given plan; different
 * workgroup counts agree to rounding.  workspace NULL with ws_bytes 0
 * selects the library-owned workspace of gqa_decode.
 */
gqa_status_t gqa_decode_ex(const gqa_shape_t *shape, const void *q,
                           const void *k_cache, const void *v_cache,
                           const int32_t *seq_lens, float scale, void *out,
                           void *workspace, size_t ws_bytes,
                           const gqa_options_t *opts, void *stream);

/*
 * gqa_decode_noalloc -- gqa_decode_ex for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): it calls no hipMalloc, hipFree or
 * other allocating routine.  (The first call on a device looks up the
 * array's address; make that call before any capture begins.)  Its
 * workspace is a fixed 64 MiB device array
 * inside libgqa, one per device, held until the process ends; a shape (and
 * options->workgroups) whose workspace exceeds it (gqa_plan_t.
 * workspace_bytes) is refused with GQA_ERR_ALLOC and a message -- fewer
 * workgroups need less.  Each call first clears the arrival counters it
 * uses with a small kernel on stream, then queues the decode as
 * gqa_decode_ex does (same plan, same kernels, same bits).  Every call on a
 * device shares that array: calls that may overlap on one device (other
 * streams, or queued work not yet finished while another host thread
 * calls) race and must be serialised by the caller.  opts may be NULL.
 */
gqa_status_t gqa_decode_noalloc(const gqa_shape_t *shape, const void *q,
                                const void *k_cache, const void *v_cache,
                                const int32_t *seq_lens, float scale,
                                void *out, const gqa_options_t *opts,
                                void *stream);

/*
 * gqa_decode_append -- the decode step with its new tokens' K/V appended:
 * the sq new rows of every (sequence b, KV head g), k_new / v_new
 * [B, G, sq, D] (dtype of the caches), are stored into the caches at rows
 * L_b - sq .. L_b - 1 (L_b = clamped seq_lens[b], which counts them; rows
 * that would fall below 0 are dropped), and attention runs over rows
 * 0 .. L_b - 1 as in gqa_decode -- one pass: the new rows are read from
 * k_new / v_new, so the result does not depend on the order of the stores.
 * The rest of the caches is not modified.  This is the incremental decode
 * loop's append-then-attend step ("GQA (Grouped-Query Attention) 분석",
 * section "동작 원리", items 2 "Projection과 RoPE" and 3 "Incremental
 * decode").
 * bf16 or fp16 (GQA_PATH_MFMA; another path or dtype is
 * GQA_ERR_UNSUPPORTED).
 * workspace NULL with ws_bytes 0: the library-owned workspace.
 */
gqa_status_t gqa_decode_append(const gqa_shape_t *shape, const void *q,
                               const void *k_new, const void *v_new,
                               void *k_cache, void *v_cache,
                               const int32_t *seq_lens, float scale, void *out,
                               void *workspace, size_t ws_bytes,
                               const gqa_options_t *opts, void *stream);

/*
 * gqa_decode_fp8 -- gqa_decode over an fp8 cache: shape->kv_dtype ==
 * GQA_FP8_E4M3 (q bf16, out fp32), k_cache / v_cache [B, G, T, D] one byte
 * per element, k_scale / v_scale [G] fp32 on the device (NULL: 1.0): the
 * cache value of a code c in KV head g is e4m3(c) * scale[g].  KV-cache
 * quantization changes only the element precision and composes with GQA
 * ("GQA (Grouped-Query Attention) 분석", section "장단점"); the format and
 * the per-KV-head scale are this library's choice.  Codes are converted to
 * bf16 exactly; accumulation is fp32.  GQA_PATH_MFMA only.  gqa_decode and
 * gqa_decode_ex also take an fp8 shape, with unit scales.
 * workspace NULL with ws_bytes 0: the library-owned workspace.
 */
gqa_status_t gqa_decode_fp8(const gqa_shape_t *shape, const void *q,
                            const void *k_cache, const void *v_cache,
                            const float *k_scale, const float *v_scale,
                            const int32_t *seq_lens, float scale, void *out,
                            void *workspace, size_t ws_bytes,
                            const gqa_options_t *opts, void *stream);

/*
 * gqa_decode_int8 -- gqa_decode_fp8 with an int8 cache: shape->kv_dtype ==
 * GQA_INT8, the cache value of a code c (-128 .. 127) in KV head g is
 * c * scale[g] (k_scale / v_scale as for gqa_decode_fp8).  KV-cache
 * quantization composes with GQA ("GQA (Grouped-Query Attention) 분석",
 * section "장단점"); int8 with one scale per KV head is the other common
 * 8-bit format.  Codes are converted to bf16 exactly (as c + 128, the offset
 * removed from the scores by the softmax and from the outputs at the end);
 * accumulation is fp32.  GQA_PATH_MFMA only.  gqa_decode and gqa_decode_ex
 * also take an int8 shape, with unit scales.
 * workspace NULL with ws_bytes 0: the library-owned workspace.
 */
gqa_status_t gqa_decode_int8(const gqa_shape_t *shape, const void *q,
                             const void *k_cache, const void *v_cache,
                             const float *k_scale, const float *v_scale,
                             const int32_t *seq_lens, float scale, void *out,
                             void *workspace, size_t ws_bytes,
                             const gqa_options_t *opts, void *stream);

/* Shape of a paged cache: page pools k_pages / v_pages [num_pages, G,
 * page_size, D]; block_table [B, max_pages] int32 (device) lists each
 * sequence's pages in order, so row t of sequence b is row
 * t % page_size of page block_table[b][t / page_size].  The capacity per
 * sequence is T = page_size * max_pages.  page_size: a power of two in
 * [16, 65536]. */
typedef struct {
    int32_t B, H, G, sq, D;
    int32_t page_size, num_pages, max_pages;
    int32_t q_dtype, kv_dtype, out_dtype; /* gqa_dtype_t values */
} gqa_paged_shape_t;

/* Device scratch bytes gqa_decode_paged needs (0 on bad shape). */
size_t gqa_paged_workspace_bytes(const gqa_paged_shape_t *shape);

/*
 * gqa_decode_paged -- gqa_decode over a paged cache (see gqa_paged_shape_t):
 * the same result as gqa_decode on the cache the block table describes
 * (paging changes only where cache rows live, so it composes with GQA:
 * "GQA (Grouped-Query Attention) 분석", section "장단점" and the checklist
 * of item 4 of "동작 원리").  Only the table entries for rows below L_b are
 * read; an entry outside [0, num_pages) is clamped into it (no fault, but
 * the result is then meaningless).  bf16 or fp16, or 8-bit codes (fp8
 * E4M3 or int8) read with unit scales: fold a K scale into `scale` and
 * multiply the output by a V scale (GQA_PATH_MFMA).
 * workspace NULL with ws_bytes 0: the library-owned workspace.
 */
gqa_status_t gqa_decode_paged(const gqa_paged_shape_t *shape, const void *q,
                              const void *k_pages, const void *v_pages,
                              const int32_t *block_table,
                              const int32_t *seq_lens, float scale, void *out,
                              void *workspace, size_t ws_bytes,
                              const gqa_options_t *opts, void *stream);

/* Fill *plan for shape and opts (opts may be NULL).  Host only, no GPU work. */
gqa_status_t gqa_plan(const gqa_shape_t *shape, const gqa_options_t *opts,
                      gqa_plan_t *plan);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *gqa_last_error(void);

/* Library version string. */
const char *gqa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
