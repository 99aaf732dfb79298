/*
 * qknorm.h -- C ABI of libqknorm: layerwise QK-Norm on AMD Instinct MI355X (gfx950).
 *
 * The operation (SwiftQK technical review, "Prerequisites", Eq. 1; "Layerwise
 * vs. headwise QK-Norm"): for every token t, the projected query row q[t] and,
 * separately, the projected key row k[t] are RMS-normalised over their FULL
 * width H, with one statistic per row,
 *
 *     y[t][j] = x[t][j] / sqrt( (1/H) * sum_i x[t][i]^2 + eps ) * gamma[j].
 *
 * The sum of squares may be formed as the sum of K per-slice partial sums
 * (review section 4b, Eqs. 3-6, and Algorithm 1's Phase A / Phase B scalar
 * reduction): the H columns are cut into K equal contiguous slices, slice 0
 * holding the first columns; each slice yields one fp32 partial, and the K
 * partials are added in ascending slice order before the scaling. The mean
 * always divides by the full width H.
 *
 * Conventions shared by every entry point
 *  - Memory: every data pointer is a DEVICE pointer owned by the caller. The
 *    library allocates no device memory and keeps no state between calls.
 *  - Layout: rows are row-major; row t of a tensor starts `stride` ELEMENTS
 *    after row t-1. Widths and strides count elements, not bytes.
 *  - Element types: QKNORM_F32 (IEEE binary32), QKNORM_BF16 (bfloat16) or
 *    QKNORM_FP8_E4M3 (OCP FP8 E4M3, the activation format of the review's
 *    Fig. 2(b) FP8 runs). gamma has the element type of the rows it scales,
 *    except that FP8 rows take bfloat16 weights. Statistics are fp32. All
 *    accumulation is fp32 (review section 5: fp32 accumulation even for bf16
 *    or FP8 data). Results are computed in fp32 and rounded to nearest-even
 *    in the output type; FP8 results saturate at +-448 (NaN stays NaN).
 *  - Vectors: data move in 16-byte vectors (16 fp8, 8 bf16 or 4 fp32
 *    elements), so every pointer must be 16-byte aligned and every width,
 *    slice width and stride a multiple of 16 (fp8), 8 (bf16) or 4 (fp32)
 *    elements.
 *  - Streams: `stream` is a hipStream_t (NULL = the null stream) on the
 *    context's device, which must also be the calling thread's current
 *    device. Calls only enqueue work; they never synchronise.
 *  - Errors: each call returns QKNORM_OK (0) or a negative qknorm_status
 *    and never throws. Arguments are validated on the host, in the order
 *    the codes are listed in each entry point's comment, before the context
 *    is looked at and before any HIP call, so bad arguments are reported
 *    even with ctx == NULL and nothing is enqueued. A failed launch returns
 *    QKNORM_ERR_DEVICE; faults inside a kernel surface at the caller's next
 *    synchronisation. Non-finite inputs propagate to the outputs.
 *  - Threads: a context is immutable after creation and may be shared by
 *    threads. Calls that write overlapping memory must be ordered by the
 *    caller (same stream, or events).
 */
#ifndef QKNORM_H
#define QKNORM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the rows (and of gamma, except for FP8 rows). */
typedef enum {
    QKNORM_F32 = 0,
    QKNORM_BF16 = 1,
    QKNORM_FP8_E4M3 = 2   /* OCP FP8 E4M3 rows (no infinities, largest finite
                             448); gamma is bfloat16 for these rows */
} qknorm_dtype;

typedef enum {
    QKNORM_OK = 0,
    QKNORM_ERR_NULL = -1,    /* a required pointer is NULL                          */
    QKNORM_ERR_SHAPE = -2,   /* T < 0, width < 1 or too wide, stride < width,
                                h_total < width                                   */
    QKNORM_ERR_SLICES = -3,  /* num_slices outside [1, 64], width not cut evenly,
                                slice width not whole vectors, slice_index out of
                                range; or head_dim not a valid head width, or
                                width not a whole number of heads               */
    QKNORM_ERR_ALIGN = -4,   /* pointer not 16-byte aligned, or width / stride not
                                a whole number of 16-byte vectors                 */
    QKNORM_ERR_DTYPE = -5,   /* dtype is not a qknorm_dtype                         */
    QKNORM_ERR_EPS = -6,     /* eps negative, NaN or infinite                       */
    QKNORM_ERR_ALIAS = -7,   /* an output overlaps an input without being that same
                                input (same pointer and stride)                   */
    QKNORM_ERR_DEVICE = -8,  /* no usable gfx950 device, wrong current device, or a
                                HIP call / launch failed                          */
    QKNORM_ERR_CONTEXT = -9  /* ctx is NULL (arguments were otherwise valid)        */
} qknorm_status;

/* Opaque context: the device, its compute-unit count and the schedule
 * options. Immutable after creation. */
typedef struct qknorm_ctx qknorm_ctx;

/* One tensor's rows: T rows of `width` elements (T is passed to the call).
 * x and y may be the same buffer (in place) only with x_stride == y_stride. */
typedef struct qknorm_rows {
    const void *x;     /* input rows, device memory                          */
    void *y;           /* output rows, device memory                         */
    int64_t width;     /* elements per row that are read and written         */
    int64_t x_stride;  /* elements from one input row start to the next      */
    int64_t y_stride;  /* elements from one output row start to the next     */
} qknorm_rows;

/* Schedule options (tuning and evidence only; the defaults are chosen from
 * the row width). */
typedef struct qknorm_options {
    int waves_per_row;   /* 0 = choose by width; else 1, 2, 4, 8 or 16 wavefronts
                            share one row (1 = several rows per workgroup)      */
    int max_workgroups;  /* 0 = one workgroup per group of rows; > 0 caps the grid
                            and workgroups loop over rows (persistent grid)     */
    int cached_rows;     /* 0 = stream the row data (non-temporal loads and
                            stores, the default); 1 = ordinary cached accesses
                            (rows cut into many narrow slices always stream)   */
} qknorm_options;

/* Create a context for `device` (a HIP device ordinal) with default options.
 *   QKNORM_ERR_NULL    ctx_out is NULL
 *   QKNORM_ERR_DEVICE  no such device, or it is not a gfx950 GPU
 * On success *ctx_out holds the context; release it with qknorm_destroy. */
int qknorm_create(qknorm_ctx **ctx_out, int device);

/* As qknorm_create, with explicit schedule options (NULL = defaults).
 *   QKNORM_ERR_SHAPE   an option is outside its documented range */
int qknorm_create_ex(qknorm_ctx **ctx_out, int device, const qknorm_options *opts);

/* Release a context (NULL is accepted). Returns QKNORM_OK. */
int qknorm_destroy(qknorm_ctx *ctx);

/*
 * Fused layerwise QK-Norm over the query rows and the key rows of T tokens
 * (SwiftQK review Eq. 1 per tensor; the K-slice scalar statistic of section
 * 4b, Eqs. 3-6), normally in one kernel launch; a large pair of which only
 * one tensor needs the narrow-slice kernels takes one launch per tensor, in
 * order on the stream. Each row is read from memory once and written once:
 * the row stays in registers between the statistic and the scaling.
 *
 *   dtype      element type of q, k, gamma_q and gamma_k
 *   T          tokens (rows of q and of k); T == 0 returns QKNORM_OK at once
 *   q, gamma_q query rows and their width-long weight vector
 *   k, gamma_k key rows and their weights; k == NULL normalises q alone
 *   eps        added to the mean of squares inside the square root (>= 0)
 *   num_slices K: each row's statistic is the ascending-order sum of K
 *              per-slice partial sums over equal contiguous column slices
 *   stream     hipStream_t to enqueue on
 * Status, in validation order: QKNORM_ERR_DTYPE, QKNORM_ERR_SHAPE (T < 0),
 * then for q and k in turn QKNORM_ERR_NULL, QKNORM_ERR_SHAPE,
 * QKNORM_ERR_ALIGN, QKNORM_ERR_SLICES, then QKNORM_ERR_EPS, QKNORM_ERR_ALIAS,
 * QKNORM_ERR_CONTEXT, QKNORM_ERR_DEVICE.
 */
int qknorm_forward(qknorm_ctx *ctx, int dtype, int64_t T,
                   const qknorm_rows *q, const qknorm_rows *k,
                   const void *gamma_q, const void *gamma_k,
                   float eps, int num_slices, void *stream);

/*
 * Fused headwise QK-Norm over the query rows and the key rows of T tokens
 * (SwiftQK review, "Layerwise vs. headwise QK-Norm": one normalisation
 * factor per attention head, the case the layerwise form is contrasted
 * with). Each row holds width / head_dim heads of head_dim contiguous
 * columns, head 0 first; every head is normalised by Eq. 1 over its own
 * columns only (its own sum of squares, the mean over head_dim, eps inside
 * the square root), and the head_dim weights of a tensor are shared by all
 * of its heads. One kernel launch; each row is read once and written once.
 *
 *   head_dim   columns per head, the same for q and k: one head must be a
 *              power of two of 16-byte vectors, at most 64 of them (fp8:
 *              16, 32, ..., 1024 columns; bf16: 8, ..., 512; fp32: 4, ...,
 *              256), and each width a multiple of head_dim
 *   gamma_q, gamma_k  head_dim weights each (gamma's element type)
 *   dtype, T, q, k, eps, stream: as for qknorm_forward
 * Rows are always streamed (the cached_rows option does not apply).
 * Status, in validation order: QKNORM_ERR_DTYPE, QKNORM_ERR_SHAPE (T < 0),
 * then for q and k in turn QKNORM_ERR_NULL, QKNORM_ERR_SHAPE,
 * QKNORM_ERR_ALIGN, QKNORM_ERR_SLICES (head_dim), then QKNORM_ERR_EPS,
 * QKNORM_ERR_ALIAS, QKNORM_ERR_CONTEXT, QKNORM_ERR_DEVICE.
 */
int qknorm_forward_headwise(qknorm_ctx *ctx, int dtype, int64_t T,
                            const qknorm_rows *q, const qknorm_rows *k,
                            const void *gamma_q, const void *gamma_k,
                            int64_t head_dim, float eps, void *stream);

/*
 * The per-token inverse RMS alone, for a consumer that applies the scaling
 * itself (review Eq. 6; the normalisation factors into a static weight and
 * one dynamic scalar per token, which a later stage such as the rotary
 * embedding or the attention kernel can fold in). For every token, over the
 * query rows and the key rows in one launch:
 *
 *     rinv[t] = 1 / sqrt( S_t / width + eps ),
 *
 * S_t formed as qknorm_forward forms it (K slice partials added in
 * ascending order). The value is bit for bit the factor qknorm_forward
 * multiplies row t by: its output is (x * gamma) * rinv in fp32, rounded to
 * the output type.
 *
 *   q, k        rows to read (only x, width and x_stride are used; k may be
 *               NULL)
 *   rinv_q, rinv_k  fp32 device arrays of T values (4-byte aligned); rinv_k
 *               is ignored when k is NULL
 *   dtype, T, eps, num_slices, stream: as for qknorm_forward
 * Status, in validation order: QKNORM_ERR_DTYPE, QKNORM_ERR_SHAPE (T < 0;
 * T == 0 returns QKNORM_OK), then for q and k in turn QKNORM_ERR_NULL,
 * QKNORM_ERR_SHAPE, QKNORM_ERR_ALIGN, QKNORM_ERR_SLICES, then
 * QKNORM_ERR_EPS, QKNORM_ERR_ALIAS (an output overlaps the rows or the other
 * output), QKNORM_ERR_CONTEXT, QKNORM_ERR_DEVICE.
 */
int qknorm_inv_rms(qknorm_ctx *ctx, int dtype, int64_t T,
                   const qknorm_rows *q, const qknorm_rows *k,
                   float eps, int num_slices,
                   float *rinv_q, float *rinv_k, void *stream);

/*
 * Split path, step 1: one slice's partial sums of squares (Algorithm 1,
 * Phase A: a block-wide sum of the local shard's squares, published as one
 * scalar per token; review Eqs. 3-4).
 *
 *   x_slice     first column of the slice: row t starts at
 *               x_slice + t*x_stride elements; slice_width columns are read
 *   slice_index s in [0, num_slices): which row of `stats` to write
 *   stats       fp32 device array laid out [num_slices][T]; the call writes
 *               stats[s*T + t] = sum over the slice's columns of x[t][j]^2
 *               for t in [0, T) and touches nothing else
 * Status, in validation order: QKNORM_ERR_DTYPE, QKNORM_ERR_SHAPE (T < 0;
 * T == 0 returns QKNORM_OK), QKNORM_ERR_NULL, QKNORM_ERR_SHAPE,
 * QKNORM_ERR_ALIGN (stats needs only 4-byte alignment), QKNORM_ERR_SLICES,
 * QKNORM_ERR_ALIAS (stats overlaps the rows), QKNORM_ERR_CONTEXT,
 * QKNORM_ERR_DEVICE.
 */
int qknorm_partial_stats(qknorm_ctx *ctx, int dtype, int64_t T,
                         const void *x_slice, int64_t x_stride,
                         int64_t slice_width, int slice_index, int num_slices,
                         float *stats, void *stream);

/*
 * Split path, step 2: combine the K partial sums of each token in ascending
 * slice order and normalise one slice's columns (Algorithm 1, Phase B's
 * scalar sum and inverse RMS, then Phase C; review Eqs. 5-8).
 *
 *   x_slice     the slice's rows: x_slice->width columns from x_slice->x,
 *               output to x_slice->y (may equal x_slice->x)
 *   gamma_slice the weights of those columns
 *   stats       fp32 [num_slices][T] partial sums, as partial_stats writes them
 *   h_total     width of the FULL row the partials cover: the mean divides by it
 * Status, in validation order: QKNORM_ERR_DTYPE, QKNORM_ERR_SHAPE (T < 0;
 * T == 0 returns QKNORM_OK), QKNORM_ERR_NULL, QKNORM_ERR_SHAPE (including
 * h_total < width or h_total > 2^24), QKNORM_ERR_ALIGN, QKNORM_ERR_SLICES (num_slices outside
 * [1, 64]), QKNORM_ERR_EPS, QKNORM_ERR_ALIAS, QKNORM_ERR_CONTEXT,
 * QKNORM_ERR_DEVICE.
 */
int qknorm_apply_stats(qknorm_ctx *ctx, int dtype, int64_t T,
                       const qknorm_rows *x_slice, const void *gamma_slice,
                       const float *stats, int num_slices, int64_t h_total,
                       float eps, void *stream);

/*
 * Split path, step 1, for the query slice and the key slice of the same
 * tokens in one launch: qknorm_partial_stats applied to each (Algorithm 1,
 * Phase A, for the two normalisations a layer makes; a rank publishes both
 * tensors' partials in one exchange).
 *
 *   q_slice, k_slice  the slices' rows: x, width (the slice width) and
 *                     x_stride are read, y is ignored; k_slice may be NULL
 *   slice_index, num_slices  as for qknorm_partial_stats, the same for both
 *   stats_q, stats_k  fp32 device arrays laid out [num_slices][T]; the call
 *                     writes row slice_index of each and touches nothing
 *                     else (stats_k is ignored when k_slice is NULL)
 * Status, in validation order: QKNORM_ERR_DTYPE, QKNORM_ERR_SHAPE (T < 0;
 * T == 0 returns QKNORM_OK), then for q and k in turn QKNORM_ERR_NULL,
 * QKNORM_ERR_SHAPE, QKNORM_ERR_ALIGN (the statistics need 4-byte alignment),
 * then QKNORM_ERR_SLICES, QKNORM_ERR_ALIAS (a written statistics row
 * overlaps the rows or the other one), QKNORM_ERR_CONTEXT, QKNORM_ERR_DEVICE.
 */
int qknorm_partial_stats_qk(qknorm_ctx *ctx, int dtype, int64_t T,
                            const qknorm_rows *q_slice, const qknorm_rows *k_slice,
                            int slice_index, int num_slices,
                            float *stats_q, float *stats_k, void *stream);

/*
 * Split path, step 2, for the query slice and the key slice of the same
 * tokens in one launch: qknorm_apply_stats applied to each (Algorithm 1,
 * Phase B's scalar sum and inverse RMS, then Phase C; review Eqs. 5-8).
 *
 *   q_slice, k_slice  the slices' rows, output to y (may equal x); k_slice
 *                     may be NULL
 *   gamma_q_slice, gamma_k_slice  the weights of those columns
 *   stats_q, stats_k  fp32 [num_slices][T] partial sums of each tensor
 *   hq_total, hk_total  widths of the FULL query and key rows (the means
 *                     divide by them)
 *   num_slices, eps, stream: as for qknorm_apply_stats
 * Status, in validation order: QKNORM_ERR_DTYPE, QKNORM_ERR_SHAPE (T < 0;
 * T == 0 returns QKNORM_OK), then for q and k in turn QKNORM_ERR_NULL,
 * QKNORM_ERR_SHAPE (including h_total < width or h_total > 2^24),
 * QKNORM_ERR_ALIGN, then QKNORM_ERR_SLICES (num_slices outside [1, 64]),
 * QKNORM_ERR_EPS, QKNORM_ERR_ALIAS (an output overlaps an input of either
 * tensor, without being that same input, or the other output),
 * QKNORM_ERR_CONTEXT, QKNORM_ERR_DEVICE.
 */
int qknorm_apply_stats_qk(qknorm_ctx *ctx, int dtype, int64_t T,
                          const qknorm_rows *q_slice, const qknorm_rows *k_slice,
                          const void *gamma_q_slice, const void *gamma_k_slice,
                          const float *stats_q, const float *stats_k, int num_slices,
                          int64_t hq_total, int64_t hk_total, float eps, void *stream);

/* Static, human-readable text for a status code (never NULL). */
const char *qknorm_status_string(int status);

/* Widest row (in elements) the fused forward accepts for a dtype, or 0 for an
 * unknown dtype. */
int64_t qknorm_max_width(int dtype);

#ifdef __cplusplus
}
#endif

#endif /* QKNORM_H */
