/*
 * lin_epi -- fp32 linear layer Y = X * W^T + b with its elementwise tail fused
 * into the GEMM epilogue, for AMD Instinct MI355X (gfx950).
 *
 * The operation is nn.Linear followed by one of three tails, as the pages
 * state the problems:
 *
 *   kind 1, scale -> Hardtanh(min, max) -> exact-erf GELU
 *       page "Kimi-K2.6 l2_p53" (POPCORNBENCH), problem statement: GEMM,
 *       scale by a constant, Hardtanh clamp, GELU.
 *   kind 2, AvgPool1d(16, stride 16, no padding, floor mode) over the output
 *       features -> exact-erf GELU -> scale -> max over the pooled features
 *       page "Kimi-K2.6 l2_p98", its step-by-step reading of the reference
 *       model (Linear, AvgPool1d defaults, GELU, scale, max over dim 1).
 *   kind 3, swish y * sigmoid(y) -> scale
 *       page "Kimi-K2.6 l2_p59", problem analysis (swish, then scaling).
 *   kind 4, exact-erf GELU -> scale -> max over the output features, with no
 *       pooling: tail (b) applied to a layer whose weights were already
 *       averaged per window (lin_epi_pool_weights), the pooled-weight form
 *       page "Kimi-K2.6 l2_p98" derives (pooling a linear layer's output
 *       equals a linear layer with window-averaged weights and bias) and
 *       adopts for its final module.
 *   kind 0, no tail (the plain linear layer), for tests.
 *
 * GELU is 0.5 * x * (1 + erf(x / sqrt 2)) (PyTorch's default form, which
 * page l2_p53 settles on).  All arithmetic is IEEE binary32: fp32 products
 * and fp32 accumulation on the matrix cores; no reduced-precision path.
 *
 * Memory: every pointer argument of lin_epi_run is a DEVICE pointer on the
 * current HIP device, owned by the caller, row-major and densely packed:
 *   X [M, K], W [N, K] (each output feature's weights K-contiguous, the
 *   nn.Linear weight layout), b [N], Y [M, N] for kinds 0, 1, 3 and Y [M]
 *   for kinds 2 and 4.
 * X and W must be 16-byte aligned and K a multiple of 4 (rows are read with
 * 128-bit loads); Y must be 4-byte aligned.  Y must not alias X, W or b.
 *
 * Threading and streams: a handle is bound to one HIP stream at creation and
 * is not thread-safe.  lin_epi_run only enqueues work on that stream and
 * returns; the caller synchronises.  The handle owns a device workspace
 * (partial sums of output tiles split over workgroups, their arrival
 * counters, per-tile row maxima) that grows on demand; two runs in flight
 * on the same handle share it, which is safe because they are ordered on the
 * handle's stream.
 *
 * Errors: every call returns a status code (LIN_EPI_OK = 0 or a negative
 * LIN_EPI_E* value).  Arguments are validated on the host before any HIP
 * call, so an invalid call enqueues nothing and leaves Y untouched.
 */
#ifndef LIN_EPI_H
#define LIN_EPI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lin_epi_ctx *lin_epi_handle;

typedef enum {
    LIN_EPI_NONE = 0,                   /* Y = X W^T + b */
    LIN_EPI_SCALE_HARDTANH_GELU = 1,    /* Y = GELU(clamp((XW^T+b)*scale, ht_min, ht_max)) */
    LIN_EPI_POOL_GELU_SCALE_ROWMAX = 2, /* Y[m] = max_j scale*GELU(mean_{t<16} y[m,16j+t]) */
    LIN_EPI_SWISH_SCALE = 3,            /* Y = (y * sigmoid(y)) * scale */
    LIN_EPI_GELU_SCALE_ROWMAX = 4       /* Y[m] = max_n scale*GELU(y[m,n]) */
} lin_epi_kind;

/* Tail parameters.  Fields a kind does not use are ignored. */
typedef struct {
    int32_t kind;        /* lin_epi_kind */
    float scale;         /* kinds 1, 2, 3, 4 */
    float ht_min;        /* kind 1: Hardtanh lower bound (inclusive clamp) */
    float ht_max;        /* kind 1: Hardtanh upper bound, ht_min <= ht_max */
    int32_t pool_kernel; /* kind 2: must be 16 */
    int32_t pool_stride; /* kind 2: must equal pool_kernel (AvgPool1d default) */
} lin_epi_desc;

enum {
    LIN_EPI_OK = 0,
    LIN_EPI_EINVAL = -1,  /* null handle/pointer/desc, negative size, unknown kind, ht_min > ht_max,
                             pool_kernel < 1 */
    LIN_EPI_EALIGN = -2,  /* X or W not 16-byte aligned, K % 4 != 0, Y not 4-byte aligned */
    LIN_EPI_ENOTSUP = -3, /* kind 2 with pool_kernel != 16, pool_stride != pool_kernel, or N < 16 */
    LIN_EPI_ENOMEM = -4,  /* workspace allocation failed */
    LIN_EPI_EHIP = -5,    /* a HIP call or kernel launch failed */
    LIN_EPI_ETOOBIG = -6  /* lin_epi_run_noalloc: the problem needs more workspace than the fixed
                             scratch array holds (lin_epi_noalloc_scratch_bytes) */
};

/* Create a handle bound to `hip_stream` (a hipStream_t; NULL = the default
 * stream).  Makes no device allocation.  *out is set to NULL on failure. */
int lin_epi_create(lin_epi_handle *out, void *hip_stream);

/* Enqueue Y = tail(X W^T + b) on the handle's stream: the forward pass of
 * the pages' model (page "Kimi-K2.6 l2_p53", its ModelNew.forward: the
 * linear layer with weight [out, in] and bias, then the tail), with the tail
 * chosen by desc->kind and the layer's parameters passed per call.
 *   X  [M, K] device, read only       W [N, K] device, read only
 *   b  [N]    device, read only       Y [M, N] (kinds 0, 1, 3) or [M]
 *                                       (kinds 2, 4) device, written
 * The caller owns every buffer and keeps it alive until the stream reaches
 * the end of the call; the handle's workspace holds any intermediate
 * (K-slice partial sums, per-tile row maxima).
 * M == 0 or N == 0 is a successful no-op.  K == 0 is allowed and gives
 * Y = tail(b) broadcast over the rows (the empty sum is 0); X and W may then
 * be NULL.  b must not be NULL (every layer on the pages has a bias).
 * Errors: EINVAL (null handle, desc, b or Y, or X/W with K > 0; negative or
 * > INT32_MAX sizes; unknown kind; ht_min > ht_max), EALIGN, ENOTSUP (kind 2
 * with another window or N < 16), ENOMEM (workspace), EHIP (launch); on an
 * error nothing is enqueued. */
int lin_epi_run(lin_epi_handle h, int64_t M, int64_t N, int64_t K,
                const float *X, const float *W, const float *b,
                const lin_epi_desc *desc, float *Y);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, arguments, errors and kernels as lin_epi_run, with every
 * intermediate (arrival counters of split tiles, their partial sums, per-tile
 * row maxima) in a fixed device array of lin_epi_noalloc_scratch_bytes()
 * bytes (64 MiB) that the library holds on each GPU it runs on until the
 * process ends, instead of the handle's workspace.  Makes no allocation of
 * any kind: the plan is chosen among those whose intermediates fit, and a
 * problem with none (a row-max tail with very many rows) returns
 * LIN_EPI_ETOOBIG before anything is enqueued.  The handle's device must be
 * the current device.  Every call on a GPU shares that GPU's array, so calls
 * that overlap on one GPU (other streams, other handles, other threads) race
 * and give wrong results; calls ordered on one stream are safe. */
int lin_epi_run_noalloc(lin_epi_handle h, int64_t M, int64_t N, int64_t K,
                        const float *X, const float *W, const float *b,
                        const lin_epi_desc *desc, float *Y);

/* Size in bytes of the fixed scratch array lin_epi_run_noalloc uses. */
int64_t lin_epi_noalloc_scratch_bytes(void);

/* Release the handle and its workspace (waits for the handle's stream
 * first).  NULL is a no-op. */
int lin_epi_destroy(lin_epi_handle h);

/* Static string for a status code. */
const char *lin_epi_status_string(int status);

/* Window-averaged weights for tail (b), once per weight (page "Kimi-K2.6
 * l2_p98": the pooled weight and bias are precomputed at construction and
 * the forward pass is a linear layer with them, followed by GELU, scale and
 * the row max).  With L = floor(N / pool_kernel):
 *   Wp[j, k] = (1/pool_kernel) * sum_{t<pool_kernel} W[j*pool_kernel + t, k],
 *   bp[j]    = (1/pool_kernel) * sum_{t<pool_kernel} b[j*pool_kernel + t],
 * the rows added in increasing t.  W [N, K], b [N] in; Wp [L, K], bp [L] out,
 * all device pointers owned by the caller; W and Wp 16-byte aligned, K a
 * multiple of 4.  Then lin_epi_run(h, M, L, K, X, Wp, bp, desc with kind 4,
 * Y) gives tail (b) of the original layer up to fp32 rounding, with a GEMM
 * pool_kernel times smaller.  Enqueued on the handle's stream.  L == 0 is a
 * no-op.  Errors as lin_epi_run (EINVAL, EALIGN, EHIP). */
int lin_epi_pool_weights(lin_epi_handle h, int64_t N, int64_t K, const float *W, const float *b,
                         int32_t pool_kernel, float *Wp, float *bp);

/* Weights with tail (a)'s scale folded in, once per weight (page "Kimi-K2.6
 * l2_p53": scaling the linear output equals a linear layer with scaled
 * weights and bias, so the multiply can leave the tail):
 *   Ws[n, k] = scale * W[n, k],  bs[n] = scale * b[n].
 * Then lin_epi_run(..., Ws, bs, desc with kind 1 and scale 1, Y) gives tail
 * (a) of the original layer; for a power-of-two scale (the pages' 0.5) the
 * result is bit-identical, since such scaling commutes with fp32 rounding
 * (barring overflow and subnormals).  Only tail (a) allows this: tails (b)
 * and (c) apply their scale after a nonlinearity.  W [N, K], b [N] in;
 * Ws [N, K], bs [N] out (may equal W, b); device pointers, W and Ws 16-byte
 * aligned, K a multiple of 4.  Enqueued on the handle's stream. */
int lin_epi_scale_weights(lin_epi_handle h, int64_t N, int64_t K, const float *W, const float *b, float scale,
                          float *Ws, float *bs);

/* ---- tuning and introspection (not needed for ordinary use) ------------- */

enum {
    /* Split-K control: 0 = automatic (default), 1 = never split (one
     * output tile per workgroup), S >= 2 = every output tile computed in S
     * K segments by S workgroups (clamped to the K steps available).  The
     * last of a tile's workgroups to finish adds the segments' partial sums
     * in K order, so results are the same on every run. */
    LIN_EPI_OPT_SPLIT_K = 1,
    /* 1 = time every kernel this handle launches with HIP events on its
     * stream (read with lin_epi_profile_read); 0 = off (default). */
    LIN_EPI_OPT_PROFILE = 2,
    /* 1 = unfused ablation: the GEMM writes the raw linear output (to Y for
     * kinds 0, 1, 3, to the workspace for kinds 2, 4) and a separate kernel
     * then applies the tail, as the pages' own solutions do after a library
     * GEMM; 0 = fused (default).  Same results within the tolerance; exists
     * to measure what fusion saves. */
    LIN_EPI_OPT_UNFUSED = 3,
    /* Tile configuration: 0 = automatic (default); 1 = 256x256 tiles with 8
     * wavefronts, 2 = 128x256 with 8, 3 = 128x128 with 4, 4 = 64x64 with 4,
     * 5 = 32x128 with 4 (few rows, weight streaming), 6 = the weight-streaming
     * kernel without LDS (16 rows of X against 64 rows of W per wavefront, any
     * M; the plan reports a 16x64 tile; automatic when 64 rows of W span
     * 1 GiB or more), 7 = 64x128 with 4 wavefronts (three workgroups per
     * CU), 8 = 128x96 with 4 wavefronts (two workgroups per CU).  The
     * split-K choice is still made (or forced) as usual. */
    LIN_EPI_OPT_TILE = 4,
    /* 1 = stage X and W tiles through registers (128-bit loads, then LDS
     * stores) even where the default direct-to-LDS buffer loads are usable;
     * 0 = automatic (default).  Both stagings feed the same MFMA sequence,
     * so results are bit-identical; exists to test and measure the
     * direct-to-LDS path against the other one. */
    LIN_EPI_OPT_REG_STAGING = 5,
    /* Stream-K grid: 0 = automatic (default), G >= 1 = run the GEMM with G
     * workgroups that divide the (tile, K step) work into G contiguous
     * ranges, balanced to within one K step (clamped to the work available);
     * tiles a range boundary cuts are finished as with LIN_EPI_OPT_SPLIT_K.
     * Overrides LIN_EPI_OPT_SPLIT_K. */
    LIN_EPI_OPT_GRID = 6
};

int lin_epi_set_option(lin_epi_handle h, int32_t option, int64_t value);

/* What the last successful lin_epi_run launched. */
typedef struct {
    int32_t tile_m, tile_n, tile_k; /* workgroup output tile and K step */
    int32_t split_k;                /* most K segments any output tile is cut into (1 = none) */
    int64_t grid_main;              /* workgroups of the GEMM kernel */
    int32_t kernels;                /* kernels launched: 1, or 2 with the row-max finalize pass (behind
                                       the weight-streaming kernel only) or the unfused tail kernel */
    int64_t workspace_bytes;        /* workspace the run used */
    int32_t schedule;               /* 0: one output tile per workgroup; 1: split-K, grid = tiles *
                                       split_k, equal K segments; 2: stream-K, workgroup ranges
                                       cross tile boundaries */
    int64_t partial_bytes;          /* partial sums the split tiles' other segments publish for the
                                       finishing one: one slot per such segment, each written once and
                                       read back once (0 when no tile is split) */
} lin_epi_plan;

int lin_epi_last_plan(lin_epi_handle h, lin_epi_plan *out);

/* The plan lin_epi_run would use for this problem, honouring the handle's
 * options, on a device with `num_cus` compute units (0 = the current
 * device's count, which needs a HIP call; any positive value makes this a
 * pure host computation).  M == 0 or N == 0 gives an all-zero plan.  Same
 * argument checks as lin_epi_run except the pointer ones. */
int lin_epi_query_plan(lin_epi_handle h, int64_t M, int64_t N, int64_t K, const lin_epi_desc *desc,
                       int32_t num_cus, lin_epi_plan *out);

/* Accumulated kernel timings since the last read (profiling on).  Waits for
 * the handle's stream.  Role 0 is the GEMM kernel, role 1 the second pass
 * (row-max finalize behind the weight-streaming kernel), role 2 the separate
 * tail kernel of the unfused ablation, lin_epi_pool_weights and
 * lin_epi_scale_weights. */
typedef struct {
    int64_t launches[3];
    double total_ms[3];
} lin_epi_profile;

int lin_epi_profile_read(lin_epi_handle h, lin_epi_profile *out);

#ifdef __cplusplus
}
#endif

#endif /* LIN_EPI_H */
