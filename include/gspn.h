/*
 * gspn.h -- C ABI of the MI355X (gfx950) GSPN line-scan library, libgspn.so.
 *
 * The operator is the 2D linear propagation of the Generalized Spatial
 * Propagation Network:
 *
 *   "Parallel Sequence Modeling via Generalized Spatial Propagation Network"
 *   (CVPR 2025 paper notes):
 *     - "Key design 1: stability-context condition": h_i = w_i h_{i-1} +
 *       lambda_i (.) x_i along the lines of the grid, with each w_i made
 *       row-stochastic by a sigmoid on the non-zero entries of each row
 *       followed by division by the row sum;
 *     - "Key design 2: tridiagonal matrix + 4-direction line scan": each pixel
 *       connects to the 3 adjacent pixels of the previous line (top-left,
 *       top, top-right for the top-to-bottom scan); the scan runs in four
 *       directions and the directions are merged;
 *     - "Key design 3: global/local variants": the local variant splits one
 *       spatial dimension into g groups that propagate independently.
 *   "GSPN-2: Efficient Parallel Sequence Modeling" (author response,
 *   paragraphs "How Channel-shared Weight Mitigates the Concurrency
 *   Bottleneck?" and "Justification for Channel-Agnostic Propagation"): one
 *   propagation weight map shared by several channels, channel diversity kept
 *   by the per-channel gains lambda (the compact multi-channel mode).
 *
 * Exact definition computed by gspn_scan_fwd (readings fixed by this ABI where
 * the pages are silent):
 *
 *   For each enabled direction d, batch b, channel c (weight set k = c / cpw):
 *     TB: line i = row i,      position p = column;   n = H lines of m = W
 *     BT: line i = row H-1-i,  position p = column;   n = H, m = W
 *     LR: line i = column i,   position p = row;      n = W, m = H
 *     RL: line i = column W-1-i, position p = row;    n = W, m = H
 *     L = n / groups lines per group.
 *     If i mod L == 0:  h_i[p] = lam[p] * x[p]            (state restarts)
 *     else:             h_i[p] = sum_t w_t * h_{i-1}[p+t-1] + lam[p] * x[p]
 *       over the taps t in {0,1,2} with 0 <= p+t-1 < m, where
 *       w_t = sigmoid(a_t) / (sum of sigmoid(a_s) over the existing taps s)
 *       and a_t = w_raw[slab(d)][b][k][t][pixel of (i, p)].
 *   y[b][c][r][q] = u[b][c][r][q] * sum over enabled d of h_d at pixel (r, q).
 *
 *   Tap t = 0, 1, 2 couples position p to positions p-1, p, p+1 of the
 *   previous line in absolute grid coordinates, for all four directions.
 *   The raw taps of a group's first line and of taps that fall outside the
 *   line are never used and may hold any value (NaN and Inf included).
 *   lam and u are shared by all directions; w_raw has one slab per enabled
 *   direction.
 *
 * Tensor layouts (all C-contiguous, all in the same dtype):
 *   x, lam, u, y : [B][C][H][W]
 *   w_raw        : [popcount(dirs)][B][C / ch_per_weight][3][H][W], one slab
 *                  per enabled direction, in ascending bit order.
 *
 * Arithmetic: inputs are widened to fp32, every product and sum is formed in
 * fp32, and y is rounded to the I/O dtype with round-to-nearest-even.
 * Results match the exact definition to fp32 rounding for raw taps >= -40;
 * rows whose taps are more negative take a slower exact-form branch.
 *
 * Memory and streams: every pointer is a device pointer owned by the caller;
 * base pointers must be 16-byte aligned; y must not overlap any input.  Calls
 * only enqueue work on `stream` and never synchronise; a kernel fault shows
 * at the caller's next synchronisation.  Shapes with H <= 64 and W <= 64 run
 * one fused kernel and allocate nothing; so do the local-group shapes of
 * GSPN_PATH_SLICE (below).  Other shapes run the general path
 * and take a workspace stream-ordered (hipMallocAsync / hipFreeAsync on
 * `stream`): with H, W <= 512 and both multiples of K (1, 2, 4 or 8 as
 * max(H, W) is <= 64, 128, 256 or 512) the line kernels use
 *   popcount(dirs) * B*C*H*W * 4 bytes (fp32 planes) + 2 KiB
 *   + if LR or RL is enabled: (2 * B*C*H*W + ncol * B*(C/cpw)*3*H*W) * s
 * (s = bytes per element, ncol = enabled column directions: transposed
 * copies of x, lambda and their taps); other shapes use the per-line
 * fallback with popcount(dirs) * B*C*H*W * 4 bytes.
 * The library keeps no other state: calls on different streams may run
 * concurrently.  Results are deterministic (fixed summation order, no atomics).
 *
 * Errors: every argument is checked on the host before anything is enqueued;
 * on an error nothing is launched and y is untouched.  A failed HIP call
 * returns GSPN_ERR_HIP and leaves its text in gspn_last_error() (per thread).
 */
#ifndef GSPN_H
#define GSPN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

#define GSPN_VERSION 1

typedef enum { GSPN_F32 = 0, GSPN_BF16 = 1 } gspn_dtype;

enum {
    GSPN_DIR_TB = 1, /* top to bottom */
    GSPN_DIR_BT = 2, /* bottom to top */
    GSPN_DIR_LR = 4, /* left to right */
    GSPN_DIR_RL = 8, /* right to left */
    GSPN_DIR_ALL = 15
};

enum {
    GSPN_OK = 0,
    GSPN_ERR_NULL = -1,   /* a pointer is null */
    GSPN_ERR_SHAPE = -2,  /* B, C, H or W <= 0, H or W > GSPN_MAX_SIDE, B*C > 2^22 */
    GSPN_ERR_DIRS = -3,   /* dirs is 0 or has a bit above 0xF */
    GSPN_ERR_GROUPS = -4, /* groups < 1, or it does not divide a scanned side */
    GSPN_ERR_CPW = -5,    /* ch_per_weight < 1 or it does not divide C */
    GSPN_ERR_DTYPE = -6,  /* unknown dtype */
    GSPN_ERR_ALIGN = -7,  /* a base pointer is not 16-byte aligned */
    GSPN_ERR_ALIAS = -8,  /* an output overlaps an input or another output */
    GSPN_ERR_HIP = -9,    /* a HIP call failed; see gspn_last_error() */
    GSPN_ERR_PATH = -10,  /* unknown path, or the path (or the backward) cannot take this shape */
    GSPN_ERR_FLAGS = -11, /* unknown bit in flags (gspn_scan_fwd_ex, gspn_scan_bwd_ex, gspn_block_fwd) */
    GSPN_ERR_SCRATCH = -12 /* the shape's workspace exceeds GSPN_NOALLOC_SCRATCH_BYTES (gspn_scan_fwd_noalloc) */
};

/* Flags of gspn_scan_fwd_ex and gspn_scan_bwd_ex. */
enum {
    GSPN_LAM_PER_DIR = 1, /* lam holds one [B][C][H][W] slab per enabled direction */
    GSPN_U_PER_DIR = 2    /* u holds one slab per enabled direction: y = sum_d u_d * h_d */
};

/* Largest H and W accepted. */
#define GSPN_MAX_SIDE 4096

/* Kernel paths for gspn_scan_fwd_path. */
enum {
    GSPN_PATH_AUTO = 0,    /* what gspn_scan_fwd uses */
    GSPN_PATH_FUSED = 1,   /* one fused 4-direction kernel; needs H <= 64 and W <= 64 */
    GSPN_PATH_GENERAL = 2, /* line (or per-line) kernels + merge; any shape; uses a workspace */
    GSPN_PATH_SLICE = 3    /* one workgroup per (b, c) slice, the sum of the directions held on chip; bf16,
                              H, W <= 128, W % 8 == 0, H even, groups >= 8, (W / groups) % 8 == 0 when LR or
                              RL is enabled; no workspace.  GSPN_PATH_AUTO takes it for such shapes when
                              they do not fit the fused kernel. */
};

/*
 * Forward 4-direction scan (definition above).
 *   x, lam, u : [B][C][H][W] inputs;  w_raw : raw taps (layout above)
 *   y         : [B][C][H][W] output, fully overwritten
 *   dirs      : bitmask of GSPN_DIR_*, 1..15
 *   groups    : g >= 1; must divide H if TB or BT is enabled, and W if LR or
 *               RL is enabled (g = 1 is the global scan)
 *   ch_per_weight : channels per weight set, divides C (1 = per-channel
 *               weights, C = one map shared by every channel)
 *   dtype     : gspn_dtype of all five tensors
 *   stream    : HIP stream the work is enqueued on (0 = null stream)
 * Returns GSPN_OK or a negative GSPN_ERR_* code.
 */
int gspn_scan_fwd(const void *x, const void *w_raw, const void *lam, const void *u, void *y,
                  int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                  int32_t ch_per_weight, int32_t dtype, hipStream_t stream);

/*
 * gspn_scan_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same operation, arguments, layouts and errors as gspn_scan_fwd, and the
 * same kernels.  It calls no hipMalloc, hipFree or allocating library
 * routine: where gspn_scan_fwd takes a stream-ordered workspace (shapes with
 * H or W above 64), this entry point uses a static device array of
 * GSPN_NOALLOC_SCRATCH_BYTES, one per GPU, held until the process ends;
 * shapes with H, W <= 64 need none.  A shape whose workspace (the formula
 * above) is larger returns GSPN_ERR_SCRATCH before anything is enqueued.
 * Every call on one GPU shares that GPU's array and leaves it holding that
 * call's intermediates (nothing in it needs to start at zero): calls that
 * overlap on one GPU (on different streams or threads) race on it and must
 * be serialised by the caller.  The first call on a device, made with that
 * device current, looks up the array's device address (hipGetSymbolAddress;
 * GSPN_ERR_HIP if that fails) and keeps it for later calls.
 */
#define GSPN_NOALLOC_SCRATCH_BYTES (64u << 20)

int gspn_scan_fwd_noalloc(const void *x, const void *w_raw, const void *lam, const void *u, void *y,
                          int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                          int32_t ch_per_weight, int32_t dtype, hipStream_t stream);

/* Same operation on a chosen kernel path (GSPN_PATH_*); used to cross-check
 * the paths against each other.  GSPN_ERR_PATH if the path cannot run the
 * shape. */
int gspn_scan_fwd_path(const void *x, const void *w_raw, const void *lam, const void *u, void *y,
                       int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                       int32_t ch_per_weight, int32_t dtype, int32_t path, hipStream_t stream);

/*
 * Variants of the forward with per-direction gains and gates:
 *   y = sum over enabled d of u_d (.) h_d,   h_d the scan of direction d driven
 *   by lam_d (.) x (otherwise exactly the definition above).
 * The pages index neither lam nor u by direction ("Key design 1"), so
 * gspn_scan_fwd shares them; "Key design 2" merges the directions with a
 * "learnable merger", which a per-direction gate u_d realises elementwise
 * (per-channel direction weights are the case of u_d constant over H, W).
 *   flags : GSPN_LAM_PER_DIR and/or GSPN_U_PER_DIR; a flagged tensor has
 *           shape [popcount(dirs)][B][C][H][W], slabs in ascending bit order.
 *           flags = 0 is gspn_scan_fwd.
 * Other arguments, layouts and errors as gspn_scan_fwd; unknown flag bits
 * give GSPN_ERR_FLAGS.  With a flag set the call runs the line kernels
 * (H, W <= 512 and multiples of K, else GSPN_ERR_PATH) and, with
 * GSPN_LAM_PER_DIR and LR or RL enabled, its workspace holds one transposed
 * lam per column direction.  gspn_scan_bwd_ex is its backward.
 */
int gspn_scan_fwd_ex(const void *x, const void *w_raw, const void *lam, const void *u, void *y,
                     int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                     int32_t ch_per_weight, uint32_t flags, int32_t dtype, hipStream_t stream);

/*
 * Several independent forward problems in one launch, for workloads too
 * small to occupy the GPU alone (GSPN-2 author response, "SM Utilization
 * for Small Workloads": micro-batching small launches).  Each problem is
 * exactly one gspn_scan_fwd call (its own tensors, sizes, dirs, groups and
 * ch_per_weight); all share `dtype` and `stream`.
 *   problems : host array of `count` descriptors (1 <= count <=
 *              GSPN_MAX_BATCH), read during the call only
 * Every problem must take the fused path (H <= 64 and W <= 64), else
 * GSPN_ERR_PATH; count outside [1, GSPN_MAX_BATCH] gives GSPN_ERR_SHAPE.
 * Each problem is validated as gspn_scan_fwd validates its arguments, and
 * no problem's y may overlap any problem's input or another problem's y
 * (GSPN_ERR_ALIAS).  On any error nothing is launched.  Results equal those
 * of separate gspn_scan_fwd calls (the same kernel code runs every problem).
 */
#define GSPN_MAX_BATCH 32

typedef struct {
    const void *x, *w_raw, *lam, *u; /* inputs, layouts as in gspn_scan_fwd */
    void *y;                         /* output */
    int64_t B, C, H, W;
    uint32_t dirs;
    int32_t groups, ch_per_weight;
} gspn_problem;

int gspn_scan_fwd_batched(const gspn_problem *problems, int32_t count, int32_t dtype, hipStream_t stream);

/* The path gspn_scan_fwd would take for these sizes (GSPN_PATH_FUSED,
 * GSPN_PATH_SLICE or GSPN_PATH_GENERAL), or a negative error code for
 * invalid sizes. */
int gspn_select_path(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                     int32_t ch_per_weight, int32_t dtype);

/*
 * Backward of gspn_scan_fwd: the exact vector-Jacobian product of the
 * definition above for a loss L with dL/dy = gy.  The pages give no formulas
 * for it ("GSPN-2: Efficient Parallel Sequence Modeling", author response,
 * "Backward Benchmark", states only that the backward's launch design and
 * speed-up follow the forward's); with
 * S = sum over enabled d of h_d and g_d the adjoint state of direction d:
 *   gu   = gy * S
 *   g_d  : for the lines of each group from its last line back to its first,
 *          g_i = gy * u (at line i) + w_{i+1}^T g_{i+1}, the second term only
 *          when line i+1 is in the same group;
 *          (w^T g)[p] = w_0[p+1] g[p+1] + w_1[p] g[p] + w_2[p-1] g[p-1]
 *   gx   = lam * sum_d g_d,   glam = x * sum_d g_d
 *   gw_raw[slab(d)][b][k][t][pixel of (i, p)] = w_t (1 - sigmoid(a_t))
 *          (D_t - sum_v D_v w_v),  D_t = sum over the channels c of weight
 *          set k of g_i[p] h_{i-1}[p+t-1],
 *          for the taps the forward reads, and 0 for every other tap
 *          (missing border neighbours, first lines of groups, lines of
 *          length 1).
 *   x, w_raw, lam, u, gy : inputs, layouts and dtype as in gspn_scan_fwd
 *   gx, glam, gu : [B][C][H][W] outputs;  gw_raw : layout of w_raw (output)
 * All four outputs are fully overwritten and must not overlap each other or
 * an input (GSPN_ERR_ALIAS).  Arithmetic in fp32, outputs rounded to the
 * dtype with round-to-nearest-even; tap gradients are summed over a set's
 * channels in a fixed order (deterministic).
 * Shapes: H, W <= 512 and both multiples of K (as for the forward's line
 * kernels), else GSPN_ERR_PATH; gspn_bwd_supported tells in advance.
 * H <= 64 and W <= 64 run one fused kernel (one workgroup per weight set,
 * all states in LDS) and allocate nothing.  Larger shapes run the line
 * kernels with a workspace taken stream-ordered on `stream`
 * (hipMallocAsync/hipFreeAsync), each part rounded up to 256 bytes:
 *   popcount(dirs) * B*C*H*W * 4 (fp32 states, then adjoints) + 2 KiB
 *   + popcount(dirs) * B*(C/cpw)*3*H*W * 4 (fp32 tap gradients)
 *   + if LR or RL is enabled: (4 * B*C*H*W + ncol * B*(C/cpw)*3*H*W) * s
 *     (transposed x, lam, gy, u and column-direction taps).
 * Enqueues only; never synchronises.
 */
int gspn_scan_bwd(const void *x, const void *w_raw, const void *lam, const void *u, const void *gy,
                  void *gx, void *gw_raw, void *glam, void *gu, int64_t B, int64_t C, int64_t H,
                  int64_t W, uint32_t dirs, int32_t groups, int32_t ch_per_weight, int32_t dtype,
                  hipStream_t stream);

/* Same operation on a chosen kernel path (GSPN_PATH_FUSED: H, W <= 64;
 * GSPN_PATH_GENERAL: the line kernels); used to cross-check the paths.
 * GSPN_ERR_PATH if the path cannot run the shape. */
int gspn_scan_bwd_path(const void *x, const void *w_raw, const void *lam, const void *u, const void *gy,
                       void *gx, void *gw_raw, void *glam, void *gu, int64_t B, int64_t C, int64_t H,
                       int64_t W, uint32_t dirs, int32_t groups, int32_t ch_per_weight, int32_t dtype,
                       int32_t path, hipStream_t stream);

/*
 * Backward of gspn_scan_fwd_ex (per-direction lam and/or u): the exact
 * vector-Jacobian product of y = sum over enabled d of u_d * h_d, h_d the scan
 * of direction d driven by lam_d * x.  With g_d the adjoint of direction d
 * (as in gspn_scan_bwd, with u_d in its source term gy * u_d):
 *   gu_d   = gy * h_d             (GSPN_U_PER_DIR; else gu = gy * sum_d h_d)
 *   glam_d = x * g_d              (GSPN_LAM_PER_DIR; else glam = x * sum_d g_d)
 *   gx     = sum_d lam_d * g_d
 *   gw_raw as in gspn_scan_bwd, from each direction's own g_d and h_d.
 *   flags : as in gspn_scan_fwd_ex; a flagged input (lam, u) and its
 *           gradient (glam, gu) are [popcount(dirs)][B][C][H][W], slabs in
 *           ascending bit order.  flags = 0 is gspn_scan_bwd.
 * With a flag set the call runs the line kernels (H, W <= 512 and multiples
 * of K, else GSPN_ERR_PATH); the workspace is that of gspn_scan_bwd, with one
 * transposed lam (GSPN_LAM_PER_DIR) and one transposed u (GSPN_U_PER_DIR)
 * per enabled column direction instead of one.  Unknown flag bits give
 * GSPN_ERR_FLAGS; other errors, aliasing rules and tolerances as
 * gspn_scan_bwd.
 */
int gspn_scan_bwd_ex(const void *x, const void *w_raw, const void *lam, const void *u, const void *gy,
                     void *gx, void *gw_raw, void *glam, void *gu, int64_t B, int64_t C, int64_t H, int64_t W,
                     uint32_t dirs, int32_t groups, int32_t ch_per_weight, uint32_t flags, int32_t dtype,
                     hipStream_t stream);

/* Flags of gspn_block_fwd. */
enum {
    GSPN_BLOCK_RMSNORM = 1 /* normalise each pixel's scan output by its RMS over C_proxy before projecting back */
};
#define GSPN_BLOCK_NORM_EPS 1e-6f

/*
 * The compressed propagation block around the scan (GSPN-2 author response,
 * "Relate Compressive Proxy Dimension to Low-rank Approximation": x is
 * projected to x_proxy with C_proxy channels by a lightweight linear layer,
 * the recurrence runs there, and the result is projected back to C; C-GSPN
 * abstract: a compressed latent-space propagation block with fused
 * normalization).  Per pixel:
 *   [x_proxy; a; lam; u] = w_in x      (a: the raw taps of the scan)
 *   y = gspn_scan_fwd(x_proxy, a, lam, u)   over C_proxy channels
 *   with GSPN_BLOCK_RMSNORM: y <- y / sqrt(mean over the C_proxy channels
 *                            of y^2 + GSPN_BLOCK_NORM_EPS)
 *   z = w_out y
 * The pages do not say how the taps, lam and u are generated; here they are
 * further rows of the input projection (plain linear, no activation).  Nor
 * do they name the block's normalisation: it is read as an RMS
 * normalisation of the propagated latent, with no learned gain (w_out
 * absorbs a per-channel gain), fused into the output projection: for bf16
 * with C_proxy in {16, 32, 64, 128, 256}, C % 32 == 0 and H*W % 8 == 0 one
 * hand-written MFMA kernel computes the RMS of each pixel from the same
 * C_proxy values it multiplies (other shapes: a rocBLAS GEMM, then a
 * scaling pass).  The taps' own sigmoid-then-row normalisation is the
 * scan's (fused in its kernels).
 *   flags : 0 or GSPN_BLOCK_RMSNORM; other bits give GSPN_ERR_FLAGS.
 *   x     : [B][C][H][W]
 *   w_in  : [gspn_block_rows(C_proxy, dirs, ch_per_weight)][C], row-major;
 *           rows: x_proxy (C_proxy), the raw taps (one slab of
 *           (C_proxy/ch_per_weight)*3 rows per enabled direction, in bit
 *           order; set k, tap t at row k*3 + t of its slab), lam (C_proxy),
 *           u (C_proxy)
 *   w_out : [C][C_proxy], row-major
 *   z     : [B][C][H][W], written
 * The generated tensors and the scan output are stored in `dtype` (bf16:
 * rounded to nearest even) in a stream-ordered workspace.  The input
 * projection is one GEMM (x read once) into g = [B][rows][H*W] (rows =
 * gspn_block_rows).  For H, W <= 64 the fused scan reads g in place
 * (workspace (rows + C_proxy) * B*H*W elements); otherwise g's row blocks
 * are copied into contiguous tensors and the scan is gspn_scan_fwd on the
 * automatic path (workspace (2*rows + C_proxy) * B*H*W elements).  When
 * the normalisation follows a library GEMM (the shapes the MFMA kernel does
 * not take) the GEMM writes fp32 into B*C*H*W*4 more workspace bytes and
 * the scaling pass rounds z once.  The input projection is a rocBLAS GEMM;
 * both projections accumulate in fp32.  The first call on a
 * device creates a rocBLAS handle that the library keeps until the process
 * ends (the scan entry points hold no state); calls are serialised on it by
 * a mutex while they enqueue, and only enqueue work on `stream`.  Sizes, dirs, groups, ch_per_weight
 * (which must divide C_proxy) and dtype are checked as in gspn_scan_fwd with
 * C_proxy in the place of C, and C >= 1; z may not overlap x, w_in or w_out
 * (GSPN_ERR_ALIAS).  GSPN_ERR_HIP if rocBLAS or a HIP call fails.
 */
int gspn_block_fwd(const void *x, const void *w_in, const void *w_out, void *z, int64_t B, int64_t C,
                   int64_t C_proxy, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                   int32_t ch_per_weight, uint32_t flags, int32_t dtype, hipStream_t stream);

/* Rows of gspn_block_fwd's w_in, 3*C_proxy + 3*popcount(dirs)*(C_proxy/ch_per_weight),
 * or a negative GSPN_ERR_* code for invalid arguments. */
int64_t gspn_block_rows(int64_t C_proxy, uint32_t dirs, int32_t ch_per_weight);

/* GSPN_OK if gspn_scan_bwd can run these sizes, GSPN_ERR_PATH if the shape is
 * outside its kernels, or another negative code for invalid sizes. */
int gspn_bwd_supported(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                       int32_t ch_per_weight, int32_t dtype);

/* Static text for a status code. */
const char *gspn_status_string(int status);

/* Detail of the calling thread's last failure ("" if none). */
const char *gspn_last_error(void);

/* GSPN_VERSION of the built library. */
int gspn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GSPN_H */
