/*
 * muon.h -- C ABI of the MI355X (gfx950) Muon Newton-Schulz update library.
 *
 * The operation (blog.hotdry.top, "How to train a GPT model in 3 minutes: an
 * analysis of modded-nanogpt's optimizations", section 2, item "customised
 * Muon optimizer"): Muon updates each hidden weight matrix with its momentum
 * orthogonalised by a Newton-Schulz iteration instead of an SVD, keeping one
 * momentum buffer per matrix. For every matrix G (rows x cols) of a set:
 *
 *   buf' = mu * buf + G           (stored back at the buffer dtype, RNE)
 *   u    = G + mu * buf'  (Nesterov)   or   u = buf'
 *   X    = u / (||u||_F + eps)
 *   if rows > cols: X = X^T        (so the Gram matrix is min(rows,cols)^2)
 *   k times:  A = X X^T;  B = b A + c A A;  X = a X + B X
 *   out  = X (transposed back), stored at the set's dtype (RNE)
 *
 * Arithmetic: momentum, norms and the X master copy are fp32. The matrix
 * products run on the matrix cores with fp32 accumulation; their operands
 * (X, A, B) are fp16 for bf16 sets by default (MUON_PRECISION_DEFAULT:
 * 11-bit significands at the same MFMA rate as bf16, and every iterate is
 * bounded by the normalisation) or bf16 (MUON_PRECISION_BF16_OPERANDS);
 * fp32 sets use fp32 operands throughout.
 *
 * Conventions shared by every entry point:
 *  - Pointers in muon_matrix, `workspace` and `stream` are device-side
 *    objects owned by the caller (`stream` is a hipStream_t; NULL = the
 *    default stream). The library never frees or retains them beyond a call,
 *    except that a plan remembers the matrix pointers it was created with.
 *  - All arguments are validated before any work is enqueued. On an error
 *    nothing is launched and nothing is written; the status says why.
 *  - Work is enqueued asynchronously on `stream`; the caller synchronises.
 *    No C++ exception crosses this interface.
 *  - Results are deterministic: equal inputs give bitwise-equal outputs.
 *  - NaN and Inf in the inputs propagate; they are not checked.
 */
#ifndef MUON_H
#define MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_ABI_VERSION 1

/* Status codes. */
typedef enum {
  MUON_OK = 0,
  MUON_E_INVALID = 1,   /* NULL where a pointer is required, bad config value */
  MUON_E_DTYPE = 2,     /* unknown dtype */
  MUON_E_SHAPE = 3,     /* negative or too large sizes, ld < cols */
  MUON_E_ALIGN = 4,     /* pointer not aligned to its element size */
  MUON_E_WORKSPACE = 5, /* workspace NULL or smaller than muon_workspace_bytes */
  MUON_E_DEVICE = 6,    /* no usable gfx950 device / HIP runtime error */
  MUON_E_LAUNCH = 7,    /* a kernel launch failed */
  MUON_E_ALLOC = 8      /* host or device allocation for a plan failed */
} muon_status;

/* Element type of grad, momentum and out (one type per call). */
typedef enum { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype;

/* Limits checked by validation (MUON_E_SHAPE beyond them). */
#define MUON_MAX_DIM 65536           /* rows and cols each */
#define MUON_MAX_ELEMS 1073741824LL  /* rows * cols per matrix (2^30) */
#define MUON_MAX_MATRICES 65536      /* matrices per call */
#define MUON_MAX_STEPS 64            /* Newton-Schulz steps */

/* One matrix of the set. Row-major: element (i, j) of grad, momentum and out
 * is at base + i * ld + j (elements of the set's dtype). rows == 0 or
 * cols == 0 is an empty matrix and is skipped. `grad` is read only;
 * `momentum` is read and overwritten with buf' (it may be NULL iff the
 * config's momentum is 0, and must then not be used); `out` is written with
 * the orthogonalised update. `out` may alias `grad` (same ld); it must not
 * overlap `momentum` or any other matrix's buffers. All three pointers must
 * be aligned to the element size; 16-byte alignment with ld and cols
 * multiples of 16 bytes selects the vectorised elementwise path. */
typedef struct {
  int64_t rows;
  int64_t cols;
  int64_t ld;
  const void* grad;
  void* momentum;
  void* out;
} muon_matrix;

/* Operand format of the matrix products (see the top of this file). */
typedef enum { MUON_PRECISION_DEFAULT = 0, MUON_PRECISION_BF16_OPERANDS = 1 } muon_precision;

/* Per-call scalars. (a, b, c) are the odd polynomial's coefficients
 * p(x) = a x + b x^3 + c x^5 (e.g. the quintic (3.4445, -4.7750, 2.0315) or
 * the cubic (1.5, -0.5, 0)); steps in [0, MUON_MAX_STEPS] (0 returns X0);
 * momentum mu in [0, 1) (0: no momentum state, u = G); nesterov 0 or 1;
 * eps >= 0 is added to ||u||_F (1e-7 is the usual value); precision is a
 * muon_precision value (ignored for fp32 sets). All must be finite. With
 * fp16 operands the iterates must stay below 65504 in magnitude, which
 * holds for polynomials that keep [0, 1] inside [-2, 2] over the steps
 * (all Newton-Schulz coefficient sets in use do). */
typedef struct {
  float a, b, c;
  int32_t steps;
  float momentum;
  int32_t nesterov;
  float eps;
  int32_t precision;
} muon_config;

/* Opaque plan: validated shapes, per-matrix workspace layout and the tile
 * schedules of every kernel, uploaded once to device memory. */
typedef struct muon_plan_s muon_plan;

/* ABI version of the loaded library (MUON_ABI_VERSION). */
int32_t muon_abi_version(void);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* muon_status_str(int32_t status);

/* Bytes of device workspace a call on this matrix set needs (host only, no
 * device calls). *bytes receives the size (0 for an all-empty set). */
muon_status muon_workspace_bytes(const muon_matrix* mats, int32_t n, muon_dtype dtype,
                                 size_t* bytes);

/* Builds a plan for `mats` (copied; pointers included) and uploads its
 * tables to the current device. Allocates a few KB to a few MB of device
 * memory owned by the plan; *plan receives NULL on error. */
muon_status muon_plan_create(const muon_matrix* mats, int32_t n, muon_dtype dtype,
                             muon_plan** plan);

/* Enqueues one Muon update of every matrix of the plan on `stream`.
 * `workspace` must hold at least muon_workspace_bytes bytes, 256-byte
 * aligned, and must not be used by anything else until the work ends.
 * Calls on the same workspace must be ordered (same stream). */
muon_status muon_plan_step(muon_plan* plan, const muon_config* cfg, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Frees a plan after waiting for the device (NULL is a no-op). */
void muon_plan_destroy(muon_plan* plan);

/* One Muon update of `mats` without an explicit plan: looks up (or builds
 * and caches, keyed by the full descriptor array including pointers) a plan
 * and calls muon_plan_step. A cache miss allocates and synchronises once;
 * training loops with stable buffers hit the cache on every later call. */
muon_status muon_step(const muon_matrix* mats, int32_t n, muon_dtype dtype,
                      const muon_config* cfg, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Orthogonalisation only: u = grad (momentum pointers ignored, cfg->momentum
 * and cfg->nesterov ignored), then normalisation and the iteration. */
muon_status muon_orthogonalize(const muon_matrix* mats, int32_t n, muon_dtype dtype,
                               const muon_config* cfg, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ---- weight application fused into the last update ---------------------
 *
 * The step after the orthogonalised update: the weight matrix W of each
 * parameter moves against it with decoupled weight decay,
 *
 *   W <- W * (1 - lr' * wd') - lr' * X,   lr' = lr * lr_mul,  wd' = wd * wd_mul
 *
 * where X is the Muon result (what muon_plan_step writes to `out`), lr and wd
 * are per call and lr_mul, wd_mul per matrix (mhpq.cn, modded-nanogpt
 * track_1_short technical guide, section 6.2, training hyper-parameters:
 * every parameter group carries its own lr and weight-decay multipliers;
 * yongjin360.com, Modded-NanoGPT green-AI article, hyper-parameter
 * paragraph: weight decay is part of the recipe). The pages give no
 * learning-rate schedule or shape rule, so all four scalars come from the
 * caller; the multipliers scale the learning rate and the decay wherever
 * they appear (decoupled decay, proportional to the effective rate). The product runs in fp32 on X before any rounding to the set's
 * dtype (the 16-bit path stages X as fp16 first), and W' is stored at the
 * set's dtype, round to nearest even. */

/* W of matrix i of a plan: same rows, cols and dtype as its grad,
 * row-major with leading dimension ld >= cols, aligned to the element size.
 * W must not overlap any grad, momentum, out or other W of the set. */
typedef struct {
  void* weight;
  int64_t ld;
  float lr_mul;
  float wd_mul;
} muon_weight;

/* Per-call scalars of a weight application; both finite. */
typedef struct {
  float lr;
  float wd;
} muon_apply;

/* Attaches the weights to a plan: w[i] for matrix i, n must equal the
 * plan's matrix count (records of empty matrices are ignored, their weight
 * may be NULL). Waits for the device, then updates the plan's device table
 * (do not call while work of this plan is in flight on another thread).
 * On error the plan keeps its previous weights. */
muon_status muon_plan_set_weights(muon_plan* plan, const muon_weight* w, int32_t n);

/* muon_plan_step, except that the last update writes W' (above) into each
 * matrix's weight instead of writing `out` (which is left untouched); with
 * cfg->steps == 0 the normalised X0 is applied. MUON_E_INVALID if the plan
 * has no weights. Momentum buffers are updated as in muon_plan_step. */
muon_status muon_plan_step_apply(muon_plan* plan, const muon_config* cfg, const muon_apply* ap,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* ---- introspection (tests, benchmarks, profiling) ---------------------- */

/* Kernels of one step, in launch order: momentum, normalise, then per
 * Newton-Schulz step gram, poly, update. */
typedef enum {
  MUON_K_MOMENTUM = 0, /* buf' and per-block sums of u^2            (HBM)  */
  MUON_K_NORMALIZE = 1,/* X0 = u/(||u||+eps), fp32 master + operand (HBM)  */
  MUON_K_GRAM = 2,     /* A = X X^T, upper-triangle tiles mirrored (MFMA) */
  MUON_K_POLY = 3,     /* B = b A + c A A, upper tiles mirrored    (MFMA) */
  MUON_K_UPDATE = 4,   /* X = a X + B X (last step writes out)     (MFMA) */
  MUON_K_COUNT = 5
} muon_kernel_kind;

/* Host-only schedule query: the work items kernel `kind` runs for `mats`
 * (for a plan split into groups, the groups' schedules one after the other,
 * each a multiple of 8 items), four int32 per item {matrix, a, b, c}
 * (momentum: {matrix, first row,
 * row count, partial slot}; normalise: {matrix, tile row, tile col, 0} of
 * 64 x 64 tiles of the rows<=cols orientation; gram/poly: {matrix, tile
 * row, tile col, 0} of the tiles on or above the diagonal; update: {matrix,
 * tile row, tile col, 0}; matrix-core tiles are 256 x 256 for bf16 sets and
 * 128 x 128 for fp32 sets), in launch order with empty slots as
 * {-1,-1,-1,-1}. Small bf16 sets whose longest Gram tiles would set the
 * Gram launch's time split those tiles' k range into S parts: such a tile
 * has S gram items with c = pbase << 16 | s << 8 | S (s = 0 .. S-1), each
 * writing an fp32 partial tile to the workspace, and kind == MUON_K_COUNT
 * queries the second Gram pass that sums them, four items {matrix, tile
 * row, tile col, pbase << 16 | q << 8 | S} per split tile, one per 128 x 128
 * quarter q (empty when nothing splits).
 * Writes min(cap, count) items to `items` (may be NULL when cap == 0) and
 * the total to *count. No device calls. */
muon_status muon_schedule_query(const muon_matrix* mats, int32_t n, muon_dtype dtype,
                                int32_t kind, int32_t* items, int64_t cap, int64_t* count);

/* Per-kernel timing. A plan may split a large set into groups of matrices
 * whose kernels run concurrently on streams of the plan (joined back to the
 * caller's stream before muon_plan_step's work ends). While timing is on,
 * every muon_plan_step instead runs each kernel over the whole set in one
 * launch on the step's stream, with HIP events recorded around each
 * launch; the results are bitwise the same. muon_plan_kernel_times (which
 * waits for the recorded events) accumulates elapsed milliseconds and
 * launch counts per muon_kernel_kind into ms[MUON_K_COUNT] and
 * launches[MUON_K_COUNT], summed over the steps since timing was enabled
 * or last read (reading resets). Off by default. */
muon_status muon_plan_set_timing(muon_plan* plan, int32_t enable);
muon_status muon_plan_kernel_times(muon_plan* plan, double* ms, int64_t* launches);

/* Workspace layout of matrix `idx` of a plan (byte offsets from the
 * workspace base; -1 where a buffer does not exist). All buffers use the
 * rows<=cols orientation, zero-padded to mp x np (X) or mp x mp (A, B),
 * with mp and np the tile multiples (256 for bf16 sets, 128 for fp32
 * sets). bf16 sets: x_op0/x_op1 hold the high part of X (the 16-bit
 * matrix-core operand, ping-pong between steps) and x_lo the low part.
 * fp16 operands: one signed byte q per element, X = hi + q * 2^(e - 33)
 * with e = max(E, 1) and E the 5-bit exponent field of hi, stored in the
 * update kernel's accumulator order (per 256 x 256 tile, 32-row blocks of
 * 8 KB). bf16 operands: a bf16 lo, X = hi + lo, row-major. gram (A) and
 * poly are 16-bit. The three 16-bit operands (x_op0/x_op1, gram, poly) are
 * stored in 32-column panels: element (r, c) is at element index
 * ((c / 32) * mp + r) * 32 + c % 32. With fp16 operands poly holds a I + B
 * (the a X term of the high part rides in the product). fp32 sets: x_op0/x_op1 are fp32 X
 * (ping-pong), gram/poly (B) fp32, all row-major, x_lo = -1. After a step
 * of k iterations X is in x_op[k % 2]. */
typedef struct {
  int64_t m, n, mp, np;
  int64_t x_lo, x_op0, x_op1, gram, poly;
} muon_buffer_info;

muon_status muon_plan_buffer_info(const muon_plan* plan, int32_t idx, muon_buffer_info* info);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H */
