/*
 * matrix_roots.h -- C ABI of the MI355X (gfx950) EMA-Gram quarter-power
 * preconditioner step.
 *
 * The step, per linear weight with gradient G (m x n), is the one described
 * on marin.community, "Sharding EMA-Gram eigensolves", section "Background":
 * keep exponential moving averages of G*G^T (left Gram, m x m) and of G^T*G
 * (right Gram, n x n), rescale them, take the inverse quarter power of each
 * rescaled Gram with a small regulariser added to its eigenvalues, and use the
 * two quarter powers to shape the update direction U = L^(-1/4) * G * R^(-1/4)
 * (the two-sided Shampoo form of tilderesearch, "Online KL Shampoo",
 * section 1).  Each Gram's root needs only that Gram (same page, section
 * "Approach"), so all calls are batched over independent problems.
 *
 * Conventions for every entry point:
 *  - Matrix pointers are DEVICE pointers, row-major, element (i, j) at
 *    ptr[i * ld + j]; ld >= number of columns.  Problem arrays (the structs)
 *    are HOST memory, read only during the call.
 *  - The caller owns every device buffer, including the workspace.  The
 *    library keeps no pointer after returning and allocates nothing on the
 *    device.  All work is enqueued on `hip_stream` (a hipStream_t passed as
 *    void*; NULL = the null stream); nothing is waited for, except where an
 *    entry point says so.  The enqueued work is kernel launches only (no
 *    copies or memsets; events only while mr_trace_enable is on), so a
 *    sequence of calls can be captured in a HIP graph and replayed on the
 *    same buffers.
 *  - Validation is all-or-nothing and happens before anything is enqueued:
 *    on an error status nothing was enqueued and mr_last_error_message()
 *    (thread-local) says what was wrong.
 *  - Numerical outcomes are never return codes: they go to per-matrix
 *    mr_root_info records in device memory that the caller reads after its
 *    own synchronisation.
 *  - Calls that share a workspace must be ordered on one stream.
 *  - Within one call, no matrix the call writes may overlap another matrix it
 *    writes or one it reads, in the same problem or in another problem of the
 *    batch (matrices it only reads may share memory); each matrix counts as
 *    the bytes from its first element to its last.  Violations return
 *    MR_ERR_ALIAS before anything is enqueued.
 */
#ifndef MATRIX_ROOTS_H
#define MATRIX_ROOTS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MR_ABI_VERSION 3

typedef int32_t mr_status;
#define MR_OK 0
#define MR_ERR_NULL 1        /* a required pointer is NULL                      */
#define MR_ERR_SHAPE 2       /* a size is <= 0, too large, or sizes disagree    */
#define MR_ERR_STRIDE 3      /* a leading dimension is smaller than the columns */
#define MR_ERR_PARAM 4       /* a scalar parameter or enum is out of range      */
#define MR_ERR_WORKSPACE 5   /* workspace NULL, too small or misaligned         */
#define MR_ERR_HIP 6         /* the HIP runtime reported an error               */
#define MR_ERR_UNSUPPORTED 7 /* valid request the library does not implement    */
#define MR_ERR_ALIAS 8       /* an output overlaps another output or an input   */

typedef int32_t mr_dtype;
#define MR_F32 0
#define MR_F64 1
/* Storage flag OR'ed into a state or input dtype (MR_F64 | MR_PACKED):
 * a symmetric d x d matrix kept as its upper triangle packed by rows,
 * element (i, j) with i <= j at offset i*d - i*(i-1)/2 + (j - i), d*(d+1)/2
 * elements in one contiguous array (the same bytes as LAPACK's lower-packed
 * column-major layout of the matrix).  Leading dimensions of packed
 * matrices are ignored.  Half the memory of full storage, and the Gram EMA
 * then reads and writes each stored element once. */
#define MR_PACKED 16

/* gram_ema_update: which Grams to update (bit mask) */
#define MR_LEFT 1
#define MR_RIGHT 2

/* inv_quarter_root_batched: rescale mode */
#define MR_NORM_NONE 0  /* s = 1                                  */
#define MR_NORM_TRACE 1 /* s = trace(A): the rescaled Gram has trace 1 */

/* inv_quarter_root_batched: method */
#define MR_AUTO 0   /* Jacobi for d <= 32, coupled Newton above              */
#define MR_JACOBI 1 /* eigendecomposition in LDS (d <= 128 only)             */
#define MR_NEWTON 2 /* GEMM-only coupled Newton inverse 4th root             */
#define MR_NEWTON_F64 3 /* the same iteration with every step in float64       */
#define MR_NEWTON_F32 4 /* float64 steps, then float32 matrix cores            */

/* mr_root_info.flags */
#define MR_INFO_NONFINITE 1     /* A held NaN or Inf; X is all NaN                          */
#define MR_INFO_ZERO_TRACE 2    /* trace(A) == 0 under MR_NORM_TRACE; X = eps^(-1/4) * I    */
#define MR_INFO_NOT_PD 4        /* Jacobi: an eigenvalue + eps <= 0; Newton: no usable bound;
                                   X is all NaN                                              */
#define MR_INFO_NOT_CONVERGED 8 /* Jacobi: still rotating after the sweep cap (default 30,
                                   mr_set_jacobi_max_sweeps); Newton: residual above
                                   r * sqrt(d), r = 2e-3 after a plain last step, 0.0243
                                   (0.135) after a degree-2 (degree-4) finish (e.g. A + eps I
                                   not positive definite), or, under MR_NORM_NONE, a floor
                                   eps/c below 1e-16                                         */

/* One weight for gram_ema_update.  G: m x n float32 (ldg >= n).
 * L: m x m, R: n x n, both of the call's state dtype (ldl >= m, ldr >= n),
 * full symmetric storage (or packed with MR_PACKED), updated in place.  L (R) may be NULL when the
 * MR_LEFT (MR_RIGHT) bit is not requested. */
typedef struct {
  int64_t m, n;
  const float* G;
  int64_t ldg;
  void* L;
  int64_t ldl;
  void* R;
  int64_t ldr;
} mr_gram_problem;

/* One matrix for inv_quarter_root_batched / inv_sqrt_root_batched.  A: d x d
 * of the call's a_dtype (symmetric; its symmetric part (A + A^T)/2 is what is
 * used), lda >= d; or packed (a_dtype | MR_PACKED, lda ignored).
 * X: d x d float32 output, ldx >= d; X must not overlap A. */
typedef struct {
  int64_t d;
  const void* A;
  int64_t lda;
  float* X;
  int64_t ldx;
} mr_root_problem;

/* Per-matrix outcome of inv_quarter_root_batched (device memory, written by
 * the call).  40 bytes. */
typedef struct {
  double scale;       /* s: trace(A) (MR_NORM_TRACE) or 1                        */
  double bound;       /* c >= lambda_max(A/s + eps I) (Newton); 0 for Jacobi      */
  int32_t iters;      /* Newton iterations run, or Jacobi sweeps                  */
  int32_t fp64_iters; /* of those Newton iterations, the ones with float64-accurate
                         products                                                */
  float residual;     /* Newton: ||M_{K-1} - I||_F, the iterate the last X update
                         used; Jacobi: off-diagonal Frobenius norm of the
                         rotated A/s at exit                                      */
  uint32_t flags;     /* MR_INFO_* bits                                           */
  int32_t final_degree; /* Newton: degree in M of the last X update (1, 2 or 4,
                           see MR_NEWTON); 0 for Jacobi and the other calls      */
  int32_t reserved;   /* 0                                                        */
} mr_root_info;

/* One weight for precondition_apply.  XL: m x m, G: m x n, XR: n x n, U: m x n,
 * all float32.  U must not overlap XL, G or XR. */
typedef struct {
  int64_t m, n;
  const float* XL;
  int64_t ldxl;
  const float* G;
  int64_t ldg;
  const float* XR;
  int64_t ldxr;
  float* U;
  int64_t ldu;
} mr_apply_problem;

/*
 * gram_ema_update -- for every problem, in place:
 *     L <- beta * L + (1 - beta) * G * G^T   (if sides & MR_LEFT)
 *     R <- beta * R + (1 - beta) * G^T * G   (if sides & MR_RIGHT)
 * The EMA of gradient products of the EMA-Gram page, section "Background";
 * the weighting convention (beta on the old state, no bias correction) is the
 * plain reading of that passage.  Products of float32 entries are formed and
 * summed in float64 on the float64 matrix cores, whatever the state dtype;
 * a float32 state receives the float64 result rounded once.
 * state_dtype: MR_F32 or MR_F64.  beta in [0, 1) (double, so that 1 - beta
 * carries no float32 rounding into a float64 state).  count >= 1 (0 is a no-op).
 * G must not overlap L or R.
 * Workspace: none needed (ws may be NULL, ws_bytes 0).
 */
mr_status gram_ema_update(const mr_gram_problem* problems, int32_t count, mr_dtype state_dtype,
                          double beta, uint32_t sides, void* ws, size_t ws_bytes, void* hip_stream);
size_t gram_ema_update_workspace(const mr_gram_problem* problems, int32_t count,
                                 mr_dtype state_dtype, uint32_t sides);

/*
 * inv_quarter_root_batched -- for every problem:
 *     X = (A/s + eps * I)^(-1/4),  s = trace(A) (MR_NORM_TRACE) or 1 (MR_NORM_NONE)
 * The regularised inverse quarter power of the rescaled Gram (EMA-Gram page,
 * section "Background": rescale, add a small regulariser to the eigenvalues,
 * raise them to -1/4, rebuild).  X is symmetric to the last bit.
 * Methods:
 *  - MR_JACOBI (d <= 128): cyclic Jacobi eigendecomposition of A/s in float64,
 *    one workgroup per matrix with A held in LDS (and V too for d <= 96),
 *    one launch per size class for any number of matrices;
 *    f = (lambda + eps)^(-1/4); X = V f V^T.
 *  - MR_NEWTON: coupled Newton iteration for the inverse 4th root,
 *        M0 = (A/s + eps I)/c, X0 = I, T = (5 I - M)/4, X <- X T, M <- T^4 M,
 *    X = c^(-1/4) X_K, with M scaled by 1/s_t before each step (per-step
 *    scales from the spectrum bounds, see mr_newton_schedule), with
 *    float64-accurate products of M and its powers while the smallest
 *    eigenvalue of M is below 5e-4, then with float32 storage on the fp16
 *    matrix cores with split operands (x = hi + 2^-11 lo, three products per
 *    product, float32 accumulation: about 2^-22 relative error per product).
 *    X is kept in that split storage from the first step.  For d >= 1024 the
 *    float64-accurate products run on the int8 matrix cores: each operand as
 *    six int8 digit planes (7 bits each, one power-of-two exponent per row of
 *    M, fixed ones for M's powers), 21 exact plane products with int32
 *    accumulation, summed in float64 (about 2^-40 relative to each row's
 *    largest entry); smaller Grams run them on the float64 matrix cores.
 *    The GEMM-only
 *    route of tilderesearch, "Online KL Shampoo", sections 2.1-2.2 (there
 *    for the -1/2 root), taken to the 4th root.  c = 1.01 times an upper
 *    bound on lambda_max(A/s + eps I): the Wolkowicz-Styan bound (the OKLS
 *    page, appendix D, normalises by an O(d^2) upper bound in the same way),
 *    or for d >= 256, where smaller, the fourth- or eighth-moment bound
 *    |B^2|_F^(1/2) or |B^4|_F^(1/4) of B = A/s + eps I from two fp16
 *    products (their fp16 and float32 rounding added, so they stay upper
 *    bounds); the iteration count follows from eps/c.  The last iteration updates X only:
 *    with the step's polynomial, or, once the spectrum of M lies within
 *    0.0162 (0.0898) of 1, with the degree-2 (degree-4) Taylor polynomial of
 *    M^(-1/4) about I, which ends the iteration a step or two earlier with a
 *    truncation error below 5e-7.
 *  - MR_NEWTON_F32: as MR_NEWTON with the float32 steps on the float32
 *    matrix cores, its float64 steps (X included) on the float64 ones.
 *  - MR_NEWTON_F64: the Newton iteration with every step on the float64
 *    matrix cores (for inputs near the float32 limit).
 *  - MR_AUTO: Jacobi for d <= 32, Newton otherwise (Jacobi's sweeps are a
 *    chain of d - 1 dependent rounds each: on MI355X it is the faster route
 *    up to d = 24 for a few matrices and up to d = 40 for hundreds, and its
 *    roots are accurate to float64 rounding).
 * a_dtype: MR_F32 or MR_F64.  eps > 0 and finite.  info_dev: device array of
 * `count` records (may be NULL).  Never synchronises: the host launches a
 * fixed number of Newton steps and each matrix runs its own schedule under
 * it.  With MR_NORM_TRACE that number covers every matrix (c <= 1.01 (1 +
 * eps)); with MR_NORM_NONE it covers floors eps/c down to 1e-16, and a
 * matrix whose floor lies lower runs the schedule of the floor 1e-16 and is
 * flagged MR_INFO_NOT_CONVERGED (float64 rounding of M0 is already of the
 * floor's size there; eigenvalues of A/c + eps/c above 1e-16 still
 * converge).
 * Workspace: at least inv_quarter_root_batched_workspace(...) bytes, 256-byte
 * aligned; its contents on entry are ignored.  Per Newton matrix it holds
 * 40 d^2 bytes (rounded up to 256), plus, for MR_NEWTON and MR_AUTO from
 * d = 1024, M's row exponents (4 dp bytes, dp = d rounded up to 128) and
 * whatever of the 18 dp x dp digit planes does not fit in the parts of the
 * 40 d^2 bytes a float64 step leaves idle (none for d a multiple of 128,
 * all of them for d not a multiple of 4).
 */
mr_status inv_quarter_root_batched(const mr_root_problem* problems, int32_t count,
                                   mr_dtype a_dtype, double eps, int32_t normalize, int32_t method,
                                   mr_root_info* info_dev, void* ws, size_t ws_bytes,
                                   void* hip_stream);
size_t inv_quarter_root_batched_workspace(const mr_root_problem* problems, int32_t count,
                                          mr_dtype a_dtype, int32_t method);

/*
 * inv_quarter_root_batched_noalloc -- inv_quarter_root_batched without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same problems, arguments, results and info records; the
 * workspace is a file-scope device array of MR_NOALLOC_SCRATCH_BYTES bytes
 * that each GPU the library runs on holds until the process ends.  The call
 * allocates nothing.  Its device address is looked up on the first call on
 * each device (the current device; hip_stream must belong to it).  A batch
 * whose workspace (inv_quarter_root_batched_workspace) exceeds that size is
 * rejected with MR_ERR_WORKSPACE before anything is enqueued: 32 MiB holds
 * for instance 16 Newton roots of 224 x 224, 256 MR_JACOBI roots of
 * 64 x 64, or one Newton root of 896 x 896.  The array's contents on entry
 * are ignored (nothing in it must start at zero), but every call on one GPU
 * uses the same array: calls that overlap on one GPU (other streams, other
 * host threads) race and give wrong results; order them on one stream.
 */
#define MR_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
mr_status inv_quarter_root_batched_noalloc(const mr_root_problem* problems, int32_t count,
                                           mr_dtype a_dtype, double eps, int32_t normalize,
                                           int32_t method, mr_root_info* info_dev, void* hip_stream);

/* inv_sqrt_root_batched: precision of the products */
#define MR_CANS_F16 0   /* fp16 products with float32 accumulation (the OKLS page's) */
#define MR_CANS_SPLIT 1 /* split-fp16 products: float32-accurate, three times the
                           matrix-core work                                        */

/*
 * inv_sqrt_root_batched -- for every problem:
 *     W = S^(-1/2),  S = (A + A^T)/2 / s + eps * I,
 *     s = trace(A) (MR_NORM_TRACE) or 1 (MR_NORM_NONE)
 * The inverse square root of a symmetric positive definite matrix by the
 * scaled CANS coupled Newton-Schulz iteration of tilderesearch, "Online KL
 * Shampoo", sections 2.3-2.4 and appendix D: L = 1.01 times the
 * Wolkowicz-Styan bound on lambda_max(S); from Y0 = S/L, Z0 = I, ten steps
 *     P = Z Y,  Q = a_k I + b_k P,  Y <- Y Q,  Z <- Q Z
 * with the page's ten CANS coefficient pairs; W = Z_10 / sqrt(L).  Every
 * intermediate is stored in fp16 (plus a second fp16 half holding its
 * float32 rounding remainder) times a power of two fixed per step by the
 * scalar recurrence, so that no entry exceeds 2^14 (the page's per-step
 * range scaling).  P is a full product; Y Q = Y Z Y and Q Z = Z Y Z are
 * computed as symmetric (upper-triangle) products.  27 products in 19
 * launches for the whole batch; no host synchronisation.
 * Accuracy: the composed CANS map reaches (lambda/L)^(-1/2) to 3e-5 for
 * lambda/L in [1e-6, 1] and fails far below; with MR_CANS_F16 the fp16
 * rounding of the operands limits the relative error to a few 1e-3 for
 * condition numbers up to 1e3 (fp16-grade, as on the page); the first step,
 * whose coefficients cancel to about y/18 for eigenvalues near L, runs on
 * split operands in both precisions; MR_CANS_SPLIT reaches about 1e-4 up to
 * 1e4.  W is symmetric to the last bit.
 * a_dtype: MR_F32 or MR_F64.  eps >= 0 and finite.  precision: MR_CANS_F16
 * or MR_CANS_SPLIT.  info_dev: device array of `count` records (may be
 * NULL): scale = s, bound = L, iters = 10, fp64_iters = 0, residual =
 * ||P_9 - I||_F (the last coupled product, which the final step maps to I);
 * flags: NONFINITE (W all NaN), ZERO_TRACE (W = eps^(-1/2) I; with eps = 0
 * also NOT_PD and W all NaN), NOT_PD (no positive bound: W all NaN),
 * NOT_CONVERGED (residual above 0.1 * sqrt(d): S not positive definite, or
 * eigenvalues below the map's reach).
 * Workspace: at least inv_sqrt_root_batched_workspace(...) bytes (24 d^2
 * bytes per matrix plus per-matrix state), 256-byte aligned; contents on
 * entry ignored.  Errors as for inv_quarter_root_batched; nothing is
 * enqueued on a validation failure.
 */
mr_status inv_sqrt_root_batched(const mr_root_problem* problems, int32_t count, mr_dtype a_dtype,
                                double eps, int32_t normalize, int32_t precision,
                                mr_root_info* info_dev, void* ws, size_t ws_bytes, void* hip_stream);
size_t inv_sqrt_root_batched_workspace(const mr_root_problem* problems, int32_t count,
                                       mr_dtype a_dtype, int32_t precision);

/* One matrix for polar_cans_batched.  G: m x n float32 (ldg >= n); O: m x n
 * float32 output (ldo >= n), must not overlap G. */
typedef struct {
  int64_t m, n;
  const float* G;
  int64_t ldg;
  float* O;
  int64_t ldo;
} mr_polar_problem;

/*
 * polar_cans_batched -- for every problem, the orthogonalised matrix of the
 * ten CANS polar steps
 *     X0 = G / sqrt(L),  L = 1.01 ||G||_F^2,  X <- a_k X + b_k X X^T X,  O = X_10
 * with the OKLS page's ten CANS coefficient pairs (tilderesearch, "Online KL
 * Shampoo", section 2.3: the coefficients were designed for Muon's polar
 * factor).  Each step maps every singular value s to s (a_k + b_k s^2) and
 * keeps the singular vectors, so O = U phi(Sigma / sqrt(L)) V^T for
 * G = U Sigma V^T; phi is within 3e-5 of 1 for sigma^2 / L in [1e-6, 0.99],
 * where O is the polar factor U V^T.  The iteration runs on the tall
 * orientation (G^T for m < n): per step the Gram A = X^T X (symmetric,
 * upper-triangle product) and X' = a X + b X A (full product), 20 launches
 * for the whole batch, intermediates stored as fp16 plus an fp16 rounding
 * remainder, times powers of two from the singular-value recurrence (no
 * entry above 2^14).  precision: MR_CANS_F16 (fp16 products, float32
 * accumulation; relative error about 3e-3) or MR_CANS_SPLIT (float32-accurate
 * products; about 1e-6).
 * info_dev: device array of `count` records (may be NULL): scale = ||G||_F^2,
 * bound = L, iters = 10, fp64_iters = 0, residual = ||A_9 - I||_F (the last
 * Gram; not small for rank-deficient G, so never a flag); flags: NONFINITE
 * (O all NaN), ZERO_TRACE (G = 0: O = 0).
 * Workspace: at least polar_cans_batched_workspace(...) bytes (4 (3 M N + N^2)
 * bytes per matrix, M = max(m, n), N = min(m, n), plus per-matrix state),
 * 256-byte aligned; contents on entry ignored.  Validation is all-or-nothing
 * before anything is enqueued; no host synchronisation.
 */
mr_status polar_cans_batched(const mr_polar_problem* problems, int32_t count, int32_t precision,
                             mr_root_info* info_dev, void* ws, size_t ws_bytes, void* hip_stream);
size_t polar_cans_batched_workspace(const mr_polar_problem* problems, int32_t count, int32_t precision);

/* One matrix for momentum_ema_batched: G (read) and M (updated in place),
 * both m x n float32, ldg, ldm >= n; M must not overlap G. */
typedef struct {
  int64_t m, n;
  const float* G;
  int64_t ldg;
  float* M;
  int64_t ldm;
} mr_momentum_problem;

/*
 * momentum_ema_batched -- for every problem, in place:
 *     M <- mu * M + (1 - mu) * G      (computed in float64, stored float32)
 * The momentum of each weight's gradient, whose preconditioned direction the
 * optimizer applies (EMA-Gram page, section "Results", compares update
 * directions at equal Grams and momentum; the MuonH notes of ai.thesatyajit.com,
 * "Marin 535B-A23B", section "A sphere for every matrix", take the momentum
 * first).  0 <= mu < 1.  One
 * HBM-bound pass (12 bytes per element; up to 48 matrices per launch).  No
 * workspace, no synchronisation.
 */
mr_status momentum_ema_batched(const mr_momentum_problem* problems, int32_t count, double mu,
                               void* hip_stream);

/* One matrix for hyperball_update_batched: W (updated in place) and U (read),
 * both m x n float32, ldw, ldu >= n; W must not overlap U. */
typedef struct {
  int64_t m, n;
  float* W;
  int64_t ldw;
  const float* U;
  int64_t ldu;
} mr_hyperball_problem;

/*
 * hyperball_update_batched -- for every problem, in place, the MuonH
 * norm-preserving step (ai.thesatyajit.com, "Marin 535B-A23B", section "A
 * sphere for every matrix"):
 *     c = lr ||W|| / max(||U||, 1e-10),  W' = W - c U,
 *     W <- W' ||W|| / max(||W'||, 1e-10)
 * (Frobenius norms of the whole matrix), so every W keeps its norm.  Two
 * HBM-bound passes: float64 partial sums of ||W||^2, ||U||^2 and <W, U>, then
 * ||W'||^2 = ||W||^2 - 2 c <W, U> + c^2 ||U||^2 and the in-place update
 * (20 bytes per element in all).  lr >= 0 and finite.  norms_dev: optional
 * device array of 3 doubles per problem, receiving ||W||, ||U||, ||W'||.
 * Workspace: at least hyperball_update_batched_workspace(...) bytes,
 * 256-byte aligned.  Deterministic (fixed summation order).
 */
mr_status hyperball_update_batched(const mr_hyperball_problem* problems, int32_t count, double lr,
                                   double* norms_dev, void* ws, size_t ws_bytes, void* hip_stream);
size_t hyperball_update_batched_workspace(const mr_hyperball_problem* problems, int32_t count);

/* Suprema over y0 in (0, 1] of the CANS scalar recurrence y <- y q, z <- z q,
 * q = a_k + b_k z y (y, z from y0, 1), at steps k = 0..10: the per-step
 * bounds inv_sqrt_root_batched scales its intermediates by (y: Y_k, z: Z_k,
 * p: P_k = Z_k Y_k).  Writes min(11, capacity) values to each non-NULL
 * array and returns 11.  Host-only. */
int32_t mr_cans_ceilings(double* y, double* z, double* p, int32_t capacity);

/*
 * precondition_apply -- for every problem:  U = alpha * XL * G * XR
 * The two-sided application of the quarter powers (EMA-Gram page, section
 * "Background"; Shampoo form of the OKLS page, section 1).  The two products
 * (W^T = XR^T G^T from a transposed split copy of XR, then U = alpha XL W;
 * any square XR, symmetric or not) run on the fp16 matrix cores with
 * float32-accurate split operands (x = hi + 2^-11 lo, three fp16 products per
 * product, float32 accumulation), each operand scaled by the power of two
 * that puts its largest magnitude in [2^14, 2^15) (exact, and undone after
 * the product): the workspace holds split copies of XR, G, XL and W^T, rows
 * padded with zeros to a multiple of 32 columns, W^T in float32 and the
 * operands' maxima, each array 256-byte aligned.  Results scale exactly with
 * power-of-two scalings of G, XL or XR.
 * Workspace: at least precondition_apply_workspace(...) bytes, 256-byte aligned.
 */
mr_status precondition_apply(const mr_apply_problem* problems, int32_t count, float alpha,
                             void* ws, size_t ws_bytes, void* hip_stream);
size_t precondition_apply_workspace(const mr_apply_problem* problems, int32_t count);

/* Iteration count of the coupled Newton p-th root iteration for a smallest
 * normalised eigenvalue m0 in (0, 1]: the number of steps of the scalar map
 * m <- m * ((p + 1 - m) / p)^p until 1 - m <= tol (the map every eigenvalue
 * of M follows).  p in {2, 4}.  Host-only; returns -1 on bad arguments. */
int32_t mr_newton_iterations(int32_t p, double m0, double tol);

/*
 * Kernel-class tracing: when enabled, every launch the library makes is
 * bracketed by a pair of HIP events recorded on the launch's own stream
 * (host-side bookkeeping only; events come from a pool created once).
 * mr_trace_collect waits for the traced launches, writes one record per
 * kernel class that ran (at most `capacity`), clears the log and returns the
 * number of records.  Not for concurrent use from several threads.
 */
typedef struct {
  char name[32];    /* kernel class, e.g. "newton_f32"             */
  int64_t launches; /* traced launches of this class               */
  double total_ms;  /* sum of event-measured launch durations      */
} mr_trace_record;
int32_t mr_trace_enable(int32_t on); /* returns the previous setting */
int32_t mr_trace_collect(mr_trace_record* out, int32_t capacity);

/* The step scales the library uses for a Newton root (MR_NEWTON) whose
 * spectrum bound is [m0, 1/1.01] (m0 = eps/c): writes min(K, capacity) scales
 * s_t, stores the count of float64 steps in *fp64_steps and the degree in M of
 * the last step's X update in *final_degree (1: the step's own (5 - M/s)/4;
 * 2 or 4: the Taylor polynomial of M^(-1/4) about I; either pointer may be
 * NULL) and returns K, the number of steps (-1 on bad arguments).  Host-only. */
int32_t mr_newton_schedule(double m0, double* scales, int32_t capacity, int32_t* fp64_steps,
                           int32_t* final_degree);

/*
 * Matrix-core peaks of the current device, for reporting rooflines (the
 * measurement the hot path's roofline figures are set against).
 * prop_tflops: multiProcessorCount x clockRate x dense MFMA flops per clock
 * per compute unit (gfx950: 256 float32, 128 float64, 4096 fp16, 8192 int8
 * operations).
 * measured_tflops: register-only MFMA loops (v_mfma_f32_32x32x2_f32,
 * v_mfma_f64_16x16x4_f64, v_mfma_f32_32x32x16_f16,
 * v_mfma_i32_32x32x32_i8), eight workgroups per CU, a few ms each, timed
 * with events on `hip_stream` after one warm-up launch, on fixed small
 * operands; measured_random_tflops: the same loops with per-lane random
 * operands (uniform in [-1, 1), int8 digits in [-64, 63]), which draw more
 * power and hold a lower clock, as real data do.  Index 0 float32,
 * 1 float64, 2 fp16, 3 int8 (TOP/s).  Synchronises the stream and
 * touches no device memory; MR_ERR_NULL for a NULL `out`, MR_ERR_HIP on a
 * runtime error (then `out` holds what was measured before it).
 */
typedef struct {
  int32_t cu_count;          /* hipDeviceProp_t::multiProcessorCount   */
  int32_t clock_khz;         /* hipDeviceProp_t::clockRate (peak, kHz) */
  double prop_tflops[4];            /* derived from CU count and clock   */
  double measured_tflops[4];        /* register-only MFMA loops         */
  double measured_random_tflops[4]; /* ... on random operands           */
} mr_peak_info;
mr_status mr_measure_peaks(mr_peak_info* out, void* hip_stream);

/* Process-wide cap on the sweeps of the Jacobi route (default 30; the
 * eigendecomposition converges in about 10 for float64 inputs).  A matrix
 * still rotating after the last allowed sweep is reconstructed from where it
 * stands and flagged MR_INFO_NOT_CONVERGED.  Takes effect for calls made
 * after it returns; returns the previous cap, or -1 (and changes nothing)
 * for a cap outside [1, 100].  Host-only. */
int32_t mr_set_jacobi_max_sweeps(int32_t sweeps);

const char* mr_status_string(mr_status status);
const char* mr_last_error_message(void);
int32_t mr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MATRIX_ROOTS_H */
