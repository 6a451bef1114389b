/*
 * pmx.h -- PRISM matrix functions for Shampoo/Muon-style preconditioners on
 * AMD Instinct MI355X (gfx950).  C ABI of libpmx.so.
 *
 * Sources of the operations (web pages; section names as printed there):
 *   [Shampoo blog]     "深度学习中的优化器之Shampoo算法原理与二阶优化机制"
 *                      (idocdown), sections 2.2, 2.3, 3.1, 6.3.
 *   [PRISM summary]    "PRISM：分布无关的自适应矩阵函数计算以加速神经网络训练"
 *                      (euno.news summary of arXiv 2601.22137), "方法论".
 *   [PRISM synthesis]  "Sintesi Tecnica: PRISM" (gist.science), Part I and
 *                      Part II ("Adaptive Polynomial Fitting",
 *                      "Randomized Sketching").
 *
 * Conventions shared by every entry point
 *   - Matrices are row-major.  "ld" is the distance in elements between
 *     consecutive rows and must be >= the number of columns.  Batched forms
 *     take a batch count and, per matrix argument, a batch stride in elements.
 *   - Every matrix, workspace and info pointer is a DEVICE pointer owned by
 *     the caller; the library never allocates, frees or retains device memory
 *     and keeps no pointer after a call returns.  Scalars are host values.
 *   - Every call validates its arguments on the host first.  On any error it
 *     returns a non-zero pmx_status and enqueues NOTHING.  On PMX_OK all work
 *     has been enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting for the device.
 *   - Numerical outcomes of the iterative functions (converged, stagnated,
 *     ...) are written asynchronously to the caller's device-resident
 *     pmx_matfn_info array (one element per matrix); the host never waits.
 *   - Input and output matrices of one call must not overlap, except that
 *     pmx_shampoo_stats_update updates L and R in place.  Overlap of
 *     distinct arguments is reported as PMX_ERR_ALIAS.
 *   - A handle serves one device; use one handle per host thread.  Calls on
 *     one stream are ordered; calls sharing a workspace must be ordered.
 */
#ifndef PMX_H
#define PMX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PMX_VERSION_MAJOR 0
#define PMX_VERSION_MINOR 1
#define PMX_OPTS_VERSION 4
#define PMX_METHOD_NEWTON_SCHULZ 0
#define PMX_METHOD_INVERSE_NEWTON 1
#define PMX_SCALE_FROBENIUS 0
#define PMX_SCALE_POWER 1
#define PMX_TRACE_LEN 64   /* alpha / residual trace entries kept per stage */
#define PMX_MAX_SKETCH 16  /* largest supported sketch width p */

/* Synchronous result of every call. */
typedef enum {
  PMX_OK = 0,
  PMX_ERR_INVALID_VALUE = 1, /* bad size, ld, pointer, option or exponent */
  PMX_ERR_NOT_SUPPORTED = 2, /* valid request this build does not implement */
  PMX_ERR_WORKSPACE = 3,     /* workspace NULL or smaller than the query says */
  PMX_ERR_ALIAS = 4,         /* an output overlaps an input or another output */
  PMX_ERR_HIP = 5            /* the HIP runtime reported an error */
} pmx_status;

/* Asynchronous numerical outcome, written to pmx_matfn_info.status. */
typedef enum {
  PMX_RUNNING = -1,  /* never left in a finished call's info */
  PMX_CONVERGED = 0, /* residual r_k <= tol */
  PMX_MAXITER = 1,   /* max_iter updates done without reaching tol */
  PMX_STAGNATED = 2, /* r_{k-1} < 1e-2 and r_k > 0.9 r_{k-1}: rounding floor */
  PMX_NONFINITE = 3, /* NaN/Inf in the input, the scale or the residual */
  PMX_DIVERGED = 4   /* r_k > 2: input not positive definite */
} pmx_numeric;

/* Element types.  The argument types pmx_dtype and pmx_op are plain 32-bit
 * integers (not enum types), so that any value a caller passes is a valid
 * value of the parameter and is rejected with PMX_ERR_INVALID_VALUE. */
typedef int32_t pmx_dtype;
enum { PMX_F32 = 0, PMX_BF16 = 1 };

/* Operation codes for pmx_workspace_size. */
typedef int32_t pmx_op;
enum {
  PMX_OP_STATS = 0,
  PMX_OP_INV_ROOT = 1,
  PMX_OP_POLAR = 2,
  PMX_OP_APPLY = 3,
  PMX_OP_POLAR_VARBATCH = 4  /* batch = number of blocks, all of sides <= PMX_VARBATCH_MAX_DIM;
                                m, n ignored */
};

/*
 * Options of the iterative matrix functions ([PRISM synthesis] Part I and
 * Part II).  pmx_matfn_opts_default fills the defaults given per field.
 */
typedef struct {
  int32_t struct_version; /* PMX_OPTS_VERSION (4); 3 (56-byte layout, ending at
                             method), 2 (48 bytes, ending at degree_max) and 1
                             (40 bytes, ending at seed) are accepted with the
                             later fields at their defaults */
  int32_t degree;         /* d in {1, 2, 3}: g(xi) = f_{d-1}(xi) + alpha xi^d; default 2;
                             d = 3 runs on the fp32 paths only (the bf16 polar
                             factor and fp64_iters > 0 return NOT_SUPPORTED) */
  int32_t sketch_p;       /* Gaussian sketch width p, 1..PMX_MAX_SKETCH; default 8 */
  int32_t max_iter;       /* updates per stage, 1..1000; default 30 */
  int32_t accelerate;     /* 1: fitted alpha (PRISM); 0: alpha = Taylor c_d; default 1 */
  float alpha_lo;         /* alpha interval; NaN selects the default:       */
  float alpha_hi;         /*   d = 1: [1/2, 1], d = 2: [3/8, 1.47],         */
                          /*   d = 3: [5/16, 2.46]                          */
  float tol;              /* stop when ||R_k||_F / sqrt(n) <= tol; default 1e-6 */
  uint64_t seed;          /* key of the Philox4x32-10 sketch stream; default 0 */
  int32_t fp64_iters;     /* inverse roots: the first fp64_iters updates of each
                             stage run in fp64 (0..max_iter), the rest in fp32;
                             for ill-conditioned inputs (kappa near 1e6) whose
                             fp32 result misses 1e-4.  Ignored by the polar
                             factor.  Default 0.  Added in struct_version 2. */
  int32_t degree_max;     /* adaptive degree ([PRISM summary], methodology step
                             3): 0 (default) or `degree` keeps d fixed; 3 with
                             degree = 2 starts every stage at d = 2 and uses
                             d = 3 for the rest of the stage after an update
                             whose sketched contraction
                             sqrt(phi_S(alpha_k)) / ||R_k S||_F exceeds
                             adapt_ratio.  Needs accelerate = 1 and
                             fp64_iters = 0; fp32 paths only (the bf16 polar
                             factor returns NOT_SUPPORTED).  Added in version 3
                             (it takes the place of version 2's zero `reserved`). */
  float adapt_ratio;      /* the contraction threshold above; default 0.3 */
  int32_t method;         /* inverse roots: PMX_METHOD_NEWTON_SCHULZ (0, default):
                             coupled Newton-Schulz square roots, chained for
                             p = 4; PMX_METHOD_INVERSE_NEWTON (1): the coupled
                             inverse Newton iteration X <- X g, M <- g^p M with
                             R = I - M and g = f_{d-1}(R) + alpha R^d, f the
                             Taylor polynomial of (1 - xi)^{-1/p} ([PRISM
                             synthesis], key contributions: inverse Newton
                             methods); alpha minimises a degree-2p sketched
                             objective over [1/4, 1/2] (d = 1) or [5/32, 0.60]
                             (d = 2) for p = 4, the square-root family's
                             intervals for p = 2.  d in {1, 2}, fp32 updates
                             only (fp64_iters = 0, no adaptive degree); X_aux =
                             A X^{p-1} is formed after the iteration.  Ignored
                             by the polar factor.  Added in version 3. */
  int32_t scale_mode;     /* the input scale c of Y_0 = A / c (inverse roots).
                             PMX_SCALE_FROBENIUS (0, default): c = ||A||_F, an
                             upper bound of the spectral norm.
                             PMX_SCALE_POWER (1): c = ||A||_F min(1, 2 mu),
                             mu = max_j ||K_8[:, j]|| / ||K_7[:, j]|| over the
                             p columns of K_t = (A / ||A||_F)^t V_0 (eight
                             skinny passes from a Gaussian block V_0 drawn as a
                             sketch of stage 2), a lower bound of
                             lambda_max / ||A||_F; so c stays within 2 lambda_max
                             of the top eigenvalue and never exceeds ||A||_F.
                             Flat spectra of large order (Shampoo statistics)
                             start much closer to convergence.  The fp32
                             polar factor with 1: X_0 = G / ||G||_F is divided
                             by s, s^2 = min(1, 2 mu) from the same passes on
                             X_0^T X_0 = I - R_0, R_0 is rewritten for X_0 / s
                             and 1 / s is folded into the first g.  The bf16
                             polar factor and the variable-size one return
                             NOT_SUPPORTED for 1 (bf16 rounding of X, amplified
                             while the top singular values overshoot under the
                             largest alpha, made the iteration diverge).
                             Order-64 calls with 1 leave the fused kernel.  The
                             pages leave the scaling open.  Added in version 4. */
  int32_t reserved;       /* 0 */
} pmx_matfn_opts;

/*
 * Per-matrix outcome, device resident, written by the library.
 * residual[s] / rtrace[s][k] hold r_k = ||R_k||_F / sqrt(n) of stage s
 * (stage 1 only for the chained inverse 4th root), alpha[s][k] the fitted
 * coefficient of update k (first PMX_TRACE_LEN entries; unused entries 0).
 */
typedef struct {
  int32_t status;          /* pmx_numeric of the whole call (worst stage) */
  int32_t iters[2];        /* updates per stage */
  int32_t gemms;           /* dense products (n x n x n, or the polar shapes) */
  int32_t sketch_products; /* skinny n x n x p products of the alpha fit */
  int32_t stages;          /* stages run */
  float scale;             /* c = ||A||_F (or ||G||_F) used to scale the input */
  float residual[2];       /* final r per stage */
  float alpha[2][PMX_TRACE_LEN];
  float rtrace[2][PMX_TRACE_LEN];
} pmx_matfn_info;

typedef struct pmx_context* pmx_handle;

/* Create a handle bound to HIP device `device` (loads nothing else; no
 * device memory is allocated).  Returns PMX_ERR_INVALID_VALUE for a NULL
 * out-pointer or a device index out of range, PMX_ERR_NOT_SUPPORTED for a
 * device that is not gfx950. */
pmx_status pmx_create(pmx_handle* handle, int device);
pmx_status pmx_destroy(pmx_handle handle);
const char* pmx_status_string(pmx_status status);
/* Library version as major * 1000 + minor. */
int pmx_version(void);

/* Fill `opts` with the defaults listed in pmx_matfn_opts. */
pmx_status pmx_matfn_opts_default(pmx_matfn_opts* opts);

/*
 * Workspace bytes a call needs.  m, n are the shapes as passed to the call
 * (for PMX_OP_INV_ROOT m is ignored; for PMX_OP_STATS and PMX_OP_APPLY the
 * gradient is m x n).  `opts` may be NULL for the operations without options.
 * The workspace must be 256-byte aligned.  `handle` may be NULL (the sizes
 * do not depend on the device), so sizes can be queried without a GPU.
 */
pmx_status pmx_workspace_size(pmx_handle handle, pmx_op op, int m, int n, int batch,
                              pmx_dtype dtype, const pmx_matfn_opts* opts, size_t* bytes);

/*
 * Shampoo statistics update ([Shampoo blog] sections 2.2 and 2.3, step 2):
 *   L <- beta L + (1 - beta) G G^T + eps I   (m x m)
 *   R <- beta R + (1 - beta) G^T G + eps I   (n x n)
 * in place on L and R (full storage, fp32).  G is m x n with element type
 * `dtype` (fp32 or bf16; products accumulate in fp32).  The Grams G G^T and
 * G^T G are computed once per pair of symmetric positions (upper-triangle
 * tiles, mirrored); each stored element takes the EMA of its own old value,
 * so L and R need not be exactly symmetric on entry.  The workspace
 * (pmx_workspace_size(PMX_OP_STATS, m, n, batch, dtype)) holds G^T in fp32
 * (and G widened to fp32 for bf16), plus the split-k partial tiles.  Either
 * L or R may be NULL to skip that side.  Requires 0 <= beta <= 1.
 */
pmx_status pmx_shampoo_stats_update(pmx_handle handle, const void* G, pmx_dtype dtype,
                                    int m, int n, int ldg, float* L, int ldl, float* R,
                                    int ldr, float beta, float eps, void* workspace,
                                    size_t workspace_bytes, void* stream);
pmx_status pmx_shampoo_stats_update_batched(pmx_handle handle, const void* G,
                                            pmx_dtype dtype, int m, int n, int ldg,
                                            int64_t stride_g, float* L, int ldl,
                                            int64_t stride_l, float* R, int ldr,
                                            int64_t stride_r, float beta, float eps,
                                            int batch, void* workspace,
                                            size_t workspace_bytes, void* stream);

/*
 * Inverse p-th root by PRISM-accelerated coupled Newton-Schulz
 * ([Shampoo blog] section 3.1; [PRISM synthesis] Part I, Part II):
 *   c = ||A||_F, Y_0 = A / c, Z_0 = I;  per update k:
 *   R_k = I - Z_k Y_k, alpha_k fitted on a Gaussian sketch of R_k,
 *   g = f_{d-1}(R_k) + alpha_k R_k^d, Y <- Y g, Z <- g Z.
 * p = 2: X = A^{-1/2} = Z / sqrt(c), X_aux = A^{1/2} = sqrt(c) Y.
 * p = 4: a second stage from the first stage's Y; X = A^{-1/4},
 *        X_aux = A^{1/4}.
 * A is n x n fp32, symmetric positive definite (full storage read).  X_aux
 * may be NULL.  info_dev points to `batch` pmx_matfn_info (may be NULL).
 * opts may be NULL for the defaults.
 */
pmx_status pmx_matfn_inv_root(pmx_handle handle, const float* A, int n, int lda, int p,
                              float* X, int ldx, float* X_aux, int ldaux,
                              const pmx_matfn_opts* opts, pmx_matfn_info* info_dev,
                              void* workspace, size_t workspace_bytes, void* stream);
pmx_status pmx_matfn_inv_root_batched(pmx_handle handle, const float* A, int n, int lda,
                                      int64_t stride_a, int p, float* X, int ldx,
                                      int64_t stride_x, float* X_aux, int ldaux,
                                      int64_t stride_aux, int batch,
                                      const pmx_matfn_opts* opts,
                                      pmx_matfn_info* info_dev, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * Polar factor U of G (m x n) by PRISM-accelerated Newton-Schulz
 * ([PRISM synthesis] Part I: sign/polar functions; Part II):
 *   X_0 = G / ||G||_F, R_k = I - X_k^T X_k, X <- X g(R_k).
 * For m < n the iteration runs on G^T.  G and U have element type `dtype`
 * (fp32: fp32 iterates; bf16: bf16 iterates with fp32 accumulation).
 */
pmx_status pmx_matfn_polar(pmx_handle handle, const void* G, pmx_dtype dtype, int m, int n,
                           int ldg, void* U, int ldu, const pmx_matfn_opts* opts,
                           pmx_matfn_info* info_dev, void* workspace,
                           size_t workspace_bytes, void* stream);
pmx_status pmx_matfn_polar_batched(pmx_handle handle, const void* G, pmx_dtype dtype,
                                   int m, int n, int ldg, int64_t stride_g, void* U,
                                   int ldu, int64_t stride_u, int batch,
                                   const pmx_matfn_opts* opts, pmx_matfn_info* info_dev,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Polar factors of many blocks of different shapes in one call (the
 * per-block orthogonalisation of block-diagonal preconditioners; [PRISM
 * synthesis] Part I, sign/polar functions).  Each block is iterated as in
 * pmx_matfn_polar with fp32 arithmetic throughout (bf16 blocks are widened
 * on load and rounded to nearest even on store).  Blocks with both sides at
 * most PMX_VARBATCH_MAX_DIM run one workgroup per block with the whole
 * iteration in LDS, all in one launch; larger blocks (sides up to
 * PMX_VARBATCH_MAX_SIDE) are grouped by shape, gathered into a packed fp32
 * batch in the workspace, iterated by the batched fp32 polar factor and
 * scattered back (a large block's sketch stream is that of its position in
 * its shape group, stage 0).
 *   blocks: HOST array of `count` descriptors; every one is checked before
 *           anything is enqueued (1 <= m, n <= PMX_VARBATCH_MAX_SIDE, ldg >= n,
 *           ldu >= n, non-null pointers, output not overlapping its input),
 *           then copied into the workspace on `stream`; the array may be
 *           reused once the call returns.
 *   info_dev: `count` pmx_matfn_info (may be NULL), in block order.
 *   opts: degree 1 or 2 (fixed), fp32 iterates, the Frobenius scale; method
 *         and fp64_iters are ignored.  dtype applies to every block.
 *   workspace: pmx_polar_varbatch_workspace_size(blocks, count, ...); when no
 *         block exceeds PMX_VARBATCH_MAX_DIM this equals
 *         pmx_workspace_size(PMX_OP_POLAR_VARBATCH, batch = count).
 * Returns PMX_ERR_NOT_SUPPORTED, enqueuing nothing, while `stream` is being
 * captured into a HIP graph: the descriptor copy reads host memory that a
 * replay could not rely on.
 */
#define PMX_VARBATCH_MAX_DIM 64
#define PMX_VARBATCH_MAX_SIDE 8192
typedef struct {
  const void* g; /* device pointer: the m x n block, row-major, leading dimension ldg */
  void* u;       /* device pointer: its polar factor, m x n, leading dimension ldu */
  int32_t m, n;
  int32_t ldg, ldu;
} pmx_polar_block;

pmx_status pmx_matfn_polar_varbatch(pmx_handle handle, const pmx_polar_block* blocks, int count,
                                    pmx_dtype dtype, const pmx_matfn_opts* opts,
                                    pmx_matfn_info* info_dev, void* workspace,
                                    size_t workspace_bytes, void* stream);
/* Workspace bytes of pmx_matfn_polar_varbatch for these blocks (host array;
 * only the shapes are read).  PMX_ERR_INVALID_VALUE for a shape out of
 * range, a NULL array or count < 1; opts may be NULL for the defaults. */
pmx_status pmx_polar_varbatch_workspace_size(const pmx_polar_block* blocks, int count,
                                             pmx_dtype dtype, const pmx_matfn_opts* opts,
                                             size_t* bytes);

/*
 * Preconditioned step ([Shampoo blog] sections 2.1 and 2.3, step 4):
 *   P = Linv * G * Rinv,  Linv m x m, G m x n, Rinv n x n (fp32),
 * G and P of element type `dtype`; accumulation in fp32.
 */
pmx_status pmx_precond_apply(pmx_handle handle, const float* Linv, int ldl, const void* G,
                             pmx_dtype dtype, int m, int n, int ldg, const float* Rinv,
                             int ldr, void* P, int ldp, void* workspace,
                             size_t workspace_bytes, void* stream);
pmx_status pmx_precond_apply_batched(pmx_handle handle, const float* Linv, int ldl,
                                     int64_t stride_l, const void* G, pmx_dtype dtype,
                                     int m, int n, int ldg, int64_t stride_g,
                                     const float* Rinv, int ldr, int64_t stride_r, void* P,
                                     int ldp, int64_t stride_p, int batch, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * pmx_precond_apply_batched without a workspace argument, for callers that
 * cannot allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc.  It runs the same kernels
 * and gives the same result; the intermediate L^{-1/4} G (and, for bf16, the
 * widened G and the fp32 P) lives in a scratch array inside the library, one
 * copy per device of PMX_NOALLOC_SCRATCH_BYTES, held until the process ends
 * (its address is resolved by pmx_create).  The call itself allocates
 * nothing.  Limit: pmx_workspace_size(PMX_OP_APPLY, m, n, batch, dtype)
 * must not exceed PMX_NOALLOC_SCRATCH_BYTES (fp32: m n batch <= 8 Mi
 * elements; bf16: <= 2.6 Mi), else PMX_ERR_WORKSPACE with nothing enqueued.
 * Every call on a device shares that device's scratch: calls that may
 * overlap in time on one device (different streams without ordering, or
 * different threads) race and must be ordered by the caller.  Other
 * arguments and errors as in pmx_precond_apply_batched.
 */
#define PMX_NOALLOC_SCRATCH_BYTES (32u << 20)
pmx_status pmx_precond_apply_noalloc(pmx_handle handle, const float* Linv, int ldl,
                                     int64_t stride_l, const void* G, pmx_dtype dtype, int m,
                                     int n, int ldg, int64_t stride_g, const float* Rinv,
                                     int ldr, int64_t stride_r, void* P, int ldp,
                                     int64_t stride_p, int batch, void* stream);

/*
 * A whole Shampoo optimizer step over the layers of a model ([Shampoo blog]
 * sections 2.3 and 6.3 for the step, 3.2 for the block-diagonal
 * approximation, 5.1 for the adaptive learning rate, 5.2 for momentum, 5.3
 * for convolution kernels):
 *   every layer's gradient is viewed as a matrix (a c_out x c_in x kh x kw
 *   kernel as the (c_out kh kw) x c_in matrix K'[(o kh + y) kw + x][i] =
 *   K[o][i][y][x]) and cut into blocks of at most block x block; each block
 *   is a parameter of its own with statistics L, R, momentum M and roots;
 *   per step t (counted by the caller from 0):
 *     L <- beta L + (1 - beta) G G^T + eps I,  R likewise       (every block)
 *     L^{-1/4}, R^{-1/4} recomputed when t % root_every == 0 (kept otherwise)
 *     P = L^{-1/4} G R^{-1/4},  M <- momentum M + P  (M = P when momentum = 0)
 *     W <- W - eta_t M,  eta_t = lr, or with adaptive_lr
 *     eta_t = lr / sqrt(1 + sum_{i <= t} ||G_i||_F^2) (the sum over all layers).
 * Blocks of equal shape are processed as one batch in every call above; the
 * plan groups them once.  All device memory is the caller's: `state`
 * (statistics, roots, momentum, the running gradient norm; kept between
 * steps, set up by pmx_shampoo_plan_init) and `workspace` (per step).
 */
typedef struct {
  int32_t struct_version;   /* 1 */
  int32_t block;            /* largest block side, 1..PMX_MAX_N; default 1024 */
  int32_t root_every;       /* >= 1; default 1 */
  int32_t adaptive_lr;      /* 0 or 1; default 0 */
  float beta, eps;          /* defaults 0.95, 1e-6 */
  float lr, momentum;       /* defaults 1e-3, 0 */
  pmx_matfn_opts root_opts; /* options of the inverse 4th roots (defaults) */
} pmx_shampoo_config;

typedef struct {
  int32_t dims;     /* 2: shape[0] x shape[1] row-major; 4: c_out x c_in x kh x kw */
  int32_t shape[4];
} pmx_layer;

typedef struct pmx_shampoo_plan_t* pmx_shampoo_plan;

/* Fill `cfg` with the defaults above. */
pmx_status pmx_shampoo_config_default(pmx_shampoo_config* cfg);
/* Block and group the layers (host only; no device memory). */
pmx_status pmx_shampoo_plan_create(pmx_handle handle, const pmx_shampoo_config* cfg,
                                   const pmx_layer* layers, int nlayers,
                                   pmx_shampoo_plan* plan);
pmx_status pmx_shampoo_plan_destroy(pmx_shampoo_plan plan);
/* Bytes of the persistent state and of the per-step workspace. */
pmx_status pmx_shampoo_plan_sizes(pmx_shampoo_plan plan, size_t* state_bytes,
                                  size_t* workspace_bytes);
/* Enqueue the state's set-up on `stream`: L = R = eps I, M = 0, the running
 * norm 0, and the block tables.  Not capturable (PMX_ERR_NOT_SUPPORTED while
 * `stream` is being captured into a HIP graph). */
pmx_status pmx_shampoo_plan_init(pmx_shampoo_plan plan, void* state, size_t state_bytes,
                                 void* stream);
/* One step: W[l] and G[l] are device pointers to layer l's weight and
 * gradient (fp32, the layer's natural layout); the HOST arrays W and G may be
 * reused once the call returns (they are copied into the workspace).  Not
 * capturable: PMX_ERR_NOT_SUPPORTED, enqueuing nothing, while `stream` is
 * being captured into a HIP graph (a replay would copy from host memory that
 * no longer holds the table). */
pmx_status pmx_shampoo_plan_step(pmx_shampoo_plan plan, float* const* W, const float* const* G,
                                 int64_t step, void* state, size_t state_bytes, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * The Gaussian sketch S_k that the alpha fit of the iterations draws
 * ([PRISM synthesis] Part II, "Randomized Sketching": a Gaussian oblivious
 * subspace embedding, S with i.i.d. N(0, 1) entries, fresh per update).  The
 * generator is Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with key
 * (seed mod 2^32, seed >> 32); the counter layout is this library's: element
 * e = i p + j of S (n x p) for matrix `matrix` of a batch, stage `stage`
 * (0 and 1: the two stages of the chained inverse 4th root, 0 for a square
 * root or polar factor; 2: the start block of the estimated input scale) and
 * update k is word e % 4 of the call with counter (e / 4, k, stage, matrix).
 * Uniforms u = ((x >> 8) + 1/2) 2^-24; Box-Muller in fp64 on the word pairs
 * (0, 1) and (2, 3): z0 = sqrt(-2 ln u0) cos(2 pi u1), z1 = ... sin(2 pi u1),
 * likewise z2, z3 from (u2, u3); S[e] = z_{e % 4} rounded to fp32.
 *   S:     device, n x p fp32, row stride lds >= p (written).
 *   words: device, n x p uint32 (row stride p) receiving the raw Philox
 *          words behind S, or NULL.  Must not overlap S (PMX_ERR_ALIAS).
 * n in [1, 32768], p in [1, PMX_MAX_SKETCH], matrix, stage, k >= 0, else
 * PMX_ERR_INVALID_VALUE with nothing enqueued.  The iterations generate
 * their sketches with the same device code.
 */
pmx_status pmx_sketch_gaussian(pmx_handle handle, uint64_t seed, int matrix, int stage, int k,
                               int n, int p, float* S, int lds, uint32_t* words, void* stream);

/*
 * Launch trace for benchmarking.  While enabled, every kernel that a call on
 * this handle enqueues is bracketed by a pair of HIP events recorded on the
 * call's stream (host-side event objects owned by the handle; no device
 * memory).  Kernels are grouped into the classes below; each class is one
 * kernel symbol family of the library.
 */
typedef enum {
  PMX_KC_GEMM_POWER = 0,   /* R^2 = R R (and R^3 = R^2 R for d = 3) */
  PMX_KC_GEMM_UPDATE = 1,  /* Y g and g Z (one launch), X g */
  PMX_KC_GEMM_RESID = 2,   /* I - Z Y, I - X^T X, Frobenius norm, convergence decision */
  PMX_KC_GEMM_STATS = 3,   /* G G^T, G^T G with the EMA epilogue */
  PMX_KC_GEMM_APPLY = 4,   /* L^{-1/4} G, then (L^{-1/4} G) R^{-1/4} */
  PMX_KC_SKINNY = 5,       /* Krylov passes R^j S */
  PMX_KC_SKINNY_ALPHA = 6, /* last Krylov pass with the Gram and the alpha solve */
  PMX_KC_OTHER = 7,        /* control reset, scaling, stage set-up, g, outputs */
  PMX_KC_COUNT = 8
} pmx_kernel_class;

/* Convergence polling by the host (off by default: chunk = 0).  A
 * matrix-function call normally enqueues all max_iter updates of a stage up
 * front; the updates after convergence exit on the device but still pay for
 * their launches (a few microseconds each).  With chunk > 0 the fp32 update
 * loops of pmx_matfn_inv_root* and pmx_matfn_polar* (and the Shampoo plan's
 * roots) publish, after every `chunk` updates, whether any matrix of the
 * batch is still iterating: a one-block kernel writes it to pinned host
 * memory behind an event.  The host reads each published value one chunk
 * later, so one chunk stays queued and the device does not wait for the
 * host, and it stops enqueuing updates once a value says that none is
 * iterating.  Results and info are the same as with chunk = 0 (the updates
 * left out are those that would have exited at once); at most 2 chunk - 1
 * updates a stage are enqueued past convergence.  The calling thread blocks
 * on those events, so a call returns only once the device is at most a
 * chunk behind it.  Polling is skipped while the stream is being captured.
 * The first enable allocates 8 bytes of pinned host memory and two events,
 * freed by pmx_destroy.  Returns PMX_ERR_INVALID_VALUE for chunk outside
 * [0, 1000], PMX_ERR_HIP when the pinned memory or events cannot be made. */
pmx_status pmx_set_host_poll(pmx_handle handle, int chunk);

/* Enable (1) or disable (0) the launch trace; enabling discards old records. */
pmx_status pmx_trace_enable(pmx_handle handle, int enable);
/* Wait for the recorded events, write per kernel class the summed
 * event-to-event time in milliseconds and the number of launches into
 * ms[PMX_KC_COUNT] and launches[PMX_KC_COUNT], then clear the records. */
pmx_status pmx_trace_collect(pmx_handle handle, double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* PMX_H */
