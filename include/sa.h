/*
 * sa.h — C interface of the Sketch Attention (SA) library for MI355X (gfx950).
 *
 * Sketch Attention compresses one user's history X (n events x d) into a fixed
 * k x d sketch against k prototypes P that every user shares:
 *
 *   Z[j,i]  = p_j . x_i / sqrt(d)                    affinities
 *   A[j,i]  = exp Z[j,i] / sum_j' exp Z[j',i]        softmax over the k
 *                                                     prototypes, per token
 *   S[j]    = sum_i A[j,i] x_i                       plain-sum sketch, or
 *   S[j]    = sum_i A[j,i] x_i / mu[j],  mu[j] = sum_i A[j,i]
 *                                                     (mass normalisation)
 *
 * Sources: "SequenceO1: End-to-End Ultra-Long (100K) Sequence Modeling in
 * Recommendation with Low-Rank Caching" — reading-notes page, section 3.1,
 * Eq. (5)-(9) (prototypes, affinities, prototype-wise softmax, sketch), and the
 * paper's HTML page, FlashSA paragraph of the system-design section (fused,
 * streaming computation of affinities, max / log-sum-exp statistics and the
 * aggregation, with no k x n matrix in memory, over ragged batches).  The
 * W_Q, W_K projections of Eq. (6) are folded into P by the caller
 * (P_eff = P W_Q W_K^T gives the same affinities).  Mass normalisation and the
 * backward pass are not printed on the pages: the first is the weighted mean
 * of the tokens a prototype receives, the second is the chain rule of the
 * lines above.
 *
 * Batches are CSR-ragged: users' histories are concatenated along the token
 * axis, and offsets[u] .. offsets[u+1] are user u's rows.  No padding.
 *
 * General conventions
 *  - All tensors are dense, row-major, contiguous, in device memory, and
 *    16-byte aligned.  The caller owns every buffer, including the workspace;
 *    the library allocates nothing and keeps no mutable global state, so calls
 *    on different streams with different workspaces may run concurrently.
 *  - GPU work is enqueued on `stream` and calls return without waiting.
 *    Argument errors are reported synchronously by the return value and
 *    nothing is enqueued.  Inconsistent device-side offsets are detected on
 *    the device, recorded in the workspace and read back by
 *    sa_get_device_status(); kernels clamp every index, so bad offsets give
 *    wrong numbers, never an out-of-bounds access.
 *  - Outputs are float32.  X and P are float32 (SA_F32, float32 arithmetic
 *    throughout) or bfloat16 (SA_BF16, bf16 matrix-core products with float32
 *    accumulation; the softmax weights enter the second product as bf16).
 *  - Results are bitwise reproducible for identical inputs, device and
 *    problem: every reduction runs in a fixed order and no floating-point
 *    atomics are used.
 *  - Shape limits: d in {32, 64, 128}; 1 <= k <= 2048; batch >= 1;
 *    0 <= total_tokens < 2^36.  Users may be empty (n_u = 0 gives S = 0 and
 *    mass = 0).
 */
#ifndef SKETCH_ATTENTION_SA_H
#define SKETCH_ATTENTION_SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL_ARG = 1,            /* a required pointer is NULL              */
  SA_ERR_BAD_SHAPE = 2,           /* k, d, batch or total_tokens out of range */
  SA_ERR_BAD_DTYPE = 3,           /* dtype is not SA_F32 / SA_BF16           */
  SA_ERR_UNSUPPORTED = 4,         /* flags or op not supported               */
  SA_ERR_WORKSPACE_TOO_SMALL = 5, /* ws_bytes < sa_workspace_size()          */
  SA_ERR_BAD_OFFSETS = 6,         /* host-checked or device-detected offsets */
  SA_ERR_MISALIGNED = 7,          /* a pointer is not 16-byte aligned        */
  SA_ERR_HIP = 8,                 /* a HIP runtime call failed               */
  SA_ERR_DEVICE_TIMEOUT = 9       /* device-detected: the single-pass forward's
                                     statistics exchange gave up waiting     */
} sa_status;

typedef enum { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;

/* Problem flags.
 *  SA_FLAG_MASS_NORM: S[j] is the mass-normalised (weighted-mean) sketch.
 *  SA_FLAG_PER_USER_PROTOTYPES: every user has its own prototype table.  P is
 *    then [B, k, d] (user u's table at P + u k d) instead of one shared
 *    [k, d] table, and sa_backward's dP is [B, k, d] with dP[u] the gradient
 *    of user u's table (instead of the sum over users).  This is the form of
 *    the refinement layers (SequenceO1 reading notes, section 3.3,
 *    Eq. (12)-(14)), whose queries are the user's own sketch from the layer
 *    before.
 *  SA_FLAG_TOKEN_WISE: the vanilla-attention baseline of Table 1 (reading
 *    notes, sections 3.5 and 7.1): the same affinities normalised over each
 *    user's tokens instead of over the prototypes,
 *        A[j,i] = exp Z[j,i] / sum_i' exp Z[j,i'],  S[j] = sum_i A[j,i] x_i,
 *    with lse per user and prototype: lse[u,j] = log sum_i exp Z[j,i]
 *    (float [B, k]; -inf for an empty user, whose S is 0).  sa_forward's lse
 *    argument is then [B, k] and mass must be NULL; sa_backward requires the
 *    forward's S and lse.  Not combinable with the other two flags. */
enum { SA_FLAG_MASS_NORM = 1u, SA_FLAG_PER_USER_PROTOTYPES = 2u, SA_FLAG_TOKEN_WISE = 4u };

/* Operation selector for sa_workspace_size. */
enum { SA_OP_FORWARD = 0, SA_OP_BACKWARD = 1 };

typedef struct {
  int32_t batch;         /* B, number of users (>= 1)                    */
  int32_t k;             /* prototypes                                   */
  int32_t d;             /* width of X rows and prototypes               */
  int64_t total_tokens;  /* T = offsets[B]                               */
  sa_dtype dtype;        /* dtype of X and P                             */
  uint32_t flags;        /* SA_FLAG_*                                    */
} sa_problem;

/* Library version, major * 10000 + minor * 100 + patch. */
int sa_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* sa_status_string(sa_status status);

/* Host-only validation of a problem description; makes no HIP call.
 * offsets_host (nullable): a host copy of the B+1 offsets; when given, it
 * must start at 0, be non-decreasing and end at total_tokens, else
 * SA_ERR_BAD_OFFSETS. */
sa_status sa_validate(const sa_problem* problem, const int64_t* offsets_host);

/* Bytes of workspace that sa_forward (op = SA_OP_FORWARD) or sa_backward
 * (op = SA_OP_BACKWARD) need for this problem.  Returns 0 for an invalid
 * problem or op.  Pure host arithmetic; makes no HIP call. */
size_t sa_workspace_size(const sa_problem* problem, int op);

/*
 * Forward.  Computes, for every user u, the sketch S[u] (k x d) and the
 * prototype masses mass[u] (k), plus the per-token log-sum-exp of the
 * affinities, lse[i] = log sum_j exp Z[j,i] (natural log), which the
 * FlashSA paragraph names as the softmax statistic and the backward reuses.
 *
 *  offsets_dev : int64 [B+1] device; offsets[0] = 0, non-decreasing,
 *                offsets[B] = total_tokens.
 *  X           : [T, d] (dtype) device.
 *  P           : [k, d] (dtype) device, shared by all users; or [B, k, d]
 *                with SA_FLAG_PER_USER_PROTOTYPES (user u uses P[u]).
 *  S           : float [B, k, d] device, written.
 *  lse         : float [T] device, written; may be NULL (kept in workspace).
 *  mass        : float [B, k] device, written; may be NULL.
 *  ws, ws_bytes: device workspace of at least
 *                sa_workspace_size(problem, SA_OP_FORWARD) bytes; its
 *                contents on entry are ignored.
 *  stream      : HIP stream (hipStream_t) the work is enqueued on.
 * Errors: SA_ERR_NULL_ARG, SA_ERR_BAD_SHAPE, SA_ERR_BAD_DTYPE,
 * SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE_TOO_SMALL, SA_ERR_MISALIGNED
 * (nothing enqueued); SA_ERR_HIP if a launch fails.
 * Two forms compute the same values (up to rounding order): the default
 * two-pass form (per-token statistics, then the aggregation) and, for bf16
 * with a shared table when the environment variable SA_FORWARD_PATH is
 * "single_pass", a single pass whose workgroups exchange per-token
 * statistics (cooperative launch; if that launch is refused the two-pass
 * form runs instead).  The single pass reports a given-up wait through
 * sa_get_device_status (SA_ERR_DEVICE_TIMEOUT).
 */
sa_status sa_forward(const sa_problem* problem, const int64_t* offsets_dev,
                     const void* X, const void* P, float* S, float* lse,
                     float* mass, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward.  Given dS = dL/dS (float [B, k, d]), writes
 *   dX = dL/dX  (float [T, d], overwritten) and
 *   dP = dL/dP  (float [k, d], overwritten; summed over all users because
 *                the prototypes are shared; with SA_FLAG_PER_USER_PROTOTYPES
 *                float [B, k, d], dP[u] from user u's tokens alone, zero for
 *                an empty user).
 * The softmax weights are recomputed tile by tile from X, P and lse; lse is
 * the forward's output (float [T]) or NULL, in which case it is recomputed.
 * With SA_FLAG_MASS_NORM, S and mass from the forward are required (float
 * [B, k, d] and [B, k]); without it they are ignored and may be NULL.
 * Formulas (chain rule, one user, c = 1/sqrt(d)):
 *   G = dS, cv = 0                     (plain sum)
 *   G[j] = dS[j] / mu[j], cv[j] = G[j] . S[j]   (mass norm; mu[j] = 0 -> 0)
 *   g_i = sum_j A[j,i] G[j];  delta_i = x_i . g_i - sum_j A[j,i] cv[j]
 *   dZ[j,i] = A[j,i] (G[j] . x_i - cv[j] - delta_i)
 *   dX_i = g_i + c sum_j dZ[j,i] p_j;   dP = c sum_u sum_i dZ[j,i] x_i
 * Same error behaviour as sa_forward.
 */
sa_status sa_backward(const sa_problem* problem, const int64_t* offsets_dev,
                      const void* X, const void* P, const float* dS,
                      const float* lse, const float* S, const float* mass,
                      float* dX, float* dP, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * Per-kernel timing for benchmarks.  The pages report no measurement of
 * their own; these variants exist so that a benchmark can time each kernel of
 * one call on the stream it runs on.  They behave exactly like sa_forward /
 * sa_backward and additionally record prof->events[2i] and
 * prof->events[2i+1] on `stream` immediately before and after the i-th
 * kernel they launch (at most SA_PROFILE_MAX_KERNELS kernels), set
 * prof->names[i] to a static kernel name and prof->n_kernels to the number of
 * kernels launched.  The caller creates all 2 * SA_PROFILE_MAX_KERNELS
 * events (hipEvent_t handles, passed as void*) beforehand; any NULL handle
 * gives SA_ERR_NULL_ARG and nothing is enqueued.  Recording events adds a
 * little host overhead; use the plain entry points for end-to-end timing.
 */
#define SA_PROFILE_MAX_KERNELS 8

typedef struct {
  void* events[2 * SA_PROFILE_MAX_KERNELS]; /* in: hipEvent_t handles        */
  int32_t n_kernels;                        /* out: kernels launched         */
  const char* names[SA_PROFILE_MAX_KERNELS]; /* out: static kernel names     */
} sa_profile;

sa_status sa_forward_profiled(const sa_problem* problem, const int64_t* offsets_dev,
                              const void* X, const void* P, float* S, float* lse,
                              float* mass, void* ws, size_t ws_bytes, void* stream,
                              sa_profile* prof);

sa_status sa_backward_profiled(const sa_problem* problem, const int64_t* offsets_dev,
                               const void* X, const void* P, const float* dS,
                               const float* lse, const float* S, const float* mass,
                               float* dX, float* dP, void* ws, size_t ws_bytes,
                               void* stream, sa_profile* prof);

/*
 * Query and key projections (SequenceO1 reading notes, section 3.1, Eq. (6):
 * Z = (P W_Q)(X W_K)^T / sqrt(d), with W_Q, W_K in R^{d x d}).  Because
 * (P W_Q)(X W_K)^T = (P W_Q W_K^T) X^T, the projected affinities are the
 * kernel's affinities of the folded table
 *     P_eff = P W_Q W_K^T,
 * so sa_forward(X, P_eff) computes the sketch of Eq. (6)-(9) with the
 * projections; the aggregation still sums the unprojected X (Eq. (9)).
 *
 *  k, d    : rows of P and P_eff, 1 <= k <= 2^24: a shared table's k, or
 *            B k for the stacked per-user tables of SA_FLAG_PER_USER_PROTOTYPES
 *            (one W_Q, W_K for all users); d in {32, 64, 128}.
 *  dtype   : dtype of P and P_eff (SA_BF16: P_eff is rounded to bf16 once,
 *            from fp32 accumulation; SA_F32: fp32 throughout).
 *  P       : [k, d] (dtype) device.
 *  Wq, Wk  : float [d, d] device, row-major (row = input feature).
 *  P_eff   : [k, d] (dtype) device, written; must not overlap P.
 * All pointers 16-byte aligned, caller-owned.  Enqueued on `stream`; returns
 * at once.  Errors (synchronous): SA_ERR_NULL_ARG, SA_ERR_BAD_SHAPE,
 * SA_ERR_BAD_DTYPE, SA_ERR_MISALIGNED, SA_ERR_HIP.
 */
sa_status sa_fold_prototypes(int k, int d, sa_dtype dtype, const void* P, const float* Wq,
                             const float* Wk, void* P_eff, void* stream);

/*
 * Backward of the fold.  Given dP_eff = dL/dP_eff (float [k, d], e.g. the dP
 * that sa_backward returns for P_eff), writes, with M = W_Q W_K^T:
 *     dP   = dP_eff M^T            float [k, d]
 *     dW_Q = P^T dP_eff W_K        float [d, d]
 *     dW_K = dP_eff^T P W_Q        float [d, d]
 * (all overwritten).  dW_Q and dW_K are sums over the k rows taken in a fixed
 * order, so repeated calls give identical bits.  `ws` is a device workspace of
 * at least sa_fold_workspace_size(k, d) bytes (per-workgroup partial sums of
 * dW_Q and dW_K); sa_fold_workspace_size returns 0 for unsupported (k, d).
 * Other arguments as for sa_fold_prototypes; errors as there, plus
 * SA_ERR_WORKSPACE_TOO_SMALL.
 */
size_t sa_fold_workspace_size(int k, int d);
sa_status sa_fold_prototypes_backward(int k, int d, sa_dtype dtype, const void* P,
                                      const float* Wq, const float* Wk, const float* dP_eff,
                                      float* dP, float* dWq, float* dWk, void* ws,
                                      size_t ws_bytes, void* stream);

/*
 * The stacked Sketch Attention block (SequenceO1 reading notes, section 3.3,
 * Eq. (12)-(16)): starting from the shared table, X~(0) = P0, each of the
 * n_layers layers computes, per user,
 *     X^     = SA(X, X~ W_Q W_K^T)            Eq. (12)-(14), plain-sum sketch
 *     X-     = LN1(X~ + X^)                    Eq. (15)
 *     X~'    = LN2(X- + FFN(X-))               Eq. (16)
 * with FFN(x) = (silu(x W1) * (x W3)) W2, the SwiGLU FFN of hidden width 2d
 * (W1, W3: [d, 2d], W2: [2d, d], no biases), and LN(v) = (v - mean) /
 * sqrt(var + 1e-5) * g + b over the d features of a row (biased variance).
 * Layer 0's queries are the shared table; later layers' queries are each
 * user's own rows (SA_FLAG_PER_USER_PROTOTYPES inside).  The output is X~ of
 * the last layer, float [B, k, d].
 *
 * All parameters are float32 device arrays, row-major.  The sketch products
 * run in the problem's dtype (X and the folded tables in bf16 with fp32
 * accumulation for SA_BF16); everything else is fp32.
 *
 *  problem  : as for sa_forward; flags must be 0 (the block's sketch is the
 *             plain sum of Eq. (14), and it manages per-user tables itself).
 *  n_layers : 1 .. 8 (the pages use 2).
 *  X        : [T, d] (dtype); P0: float [k, d]; out: float [B, k, d].
 *  layers   : host array of n_layers parameter sets (device pointers).
 *  ws       : device workspace of sa_block_workspace_size(problem, n_layers)
 *             bytes.  sa_block_forward leaves in it the activations that
 *             sa_block_backward reads: a backward must use the workspace of
 *             the forward on the same inputs, untouched in between.
 * Errors as for sa_forward (SA_ERR_UNSUPPORTED for flags or n_layers out of
 * range).
 */
typedef struct {
  const float* Wq;      /* [d, d]   */
  const float* Wk;      /* [d, d]   */
  const float* ln1_g;   /* [d]      */
  const float* ln1_b;   /* [d]      */
  const float* W1;      /* [d, 2d]  */
  const float* W3;      /* [d, 2d]  */
  const float* W2;      /* [2d, d]  */
  const float* ln2_g;   /* [d]      */
  const float* ln2_b;   /* [d]      */
} sa_block_layer;

/* Gradients of one layer's parameters (device pointers, same shapes as
 * sa_block_layer; all overwritten). */
typedef struct {
  float* Wq;
  float* Wk;
  float* ln1_g;
  float* ln1_b;
  float* W1;
  float* W3;
  float* W2;
  float* ln2_g;
  float* ln2_b;
} sa_block_layer_grad;

size_t sa_block_workspace_size(const sa_problem* problem, int n_layers);
sa_status sa_block_forward(const sa_problem* problem, int n_layers, const int64_t* offsets_dev,
                           const void* X, const float* P0, const sa_block_layer* layers,
                           float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of the block: given dout = dL/dout (float [B, k, d]), writes
 * dX = dL/dX (float [T, d]), dP0 = dL/dP0 (float [k, d]) and every layer's
 * parameter gradients (all overwritten).  Weight and layer-norm gradients
 * sum over all users' rows in a fixed order (deterministic).  `ws` must hold
 * the state left by sa_block_forward for the same problem, X, P0 and layers.
 */
sa_status sa_block_backward(const sa_problem* problem, int n_layers, const int64_t* offsets_dev,
                            const void* X, const float* P0, const sa_block_layer* layers,
                            const float* dout, float* dX, float* dP0,
                            const sa_block_layer_grad* grads, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * Action-side SwiGLU fusion (SequenceO1 reading notes, section 3.6,
 * Eq. (20)): the history rows the sketch consumes,
 *     x_i = e_i + (silu(v_i W1) * (v_i W3)) W2,   v_i = [e_i; A[t_i]],
 * from item embeddings e (the history's dtype) and action types t_i that
 * index an action table A (float [n_types, d]).  W1, W3: float [2d, 2d]
 * (rows 0 .. d-1 act on e, rows d .. 2d-1 on the action row), W2: float
 * [2d, d]; hidden width 2d, no biases.  The page leaves the FFN's sizes
 * open; the hidden width 2d (twice the width of e_i, half of what Eq. (23)'s
 * rule would give for the 2d-wide v_i) is this library's choice.
 *
 *  d       : 32, 64 or 128;  T: events, 0 <= T <= 2^30;  1 <= n_types <= 16.
 *  dtype   : of e and x.  SA_BF16 runs the fused matrix-core kernel (bf16
 *            products, fp32 accumulation); SA_F32 is fp32 throughout.
 *  types   : int32 [T] device (values outside [0, n_types) are clamped).
 *  x       : [T, d] (dtype) device, written; the sketch's X.
 *  ws      : sa_action_fusion_workspace_size(d, dtype, T, n_types, op) bytes.
 * Backward: given dx = dL/dx (float [T, d], e.g. sa_backward's dX), writes
 * de (float [T, d]), dA (float [n_types, d]), dW1, dW3 (float [2d, 2d]) and
 * dW2 (float [2d, d]), all overwritten; the weight and table gradients sum
 * over events in a fixed order.  With SA_BF16 the backward keeps its
 * per-event intermediates in bf16 and runs its products on the matrix cores
 * (bf16 operands, fp32 accumulation); with SA_F32 it is fp32 throughout.
 * Errors as for the fold.
 */
size_t sa_action_fusion_workspace_size(int d, sa_dtype dtype, int64_t T, int n_types, int op);
sa_status sa_action_fusion_forward(int d, sa_dtype dtype, int64_t T, int n_types, const void* e,
                                   const int32_t* types, const float* A, const float* W1,
                                   const float* W3, const float* W2, void* x, void* ws,
                                   size_t ws_bytes, void* stream);
sa_status sa_action_fusion_backward(int d, sa_dtype dtype, int64_t T, int n_types, const void* e,
                                    const int32_t* types, const float* A, const float* W1,
                                    const float* W3, const float* W2, const float* dx, float* de,
                                    float* dA, float* dW1, float* dW3, float* dW2, void* ws,
                                    size_t ws_bytes, void* stream);

/*
 * Reordered single-query STCA attention (SequenceO1 reading notes, section
 * 5.1, Eq. (24)-(25)): each target r has one query q_r (width D) and attends,
 * per head j (h heads of width d_h = D / h, head j = columns j d_h ..
 * (j+1) d_h - 1 of W_Q, W_K, W_V), over the history rows of its user:
 *     u     = (q_r W_Q[:, j]) W_K[:, j]^T                (width D)
 *     alpha = softmax(X_u u / sqrt(d_h)),   o[r, j] = (alpha X_u) W_V[:, j]
 * so X W_K and X W_V are never formed; the length-dependent work is the two
 * reductions, 4 L D flops per head and target, on the matrix cores (X and u
 * in bf16, fp32 accumulation).  The output projection and the FFN that
 * follow in the pages' STCA layer are added by sa_stca_layer below.
 *
 *  B           : users; x_off: int64 [B+1] device, rows of X per user;
 *                t_off: int64 [B+1] device, targets (rows of Q and o) per user.
 *  D, h        : D in {256, 512, 1024}, h divides D.
 *  X           : bf16 [L, D] device (the sketch rows after the width adapter,
 *                or the recent suffix); Q: float [R, D]; Wq, Wk, Wv: float [D, D].
 *  o           : float [R, D], written (heads concatenated; 0 for a user
 *                without rows); lse: float [R, h] or NULL (log-sum-exp of the
 *                scaled scores, -inf for a user without rows).
 *  ws          : sa_stca_workspace_size(D, h, R) bytes.
 * x_off must be nondecreasing in [0, L] and t_off nondecreasing in [0, R]
 * with t_off[B] = R.  The kernels clamp every user's row range to [0, L] and
 * map every target to a user in [0, B), so malformed offsets give wrong
 * numbers but never an access outside X, Q or o; they are not reported.
 * The query, key and value products round their fp32 operands to bf16 on
 * the matrix cores when d_h is a multiple of 32 and run in fp32 otherwise.
 * Errors as for the fold.
 */
size_t sa_stca_workspace_size(int D, int h, int64_t R);
sa_status sa_stca_attention(int B, int D, int h, int64_t L, int64_t R, const int64_t* x_off,
                            const int64_t* t_off, const void* X, const float* Q, const float* Wq,
                            const float* Wk, const float* Wv, float* o, float* lse, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * One whole STCA layer per target (reading notes section 5.1, Eq. (26)): the
 * reordered attention above, then the output projection W_O (2 D^2 flops
 * per target) and the query-side SwiGLU FFN of hidden width 2D (12 D^2, the
 * pages' Eq. (23) with w_f = 2w).  The page counts their flops and prints no
 * residual connection or normalisation; they are read as residual sublayers
 * without normalisation:
 *     a = q + o W_O,     y = a + (silu(a W1) * (a W3)) W2.
 *
 *  Wo : float [D, D];  W1, W3 : float [D, 2D];  W2 : float [2D, D]; no biases.
 *  y  : float [R, D], written.
 *  o  : float [R, D] or NULL: the attention output, also written when given.
 *  lse, and every other argument: as for sa_stca_attention.
 *  ws : sa_stca_layer_workspace_size(D, h, R) bytes.
 * The four products round their fp32 operands to bf16 on the matrix cores
 * with fp32 accumulation; the SwiGLU is fp32.  Errors as for
 * sa_stca_attention, checked before anything is enqueued.
 */
size_t sa_stca_layer_workspace_size(int D, int h, int64_t R);
sa_status sa_stca_layer(int B, int D, int h, int64_t L, int64_t R, const int64_t* x_off,
                        const int64_t* t_off, const void* X, const float* Q, const float* Wq,
                        const float* Wk, const float* Wv, const float* Wo, const float* W1,
                        const float* W3, const float* W2, float* y, float* o, float* lse,
                        void* ws, size_t ws_bytes, void* stream);

/* Waits for `stream`, then reports whether a kernel of the last call that
 * used this workspace found inconsistent offsets (SA_ERR_BAD_OFFSETS), or the
 * single-pass forward's statistics exchange between workgroups gave up
 * waiting (SA_ERR_DEVICE_TIMEOUT: every wait is bounded, so the kernel ends,
 * but that call's results are wrong), or neither (SA_OK).  SA_ERR_HIP if the
 * wait or the read fails. */
sa_status sa_get_device_status(const void* ws, void* stream);

/*
 * sa_forward without a caller workspace, for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc.  The caller still owns every input and
 * output (same arguments and meaning as sa_forward); the workspace is a
 * device array of SA_NOALLOC_SCRATCH_BYTES bytes inside the library, one
 * per GPU, which that GPU holds until the process ends.  The call allocates
 * and frees nothing.  The first call on a device (the current device, which
 * must be the stream's) looks the array's device address up once.
 *
 * Returns SA_ERR_WORKSPACE_TOO_SMALL, with nothing enqueued, when the
 * problem's sa_workspace_size(problem, SA_OP_FORWARD) exceeds
 * SA_NOALLOC_SCRATCH_BYTES (64 MiB: for k = 1024, d = 128 that holds about
 * 100 partial sketches, e.g. one user of any length, or a few tens of users
 * of 100K tokens when lse is passed); SA_ERR_HIP if the lookup fails; other
 * errors as sa_forward.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (two streams, two threads) race and
 * give wrong results; serialize them.  Each call rewrites every byte of the
 * array it reads, so nothing carries over from the previous call.  Offsets
 * errors are flagged in the library's array, which the caller cannot read:
 * validate offsets on the host (sa_validate) where that matters.
 */
#define SA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
sa_status sa_forward_noalloc(const sa_problem* problem, const int64_t* offsets_dev,
                             const void* X, const void* P, float* S, float* lse, float* mass,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SKETCH_ATTENTION_SA_H */
