// sa_kernels.h — internal interface between the C-ABI layer (sa_api.cpp) and
// the kernel launchers.  Not installed; the public interface is include/sa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

// Work partition constants (MI355X: 256 compute units, one aggregation
// workgroup per unit).
constexpr int kTargetWorkgroups = 256;
constexpr int kChunkBf16 = 256;     // prototypes per bf16 prototype-stationary workgroup
constexpr int kChunkF32 = 64;       // prototypes per fp32 forward aggregation workgroup
constexpr int kChunkF32Bwd = 32;    // prototypes per fp32 backward dP workgroup
constexpr int kBwdxTokensBf16 = 256;  // tokens per bf16 dX workgroup (8 waves x 32)
constexpr int kBwdxChunkBf16 = 64;    // prototypes per chunk of the bf16 dX pass (and row padding)
constexpr int kBwdxTokensF32 = 32;    // tokens per fp32 dX workgroup
constexpr int kBwdpWaves = 8;         // waves of a bf16 dP workgroup (32 prototypes each)

// Device status word values written into the first bytes of the workspace.
constexpr uint32_t kStatusOk = 0u;
constexpr uint32_t kStatusBadOffsets = 1u;
// Second status word (byte 4 of the workspace): the single-pass forward's
// exchange gave up waiting.  A distinctive value, so that an unwritten word
// is not mistaken for it.
constexpr uint32_t kStatusExchangeTimeout = 0x7E4C7105u;

struct Plan {
  int B, k, d;
  int64_t T;
  int dtype;            // 0 = fp32, 1 = bf16
  bool mass_norm;
  bool per_user;        // P is [B, k, d] (one table per user), dP likewise
  // forward
  int chunk, nchunks, G;
  int64_t nslots;       // G + B - 1 partial slots
  // backward (dP pass)
  int bchunk, bnchunks, Gb;
  int64_t bslots;       // dP partial slots: Gb, or Gb + B - 1 with per-user tables
  int kp;               // row stride of G and cv: k rounded up to the dX chunk (bf16), else k
  // forward workspace layout (byte offsets)
  size_t off_status, off_lse, off_lse2, off_part, off_pmass, off_pl, off_tlse, off_xchg, fwd_bytes;
  // backward workspace layout (byte offsets)
  size_t off_G, off_cv, off_cvs, off_Pq, off_delta, off_dpp, off_blse, off_blse2, off_tlse2,
      off_dz, bwd_bytes;
};

// Fills the plan; returns false for an unsupported problem.
bool make_plan(int B, int k, int d, int64_t T, int dtype, bool mass_norm, bool per_user,
               Plan* p);

struct FwdArgs {
  const int64_t* offsets;
  int B, k, d;
  int64_t T;
  const void* X;
  const void* P;
  int64_t pstride;     // elements between users' tables: 0 (shared P) or k d
  float* lse;          // [T] (caller's buffer or workspace)
  float* lse2;         // [T + 1] log2-unit lse and +inf sentinel, or nullptr (bf16 stats only)
  float* S;            // [B, k, d]
  float* mass;         // [B, k] or nullptr
  float* part;         // [nslots, k, d]
  float* pmass;        // [nslots, k] (token-wise: per-slot running maxima)
  float* pl;           // [nslots, k] token-wise: per-slot sums of weights
  uint32_t* status;    // device status words: [0] offsets, [1] exchange
  uint64_t* xchg;      // [nchunks, T] exchange words of the single-pass forward
  int G, nchunks;
  int mass_norm;
};

struct BwdArgs {
  const int64_t* offsets;
  int B, k, d;
  int64_t T;
  const void* X;
  const void* P;
  int64_t pstride;     // elements between users' tables: 0 (shared P) or k d
  const float* dS;     // [B, k, d]
  const float* lse;    // [T] (caller's, or lse_ws after recomputation)
  float* lse_ws;       // [T]
  float* lse2;         // [T + 1] log2-unit lse with +inf sentinel (bf16 dP pass)
  const float* S;      // [B, k, d] (mass norm only)
  const float* mass;   // [B, k]    (mass norm only)
  float* dX;           // [T, d]
  int acc_dx;          // 1: add to dX instead of overwriting it
  float* dP;           // [k, d], or [B, k, d] with per-user tables
  void* Gq;            // [B, kp, d] G = dS (or dS / mass) in the input dtype, rows >= k zero
  float* cv;           // [B, kp]   G[j] . S[j] (mass norm) or 0
  float* cvs;          // [B, kp]   -cv (bf16 dX pass)
  void* Pq;            // [kp, d] (or [B, kp, d] per user): P with zero rows from k on (bf16)
  int kp;
  float* delta;        // [T]
  float* dpp;          // [bslots, k, d] dP partial per segment (per piece with per-user tables)
  uint32_t* status;
  int Gb, bnchunks;
  int64_t bslots;
  int mass_norm;
  int recompute_lse;
  int tokwise;         // token-wise normalisation: lse is [B, k] and S is required
  float* tlse2;        // [B, kp] token-wise: log2-unit lse per prototype (bf16 path)
  void* dz;            // bf16 c dZ from the dX pass for the dP pass, in MFMA fragment order:
                       // [ceil(T / 32) + 1 token tiles][kz / 32 prototype tiles][64 lanes][16]
  int kz;              // prototypes per token tile of dz: bnchunks x kChunkBf16 (>= kp)
};

// Optional per-kernel timing: when ev is non-null, the launchers record
// ev[2i] / ev[2i+1] on the launch stream right before / after the i-th kernel
// and store a static name for it.
struct Prof {
  hipEvent_t* ev;
  int cap;
  int n;
  const char** names;
};

inline void prof_begin(Prof* p, const char* name, hipStream_t st) {
  if (p != nullptr && p->ev != nullptr && p->n < p->cap) {
    p->names[p->n] = name;
    (void)hipEventRecord(p->ev[2 * p->n], st);
  }
}

inline void prof_end(Prof* p, hipStream_t st) {
  if (p != nullptr && p->ev != nullptr && p->n < p->cap) {
    (void)hipEventRecord(p->ev[2 * p->n + 1], st);
    p->n++;
  }
}

hipError_t launch_stats_bf16(const FwdArgs& a, hipStream_t st, Prof* prof);
// P_eff = P W_Q W_K^T and its backward.
hipError_t launch_fold(int k, int d, int dtype, const void* P, const float* Wq, const float* Wk,
                       void* Peff, hipStream_t st);
hipError_t launch_fold_backward(int k, int d, int dtype, const void* P, const float* Wq,
                                const float* Wk, const float* G, float* dP, float* dWq,
                                float* dWk, float* parts, hipStream_t st);
// The fold of an fp32 table, P_eff written in out_dtype (0 fp32, 1 bf16).
hipError_t launch_fold_from_f32(int k, int d, int out_dtype, const float* P, const float* Wq,
                                const float* Wk, void* Peff, hipStream_t st);
// Workspace of the fold's backward: Q, dQ and per-slice parts of dW_Q, dW_K.
size_t fold_workspace_bytes(int k, int d);

// Dense pieces of the stacked block (sa_block.hip), fp32.
hipError_t launch_gemm(bool ta, bool tb, const float* A, int lda, const float* B, int ldb,
                       float* C, int ldc, int M, int N, int K, int slices, int accumulate,
                       hipStream_t st);
// fp32 operands rounded to bf16 on the matrix cores, fp32 accumulation
// (sa_gemm_mx.hip): C (fp32, or bf16 when out_bf16) = A B(k, n) per batch z,
// A row-major, B(k, n) = tb ? B[n ldb + k] : B[k ldb + n].  K % 32 == 0 and
// 16-byte aligned rows, else hipErrorInvalidValue.  a_bf16: A is bf16 (then
// tb and out_bf16 must be false).
hipError_t launch_gemm_mx(bool tb, bool out_bf16, bool a_bf16, const void* A, int lda, int64_t sA,
                          const float* B, int ldb, int64_t sB, void* C, int ldc, int64_t sC, int M,
                          int N, int K, int batch, hipStream_t st);
// The same with A(m, k) = ta ? A[k lda + m] : A[m lda + k] and the
// reduction split into `slices` slices written to C + z M ldc (accumulate:
// C += instead of C =); K is free when both operands are stored [k][row].
// init (one slice, not accumulating): C = init + op(A) op(B).
hipError_t launch_gemm_mx_sliced(bool ta, bool tb, const float* A, int lda, const float* B, int ldb,
                                 float* C, int ldc, int M, int N, int K, int slices, int accumulate,
                                 hipStream_t st, const float* init = nullptr);
// bf16 operands (a_bf16, b_bf16) and a bf16 output (out_bf16) for the
// action-fusion backward's intermediates (sa_gemm_mx.hip); the combinations
// it does not use return hipErrorInvalidValue.
hipError_t launch_gemm_mx_typed(bool ta, bool tb, bool a_bf16, bool b_bf16, bool out_bf16,
                                const void* A, int lda, const void* B, int ldb, void* C, int ldc,
                                int M, int N, int K, int slices, int accumulate, const float* init,
                                hipStream_t st);
// Batch z of the product: A + z sA, B + z sB -> C + z sC, over all of K.
hipError_t launch_gemm_batched(bool ta, bool tb, const float* A, int lda, int64_t sA,
                               const float* B, int ldb, int64_t sB, float* C, int ldc, int64_t sC,
                               int M, int N, int K, int batch, int accumulate, hipStream_t st);
hipError_t launch_sum_slices(const float* parts, int nslices, int64_t n, const float* init,
                             float* out, hipStream_t st);
hipError_t launch_ln_fwd(int d, const float* a, const float* res, int64_t res_rows, int64_t R,
                         const float* g, const float* b, float* y, float* mean, float* rstd,
                         hipStream_t st);
hipError_t launch_ln_bwd(int d, const float* dy, const float* a, const float* res,
                         int64_t res_rows, int64_t R, const float* mean, const float* rstd,
                         const float* g, float* dv, int acc_dv, float* part, int nblk,
                         hipStream_t st);
hipError_t launch_swiglu_fwd(const float* U1, const float* U3, int64_t n, float* G,
                             hipStream_t st);
hipError_t launch_swiglu_bwd(const float* dG, const float* U1, const float* U3, int64_t n,
                             float* dU1, float* dU3, hipStream_t st);

// Action-side SwiGLU fusion (sa_action.hip).
constexpr int kActionTypesMax = 16;
hipError_t launch_action_fwd(int d, int dtype, int64_t T, int n_types, const void* e,
                             const int32_t* types, const float* A, const float* W1,
                             const float* W3, const float* W2, void* prep, void* x,
                             hipStream_t st);
size_t action_prep_bytes(int d);
hipError_t launch_action_build_v(int d, int dtype, int64_t T, int n_types, const void* e,
                                 const int32_t* types, const float* A, float* V, hipStream_t st);
// Backward without V: the SwiGLU with the type rows added on the fly (bwd:
// dU1, dU3 from dG; fwd: G into out1), its intermediates fp32 or bf16
// (bf16_io); the per-type row sums of X [T, ncol] per block (part [nblk,
// n_types, ncol]).
hipError_t launch_action_swiglu(bool bwd, bool bf16_io, const void* dG, const void* U1,
                                const void* U3, const int32_t* types, const float* T1,
                                const float* T3, int n_types, int H, int64_t T, void* out1,
                                void* out3, hipStream_t st);
hipError_t launch_action_type_sums(bool bf16_in, const void* X, const int32_t* types, int n_types,
                                   int ncol, int64_t T, float* part, int nblk, hipStream_t st);
// mode 0: T1 = A W1a, T3 = A W3a; mode 1: dA = S1 W1a^T + S3 W3a^T and the
// action rows of dW1, dW3 (A^T S1, A^T S3).
hipError_t launch_action_small(int mode, int d, int n_types, const float* A, const float* W1,
                               const float* W3, const float* S1, const float* S3, float* T1,
                               float* T3, float* dA, float* dW1, float* dW3, hipStream_t st);

// Reordered single-query STCA attention core (sa_stca.hip).
// U, X: bf16 device arrays; C fp32, or bf16 when c_bf16.
hipError_t launch_stca_core(int D, int h, int B, const int64_t* x_off, const int64_t* t_off,
                            const void* U, const void* X, int64_t L, int64_t rows, void* C,
                            int c_bf16, float* lse, hipStream_t st);
hipError_t launch_to_bf16(const float* a, int64_t n, void* b, hipStream_t st);

// Argument blocks of the sketch kernels for a plan and a workspace (sa_api.cpp).
FwdArgs fwd_args(const Plan& p, char* ws, const int64_t* offsets, const void* X, const void* P,
                 int64_t pstride, float* S, float* lse, float* mass);
BwdArgs bwd_args(const Plan& p, char* ws, const int64_t* offsets, const void* X, const void* P,
                 int64_t pstride, const float* dS, const float* lse, const float* S,
                 const float* mass, float* dX, float* dP);
hipError_t launch_stats_f32(const FwdArgs& a, hipStream_t st, Prof* prof);
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st, Prof* prof);
// Single-pass forward (sa_fused_bf16.hip): the exchange clear, the fused
// kernel (cooperative launch) and the reduce.  An error means the fused
// kernel did not run.
hipError_t launch_fwd_fused_bf16(const FwdArgs& a, hipStream_t st, Prof* prof);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st, Prof* prof);
// keep_exchange_status: leave the second status word as the single-pass
// forward's kernel left it.  skip_single: users that lie in one segment were
// written to S (and mass) by the aggregation pass; leave them.
hipError_t launch_reduce(const FwdArgs& a, hipStream_t st, Prof* prof,
                         bool keep_exchange_status = false, bool skip_single = false);
// Token-wise normalisation (sa_tok.hip): S [B, k, d] and lse [B, k].
hipError_t launch_tok_fwd(const FwdArgs& a, int dtype, hipStream_t st, Prof* prof);
// out[u] = scale * sum of user u's piece partials (slot s + u of segment s of
// G), in piece order; also checks the offsets.  Per-user dP.
hipError_t launch_piece_sum(const int64_t* offsets, int B, int k, int d, int64_t T, int G,
                            const float* parts, float scale, float* out, uint32_t* status,
                            hipStream_t st, Prof* prof);
hipError_t launch_bwd(const BwdArgs& a, int dtype, hipStream_t st, Prof* prof);

}  // namespace sa
