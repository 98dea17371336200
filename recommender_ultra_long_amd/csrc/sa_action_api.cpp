// sa_action_api.cpp — the action-side SwiGLU fusion of include/sa.h
// (SequenceO1 reading notes, section 3.6, Eq. (20)): validation, workspace
// layout and the launch sequence.  Host code only.
//
// bf16 histories: the fused matrix-core kernel of sa_action.hip forward; the
// backward on materialised intermediates with its products on the matrix
// cores (fp32 operands rounded to bf16, fp32 accumulation, sa_gemm_mx.hip).
// fp32 histories: fp32 arithmetic throughout, like the sketch's fp32 path
// (the fp32 products of sa_block.hip).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "sa.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr int kTypeBlocks = 256;      // event blocks of the per-type partial sums
constexpr int kMaxSlices = 64;        // reduction slices of a weight-gradient product

size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }

bool shape_ok(int d, int64_t T, int n_types) {
  return (d == 32 || d == 64 || d == 128) && T >= 0 && T <= ((int64_t)1 << 30) && n_types >= 1 &&
         n_types <= kActionTypesMax;
}

int slices_for(int64_t T) {
  const int64_t s = T / 512;
  return (int)(s < 1 ? 1 : (s > kMaxSlices ? kMaxSlices : s));
}

// Forward workspace (fp32 histories): V [T, 2d], U1, U3, G [T, H] (H = 2d), F
// [T, d].  Backward: U1' = e W1e, U3' = e W3e, G, dG, dU1, dU3 [T, H] (bf16
// for bf16 histories, fp32 otherwise), the weight-gradient slices, the
// per-type partial sums, S1, S3 (per-type sums of dU1, dU3) and T1, T3
// (= A W1a, A W3a).
struct ActionPlan {
  size_t prep, V, U1, U3, G, F, fwd_bf16, fwd_f32;
  size_t bU1, bU3, bG, bdG, bdU1, bdU3, bparts, btparts, bS1, bS3, bT1, bT3, bwd;
};

ActionPlan action_plan(int d, int64_t T, int n_types, int dtype) {
  ActionPlan p;
  memset(&p, 0, sizeof(p));
  const size_t Tn = (size_t)T, H = 2 * (size_t)d, nt = (size_t)n_types;
  size_t off = 0;
  p.prep = off; off = a256(off + action_prep_bytes(d));
  p.fwd_bf16 = off;
  const size_t base = off;
  p.V = off; off = a256(off + Tn * 2 * d * 4);
  p.U1 = off; off = a256(off + Tn * H * 4);
  p.U3 = off; off = a256(off + Tn * H * 4);
  p.G = off; off = a256(off + Tn * H * 4);
  p.F = off; off = a256(off + Tn * d * 4);
  p.fwd_f32 = off;
  off = base;
  const size_t es = dtype == SA_BF16 ? 2 : 4;     // intermediates' element size
  p.bU1 = off; off = a256(off + Tn * H * es);
  p.bU3 = off; off = a256(off + Tn * H * es);
  p.bG = off; off = a256(off + Tn * H * es);
  p.bdG = off; off = a256(off + Tn * H * es);
  p.bdU1 = off; off = a256(off + Tn * H * es);
  p.bdU3 = off; off = a256(off + Tn * H * es);
  p.bparts = off; off = a256(off + (size_t)slices_for(T) * d * H * 4);
  p.btparts = off; off = a256(off + (size_t)kTypeBlocks * nt * H * 4);
  p.bS1 = off; off = a256(off + nt * H * 4);
  p.bS3 = off; off = a256(off + nt * H * 4);
  p.bT1 = off; off = a256(off + nt * H * 4);
  p.bT3 = off; off = a256(off + nt * H * 4);
  p.bwd = off;
  return p;
}

bool a16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

#define SA_TRY(call)                            \
  do {                                          \
    const hipError_t e_ = (call);               \
    if (e_ != hipSuccess) return SA_ERR_HIP;    \
  } while (0)

// The products of the materialised path: fp32 operands rounded to bf16 on the
// matrix cores for bf16 histories (the sketch's own precision: bf16 in, fp32
// accumulate), fp32 on the vector ALU for fp32 histories.
hipError_t product(int dtype, bool ta, bool tb, const float* A, int lda, const float* B, int ldb,
                   float* C, int ldc, int M, int N, int K, int slices, int accumulate,
                   hipStream_t st) {
  if (dtype == SA_BF16)
    return launch_gemm_mx_sliced(ta, tb, A, lda, B, ldb, C, ldc, M, N, K, slices, accumulate, st);
  return launch_gemm(ta, tb, A, lda, B, ldb, C, ldc, M, N, K, slices, accumulate, st);
}

// U1 = V W1, U3 = V W3, G = silu(U1) U3 (fp32).
sa_status fp32_hidden(int d, int dtype, int64_t T, int n_types, const void* e,
                      const int32_t* types, const float* A, const float* W1, const float* W3,
                      char* w, const ActionPlan& p, hipStream_t st) {
  const int H = 2 * d;
  float* V = (float*)(w + p.V);
  SA_TRY(launch_action_build_v(d, dtype, T, n_types, e, types, A, V, st));
  SA_TRY(product(dtype, false, false, V, 2 * d, W1, H, (float*)(w + p.U1), H, (int)T, H, 2 * d, 1,
                 0, st));
  SA_TRY(product(dtype, false, false, V, 2 * d, W3, H, (float*)(w + p.U3), H, (int)T, H, 2 * d, 1,
                 0, st));
  SA_TRY(launch_swiglu_fwd((const float*)(w + p.U1), (const float*)(w + p.U3), T * H,
                           (float*)(w + p.G), st));
  return SA_OK;
}

}  // namespace
}  // namespace sa

using namespace sa;

extern "C" {

size_t sa_action_fusion_workspace_size(int d, sa_dtype dtype, int64_t T, int n_types, int op) {
  if (!shape_ok(d, T, n_types) || (dtype != SA_F32 && dtype != SA_BF16)) return 0;
  const ActionPlan p = action_plan(d, T, n_types, (int)dtype);
  if (op == SA_OP_FORWARD) return dtype == SA_BF16 ? p.fwd_bf16 : p.fwd_f32;
  if (op == SA_OP_BACKWARD) return p.bwd;
  return 0;
}

sa_status sa_action_fusion_forward(int d, sa_dtype dtype, int64_t T, int n_types, const void* e,
                                   const int32_t* types, const float* A, const float* W1,
                                   const float* W3, const float* W2, void* x, void* ws,
                                   size_t ws_bytes, void* stream) {
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_BAD_DTYPE;
  if (!shape_ok(d, T, n_types)) return SA_ERR_BAD_SHAPE;
  if (A == nullptr || W1 == nullptr || W3 == nullptr || W2 == nullptr || ws == nullptr)
    return SA_ERR_NULL_ARG;
  if (T > 0 && (e == nullptr || types == nullptr || x == nullptr)) return SA_ERR_NULL_ARG;
  if (!a16(A) || !a16(W1) || !a16(W3) || !a16(W2) || !a16(ws) || (e && !a16(e)) ||
      (x && !a16(x)) || (types && ((uintptr_t)types & 3u) != 0u))
    return SA_ERR_MISALIGNED;
  if (ws_bytes < sa_action_fusion_workspace_size(d, dtype, T, n_types, SA_OP_FORWARD))
    return SA_ERR_WORKSPACE_TOO_SMALL;
  const ActionPlan p = action_plan(d, T, n_types, (int)dtype);
  char* w = (char*)ws;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == SA_BF16) {
    SA_TRY(launch_action_fwd(d, 1, T, n_types, e, types, A, W1, W3, W2, w + p.prep, x, st));
    return SA_OK;
  }
  if (T == 0) return SA_OK;
  const sa_status v = fp32_hidden(d, 0, T, n_types, e, types, A, W1, W3, w, p, st);
  if (v != SA_OK) return v;
  float* F = (float*)(w + p.F);
  SA_TRY(launch_gemm(false, false, (const float*)(w + p.G), 2 * d, W2, d, F, d, (int)T, d, 2 * d, 1,
                     0, st));
  SA_TRY(launch_sum_slices(F, 1, T * d, (const float*)e, (float*)x, st));   // x = e + F
  return SA_OK;
}

sa_status sa_action_fusion_backward(int d, sa_dtype dtype, int64_t T, int n_types, const void* e,
                                    const int32_t* types, const float* A, const float* W1,
                                    const float* W3, const float* W2, const float* dx, float* de,
                                    float* dA, float* dW1, float* dW3, float* dW2, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_BAD_DTYPE;
  if (!shape_ok(d, T, n_types)) return SA_ERR_BAD_SHAPE;
  if (A == nullptr || W1 == nullptr || W3 == nullptr || W2 == nullptr || ws == nullptr ||
      dA == nullptr || dW1 == nullptr || dW3 == nullptr || dW2 == nullptr)
    return SA_ERR_NULL_ARG;
  if (T > 0 && (e == nullptr || types == nullptr || dx == nullptr || de == nullptr))
    return SA_ERR_NULL_ARG;
  const void* ptrs[] = {A, W1, W3, W2, ws, dA, dW1, dW3, dW2};
  for (const void* q : ptrs)
    if (!a16(q)) return SA_ERR_MISALIGNED;
  if ((e && !a16(e)) || (dx && !a16(dx)) || (de && !a16(de)) ||
      (types && ((uintptr_t)types & 3u) != 0u))
    return SA_ERR_MISALIGNED;
  if (ws_bytes < sa_action_fusion_workspace_size(d, dtype, T, n_types, SA_OP_BACKWARD))
    return SA_ERR_WORKSPACE_TOO_SMALL;
  const ActionPlan p = action_plan(d, T, n_types, (int)dtype);
  char* w = (char*)ws;
  hipStream_t st = (hipStream_t)stream;
  const int H = 2 * d, dt = (int)dtype, nt = n_types;
  const int ns = slices_for(T);
  // With V = [e | A[type]]: U1 = e W1e + T1[type] (T1 = A W1a), likewise U3;
  // de = dx + dU1 W1e^T + dU3 W3e^T; dA = S1 W1a^T + S3 W3a^T and
  // dW1 = [e^T dU1 ; A^T S1], dW3 likewise, with S1[t], S3[t] the sums of the
  // rows of dU1, dU3 over the events of type t.  V is never formed.  bf16
  // histories keep the [T, H] intermediates in bf16 and run every product on
  // the matrix cores; fp32 histories are fp32 throughout.
  const bool bf = dtype == SA_BF16;
  void* U1 = w + p.bU1;
  void* U3 = w + p.bU3;
  void* G = w + p.bG;
  void* dG = w + p.bdG;
  void* dU1 = w + p.bdU1;
  void* dU3 = w + p.bdU3;
  float* parts = (float*)(w + p.bparts);
  float* tparts = (float*)(w + p.btparts);
  float* S1 = (float*)(w + p.bS1);
  float* S3 = (float*)(w + p.bS3);
  float* T1 = (float*)(w + p.bT1);
  float* T3 = (float*)(w + p.bT3);
  // C (+)= op(A) op(B): typed matrix-core products for bf16 histories, fp32
  // vector-ALU products otherwise.
  auto prod = [&](bool ta, bool tb, bool abf, bool bbf, bool obf, const void* A_, int lda,
                  const void* B_, int ldb, void* C_, int ldc, int M, int N, int K, int sl,
                  int accumulate, const float* init) -> hipError_t {
    if (bf)
      return launch_gemm_mx_typed(ta, tb, abf, bbf, obf, A_, lda, B_, ldb, C_, ldc, M, N, K, sl,
                                  accumulate, init, st);
    if (init != nullptr) {
      const hipError_t e_ = launch_sum_slices(init, 1, (int64_t)M * N, nullptr, (float*)C_, st);
      if (e_ != hipSuccess) return e_;
      accumulate = 1;
    }
    return launch_gemm(ta, tb, (const float*)A_, lda, (const float*)B_, ldb, (float*)C_, ldc, M,
                       N, K, sl, accumulate, st);
  };
  SA_TRY(launch_action_small(0, d, nt, A, W1, W3, nullptr, nullptr, T1, T3, nullptr, nullptr,
                             nullptr, st));
  if (T > 0) {
    // U1' = e W1e, U3' = e W3e (rows 0 .. d-1 of W1, W3); G.
    SA_TRY(prod(false, false, bf, false, bf, e, d, W1, H, U1, H, (int)T, H, d, 1, 0, nullptr));
    SA_TRY(prod(false, false, bf, false, bf, e, d, W3, H, U3, H, (int)T, H, d, 1, 0, nullptr));
    SA_TRY(launch_action_swiglu(false, bf, nullptr, U1, U3, types, T1, T3, nt, H, T, G, nullptr,
                                st));
    // dG = dx W2^T; dU1, dU3.
    SA_TRY(prod(false, true, false, false, bf, dx, d, W2, d, dG, H, (int)T, H, d, 1, 0, nullptr));
    SA_TRY(launch_action_swiglu(true, bf, dG, U1, U3, types, T1, T3, nt, H, T, dU1, dU3, st));
    // de = dx + dU1 W1e^T + dU3 W3e^T.
    SA_TRY(prod(false, true, bf, false, false, dU1, H, W1, H, de, d, (int)T, d, H, 1, 0, dx));
    SA_TRY(prod(false, true, bf, false, false, dU3, H, W3, H, de, d, (int)T, d, H, 1, 1, nullptr));
  }
  // dW2 = G^T dx (zero without events).
  SA_TRY(prod(true, false, bf, false, false, G, H, dx, d, parts, d, H, d, (int)T, ns, 0, nullptr));
  SA_TRY(launch_sum_slices(parts, ns, (int64_t)H * d, nullptr, dW2, st));
  // S1, S3; dA and the action rows of dW1, dW3 (A^T S1, A^T S3).
  SA_TRY(launch_action_type_sums(bf, dU1, types, nt, H, T, tparts, kTypeBlocks, st));
  SA_TRY(launch_sum_slices(tparts, kTypeBlocks, (int64_t)nt * H, nullptr, S1, st));
  SA_TRY(launch_action_type_sums(bf, dU3, types, nt, H, T, tparts, kTypeBlocks, st));
  SA_TRY(launch_sum_slices(tparts, kTypeBlocks, (int64_t)nt * H, nullptr, S3, st));
  SA_TRY(launch_action_small(1, d, nt, A, W1, W3, S1, S3, nullptr, nullptr, dA, dW1, dW3, st));
  // The event rows of dW1, dW3: e^T dU1, e^T dU3.
  SA_TRY(prod(true, false, bf, bf, false, e, d, dU1, H, parts, H, d, H, (int)T, ns, 0, nullptr));
  SA_TRY(launch_sum_slices(parts, ns, (int64_t)d * H, nullptr, dW1, st));
  SA_TRY(prod(true, false, bf, bf, false, e, d, dU3, H, parts, H, d, H, (int)T, ns, 0, nullptr));
  SA_TRY(launch_sum_slices(parts, ns, (int64_t)d * H, nullptr, dW3, st));
  return SA_OK;
}

}  // extern "C"
