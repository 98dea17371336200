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

constexpr int kDedABlocks = 256;      // event blocks of the per-type dA partial sums
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

// Workspace of the fp32 composition: V [T, 2d], U1, U3, G [T, 2d] (H = 2d),
// then F (forward) or dG, dU1, dU3, dV (backward), slices and dA partials.
struct ActionPlan {
  size_t prep, V, U1, U3, G, F, dG, dU1, dU3, dV, parts, dAparts, fwd_bf16, fwd_f32, bwd;
};

ActionPlan action_plan(int d, int64_t T, int n_types) {
  ActionPlan p;
  memset(&p, 0, sizeof(p));
  const size_t Tn = (size_t)T, H = 2 * (size_t)d;
  size_t off = 0;
  p.prep = off; off = a256(off + action_prep_bytes(d));
  p.fwd_bf16 = off;
  p.V = off; off = a256(off + Tn * 2 * d * 4);
  p.U1 = off; off = a256(off + Tn * H * 4);
  p.U3 = off; off = a256(off + Tn * H * 4);
  p.G = off; off = a256(off + Tn * H * 4);
  const size_t common = off;
  p.F = off; off = a256(off + Tn * d * 4);
  p.fwd_f32 = off;
  off = common;
  p.dG = off; off = a256(off + Tn * H * 4);
  p.dU1 = off; off = a256(off + Tn * H * 4);
  p.dU3 = off; off = a256(off + Tn * H * 4);
  p.dV = off; off = a256(off + Tn * 2 * d * 4);
  p.parts = off; off = a256(off + (size_t)slices_for(T) * 2 * d * H * 4);
  p.dAparts = off; off = a256(off + (size_t)kDedABlocks * n_types * d * 4);
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
  const ActionPlan p = action_plan(d, T, n_types);
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
  const ActionPlan p = action_plan(d, T, n_types);
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
  const ActionPlan p = action_plan(d, T, n_types);
  char* w = (char*)ws;
  hipStream_t st = (hipStream_t)stream;
  const int H = 2 * d;
  const int ns = slices_for(T);
  float* parts = (float*)(w + p.parts);
  if (T > 0) {
    const sa_status v = fp32_hidden(d, (int)dtype, T, n_types, e, types, A, W1, W3, w, p, st);
    if (v != SA_OK) return v;
  }
  const float* V = (const float*)(w + p.V);
  const float* U1 = (const float*)(w + p.U1);
  const float* U3 = (const float*)(w + p.U3);
  const float* G = (const float*)(w + p.G);
  float* dG = (float*)(w + p.dG);
  float* dU1 = (float*)(w + p.dU1);
  float* dU3 = (float*)(w + p.dU3);
  float* dV = (float*)(w + p.dV);
  const int dt = (int)dtype;
  // dG = dx W2^T; dW2 = G^T dx.
  SA_TRY(product(dt, false, true, dx, d, W2, d, dG, H, (int)T, H, d, 1, 0, st));
  SA_TRY(product(dt, true, false, G, H, dx, d, parts, d, H, d, (int)T, ns, 0, st));
  SA_TRY(launch_sum_slices(parts, ns, (int64_t)H * d, nullptr, dW2, st));
  // Through the SwiGLU; dV = dU1 W1^T + dU3 W3^T; dW1 = V^T dU1, dW3 = V^T dU3.
  SA_TRY(launch_swiglu_bwd(dG, U1, U3, T * H, dU1, dU3, st));
  SA_TRY(product(dt, false, true, dU1, H, W1, H, dV, 2 * d, (int)T, 2 * d, H, 1, 0, st));
  SA_TRY(product(dt, false, true, dU3, H, W3, H, dV, 2 * d, (int)T, 2 * d, H, 1, 1, st));
  SA_TRY(product(dt, true, false, V, 2 * d, dU1, H, parts, H, 2 * d, H, (int)T, ns, 0, st));
  SA_TRY(launch_sum_slices(parts, ns, (int64_t)2 * d * H, nullptr, dW1, st));
  SA_TRY(product(dt, true, false, V, 2 * d, dU3, H, parts, H, 2 * d, H, (int)T, ns, 0, st));
  SA_TRY(launch_sum_slices(parts, ns, (int64_t)2 * d * H, nullptr, dW3, st));
  // de = dx + dV[:, :d]; dA[t] = sum over events of type t of dV[:, d:].
  float* dAparts = (float*)(w + p.dAparts);
  SA_TRY(launch_action_dedA(d, T, n_types, dx, dV, types, de, dAparts, kDedABlocks, st));
  SA_TRY(launch_sum_slices(dAparts, kDedABlocks, (int64_t)n_types * d, nullptr, dA, st));
  return SA_OK;
}

}  // extern "C"
