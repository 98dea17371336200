// sa_stca_api.cpp — the reordered single-query STCA attention of include/sa.h
// (SequenceO1 reading notes, section 5.1, Eq. (24)) and the whole STCA layer
// of Eq. (26) around it: validation, workspace layout and the launch sequence
// (query projections, the length-dependent core, value projections; then the
// output projection and the query-side SwiGLU FFN).  Host code only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa.h"
#include "sa_kernels.h"

namespace sa {
namespace {

size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }

bool stca_shape_ok(int B, int D, int h, int64_t L, int64_t R) {
  return B >= 1 && (D == 256 || D == 512 || D == 1024) && h >= 1 && D % h == 0 && L >= 0 &&
         L < ((int64_t)1 << 34) && R >= 0 && (int64_t)R * h < ((int64_t)1 << 31) / 32 * 32;
}

// Qp [R, D] fp32 | Uf [R h, D] fp32 | U [R h, D] bf16 | C [R h, D] fp32 (or
// bf16) | lse [R h]
struct StcaPlan {
  size_t Qp, Uf, U, C, lse, total;
};

StcaPlan stca_plan(int D, int h, int64_t R) {
  StcaPlan p;
  const size_t rows = (size_t)R * h;
  size_t off = 0;
  p.Qp = off; off = a256(off + (size_t)R * D * 4);
  p.Uf = off; off = a256(off + rows * D * 4);
  p.U = off; off = a256(off + rows * D * 2);
  p.C = off; off = a256(off + rows * D * 4);
  p.lse = off; off = a256(off + rows * 4);
  p.total = off;
  return p;
}

bool a16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

#define SA_TRY(call)                            \
  do {                                          \
    const hipError_t e_ = (call);               \
    if (e_ != hipSuccess) return SA_ERR_HIP;    \
  } while (0)

}  // namespace
}  // namespace sa

using namespace sa;

extern "C" {

size_t sa_stca_workspace_size(int D, int h, int64_t R) {
  if (!stca_shape_ok(1, D, h, 0, R)) return 0;
  return stca_plan(D, h, R).total;
}

sa_status sa_stca_attention(int B, int D, int h, int64_t L, int64_t R, const int64_t* x_off,
                            const int64_t* t_off, const void* X, const float* Q, const float* Wq,
                            const float* Wk, const float* Wv, float* o, float* lse, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!stca_shape_ok(B, D, h, L, R)) return SA_ERR_BAD_SHAPE;
  if (x_off == nullptr || t_off == nullptr || Wq == nullptr || Wk == nullptr || Wv == nullptr ||
      ws == nullptr)
    return SA_ERR_NULL_ARG;
  if ((L > 0 && X == nullptr) || (R > 0 && (Q == nullptr || o == nullptr))) return SA_ERR_NULL_ARG;
  if (((uintptr_t)x_off & 7u) != 0u || ((uintptr_t)t_off & 7u) != 0u || !a16(Wq) || !a16(Wk) ||
      !a16(Wv) || !a16(ws) || (X && !a16(X)) || (Q && !a16(Q)) || (o && !a16(o)) ||
      (lse && !a16(lse)))
    return SA_ERR_MISALIGNED;
  const StcaPlan p = stca_plan(D, h, R);
  if (ws_bytes < p.total) return SA_ERR_WORKSPACE_TOO_SMALL;
  if (R == 0) return SA_OK;
  char* w = (char*)ws;
  hipStream_t st = (hipStream_t)stream;
  const int dh = D / h;
  const int64_t rows = R * h;
  float* Qp = (float*)(w + p.Qp);
  float* Uf = (float*)(w + p.Uf);
  float* C = (float*)(w + p.C);
  float* l = lse ? lse : (float*)(w + p.lse);
  // q W_Q, then per head u_j = (q W_Q)[:, j] W_K[:, j]^T (row r h + j of U),
  // all heads in one batched launch; o[:, j] = C[r, j] W_V[:, j] likewise.
  // Head widths that are multiples of 32 run on the matrix cores with the
  // operands rounded to bf16 (the precision the core consumes them in); other
  // widths use the fp32 products.
  if (dh % 32 == 0) {
    SA_TRY(launch_gemm_mx(false, false, false, Q, D, 0, Wq, D, 0, Qp, D, 0, (int)R, D, D, 1, st));
    SA_TRY(launch_gemm_mx(true, true, false, Qp, D, dh, Wk, D, dh, w + p.U, h * D, D, (int)R, D,
                          dh, h, st));
  } else {
    SA_TRY(launch_gemm(false, false, Q, D, Wq, D, Qp, D, (int)R, D, D, 1, 0, st));
    SA_TRY(launch_gemm_batched(false, true, Qp, D, dh, Wk, D, dh, Uf, h * D, D, (int)R, D, dh, h,
                               0, st));
    SA_TRY(launch_to_bf16(Uf, rows * D, w + p.U, st));
  }
  // The length-dependent core: C[r, j] = softmax(X_u u_j / sqrt(d_h)) X_u,
  // written in bf16 when the value product consumes it on the matrix cores.
  const bool mx = dh % 32 == 0;
  SA_TRY(launch_stca_core(D, h, B, x_off, t_off, w + p.U, X, L, rows, C, mx ? 1 : 0, l, st));
  if (mx)
    SA_TRY(launch_gemm_mx(false, false, true, C, h * D, D, Wv, D, dh, o, D, dh, (int)R, dh, D, h,
                          st));
  else
    SA_TRY(launch_gemm_batched(false, false, C, h * D, D, Wv, D, dh, o, D, dh, (int)R, dh, D, h,
                               0, st));
  return SA_OK;
}

// Workspace of the whole layer: the attention's, then o [R, D] (when the
// caller passes none), a [R, D], U1, U3, G [R, 2D], all fp32.
struct StcaLayerPlan {
  size_t attn, o, a, U1, U3, G, total;
};

static StcaLayerPlan stca_layer_plan(int D, int h, int64_t R) {
  StcaLayerPlan p;
  size_t off = 0;
  p.attn = off; off = a256(off + stca_plan(D, h, R).total);
  p.o = off; off = a256(off + (size_t)R * D * 4);
  p.a = off; off = a256(off + (size_t)R * D * 4);
  p.U1 = off; off = a256(off + (size_t)R * 2 * D * 4);
  p.U3 = off; off = a256(off + (size_t)R * 2 * D * 4);
  p.G = off; off = a256(off + (size_t)R * 2 * D * 4);
  p.total = off;
  return p;
}

size_t sa_stca_layer_workspace_size(int D, int h, int64_t R) {
  if (!stca_shape_ok(1, D, h, 0, R)) return 0;
  return stca_layer_plan(D, h, R).total;
}

sa_status sa_stca_layer(int B, int D, int h, int64_t L, int64_t R, const int64_t* x_off,
                        const int64_t* t_off, const void* X, const float* Q, const float* Wq,
                        const float* Wk, const float* Wv, const float* Wo, const float* W1,
                        const float* W3, const float* W2, float* y, float* o, float* lse,
                        void* ws, size_t ws_bytes, void* stream) {
  if (!stca_shape_ok(B, D, h, L, R)) return SA_ERR_BAD_SHAPE;
  if (Wo == nullptr || W1 == nullptr || W3 == nullptr || W2 == nullptr || ws == nullptr)
    return SA_ERR_NULL_ARG;
  if (R > 0 && y == nullptr) return SA_ERR_NULL_ARG;
  if (!a16(Wo) || !a16(W1) || !a16(W3) || !a16(W2) || !a16(ws) || (y && !a16(y)) ||
      (o && !a16(o)))
    return SA_ERR_MISALIGNED;
  const StcaLayerPlan p = stca_layer_plan(D, h, R);
  if (ws_bytes < p.total) return SA_ERR_WORKSPACE_TOO_SMALL;
  char* w = (char*)ws;
  float* ob = o ? o : (float*)(w + p.o);
  // The attention validates its own arguments (x_off, t_off, X, Q, W_Q, W_K,
  // W_V) before enqueueing anything.
  const sa_status v = sa_stca_attention(B, D, h, L, R, x_off, t_off, X, Q, Wq, Wk, Wv, ob, lse,
                                        w + p.attn, stca_plan(D, h, R).total, stream);
  if (v != SA_OK || R == 0) return v;
  hipStream_t st = (hipStream_t)stream;
  float* a = (float*)(w + p.a);
  float* U1 = (float*)(w + p.U1);
  float* U3 = (float*)(w + p.U3);
  float* G = (float*)(w + p.G);
  const int M = (int)R;
  // a = q + o W_O; U1 = a W1, U3 = a W3; G = silu(U1) * U3; y = a + G W2.
  // The products round their fp32 operands to bf16 on the matrix cores with
  // fp32 accumulation, as the attention's projections do.
  SA_TRY(launch_gemm_mx_sliced(false, false, ob, D, Wo, D, a, D, M, D, D, 1, 0, st, Q));
  SA_TRY(launch_gemm_mx_sliced(false, false, a, D, W1, 2 * D, U1, 2 * D, M, 2 * D, D, 1, 0, st));
  SA_TRY(launch_gemm_mx_sliced(false, false, a, D, W3, 2 * D, U3, 2 * D, M, 2 * D, D, 1, 0, st));
  SA_TRY(launch_swiglu_fwd(U1, U3, (int64_t)R * 2 * D, G, st));
  SA_TRY(launch_gemm_mx_sliced(false, false, G, 2 * D, W2, D, y, D, M, D, 2 * D, 1, 0, st, a));
  return SA_OK;
}

}  // extern "C"
