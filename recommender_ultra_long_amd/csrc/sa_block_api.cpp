// sa_block_api.cpp — the stacked Sketch Attention block of include/sa.h
// (SequenceO1 reading notes, section 3.3, Eq. (12)-(16)): workspace layout and
// the sequence of kernel launches of its forward and backward.  Host code
// only; the kernels are those of sa_fold.hip, sa_fwd_*.hip, sa_bwd.hip and
// sa_block.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "sa.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr int kMaxLayers = 8;
constexpr int kLnBlocks = 256;       // row blocks of the layer-norm backward (partial sums)
constexpr int kMaxWeightSlices = 64; // reduction slices of a weight-gradient product

size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }

// Byte offsets of one layer's saved activations.
struct LayerBufs {
  size_t peff;            // folded queries, [rows, d] in the sketch dtype
  size_t lse;             // [T]
  size_t xh;              // sketch X^, [R, d]
  size_t xbar;            // LN1 output, [R, d]
  size_t F;               // FFN output, [R, d]
  size_t out;             // LN2 output (the next layer's queries), [R, d]; not the last layer's
  size_t u1, u3;          // x W1, x W3, [R, 2d]
  size_t mean1, rstd1, mean2, rstd2;   // [R]
};

struct BlockPlan {
  Plan sa;                // the sketch's plan with per-user tables (the larger workspace)
  int L;
  int64_t R;              // B k sketch rows
  LayerBufs lay[kMaxLayers];
  // temporaries (used by the forward's FFN and by the backward)
  size_t G, dG, dU1, dU3, dxbar, dr1, dq, dpeff, dqf, fold_ws, wparts, lnparts;
  int wslices;
  size_t total;
};

bool block_plan(const sa_problem* pr, int L, BlockPlan* bp) {
  if (L < 1 || L > kMaxLayers) return false;
  memset(bp, 0, sizeof(*bp));
  if (!make_plan(pr->batch, pr->k, pr->d, pr->total_tokens, (int)pr->dtype, false, true, &bp->sa))
    return false;
  const int B = pr->batch, k = pr->k, d = pr->d;
  const size_t T = (size_t)pr->total_tokens;
  const size_t esz = pr->dtype == SA_BF16 ? 2 : 4;
  bp->L = L;
  bp->R = (int64_t)B * k;
  if (bp->R > (1 << 24)) return false;      // the fold's row limit
  const size_t Rd = (size_t)bp->R * d * 4, R2d = 2 * Rd, R4 = (size_t)bp->R * 4;
  // The sketch's own workspace comes first, so that its status word is the
  // block workspace's first word (sa_get_device_status).
  size_t off = a256(bp->sa.fwd_bytes > bp->sa.bwd_bytes ? bp->sa.fwd_bytes : bp->sa.bwd_bytes);
  for (int l = 0; l < L; ++l) {
    LayerBufs& b = bp->lay[l];
    const size_t rows = l == 0 ? (size_t)k : (size_t)bp->R;
    b.peff = off; off = a256(off + rows * d * esz);
    b.lse = off; off = a256(off + T * 4);
    b.xh = off; off = a256(off + Rd);
    b.xbar = off; off = a256(off + Rd);
    b.F = off; off = a256(off + Rd);
    if (l + 1 < L) { b.out = off; off = a256(off + Rd); }
    b.u1 = off; off = a256(off + R2d);
    b.u3 = off; off = a256(off + R2d);
    b.mean1 = off; off = a256(off + R4);
    b.rstd1 = off; off = a256(off + R4);
    b.mean2 = off; off = a256(off + R4);
    b.rstd2 = off; off = a256(off + R4);
  }
  bp->G = off; off = a256(off + R2d);
  bp->dG = off; off = a256(off + R2d);
  bp->dU1 = off; off = a256(off + R2d);
  bp->dU3 = off; off = a256(off + R2d);
  bp->dxbar = off; off = a256(off + Rd);
  bp->dr1 = off; off = a256(off + Rd);
  bp->dq = off; off = a256(off + Rd);
  bp->dpeff = off; off = a256(off + Rd);
  bp->dqf = off; off = a256(off + Rd);
  bp->fold_ws = off; off = a256(off + fold_workspace_bytes((int)bp->R, d));
  int ws = (int)(bp->R / 512);
  bp->wslices = ws < 1 ? 1 : (ws > kMaxWeightSlices ? kMaxWeightSlices : ws);
  bp->wparts = off; off = a256(off + (size_t)bp->wslices * 2 * d * d * 4);
  bp->lnparts = off; off = a256(off + (size_t)2 * kLnBlocks * d * 4);
  bp->total = off;
  return true;
}

bool a16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

// The FFN products of Eq. (16) and their gradients: fp32 operands rounded to
// bf16 on the matrix cores when the sketch runs in bf16 (bf16 in, fp32
// accumulate, as the sketch), fp32 on the vector ALU otherwise.
hipError_t product(int dtype, bool ta, bool tb, const float* A, int lda, const float* B, int ldb,
                   float* C, int ldc, int M, int N, int K, int slices, int accumulate,
                   hipStream_t st) {
  if (dtype == SA_BF16)
    return launch_gemm_mx_sliced(ta, tb, A, lda, B, ldb, C, ldc, M, N, K, slices, accumulate, st);
  return launch_gemm(ta, tb, A, lda, B, ldb, C, ldc, M, N, K, slices, accumulate, st);
}

sa_status check_common(const sa_problem* pr, int L, const int64_t* offsets, const void* X,
                       const float* P0, const sa_block_layer* layers, void* ws) {
  const sa_status v = sa_validate(pr, nullptr);
  if (v != SA_OK) return v;
  if (pr->flags != 0u || L < 1 || L > kMaxLayers) return SA_ERR_UNSUPPORTED;
  if (offsets == nullptr || P0 == nullptr || layers == nullptr || ws == nullptr)
    return SA_ERR_NULL_ARG;
  if (X == nullptr && pr->total_tokens > 0) return SA_ERR_NULL_ARG;
  for (int l = 0; l < L; ++l) {
    const sa_block_layer& p = layers[l];
    const void* ptrs[] = {p.Wq, p.Wk, p.ln1_g, p.ln1_b, p.W1, p.W3, p.W2, p.ln2_g, p.ln2_b};
    for (const void* q : ptrs) {
      if (q == nullptr) return SA_ERR_NULL_ARG;
      if (!a16(q)) return SA_ERR_MISALIGNED;
    }
  }
  if (((uintptr_t)offsets & 7u) != 0u || (X && !a16(X)) || !a16(P0) || !a16(ws))
    return SA_ERR_MISALIGNED;
  return SA_OK;
}

#define SA_TRY(call)                            \
  do {                                          \
    const hipError_t e_ = (call);               \
    if (e_ != hipSuccess) return SA_ERR_HIP;    \
  } while (0)

}  // namespace
}  // namespace sa

using namespace sa;

extern "C" {

size_t sa_block_workspace_size(const sa_problem* pr, int n_layers) {
  if (sa_validate(pr, nullptr) != SA_OK || pr->flags != 0u) return 0;
  BlockPlan bp;
  if (!block_plan(pr, n_layers, &bp)) return 0;
  return bp.total;
}

sa_status sa_block_forward(const sa_problem* pr, int L, const int64_t* offsets, const void* X,
                           const float* P0, const sa_block_layer* layers, float* out, void* ws,
                           size_t ws_bytes, void* stream) {
  sa_status v = check_common(pr, L, offsets, X, P0, layers, ws);
  if (v != SA_OK) return v;
  if (out == nullptr) return SA_ERR_NULL_ARG;
  if (!a16(out)) return SA_ERR_MISALIGNED;
  BlockPlan bp;
  if (!block_plan(pr, L, &bp)) return SA_ERR_BAD_SHAPE;
  if (ws_bytes < bp.total) return SA_ERR_WORKSPACE_TOO_SMALL;

  char* w = (char*)ws;
  hipStream_t st = (hipStream_t)stream;
  const int k = pr->k, d = pr->d, dt = (int)pr->dtype;
  const int64_t R = bp.R;
  const float* q = P0;                 // this layer's queries: the shared table, then per user
  int64_t q_rows = k;
  for (int l = 0; l < L; ++l) {
    const LayerBufs& b = bp.lay[l];
    const sa_block_layer& p = layers[l];
    float* xh = (float*)(w + b.xh);
    float* xbar = (float*)(w + b.xbar);
    float* F = (float*)(w + b.F);
    float* u1 = (float*)(w + b.u1);
    float* u3 = (float*)(w + b.u3);
    float* G = (float*)(w + bp.G);
    float* y = l + 1 < L ? (float*)(w + b.out) : out;
    // Eq. (12): the folded queries X~ W_Q W_K^T, in the sketch dtype.
    SA_TRY(launch_fold_from_f32((int)q_rows, d, dt, q, p.Wq, p.Wk, w + b.peff, st));
    // Eq. (13)-(14): the plain-sum sketch, per-user tables after layer 0.
    const FwdArgs a = fwd_args(bp.sa, w, offsets, X, w + b.peff, l == 0 ? 0 : (int64_t)k * d, xh,
                               (float*)(w + b.lse), nullptr);
    SA_TRY(dt == 1 ? launch_fwd_bf16(a, st, nullptr) : launch_fwd_f32(a, st, nullptr));
    // Eq. (15): LN1(X~ + X^); layer 0's X~ is the shared table, row j % k.
    SA_TRY(launch_ln_fwd(d, xh, q, q_rows, R, p.ln1_g, p.ln1_b, xbar, (float*)(w + b.mean1),
                         (float*)(w + b.rstd1), st));
    // Eq. (16): LN2(X- + FFN(X-)), FFN = (silu(X- W1) * (X- W3)) W2.
    SA_TRY(product(dt, false, false, xbar, d, p.W1, 2 * d, u1, 2 * d, (int)R, 2 * d, d, 1, 0, st));
    SA_TRY(product(dt, false, false, xbar, d, p.W3, 2 * d, u3, 2 * d, (int)R, 2 * d, d, 1, 0, st));
    SA_TRY(launch_swiglu_fwd(u1, u3, R * 2 * d, G, st));
    SA_TRY(product(dt, false, false, G, 2 * d, p.W2, d, F, d, (int)R, d, 2 * d, 1, 0, st));
    SA_TRY(launch_ln_fwd(d, xbar, F, R, R, p.ln2_g, p.ln2_b, y, (float*)(w + b.mean2),
                         (float*)(w + b.rstd2), st));
    q = y;
    q_rows = R;
  }
  return SA_OK;
}

sa_status sa_block_backward(const sa_problem* pr, int L, const int64_t* offsets, const void* X,
                            const float* P0, const sa_block_layer* layers, const float* dout,
                            float* dX, float* dP0, const sa_block_layer_grad* grads, void* ws,
                            size_t ws_bytes, void* stream) {
  sa_status v = check_common(pr, L, offsets, X, P0, layers, ws);
  if (v != SA_OK) return v;
  if (dout == nullptr || dP0 == nullptr || grads == nullptr) return SA_ERR_NULL_ARG;
  if (dX == nullptr && pr->total_tokens > 0) return SA_ERR_NULL_ARG;
  if (!a16(dout) || !a16(dP0) || (dX && !a16(dX))) return SA_ERR_MISALIGNED;
  for (int l = 0; l < L; ++l) {
    const sa_block_layer_grad& g = grads[l];
    const void* ptrs[] = {g.Wq, g.Wk, g.ln1_g, g.ln1_b, g.W1, g.W3, g.W2, g.ln2_g, g.ln2_b};
    for (const void* q : ptrs) {
      if (q == nullptr) return SA_ERR_NULL_ARG;
      if (!a16(q)) return SA_ERR_MISALIGNED;
    }
  }
  BlockPlan bp;
  if (!block_plan(pr, L, &bp)) return SA_ERR_BAD_SHAPE;
  if (ws_bytes < bp.total) return SA_ERR_WORKSPACE_TOO_SMALL;

  char* w = (char*)ws;
  hipStream_t st = (hipStream_t)stream;
  const int B = pr->batch, k = pr->k, d = pr->d, dt = (int)pr->dtype;
  const int64_t R = bp.R;
  float* G = (float*)(w + bp.G);
  float* dG = (float*)(w + bp.dG);
  float* dU1 = (float*)(w + bp.dU1);
  float* dU3 = (float*)(w + bp.dU3);
  float* dxbar = (float*)(w + bp.dxbar);
  float* dr1 = (float*)(w + bp.dr1);
  float* dqbuf = (float*)(w + bp.dq);
  float* dpeff = (float*)(w + bp.dpeff);
  float* dqf = (float*)(w + bp.dqf);
  float* wparts = (float*)(w + bp.wparts);
  float* lnparts = (float*)(w + bp.lnparts);
  const int ns = bp.wslices;

  const float* dq = dout;              // dL/d(this layer's output)
  for (int l = L - 1; l >= 0; --l) {
    const LayerBufs& b = bp.lay[l];
    const sa_block_layer& p = layers[l];
    const sa_block_layer_grad& g = grads[l];
    const float* q = l == 0 ? P0 : (const float*)(w + bp.lay[l - 1].out);
    const int64_t q_rows = l == 0 ? k : R;
    const float* xh = (const float*)(w + b.xh);
    const float* xbar = (const float*)(w + b.xbar);
    const float* F = (const float*)(w + b.F);
    const float* u1 = (const float*)(w + b.u1);
    const float* u3 = (const float*)(w + b.u3);

    // LN2: dxbar = dL/d(X- + F) for now; dg2, db2.
    SA_TRY(launch_ln_bwd(d, dq, xbar, F, R, R, (const float*)(w + b.mean2),
                         (const float*)(w + b.rstd2), p.ln2_g, dxbar, 0, lnparts, kLnBlocks, st));
    SA_TRY(launch_sum_slices(lnparts, kLnBlocks, d, nullptr, g.ln2_g, st));
    SA_TRY(launch_sum_slices(lnparts + (size_t)kLnBlocks * d, kLnBlocks, d, nullptr, g.ln2_b, st));
    // FFN: dG = dF W2^T, dW2 = G^T dF (G recomputed), then the SwiGLU.
    SA_TRY(launch_swiglu_fwd(u1, u3, R * 2 * d, G, st));
    SA_TRY(product(dt, false, true, dxbar, d, p.W2, d, dG, 2 * d, (int)R, 2 * d, d, 1, 0, st));
    SA_TRY(product(dt, true, false, G, 2 * d, dxbar, d, wparts, d, 2 * d, d, (int)R, ns, 0, st));
    SA_TRY(launch_sum_slices(wparts, ns, (int64_t)2 * d * d, nullptr, g.W2, st));
    SA_TRY(launch_swiglu_bwd(dG, u1, u3, R * 2 * d, dU1, dU3, st));
    SA_TRY(product(dt, true, false, xbar, d, dU1, 2 * d, wparts, 2 * d, d, 2 * d, (int)R, ns, 0, st));
    SA_TRY(launch_sum_slices(wparts, ns, (int64_t)2 * d * d, nullptr, g.W1, st));
    SA_TRY(product(dt, true, false, xbar, d, dU3, 2 * d, wparts, 2 * d, d, 2 * d, (int)R, ns, 0, st));
    SA_TRY(launch_sum_slices(wparts, ns, (int64_t)2 * d * d, nullptr, g.W3, st));
    // dL/dX- = dF (residual) + dU1 W1^T + dU3 W3^T.
    SA_TRY(product(dt, false, true, dU1, 2 * d, p.W1, 2 * d, dxbar, d, (int)R, d, 2 * d, 1, 1, st));
    SA_TRY(product(dt, false, true, dU3, 2 * d, p.W3, 2 * d, dxbar, d, (int)R, d, 2 * d, 1, 1, st));
    // LN1: dr1 = dL/d(X~ + X^); dg1, db1.
    SA_TRY(launch_ln_bwd(d, dxbar, xh, q, q_rows, R, (const float*)(w + b.mean1),
                         (const float*)(w + b.rstd1), p.ln1_g, dr1, 0, lnparts, kLnBlocks, st));
    SA_TRY(launch_sum_slices(lnparts, kLnBlocks, d, nullptr, g.ln1_g, st));
    SA_TRY(launch_sum_slices(lnparts + (size_t)kLnBlocks * d, kLnBlocks, d, nullptr, g.ln1_b, st));
    // The sketch: dS = dr1 -> dX (added over layers) and dL/dP_eff.
    BwdArgs a = bwd_args(bp.sa, w, offsets, X, w + b.peff, l == 0 ? 0 : (int64_t)k * d, dr1,
                         (const float*)(w + b.lse), nullptr, nullptr, dX, dpeff);
    a.acc_dx = l == L - 1 ? 0 : 1;
    SA_TRY(launch_bwd(a, dt, st, nullptr));
    // The fold: dL/dX~ through P_eff, and dW_Q, dW_K.
    SA_TRY(launch_fold_backward((int)q_rows, d, 0, q, p.Wq, p.Wk, dpeff, dqf, g.Wq, g.Wk,
                                (float*)(w + bp.fold_ws), st));
    // The residual of Eq. (15): X~ enters LN1 directly.  Layer 0's X~ is the
    // shared table, so its gradient sums over users.
    if (l > 0) {
      SA_TRY(launch_sum_slices(dr1, 1, R * d, dqf, dqbuf, st));
      dq = dqbuf;
    } else {
      SA_TRY(launch_sum_slices(dr1, B, (int64_t)k * d, dqf, dP0, st));
    }
  }
  return SA_OK;
}

}  // extern "C"
