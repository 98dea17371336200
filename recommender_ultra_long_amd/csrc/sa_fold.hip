// sa_fold.hip — folding the query and key projections of the affinities into
// the prototype table (SequenceO1 reading notes, section 3.1, Eq. (6):
// Z = (P W_Q)(X W_K)^T / sqrt(d) = (P W_Q W_K^T) X^T / sqrt(d)), and the
// backward of the fold.  With G = dL/dP_eff:
//   forward   Q = P W_Q,  P_eff = Q W_K^T
//   backward  dQ = G W_K,  dP = dQ W_Q^T,  dW_Q = P^T dQ,  dW_K = G^T Q
// (dW_Q = dM W_K and dW_K = dM^T W_Q for M = W_Q W_K^T and dM = P^T G,
// regrouped so that every product is k x d x d).
//
// The products are small (k x 128 x 128 with k in the thousands for a shared
// table; fp32 on the vector ALU):
// their cost is load latency and LDS reads, not arithmetic.  So every weight
// matrix is brought into LDS with one batch of loads (the second one
// prefetched into registers while the first product runs), and the row
// products work on tiles of 4 rows (8 at d = 32) so that k = 1024 spreads
// over 256 workgroups.
//
// Row kernels (grid = ceil(k / rows per tile)): each row of Q, dQ, P_eff and
// dP depends only on the same row of P and G.  The d x d gradients sum over all k rows:
// the gram kernel splits the rows into at most 256 slices (whole 128-row
// sub-chunks), one workgroup per (32 x 32 output tile, gradient, slice), and
// sa_fold_sum adds the slices in slice order, so results do not depend on
// scheduling.  The rows can be one shared table (k) or the stacked tables of
// all users (B k rows, one W_Q and W_K for all).
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

// Rows per row-kernel workgroup: as few as keep all 256 threads busy (one
// output column per thread and 256 / D rows per pass), at least 4, so that
// small k still spreads over many compute units.
template <int D>
constexpr int fold_rows() { return 256 / D > 4 ? 256 / D : 4; }
constexpr int kGramRows = 128;     // rows per gram sub-chunk (a slice is a whole number of them)
constexpr int kMaxSlices = 256;    // at most this many slices (partial sums) per gradient
constexpr int kGramTile = 32;      // gram output tile edge

template <int D>
struct FoldW {
  static constexpr int kPerThread = D * D / 4 / 256;   // float4 loads per thread
  float4 v[kPerThread > 0 ? kPerThread : 1];
};

// Issues the loads of a row-major D x D fp32 matrix into registers.
template <int D>
__device__ __forceinline__ void fetch_w(const float* __restrict__ W, FoldW<D>& r) {
  if constexpr (D * D / 4 >= 256) {
#pragma unroll
    for (int j = 0; j < FoldW<D>::kPerThread; ++j)
      r.v[j] = reinterpret_cast<const float4*>(W)[threadIdx.x + 256 * j];
  } else {
    if (threadIdx.x < D * D / 4) r.v[0] = reinterpret_cast<const float4*>(W)[threadIdx.x];
  }
}

// Stores the fetched matrix into LDS, sW[row][col] with row stride D + 1.
template <int D>
__device__ __forceinline__ void store_w(const FoldW<D>& r, float (*sW)[D + 1]) {
  constexpr int J = FoldW<D>::kPerThread > 0 ? FoldW<D>::kPerThread : 1;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i < D * D / 4) {
      const int e = 4 * i, row = e / D, col = e % D;
      sW[row][col] = r.v[j].x;
      sW[row][col + 1] = r.v[j].y;
      sW[row][col + 2] = r.v[j].z;
      sW[row][col + 3] = r.v[j].w;
    }
  }
}

// Rows r0 .. r0 + fold_rows<D>() - 1 of a k x D matrix into LDS as fp32
// (rows at or beyond k read as zero).
template <typename T, int D>
__device__ __forceinline__ void load_rows(const T* __restrict__ src, int r0, int k,
                                          float (*dst)[D + 4]) {
  for (int i = threadIdx.x; i < fold_rows<D>() * D; i += 256) {
    const int r = i / D, c = i % D;
    dst[r][c] = r0 + r < k ? (float)src[(int64_t)(r0 + r) * D + c] : 0.f;
  }
}

// acc[i] = sum_q In[rr + RS i][q] * (WT ? W[n][q] : W[q][n]) for the thread's
// column n = t % D and rows rr = t / D + RS i (RS = 256 / D).  Reads of In are
// broadcasts; reads of W hit consecutive banks across the lanes (W's row
// stride D + 1 keeps the transposed reads conflict-free too).
template <int D, bool WT>
__device__ __forceinline__ void rows_times_w(const float (*In)[D + 4], const float (*W)[D + 1],
                                             float* acc) {
  constexpr int RS = 256 / D, NR = fold_rows<D>() / RS;
  const int n = threadIdx.x % D, rr = threadIdx.x / D;
#pragma unroll
  for (int i = 0; i < NR; ++i) acc[i] = 0.f;
#pragma unroll 4
  for (int q = 0; q < D; q += 4) {
    float w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = WT ? W[n][q + j] : W[q + j][n];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float4 x = *reinterpret_cast<const float4*>(&In[rr + RS * i][q]);
      acc[i] = fmaf(x.x, w[0], acc[i]);
      acc[i] = fmaf(x.y, w[1], acc[i]);
      acc[i] = fmaf(x.z, w[2], acc[i]);
      acc[i] = fmaf(x.w, w[3], acc[i]);
    }
  }
}

// grid = ceil(k / fold_rows<D>()); block 256.  P_eff is written in OT (the
// sketch's input dtype), rounded once from the fp32 result.
template <typename PT, typename OT, int D>
__global__ __launch_bounds__(256) void sa_fold_fwd(const PT* __restrict__ P,
                                                   const float* __restrict__ Wq,
                                                   const float* __restrict__ Wk,
                                                   OT* __restrict__ Peff, int k) {
  constexpr int RB = fold_rows<D>(), RS = 256 / D, NR = RB / RS;
  __shared__ float sW[D][D + 1];
  __shared__ __align__(16) float sP[RB][D + 4];
  __shared__ __align__(16) float sQ[RB][D + 4];
  const int r0 = blockIdx.x * RB;
  const int n = threadIdx.x % D, rr = threadIdx.x / D;
  FoldW<D> wr;
  fetch_w<D>(Wq, wr);
  load_rows<PT, D>(P, r0, k, sP);
  store_w<D>(wr, sW);
  fetch_w<D>(Wk, wr);                                  // in flight during Q = P W_Q
  __syncthreads();
  float acc[NR];
  rows_times_w<D, false>(sP, sW, acc);                 // Q = P W_Q
#pragma unroll
  for (int i = 0; i < NR; ++i) sQ[rr + RS * i][n] = acc[i];
  __syncthreads();
  store_w<D>(wr, sW);
  __syncthreads();
  rows_times_w<D, true>(sQ, sW, acc);                  // P_eff = Q W_K^T
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = r0 + rr + RS * i;
    if (r < k) Peff[(int64_t)r * D + n] = (OT)acc[i];
  }
}

// grid = ceil(k / fold_rows<D>()); block 256.  Writes dP and the workspace rows
// Q = P W_Q and dQ = G W_K that the gram kernel reads.
template <typename PT, int D>
__global__ __launch_bounds__(256) void sa_fold_bwd_rows(const PT* __restrict__ P,
                                                        const float* __restrict__ Wq,
                                                        const float* __restrict__ Wk,
                                                        const float* __restrict__ G,
                                                        float* __restrict__ dP,
                                                        float* __restrict__ Qw,
                                                        float* __restrict__ dQw, int k) {
  constexpr int RB = fold_rows<D>(), RS = 256 / D, NR = RB / RS;
  __shared__ float sW[D][D + 1];
  __shared__ __align__(16) float sP[RB][D + 4];
  __shared__ __align__(16) float sG[RB][D + 4];
  __shared__ __align__(16) float sdQ[RB][D + 4];
  const int r0 = blockIdx.x * RB;
  const int n = threadIdx.x % D, rr = threadIdx.x / D;
  FoldW<D> wr;
  fetch_w<D>(Wk, wr);
  load_rows<float, D>(G, r0, k, sG);
  load_rows<PT, D>(P, r0, k, sP);
  store_w<D>(wr, sW);
  fetch_w<D>(Wq, wr);                                  // in flight during dQ = G W_K
  __syncthreads();
  float acc[NR];
  rows_times_w<D, false>(sG, sW, acc);                 // dQ = G W_K
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = rr + RS * i;
    sdQ[r][n] = acc[i];
    if (r0 + r < k) dQw[(int64_t)(r0 + r) * D + n] = acc[i];
  }
  __syncthreads();
  store_w<D>(wr, sW);
  __syncthreads();
  rows_times_w<D, false>(sP, sW, acc);                 // Q = P W_Q
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = r0 + rr + RS * i;
    if (r < k) Qw[(int64_t)r * D + n] = acc[i];
  }
  rows_times_w<D, true>(sdQ, sW, acc);                 // dP = dQ W_Q^T
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = r0 + rr + RS * i;
    if (r < k) dP[(int64_t)r * D + n] = acc[i];
  }
}

// grid = ((D / 32)^2, 2, slices); block 256.  blockIdx.y = 0: slice part of
// dW_Q = P^T dQ; 1: of dW_K = G^T Q.  Slice z is rows [z span, (z+1) span),
// taken in 128-row sub-chunks in order; the 32 x 32 output tile (a0, b0) sums
// them into parts[(z * 2 + y) * D * D + a * D + b].
template <typename PT, int D>
__global__ __launch_bounds__(256) void sa_fold_gram(const PT* __restrict__ P,
                                                    const float* __restrict__ G,
                                                    const float* __restrict__ Qw,
                                                    const float* __restrict__ dQw,
                                                    float* __restrict__ parts, int k, int span) {
  constexpr int T = kGramTile, TPR = D / T;
  __shared__ __align__(16) float sL[kGramRows][T + 4];
  __shared__ float sR[kGramRows][T + 1];
  const int a0 = (blockIdx.x / TPR) * T, b0 = (blockIdx.x % TPR) * T;
  const int which = blockIdx.y, z = blockIdx.z;
  const float* R = which == 0 ? dQw : Qw;
  constexpr int PER = kGramRows * T / 256;
  // thread t: output column b = t % T, rows a = 4 (t / T) .. + 3
  const int b = threadIdx.x % T, a = 4 * (threadIdx.x / T);
  static_assert(T * T / 256 == 4, "four outputs per thread");
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int end = (z + 1) * span < k ? (z + 1) * span : k;
  for (int row0 = z * span; row0 < end; row0 += kGramRows) {
    float lv[PER], rv[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = threadIdx.x + 256 * j, r = e / T, c = e % T;
      const bool in = row0 + r < end;
      const int64_t g = (int64_t)(row0 + r) * D;
      lv[j] = in ? (which == 0 ? (float)P[g + a0 + c] : G[g + a0 + c]) : 0.f;
      rv[j] = in ? R[g + b0 + c] : 0.f;
    }
    __syncthreads();   // the previous sub-chunk's LDS reads are done
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = threadIdx.x + 256 * j, r = e / T, c = e % T;
      sL[r][c] = lv[j];
      sR[r][c] = rv[j];
    }
    __syncthreads();
#pragma unroll 8
    for (int r = 0; r < kGramRows; ++r) {
      const float x = sR[r][b];
      const float4 l = *reinterpret_cast<const float4*>(&sL[r][a]);
      acc[0] = fmaf(l.x, x, acc[0]);
      acc[1] = fmaf(l.y, x, acc[1]);
      acc[2] = fmaf(l.z, x, acc[2]);
      acc[3] = fmaf(l.w, x, acc[3]);
    }
  }
  float* part = parts + (int64_t)(2 * z + which) * D * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) part[(int64_t)(a0 + a + i) * D + b0 + b] = acc[i];
}

// dW_Q and dW_K: the slices' parts added in slice order.
__global__ __launch_bounds__(256) void sa_fold_sum(const float* __restrict__ parts, int nslices,
                                                   int dd, float* __restrict__ dWq,
                                                   float* __restrict__ dWk) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * dd) return;
  const int which = i / dd, e = i % dd;
  float s = 0.f;
#pragma unroll 4
  for (int z = 0; z < nslices; ++z) s += parts[(int64_t)(2 * z + which) * dd + e];
  (which == 0 ? dWq : dWk)[e] = s;
}

template <int D>
static unsigned fold_row_blocks(int k) {
  return (unsigned)((k + fold_rows<D>() - 1) / fold_rows<D>());
}
// Rows per gram slice (a multiple of kGramRows, so that at most kMaxSlices
// slices cover k rows) and the number of slices.
static int fold_span(int k) {
  const int chunks = (k + kGramRows - 1) / kGramRows;
  const int ns = chunks < kMaxSlices ? chunks : kMaxSlices;
  return (chunks + ns - 1) / ns * kGramRows;
}
static int fold_slices(int k) { return (k + fold_span(k) - 1) / fold_span(k); }

template <typename PT, int D, typename OT = PT>
static hipError_t fold_t(int k, const void* P, const float* Wq, const float* Wk, void* Peff,
                         hipStream_t st) {
  hipLaunchKernelGGL((sa_fold_fwd<PT, OT, D>), dim3(fold_row_blocks<D>(k)), dim3(256), 0, st,
                     (const PT*)P, Wq, Wk, (OT*)Peff, k);
  return hipGetLastError();
}

hipError_t launch_fold_from_f32(int k, int d, int out_dtype, const float* P, const float* Wq,
                                const float* Wk, void* Peff, hipStream_t st) {
  switch (d) {
    case 32: return out_dtype == 1 ? fold_t<float, 32, bf16>(k, P, Wq, Wk, Peff, st)
                                   : fold_t<float, 32>(k, P, Wq, Wk, Peff, st);
    case 64: return out_dtype == 1 ? fold_t<float, 64, bf16>(k, P, Wq, Wk, Peff, st)
                                   : fold_t<float, 64>(k, P, Wq, Wk, Peff, st);
    case 128: return out_dtype == 1 ? fold_t<float, 128, bf16>(k, P, Wq, Wk, Peff, st)
                                    : fold_t<float, 128>(k, P, Wq, Wk, Peff, st);
  }
  return hipErrorInvalidValue;
}

template <typename PT, int D>
static hipError_t fold_backward_t(int k, const void* P, const float* Wq, const float* Wk,
                                  const float* G, float* dP, float* dWq, float* dWk, float* ws,
                                  hipStream_t st) {
  float* Qw = ws;
  float* dQw = Qw + (size_t)k * D;
  float* parts = dQw + (size_t)k * D;
  hipLaunchKernelGGL((sa_fold_bwd_rows<PT, D>), dim3(fold_row_blocks<D>(k)), dim3(256), 0, st,
                     (const PT*)P, Wq, Wk, G, dP, Qw, dQw, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ns = fold_slices(k);
  constexpr int tiles = (D / kGramTile) * (D / kGramTile);
  hipLaunchKernelGGL((sa_fold_gram<PT, D>), dim3(tiles, 2, (unsigned)ns), dim3(256), 0, st,
                     (const PT*)P, G, Qw, dQw, parts, k, fold_span(k));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sa_fold_sum, dim3((unsigned)((2 * D * D + 255) / 256)), dim3(256), 0, st,
                     parts, ns, D * D, dWq, dWk);
  return hipGetLastError();
}

hipError_t launch_fold(int k, int d, int dtype, const void* P, const float* Wq, const float* Wk,
                       void* Peff, hipStream_t st) {
  switch (d) {
    case 32: return dtype == 1 ? fold_t<bf16, 32>(k, P, Wq, Wk, Peff, st)
                               : fold_t<float, 32>(k, P, Wq, Wk, Peff, st);
    case 64: return dtype == 1 ? fold_t<bf16, 64>(k, P, Wq, Wk, Peff, st)
                               : fold_t<float, 64>(k, P, Wq, Wk, Peff, st);
    case 128: return dtype == 1 ? fold_t<bf16, 128>(k, P, Wq, Wk, Peff, st)
                                : fold_t<float, 128>(k, P, Wq, Wk, Peff, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fold_backward(int k, int d, int dtype, const void* P, const float* Wq,
                                const float* Wk, const float* G, float* dP, float* dWq,
                                float* dWk, float* ws, hipStream_t st) {
  switch (d) {
    case 32: return dtype == 1 ? fold_backward_t<bf16, 32>(k, P, Wq, Wk, G, dP, dWq, dWk, ws, st)
                               : fold_backward_t<float, 32>(k, P, Wq, Wk, G, dP, dWq, dWk, ws, st);
    case 64: return dtype == 1 ? fold_backward_t<bf16, 64>(k, P, Wq, Wk, G, dP, dWq, dWk, ws, st)
                               : fold_backward_t<float, 64>(k, P, Wq, Wk, G, dP, dWq, dWk, ws, st);
    case 128: return dtype == 1 ? fold_backward_t<bf16, 128>(k, P, Wq, Wk, G, dP, dWq, dWk, ws, st)
                                : fold_backward_t<float, 128>(k, P, Wq, Wk, G, dP, dWq, dWk, ws, st);
  }
  return hipErrorInvalidValue;
}

size_t fold_workspace_bytes(int k, int d) {
  return (2 * (size_t)k * d + 2 * (size_t)fold_slices(k) * d * d) * sizeof(float);
}

}  // namespace sa
