// sa_block.hip — the dense pieces of the stacked Sketch Attention block
// (SequenceO1 reading notes, section 3.3, Eq. (15)-(16)): residual + layer
// normalisation, the SwiGLU FFN of hidden width 2d, and their backward.  The
// sketch itself and the query/key fold are the kernels of sa_fwd_*.hip,
// sa_bwd.hip and sa_fold.hip.
//
// Everything here is fp32 on the vector ALU.  These pieces act on the B k x d
// sketch rows, not on the history, so their work is a small fraction of the
// sketch's (12 k d^2 against 4 n k d flops per user and layer).
//
// Kernels
//  sa_gemm_f32<TA, TB>  C (+)= op(A) op(B), 64 x 64 tiles; blockIdx.z splits the
//                       reduction into slices written to separate outputs
//                       (added later in slice order, so sums are deterministic).
//  sa_sum_slices        out = init + sum over slices, in slice order.
//  sa_ln_fwd<D>         y = LN(a + res) per row, res broadcast over users when
//                       it is the shared table; saves mean and 1/std.
//  sa_ln_bwd<D>         dv = LN backward, per-workgroup partial dg, db.
//  sa_swiglu_fwd/bwd    G = silu(U1) U3 and its backward.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

constexpr float kLnEps = 1e-5f;

// ----------------------------------------------------------------------------
// C[m][n] (+)= sum_kk A(m, kk) B(kk, n), where
// A(m, kk) = TA ? A[kk lda + m] : A[m lda + kk] and
// B(kk, n) = TB ? B[n ldb + kk] : B[kk ldb + n].
// grid = (ceil(M / 64), ceil(N / 64), Z) (rows in x: M can be B k, far
// beyond the 65535 limit of y and z).  With zk = 1, z is a reduction slice:
// it covers kk in [z kc, (z + 1) kc) and writes C + z M ldc.  With zk = 0, z
// is a batch index: the product of A + z sA and B + z sB over all of K goes to
// C + z sC.  Thread (tx, ty) = (t % 16, t / 16) owns rows 4 ty .. +3 and
// columns 4 tx .. +3 of the tile.
template <bool TA, bool TB>
__global__ __launch_bounds__(256) void sa_gemm_f32(const float* __restrict__ A, int lda,
                                                   int64_t sA, const float* __restrict__ B,
                                                   int ldb, int64_t sB, float* __restrict__ C,
                                                   int ldc, int64_t sC, int M, int N, int K,
                                                   int kc, int zk, int accumulate) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ __align__(16) float As[2][BK][BM + 4];
  __shared__ __align__(16) float Bs[2][BK][BN + 4];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int k0 = zk ? (int)blockIdx.z * kc : 0;
  const int k1 = zk ? (k0 + kc < K ? k0 + kc : K) : K;
  A += (int64_t)blockIdx.z * sA;
  B += (int64_t)blockIdx.z * sB;
  C += (int64_t)blockIdx.z * sC;

  // Element e = tid + 256 i of a tile, laid out so that consecutive threads
  // read consecutive addresses of the source.
  float ra[4], rb[4];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int m = TA ? e % BM : e / BK, kk = TA ? e / BM : e % BK;
      const int gm = m0 + m, gk = kb + kk;
      ra[i] = (gm < M && gk < k1) ? (TA ? A[(int64_t)gk * lda + gm] : A[(int64_t)gm * lda + gk])
                                  : 0.f;
      const int n = TB ? e / BK : e % BN, kb2 = TB ? e % BK : e / BN;
      const int gn = n0 + n, gk2 = kb + kb2;
      rb[i] = (gn < N && gk2 < k1) ? (TB ? B[(int64_t)gn * ldb + gk2] : B[(int64_t)gk2 * ldb + gn])
                                   : 0.f;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int m = TA ? e % BM : e / BK, kk = TA ? e / BM : e % BK;
      As[buf][kk][m] = ra[i];
      const int n = TB ? e / BK : e % BN, kb2 = TB ? e % BK : e / BN;
      Bs[buf][kb2][n] = rb[i];
    }
  };

  float acc[4][4] = {};
  int buf = 0;
  if (k0 < k1) {
    fetch(k0);
    stash(0);
    __syncthreads();
  }
  for (int kb = k0; kb < k1; kb += BK) {
    const bool more = kb + BK < k1;
    if (more) fetch(kb + BK);                   // next tile in flight meanwhile
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(&As[buf][kk][4 * ty]);
      const float4 b = *reinterpret_cast<const float4*>(&Bs[buf][kk][4 * tx]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    if (more) {
      stash(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * ty + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 4 * tx + j;
      if (n < N) {
        float* c = C + (int64_t)m * ldc + n;
        *c = accumulate ? *c + acc[i][j] : acc[i][j];
      }
    }
  }
}

// out[i] = (init ? init[i] : 0) + sum_s parts[s n + i].  Four running sums
// take slices z = 4 m + r (r = 0..3, m increasing) and are combined as
// ((s0 + s1) + (s2 + s3)): a fixed order, so the result is deterministic, with
// four independent load/add chains per thread.
__global__ __launch_bounds__(256) void sa_sum_slices(const float* __restrict__ parts, int nslices,
                                                     int64_t n, const float* __restrict__ init,
                                                     float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  const float* p = parts + i;
  int z = 0;
  for (; z + 15 < nslices; z += 16) {   // sixteen loads in flight
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = p[(int64_t)(z + r) * n];
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      s0 += v[r];
      s1 += v[r + 1];
      s2 += v[r + 2];
      s3 += v[r + 3];
    }
  }
  for (; z + 3 < nslices; z += 4) {
    s0 += p[(int64_t)z * n];
    s1 += p[(int64_t)(z + 1) * n];
    s2 += p[(int64_t)(z + 2) * n];
    s3 += p[(int64_t)(z + 3) * n];
  }
  if (z < nslices) s0 += p[(int64_t)z * n];
  if (z + 1 < nslices) s1 += p[(int64_t)(z + 1) * n];
  if (z + 2 < nslices) s2 += p[(int64_t)(z + 2) * n];
  const float s = (s0 + s1) + (s2 + s3);
  out[i] = init != nullptr ? init[i] + s : s;
}

// ----------------------------------------------------------------------------
// Layer normalisation of v = a + res over the D features of a row (biased
// variance, eps 1e-5), y = (v - mean) rstd g + b.  res row r % res_rows is
// added (the shared table broadcast over users when res_rows = k).  One wave
// per row, four rows per block.
template <int D>
__global__ __launch_bounds__(256) void sa_ln_fwd(const float* __restrict__ a,
                                                 const float* __restrict__ res, int64_t res_rows,
                                                 int64_t R, const float* __restrict__ g,
                                                 const float* __restrict__ b,
                                                 float* __restrict__ y, float* __restrict__ mean_out,
                                                 float* __restrict__ rstd_out) {
  constexpr int E = (D + 63) / 64;       // features per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;                  // whole wave; no barriers below
  const float* ar = a + row * D;
  const float* rr = res + (row % res_rows) * D;
  float v[E];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < D ? ar[e] + rr[e] : 0.f;
    s += v[i];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  const float mean = s * (1.0f / D);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int e = lane + 64 * i;
    const float c = e < D ? v[i] - mean : 0.f;
    q = fmaf(c, c, q);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) q += __shfl_xor(q, off, 64);
  const float rstd = 1.0f / sqrtf(q * (1.0f / D) + kLnEps);
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int e = lane + 64 * i;
    if (e < D) y[row * D + e] = (v[i] - mean) * rstd * g[e] + b[e];
  }
  if (lane == 0) {
    mean_out[row] = mean;
    rstd_out[row] = rstd;
  }
}

// Backward of sa_ln_fwd.  With xhat = (v - mean) rstd and h = dy g:
//   dv = rstd (h - mean(h) - xhat mean(h xhat))   (added to dv when acc_dv)
// and this block's partial sums over its rows of dy xhat (-> dg) and dy
// (-> db), written to part[blockIdx.x D + e] and part[(nblk + blockIdx.x) D + e].
// Block b owns rows [b rpb, (b + 1) rpb); wave w takes rows w, w + 4, ...; the
// four waves' partials are added in wave order.
template <int D>
__global__ __launch_bounds__(256) void sa_ln_bwd(const float* __restrict__ dy,
                                                 const float* __restrict__ a,
                                                 const float* __restrict__ res, int64_t res_rows,
                                                 int64_t R, int64_t rpb,
                                                 const float* __restrict__ mean,
                                                 const float* __restrict__ rstd,
                                                 const float* __restrict__ g,
                                                 float* __restrict__ dv, int acc_dv,
                                                 float* __restrict__ part) {
  constexpr int E = (D + 63) / 64;
  __shared__ float red[2][4][64 * E];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * rpb;
  const int64_t r1 = r0 + rpb < R ? r0 + rpb : R;
  float pg[E], pb[E], gv[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int e = lane + 64 * i;
    pg[i] = 0.f;
    pb[i] = 0.f;
    gv[i] = e < D ? g[e] : 0.f;
  }
  for (int64_t row = r0 + wave; row < r1; row += 4) {
    const float mu = mean[row], rs = rstd[row];
    const float* ar = a + row * D;
    const float* rr = res + (row % res_rows) * D;
    float xh[E], h[E];
    float sh = 0.f, shx = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int e = lane + 64 * i;
      const bool in = e < D;
      const float d = in ? dy[row * D + e] : 0.f;
      xh[i] = in ? (ar[e] + rr[e] - mu) * rs : 0.f;
      h[i] = d * gv[i];
      sh += h[i];
      shx = fmaf(h[i], xh[i], shx);
      pg[i] = fmaf(d, xh[i], pg[i]);
      pb[i] += d;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      sh += __shfl_xor(sh, off, 64);
      shx += __shfl_xor(shx, off, 64);
    }
    const float mh = sh * (1.0f / D), mhx = shx * (1.0f / D);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int e = lane + 64 * i;
      if (e < D) {
        const float v = rs * (h[i] - mh - xh[i] * mhx);
        float* dst = dv + row * D + e;
        *dst = acc_dv ? *dst + v : v;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < E; ++i) {
    red[0][wave][lane + 64 * i] = pg[i];
    red[1][wave][lane + 64 * i] = pb[i];
  }
  __syncthreads();
  const int nblk = gridDim.x;
  for (int e = threadIdx.x; e < D; e += 256) {
    part[(int64_t)blockIdx.x * D + e] = ((red[0][0][e] + red[0][1][e]) + red[0][2][e]) + red[0][3][e];
    part[(int64_t)(nblk + blockIdx.x) * D + e] =
        ((red[1][0][e] + red[1][1][e]) + red[1][2][e]) + red[1][3][e];
  }
}

// ----------------------------------------------------------------------------
// SwiGLU: G = silu(U1) U3 with silu(u) = u s(u), s the logistic function.
__device__ __forceinline__ float logistic(float u) { return 1.0f / (1.0f + __expf(-u)); }

__global__ __launch_bounds__(256) void sa_swiglu_fwd(const float* __restrict__ U1,
                                                     const float* __restrict__ U3, int64_t n,
                                                     float* __restrict__ G) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float u = U1[i];
  G[i] = u * logistic(u) * U3[i];
}

// dU1 = dG U3 s (1 + u (1 - s)),  dU3 = dG u s.
__global__ __launch_bounds__(256) void sa_swiglu_bwd(const float* __restrict__ dG,
                                                     const float* __restrict__ U1,
                                                     const float* __restrict__ U3, int64_t n,
                                                     float* __restrict__ dU1,
                                                     float* __restrict__ dU3) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float u = U1[i], s = logistic(u), d = dG[i];
  dU1[i] = d * U3[i] * s * (1.0f + u * (1.0f - s));
  dU3[i] = d * u * s;
}

// ----------------------------------------------------------------------------
// Launchers.
static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

namespace {

hipError_t gemm_dispatch(bool ta, bool tb, dim3 grid, const float* A, int lda, int64_t sA,
                         const float* B, int ldb, int64_t sB, float* C, int ldc, int64_t sC, int M,
                         int N, int K, int kc, int zk, int accumulate, hipStream_t st) {
#define SA_GEMM_LAUNCH(TA_, TB_)                                                                  \
  hipLaunchKernelGGL((sa_gemm_f32<TA_, TB_>), grid, dim3(256), 0, st, A, lda, sA, B, ldb, sB, C, \
                     ldc, sC, M, N, K, kc, zk, accumulate)
  if (!ta && !tb) SA_GEMM_LAUNCH(false, false);
  else if (!ta && tb) SA_GEMM_LAUNCH(false, true);
  else if (ta && !tb) SA_GEMM_LAUNCH(true, false);
  else SA_GEMM_LAUNCH(true, true);
#undef SA_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(bool ta, bool tb, const float* A, int lda, const float* B, int ldb,
                       float* C, int ldc, int M, int N, int K, int slices, int accumulate,
                       hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (slices < 1) slices = 1;
  int kc = (K + slices - 1) / slices;
  kc = (kc + 15) / 16 * 16;
  const dim3 grid((unsigned)((M + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)slices);
  return gemm_dispatch(ta, tb, grid, A, lda, 0, B, ldb, 0, C, ldc, (int64_t)M * ldc, M, N, K, kc,
                       1, accumulate, st);
}

hipError_t launch_gemm_batched(bool ta, bool tb, const float* A, int lda, int64_t sA,
                               const float* B, int ldb, int64_t sB, float* C, int ldc, int64_t sC,
                               int M, int N, int K, int batch, int accumulate, hipStream_t st) {
  if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
  if (batch > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((M + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)batch);
  return gemm_dispatch(ta, tb, grid, A, lda, sA, B, ldb, sB, C, ldc, sC, M, N, K, K, 0, accumulate,
                       st);
}

hipError_t launch_sum_slices(const float* parts, int nslices, int64_t n, const float* init,
                             float* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sa_sum_slices, dim3(blocks_for(n)), dim3(256), 0, st, parts, nslices, n,
                     init, out);
  return hipGetLastError();
}

hipError_t launch_ln_fwd(int d, const float* a, const float* res, int64_t res_rows, int64_t R,
                         const float* g, const float* b, float* y, float* mean, float* rstd,
                         hipStream_t st) {
  if (R <= 0) return hipSuccess;
  const dim3 grid((unsigned)((R + 3) / 4));
  switch (d) {
    case 32: hipLaunchKernelGGL(sa_ln_fwd<32>, grid, dim3(256), 0, st, a, res, res_rows, R, g, b, y, mean, rstd); break;
    case 64: hipLaunchKernelGGL(sa_ln_fwd<64>, grid, dim3(256), 0, st, a, res, res_rows, R, g, b, y, mean, rstd); break;
    case 128: hipLaunchKernelGGL(sa_ln_fwd<128>, grid, dim3(256), 0, st, a, res, res_rows, R, g, b, y, mean, rstd); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_ln_bwd(int d, const float* dy, const float* a, const float* res,
                         int64_t res_rows, int64_t R, const float* mean, const float* rstd,
                         const float* g, float* dv, int acc_dv, float* part, int nblk,
                         hipStream_t st) {
  if (R <= 0) return hipSuccess;
  const int64_t rpb = (R + nblk - 1) / nblk;
  switch (d) {
    case 32: hipLaunchKernelGGL(sa_ln_bwd<32>, dim3(nblk), dim3(256), 0, st, dy, a, res, res_rows, R, rpb, mean, rstd, g, dv, acc_dv, part); break;
    case 64: hipLaunchKernelGGL(sa_ln_bwd<64>, dim3(nblk), dim3(256), 0, st, dy, a, res, res_rows, R, rpb, mean, rstd, g, dv, acc_dv, part); break;
    case 128: hipLaunchKernelGGL(sa_ln_bwd<128>, dim3(nblk), dim3(256), 0, st, dy, a, res, res_rows, R, rpb, mean, rstd, g, dv, acc_dv, part); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const float* U1, const float* U3, int64_t n, float* G,
                             hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sa_swiglu_fwd, dim3(blocks_for(n)), dim3(256), 0, st, U1, U3, n, G);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* dG, const float* U1, const float* U3, int64_t n,
                             float* dU1, float* dU3, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sa_swiglu_bwd, dim3(blocks_for(n)), dim3(256), 0, st, dG, U1, U3, n, dU1,
                     dU3);
  return hipGetLastError();
}

}  // namespace sa
