// sa_fwd_f32.hip — Sketch Attention forward with float32 inputs and float32
// arithmetic throughout (vector ALU; there is no reduced-precision step).
//
// Method: SequenceO1 reading notes, section 3.1, Eq. (6)-(9).  Same two-pass
// structure as the bf16 path: per-token log-sum-exp over all prototypes, then
// prototype-chunk aggregation per (segment, user) piece, then sa_reduce.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

// Log-sum-exp of the thread's token x over the k rows of table Pu, which the
// block streams through LDS 32 rows at a time (every thread of the block must
// call it).
template <int D>
__device__ float table_lse(const float* __restrict__ Pu, int k, const float (&x)[D], float alpha,
                           float scale, float (*sP)[D]) {
  constexpr int PC = 32;
  const int tid = threadIdx.x;
  float m = -INFINITY, l = 0.f;
  for (int p0 = 0; p0 < k; p0 += PC) {
    __syncthreads();
    for (int q = tid; q < PC * D; q += 256) {
      const int r = q / D, c = q % D;
      sP[r][c] = (p0 + r < k) ? Pu[(int64_t)(p0 + r) * D + c] : 0.f;
    }
    __syncthreads();
    const int np = k - p0 < PC ? k - p0 : PC;
    float z[PC];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < PC; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) acc = fmaf(sP[j][e], x[e], acc);
      z[j] = j < np ? acc : -INFINITY;
      tmax = fmaxf(tmax, z[j]);
    }
    const float mnew = fmaxf(m, tmax);
    const float ma = mnew * alpha;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < PC; ++j) s += exp2_fast(fmaf(z[j], alpha, -ma));
    l = fmaf(l, exp2_fast(fmaf(m, alpha, -ma)), s);
    m = mnew;
  }
  return m * scale + __logf(l);
}

// Pass 1: one token per thread, prototypes streamed through LDS 32 at a time.
// With one table per user (user u's table at P + u pstride, pstride != 0),
// the block makes one pass per user among its tokens and each token keeps
// the result of its own user's pass.
template <int D>
__global__ __launch_bounds__(256) void sa_stats_f32(const float* __restrict__ X,
                                                    const float* __restrict__ P, int k, int64_t T,
                                                    float alpha, float scale,
                                                    float* __restrict__ lse_out,
                                                    const int64_t* __restrict__ offsets, int B,
                                                    int64_t pstride) {
  __shared__ float sP[32][D];
  const int64_t b0 = (int64_t)blockIdx.x * 256;
  const int64_t b1 = b0 + 256 < T ? b0 + 256 : T;
  const int64_t tok = b0 + threadIdx.x;
  float x[D];
#pragma unroll
  for (int e = 0; e < D; ++e) x[e] = tok < T ? X[tok * D + e] : 0.f;
  if (pstride == 0) {
    const float v = table_lse<D>(P, k, x, alpha, scale, sP);
    if (tok < T) lse_out[tok] = v;
    return;
  }
  for (int u = first_user_after(offsets, B, b0);; ++u) {
    const int64_t ulo = clamp64(uload64(offsets + u), b0, b1);
    const int64_t uhi = clamp64(uload64(offsets + u + 1), ulo, b1);
    if (uhi > ulo) {
      // (table_lse starts every chunk with a barrier, so the previous pass's
      // LDS reads are done before sP is refilled)
      const float v = table_lse<D>(P + (int64_t)u * pstride, k, x, alpha, scale, sP);
      if (tok >= ulo && tok < uhi) lse_out[tok] = v;
    }
    if (uhi >= b1 || u + 1 >= B) break;
  }
}

// Pass 2: grid = (G, nchunks), block 256.  Workgroup owns 64 prototypes;
// thread t owns prototype t / 4 and columns (t % 4) D/4 .. +D/4 of U.  With
// one table per user, the workgroup's rows of it are reloaded at a user change.
template <int D>
__global__ __launch_bounds__(256) void sa_agg_f32(const int64_t* __restrict__ offsets, int B,
                                                  const float* __restrict__ X,
                                                  const float* __restrict__ P, int64_t pstride,
                                                  int k, int64_t T,
                                                  int G, float alpha,
                                                  const float* __restrict__ lse,
                                                  float* __restrict__ part,
                                                  float* __restrict__ pmass) {
  constexpr int PC = kChunkF32;   // 64
  constexpr int TILE = 32;
  constexpr int DQ = D / 4;
  __shared__ float sP[PC][D + 1];
  __shared__ float sX[TILE][D + 1];
  __shared__ float sA[PC][TILE + 1];
  __shared__ float sL[TILE];
  const int tid = threadIdx.x;
  const int j = tid >> 2, q = tid & 3;
  const int s = blockIdx.x;
  const int p0 = blockIdx.y * PC;

  const int64_t lo = seg_lo(T, G, s), hi = seg_lo(T, G, s + 1);
  TileWalker<TILE> cur;
  cur.start(offsets, B, lo, hi);

  float acc[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) acc[e] = 0.f;
  float ms = 0.f;
  int table = -1;   // user whose table is in sP (any user's, with a shared P)

  while (cur.valid) {
    __syncthreads();
    if (table < 0 || (pstride != 0 && cur.user != table)) {
      table = cur.user;
      const float* Pu = P + (int64_t)table * pstride;
      for (int i = tid; i < PC * D; i += 256) {
        const int r = i / D, c = i % D;
        sP[r][c] = (p0 + r < k) ? Pu[(int64_t)(p0 + r) * D + c] : 0.f;
      }
    }
    for (int i = tid; i < TILE * D; i += 256) {
      const int r = i / D, c = i % D;
      sX[r][c] = (cur.t0 + r < cur.t1) ? X[(cur.t0 + r) * D + c] : 0.f;
    }
    if (tid < TILE) sL[tid] = (cur.t0 + tid < cur.t1) ? lse[cur.t0 + tid] * kLog2e : INFINITY;
    __syncthreads();
    // 8 softmax weights per thread: prototype j, tokens 8q .. 8q+7.
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int tt = 8 * q + t;
      float z = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) z = fmaf(sP[j][e], sX[tt][e], z);
      const float a = exp2_fast(fmaf(z, alpha, -sL[tt]));
      sA[j][tt] = a;
      ms += a;
    }
    __syncthreads();
#pragma unroll 4
    for (int tt = 0; tt < TILE; ++tt) {
      const float a = sA[j][tt];
#pragma unroll
      for (int e = 0; e < DQ; ++e) acc[e] = fmaf(a, sX[tt][q * DQ + e], acc[e]);
    }
    if (cur.last_in_piece()) {
      const int64_t slot = (int64_t)s + cur.user;
      float mt = ms + __shfl_xor(ms, 1, 64);
      mt += __shfl_xor(mt, 2, 64);
      if (p0 + j < k) {
        float* dst = part + (slot * k + p0 + j) * D + q * DQ;
#pragma unroll
        for (int e = 0; e < DQ; ++e) dst[e] = acc[e];
        if (q == 0) pmass[slot * k + p0 + j] = mt;
      }
#pragma unroll
      for (int e = 0; e < DQ; ++e) acc[e] = 0.f;
      ms = 0.f;
    }
    cur.advance();
  }
}

template <int D>
static hipError_t launch_stats_f32_t(const FwdArgs& a, hipStream_t st, Prof* prof) {
  const float scale = 1.0f / sqrtf((float)D);
  const float alpha = scale * kLog2e;
  const unsigned nb = (unsigned)((a.T + 255) / 256);
  prof_begin(prof, "sa_stats_f32", st);
  hipLaunchKernelGGL(sa_stats_f32<D>, dim3(nb), dim3(256), 0, st, (const float*)a.X,
                     (const float*)a.P, a.k, a.T, alpha, scale, a.lse, a.offsets, a.B, a.pstride);
  const hipError_t e = hipGetLastError();
  prof_end(prof, st);
  return e;
}

template <int D>
static hipError_t launch_fwd_f32_t(const FwdArgs& a, hipStream_t st, Prof* prof) {
  const float scale = 1.0f / sqrtf((float)D);
  const float alpha = scale * kLog2e;
  if (a.T > 0) {
    hipError_t e = launch_stats_f32_t<D>(a, st, prof);
    if (e != hipSuccess) return e;
    prof_begin(prof, "sa_agg_f32", st);
    hipLaunchKernelGGL(sa_agg_f32<D>, dim3(a.G, a.nchunks), dim3(256), 0, st, a.offsets, a.B,
                       (const float*)a.X, (const float*)a.P, a.pstride, a.k, a.T, a.G, alpha,
                       a.lse, a.part, a.pmass);
    e = hipGetLastError();
    prof_end(prof, st);
    if (e != hipSuccess) return e;
  }
  return launch_reduce(a, st, prof);
}

hipError_t launch_stats_f32(const FwdArgs& a, hipStream_t st, Prof* prof) {
  if (a.T == 0) return hipSuccess;
  switch (a.d) {
    case 32: return launch_stats_f32_t<32>(a, st, prof);
    case 64: return launch_stats_f32_t<64>(a, st, prof);
    case 128: return launch_stats_f32_t<128>(a, st, prof);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st, Prof* prof) {
  switch (a.d) {
    case 32: return launch_fwd_f32_t<32>(a, st, prof);
    case 64: return launch_fwd_f32_t<64>(a, st, prof);
    case 128: return launch_fwd_f32_t<128>(a, st, prof);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
