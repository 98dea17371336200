// sa_gemm_mx.hip — dense products with fp32 operands rounded to bf16 on the
// matrix cores (fp32 accumulation): the query, key and value projections of
// the single-query STCA attention (SequenceO1 reading notes, section 5.1,
// Eq. (24)), whose history and query rows enter its core in bf16 anyway.
//
// sa_gemm_mx<TB, OBF>: C[m][n] = sum_k A[m][k] B(k, n) for batch z, with
//   A row-major (lda), B(k, n) = TB ? B[n ldb + k] : B[k ldb + n],
//   A + z sA, B + z sB, C + z sC; C fp32 or (OBF) bf16, row-major (ldc).
// 64 x 64 output tile per workgroup of 4 waves (2 x 2 waves of 32 x 32), K in
// steps of 32.  The operands are staged in LDS as [row][k] bf16 (row stride 40
// elements, so 16 lanes reading one 16-byte column of 16 rows hit distinct
// banks); the next four K steps are in flight in registers meanwhile.
// Requires K % 32 == 0, 16-byte aligned rows (lda, ldb multiples of 4; N a
// multiple of 4 when TB is false) — the launcher checks and reports
// hipErrorInvalidValue otherwise.  M and N are bounds-checked.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

namespace {

constexpr int kMxTile = 64, kMxK = 32, kMxStride = 40;

__device__ __forceinline__ bf16x8 to_bf16x8(const float4 a, const float4 b) {
  bf16x8 r;
  r[0] = (bf16)a.x; r[1] = (bf16)a.y; r[2] = (bf16)a.z; r[3] = (bf16)a.w;
  r[4] = (bf16)b.x; r[5] = (bf16)b.y; r[6] = (bf16)b.z; r[7] = (bf16)b.w;
  return r;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

}  // namespace

template <bool TB, bool OBF>
__global__ __launch_bounds__(256) void sa_gemm_mx(const float* __restrict__ A, int lda, int64_t sA,
                                                  const float* __restrict__ B, int ldb, int64_t sB,
                                                  void* __restrict__ Cv, int ldc, int64_t sC, int M,
                                                  int N, int K) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][kMxTile * kMxStride];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][kMxTile * kMxStride];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int m0 = blockIdx.x * kMxTile, n0 = blockIdx.y * kMxTile;
  A += (int64_t)blockIdx.z * sA;
  B += (int64_t)blockIdx.z * sB;

  // Staging geometry.  A (and B when TB): thread -> row t / 4, k 8 (t % 4) ..
  // +7.  B when !TB: thread -> k rows 2 (t / 16), +1, columns 4 (t % 16) .. +3.
  const int ar = tid >> 2, ak = (tid & 3) * 8;
  const bool a_ok = m0 + ar < M;
  const float* ap = A + (int64_t)(a_ok ? m0 + ar : 0) * lda + ak;
  const int bkp = TB ? 0 : (tid >> 4) * 2, bn = TB ? 0 : (tid & 15) * 4;
  const bool b_ok = TB ? (n0 + ar < N) : (n0 + bn < N);
  const float* bp = TB ? B + (int64_t)(b_ok ? n0 + ar : 0) * ldb + ak
                       : B + (int64_t)bkp * ldb + (b_ok ? n0 + bn : 0);

  // NPF K steps in flight: register stage s holds K step kt while steps
  // kt + 1 .. kt + NPF - 1 load; LDS is double-buffered.
  constexpr int NPF = 4;
  float4 ra[NPF][2], rb[NPF][2];
  // Rows of A (columns of C) past M (N) read row (column) 0 instead: they only
  // feed outputs that are never stored, so no load is conditional.
  auto load = [&](int s, int k0) {
    ra[s][0] = *(const float4*)(ap + k0);
    ra[s][1] = *(const float4*)(ap + k0 + 4);
    if (TB) {
      rb[s][0] = *(const float4*)(bp + k0);
      rb[s][1] = *(const float4*)(bp + k0 + 4);
    } else {
      rb[s][0] = *(const float4*)(bp + (int64_t)k0 * ldb);
      rb[s][1] = *(const float4*)(bp + (int64_t)(k0 + 1) * ldb);
    }
  };
  auto store = [&](int s, int buf) {
    *(bf16x8*)&As[buf][ar * kMxStride + ak] = to_bf16x8(ra[s][0], ra[s][1]);
    if (TB) {
      *(bf16x8*)&Bs[buf][ar * kMxStride + ak] = to_bf16x8(rb[s][0], rb[s][1]);
    } else {
      const float x0[4] = {rb[s][0].x, rb[s][0].y, rb[s][0].z, rb[s][0].w};
      const float x1[4] = {rb[s][1].x, rb[s][1].y, rb[s][1].z, rb[s][1].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x2 v;
        v[0] = (bf16)x0[i];
        v[1] = (bf16)x1[i];
        *(bf16x2*)&Bs[buf][(bn + i) * kMxStride + bkp] = v;
      }
    }
  };

  f32x16 acc = f32x16{};
  const int nk = K / kMxK;
#pragma unroll
  for (int s = 0; s < NPF; ++s)
    if (s < nk) load(s, s * kMxK);
  for (int kt0 = 0; kt0 < nk; kt0 += NPF) {
#pragma unroll
    for (int s = 0; s < NPF; ++s) {
      const int kt = kt0 + s;
      if (kt >= nk) break;
      const int buf = kt & 1;
      // Readers of this buffer (step kt - 2) finished before the barrier of
      // step kt - 1.
      store(s, buf);
      __syncthreads();
      if (kt + NPF < nk) load(s, (kt + NPF) * kMxK);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = *(const bf16x8*)&As[buf][(wm + l32) * kMxStride + 16 * ks + 8 * h];
        const bf16x8 b = *(const bf16x8*)&Bs[buf][(wn + l32) * kMxStride + 16 * ks + 8 * h];
        acc = mfma32(a, b, acc);
      }
    }
  }
  // Register i holds C[wm + crow(i, h)][wn + l32].
  const int n = n0 + wn + l32;
  if (n < N) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + wm + crow(i, h);
      if (m < M) {
        const int64_t o = (int64_t)blockIdx.z * sC + (int64_t)m * ldc + n;
        if (OBF) ((bf16*)Cv)[o] = (bf16)acc[i];
        else ((float*)Cv)[o] = acc[i];
      }
    }
  }
}

hipError_t launch_gemm_mx(bool tb, bool out_bf16, const float* A, int lda, int64_t sA,
                          const float* B, int ldb, int64_t sB, void* C, int ldc, int64_t sC, int M,
                          int N, int K, int batch, hipStream_t st) {
  if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
  const bool shape_ok = K % kMxK == 0 && lda % 4 == 0 && ldb % 4 == 0 && sA % 4 == 0 &&
                        sB % 4 == 0 && (tb || N % 4 == 0) && batch <= 65535 &&
                        ((uintptr_t)A & 15u) == 0 && ((uintptr_t)B & 15u) == 0;
  if (!shape_ok) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((M + kMxTile - 1) / kMxTile), (unsigned)((N + kMxTile - 1) / kMxTile),
                  (unsigned)batch);
#define SA_MX(TB_, OBF_)                                                                        \
  hipLaunchKernelGGL((sa_gemm_mx<TB_, OBF_>), grid, dim3(256), 0, st, A, lda, sA, B, ldb, sB, C, \
                     ldc, sC, M, N, K)
  if (tb) {
    if (out_bf16) SA_MX(true, true);
    else SA_MX(true, false);
  } else {
    if (out_bf16) SA_MX(false, true);
    else SA_MX(false, false);
  }
#undef SA_MX
  return hipGetLastError();
}

}  // namespace sa
