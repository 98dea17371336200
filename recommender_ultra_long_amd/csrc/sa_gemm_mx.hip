// sa_gemm_mx.hip — dense products with fp32 operands rounded to bf16 on the
// matrix cores (fp32 accumulation).  They serve the products around the
// sketch whose inputs enter the matrix cores in bf16 anyway: the query, key
// and value projections of the single-query STCA attention (SequenceO1
// reading notes, section 5.1, Eq. (24)) and the backward of the action-side
// SwiGLU fusion (section 3.6, Eq. (20)) on bf16 histories.
//
// sa_gemm_mx<TA, TB, OBF>: C (+)= op(A) op(B) with
//   A(m, k) = TA ? A[k lda + m] : A[m lda + k],
//   B(k, n) = TB ? B[n ldb + k] : B[k ldb + n],
//   C fp32, or bf16 when OBF, row-major (ldc).
// With C0 (one slice, not accumulating) the output is C0 + op(A) op(B), C0
// laid out like C.
// blockIdx.z is either a batch index (zk = 0: A + z sA, B + z sB, all of K)
// or a reduction slice (zk = 1: k in [z kc, min((z + 1) kc, K))); either way
// the output goes to C + z sC.
// 64 x 64 output tile per workgroup of 4 waves (2 x 2 waves of 32 x 32), K in
// steps of 32.  The operands are staged in LDS as [row][k] bf16 (row stride 40
// elements, so 16 lanes reading one 16-byte column of 16 rows hit distinct
// banks); four K steps are in flight in registers meanwhile.  An operand
// stored [row][k] is loaded 8 k-values per lane and needs K % 32 == 0; one
// stored [k][row] is loaded as pairs of k rows, 4 values each, with the rows
// past the end of K read clamped and zeroed, so K is free there.  Rows of A
// (columns of C) past M (N) read row (column) 0 instead: they only feed
// outputs that are never stored, so no load is conditional.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

namespace {

constexpr int kMxTile = 64, kMxK = 32, kMxStride = 40, kMxPf = 4;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 to_bf16x8(const float4 a, const float4 b) {
  bf16x8 r;
  r[0] = (bf16)a.x; r[1] = (bf16)a.y; r[2] = (bf16)a.z; r[3] = (bf16)a.w;
  r[4] = (bf16)b.x; r[5] = (bf16)b.y; r[6] = (bf16)b.z; r[7] = (bf16)b.w;
  return r;
}

// One operand tile (64 rows x 32 k) of an fp32 (ST = float) or bf16 (ST =
// bf16) matrix, staged into LDS as [row][k] bf16.  KROW: the matrix is stored
// [k][row] (ld between k rows); otherwise [row][k] (ld between rows).  `rows`
// bounds the row index.
template <bool KROW, typename ST>
struct MxOperand {
  static constexpr bool B16 = sizeof(ST) == 2;
  const ST* base;      // this thread's first element (row clamped)
  int ld;
  int row_s, k_s;      // staging position: LDS row and first k of this thread
  float4 r[kMxPf][2];  // fp32 source
  bf16x4 rb[kMxPf][2]; // bf16 source, [k][row]: two k rows of 4 values
  bf16x8 rr[kMxPf];    // bf16 source, [row][k]: 8 k values

  __device__ void init(const ST* m, int ldm, int row0, int rows, int tid) {
    ld = ldm;
    if (KROW) {
      k_s = (tid >> 4) * 2;
      row_s = (tid & 15) * 4;
      const int row = row0 + row_s < rows ? row0 + row_s : 0;
      base = m + row;
    } else {
      row_s = tid >> 2;
      k_s = (tid & 3) * 8;
      const int row = row0 + row_s < rows ? row0 + row_s : 0;
      base = m + (int64_t)row * ld + k_s;
    }
  }
  // K step at k0 into stage s; k1 bounds k (KROW only: rows past it are 0).
  __device__ void load(int s, int k0, int k1) {
    if (KROW) {
      const int ka = k0 + k_s, kb = ka + 1;
      const int kac = ka < k1 ? ka : k1 - 1, kbc = kb < k1 ? kb : k1 - 1;
      if constexpr (B16) {
        const bf16x4 va = *(const bf16x4*)(base + (int64_t)kac * ld);
        const bf16x4 vb = *(const bf16x4*)(base + (int64_t)kbc * ld);
        rb[s][0] = ka < k1 ? va : bf16x4{};
        rb[s][1] = kb < k1 ? vb : bf16x4{};
      } else {
        const float4 va = *(const float4*)(base + (int64_t)kac * ld);
        const float4 vb = *(const float4*)(base + (int64_t)kbc * ld);
        const float4 z = {0.f, 0.f, 0.f, 0.f};
        r[s][0] = ka < k1 ? va : z;
        r[s][1] = kb < k1 ? vb : z;
      }
    } else {
      if constexpr (B16) {
        rr[s] = *(const bf16x8*)(base + k0);
      } else {
        r[s][0] = *(const float4*)(base + k0);
        r[s][1] = *(const float4*)(base + k0 + 4);
      }
    }
  }
  __device__ void store(int s, bf16* S) const {
    if (KROW) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x2 v;
        if constexpr (B16) {
          v[0] = rb[s][0][i];
          v[1] = rb[s][1][i];
        } else {
          const float x0[4] = {r[s][0].x, r[s][0].y, r[s][0].z, r[s][0].w};
          const float x1[4] = {r[s][1].x, r[s][1].y, r[s][1].z, r[s][1].w};
          v[0] = (bf16)x0[i];
          v[1] = (bf16)x1[i];
        }
        *(bf16x2*)&S[(row_s + i) * kMxStride + k_s] = v;
      }
    } else {
      if constexpr (B16) *(bf16x8*)&S[row_s * kMxStride + k_s] = rr[s];
      else *(bf16x8*)&S[row_s * kMxStride + k_s] = to_bf16x8(r[s][0], r[s][1]);
    }
  }
};

}  // namespace

template <bool TA, bool TB, bool OBF, typename AT = float, typename BT = float>
__global__ __launch_bounds__(256) void sa_gemm_mx(const AT* __restrict__ A, int lda, int64_t sA,
                                                  const BT* __restrict__ B, int ldb, int64_t sB,
                                                  void* __restrict__ Cv, int ldc, int64_t sC, int M,
                                                  int N, int K, int kc, int zk, int accumulate,
                                                  const float* __restrict__ C0) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][kMxTile * kMxStride];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][kMxTile * kMxStride];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int m0 = blockIdx.x * kMxTile, n0 = blockIdx.y * kMxTile;
  const int z = blockIdx.z;
  int kbeg = 0, kend = K;
  if (zk) {
    kbeg = z * kc;
    kend = kbeg + kc < K ? kbeg + kc : K;
  } else {
    A += (int64_t)z * sA;
    B += (int64_t)z * sB;
  }

  MxOperand<TA, AT> a;     // A stored [k][m] when TA
  MxOperand<!TB, BT> b;    // B stored [k][n] when !TB
  a.init(A, lda, m0, M, tid);
  b.init(B, ldb, n0, N, tid);

  f32x16 acc = f32x16{};
  const int nk = kend > kbeg ? (kend - kbeg + kMxK - 1) / kMxK : 0;
#pragma unroll
  for (int s = 0; s < kMxPf; ++s)
    if (s < nk) {
      a.load(s, kbeg + s * kMxK, kend);
      b.load(s, kbeg + s * kMxK, kend);
    }
  for (int kt0 = 0; kt0 < nk; kt0 += kMxPf) {
#pragma unroll
    for (int s = 0; s < kMxPf; ++s) {
      const int kt = kt0 + s;
      if (kt >= nk) break;
      const int buf = kt & 1;
      // Readers of this buffer (step kt - 2) finished before the barrier of
      // step kt - 1.
      a.store(s, As[buf]);
      b.store(s, Bs[buf]);
      __syncthreads();
      if (kt + kMxPf < nk) {
        a.load(s, kbeg + (kt + kMxPf) * kMxK, kend);
        b.load(s, kbeg + (kt + kMxPf) * kMxK, kend);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 av = *(const bf16x8*)&As[buf][(wm + l32) * kMxStride + 16 * ks + 8 * h];
        const bf16x8 bv = *(const bf16x8*)&Bs[buf][(wn + l32) * kMxStride + 16 * ks + 8 * h];
        acc = mfma32(av, bv, acc);
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
        const int64_t o = (int64_t)z * sC + (int64_t)m * ldc + n;
        if (OBF) {
          ((bf16*)Cv)[o] = (bf16)acc[i];
        } else {
          float* c = (float*)Cv + o;
          *c = accumulate ? *c + acc[i] : (C0 != nullptr ? C0[o] + acc[i] : acc[i]);
        }
      }
    }
  }
}

namespace {

hipError_t mx_dispatch(bool ta, bool tb, bool obf, dim3 grid, const float* A, int lda, int64_t sA,
                       const float* B, int ldb, int64_t sB, void* C, int ldc, int64_t sC, int M,
                       int N, int K, int kc, int zk, int accumulate, const float* C0,
                       hipStream_t st) {
#define SA_MX(TA_, TB_, OBF_)                                                                   \
  hipLaunchKernelGGL((sa_gemm_mx<TA_, TB_, OBF_>), grid, dim3(256), 0, st, A, lda, sA, B, ldb, \
                     sB, C, ldc, sC, M, N, K, kc, zk, accumulate, C0)
  if (obf) {
    if (ta || !tb) return hipErrorInvalidValue;   // bf16 output: the key product only
    SA_MX(false, true, true);
  } else if (!ta && !tb) SA_MX(false, false, false);
  else if (!ta && tb) SA_MX(false, true, false);
  else if (ta && !tb) SA_MX(true, false, false);
  else SA_MX(true, true, false);
#undef SA_MX
  return hipGetLastError();
}

// Operands stored [row][k] need K % 32 == 0 (per slice too); all rows must be
// 16-byte aligned, and so must the [k][row] operands' row extents.
bool mx_shape_ok(bool ta, bool tb, const float* A, int lda, int64_t sA, const float* B, int ldb,
                 int64_t sB, int M, int N, int K, int kc) {
  const bool rowk_a = !ta, rowk_b = tb;
  if ((rowk_a || rowk_b) && (K % kMxK != 0 || kc % kMxK != 0)) return false;
  if (ta && M % 4 != 0) return false;
  if (!tb && N % 4 != 0) return false;
  return lda % 4 == 0 && ldb % 4 == 0 && sA % 4 == 0 && sB % 4 == 0 &&
         ((uintptr_t)A & 15u) == 0 && ((uintptr_t)B & 15u) == 0;
}

}  // namespace

hipError_t launch_gemm_mx(bool tb, bool out_bf16, bool a_bf16, const void* A, int lda, int64_t sA,
                          const float* B, int ldb, int64_t sB, void* C, int ldc, int64_t sC, int M,
                          int N, int K, int batch, hipStream_t st) {
  if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
  if (batch > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((M + kMxTile - 1) / kMxTile), (unsigned)((N + kMxTile - 1) / kMxTile),
                  (unsigned)batch);
  if (a_bf16) {
    // bf16 A stored [row][k] (the STCA context): 16-byte aligned rows.
    if (tb || out_bf16 || K % kMxK != 0 || lda % 8 != 0 || sA % 8 != 0 ||
        ((uintptr_t)A & 15u) != 0 || N % 4 != 0 || ldb % 4 != 0 || sB % 4 != 0 ||
        ((uintptr_t)B & 15u) != 0)
      return hipErrorInvalidValue;
    hipLaunchKernelGGL((sa_gemm_mx<false, false, false, bf16, float>), grid, dim3(256), 0, st,
                       (const bf16*)A, lda, sA, B, ldb, sB, C, ldc, sC, M, N, K, K, 0, 0, nullptr);
    return hipGetLastError();
  }
  const float* Af = (const float*)A;
  if (!mx_shape_ok(false, tb, Af, lda, sA, B, ldb, sB, M, N, K, K)) return hipErrorInvalidValue;
  return mx_dispatch(false, tb, out_bf16, grid, Af, lda, sA, B, ldb, sB, C, ldc, sC, M, N, K, K, 0,
                     0, nullptr, st);
}

hipError_t launch_gemm_mx_sliced(bool ta, bool tb, const float* A, int lda, const float* B, int ldb,
                                 float* C, int ldc, int M, int N, int K, int slices, int accumulate,
                                 hipStream_t st, const float* init) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (slices < 1) slices = 1;
  int kc = (K + slices - 1) / slices;
  kc = (kc + kMxK - 1) / kMxK * kMxK;
  if (kc < kMxK) kc = kMxK;
  if (slices > 65535 || !mx_shape_ok(ta, tb, A, lda, 0, B, ldb, 0, M, N, K, slices > 1 ? kc : K) ||
      (init != nullptr && (slices != 1 || accumulate)))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((M + kMxTile - 1) / kMxTile), (unsigned)((N + kMxTile - 1) / kMxTile),
                  (unsigned)slices);
  return mx_dispatch(ta, tb, false, grid, A, lda, 0, B, ldb, 0, C, ldc, (int64_t)M * ldc, M, N, K,
                     kc, 1, accumulate, init, st);
}

// Operands in bf16 as well as fp32 (a_bf16, b_bf16) and a bf16 output
// (out_bf16), for the intermediates of the action-fusion backward; only the
// combinations it uses are built.  bf16 operands stored [row][k] need
// 16-byte aligned rows (ld % 8 == 0), those stored [k][row] 8-byte aligned
// rows.
hipError_t launch_gemm_mx_typed(bool ta, bool tb, bool a_bf16, bool b_bf16, bool out_bf16,
                                const void* A, int lda, const void* B, int ldb, void* C, int ldc,
                                int M, int N, int K, int slices, int accumulate, const float* init,
                                hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (slices < 1) slices = 1;
  int kc = (K + slices - 1) / slices;
  kc = (kc + kMxK - 1) / kMxK * kMxK;
  if (kc < kMxK) kc = kMxK;
  const int kcheck = slices > 1 ? kc : K;
  const bool rowk_a = !ta, rowk_b = tb;
  bool ok = slices <= 65535 && ((uintptr_t)A & 7u) == 0 && ((uintptr_t)B & 7u) == 0;
  if ((rowk_a || rowk_b) && (K % kMxK != 0 || kcheck % kMxK != 0)) ok = false;
  if (ta && M % 4 != 0) ok = false;
  if (!tb && N % 4 != 0) ok = false;
  if (lda % (a_bf16 && rowk_a ? 8 : 4) != 0 || ldb % (b_bf16 && rowk_b ? 8 : 4) != 0) ok = false;
  if ((!a_bf16 || rowk_a) && ((uintptr_t)A & 15u) != 0) ok = false;
  if ((!b_bf16 || rowk_b) && ((uintptr_t)B & 15u) != 0) ok = false;
  if (init != nullptr && (slices != 1 || accumulate || out_bf16)) ok = false;
  if (out_bf16 && (slices != 1 || accumulate)) ok = false;
  if (!ok) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((M + kMxTile - 1) / kMxTile), (unsigned)((N + kMxTile - 1) / kMxTile),
                  (unsigned)slices);
  const int64_t sC = (int64_t)M * ldc;
#define SA_MXT(TA_, TB_, OBF_, AT_, BT_)                                                         \
  hipLaunchKernelGGL((sa_gemm_mx<TA_, TB_, OBF_, AT_, BT_>), grid, dim3(256), 0, st,             \
                     (const AT_*)A, lda, 0, (const BT_*)B, ldb, 0, C, ldc, sC, M, N, K, kc, 1,     \
                     accumulate, init)
  if (!a_bf16 && !b_bf16 && !out_bf16)
    return mx_dispatch(ta, tb, false, grid, (const float*)A, lda, 0, (const float*)B, ldb, 0, C,
                       ldc, sC, M, N, K, kc, 1, accumulate, init, st);
  if (!ta && !tb && a_bf16 && !b_bf16 && out_bf16) SA_MXT(false, false, true, bf16, float);
  else if (!ta && tb && !a_bf16 && !b_bf16 && out_bf16) SA_MXT(false, true, true, float, float);
  else if (!ta && tb && a_bf16 && !b_bf16 && !out_bf16) SA_MXT(false, true, false, bf16, float);
  else if (ta && !tb && a_bf16 && !b_bf16 && !out_bf16) SA_MXT(true, false, false, bf16, float);
  else if (ta && !tb && a_bf16 && b_bf16 && !out_bf16) SA_MXT(true, false, false, bf16, bf16);
  else return hipErrorInvalidValue;
#undef SA_MXT
  return hipGetLastError();
}

}  // namespace sa
