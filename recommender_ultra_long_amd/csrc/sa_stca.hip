// sa_stca.hip — the length-dependent core of the reordered single-query STCA
// attention (SequenceO1 reading notes, section 5.1, Eq. (24)-(25)).  For every
// (target r, head j) query row u = (q_r W_Q[:, j]) W_K[:, j]^T (width D, formed
// by sa_gemm_f32 beforehand), over the rows X_u of the target's user:
//     alpha = softmax(X_u u / sqrt(d_h)),   C[r, j] = alpha X_u   (width D)
// and then o[r, j] = C[r, j] W_V[:, j] (sa_gemm_f32 again).  The two
// reductions are 4 L D flops per query row, the whole length-dependent cost.
//
// sa_stca_core<DW>: one workgroup per 32 query rows, 8 waves; wave w owns the
// D-columns [w DW, (w+1) DW) (DW = D / 8).  Per 32-row tile of X:
//   - the wave copies its 32 x DW slice of the tile into its own LDS region
//     (the tile layout and swizzle of the sketch's aggregation), prefetched a
//     tile ahead in registers;
//   - partial scores S_w^T = X_w U_w^T on the matrix cores (lane = query row,
//     registers = history rows), exchanged through LDS and added in wave
//     order, so every wave holds the same full scores;
//   - online softmax per query row (a lane register), rescaled lazily as in
//     the token-wise sketch (weights below 2^8);
//   - C_w^T += X_w^T A^T with X_w^T read transposed from the wave's slice.
// Query rows of a tile may belong to several users: the tile streams each of
// those users' rows in turn, with the other users' rows masked (weight 0).
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

constexpr float kStcaTau = 8.0f;   // lazy rescale threshold, log2 units

// Last user whose first target is at or before target t (t_off[u] <= t).
// UNIFORM: t is the same in every lane (scalar loads); otherwise each lane
// searches with its own loads.
template <bool UNIFORM>
__device__ __forceinline__ int user_of_target(const int64_t* t_off, int B, int64_t t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int64_t v = UNIFORM ? uload64(t_off + mid) : t_off[mid];
    if (v <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// grid = ceil(rows / 32), rows = R h; block 512 (8 waves).
// U: [rows, D] bf16 (row r h + j), X: [L_total, D] bf16, C: [rows, D] fp32,
// lse: [rows] (natural log; -inf for a user without history rows).
template <int DW>
__global__ __launch_bounds__(512, 1) void sa_stca_core(const int64_t* __restrict__ x_off,
                                                      const int64_t* __restrict__ t_off, int B,
                                                      int h, const bf16* __restrict__ U,
                                                      const bf16* __restrict__ X, int64_t rows,
                                                      float alpha, float scale,
                                                      float* __restrict__ C,
                                                      float* __restrict__ lse) {
  constexpr int NW = 8;
  constexpr int D = DW * NW;
  constexpr int KS = DW / 16;              // K steps of the partial scores
  constexpr int DB = DW / 32;              // 32-row blocks of the wave's C^T
  constexpr int U16 = DW / 8;              // 16-byte units per slice row
  constexpr int CPL = 32 * U16 / 64;       // 16-byte copies per lane per tile
  __shared__ __attribute__((aligned(16))) bf16 sX[NW][32 * DW];
  __shared__ __attribute__((aligned(16))) f32x4 sS[2][NW][4][64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h2 = lane >> 5, l32 = lane & 31;
  const int64_t q0 = (int64_t)blockIdx.x * 32;
  const int64_t q = q0 + l32;                       // this lane's query row
  const bool qvalid = q < rows;
  const int c0 = wave * DW;                         // this wave's D-columns
  const uint32_t sx = lds_addr((const SA_LDS void*)&sX[wave][0]);
  const SA_LDS char* lds = (const SA_LDS char*)0;

  // The wave's query slice as B operands: ub[ks] = U[q][c0 + 16 ks + 8 h2 ..].
  bf16x8 ub[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    ub[ks] = qvalid ? *(const bf16x8*)(U + q * D + c0 + 16 * ks + 8 * h2) : bf16x8{};
  const int quser = qvalid ? user_of_target<false>(t_off, B, q / h) : -1;

  // LDS offsets within the slice (the aggregation tile layout with width DW).
  const int tr_r = (lane & 15) >> 2, tr_c = lane & 3, tr_half = (lane >> 4) & 1;
  uint32_t aoff[KS], toff[DB][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) aoff[ks] = (uint32_t)xoff<DW>(l32, 2 * ks + h2) * 2;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      toff[db][e] = (uint32_t)(xoff<DW>(4 * h2 + tr_r + 8 * e, 4 * db + 2 * tr_half + (tr_c >> 1)) +
                               (tr_c & 1) * 4) * 2;
  // Copy geometry: copy j of this lane moves unit v = lane + 64 j of the
  // slice (row v / U16, unit v % U16 of the wave's columns).
  auto fetch = [&](int64_t t0, int nr, bf16x8 (&reg)[CPL]) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int v = lane + 64 * j, r = v / U16, uu = v % U16;
      reg[j] = r < nr ? *(const bf16x8*)(X + (t0 + r) * D + c0 + 8 * uu) : bf16x8{};
    }
  };
  auto stash = [&](const bf16x8 (&reg)[CPL]) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int v = lane + 64 * j, r = v / U16, uu = v % U16;
      *(SA_LDS bf16x8*)(lds + sx + xoff<DW>(r, uu) * 2) = reg[j];
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float mrun = -INFINITY, lsum = 0.f;
  const float tau_raw = kStcaTau / alpha;
  uint32_t it = 0;                                  // tile counter (sS buffer parity)

  // Users of this tile's query rows (uniform over the workgroup).
  const int64_t qlast = (q0 + 31 < rows ? q0 + 31 : rows - 1);
  const int u_first = user_of_target<true>(t_off, B, q0 / h);
  const int u_last = user_of_target<true>(t_off, B, qlast / h);
  for (int u = u_first; u <= u_last; ++u) {
    if (uload64(t_off + u) == uload64(t_off + u + 1)) continue;   // no targets here
    const int64_t xlo = uload64(x_off + u), xhi = uload64(x_off + u + 1);
    const bool mine = quser == u;
    bf16x8 pre[CPL];
    if (xlo < xhi) fetch(xlo, (int)(xhi - xlo < 32 ? xhi - xlo : 32), pre);
    for (int64_t t0 = xlo; t0 < xhi; t0 += 32) {
      const int nr = (int)(xhi - t0 < 32 ? xhi - t0 : 32);
      stash(pre);                                   // this tile's slice (own region)
      __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): the slice is written
      if (t0 + 32 < xhi) fetch(t0 + 32, (int)(xhi - t0 - 32 < 32 ? xhi - t0 - 32 : 32), pre);
      // Partial S^T over this wave's columns: rows = history rows, lane = query.
      f32x16 sp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sp = mfma32(*(const SA_LDS bf16x8*)(lds + sx + aoff[ks]), ub[ks], sp);
      // X_w^T operands for the context product (rows 16 kb .. of the slice,
      // 32 DW bytes apart), read before the slice is overwritten.
      bf16x8 xt[2][DB];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          xt[kb][db] = concat4(
              lds_read_tr16((const SA_LDS bf16*)(lds + sx + toff[db][0] + kb * 32 * DW)),
              lds_read_tr16((const SA_LDS bf16*)(lds + sx + toff[db][1] + kb * 32 * DW)));
      // Exchange the partial scores; every wave adds them in wave order.
      const uint32_t pb = it & 1;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        sS[pb][wave][g][lane] = f32x4{sp[4 * g], sp[4 * g + 1], sp[4 * g + 2], sp[4 * g + 3]};
      __syncthreads();
      f32x16 s = f32x16{};
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = sS[pb][w][g][lane];
          s[4 * g] += v[0]; s[4 * g + 1] += v[1]; s[4 * g + 2] += v[2]; s[4 * g + 3] += v[3];
        }
      // Register i is history row crow(i, h2) of the tile.
      float tm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (!mine || crow(i, h2) >= nr) s[i] = -INFINITY;
        tm = fmaxf(tm, s[i]);
      }
      tm = fmaxf(tm, shfl_xor32(tm));
      const bool need = tm > mrun + tau_raw;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float mnew = need ? tm : mrun;
        const float f = mrun == -INFINITY ? 0.f : exp2_fast((mrun - mnew) * alpha);
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= f;
        lsum *= f;
        mrun = mnew;
      }
      const float ma = mrun == -INFINITY ? 0.f : mrun * alpha;
      bf16x8 abf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float a = exp2_fast(fmaf(s[8 * kb + j], alpha, -ma));
          lsum += a;
          abf[kb][j] = (bf16)a;
        }
      // C^T (columns x queries) += X_w^T (columns x rows) A^T (rows x queries).
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = mfma32(xt[kb][db], abf[kb], acc[db]);
      ++it;
    }
  }
  // Output: acc[db] register i is C[q][c0 + 32 db + crow(i, h2)] (unnormalised).
  const float L = lsum + shfl_xor32(lsum);
  if (qvalid) {
    const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = {acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv,
                         acc[db][4 * g + 3] * inv};
        *(f32x4*)(C + q * D + c0 + 32 * db + 8 * g + 4 * h2) = v;
      }
    if (wave == 0 && h2 == 0) lse[q] = L > 0.f ? mrun * scale + __logf(L) : -INFINITY;
  }
}

hipError_t launch_stca_core(int D, int h, int B, const int64_t* x_off, const int64_t* t_off,
                            const void* Uv, const void* Xv, int64_t rows, float* C, float* lse,
                            hipStream_t st) {
  const bf16* U = (const bf16*)Uv;
  const bf16* X = (const bf16*)Xv;
  if (rows <= 0) return hipSuccess;
  const int dh = D / h;
  const float scale = 1.0f / sqrtf((float)dh);
  const float alpha = scale * kLog2e;
  const dim3 grid((unsigned)((rows + 31) / 32));
  switch (D) {
    case 256: hipLaunchKernelGGL(sa_stca_core<32>, grid, dim3(512), 0, st, x_off, t_off, B, h, U, X, rows, alpha, scale, C, lse); break;
    case 512: hipLaunchKernelGGL(sa_stca_core<64>, grid, dim3(512), 0, st, x_off, t_off, B, h, U, X, rows, alpha, scale, C, lse); break;
    case 1024: hipLaunchKernelGGL(sa_stca_core<128>, grid, dim3(512), 0, st, x_off, t_off, B, h, U, X, rows, alpha, scale, C, lse); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// fp32 -> bf16 rows (the query rows u for the matrix cores).
__global__ __launch_bounds__(256) void sa_to_bf16(const float* __restrict__ a, int64_t n,
                                                  bf16* __restrict__ b) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) b[i] = (bf16)a[i];
}

hipError_t launch_to_bf16(const float* a, int64_t n, void* b, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sa_to_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a, n,
                     (bf16*)b);
  return hipGetLastError();
}

}  // namespace sa
