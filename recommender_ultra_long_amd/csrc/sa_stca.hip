// sa_stca.hip — the length-dependent core of the reordered single-query STCA
// attention (SequenceO1 reading notes, section 5.1, Eq. (24)-(25)).  For every
// (target r, head j) query row u = (q_r W_Q[:, j]) W_K[:, j]^T (width D, formed
// by the projection products beforehand: sa_gemm_mx on the matrix cores, or
// the fp32 sa_gemm_f32 when d_h is not a multiple of 32), over the rows X_u
// of the target's user:
//     alpha = softmax(X_u u / sqrt(d_h)),   C[r, j] = alpha X_u   (width D)
// and then o[r, j] = C[r, j] W_V[:, j] (a projection product again).  The two
// reductions are 4 L D flops per query row, the whole length-dependent cost.
//
// sa_stca_core<DW>: one workgroup per 32 query rows, 8 waves; wave w owns the
// D-columns [w DW, (w+1) DW) (DW = D / 8) of the context product and the
// softmax of query rows 4w .. 4w+3.  Per 32-row tile of X:
//   - the wave copies its 32 x DW slice of the tile into its own LDS region
//     (the tile layout and swizzle of the sketch's aggregation), prefetched a
//     tile ahead in registers;
//   - partial scores S_w^T = X_w U_w^T on the matrix cores (lane = query row,
//     registers = history rows), written to LDS;
//   - reduce-scatter: wave w adds the 8 partials of its 4 query rows (in wave
//     order), keeps their online-softmax state (running maximum, rescaled
//     lazily when it grows past 2^8, and running sum) and publishes bf16
//     weights and the rescale factor of each of its rows;
//   - every wave reads the 32 x 32 weight tile back as the B operand of
//     C_w^T += X_w^T A^T, with X_w^T read transposed from the wave's slice.
// Query rows of a tile may belong to several users: the tile streams each of
// those users' rows in turn, with the other users' rows masked (weight 0).
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

constexpr float kStcaTau = 8.0f;   // lazy rescale threshold, log2 units

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr int kXcds = 8;           // accelerator complex dies, each with its own L2

// Cross-lane max / sum over each row of 16 lanes with DPP moves: swap
// neighbours, swap pairs, then mirror within 8 and within 16 lanes; after
// each step every lane holds the combination of a group twice as large.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));     // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_mov<0x4E>(v));     // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_mov<0x141>(v));    // row_half_mirror
  return fmaxf(v, dpp_mov<0x140>(v)); // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  return v + dpp_mov<0x140>(v);
}

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
// lse: [rows] (natural log; -inf for a user without history rows).  C is
// written in bf16 when CBF (the value product rounds it to bf16 anyway).
template <int DW, bool CBF>
__global__ __launch_bounds__(512, 1) void sa_stca_core(const int64_t* __restrict__ x_off,
                                                      const int64_t* __restrict__ t_off, int B,
                                                      int h, const bf16* __restrict__ U,
                                                      const bf16* __restrict__ X,
                                                      int64_t nrows_x, int64_t rows,
                                                      float alpha, float scale,
                                                      void* __restrict__ Cv,
                                                      float* __restrict__ lse) {
  constexpr int NW = 8;
  constexpr int D = DW * NW;
  constexpr int KS = DW / 16;              // K steps of the partial scores
  constexpr int DB = DW / 32;              // 32-row blocks of the wave's C^T
  constexpr int U16 = DW / 8;              // 16-byte units per slice row
  constexpr int CPL = 32 * U16 / 64;       // 16-byte copies per lane per tile
  constexpr int WST = 40;                  // bf16 stride of a weight row (80 bytes)
  __shared__ __attribute__((aligned(16))) bf16 sX[NW][32 * DW];
  __shared__ __attribute__((aligned(16))) float sS[NW][32 * 32];   // [wave][query][row]
  // Float index of 16-byte unit u (history rows 4 u .. 4 u + 3) of query q's
  // partial scores.  The unit is XOR-swizzled with q / 2 so that 16 lanes
  // writing one unit of 16 queries, and 32 lanes reading two queries' rows,
  // each touch every bank once.
  auto sidx = [](int q, int u) { return q * 32 + ((u ^ ((q >> 1) & 7)) << 2); };
  __shared__ __attribute__((aligned(16))) bf16 sW[32 * WST];       // [query][slot]
  __shared__ float sF[32];                                         // rescale factor / 1 / sum

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h2 = lane >> 5, l32 = lane & 31;
  // Workgroups are dealt to the 8 XCDs in turn (block b runs on XCD b % 8).
  // Give each XCD a contiguous range of query tiles instead: the workgroups
  // resident on one XCD then serve the same user and stream the same history
  // rows through that XCD's L2 at about the same pace.
  const int nb = (int)gridDim.x, xcd = (int)blockIdx.x % kXcds, per = nb / kXcds,
            extra = nb % kXcds;
  const int tile = xcd * per + (xcd < extra ? xcd : extra) + (int)blockIdx.x / kXcds;
  const int64_t q0 = (int64_t)tile * 32;
  const int64_t q = q0 + l32;                       // this lane's query row (context product)
  const bool qvalid = q < rows;
  const int c0 = wave * DW;                         // this wave's D-columns
  const uint32_t sx = lds_addr((const SA_LDS void*)&sX[wave][0]);
  const SA_LDS char* lds = (const SA_LDS char*)0;

  // Reduce-scatter role: lane -> query row rq = 4 wave + (lane >> 4) of the
  // tile, history rows 2 m and 2 m + 1 (m = lane & 15).
  const int rqi = 4 * wave + (lane >> 4), rm = lane & 15;
  const int64_t rq = q0 + rqi;
  const int ruser = rq < rows ? user_of_target<false>(t_off, B, rq / h) : -1;
  // Weight slot of history row r: rows 16 kb + 8 e + 4 hh + c go to slot
  // 16 kb + 8 hh + 4 e + c, so that a context-product lane (query, half hh)
  // reads its 8 K slots of block kb as one 16-byte unit.
  const int wrow = 2 * rm;
  const int wslot = (wrow & ~12) | (((wrow >> 2) & 1) << 3) | (((wrow >> 3) & 1) << 2);

  // The wave's query slice as B operands: ub[ks] = U[q][c0 + 16 ks + 8 h2 ..].
  bf16x8 ub[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    ub[ks] = qvalid ? *(const bf16x8*)(U + q * D + c0 + 16 * ks + 8 * h2) : bf16x8{};

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
  // slice (row v / U16, unit v % U16 of the wave's columns).  Rows past the
  // user's last row load that last row instead (no branch per load): their
  // scores are masked, so they enter the context product with weight 0.
  // Addressing: a tile base uniform over the workgroup plus a 32-bit lane
  // offset (row r clamped to the tile's last valid row, times the row pitch).
  const uint32_t ucol = (uint32_t)(c0 + 8 * (lane % U16)) * 2;
  auto fetch = [&](int64_t t0, int64_t xlast, bf16x8 (&reg)[CPL]) {
    const int64_t tb = t0 < xlast ? t0 : xlast;     // tiles past the end load row xlast
    const char* base = (const char*)(X + tb * D);
    const int64_t mr = xlast - tb;                  // >= 0
    const int rmax = mr < 31 ? (int)mr : 31;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int r = (lane + 64 * j) / U16;
      const int rc = r < rmax ? r : rmax;
      reg[j] = *(const bf16x8*)(base + ((uint32_t)rc * (uint32_t)(D * 2) + ucol));
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
  float mrun = -INFINITY, lsum = 0.f;               // softmax state of query row rq
  const float tau_raw = kStcaTau / alpha;

  // Users of this tile's query rows (uniform over the workgroup).
  const int64_t qlast = (q0 + 31 < rows ? q0 + 31 : rows - 1);
  const int u_first = user_of_target<true>(t_off, B, q0 / h);
  const int u_last = user_of_target<true>(t_off, B, qlast / h);
  for (int u = u_first; u <= u_last; ++u) {
    if (uload64(t_off + u) == uload64(t_off + u + 1)) continue;   // no targets here
    // Row ranges are clamped to the nrows_x rows of X: corrupt offsets give
    // wrong numbers, never an access outside X.
    const int64_t xlo = clamp64(uload64(x_off + u), 0, nrows_x);
    const int64_t xhi = clamp64(uload64(x_off + u + 1), xlo, nrows_x);
    if (xlo >= xhi) continue;
    const bool mine = ruser == u;
    const int nt = (int)((xhi - xlo + 31) / 32);
    // Rows of the tile starting at t0 (0 past the end).
    auto nrows = [&](int64_t t0) -> int {
      const int64_t n = xhi - t0;
      return n <= 0 ? 0 : (n >= 32 ? 32 : (int)n);
    };
    // Partial S^T over this wave's columns: rows = history rows, lane = query.
    auto scores = [&]() {
      f32x16 sp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sp = mfma32(*(const SA_LDS bf16x8*)(lds + sx + aoff[ks]), ub[ks], sp);
      return sp;
    };
    // X_w^T operands of the context product (rows 16 kb .. of the slice, 32 DW
    // bytes apart).
    auto read_xt = [&](bf16x8 (&xt)[2][DB]) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          xt[kb][db] = concat4(
              lds_read_tr16((const SA_LDS bf16*)(lds + sx + toff[db][0] + kb * 32 * DW)),
              lds_read_tr16((const SA_LDS bf16*)(lds + sx + toff[db][1] + kb * 32 * DW)));
    };
    // Register i of sp is history row crow(i, h2) = 8 (i / 4) + 4 h2 + i % 4:
    // 16-byte unit 2 g + h2 of the query's row of partial scores.
    auto publish = [&](const f32x16& sp) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)&sS[wave][sidx(l32, 2 * g + h2)] =
            f32x4{sp[4 * g], sp[4 * g + 1], sp[4 * g + 2], sp[4 * g + 3]};
    };

    // Pipeline: the slice holds tile t + 1 and the registers tile t + 2 while
    // tile t's softmax and context product run.
    bf16x8 pre[CPL], xt[2][DB];
    const int64_t xlast = xhi - 1;
    fetch(xlo, xlast, pre);
    stash(pre);
    __builtin_amdgcn_s_waitcnt(0xC07F);             // lgkmcnt(0): the slice is written
    fetch(xlo + 32, xlast, pre);
    {
      const f32x16 sp = scores();
      read_xt(xt);
      publish(sp);
    }
    stash(pre);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    fetch(xlo + 64, xlast, pre);
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      const int nr = nrows(xlo + 32 * (int64_t)t);
      // Scores of tile t + 1 (unused after the last tile), then the
      // reduce-scatter of tile t: query row rq, history rows 2 rm, 2 rm + 1.
      const f32x16 spn = scores();
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float2 pv = *(const float2*)&sS[w][sidx(rqi, rm >> 1) + 2 * (rm & 1)];
        v0 += pv.x;
        v1 += pv.y;
      }
      v0 = (mine && 2 * rm < nr) ? v0 : -INFINITY;
      v1 = (mine && 2 * rm + 1 < nr) ? v1 : -INFINITY;
      const float tm = row16_max(fmaxf(v0, v1));
      const bool raise = tm > mrun + tau_raw;
      const float fr = mrun == -INFINITY ? 0.f : exp2_fast((mrun - tm) * alpha);
      const float f = raise ? fr : 1.f;
      mrun = raise ? tm : mrun;
      const float ma = mrun == -INFINITY ? 0.f : mrun * alpha;
      const float a0 = exp2_fast(fmaf(v0, alpha, -ma)), a1 = exp2_fast(fmaf(v1, alpha, -ma));
      lsum = fmaf(lsum, f, a0 + a1);
      bf16x2 wv;
      wv[0] = (bf16)a0;
      wv[1] = (bf16)a1;
      *(bf16x2*)&sW[rqi * WST + wslot] = wv;
      sF[rqi] = f;                                  // the 16 lanes of a row agree
      __syncthreads();
      // Rescale and accumulate tile t: C^T (columns x queries) += X_w^T A^T.
      const float fq = sF[l32];
      if (__builtin_amdgcn_ballot_w64(fq != 1.f) != 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= fq;
      }
      bf16x8 abf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) abf[kb] = *(const bf16x8*)&sW[l32 * WST + 16 * kb + 8 * h2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = mfma32(xt[kb][db], abf[kb], acc[db]);
      // Advance: operands of tile t + 1, its partial scores out, tile t + 2
      // into the slice, tile t + 3 into registers.
      read_xt(xt);
      publish(spn);
      stash(pre);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      fetch(xlo + 32 * (int64_t)(t + 3), xlast, pre);
      __syncthreads();
    }
  }
  // Totals of the reduce-scatter rows: 1 / sum to the context lanes, lse out.
  const float L = row16_sum(lsum);
  if (rm == 0) {
    sF[rqi] = L > 0.f ? 1.0f / L : 0.f;
    if (rq < rows) lse[rq] = L > 0.f ? mrun * scale + __logf(L) : -INFINITY;
  }
  __syncthreads();
  // Output: acc[db] register i is C[q][c0 + 32 db + crow(i, h2)] (unnormalised).
  if (qvalid) {
    const float inv = sF[l32];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = {acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv,
                         acc[db][4 * g + 3] * inv};
        const int64_t o = q * D + c0 + 32 * db + 8 * g + 4 * h2;
        if constexpr (CBF) {
          bf16x4 b;
          b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
          *(bf16x4*)((bf16*)Cv + o) = b;
        } else {
          *(f32x4*)((float*)Cv + o) = v;
        }
      }
  }
}

hipError_t launch_stca_core(int D, int h, int B, const int64_t* x_off, const int64_t* t_off,
                            const void* Uv, const void* Xv, int64_t L, int64_t rows, void* C,
                            int c_bf16, float* lse, hipStream_t st) {
  const bf16* U = (const bf16*)Uv;
  const bf16* X = (const bf16*)Xv;
  if (rows <= 0) return hipSuccess;
  const int dh = D / h;
  const float scale = 1.0f / sqrtf((float)dh);
  const float alpha = scale * kLog2e;
  const dim3 grid((unsigned)((rows + 31) / 32));
#define SA_STCA(DW_, CBF_)                                                                       \
  hipLaunchKernelGGL((sa_stca_core<DW_, CBF_>), grid, dim3(512), 0, st, x_off, t_off, B, h, U, X, \
                     L, rows, alpha, scale, C, lse)
  switch (D) {
    case 256: if (c_bf16) SA_STCA(32, true); else SA_STCA(32, false); break;
    case 512: if (c_bf16) SA_STCA(64, true); else SA_STCA(64, false); break;
    case 1024: if (c_bf16) SA_STCA(128, true); else SA_STCA(128, false); break;
    default: return hipErrorInvalidValue;
  }
#undef SA_STCA
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
