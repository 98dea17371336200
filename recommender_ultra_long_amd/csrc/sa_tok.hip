// sa_tok.hip — the token-wise normalised sketch, the vanilla-attention
// baseline of Table 1 (SequenceO1 reading notes, sections 3.5 and 7.1): the
// affinities of Eq. (6) normalised over each user's tokens instead of over
// the prototypes,
//   A[j,i] = exp z[j,i] / sum_i' exp z[j,i'],  S[j] = sum_i A[j,i] x_i,
//   lse[j] = log sum_i exp z[j,i]  (per user and prototype).
// This is attention with the k prototypes as queries and the history as keys
// and values, so one pass suffices: each prototype keeps a running maximum
// and sum (online softmax) while its weighted sum of rows accumulates.
//
// Forward
//  sa_tok_fwd_bf16: the tiling and copy pipeline of the prototype-wise
//    aggregation (prototype-stationary workgroups over token segments, X tiles
//    copied global -> LDS six ahead, transposed reads for the second
//    product).  The lane owns a prototype, so its running maximum is a lane
//    register; the fp32 accumulators live in the matrix cores' registers and
//    are rescaled only when a maximum grows by more than 2^8 (the weights
//    exp2((z - m) alpha) then stay below 256), which after the first tiles
//    almost never happens.  One partial (U, m, l) per (segment, user) piece.
//  sa_tok_fwd_f32:  the same on the vector ALU, exact online softmax.
//  sa_tok_reduce:   per user, combines its pieces in order:
//    M = max m_s,  L = sum l_s e^{c (m_s - M)},  S = sum U_s e^{c (m_s - M)} / L,
//    lse = c M + ln L.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

constexpr float kTokTau = 8.0f;   // lazy rescale threshold, log2 units

// ----------------------------------------------------------------------------
// grid = (G segments, nchunks); block = NW waves of PT x 32 prototypes.
// part[slot][proto][d], pm[slot][proto] (raw dot products p . x, the running
// maximum the partial is scaled by), pl[slot][proto] (sum of weights), slot =
// segment + user.
template <int D, int NW, int PT>
__global__ __launch_bounds__(NW * 64, 1) void sa_tok_fwd_bf16(
    const int64_t* __restrict__ offsets, int B, const bf16* __restrict__ X,
    const bf16* __restrict__ P, int k, int64_t T, int G, float alpha, float* __restrict__ part,
    float* __restrict__ pm, float* __restrict__ pl) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int U = D / 8;
  constexpr int KC = NW * PT * 32;
  static_assert(KC == kChunkBf16, "one workgroup covers one prototype chunk");
  constexpr int TILE = 32;
  constexpr int UNITS = TILE * U;
  constexpr int UPW = UNITS / NW;
  static_assert(UNITS % NW == 0 && (UPW <= 64 || UPW % 64 == 0), "");
  constexpr int XI = (UPW + 63) / 64;    // copy instructions (= loads) per wave per tile
  constexpr int NBUF = 8, AHEAD = 6;
  constexpr int L = XI;
  constexpr uint32_t XBYTES = TILE * D * 2;
  const float tau_raw = kTokTau / alpha;  // the threshold in raw dot-product units

  __shared__ __attribute__((aligned(16))) bf16 sX[NBUF][TILE * D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int s = blockIdx.x, chunk = blockIdx.y;
  const int pw0 = chunk * KC + wave * PT * 32;
  const uint32_t sx0 = lds_addr((const SA_LDS void*)&sX[0][0]);
  const SA_LDS char* lds = (const SA_LDS char*)0;

  const int64_t lo = seg_lo(T, G, s), hi = seg_lo(T, G, s + 1);
  TileWalker<TILE> cw;
  cw.start(offsets, B, lo, hi);
  if (!cw.valid) return;
  TileWalker<TILE> qw = cw;

  bf16x8 pw[PT][KS];
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    const int row = pw0 + pt * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      pw[pt][ks] = row < k ? *(const bf16x8*)(P + (int64_t)row * D + 16 * ks + 8 * h) : bf16x8{};
  }

  int crow_[XI];
  uint32_t ccol[XI];
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int v = wave * UPW + j * 64 + lane;
    crow_[j] = v / U;
    ccol[j] = (uint32_t)(((v % U) ^ xswz<D>(v / U)) * 16);
  }
  // Every wave issues exactly L loads per tile (past the end of the stream
  // too), so that the vmcnt counts below hold.  Rows past a tile's end copy
  // its first row; their weights are masked to zero.
  auto copy_next = [&](uint32_t b) {
    const bool valid = qw.valid;
    const int64_t base = valid ? qw.t0 : 0;
    const int nr = valid ? (int)(qw.t1 - qw.t0) : 0;
    const bf16* xb = X + base * D;
#pragma unroll
    for (int j = 0; j < XI; ++j) {
      const int r = crow_[j] < nr ? crow_[j] : 0;
      if (UPW >= 64 || lane < UPW)
        lds_copy16(xb, (uint32_t)(r * D * 2) + ccol[j],
                   sx0 + b * XBYTES + (uint32_t)(wave * UPW + j * 64) * 16);
    }
    if (valid) qw.advance();
  };

#pragma unroll
  for (int b = 0; b < AHEAD; ++b) copy_next(b);
#pragma unroll
  for (int pt = 0; pt < PT; ++pt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(pw[pt][ks]));
  wait_vmcnt<0>();
  __syncthreads();

  const int tr_r = (lane & 15) >> 2, tr_c = lane & 3, tr_half = (lane >> 4) & 1;
  uint32_t aoff[KS], toff[DB][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) aoff[ks] = (uint32_t)xoff<D>(l32, 2 * ks + h) * 2;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      toff[db][e] = (uint32_t)(xoff<D>(4 * h + tr_r + 8 * e, 4 * db + 2 * tr_half + (tr_c >> 1)) +
                               (tr_c & 1) * 4) * 2;

  f32x16 znext[PT];
  {
    bf16x8 a0[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a0[ks] = *(const SA_LDS bf16x8*)(lds + sx0 + aoff[ks]);
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      znext[pt] = mfma32(a0[0], pw[pt][0], f32x16{});
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) znext[pt] = mfma32(a0[ks], pw[pt][ks], znext[pt]);
    }
  }

  uint32_t t = 0;
  while (cw.valid) {
    const int64_t slot = (int64_t)s + cw.user;
    f32x16 acc[PT][DB];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[pt][db] = f32x16{};
    float mrun[PT], lsum[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) { mrun[pt] = -INFINITY; lsum[pt] = 0.f; }
    bool last;
    do {
      const uint32_t buf = t & (NBUF - 1), b1 = (t + 1) & (NBUF - 1);
      copy_next((t + AHEAD) & (NBUF - 1));
      const SA_LDS char* xs = lds + sx0 + buf * XBYTES;
      const SA_LDS char* xs1 = lds + sx0 + b1 * XBYTES;
      const int nr = (int)(cw.t1 - cw.t0);        // valid rows of this tile

      bf16x8 an[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) an[ks] = *(const SA_LDS bf16x8*)(xs1 + aoff[ks]);
      f32x16 z[PT];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) z[pt] = znext[pt];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
          znext[pt] = mfma32(an[ks], pw[pt][ks], ks == 0 ? f32x16{} : znext[pt]);

      bf16x8 xt[2][DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const SA_LDS char* p0 = xs + toff[db][0];
        const SA_LDS char* p1 = xs + toff[db][1];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          xt[kb][db] = concat4(lds_read_tr16((const SA_LDS bf16*)(p0 + kb * 32 * D)),
                               lds_read_tr16((const SA_LDS bf16*)(p1 + kb * 32 * D)));
      }

      // Weights of tile t for the lane's prototype: register i is token
      // crow(i, h) of the tile.
      bf16x8 abf[PT][2];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        if (nr < TILE) {   // the last tile of a piece: rows past its end weigh 0
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (crow(i, h) >= nr) z[pt][i] = -INFINITY;
        }
        float tm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) tm = fmaxf(tm, z[pt][i]);
        tm = fmaxf(tm, shfl_xor32(tm));            // both halves of the prototype
        const bool need = tm > mrun[pt] + tau_raw;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
          // Rare: rescale the lanes whose maximum grew past the threshold.
          const float mnew = need ? tm : mrun[pt];
          const float f = mrun[pt] == -INFINITY ? 0.f : exp2_fast((mrun[pt] - mnew) * alpha);
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[pt][db] *= f;
          lsum[pt] *= f;
          mrun[pt] = mnew;
        }
        const float ma = mrun[pt] * alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float a = exp2_fast(fmaf(z[pt][8 * kb + j], alpha, -ma));
            lsum[pt] += a;
            abf[pt][kb][j] = (bf16)a;
          }
      }
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[pt][db] = mfma32(xt[kb][db], abf[pt][kb], acc[pt][db]);

      if (t & 1) {
        wait_vmcnt<3 * L>();
        barrier_lds();
      }
      last = cw.last_in_piece();
      cw.advance();
      ++t;
    } while (!last);

#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const int proto = pw0 + pt * 32 + l32;
      const float lo_ = shfl_xor32(lsum[pt]);
      if (proto < k) {
        float* dst = part + (slot * k + proto) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 v = {acc[pt][db][4 * g], acc[pt][db][4 * g + 1], acc[pt][db][4 * g + 2],
                       acc[pt][db][4 * g + 3]};
            *(f32x4*)(dst + 32 * db + 8 * g + 4 * h) = v;
          }
        if (h == 0) {
          pm[slot * k + proto] = mrun[pt];
          pl[slot * k + proto] = lsum[pt] + lo_;
        }
      }
    }
    wait_vmem_all();
  }
  wait_vmcnt<0>();
}

// ----------------------------------------------------------------------------
// fp32: grid = (G, ceil(k / 64)), block 256; thread (j = t / 4, q = t % 4)
// owns prototype j, columns q D/4 .. +D/4 of the partial, and the weights of
// tokens 8q .. 8q+7 of each 32-token tile.  Exact online softmax per tile.
template <int D>
__global__ __launch_bounds__(256) void sa_tok_fwd_f32(const int64_t* __restrict__ offsets, int B,
                                                      const float* __restrict__ X,
                                                      const float* __restrict__ P, int k,
                                                      int64_t T, int G, float alpha,
                                                      float* __restrict__ part,
                                                      float* __restrict__ pm,
                                                      float* __restrict__ pl) {
  constexpr int PC = kChunkF32, TILE = 32, DQ = D / 4;
  __shared__ float sP[PC][D + 1];
  __shared__ float sX[TILE][D + 1];
  __shared__ float sA[PC][TILE + 1];
  const int tid = threadIdx.x;
  const int j = tid >> 2, q = tid & 3;
  const int s = blockIdx.x;
  const int p0 = blockIdx.y * PC;
  for (int i = tid; i < PC * D; i += 256) {
    const int r = i / D, c = i % D;
    sP[r][c] = (p0 + r < k) ? P[(int64_t)(p0 + r) * D + c] : 0.f;
  }
  const int64_t lo = seg_lo(T, G, s), hi = seg_lo(T, G, s + 1);
  TileWalker<TILE> cur;
  cur.start(offsets, B, lo, hi);
  float acc[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  while (cur.valid) {
    __syncthreads();
    for (int i = tid; i < TILE * D; i += 256) {
      const int r = i / D, c = i % D;
      sX[r][c] = (cur.t0 + r < cur.t1) ? X[(cur.t0 + r) * D + c] : 0.f;
    }
    __syncthreads();
    const int nr = (int)(cur.t1 - cur.t0);
    float z[8];
    float tm = -INFINITY;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int tt = 8 * q + t;
      float v = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) v = fmaf(sP[j][e], sX[tt][e], v);
      z[t] = tt < nr ? v : -INFINITY;
      tm = fmaxf(tm, z[t]);
    }
    tm = fmaxf(tm, __shfl_xor(tm, 1, 64));
    tm = fmaxf(tm, __shfl_xor(tm, 2, 64));
    const float mnew = fmaxf(m, tm);
    const float f = m == -INFINITY ? 0.f : exp2_fast((m - mnew) * alpha);   // 0 on a piece's first tile
#pragma unroll
    for (int e = 0; e < DQ; ++e) acc[e] *= f;
    l *= f;
    m = mnew;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float a = exp2_fast((z[t] - m) * alpha);
      sA[j][8 * q + t] = a;
      l += a;
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
      float lt = l + __shfl_xor(l, 1, 64);
      lt += __shfl_xor(lt, 2, 64);
      if (p0 + j < k) {
        float* dst = part + (slot * k + p0 + j) * D + q * DQ;
#pragma unroll
        for (int e = 0; e < DQ; ++e) dst[e] = acc[e];
        if (q == 0) {
          pm[slot * k + p0 + j] = m;
          pl[slot * k + p0 + j] = lt;
        }
      }
#pragma unroll
      for (int e = 0; e < DQ; ++e) acc[e] = 0.f;
      m = -INFINITY;
      l = 0.f;
    }
    cur.advance();
  }
}

// ----------------------------------------------------------------------------
// grid = (B, ceil(k d / 256)); block 256 = 4 waves; lane -> 4 consecutive
// elements of S[u] (one prototype).  Pieces of user u are slots s0 + u ..
// s1 + u.  Every wave finds the maximum M over the pieces; wave w then adds
// pieces w, w + 4, ... (eight loads in flight) and the four wave sums are
// added in wave order, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void sa_tok_reduce(const int64_t* __restrict__ offsets, int B,
                                                     int k, int d, int64_t T, int G, float scale,
                                                     float alpha, const float* __restrict__ part,
                                                     const float* __restrict__ pm,
                                                     const float* __restrict__ pl,
                                                     float* __restrict__ S, float* __restrict__ lse,
                                                     uint32_t* __restrict__ status) {
  __shared__ f32x4 red[4][64];
  __shared__ float redl[4][64];
  __shared__ float redm[4][64];
  const int u = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (blockIdx.y == 0 && u == 0) check_offsets_block(offsets, B, T, status, kStatusOk, kStatusBadOffsets);
  const int64_t kd = (int64_t)k * d;
  const int64_t e = ((int64_t)blockIdx.y * 64 + lane) * 4;
  const bool live = e < kd;
  const int j = live ? (int)(e / d) : 0;
  const int64_t lo = clamp64(uload64(offsets + u), 0, T);
  const int64_t hi = clamp64(uload64(offsets + u + 1), lo, T);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float Ls = 0.f, M = -INFINITY;
  const bool work = hi > lo && live;
  const int s0 = work ? seg_of(T, G, lo) : 0, s1 = work ? seg_of(T, G, hi - 1) : -1;
  const int n = s1 - s0 + 1;                     // pieces of user u (0 without work)
  const int64_t b0 = (int64_t)s0 + u;
  // The maximum over the pieces: wave w takes pieces w, w + 4, ... with eight
  // loads in flight; the four wave maxima meet in LDS.
  {
    float Mw = -INFINITY;
    int q = wave;
    for (; q + 28 < n; q += 32) {
      float t8[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) t8[r] = pm[(b0 + q + 4 * r) * k + j];
#pragma unroll
      for (int r = 0; r < 8; ++r) Mw = fmaxf(Mw, t8[r]);
    }
    for (; q < n; q += 4) Mw = fmaxf(Mw, pm[(b0 + q) * k + j]);
    redm[wave][lane] = Mw;
    __syncthreads();
    M = fmaxf(fmaxf(redm[0][lane], redm[1][lane]), fmaxf(redm[2][lane], redm[3][lane]));
  }
  if (work) {
    int q = wave;
    for (; q + 28 < n; q += 32) {
      f32x4 v[8];
      float f[8], lv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int64_t sl = b0 + q + 4 * r;
        v[r] = *(const f32x4*)(part + sl * kd + e);
        f[r] = pm[sl * k + j];
        lv[r] = pl[sl * k + j];
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float w = exp2_fast((f[r] - M) * alpha);
        acc += v[r] * w;
        Ls = fmaf(lv[r], w, Ls);
      }
    }
    for (; q < n; q += 4) {
      const int64_t sl = b0 + q;
      const float w = exp2_fast((pm[sl * k + j] - M) * alpha);
      acc += *(const f32x4*)(part + sl * kd + e) * w;
      Ls = fmaf(pl[sl * k + j], w, Ls);
    }
  }
  red[wave][lane] = acc;
  redl[wave][lane] = Ls;
  __syncthreads();
  if (wave != 0 || !live) return;
  acc = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
  Ls = ((redl[0][lane] + redl[1][lane]) + redl[2][lane]) + redl[3][lane];
  const bool any = hi > lo;
  *(f32x4*)(S + (int64_t)u * kd + e) = any ? acc * (1.0f / Ls) : f32x4{0.f, 0.f, 0.f, 0.f};
  if (e % d == 0) lse[(int64_t)u * k + j] = any ? M * scale + __logf(Ls) : -INFINITY;
}

// ----------------------------------------------------------------------------
#ifndef SA_AGG_WAVES
#define SA_AGG_WAVES 8
#endif

template <int D>
static hipError_t tok_fwd_t(const FwdArgs& a, int dtype, hipStream_t st, Prof* prof) {
  const float scale = 1.0f / sqrtf((float)D);
  const float alpha = scale * kLog2e;
  float* pm = a.pmass;         // per-slot running maxima
  float* pl = a.pl;            // per-slot sums of weights
  if (a.T > 0) {
    prof_begin(prof, dtype == 1 ? "sa_tok_fwd_bf16" : "sa_tok_fwd_f32", st);
    if (dtype == 1) {
      constexpr int NW = SA_AGG_WAVES, PT = kChunkBf16 / (32 * NW);
      hipLaunchKernelGGL((sa_tok_fwd_bf16<D, NW, PT>), dim3(a.G, a.nchunks), dim3(64 * NW), 0, st,
                         a.offsets, a.B, (const bf16*)a.X, (const bf16*)a.P, a.k, a.T, a.G, alpha,
                         a.part, pm, pl);
    } else {
      hipLaunchKernelGGL(sa_tok_fwd_f32<D>, dim3(a.G, a.nchunks), dim3(256), 0, st, a.offsets,
                         a.B, (const float*)a.X, (const float*)a.P, a.k, a.T, a.G, alpha, a.part,
                         pm, pl);
    }
    const hipError_t e = hipGetLastError();
    prof_end(prof, st);
    if (e != hipSuccess) return e;
  }
  const int64_t kd = (int64_t)a.k * a.d;
  prof_begin(prof, "sa_tok_reduce", st);
  hipLaunchKernelGGL(sa_tok_reduce, dim3(a.B, (unsigned)((kd + 255) / 256)), dim3(256), 0, st,
                     a.offsets, a.B, a.k, a.d, a.T, a.G, scale, alpha, a.part, pm, pl, a.S, a.lse,
                     a.status);
  const hipError_t e = hipGetLastError();
  prof_end(prof, st);
  return e;
}

hipError_t launch_tok_fwd(const FwdArgs& a, int dtype, hipStream_t st, Prof* prof) {
  switch (a.d) {
    case 32: return tok_fwd_t<32>(a, dtype, st, prof);
    case 64: return tok_fwd_t<64>(a, dtype, st, prof);
    case 128: return tok_fwd_t<128>(a, dtype, st, prof);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
