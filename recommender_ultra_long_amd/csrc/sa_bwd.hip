// sa_bwd.hip — Sketch Attention backward: dX and dP from dS.
//
// The pages state only that the sketch is fully differentiable (SequenceO1
// reading notes, section 3.1, after Eq. (9)); the formulas are the chain rule
// of Eq. (6)-(9) with the optional mass normalisation:
//   G = dS, cv = 0                 (plain sum)
//   G_j = dS_j / mu_j, cv_j = G_j . S_j          (mass norm, mu_j = 0 -> 0)
//   dA'_ji = G_j . x_i,  w_ji = A_ji (dA'_ji - cv_j),  delta_i = sum_j w_ji
//   dZ_ji = w_ji - A_ji delta_i
//   dX_i = sum_j A_ji G_j + c sum_j dZ_ji p_j
//        = g_i + c (b_i - delta_i a_i),  g = A^T G,  a = A^T P,  b = w^T P
//   dP = c sum_u sum_i dZ_ji x_i
// The softmax weights A are recomputed per tile from X, P and the forward's
// per-token log-sum-exp; nothing of size k x n is stored.
//
// Kernels
//  sa_bwd_prep:   G (input dtype) and cv per user and prototype.
//  sa_bwdx_bf16:  token-stationary, one pass over all prototypes per token
//                 tile, twice: Z and g^T = G^T A, giving delta, then Z, dA'
//                 and dX^T += P^T dZ (Z = P X^T orientation, token per lane;
//                 the accumulation operands read transposed from LDS).
//                 Writes dX and delta.  10 k d MFMA flops per token.
//  sa_bwdp_bf16:  prototype-stationary (256 prototypes per workgroup, like
//                 the forward aggregation): Z^T, dA'^T, dZ, then
//                 dP^T += X^T dZ^T.  One partial per token segment.  6 k d.
//  sa_dp_reduce:  dP = c sum over segments in order (deterministic).
// The fp32 variants do the same arithmetic on the vector ALU.
#include <type_traits>

#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

// ----------------------------------------------------------------------------
// G, cv and the padded copies.  Rows of G and cv have stride kp >= k; rows
// from k on are zero.  Block ranges:
//   [0, nbg)          one group of D/4 threads per (user, prototype) row: G in
//                     the input dtype, cv, and -cv (when cvs is not null);
//   [nbg, nbg + nbq)  Pq = P with zero rows k .. kp - 1, 16 bytes per thread
//                     (bf16 only); one copy per user (pq_users = B, user u's
//                     table at P + u pstride) or one shared copy (pq_users = 1);
//   from nbg + nbq    lse2 = lse log2(e), with the +inf sentinel at index T;
//                     token-wise (mode 2): per (user, prototype), rows of
//                     stride kp, +inf on padding rows.
// mode: 0 plain sum (G = dS, cv = 0), 1 mass normalisation (G = dS / mu,
// cv = G . S), 2 token-wise normalisation (G = dS, cv = G . S).
template <typename OutT, int D>
__global__ __launch_bounds__(256) void sa_bwd_prep(
    const float* __restrict__ dS, const float* __restrict__ S, const float* __restrict__ mass,
    int B, int k, int kp, int mode, float scale, OutT* __restrict__ Gq,
    float* __restrict__ cv, float* __restrict__ cvs, unsigned nbg, const bf16* __restrict__ P,
    int64_t pstride, int pq_users, bf16* __restrict__ Pq, unsigned nbq,
    const float* __restrict__ lse, int64_t T, float* __restrict__ lse2) {
  if (blockIdx.x >= nbg + nbq) {
    const int64_t i = (int64_t)(blockIdx.x - nbg - nbq) * 256 + threadIdx.x;
    if (mode == 2) {
      // token-wise: per (user, prototype) rows of stride kp, +inf for padding
      if (i < (int64_t)B * kp) {
        const int64_t u = i / kp;
        const int j = (int)(i % kp);
        lse2[i] = j < k ? lse[u * k + j] * kLog2e : INFINITY;
      }
      return;
    }
    if (i < T) lse2[i] = lse[i] * kLog2e;
    else if (i == T) lse2[i] = INFINITY;
    return;
  }
  if (blockIdx.x >= nbg) {
    constexpr int UPR = D / 8;   // 16-byte units per row
    const int64_t unit = (int64_t)(blockIdx.x - nbg) * 256 + threadIdx.x;
    const int64_t row = unit / UPR;                    // over pq_users x kp rows
    const int part = (int)(unit % UPR);
    if (row < (int64_t)pq_users * kp) {
      const int64_t u = row / kp;
      const int j = (int)(row % kp);
      bf16x8 v = {};
      if (j < k) v = *(const bf16x8*)(P + u * pstride + (int64_t)j * D + 8 * part);
      *(bf16x8*)(Pq + row * D + 8 * part) = v;
    }
    return;
  }
  constexpr int TPR = D / 4;   // threads per row (8, 16 or 32)
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gt / TPR;
  const int part = (int)(gt % TPR);
  const int64_t rows = (int64_t)B * kp;
  const int u = (int)(row / kp), j = (int)(row % kp);
  const bool inrange = row < rows;
  const bool live = inrange && j < k;
  const int64_t r = live ? (int64_t)u * k + j : 0;   // source row of dS, S, mass
  f32x4 g = {0.f, 0.f, 0.f, 0.f};
  float c = 0.f;
  if (live) {
    g = *(const f32x4*)(dS + r * D + 4 * part);
    if (mode == 1) {
      const float mu = mass[r];
      const float inv = mu > 0.f ? 1.0f / mu : 0.f;
      g = mu > 0.f ? g * inv : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (mode != 0) {
      // cv = G . S: the mass-normalised sketch's rows, or, token-wise, the
      // softmax term D_j = sum_i A_ji dA_ji = dS_j . S_j
      const f32x4 sv = *(const f32x4*)(S + r * D + 4 * part);
      c = g[0] * sv[0] + g[1] * sv[1] + g[2] * sv[2] + g[3] * sv[3];
    }
  }
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) c += __shfl_xor(c, off, 64);
  if (inrange) {
#pragma unroll
    for (int e = 0; e < 4; ++e) Gq[row * D + 4 * part + e] = (OutT)g[e];
    if (part == 0) {
      cv[row] = c;
      if (cvs != nullptr) cvs[row] = -c;
    }
  }
}

// ----------------------------------------------------------------------------
// bf16 dX pass.  grid = ceil(T / 256); block 512 = 8 waves x 32 tokens, two
// waves per SIMD so that one wave's vector work overlaps the other's matrix
// products.  Tokens of the workgroup that belong to different users are
// handled one user at a time (the others get weight 0), because G depends on
// the user; in a user's round, waves that hold none of its tokens only copy
// their share of the chunks and meet the barriers.
//
// With w'_ji = c A_ji (dA'_ji - cv_j) and s_i = sum_j w'_ji (= c delta_i),
//   dX_i = g_i + sum_j (w'_ji - s_i A_ji) p_j,   g_i = sum_j A_ji G_j,
// and, since dA'_ji = G_j . x_i,  s_i = c (x_i . g_i - sum_j A_ji cv_j).
// s_i needs every prototype before any w' - s A can be formed, so the pass
// runs over the prototypes twice:
//   stage 1: Z, A;  acc^T = G^T A (= g^T), e += A (-cv);  s = c (x . g + e);
//   stage 2: Z, dA' - cv, A;  acc^T += P^T (c A (dA' - cv) - s A).
// 4 + 6 = 10 k d matrix flops per token; the weight of stage 2 is c dZ
// itself, rounded to bf16 once.
//
// Prototypes stream through LDS in chunks of 64 rows: P, G and -cv in both
// stages, copied global -> LDS by the direct-to-LDS loads three
// chunks ahead into four buffers (rows stored with the tile swizzle of
// sa_device.h), one barrier per chunk.  P, G and cv are padded with zero rows
// to a whole number of chunks: a padded prototype's weight is at most 1 and
// multiplies zero rows.  The token is the lane (Z = P X^T orientation, X rows
// resident as B operands); the A operands of the accumulation are
// transpose-read from LDS.  dX goes out through LDS so that every store
// covers whole token rows.
//
// A wave runs its products at raised priority and its vector work (the
// weights) at the normal one (s_setprio): when the two waves of a SIMD are in
// different phases, the one with products ready issues them first and the
// other's vector instructions fill the matrix cores' busy cycles (about 4 %
// faster than equal priorities).
//
// Token-wise normalisation (TW): the weights A_ji = exp(z_ji - lse_j) use the
// prototype's statistic, streamed with each chunk beside -cv (= -D_j); with
// w'_ji = c A_ji (dA'_ji - D_j) = c dZ_ji there is no per-token coupling:
// one round (stage 2 with s = 0, also adding G^T A) gives
// dX_i = sum_j (A_ji G_j + w'_ji p_j), 8 k d, and no delta.
//
// CV: cv is not zero (mass normalisation, token-wise); without it (the plain
// sum) the -cv terms are left out.
template <int D, bool TW, bool CV>
__global__ __launch_bounds__(512) void sa_bwdx_bf16(
    const int64_t* __restrict__ offsets, int B, const bf16* __restrict__ X,
    const bf16* __restrict__ Pq, int64_t pq_ustride, const bf16* __restrict__ Gq,
    const float* __restrict__ cvn, int kp, int64_t T, float alpha, float scale,
    const float* __restrict__ lse, const float* __restrict__ lq2, float* __restrict__ dX,
    int acc_dx, float* __restrict__ delta_out, bf16* __restrict__ wz, int kz) {
  constexpr int NW = 8;                   // waves
  static_assert(NW * 32 == kBwdxTokensBf16, "");
  constexpr int KS = D / 16, DB = D / 32, U = D / 8;
  constexpr int PCH = kBwdxChunkBf16;     // prototypes per chunk
  static_assert(PCH == 64, "two 32-prototype tiles per chunk");
  constexpr int NB = 4;                   // chunk buffers
  constexpr int CU = PCH * U;             // 16-byte units per matrix chunk
  constexpr int UPW = CU / NW;            // units per wave per matrix
  static_assert(UPW < 64 || UPW % 64 == 0, "");
  constexpr int XI = (UPW + 63) / 64;     // copy instructions per wave per matrix
  constexpr int LC = 2 * XI + 1 + (TW ? 1 : 0);   // loads per wave per chunk copy
  constexpr int NST = TW ? 1 : 2;         // rounds over the prototypes
  constexpr int CW = PCH / NW;            // cv entries copied per wave
  constexpr uint32_t MB = PCH * D * 2;    // bytes of one matrix chunk
  constexpr uint32_t GOFF = MB;           // G follows P in a buffer
  constexpr uint32_t CB = 2 * MB;         // bytes of one chunk buffer
  constexpr uint32_t TB = 32 * D * 2;     // bytes of a 32-row tile
  constexpr uint32_t KB = 16 * D * 2;     // bytes of 16 rows
  static_assert(NW * 32 * D * 4 <= NB * CB, "dX staging fits in the chunk buffers");
  __shared__ __attribute__((aligned(16))) bf16 sbuf[NB * 2 * PCH * D];
  __shared__ __attribute__((aligned(16))) float sC[NB][PCH];
  __shared__ __attribute__((aligned(16))) float sQ[TW ? NB : 1][PCH];   // TW: lse2 per prototype

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int64_t r0 = (int64_t)blockIdx.x * kBwdxTokensBf16;
  const int64_t r1 = r0 + kBwdxTokensBf16 < T ? r0 + kBwdxTokensBf16 : T;
  const int64_t tok = r0 + wave * 32 + l32;
  const uint32_t sb0 = lds_addr((const SA_LDS void*)&sbuf[0]);
  const uint32_t sc0 = lds_addr((const SA_LDS void*)&sC[0][0]);
  const uint32_t sq0 = lds_addr((const SA_LDS void*)&sQ[0][0]);
  const SA_LDS char* lds = (const SA_LDS char*)0;

  bf16x8 xb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    xb[ks] = tok < r1 ? *(const bf16x8*)(X + tok * D + 16 * ks + 8 * h) : bf16x8{};
  const float l2 = (!TW && tok < r1) ? lse[tok] * kLog2e : INFINITY;

  // Copy geometry (per matrix): instruction j of this wave moves units
  // v0 .. v0 + 63, v0 = wave UPW + 64 j; unit v is row v / U at stored
  // position v % U, holding global unit (v % U) ^ g(row).
  uint32_t cgo[XI];   // global byte offset within a chunk
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int v = wave * UPW + j * 64 + lane;
    cgo[j] = (uint32_t)((v / U) * D * 2 + ((v % U) ^ xswz<D>(v / U)) * 16);
  }
  // Per-lane LDS byte offsets within a chunk buffer: aoff for the A operand
  // of Z and dA' (row l32, unit 2 ks + h), toff for the transpose reads.
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
  const int nch = kp / PCH;

  int u = first_user_after(offsets, B, r0);
  for (; u < B; ++u) {
    const int64_t ulo = clamp64(uload64(offsets + u), r0, r1);
    const int64_t uhi = clamp64(uload64(offsets + u + 1), ulo, r1);
    if (ulo >= r1) break;
    if (uhi <= ulo) continue;
    const bool mine = tok >= ulo && tok < uhi;
    const float lsh = mine ? l2 : INFINITY;
    // A wave none of whose tokens belong to user u only copies its share of
    // the chunks and meets the barriers: its products would all get weight 0.
    const int64_t wt0 = r0 + (int64_t)__builtin_amdgcn_readfirstlane(wave) * 32;
    const bool active = wt0 < uhi && wt0 + 32 > ulo;
    const bf16* Gu = Gq + (int64_t)u * kp * D;
    const bf16* Pu = Pq + (int64_t)u * pq_ustride;   // the user's table (or the shared one)
    const float* cvu = cvn + (int64_t)u * kp;
    const float* lqu = TW ? lq2 + (int64_t)u * kp : nullptr;

    // Chunk q of the stream is prototype chunk q mod nch (P, G, -cv) while
    // q < NST nch (one round per stage), then copies of chunk 0 that are
    // never read, so that every copy is the same number of loads.  Into
    // buffer q % NB.
    auto copy_chunk = [&](int q) {
      const uint32_t dst = sb0 + (uint32_t)(q & (NB - 1)) * CB + (uint32_t)(wave * UPW) * 16;
      const int c = q < nch ? q : (q < NST * nch ? q - nch : 0);
      const uint32_t goff = (uint32_t)c * MB;
#pragma unroll
      for (int j = 0; j < XI; ++j) {
        if (UPW >= 64 || lane < UPW) {
          lds_copy16(Pu, goff + cgo[j], dst + j * 1024);
          lds_copy16(Gu, goff + cgo[j], dst + GOFF + j * 1024);
        }
      }
      if (lane < CW)
        lds_copy4v(cvu + c * PCH + wave * CW + lane, sc0 + ((q & (NB - 1)) * PCH + wave * CW) * 4);
      if constexpr (TW) {
        if (lane < CW)
          lds_copy4v(lqu + c * PCH + wave * CW + lane, sq0 + ((q & (NB - 1)) * PCH + wave * CW) * 4);
      }
    };
    // After chunk q: wait until chunk q + 1 has landed (q + 2 may still be in
    // flight); after the barrier no wave reads chunk q - 1 any more, and its
    // buffer takes chunk q + 3.
    // Stage-2 chunks also issued their NZS stores of W after chunk q + 2's copy.
    constexpr int NZS = 4;                 // stores of W per wave per chunk (2 per tile)
    auto advance = [&](int q, auto stores) {
      wait_vmcnt<LC + decltype(stores)::value>();
      barrier_lds();
      copy_chunk(q + 3);
    };
    using NoStores = std::integral_constant<int, 0>;
    using WStores = std::integral_constant<int, NZS>;

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

    __syncthreads();   // the previous user's buffers are no longer read
#pragma unroll
    for (int q = 0; q < 3; ++q) copy_chunk(q);
    wait_vmcnt<2 * LC>();
    __syncthreads();   // chunk 0 has landed

    // The loops below are written in the order the instructions should
    // issue: LDS operands are read a few products ahead of their use, and
    // scheduling fences keep the compiler from moving the reads back next to
    // the products (where each product would wait for its read).
    constexpr int NS = 2 * DB;               // accumulation steps (db, kb) per tile
    constexpr int ZA = KS < 3 ? KS : 3;      // Z / dA' operand look-ahead (products)
    constexpr int ZB = KS < 4 ? KS : 4;      // Z operand look-ahead when Z is alone
    constexpr int TA = NS < 2 ? NS : 2;      // look-ahead of two accumulation operands (steps)
    constexpr int TB2 = NS < 3 ? NS : 3;     // look-ahead of one accumulation operand
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    auto rd16 = [&](uint32_t a) { return *(const SA_LDS bf16x8*)(lds + a); };
    auto rdtr = [&](uint32_t a0, uint32_t a1) {
      return concat4(lds_read_tr16((const SA_LDS bf16*)(lds + a0)),
                     lds_read_tr16((const SA_LDS bf16*)(lds + a1)));
    };
    // Transpose-read addresses of accumulation step st = 2 db + kb.
    auto tra = [&](uint32_t base, int st, int e) {
      return base + toff[st >> 1][e] + (uint32_t)((st & 1) * KB);
    };
    // -cv of prototypes crow(i, h) of tile pt, as register i.
    auto cv_regs = [&](uint32_t cb, int pt) {
      f32x16 c;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 c4 = *(const SA_LDS f32x4*)(lds + cb + pt * 128 + 32 * g4);
#pragma unroll
        for (int r = 0; r < 4; ++r) c[4 * g4 + r] = c4[r];
      }
      return c;
    };

    // Stage 1 (softmax weights only): acc^T = g^T = G^T A and
    // e = sum_j A_ji (-cv_j); then s = c (x_i . g_i + e) = c delta_i.
    float s = 0.f;
    if constexpr (!TW) {
      float eneg = 0.f;
      for (int q = 0; q < nch; ++q) {
        const uint32_t buf = sb0 + (uint32_t)(q & (NB - 1)) * CB;
        const uint32_t cb = sc0 + (uint32_t)((q & (NB - 1)) * PCH * 4 + 16 * h);
#pragma unroll
        for (int pt = 0; pt < 2 && active; ++pt) {
          const uint32_t tbuf = buf + pt * TB;
          f32x16 z = f32x16{};
          bf16x8 pa[KS];
#pragma unroll
          for (int ks = 0; ks < ZB; ++ks) pa[ks] = rd16(tbuf + aoff[ks]);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            fence();
            if (ks + ZB < KS) pa[ks + ZB] = rd16(tbuf + aoff[ks + ZB]);
            z = mfma32(pa[ks], xb[ks], z);
          }
          fence();
          bf16x8 gt[NS];
#pragma unroll
          for (int st = 0; st < TB2; ++st)
            gt[st] = rdtr(tra(tbuf, st, 0) + GOFF, tra(tbuf, st, 1) + GOFF);
          const f32x16 cvn = CV ? cv_regs(cb, pt) : f32x16{};
          fence();
          __builtin_amdgcn_s_setprio(0);
          bf16x8 abf[2];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float a = __builtin_amdgcn_fmed3f(exp2_fast(fmaf(z[i], alpha, -lsh)), 0.f, 1.f);
            if constexpr (CV) eneg = fmaf(a, cvn[i], eneg);
            abf[i >> 3][i & 7] = (bf16)a;
          }
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            fence();
            if (st + TB2 < NS)
              gt[st + TB2] = rdtr(tra(tbuf, st + TB2, 0) + GOFF, tra(tbuf, st + TB2, 1) + GOFF);
            acc[st >> 1] = mfma32(gt[st], abf[st & 1], acc[st >> 1]);
          }
          fence();
        }
        advance(q, NoStores{});
      }
      // x_i . g_i.  Register 4 g4 + r of block db is column
      // 32 db + 8 g4 + 4h + r = 16 ks + 8 (g4 % 2) + 4h + r with ks = 2 db + g4 / 2,
      // which lane (l32, g4 % 2) holds in xb[ks] at position 4h + r.  Each
      // lane keeps the positions 4h .. 4h + 3 of its own xb and takes the
      // others from the partner lane l ^ 32.
      float dot = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 xv = __builtin_bit_cast(u32x4, xb[ks]);
        const uint32_t o0 = h ? xv[2] : xv[0], o1 = h ? xv[3] : xv[1];   // own 4h .. 4h + 3
        const uint32_t p0 = h ? xv[0] : xv[2], p1 = h ? xv[1] : xv[3];   // the partner's
        const uint32_t r0w = (uint32_t)__shfl_xor((int)p0, 32, 64);
        const uint32_t r1w = (uint32_t)__shfl_xor((int)p1, 32, 64);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int db = ks >> 1, g4 = 2 * (ks & 1) + half;
          const bool own = half == h;
          const uint32_t w0 = own ? o0 : r0w, w1 = own ? o1 : r1w;
          dot = fmaf(__uint_as_float(w0 << 16), acc[db][4 * g4 + 0], dot);
          dot = fmaf(__uint_as_float(w0 & 0xFFFF0000u), acc[db][4 * g4 + 1], dot);
          dot = fmaf(__uint_as_float(w1 << 16), acc[db][4 * g4 + 2], dot);
          dot = fmaf(__uint_as_float(w1 & 0xFFFF0000u), acc[db][4 * g4 + 3], dot);
        }
      }
      const float part = dot + eneg;
      s = scale * (part + shfl_xor32(part));
    }

    // Stage 2 (the only one with token-wise weights): Z, dA' - cv, A and
    // w_ji = c A_ji (dA'_ji - cv_j) - s_i A_ji = c dZ_ji;  acc^T += P^T w
    // (+ G^T A with token-wise weights, where s = 0 and acc starts at 0).
    const int q0 = TW ? 0 : nch;
    for (int q = q0; q < NST * nch; ++q) {
      const uint32_t buf = sb0 + (uint32_t)(q & (NB - 1)) * CB;
      const uint32_t cb = sc0 + (uint32_t)((q & (NB - 1)) * PCH * 4 + 16 * h);
      const uint32_t qb = sq0 + (uint32_t)((q & (NB - 1)) * PCH * 4 + 16 * h);
      if (!active) {
        advance(q, NoStores{});   // no stores of W issued
        continue;
      }
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const uint32_t tbuf = buf + pt * TB;
        // Z and dA' - cv: rows = prototypes crow(i, h), column = this token.
        f32x16 z = f32x16{};
        f32x16 da = CV ? cv_regs(cb, pt) : f32x16{};
        bf16x8 pa[KS], ga[KS];
#pragma unroll
        for (int ks = 0; ks < ZA; ++ks) {
          pa[ks] = rd16(tbuf + aoff[ks]);
          ga[ks] = rd16(tbuf + aoff[ks] + GOFF);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          fence();
          if (ks + ZA < KS) {
            pa[ks + ZA] = rd16(tbuf + aoff[ks + ZA]);
            ga[ks + ZA] = rd16(tbuf + aoff[ks + ZA] + GOFF);
          }
          z = mfma32(pa[ks], xb[ks], z);
          da = mfma32(ga[ks], xb[ks], da);
        }
        fence();
        // The first accumulation operands, read while the weights are formed.
        constexpr int LA = TA;
        bf16x8 gt[NS], ptr[NS];
#pragma unroll
        for (int st = 0; st < LA; ++st) {
          if constexpr (TW) gt[st] = rdtr(tra(tbuf, st, 0) + GOFF, tra(tbuf, st, 1) + GOFF);
          ptr[st] = rdtr(tra(tbuf, st, 0), tra(tbuf, st, 1));
        }
        fence();
        __builtin_amdgcn_s_setprio(0);
        bf16x8 abf[2], wbf[2];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 l4 = {lsh, lsh, lsh, lsh};
          if constexpr (TW) l4 = *(const SA_LDS f32x4*)(lds + qb + pt * 128 + 32 * g4);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * g4 + r;
            // A <= 1 for real prototypes; the clamp keeps padded ones finite.
            const float a = __builtin_amdgcn_fmed3f(exp2_fast(fmaf(z[i], alpha, -l4[r])), 0.f, 1.f);
            const float w = a * fmaf(da[i], scale, -s);
            if constexpr (TW) abf[i >> 3][i & 7] = (bf16)a;
            wbf[i >> 3][i & 7] = (bf16)w;
          }
        }
        // W = c dZ for the dP pass, in fragment order: block (token tile
        // tok / 32, prototype tile) of wz holds the 64 lanes' 16 weights
        // (32 bytes each) as they are here, so each lane writes 32 contiguous
        // bytes and a wave 2 KiB.  Every lane stores (a token of another user,
        // or past the end, writes to the scratch tile after the last one), so
        // that each wave issues exactly NZS stores per chunk.
        {
          const int64_t zt = mine ? (tok >> 5) : ((T + 31) >> 5);
          bf16* zd = wz + ((zt * (kz >> 5) + ((q - q0) * 2 + pt)) * 64 + lane) * 16;
          *(bf16x8*)zd = wbf[0];
          *(bf16x8*)(zd + 8) = wbf[1];
        }
        __builtin_amdgcn_s_setprio(1);
        // K slot j of half h in block kb is prototype 16 kb + 8 (j / 4) + 4h + (j % 4).
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          fence();
          if (st + LA < NS) {
            if constexpr (TW)
              gt[st + LA] = rdtr(tra(tbuf, st + LA, 0) + GOFF, tra(tbuf, st + LA, 1) + GOFF);
            ptr[st + LA] = rdtr(tra(tbuf, st + LA, 0), tra(tbuf, st + LA, 1));
          }
          if constexpr (TW) acc[st >> 1] = mfma32(gt[st], abf[st & 1], acc[st >> 1]);
          acc[st >> 1] = mfma32(ptr[st], wbf[st & 1], acc[st >> 1]);
        }
        fence();
      }
      advance(q, WStores{});
    }
    wait_vmcnt<0>();
    __syncthreads();   // every wave's copies have landed and every read is done

    // dX rows through LDS.  Register i of accumulator block db is column
    // 32 db + crow(i, h) of this lane's token.  16-byte unit q of staging
    // row r sits at unit q ^ f(r), which keeps the 16-lane groups of both the
    // writes and the reads on distinct banks.
    auto sw = [](int r) { return D >= 64 ? (r & 15) : ((r >> 1) & 7); };
    SA_LDS f32x4* st = (SA_LDS f32x4*)(lds + sb0) + wave * 32 * (D / 4);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 v = {acc[db][4 * g4], acc[db][4 * g4 + 1], acc[db][4 * g4 + 2],
                         acc[db][4 * g4 + 3]};
        st[l32 * (D / 4) + ((8 * db + 2 * g4 + h) ^ sw(l32))] = v;
      }
    if (!TW && mine && h == 0) delta_out[tok] = s / scale;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's staging writes are done
    // Each store instruction writes 64 x 16 bytes = 256 / D whole rows.
    constexpr int RPI = 256 / D;
    int rr = lane / (D / 4), cc = lane % (D / 4);
    // Opaque here, so that the row addresses below are not computed once
    // before the user loop and kept (spilled) across it.
    asm volatile("" : "+v"(rr), "+v"(cc));
#pragma unroll
    for (int q = 0; q < 32 / RPI; ++q) {
      const int row = q * RPI + rr;
      const int64_t t = r0 + wave * 32 + row;
      const f32x4 v = st[row * (D / 4) + (cc ^ sw(row))];
      if (t >= ulo && t < uhi) {
        f32x4* dst = (f32x4*)(dX + t * D + 4 * cc);
        *dst = acc_dx ? *dst + v : v;   // acc_dx: add to the caller's dX
      }
    }
  }
}

// ----------------------------------------------------------------------------
// bf16 dP pass, a product of two stored operands: dP^T (d x prototypes) =
// X^T (d x tokens) W (tokens x prototypes) with W = c dZ, the bf16 weights the
// dX pass formed and stored in its fragment order: 2 KiB blocks per (aligned
// 32-token tile, 32-prototype tile), lane L = 32 h + token % 32 holding the
// 16 weights of prototypes crow(i, h) (i = 0 .. 15), kz / 32 blocks per token
// tile.  grid = (Gb segments, nchunks); block = NW waves x 32 prototypes (one
// 256-prototype chunk).  The segment's token stream is cut into 32-token
// tiles that never straddle two users (nor align with the stored ones); the X
// tile and the tile's W entries of this chunk are copied global -> LDS by the
// direct-to-LDS loads three tiles ahead into four buffers, one barrier per
// tile.  In LDS, wave w's W is [token row][h][16 weights]: 8 bytes at (row,
// h, 4 (c / 2)) are the row's prototypes 4c .. 4c + 3 (c % 2 = h), so both
// operands are transpose-read like a row-major tile (K = tokens, in the same
// order for both).  Rows of a tile past its end are copies of the tile's
// first row; their W entries are zeroed in registers.
// With a shared P the partial spans the whole segment, across users (slot
// s); with one table per user (PU) each (segment, user) piece has its own
// partial (slot s + u).
template <int D, int NW, bool PU>
__global__ __launch_bounds__(NW * 64, 1) void sa_bwdp_bf16(
    const int64_t* __restrict__ offsets, int B, const bf16* __restrict__ X,
    const bf16* __restrict__ W, int kz, int k, int64_t T, int G, float* __restrict__ dpp) {
  // W units (16 bytes) of one tile: 8 prototype tiles x 32 rows x 2 halves x 2.
  constexpr int DB = D / 32;             // 32-row blocks of the transposed partial
  constexpr int U = D / 8;               // 16-byte units per X row
  constexpr int KC = NW * 32;            // prototypes per workgroup
  static_assert(KC == kChunkBf16, "one workgroup covers one prototype chunk");
  constexpr int TILE = 32;
  constexpr int XUN = TILE * U, ZUN = TILE * (KC / 8);
  constexpr int XPW = XUN / NW, ZPW = ZUN / NW;   // units copied by each wave
  static_assert(XUN % NW == 0 && (XPW <= 64 || XPW % 64 == 0), "");
  static_assert(ZPW % 64 == 0, "");
  constexpr int XI = (XPW + 63) / 64, ZI = ZPW / 64;   // copy instructions per wave per tile
  constexpr int L = XI + ZI;             // loads per wave per tile
  constexpr int NBUF = 4, AHEAD = 3;
  constexpr uint32_t XBYTES = TILE * D * 2, ZBYTES = TILE * KC * 2;

  __shared__ __attribute__((aligned(16))) bf16 sX[NBUF][TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 sW[NBUF][TILE * KC];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int s = blockIdx.x, chunk = blockIdx.y;
  const int proto = chunk * KC + wave * 32 + l32;   // this lane's prototype (output column)
  const uint32_t sx0 = lds_addr((const SA_LDS void*)&sX[0][0]);
  const uint32_t sw0 = lds_addr((const SA_LDS void*)&sW[0][0]);
  const SA_LDS char* lds = (const SA_LDS char*)0;

  const int64_t lo = seg_lo(T, G, s), hi = seg_lo(T, G, s + 1);
  TileWalker<TILE> cw_;                // tile being computed
  cw_.start(offsets, B, lo, hi);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  // acc[db] register i is dP[proto][d = 32 db + crow(i, h)].
  auto flush = [&](int64_t slot) {
    if (proto < k) {
      float* dst = dpp + (slot * k + proto) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v = {acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
          *(f32x4*)(dst + 32 * db + 8 * g + 4 * h) = v;
        }
    }
  };

  int guser = -1;
  if (cw_.valid) {
    TileWalker<TILE> qw = cw_;         // next tile to copy

    // Copy geometry.  X: unit v of the tile is row v / U at stored position
    // v % U, holding global unit (v % U) ^ xswz<D>(row).  W: unit v of wave
    // w's 128 is (row (v / 4) % 32, half (v / 2) % 2, 16 bytes v % 2) of
    // prototype tile w of the chunk.
    int xrow[XI], zrow[ZI];
    uint32_t xcol[XI], zcol[ZI];
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // uniform: a scalar base
#pragma unroll
    for (int j = 0; j < XI; ++j) {
      const int v = wave * XPW + j * 64 + lane;
      xrow[j] = v / U;
      xcol[j] = (uint32_t)(((v % U) ^ xswz<D>(v / U)) * 16);
    }
#pragma unroll
    for (int j = 0; j < ZI; ++j) {
      const int v = j * 64 + lane;
      zrow[j] = (v >> 2) & 31;
      zcol[j] = (uint32_t)((((v >> 1) & 1) * 32) * 32 + (v & 1) * 16);   // + 32 (row % 32) later
    }

    // Every wave issues exactly L loads per tile (also past the end of the
    // stream, re-reading the segment's first tile), so that vmcnt counts are
    // the same every time.
    auto copy_next = [&](uint32_t b) {
      const bool valid = qw.valid;
      const int64_t base = valid ? qw.t0 : cw_.t0;
      const int nr = valid ? (int)(qw.t1 - qw.t0) : 1;
      const bf16* xb = X + base * D;
      // W blocks of the stored token tile holding row 0 of this tile, and of
      // the next one (rows may run into it).
      const int64_t tau0 = base >> 5;
      const bf16* zb = W + (tau0 * (kz >> 5) + chunk * NW + wave_s) * 1024;
      const uint32_t nextb = (uint32_t)(kz >> 5) * 2048u;
#pragma unroll
      for (int j = 0; j < XI; ++j) {
        const int r = xrow[j] < nr ? xrow[j] : 0;
        if (XPW >= 64 || lane < XPW)
          lds_copy16(xb, (uint32_t)(r * D * 2) + xcol[j],
                     sx0 + b * XBYTES + (uint32_t)(wave * XPW + j * 64) * 16);
      }
#pragma unroll
      for (int j = 0; j < ZI; ++j) {
        const int r = zrow[j] < nr ? zrow[j] : 0;
        const int tl = (int)(base & 31) + r;              // row within the stored tiles
        lds_copy16(zb, (tl >> 5) * nextb + (uint32_t)(tl & 31) * 32u + zcol[j],
                   sw0 + b * ZBYTES + (uint32_t)(wave * ZPW + j * 64) * 16);
      }
      if (valid) qw.advance();
    };

    guser = cw_.user;
#pragma unroll
    for (int b = 0; b < AHEAD; ++b) copy_next(b);

    // Transpose-read offsets: X^T block db (A operand, rows = d) and this
    // wave's W columns (B operand, columns = its 32 prototypes); token rows
    // 4h + tr_r + 8e (+ 16 kb), so K slot j of half h in block kb is token
    // 16 kb + 8 (j / 4) + 4h + (j % 4) for both operands.
    const int tr_r = (lane & 15) >> 2, tr_c = lane & 3, tr_half = (lane >> 4) & 1;
    uint32_t toff[DB][2], woff[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 4 * h + tr_r + 8 * e;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        toff[db][e] = (uint32_t)(xoff<D>(r, 4 * db + 2 * tr_half + (tr_c >> 1)) + (tr_c & 1) * 4) * 2;
      // columns 4c .. 4c + 3, c = 4 tr_half + tr_c: half c % 2, bytes 8 (c / 2)
      woff[e] = (uint32_t)(wave * 2048 + r * 64 + (tr_c & 1) * 32 + 8 * (2 * tr_half + (tr_c >> 1)));
    }

    uint32_t t = 0;
    while (true) {
      const uint32_t buf = t & (NBUF - 1);
      // Tile t has landed (t + 1 and t + 2 may be in flight); after the
      // barrier every wave's copies of it are visible and nobody reads tile
      // t - 1 any more, whose buffer takes tile t + 3.
      wait_vmcnt<(AHEAD - 1) * L>();
      barrier_lds();
      copy_next((t + AHEAD) & (NBUF - 1));
      if (PU && cw_.user != guser) {
        // The finished piece's partial (its stores only make later vmcnt
        // waits stricter).
        flush((int64_t)s + guser);
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
        guser = cw_.user;
      }
      const int nr = (int)(cw_.t1 - cw_.t0);   // valid rows of this tile
      const SA_LDS char* xs = lds + sx0 + buf * XBYTES;
      const SA_LDS char* ws = lds + sw0 + buf * ZBYTES;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 wt = concat4(lds_read_tr16((const SA_LDS bf16*)(ws + woff[0] + kb * 16 * 64)),
                            lds_read_tr16((const SA_LDS bf16*)(ws + woff[1] + kb * 16 * 64)));
        if (nr < TILE) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (16 * kb + 8 * (j >> 2) + 4 * h + (j & 3) >= nr) wt[j] = (bf16)0.f;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 xt =
              concat4(lds_read_tr16((const SA_LDS bf16*)(xs + toff[db][0] + kb * 16 * D * 2)),
                      lds_read_tr16((const SA_LDS bf16*)(xs + toff[db][1] + kb * 16 * D * 2)));
          acc[db] = mfma32(xt, wt, acc[db]);
        }
      }
      cw_.advance();
      if (!cw_.valid) break;
      ++t;
    }
    wait_vmcnt<0>();   // no copy left in flight
  }
  // This segment's partial (shared P: every segment writes its slot), or the
  // last piece's.
  if (!PU) flush(s);
  else if (guser >= 0) flush((int64_t)s + guser);
}


// ----------------------------------------------------------------------------
// fp32 dX pass.  grid = ceil(T / 32); block 256 = 32 tokens x 8 threads, each
// thread owning D/8 columns.  Prototypes stream through LDS 32 at a time.
// tw: token-wise normalisation, A_ji = exp2(z alpha - lse2_j) with the
// prototype's statistic (lse [B, k], natural log), cv = D_j, and
// dX_i = sum_j (A_ji G_j + c dZ_ji p_j) with no per-token term.
template <int D>
__global__ __launch_bounds__(256) void sa_bwdx_f32(
    const int64_t* __restrict__ offsets, int B, const float* __restrict__ X,
    const float* __restrict__ P, int64_t pstride, const float* __restrict__ Gq,
    const float* __restrict__ cv, int k,
    int64_t T, float alpha, float scale, const float* __restrict__ lse, int tw,
    float* __restrict__ dX, int acc_dx, float* __restrict__ delta_out) {
  constexpr int PC = 32, DS = D / 8;
  __shared__ float sP[PC][D + 4];
  __shared__ float sG[PC][D + 4];
  __shared__ float sC[PC];
  __shared__ float sQ[PC];   // tw: lse2 of the chunk's prototypes
  const int tid = threadIdx.x;
  const int q = tid & 7;
  const int64_t r0 = (int64_t)blockIdx.x * kBwdxTokensF32;
  const int64_t r1 = r0 + kBwdxTokensF32 < T ? r0 + kBwdxTokensF32 : T;
  const int64_t tok = r0 + (tid >> 3);
  float x[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) x[e] = tok < r1 ? X[tok * D + q * DS + e] : 0.f;
  const float l2 = (!tw && tok < r1) ? lse[tok] * kLog2e : INFINITY;

  int u = first_user_after(offsets, B, r0);
  for (; u < B; ++u) {
    const int64_t ulo = clamp64(offsets[u], r0, r1), uhi = clamp64(offsets[u + 1], ulo, r1);
    if (ulo >= r1) break;
    if (uhi <= ulo) continue;
    const bool mine = tok >= ulo && tok < uhi;
    const float lsh = mine ? l2 : INFINITY;
    const float* Gu = Gq + (int64_t)u * k * D;
    const float* Pu = P + (int64_t)u * pstride;   // the user's table (or the shared one)
    float g[DS], aa[DS], bb[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) { g[e] = 0.f; aa[e] = 0.f; bb[e] = 0.f; }
    float dsum = 0.f;
    for (int p0 = 0; p0 < k; p0 += PC) {
      __syncthreads();
      for (int i = tid; i < PC * D; i += 256) {
        const int r = i / D, c = i % D;
        const bool v = p0 + r < k;
        sP[r][c] = v ? Pu[(int64_t)(p0 + r) * D + c] : 0.f;
        sG[r][c] = v ? Gu[(int64_t)(p0 + r) * D + c] : 0.f;
      }
      if (tid < PC) sC[tid] = p0 + tid < k ? cv[(int64_t)u * k + p0 + tid] : 0.f;
      if (tw && tid < PC) sQ[tid] = p0 + tid < k ? lse[(int64_t)u * k + p0 + tid] * kLog2e : INFINITY;
      __syncthreads();
      const int np = k - p0 < PC ? k - p0 : PC;
      for (int j = 0; j < np; ++j) {
        float pz = 0.f, pg = 0.f;
#pragma unroll
        for (int e = 0; e < DS; ++e) {
          pz = fmaf(sP[j][q * DS + e], x[e], pz);
          pg = fmaf(sG[j][q * DS + e], x[e], pg);
        }
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {
          pz += __shfl_xor(pz, off, 64);
          pg += __shfl_xor(pg, off, 64);
        }
        const float a = exp2_fast(fmaf(pz, alpha, -(tw ? sQ[j] : lsh)));
        const float w = a * (pg - sC[j]);
        dsum += w;
#pragma unroll
        for (int e = 0; e < DS; ++e) {
          g[e] = fmaf(a, sG[j][q * DS + e], g[e]);
          aa[e] = fmaf(a, sP[j][q * DS + e], aa[e]);
          bb[e] = fmaf(w, sP[j][q * DS + e], bb[e]);
        }
      }
    }
    if (mine) {
#pragma unroll
      for (int e = 0; e < DS; ++e) {
        const float v = g[e] + scale * (tw ? bb[e] : bb[e] - dsum * aa[e]);
        float* dst = dX + tok * D + q * DS + e;
        *dst = acc_dx ? *dst + v : v;   // acc_dx: add to the caller's dX
      }
      if (q == 0 && !tw) delta_out[tok] = dsum;
    }
  }
}

// fp32 dP pass.  grid = (Gb, ceil(k / 32)); block 256: thread (j = t / 8,
// q = t % 8) owns prototype j, columns q D/8 .. +D/8 of the partial, and
// computes the weights of tokens 4q .. 4q+3 of each 32-token tile.  With one
// table per user (pstride != 0) each (segment, user) piece writes its own
// partial (slot s + u) and a user change reloads the table's rows.
template <int D>
__global__ __launch_bounds__(256) void sa_bwdp_f32(
    const int64_t* __restrict__ offsets, int B, const float* __restrict__ X,
    const float* __restrict__ P, int64_t pstride, const float* __restrict__ Gq,
    const float* __restrict__ cv, int k,
    int64_t T, int G, float alpha, const float* __restrict__ lse, const float* __restrict__ delta,
    int tw, float* __restrict__ dpp) {
  constexpr int PC = kChunkF32Bwd, TILE = 32, DS = D / 8;
  __shared__ float sP[PC][D + 1];
  __shared__ float sG[PC][D + 1];
  __shared__ float sX[TILE][D + 1];
  __shared__ float sZ[PC][TILE + 1];
  __shared__ float sL[TILE], sDl[TILE], sC[PC], sQ[PC];
  const int tid = threadIdx.x;
  const int j = tid >> 3, q = tid & 7;
  const int s = blockIdx.x;
  const int p0 = blockIdx.y * PC;
  float acc[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) acc[e] = 0.f;
  auto flush = [&](int64_t slot) {
    if (p0 + j < k) {
      float* dst = dpp + (slot * k + p0 + j) * D + q * DS;
#pragma unroll
      for (int e = 0; e < DS; ++e) dst[e] = acc[e];
    }
  };

  const int64_t lo = seg_lo(T, G, s), hi = seg_lo(T, G, s + 1);
  TileWalker<TILE> cur;
  cur.start(offsets, B, lo, hi);
  int loaded_user = -1;
  while (cur.valid) {
    __syncthreads();
    if (cur.user != loaded_user) {
      if (pstride != 0 && loaded_user >= 0) {
        flush((int64_t)s + loaded_user);   // the finished piece
#pragma unroll
        for (int e = 0; e < DS; ++e) acc[e] = 0.f;
      }
      const float* Gu = Gq + (int64_t)cur.user * k * D;
      if (pstride != 0 || loaded_user < 0) {
        const float* Pu = P + (int64_t)cur.user * pstride;
        for (int i = tid; i < PC * D; i += 256) {
          const int r = i / D, c = i % D;
          sP[r][c] = (p0 + r < k) ? Pu[(int64_t)(p0 + r) * D + c] : 0.f;
        }
      }
      for (int i = tid; i < PC * D; i += 256) {
        const int r = i / D, c = i % D;
        sG[r][c] = (p0 + r < k) ? Gu[(int64_t)(p0 + r) * D + c] : 0.f;
      }
      if (tid < PC) sC[tid] = p0 + tid < k ? cv[(int64_t)cur.user * k + p0 + tid] : 0.f;
      if (tw && tid < PC)
        sQ[tid] = p0 + tid < k ? lse[(int64_t)cur.user * k + p0 + tid] * kLog2e : INFINITY;
      loaded_user = cur.user;
    }
    for (int i = tid; i < TILE * D; i += 256) {
      const int r = i / D, c = i % D;
      sX[r][c] = (cur.t0 + r < cur.t1) ? X[(cur.t0 + r) * D + c] : 0.f;
    }
    if (!tw && tid < TILE) {
      const bool in = cur.t0 + tid < cur.t1;
      sL[tid] = in ? lse[cur.t0 + tid] * kLog2e : INFINITY;
      sDl[tid] = in ? delta[cur.t0 + tid] : 0.f;
    }
    const int nr = (int)(cur.t1 - cur.t0);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tt = 4 * q + t;
      float z = 0.f, ga = 0.f;
#pragma unroll 8
      for (int e = 0; e < D; ++e) {
        z = fmaf(sP[j][e], sX[tt][e], z);
        ga = fmaf(sG[j][e], sX[tt][e], ga);
      }
      if (tw) {
        const float a = tt < nr ? exp2_fast(fmaf(z, alpha, -sQ[j])) : 0.f;
        sZ[j][tt] = a * (ga - sC[j]);
      } else {
        const float a = exp2_fast(fmaf(z, alpha, -sL[tt]));
        sZ[j][tt] = a * (ga - sC[j] - sDl[tt]);
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int tt = 0; tt < TILE; ++tt) {
      const float dz = sZ[j][tt];
#pragma unroll
      for (int e = 0; e < DS; ++e) acc[e] = fmaf(dz, sX[tt][q * DS + e], acc[e]);
    }
    cur.advance();
  }
  if (pstride == 0) flush(s);
  else if (loaded_user >= 0) flush((int64_t)s + loaded_user);
}

// ----------------------------------------------------------------------------
// dP = c * sum_s dpp[s]; block 0 also checks the offsets.  Block = 4 waves
// over 256 consecutive elements: wave w adds segments w, w + 4, ... (eight
// loads in flight), and the four wave sums are added in wave order, so the
// result does not depend on scheduling.
__global__ __launch_bounds__(256) void sa_dp_reduce(const int64_t* __restrict__ offsets, int B,
                                                    int64_t T, int k, int d, int G, float scale,
                                                    const float* __restrict__ dpp,
                                                    float* __restrict__ dP,
                                                    uint32_t* __restrict__ status) {
  __shared__ f32x4 red[4][64];
  if (blockIdx.x == 0) check_offsets_block(offsets, B, T, status, kStatusOk, kStatusBadOffsets);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t kd = (int64_t)k * d;
  const int64_t e = ((int64_t)blockIdx.x * 64 + lane) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (T > 0 && e < kd) {
    const float* pp = dpp + e;
    int q = wave;
    for (; q + 28 < G; q += 32) {
      f32x4 v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = *(const f32x4*)(pp + (int64_t)(q + 4 * r) * kd);
#pragma unroll
      for (int r = 0; r < 8; ++r) acc += v[r];
    }
    for (; q < G; q += 4) acc += *(const f32x4*)(pp + (int64_t)q * kd);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && e < kd)
    *(f32x4*)(dP + e) = (red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane]) * scale;
}

// ----------------------------------------------------------------------------
template <int D, bool TW, bool CV>
static void launch_bwdx_bf16(const BwdArgs& a, unsigned nbx, bool pu, float alpha, float scale,
                             hipStream_t st) {
  hipLaunchKernelGGL((sa_bwdx_bf16<D, TW, CV>), dim3(nbx), dim3(kBwdxTokensBf16 * 2), 0, st,
                     a.offsets, a.B, (const bf16*)a.X, (const bf16*)a.Pq,
                     (!TW && pu) ? (int64_t)a.kp * D : (int64_t)0, (const bf16*)a.Gq, a.cvs, a.kp,
                     a.T, alpha, scale, a.lse, TW ? (const float*)a.tlse2 : (const float*)nullptr,
                     a.dX, a.acc_dx, a.delta, (bf16*)a.dz, a.kz);
}

template <int D>
static hipError_t launch_bwd_t(const BwdArgs& a, int dtype, hipStream_t st, Prof* prof) {
  const float scale = 1.0f / sqrtf((float)D);
  const float alpha = scale * kLog2e;
  hipError_t e;
  const bool pu = a.pstride != 0;
  const bool tw = a.tokwise != 0;   // token-wise normalisation: lse is [B, k], S required
  if (a.recompute_lse && a.T > 0 && !tw) {
    FwdArgs f = {};
    f.offsets = a.offsets; f.B = a.B; f.pstride = a.pstride;
    f.X = a.X; f.P = a.P; f.k = a.k; f.d = a.d; f.T = a.T; f.lse = a.lse_ws;
    f.lse2 = nullptr;
    e = dtype == 1 ? launch_stats_bf16(f, st, prof) : launch_stats_f32(f, st, prof);
    if (e != hipSuccess) return e;
  }
  // G and cv rows (padded to kp per user), the zero-padded copy of P (bf16),
  // and, token-wise, lse2 per (user, prototype) for the bf16 dX pass.
  const int64_t rows = (int64_t)a.B * a.kp;
  const unsigned nbg = (unsigned)((rows * (D / 4) + 255) / 256);
  const bool bf = dtype == 1;
  const int pq_users = pu ? a.B : 1;
  const unsigned nbq =
      bf ? (unsigned)(((int64_t)pq_users * a.kp * (D / 8) + 255) / 256) : 0u;
  const bool lse2 = bf && a.T > 0 && tw;
  const int64_t nl = tw ? (int64_t)a.B * a.kp : a.T + 1;
  const unsigned nbl = lse2 ? (unsigned)((nl + 255) / 256) : 0u;
  const int mode = tw ? 2 : (a.mass_norm ? 1 : 0);
  float* lse2_out = tw ? a.tlse2 : a.lse2;
  prof_begin(prof, "sa_bwd_prep", st);
  if (bf)
    hipLaunchKernelGGL((sa_bwd_prep<bf16, D>), dim3(nbg + nbq + nbl), dim3(256), 0, st, a.dS, a.S,
                       a.mass, a.B, a.k, a.kp, mode, scale, (bf16*)a.Gq, a.cv, a.cvs, nbg,
                       (const bf16*)a.P, a.pstride, pq_users, (bf16*)a.Pq, nbq, a.lse, a.T,
                       lse2_out);
  else
    hipLaunchKernelGGL((sa_bwd_prep<float, D>), dim3(nbg), dim3(256), 0, st, a.dS, a.S, a.mass,
                       a.B, a.k, a.kp, mode, scale, (float*)a.Gq, a.cv, (float*)nullptr,
                       nbg, (const bf16*)nullptr, (int64_t)0, 1, (bf16*)nullptr, 0u, a.lse, a.T,
                       a.lse2);
  e = hipGetLastError();
  prof_end(prof, st);
  if (e != hipSuccess) return e;
  if (a.T > 0) {
    if (bf) {
      const unsigned nbx = (unsigned)((a.T + kBwdxTokensBf16 - 1) / kBwdxTokensBf16);
      prof_begin(prof, "sa_bwdx_bf16", st);
      // cv is zero for the plain sum.
      if (tw) launch_bwdx_bf16<D, true, true>(a, nbx, pu, alpha, scale, st);
      else if (a.mass_norm) launch_bwdx_bf16<D, false, true>(a, nbx, pu, alpha, scale, st);
      else launch_bwdx_bf16<D, false, false>(a, nbx, pu, alpha, scale, st);
      e = hipGetLastError();
      prof_end(prof, st);
      if (e != hipSuccess) return e;
      prof_begin(prof, "sa_bwdp_bf16", st);
      const dim3 pg(a.Gb, a.bnchunks), pb(64 * kBwdpWaves);
      if (pu && !tw)
        hipLaunchKernelGGL((sa_bwdp_bf16<D, kBwdpWaves, true>), pg, pb, 0, st, a.offsets, a.B,
                           (const bf16*)a.X, (const bf16*)a.dz, a.kz, a.k, a.T, a.Gb, a.dpp);
      else
        hipLaunchKernelGGL((sa_bwdp_bf16<D, kBwdpWaves, false>), pg, pb, 0, st, a.offsets, a.B,
                           (const bf16*)a.X, (const bf16*)a.dz, a.kz, a.k, a.T, a.Gb, a.dpp);
      e = hipGetLastError();
      prof_end(prof, st);
      if (e != hipSuccess) return e;
    } else {
      const unsigned nbx = (unsigned)((a.T + kBwdxTokensF32 - 1) / kBwdxTokensF32);
      prof_begin(prof, "sa_bwdx_f32", st);
      hipLaunchKernelGGL(sa_bwdx_f32<D>, dim3(nbx), dim3(256), 0, st, a.offsets, a.B,
                         (const float*)a.X, (const float*)a.P, a.pstride, (const float*)a.Gq,
                         a.cv, a.k, a.T, alpha, scale, a.lse, tw ? 1 : 0, a.dX, a.acc_dx,
                         a.delta);
      e = hipGetLastError();
      prof_end(prof, st);
      if (e != hipSuccess) return e;
      prof_begin(prof, "sa_bwdp_f32", st);
      hipLaunchKernelGGL(sa_bwdp_f32<D>, dim3(a.Gb, a.bnchunks), dim3(256), 0, st, a.offsets, a.B,
                         (const float*)a.X, (const float*)a.P, a.pstride, (const float*)a.Gq,
                         a.cv, a.k, a.T, a.Gb, alpha, a.lse, a.delta, tw ? 1 : 0, a.dpp);
      e = hipGetLastError();
      prof_end(prof, st);
      if (e != hipSuccess) return e;
    }
  }
  // The bf16 partials already hold c dZ; the fp32 ones dZ.
  const float rscale = bf ? 1.0f : scale;
  if (pu)   // dP[u] = sum of user u's pieces, like the forward's sketch
    return launch_piece_sum(a.offsets, a.B, a.k, a.d, a.T, a.Gb, a.dpp, rscale, a.dP, a.status, st,
                            prof);
  const int64_t kd = (int64_t)a.k * a.d;
  prof_begin(prof, "sa_dp_reduce", st);
  hipLaunchKernelGGL(sa_dp_reduce, dim3((unsigned)((kd + 255) / 256)), dim3(256), 0, st,
                     a.offsets, a.B, a.T, a.k, a.d, a.Gb, rscale, a.dpp, a.dP, a.status);
  e = hipGetLastError();
  prof_end(prof, st);
  return e;
}

hipError_t launch_bwd(const BwdArgs& a, int dtype, hipStream_t st, Prof* prof) {
  switch (a.d) {
    case 32: return launch_bwd_t<32>(a, dtype, st, prof);
    case 64: return launch_bwd_t<64>(a, dtype, st, prof);
    case 128: return launch_bwd_t<128>(a, dtype, st, prof);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
