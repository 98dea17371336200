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
//                 tile: Z and dA' on the matrix cores (Z = P X^T orientation,
//                 token per lane), then g^T, a^T, b^T += {G,P}^T {A,w} with
//                 the A operands read transposed from LDS.  Writes dX and
//                 delta.  10 k d MFMA flops per token.
//  sa_bwdp_bf16:  prototype-stationary (256 prototypes per workgroup, like
//                 the forward aggregation): Z^T, dA'^T, dZ, then
//                 dP^T += X^T dZ^T.  One partial per token segment.  6 k d.
//  sa_dp_reduce:  dP = c sum over segments in order (deterministic).
// The fp32 variants do the same arithmetic on the vector ALU.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

// ----------------------------------------------------------------------------
// G and cv.  One group of D/4 threads per (user, prototype) row.  Blocks from
// nbrows on instead write lse2 = lse log2(e) for the dP pass, with the +inf
// sentinel at index T (when lse2 is not null).
template <typename OutT, int D>
__global__ __launch_bounds__(256) void sa_bwd_prep(const float* __restrict__ dS,
                                                   const float* __restrict__ S,
                                                   const float* __restrict__ mass, int64_t rows,
                                                   int mass_norm, OutT* __restrict__ Gq,
                                                   float* __restrict__ cv, unsigned nbrows,
                                                   const float* __restrict__ lse, int64_t T,
                                                   float* __restrict__ lse2) {
  if (blockIdx.x >= nbrows) {
    const int64_t i = (int64_t)(blockIdx.x - nbrows) * 256 + threadIdx.x;
    if (i < T) lse2[i] = lse[i] * kLog2e;
    else if (i == T) lse2[i] = INFINITY;
    return;
  }
  constexpr int TPR = D / 4;   // threads per row (8, 16 or 32)
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gt / TPR;
  const int part = (int)(gt % TPR);
  const bool live = row < rows;
  const int64_t r = live ? row : 0;
  f32x4 g = *(const f32x4*)(dS + r * D + 4 * part);
  float c = 0.f;
  if (mass_norm) {
    const float mu = mass[r];
    const float inv = mu > 0.f ? 1.0f / mu : 0.f;
    g = mu > 0.f ? g * inv : f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 s = *(const f32x4*)(S + r * D + 4 * part);
    c = g[0] * s[0] + g[1] * s[1] + g[2] * s[2] + g[3] * s[3];
  }
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) c += __shfl_xor(c, off, 64);
  if (live) {
#pragma unroll
    for (int e = 0; e < 4; ++e) Gq[r * D + 4 * part + e] = (OutT)g[e];
    if (part == 0) cv[r] = mass_norm ? c : 0.f;
  }
}

// ----------------------------------------------------------------------------
// bf16 dX pass.  grid = ceil(T / 128); block 256 = 4 waves x 32 tokens.
// Tokens of the workgroup that belong to different users are handled one
// user at a time (the others are masked), because G depends on the user.
// For each user, 64-prototype chunks of P and G (and cv) are copied
// global -> LDS by the direct-to-LDS loads three chunks ahead into four
// buffers (rows stored with the tile swizzle of sa_device.h), one barrier per
// chunk.  Per 32-prototype tile: Z and dA' on the matrix cores (Z = P X^T
// orientation, a token per lane, X rows resident as B operands), the weights
// A and w on the vector ALU, then
//   acc1^T += G^T A + P^T (c w),  acc2^T += P^T A
// with the A operands transpose-read from LDS; dX = acc1 - c delta acc2.
template <int D>
__global__ __launch_bounds__(256, 1) void sa_bwdx_bf16(
    const int64_t* __restrict__ offsets, int B, const bf16* __restrict__ X,
    const bf16* __restrict__ P, const bf16* __restrict__ Gq, const float* __restrict__ cv, int k,
    int64_t T, float alpha, float scale, const float* __restrict__ lse, float* __restrict__ dX,
    float* __restrict__ delta_out) {
  constexpr int KS = D / 16, DB = D / 32, U = D / 8;
  constexpr int PCH = 64;                 // prototypes per chunk
  constexpr int NB = 4, AHEAD = 3;        // chunk buffers, copy distance
  constexpr int CU = PCH * U;             // 16-byte units per matrix chunk
  constexpr int UPW = CU / 4;             // units per wave per matrix
  static_assert(UPW % 64 == 0, "");
  constexpr int XI = UPW / 64;            // copy instructions per wave per matrix
  constexpr int L = 2 * XI + 1;           // loads per wave per chunk
  constexpr uint32_t CBYTES = PCH * D * 2;
  __shared__ __attribute__((aligned(16))) bf16 sP[NB][PCH * D];
  __shared__ __attribute__((aligned(16))) bf16 sG[NB][PCH * D];
  __shared__ __attribute__((aligned(16))) float sC[NB][PCH];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int64_t r0 = (int64_t)blockIdx.x * kBwdxTokensBf16;
  const int64_t r1 = r0 + kBwdxTokensBf16 < T ? r0 + kBwdxTokensBf16 : T;
  const int64_t tok = r0 + wave * 32 + l32;
  const uint32_t sp0 = lds_addr((const SA_LDS void*)&sP[0][0]);
  const uint32_t sg0 = lds_addr((const SA_LDS void*)&sG[0][0]);
  const uint32_t sc0 = lds_addr((const SA_LDS void*)&sC[0][0]);
  const SA_LDS char* lds = (const SA_LDS char*)0;

  bf16x8 xb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    xb[ks] = tok < r1 ? *(const bf16x8*)(X + tok * D + 16 * ks + 8 * h) : bf16x8{};
  const float l2 = tok < r1 ? lse[tok] * kLog2e : INFINITY;

  // Copy geometry (per matrix): instruction j of this wave moves units
  // v0 .. v0 + 63, v0 = wave UPW + 64 j; unit v is row v / U at stored
  // position v % U, holding global unit (v % U) ^ g(row).
  int crow_[XI];
  uint32_t ccol[XI];
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int v = wave * UPW + j * 64 + lane;
    crow_[j] = v / U;
    ccol[j] = (uint32_t)(((v % U) ^ xswz<D>(v / U)) * 16);
  }
  // LDS byte offsets within a chunk buffer (prototype rows).
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
  const uint32_t cqoff = (uint32_t)(4 * h) * 4;
  const int nch = (k + PCH - 1) / PCH;

  int u = first_user_after(offsets, B, r0);
  for (; u < B; ++u) {
    const int64_t ulo = clamp64(uload64(offsets + u), r0, r1);
    const int64_t uhi = clamp64(uload64(offsets + u + 1), ulo, r1);
    if (ulo >= r1) break;
    if (uhi <= ulo) continue;
    const bool mine = tok >= ulo && tok < uhi;
    const float lsh = mine ? l2 : INFINITY;
    const bf16* Gu = Gq + (int64_t)u * k * D;
    const float* cvu = cv + (int64_t)u * k;

    // Copy chunk c (rows past k repeat row k - 1, and cv past k reads
    // cv[k - 1]; their weights are zeroed below) into buffer b.  Every wave
    // issues exactly L loads per chunk, also for chunks past the end.
    auto copy_chunk = [&](int c, uint32_t b) {
      const int p0 = c < nch ? c * PCH : 0;
#pragma unroll
      for (int j = 0; j < XI; ++j) {
        const int row = min(p0 + crow_[j], k - 1);
        const uint32_t dst = b * CBYTES + (uint32_t)(wave * UPW + j * 64) * 16;
        lds_copy16(P, (uint32_t)row * (D * 2) + ccol[j], sp0 + dst);
        lds_copy16(Gu, (uint32_t)row * (D * 2) + ccol[j], sg0 + dst);
      }
      if (lane < PCH / 4)
        lds_copy4v(cvu + min(p0 + wave * (PCH / 4) + lane, k - 1),
                   sc0 + (b * PCH + wave * (PCH / 4)) * 4);
    };

    // acc1 = g + c b = sum_j (A_ji G_j + c w_ji p_j) (one accumulator for
    // both products), acc2 = a = sum_j A_ji p_j.
    f32x16 acc1[DB], acc2[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { acc1[db] = f32x16{}; acc2[db] = f32x16{}; }
    float dsum = 0.f;

    barrier_lds();   // the previous user's chunks are fully consumed
#pragma unroll
    for (int c = 0; c < AHEAD; ++c) copy_chunk(c, c);
    wait_vmcnt<0>();
    barrier_lds();
    for (int ci = 0; ci < nch; ++ci) {
      const uint32_t buf = ci & (NB - 1);
      copy_chunk(ci + AHEAD, (ci + AHEAD) & (NB - 1));   // into the buffer of chunk ci - 1
      const SA_LDS char* ps = lds + sp0 + buf * CBYTES;
      const SA_LDS char* gs = lds + sg0 + buf * CBYTES;
      const SA_LDS char* cs = lds + sc0 + buf * (PCH * 4) + cqoff;
#pragma unroll
      for (int pt = 0; pt < PCH / 32; ++pt) {
        const int pbase = ci * PCH + pt * 32;
        if (pbase >= k) break;   // uniform
        const uint32_t rb = (uint32_t)(pt * 32 * D * 2);   // byte offset of the tile's rows
        // Z and dA' tiles: rows = prototypes pbase + crow(i, h), column = token.
        f32x16 z = f32x16{}, da = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 ap = *(const SA_LDS bf16x8*)(ps + rb + aoff[ks]);
          const bf16x8 agr = *(const SA_LDS bf16x8*)(gs + rb + aoff[ks]);
          z = mfma32(ap, xb[ks], z);
          da = mfma32(agr, xb[ks], da);
        }
        f32x4 cq[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) cq[g4] = *(const SA_LDS f32x4*)(cs + pt * 128 + 32 * g4);
        const bool partial = pbase + 32 > k;
        bf16x8 abf[2], wbf[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float a = exp2_fast(fmaf(z[i], alpha, -lsh));
          if (partial && pbase + crow(i, h) >= k) a = 0.f;
          const float w = a * (da[i] - cq[i >> 2][i & 3]);
          dsum += w;
          abf[i >> 3][i & 7] = (bf16)a;
          wbf[i >> 3][i & 7] = (bf16)(scale * w);
        }
        // {acc1, acc2}^T (d x tokens) += {G, P, P}^T (d x prototypes) {A, c w, A}.
        // K slot j of half h in block kb is prototype 16 kb + 8 (j / 4) + 4h + (j % 4).
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const uint32_t o0 = rb + (uint32_t)(kb * 16 * D * 2) + toff[db][0];
            const uint32_t o1 = rb + (uint32_t)(kb * 16 * D * 2) + toff[db][1];
            const bf16x8 gT = concat4(lds_read_tr16((const SA_LDS bf16*)(gs + o0)),
                                      lds_read_tr16((const SA_LDS bf16*)(gs + o1)));
            const bf16x8 pT = concat4(lds_read_tr16((const SA_LDS bf16*)(ps + o0)),
                                      lds_read_tr16((const SA_LDS bf16*)(ps + o1)));
            acc1[db] = mfma32(gT, abf[kb], acc1[db]);
            acc1[db] = mfma32(pT, wbf[kb], acc1[db]);
            acc2[db] = mfma32(pT, abf[kb], acc2[db]);
          }
        }
      }
      // Chunk ci + 1 must be complete before the barrier; chunks ci + 2 and
      // ci + 3 may still be in flight.
      wait_vmcnt<2 * L>();
      barrier_lds();
    }
    wait_vmcnt<0>();

    const float delta = dsum + shfl_xor32(dsum);
    if (mine) {
      // C layout: lane -> token, register i -> d = 32 db + crow(i, h).
      float* dst = dX + tok * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * g4 + r;
            v[r] = acc1[db][i] - scale * delta * acc2[db][i];
          }
          *(f32x4*)(dst + 32 * db + 8 * g4 + 4 * h) = v;
        }
      if (h == 0) delta_out[tok] = delta;
    }
  }
}

// ----------------------------------------------------------------------------
// bf16 dP pass.  grid = (Gb segments, nchunks); block = NW waves x 32
// prototypes, the tiling and copy pipeline of the forward aggregation:
// 32-token tiles copied global -> LDS (X, lse2, delta) six tiles ahead into
// eight buffers, a barrier after every second tile.  Per tile: Z^T and dA'^T
// (matrix cores), dZ (vector ALU), dP^T += X^T dZ^T (matrix cores).  The
// partial spans the whole segment, across users (P is shared).
//
// lse2 holds the log-sum-exp in log2 units with lse2[T] = +inf, which rows
// past the end of a tile read (weight 0, so dZ = 0).
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 1) void sa_bwdp_bf16(
    const int64_t* __restrict__ offsets, int B, const bf16* __restrict__ X,
    const bf16* __restrict__ P, const bf16* __restrict__ Gq, const float* __restrict__ cv, int k,
    int64_t T, int G, float alpha, const float* __restrict__ lse2, const float* __restrict__ delta,
    float* __restrict__ dpp) {
  constexpr int KS = D / 16;             // reduction steps over d
  constexpr int DB = D / 32;             // 32-row blocks of the transposed partial
  constexpr int U = D / 8;               // 16-byte units per token row
  constexpr int KC = NW * 32;            // prototypes per workgroup
  static_assert(KC == kChunkBf16, "one workgroup covers one prototype chunk");
  constexpr int TILE = 32;
  constexpr int UNITS = TILE * U;
  constexpr int UPW = UNITS / NW;        // units copied by each wave
  static_assert(UNITS % NW == 0 && (UPW <= 64 || UPW % 64 == 0), "");
  constexpr int XI = (UPW + 63) / 64;    // X copy instructions per wave per tile
  constexpr int LPW = TILE / NW;         // lse and delta entries copied by each wave
  constexpr int NBUF = 8, AHEAD = 6;
  constexpr int L = XI + 2;              // loads per wave per tile
  constexpr uint32_t XBYTES = TILE * D * 2;

  __shared__ __attribute__((aligned(16))) bf16 sX[NBUF][TILE * D];
  __shared__ __attribute__((aligned(16))) float sL[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) float sD[NBUF][TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int s = blockIdx.x, chunk = blockIdx.y;
  const int proto = chunk * KC + wave * 32 + l32;   // this lane's prototype
  const int prow = proto < k ? proto : k - 1;       // rows past k: results unused
  const uint32_t sx0 = lds_addr((const SA_LDS void*)&sX[0][0]);
  const uint32_t sl0 = lds_addr((const SA_LDS void*)&sL[0][0]);
  const uint32_t sd0 = lds_addr((const SA_LDS void*)&sD[0][0]);
  const SA_LDS char* lds = (const SA_LDS char*)0;

  // B operands: pw[ks] = P[proto][16 ks + 8h .. +7], gw likewise for the
  // current user's G; cw = cv[user][proto].
  bf16x8 pw[KS], gw[KS];
  float cw;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) pw[ks] = *(const bf16x8*)(P + (int64_t)prow * D + 16 * ks + 8 * h);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  const int64_t lo = seg_lo(T, G, s), hi = seg_lo(T, G, s + 1);
  TileWalker<TILE> cw_;                // tile being computed
  cw_.start(offsets, B, lo, hi);
  if (cw_.valid) {
    TileWalker<TILE> qw = cw_;         // next tile to copy

    int crow_[XI];
    uint32_t ccol[XI];
#pragma unroll
    for (int j = 0; j < XI; ++j) {
      const int v = wave * UPW + j * 64 + lane;
      crow_[j] = v / U;
      ccol[j] = (uint32_t)(((v % U) ^ xswz<D>(v / U)) * 16);
    }
    const int lrow = wave * LPW + lane;

    // Every wave issues exactly L loads per tile (also past the end of the
    // stream), so that vmcnt counts are the same every time.
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
      if (lane < LPW) {
        const bool in = lrow < nr;
        lds_copy4v(in ? lse2 + base + lrow : lse2 + T, sl0 + (b * TILE + wave * LPW) * 4);
        lds_copy4v(delta + base + (in ? lrow : 0), sd0 + (b * TILE + wave * LPW) * 4);
      }
      if (valid) qw.advance();
    };

    int guser = cw_.user;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      gw[ks] = *(const bf16x8*)(Gq + ((int64_t)guser * k + prow) * D + 16 * ks + 8 * h);
    cw = cv[(int64_t)guser * k + prow];
#pragma unroll
    for (int b = 0; b < AHEAD; ++b) copy_next(b);
    // The compiler must see the waits for the operand loads above here, not
    // inside the loop (where they would also wait for every copy in flight).
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(pw[ks]), "v"(gw[ks]));
    asm volatile("" ::"v"(cw));
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
    const uint32_t lqoff = (uint32_t)(4 * h) * 4;

    uint32_t t = 0;
    while (true) {
      const uint32_t buf = t & (NBUF - 1);
      copy_next((t + AHEAD) & (NBUF - 1));
      if (cw_.user != guser) {
        // A new user: its G rows and cv (rare; waits for the loads here).
        guser = cw_.user;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          gw[ks] = *(const bf16x8*)(Gq + ((int64_t)guser * k + prow) * D + 16 * ks + 8 * h);
        cw = cv[(int64_t)guser * k + prow];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(gw[ks]));
        asm volatile("" ::"v"(cw));
      }

      const SA_LDS char* xs = lds + sx0 + buf * XBYTES;
      // Z^T and dA'^T (tokens x prototypes) of this tile.
      f32x16 z = f32x16{}, da = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = *(const SA_LDS bf16x8*)(xs + aoff[ks]);
        z = mfma32(a, pw[ks], z);
        da = mfma32(a, gw[ks], da);
      }
      // dZ = A (dA' - cv - delta); register i of a lane is token crow(i, h).
      const SA_LDS char* ls = lds + sl0 + buf * (TILE * 4) + lqoff;
      const SA_LDS char* ds = lds + sd0 + buf * (TILE * 4) + lqoff;
      f32x4 lq[4], dq[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        lq[g] = *(const SA_LDS f32x4*)(ls + 32 * g);
        dq[g] = *(const SA_LDS f32x4*)(ds + 32 * g);
      }
      bf16x8 zbf[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = exp2_fast(fmaf(z[i], alpha, -lq[i >> 2][i & 3]));
        zbf[i >> 3][i & 7] = (bf16)(a * (da[i] - cw - dq[i >> 2][i & 3]));
      }
      // dP^T (d x prototypes) += X^T (d x tokens) dZ^T (tokens x prototypes).
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const SA_LDS char* p0 = xs + toff[db][0];
        const SA_LDS char* p1 = xs + toff[db][1];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 xt = concat4(lds_read_tr16((const SA_LDS bf16*)(p0 + kb * 32 * D)),
                                    lds_read_tr16((const SA_LDS bf16*)(p1 + kb * 32 * D)));
          acc[db] = mfma32(xt, zbf[kb], acc[db]);
        }
      }

      cw_.advance();
      if (!cw_.valid) break;
      if (t & 1) {
        // The next two steps read tiles up to t+2; t+3 .. t+6 may be in flight.
        wait_vmcnt<4 * L>();
        barrier_lds();
      }
      ++t;
    }
    wait_vmcnt<0>();   // no copy left in flight
  }
  // Flush this segment's partial: acc[db] register i is
  // dP[proto][d = 32 db + crow(i, h)] / c.
  if (proto < k) {
    float* dst = dpp + ((int64_t)s * k + proto) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
        *(f32x4*)(dst + 32 * db + 8 * g + 4 * h) = v;
      }
  }
}


// ----------------------------------------------------------------------------
// fp32 dX pass.  grid = ceil(T / 32); block 256 = 32 tokens x 8 threads, each
// thread owning D/8 columns.  Prototypes stream through LDS 32 at a time.
template <int D>
__global__ __launch_bounds__(256) void sa_bwdx_f32(
    const int64_t* __restrict__ offsets, int B, const float* __restrict__ X,
    const float* __restrict__ P, const float* __restrict__ Gq, const float* __restrict__ cv, int k,
    int64_t T, float alpha, float scale, const float* __restrict__ lse, float* __restrict__ dX,
    float* __restrict__ delta_out) {
  constexpr int PC = 32, DS = D / 8;
  __shared__ float sP[PC][D + 4];
  __shared__ float sG[PC][D + 4];
  __shared__ float sC[PC];
  const int tid = threadIdx.x;
  const int q = tid & 7;
  const int64_t r0 = (int64_t)blockIdx.x * kBwdxTokensF32;
  const int64_t r1 = r0 + kBwdxTokensF32 < T ? r0 + kBwdxTokensF32 : T;
  const int64_t tok = r0 + (tid >> 3);
  float x[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) x[e] = tok < r1 ? X[tok * D + q * DS + e] : 0.f;
  const float l2 = tok < r1 ? lse[tok] * kLog2e : INFINITY;

  int u = first_user_after(offsets, B, r0);
  for (; u < B; ++u) {
    const int64_t ulo = clamp64(offsets[u], r0, r1), uhi = clamp64(offsets[u + 1], ulo, r1);
    if (ulo >= r1) break;
    if (uhi <= ulo) continue;
    const bool mine = tok >= ulo && tok < uhi;
    const float lsh = mine ? l2 : INFINITY;
    const float* Gu = Gq + (int64_t)u * k * D;
    float g[DS], aa[DS], bb[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) { g[e] = 0.f; aa[e] = 0.f; bb[e] = 0.f; }
    float dsum = 0.f;
    for (int p0 = 0; p0 < k; p0 += PC) {
      __syncthreads();
      for (int i = tid; i < PC * D; i += 256) {
        const int r = i / D, c = i % D;
        const bool v = p0 + r < k;
        sP[r][c] = v ? P[(int64_t)(p0 + r) * D + c] : 0.f;
        sG[r][c] = v ? Gu[(int64_t)(p0 + r) * D + c] : 0.f;
      }
      if (tid < PC) sC[tid] = p0 + tid < k ? cv[(int64_t)u * k + p0 + tid] : 0.f;
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
        const float a = exp2_fast(fmaf(pz, alpha, -lsh));
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
      for (int e = 0; e < DS; ++e) dX[tok * D + q * DS + e] = g[e] + scale * (bb[e] - dsum * aa[e]);
      if (q == 0) delta_out[tok] = dsum;
    }
  }
}

// fp32 dP pass.  grid = (Gb, ceil(k / 32)); block 256: thread (j = t / 8,
// q = t % 8) owns prototype j, columns q D/8 .. +D/8 of the partial, and
// computes the weights of tokens 4q .. 4q+3 of each 32-token tile.
template <int D>
__global__ __launch_bounds__(256) void sa_bwdp_f32(
    const int64_t* __restrict__ offsets, int B, const float* __restrict__ X,
    const float* __restrict__ P, const float* __restrict__ Gq, const float* __restrict__ cv, int k,
    int64_t T, int G, float alpha, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dpp) {
  constexpr int PC = kChunkF32Bwd, TILE = 32, DS = D / 8;
  __shared__ float sP[PC][D + 1];
  __shared__ float sG[PC][D + 1];
  __shared__ float sX[TILE][D + 1];
  __shared__ float sZ[PC][TILE + 1];
  __shared__ float sL[TILE], sDl[TILE], sC[PC];
  const int tid = threadIdx.x;
  const int j = tid >> 3, q = tid & 7;
  const int s = blockIdx.x;
  const int p0 = blockIdx.y * PC;
  for (int i = tid; i < PC * D; i += 256) {
    const int r = i / D, c = i % D;
    sP[r][c] = (p0 + r < k) ? P[(int64_t)(p0 + r) * D + c] : 0.f;
  }
  float acc[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) acc[e] = 0.f;

  const int64_t lo = seg_lo(T, G, s), hi = seg_lo(T, G, s + 1);
  TileWalker<TILE> cur;
  cur.start(offsets, B, lo, hi);
  int loaded_user = -1;
  while (cur.valid) {
    __syncthreads();
    if (cur.user != loaded_user) {
      const float* Gu = Gq + (int64_t)cur.user * k * D;
      for (int i = tid; i < PC * D; i += 256) {
        const int r = i / D, c = i % D;
        sG[r][c] = (p0 + r < k) ? Gu[(int64_t)(p0 + r) * D + c] : 0.f;
      }
      if (tid < PC) sC[tid] = p0 + tid < k ? cv[(int64_t)cur.user * k + p0 + tid] : 0.f;
      loaded_user = cur.user;
    }
    for (int i = tid; i < TILE * D; i += 256) {
      const int r = i / D, c = i % D;
      sX[r][c] = (cur.t0 + r < cur.t1) ? X[(cur.t0 + r) * D + c] : 0.f;
    }
    if (tid < TILE) {
      const bool in = cur.t0 + tid < cur.t1;
      sL[tid] = in ? lse[cur.t0 + tid] * kLog2e : INFINITY;
      sDl[tid] = in ? delta[cur.t0 + tid] : 0.f;
    }
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
      const float a = exp2_fast(fmaf(z, alpha, -sL[tt]));
      sZ[j][tt] = a * (ga - sC[j] - sDl[tt]);
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
  if (p0 + j < k) {
    float* dst = dpp + ((int64_t)s * k + p0 + j) * D + q * DS;
#pragma unroll
    for (int e = 0; e < DS; ++e) dst[e] = acc[e];
  }
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
template <int D>
static hipError_t launch_bwd_t(const BwdArgs& a, int dtype, hipStream_t st, Prof* prof) {
  const float scale = 1.0f / sqrtf((float)D);
  const float alpha = scale * kLog2e;
  hipError_t e;
  if (a.recompute_lse && a.T > 0) {
    FwdArgs f = {};
    f.X = a.X; f.P = a.P; f.k = a.k; f.d = a.d; f.T = a.T; f.lse = a.lse_ws;
    f.lse2 = dtype == 1 ? a.lse2 : nullptr;
    e = dtype == 1 ? launch_stats_bf16(f, st, prof) : launch_stats_f32(f, st, prof);
    if (e != hipSuccess) return e;
  }
  const int64_t rows = (int64_t)a.B * a.k;
  const unsigned nbp = (unsigned)((rows * (D / 4) + 255) / 256);
  // The bf16 dP pass reads lse in log2 units; when the caller supplied lse
  // (not recomputed above), the prep kernel's extra blocks convert it.
  const bool lse2 = dtype == 1 && a.T > 0 && !a.recompute_lse;
  const unsigned nbl = lse2 ? (unsigned)((a.T + 1 + 255) / 256) : 0u;
  prof_begin(prof, "sa_bwd_prep", st);
  if (dtype == 1)
    hipLaunchKernelGGL((sa_bwd_prep<bf16, D>), dim3(nbp + nbl), dim3(256), 0, st, a.dS, a.S, a.mass,
                       rows, a.mass_norm, (bf16*)a.Gq, a.cv, nbp, a.lse, a.T, a.lse2);
  else
    hipLaunchKernelGGL((sa_bwd_prep<float, D>), dim3(nbp), dim3(256), 0, st, a.dS, a.S, a.mass,
                       rows, a.mass_norm, (float*)a.Gq, a.cv, nbp, a.lse, a.T, a.lse2);
  e = hipGetLastError();
  prof_end(prof, st);
  if (e != hipSuccess) return e;
  if (a.T > 0) {
    if (dtype == 1) {
      const unsigned nbx = (unsigned)((a.T + kBwdxTokensBf16 - 1) / kBwdxTokensBf16);
      prof_begin(prof, "sa_bwdx_bf16", st);
      hipLaunchKernelGGL(sa_bwdx_bf16<D>, dim3(nbx), dim3(256), 0, st, a.offsets, a.B,
                         (const bf16*)a.X, (const bf16*)a.P, (const bf16*)a.Gq, a.cv, a.k, a.T,
                         alpha, scale, a.lse, a.dX, a.delta);
      e = hipGetLastError();
      prof_end(prof, st);
      if (e != hipSuccess) return e;
      prof_begin(prof, "sa_bwdp_bf16", st);
      hipLaunchKernelGGL((sa_bwdp_bf16<D, kBwdpWaves>), dim3(a.Gb, a.bnchunks), dim3(64 * kBwdpWaves),
                         0, st, a.offsets, a.B, (const bf16*)a.X, (const bf16*)a.P,
                         (const bf16*)a.Gq, a.cv, a.k, a.T, a.Gb, alpha, a.lse2, a.delta, a.dpp);
      e = hipGetLastError();
      prof_end(prof, st);
      if (e != hipSuccess) return e;
    } else {
      const unsigned nbx = (unsigned)((a.T + kBwdxTokensF32 - 1) / kBwdxTokensF32);
      prof_begin(prof, "sa_bwdx_f32", st);
      hipLaunchKernelGGL(sa_bwdx_f32<D>, dim3(nbx), dim3(256), 0, st, a.offsets, a.B,
                         (const float*)a.X, (const float*)a.P, (const float*)a.Gq, a.cv, a.k, a.T,
                         alpha, scale, a.lse, a.dX, a.delta);
      e = hipGetLastError();
      prof_end(prof, st);
      if (e != hipSuccess) return e;
      prof_begin(prof, "sa_bwdp_f32", st);
      hipLaunchKernelGGL(sa_bwdp_f32<D>, dim3(a.Gb, a.bnchunks), dim3(256), 0, st, a.offsets, a.B,
                         (const float*)a.X, (const float*)a.P, (const float*)a.Gq, a.cv, a.k, a.T,
                         a.Gb, alpha, a.lse, a.delta, a.dpp);
      e = hipGetLastError();
      prof_end(prof, st);
      if (e != hipSuccess) return e;
    }
  }
  const int64_t kd = (int64_t)a.k * a.d;
  prof_begin(prof, "sa_dp_reduce", st);
  hipLaunchKernelGGL(sa_dp_reduce, dim3((unsigned)((kd + 255) / 256)), dim3(256), 0, st,
                     a.offsets, a.B, a.T, a.k, a.d, a.Gb, scale, a.dpp, a.dP, a.status);
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
