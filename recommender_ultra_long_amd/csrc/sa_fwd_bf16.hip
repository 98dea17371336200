// sa_fwd_bf16.hip — Sketch Attention forward, bf16 inputs, fp32 accumulation,
// matrix cores (v_mfma_f32_32x32x16_bf16) for both contractions.
//
// Method: SequenceO1 reading notes, section 3.1, Eq. (6)-(9); FlashSA
// paragraph of the paper's HTML page (streamed affinities, per-token max and
// log-sum-exp, aggregation, no k x n matrix in memory).
//
// Two passes over the history, because the softmax normalises over all k
// prototypes of a token while one compute unit cannot hold the k x d fp32
// accumulator for k = 1024 (512 KiB, the whole register file):
//
//  1. sa_stats_bf16: token-stationary.  Each wave keeps 32 tokens' rows in
//     registers as MFMA B operands (four waves per SIMD, so that one wave's
//     products overlap another's exponentials), streams every prototype
//     through LDS, and
//     reduces the per-token max and sum of exponentials inside each lane
//     (orientation Z = P X^T puts a token in each lane and prototypes in the
//     registers).  Writes lse (natural log) per token.
//  2. sa_agg_bf16: prototype-stationary.  A workgroup owns 256 prototypes
//     (waves x prototype tiles, B operands in registers, fp32 accumulators in
//     AGPRs) and a contiguous segment of tokens.  Per 32-token tile:
//     Z^T = X P_w^T on the matrix cores, A = exp2(Z alpha - lse2) in
//     registers, then U^T += X^T A^T, whose B operand is the first product's C
//     fragment as is (prototype per lane, tokens per register) and whose A
//     operand (X^T) is read from the LDS tile with the gfx950 transpose read.
//     Partial sketches go to a workspace slot per (segment, user) piece;
//     sa_reduce sums them in segment order.
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

// ----------------------------------------------------------------------------
// Pass 1: per-token log-sum-exp over all k prototypes.
// Block: 256 tokens in NW = 8 / NT waves; wave w handles tokens
// blk*256 + 32 NT w .. +32 NT - 1 as NT 32-token MFMA tiles.  With NT = 1 (the
// shared table at d >= 64) two blocks give every SIMD four waves, which keeps
// the matrix cores fed while other waves exponentiate (measured 38.4 -> 36.6
// us at 100,000 tokens, k = 1024, d = 128, against NT = 2 with two waves per
// SIMD); each prototype fragment read from LDS then feeds one product instead
// of two.  Prototypes stream through LDS in chunks of 64 rows, stored in MFMA fragment order and copied global -> LDS by the
// direct-to-LDS loads three chunks ahead into four buffers, one barrier per
// chunk.  Every block reads the same chunk at about the same time, so the
// first request for a chunk's lines usually goes past the L2; the copies are
// issued early enough to cover that latency.
// With one table per user (PU), the block makes one pass over the prototypes
// per user among its tokens, with that user's table, and each pass writes the
// statistics of its user's tokens only.
#ifndef SA_STATS_TILES
#define SA_STATS_TILES 1
#endif
template <int D, bool PU, int NT>
__global__ __launch_bounds__(512 / NT, 2) void sa_stats_bf16(const bf16* __restrict__ X,
                                                     const bf16* __restrict__ P, int k,
                                                     int64_t T, float alpha, float scale,
                                                     float* __restrict__ lse_out,
                                                     float* __restrict__ lse2_out,
                                                     const int64_t* __restrict__ offsets, int B,
                                                     int64_t pstride) {
  constexpr int KS = D / 16;            // 16-wide reduction steps over d
  constexpr int PCH = 64;               // prototypes per LDS chunk
  constexpr int NPIECE = PCH * D / 8;   // 16-byte slots per chunk
  constexpr int NW = 8 / NT;            // waves per block
  static_assert(NT == 1 || NT == 2, "");
  constexpr int SPW = NPIECE / NW;      // slots copied by each wave
  constexpr int XI = SPW / 64;          // copy instructions per wave per chunk
  static_assert(SPW % 64 == 0 && XI >= 1, "");
  constexpr int NB = 4;                 // chunk buffers
  constexpr uint32_t CBYTES = NPIECE * 16;
  __shared__ __attribute__((aligned(16))) bf16x8 sP[NB][NPIECE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int64_t tok0 = (int64_t)blockIdx.x * 256 + wave * 32 * NT;
  const uint32_t sp0 = lds_addr((const SA_LDS void*)&sP[0][0]);
  const int nch = (k + PCH - 1) / PCH;

  // Copy geometry.  Slot (pt KS + ks) 64 + L of a chunk buffer is lane L's A
  // operand for prototype tile pt and step ks: chunk row 32 pt + L % 32,
  // 16-byte unit 2 ks + L / 32.  Copy instruction j of this wave fills the
  // slots wave SPW + 64 j + lane (consecutive lanes, consecutive slots: the
  // reads below are free of bank conflicts).
  int crow_[XI];
  uint32_t cunit[XI];
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int slot = wave * SPW + 64 * j + lane;
    crow_[j] = (slot / (KS * 64)) * 32 + l32;
    cunit[j] = (uint32_t)(2 * ((slot / 64) % KS) + h) * 16;
  }
  const bf16* Pu = P;                    // the current user's table
  // Copy chunk q of the stream into buffer q % NB: prototype chunk q while
  // q < nch, afterwards chunk 0 again (never read), so that every chunk is
  // the same number of loads.  Rows past k copy row k - 1; the last chunk
  // masks them.
  auto copy_chunk = [&](int q) {
    const int c = q < nch ? q : 0;
    const uint32_t dst = sp0 + (uint32_t)(q & (NB - 1)) * CBYTES + (uint32_t)(wave * SPW) * 16;
#pragma unroll
    for (int j = 0; j < XI; ++j) {
      const int row = c * PCH + crow_[j] < k ? c * PCH + crow_[j] : k - 1;
      lds_copy16(Pu, (uint32_t)row * (uint32_t)(D * 2) + cunit[j], dst + 1024 * j);
    }
  };

  // The first pass's chunks are requested before the token rows, so that
  // both streams are in flight together.
  if constexpr (PU) Pu = P + (int64_t)first_user_after(offsets, B, (int64_t)blockIdx.x * 256) * pstride;
#pragma unroll
  for (int q = 0; q < 3; ++q) copy_chunk(q);
  bool primed = true;

  // This lane's token rows as B operands: xb[tt][ks] = X[tok][16 ks + 8h .. +7].
  bf16x8 xb[NT][KS];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int64_t tok = tok0 + tt * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (tok < T) xb[tt][ks] = *(const bf16x8*)(X + tok * D + 16 * ks + 8 * h);
      else xb[tt][ks] = bf16x8{};
    }
  }
  // The compiler waits for the rows here, where it also sees the wait, and
  // adds none inside the loops (where it would hold up every copy in flight).
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(xb[tt][ks]));

  // Per-token statistics of one pass, per lane (its token, half h of the
  // prototypes): ref = reference maximum, l = sum of exp2((z - ref) alpha).
  float ref[NT], l[NT];

  // Exact form (running maximum, the sum rescaled whenever it grows).  Folds
  // one 32-prototype x 32-token product tile (register i of a lane is
  // prototype crow(i, h) of the tile, the lane's token is tt 32 + l32).
  auto fold_exact = [&](const f32x16& v, int tt) {
    float t0 = fmaxf(fmaxf(v[0], v[1]), v[2]), t1 = fmaxf(fmaxf(v[3], v[4]), v[5]);
    float t2 = fmaxf(fmaxf(v[6], v[7]), v[8]), t3 = fmaxf(fmaxf(v[9], v[10]), v[11]);
    float t4 = fmaxf(fmaxf(v[12], v[13]), fmaxf(v[14], v[15]));
    const float tmax = fmaxf(fmaxf(fmaxf(t0, t1), t2), fmaxf(t3, t4));
    const float mnew = fmaxf(ref[tt], tmax);
    // A lane whose prototypes are all padding so far keeps m = -inf; a zero
    // shift then keeps every term at exp2(-inf) = 0 instead of NaN.
    const float ma = mnew == -INFINITY ? 0.f : mnew * alpha;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      s0 += exp2_fast(fmaf(v[i], alpha, -ma));
      s1 += exp2_fast(fmaf(v[i + 1], alpha, -ma));
      s2 += exp2_fast(fmaf(v[i + 2], alpha, -ma));
      s3 += exp2_fast(fmaf(v[i + 3], alpha, -ma));
    }
    l[tt] = fmaf(l[tt], exp2_fast(fmaf(ref[tt], alpha, -ma)), (s0 + s1) + (s2 + s3));
    ref[tt] = mnew;
  };
  // Fast form: the reference is the maximum over the first tile and stays
  // fixed, so a fold is one fma, one exp2 and one add per product.  A term
  // overflows only when a later product exceeds the reference by more than
  // 128 / alpha; the pass then ends with a non-finite sum and is redone in
  // the exact form.
  auto fold_fast = [&](const f32x16& v, int tt) {
    const float ma = ref[tt] * alpha;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      s0 += exp2_fast(fmaf(v[i], alpha, -ma));
      s1 += exp2_fast(fmaf(v[i + 1], alpha, -ma));
      s2 += exp2_fast(fmaf(v[i + 2], alpha, -ma));
      s3 += exp2_fast(fmaf(v[i + 3], alpha, -ma));
    }
    l[tt] += (s0 + s1) + (s2 + s3);
  };
  auto set_ref = [&](const f32x16& v, int tt) {
    float t0 = fmaxf(fmaxf(v[0], v[1]), v[2]), t1 = fmaxf(fmaxf(v[3], v[4]), v[5]);
    float t2 = fmaxf(fmaxf(v[6], v[7]), v[8]), t3 = fmaxf(fmaxf(v[9], v[10]), v[11]);
    float t4 = fmaxf(fmaxf(v[12], v[13]), fmaxf(v[14], v[15]));
    const float tmax = fmaxf(fmaxf(fmaxf(t0, t1), t2), fmaxf(t3, t4));
    // all padding (k < 32): any finite reference; the lane's sum stays 0
    ref[tt] = tmax == -INFINITY ? 0.f : tmax;
  };

  // Products of prototype tile pt of the chunk in LDS buffer buf.
  using Tiles = f32x16[NT];
  auto products = [&](int buf, int pt, Tiles& c) {
    {
      const bf16x8 a = sP[buf][(pt * KS) * 64 + lane];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) c[tt] = mfma32(a, xb[tt][0], f32x16{});
    }
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) {
      const bf16x8 a = sP[buf][(pt * KS + ks) * 64 + lane];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) c[tt] = mfma32(a, xb[tt][ks], c[tt]);
    }
  };

  // One pass over all prototypes of table Pu; writes the statistics of the
  // tokens in [ulo, uhi).  Returns false (block-uniform) when the fast form
  // overflowed and nothing was written.
  auto run_pass = [&](int64_t ulo, int64_t uhi, auto exact_tag) -> bool {
    constexpr bool EXACT = decltype(exact_tag)::value;
    auto fold = [&](const f32x16& v, int tt) {
      if constexpr (EXACT) fold_exact(v, tt);
      else fold_fast(v, tt);
    };
    // Tiles folded so far (block-uniform); the first real tile sets the
    // reference in the fast form.
    int nfold = 0;
    auto consume = [&](const Tiles& v) {
      if (!EXACT && nfold == 0) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) set_ref(v[tt], tt);
      }
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) fold(v[tt], tt);
      ++nfold;
    };
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) { ref[tt] = -INFINITY; l[tt] = 0.f; }
    // The chunk stream: chunks 0 .. 2 in flight (the first pass requested
    // them before the token rows), then wait for chunk 0.
    if (!primed) {
#pragma unroll
      for (int q = 0; q < 3; ++q) copy_chunk(q);
    }
    primed = false;
    wait_vmcnt<2 * XI>();
    barrier_lds();
    // Software pipeline over prototype tiles: the products of tile p are
    // issued in the same straight-line block as the vector work on tile p - 1,
    // so the matrix cores and the vector ALU overlap.  All chunks but the last
    // are full.
    Tiles q;                             // the tiles whose fold is pending
    bool qreal = false;
    static_assert(PCH == 64, "two prototype tiles per chunk");
    for (int ci = 0; ci + 1 < nch; ++ci) {
      const int buf = ci & (NB - 1);
      // The two tiles of the chunk swap roles with q, so nothing is copied.
      Tiles c;
      products(buf, 0, c);
      if (ci > 0) consume(q);
      products(buf, 1, q);
      consume(c);
      qreal = true;
      // Chunk ci + 1 has landed (ci + 2 may still be in flight); after the
      // barrier no wave reads chunk ci any more, and chunk ci + 3 goes into
      // the buffer of chunk ci - 1.
      wait_vmcnt<XI>();
      barrier_lds();
      copy_chunk(ci + 3);
    }
    {
      // Last chunk: tiles may be partial or past k; padding rows drop out as
      // -inf.
      const int ci = nch - 1, buf = ci & (NB - 1);
#pragma unroll
      for (int pt = 0; pt < PCH / 32; ++pt) {
        const int pbase = ci * PCH + pt * 32;
        if (pbase >= k) break;             // uniform across the block
        Tiles c;
        products(buf, pt, c);
        if (qreal) consume(q);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) q[tt] = c[tt];
        qreal = true;
        if (pbase + 32 > k) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (pbase + crow(i, h) >= k) {
#pragma unroll
              for (int tt = 0; tt < NT; ++tt) q[tt][i] = -INFINITY;
            }
        }
      }
      consume(q);
    }
    wait_vmcnt<0>();   // the copies past the end have landed: none is in flight after the pass

    if constexpr (!EXACT) {
      // Redo in the exact form if any lane's sum overflowed.
      bool bad = false;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) bad = bad || !__builtin_isfinite(l[tt]);
      if (__syncthreads_or(bad)) return false;
    }
    // Lanes l and l ^ 32 saw disjoint halves of the prototypes of one token.
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const float m = l[tt] > 0.f ? ref[tt] : -INFINITY;   // a lane with no terms
      const float mo = shfl_xor32(m), lo = shfl_xor32(l[tt]);
      const float M = fmaxf(m, mo);
      const float Ma = M * alpha;
      const float L = l[tt] * exp2_fast(fmaf(m, alpha, -Ma)) + lo * exp2_fast(fmaf(mo, alpha, -Ma));
      const int64_t tok = tok0 + tt * 32 + l32;
      if (h == 0 && tok >= ulo && tok < uhi) {
        lse_out[tok] = M * scale + __logf(L);
        if (lse2_out != nullptr) lse2_out[tok] = Ma + __log2f(L);
      }
    }
    return true;
  };
  auto pass = [&](int64_t ulo, int64_t uhi) {
    if (!run_pass(ulo, uhi, std::false_type{})) {
      __syncthreads();   // the fast pass's LDS reads are done before the next store
      run_pass(ulo, uhi, std::true_type{});
    }
  };

  if constexpr (!PU) {
    pass(0, T);
  } else {
    // One pass per user among this block's tokens, with that user's table.
    const int64_t b0 = (int64_t)blockIdx.x * 256;
    const int64_t b1 = b0 + 256 < T ? b0 + 256 : T;
    for (int u = first_user_after(offsets, B, b0);; ++u) {
      const int64_t ulo = clamp64(uload64(offsets + u), b0, b1);
      const int64_t uhi = clamp64(uload64(offsets + u + 1), ulo, b1);
      if (uhi > ulo) {
        const bf16* tab = P + (int64_t)u * pstride;
        if (primed && tab != Pu) {   // only with corrupt offsets: drop the early copies
          wait_vmcnt<0>();
          primed = false;
        }
        Pu = tab;
        pass(ulo, uhi);
      }
      if (uhi >= b1 || u + 1 >= B) break;
      __syncthreads();   // the last pass's LDS reads are done before the next store
    }
  }
  // Sentinel read by the aggregation pass for rows past the end of a tile.
  if (lse2_out != nullptr && blockIdx.x == 0 && tid == 0) lse2_out[T] = INFINITY;
  wait_vmcnt<0>();   // no copy into this block's LDS is left in flight at exit
}

// ----------------------------------------------------------------------------
// Pass 2: partial sketches per (segment, user) piece for one 256-prototype
// chunk.  grid = (G segments, nchunks); block = NW waves, each owning PT x 32
// prototypes: their rows as MFMA B operands in registers and their PT x 32 x D
// fp32 partial sketch as MFMA accumulators (AGPRs).
//
// The token stream of the segment is cut into 32-token tiles that never
// straddle two users.  Tile t + 8 is copied global -> LDS by the
// direct-to-LDS loads while tile t is computed, into sixteen rotating
// buffers; a barrier after every fourth tile publishes the copies (waits are
// explicit vmcnt counts and the barrier carries no fence).  Fewer barriers
// leave the waves less time waiting for the slowest one (a barrier every
// second tile was 2-3 % slower).  Step t computes the
// affinities of tile t+1 on the matrix cores while the vector ALU turns those
// of tile t into softmax weights, then the sketch update of tile t.
//
// lse2 holds the per-token log-sum-exp in log2 units, with lse2[T] = +inf:
// rows of a tile past its end read that entry and get weight 0.
//
// With one table per user (PU, user u's table at P + u pstride), every piece
// after the segment's first reloads the prototype rows and recomputes the
// affinities of its first tile (the step before computed them with the
// previous user's table).
//
// DIRECT (batches of many short users): a user whose tokens all lie
// in this segment has this one piece, and its sketch (normalised by its mass
// with mass_norm) and its mass go straight to S and mass_out, which sa_reduce
// then leaves alone; this saves the k x d partial and its read-back per short
// user.  Without DIRECT every piece goes to its partial (the extra per-piece
// state costs the main loop about 2 % when pieces are long).
template <int D, bool MASS, int NW, int PT, bool PU, bool DIRECT>
__global__ __launch_bounds__(NW * 64, 1) void sa_agg_bf16(
    const int64_t* __restrict__ offsets, int B, const bf16* __restrict__ X,
    const bf16* __restrict__ P, int64_t pstride, int k, int64_t T, int G, float alpha,
    const float* __restrict__ lse2, float* __restrict__ part, float* __restrict__ pmass,
    float* __restrict__ S, float* __restrict__ mass_out, int mass_norm) {
  constexpr int KS = D / 16;             // reduction steps of the affinity product
  constexpr int DB = D / 32;             // 32-row blocks of the transposed sketch
  constexpr int U = D / 8;               // 16-byte units per token row
  constexpr int KC = NW * PT * 32;       // prototypes per workgroup
  static_assert(KC == kChunkBf16, "one workgroup covers one prototype chunk");
  constexpr int TILE = 32;               // tokens per step
  constexpr int UNITS = TILE * U;        // 16-byte units per tile
  constexpr int UPW = UNITS / NW;        // units copied by each wave
  static_assert(UNITS % NW == 0 && (UPW <= 64 || UPW % 64 == 0), "");
  constexpr int XI = (UPW + 63) / 64;    // copy instructions per wave per tile
  constexpr int LPW = TILE / NW;         // lse entries copied by each wave
  constexpr int NBUF = 16;               // tile buffers (a power of two)
  constexpr int AHEAD = 8;               // copy distance in tiles
  static_assert((NBUF & (NBUF - 1)) == 0 && AHEAD >= 6 && AHEAD + 4 <= NBUF, "");
  constexpr int L = XI + 1;              // loads per wave per tile
  constexpr uint32_t XBYTES = TILE * D * 2;

  __shared__ __attribute__((aligned(16))) bf16 sX[NBUF][TILE * D];
  __shared__ __attribute__((aligned(16))) float sL[NBUF][TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int s = blockIdx.x, chunk = blockIdx.y;
  const int pw0 = chunk * KC + wave * PT * 32;   // first prototype of this wave
  const uint32_t sx0 = lds_addr((const SA_LDS void*)&sX[0][0]);
  const uint32_t sl0 = lds_addr((const SA_LDS void*)&sL[0][0]);
  const SA_LDS char* lds = (const SA_LDS char*)0;

  const int64_t lo = seg_lo(T, G, s), hi = seg_lo(T, G, s + 1);
  TileWalker<TILE> cw;                 // tile being computed
  cw.start(offsets, B, lo, hi);
  if (!cw.valid) return;
  TileWalker<TILE> qw = cw;            // next tile to copy

  // Prototype rows as B operands of Z^T = X P^T: pw[pt][ks] holds
  // P[pw0 + 32 pt + l32][16 ks + 8h .. +7] (of the piece's user's table).
  bf16x8 pw[PT][KS];
  auto load_prototypes = [&](const bf16* Pu) {
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const int row = pw0 + pt * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        pw[pt][ks] = row < k ? *(const bf16x8*)(Pu + (int64_t)row * D + 16 * ks + 8 * h) : bf16x8{};
    }
  };
  load_prototypes(PU ? P + (int64_t)cw.user * pstride : P);

  // Copy geometry.  Copy instruction j of this wave moves units
  // v0 .. v0 + 63 of the tile, v0 = wave UPW + 64 j; the lane's unit v sits in
  // row v / U at stored position v % U and holds global unit (v % U) ^ g(row).
  int crow_[XI];
  uint32_t ccol[XI];
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int v = wave * UPW + j * 64 + lane;
    crow_[j] = v / U;
    ccol[j] = (uint32_t)(((v % U) ^ xswz<D>(v / U)) * 16);
  }
  const int lrow = wave * LPW + lane;            // lse row copied (lane < LPW)

  // Copy the tile of qw into buffer b and advance qw.  Every wave issues
  // exactly L loads per tile, also past the end of the stream (then row 0 of
  // X and lse2[T]), so that vmcnt counts are the same every time.  Rows past
  // the tile's end copy its first row of X and lse2[T] = +inf.
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
    if (lane < LPW)
      lds_copy4v(lrow < nr ? lse2 + base + lrow : lse2 + T, sl0 + (b * TILE + wave * LPW) * 4);
    if (valid) qw.advance();
  };

#pragma unroll
  for (int b = 0; b < AHEAD; ++b) copy_next(b);
  // The prototype rows must have arrived before the loop, and the compiler
  // must see the wait for them here: otherwise it places one inside the loop,
  // where it would also wait for every copy in flight.  The copies above are
  // waited for as well, which the first tiles need anyway.
#pragma unroll
  for (int pt = 0; pt < PT; ++pt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(pw[pt][ks]));
  wait_vmcnt<0>();
  __syncthreads();

  // LDS byte offsets within a tile buffer (loop invariant).
  //  aoff[ks]: affinity A operand, token row l32, unit 2 ks + h.
  //  toff[db][e]: transpose read for token rows 4h + tr_r + 8e (+ 16 kb, which
  //  the swizzle leaves additive) and the lane's 4-column piece of d block db.
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

  // Affinities of the first tile.
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

  uint32_t t = 0;                                 // tile counter of the segment
  // Outer loop: one (segment, user) piece per iteration; inner loop: its
  // tiles.  The accumulators are only touched by the matrix cores inside the
  // inner loop, and flushed once per piece.
  while (cw.valid) {
    if constexpr (PU) {
      if (t > 0) {
        // A later piece: the next user's rows.  No load is in flight here (the
        // previous flush waited for all), and tile t's buffer is complete and
        // published (the previous step read it).
        load_prototypes(P + (int64_t)cw.user * pstride);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(pw[pt][ks]));
        wait_vmcnt<0>();
        const SA_LDS char* xs = lds + sx0 + (t & (NBUF - 1)) * XBYTES;
        bf16x8 a0[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a0[ks] = *(const SA_LDS bf16x8*)(xs + aoff[ks]);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          znext[pt] = mfma32(a0[0], pw[pt][0], f32x16{});
#pragma unroll
          for (int ks = 1; ks < KS; ++ks) znext[pt] = mfma32(a0[ks], pw[pt][ks], znext[pt]);
        }
      }
    }
    const int64_t slot = (int64_t)s + cw.user;
    bool whole = false;                          // the user's only piece
    if constexpr (DIRECT) {
      const int64_t ulo = clamp64(uload64(offsets + cw.user), 0, T);
      const int64_t uhi = clamp64(uload64(offsets + cw.user + 1), ulo, T);
      whole = ulo >= lo && uhi <= hi;
    }
    const int64_t urow = (int64_t)cw.user;
    f32x16 acc[PT][DB];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[pt][db] = f32x16{};
    float mass[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) mass[pt] = 0.f;
    bool last;
    do {
      const uint32_t buf = t & (NBUF - 1), b1 = (t + 1) & (NBUF - 1);
      copy_next((t + AHEAD) & (NBUF - 1));        // into the buffer of tile t-8

      const SA_LDS char* xs = lds + sx0 + buf * XBYTES;
      const SA_LDS char* xs1 = lds + sx0 + b1 * XBYTES;
      const SA_LDS char* ls = lds + sl0 + buf * (TILE * 4) + lqoff;

      // Affinities of tile t+1 (unused after the last tile of the stream).
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

      // This tile's lse and transposed token block (sketch-update operands).
      f32x4 lq[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) lq[g] = *(const SA_LDS f32x4*)(ls + 32 * g);
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

      // Softmax weights of tile t.  Register i of a lane is token crow(i, h)
      // of the tile; the lane's prototype is pw0 + 32 pt + l32.
      bf16x8 abf[PT][2];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 8 * kb + j;
            const float a = exp2_fast(fmaf(z[pt][i], alpha, -lq[i >> 2][i & 3]));
            if (MASS) mass[pt] += a;
            abf[pt][kb][j] = (bf16)a;
          }

      // U^T (d x prototypes) += X^T (d x tokens) A^T (tokens x prototypes).
      // K slot j of half h in block kb is token 16 kb + 8 (j / 4) + 4h + (j % 4),
      // matching the C fragment rows above.
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[pt][db] = mfma32(xt[kb][db], abf[pt][kb], acc[pt][db]);

      if ((t & 3) == 3) {
        // Tiles up to t+5 must be complete before the barrier (the next four
        // steps read up to tile t+5); those of t+6 .. t+AHEAD may be in flight.
        // The buffer a step copies into held tile t-8 or later, which every
        // wave finished before the previous barrier (at most four steps ago).
        wait_vmcnt<(AHEAD - 5) * L>();
        barrier_lds();
      }
      last = cw.last_in_piece();
      cw.advance();
      ++t;
    } while (!last);

    // Flush the piece.  acc[pt][db] register i holds
    // U[proto = pw0 + 32 pt + l32][d = 32 db + crow(i, h)].
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const int proto = pw0 + pt * 32 + l32;
      const float mo = MASS ? shfl_xor32(mass[pt]) : 0.f;
      if (proto < k) {
        const float mu = mass[pt] + mo;
        // The direct row is what sa_reduce forms from a single piece: the
        // partial, divided by the mass when normalised (zero mass: zero row).
        const bool nz = !(MASS && mass_norm) || mu > 0.f;
        const float inv = (MASS && mass_norm && mu > 0.f) ? 1.0f / mu : 1.0f;
        float* dst = whole ? S + (urow * k + proto) * D : part + (slot * k + proto) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 v = {acc[pt][db][4 * g], acc[pt][db][4 * g + 1], acc[pt][db][4 * g + 2],
                       acc[pt][db][4 * g + 3]};
            if (whole && MASS && mass_norm) v = nz ? v * inv : f32x4{0.f, 0.f, 0.f, 0.f};
            *(f32x4*)(dst + 32 * db + 8 * g + 4 * h) = v;
          }
        if (MASS && h == 0) {
          if (!whole) pmass[slot * k + proto] = mu;
          else if (mass_out != nullptr) mass_out[urow * k + proto] = mu;
        }
      }
    }
    // With one table per user the next piece reloads the prototype rows and
    // waits for them (and so for everything in flight) anyway.  With a shared
    // table the stores stay in flight: the copy waits of the tile loop count
    // them among the newer operations, which only makes those waits longer.
    if constexpr (PU) wait_vmem_all();
  }
  wait_vmcnt<0>();   // no copy left in flight at exit
}

// ----------------------------------------------------------------------------
// Host-side launchers.
#ifndef SA_AGG_WAVES
#define SA_AGG_WAVES 8
#endif
constexpr int kAggWaves = SA_AGG_WAVES;   // waves per aggregation workgroup
constexpr int kStatsTiles = SA_STATS_TILES;   // 32-token tiles per statistics wave

template <int D>
static hipError_t launch_stats_bf16_t(const FwdArgs& a, hipStream_t st, Prof* prof) {
  const float scale = 1.0f / sqrtf((float)D);
  const float alpha = scale * kLog2e;
  const unsigned nb = (unsigned)((a.T + 255) / 256);
  // Eight single-tile waves need at least 64 copy slots per wave (d >= 64).
  // With one table per user the block keeps two tiles per wave: its extra
  // per-user state would not fit the 128 registers of four waves per SIMD.
  constexpr int NT = D >= 64 ? kStatsTiles : 2;
  prof_begin(prof, "sa_stats_bf16", st);
  if (a.pstride != 0)
    hipLaunchKernelGGL((sa_stats_bf16<D, true, 2>), dim3(nb), dim3(256), 0, st,
                       (const bf16*)a.X,
                       (const bf16*)a.P, a.k, a.T, alpha, scale, a.lse, a.lse2, a.offsets, a.B,
                       a.pstride);
  else
    hipLaunchKernelGGL((sa_stats_bf16<D, false, NT>), dim3(nb), dim3(512 / NT), 0, st,
                       (const bf16*)a.X,
                       (const bf16*)a.P, a.k, a.T, alpha, scale, a.lse, a.lse2, a.offsets, a.B,
                       (int64_t)0);
  const hipError_t e = hipGetLastError();
  prof_end(prof, st);
  return e;
}

template <int D, bool MASS, int PT, bool PU>
static void launch_agg_bf16(const FwdArgs& a, bool direct, float alpha, hipStream_t st) {
  const dim3 grid(a.G, a.nchunks), block(64 * kAggWaves);
  const bf16* X = (const bf16*)a.X;
  const bf16* P = (const bf16*)a.P;
  if (direct)
    hipLaunchKernelGGL((sa_agg_bf16<D, MASS, kAggWaves, PT, PU, true>), grid, block, 0, st,
                       a.offsets, a.B, X, P, a.pstride, a.k, a.T, a.G, alpha, a.lse2, a.part,
                       a.pmass, a.S, a.mass, a.mass_norm);
  else
    hipLaunchKernelGGL((sa_agg_bf16<D, MASS, kAggWaves, PT, PU, false>), grid, block, 0, st,
                       a.offsets, a.B, X, P, a.pstride, a.k, a.T, a.G, alpha, a.lse2, a.part,
                       a.pmass, a.S, a.mass, a.mass_norm);
}

template <int D>
static hipError_t launch_fwd_bf16_t(const FwdArgs& a, hipStream_t st, Prof* prof) {
  const float scale = 1.0f / sqrtf((float)D);
  const float alpha = scale * kLog2e;
  constexpr int PT = kChunkBf16 / (32 * kAggWaves);
  // Single-piece users write S directly when users outnumber segments four
  // to one (most users then lie inside one segment).  With fewer, longer
  // users the partials saved do not pay for the slower main loop.
  const bool direct = (int64_t)a.B >= 4 * (int64_t)a.G;
  if (a.T > 0) {
    hipError_t e = launch_stats_bf16_t<D>(a, st, prof);
    if (e != hipSuccess) return e;
    prof_begin(prof, "sa_agg_bf16", st);
    const bool ms = a.mass_norm || a.mass != nullptr, pu = a.pstride != 0;
    if (ms && pu) launch_agg_bf16<D, true, PT, true>(a, direct, alpha, st);
    else if (ms) launch_agg_bf16<D, true, PT, false>(a, direct, alpha, st);
    else if (pu) launch_agg_bf16<D, false, PT, true>(a, direct, alpha, st);
    else launch_agg_bf16<D, false, PT, false>(a, direct, alpha, st);
    e = hipGetLastError();
    prof_end(prof, st);
    if (e != hipSuccess) return e;
  }
  return launch_reduce(a, st, prof, false, direct);
}

hipError_t launch_stats_bf16(const FwdArgs& a, hipStream_t st, Prof* prof) {
  if (a.T == 0) return hipSuccess;
  switch (a.d) {
    case 32: return launch_stats_bf16_t<32>(a, st, prof);
    case 64: return launch_stats_bf16_t<64>(a, st, prof);
    case 128: return launch_stats_bf16_t<128>(a, st, prof);
  }
  return hipErrorInvalidValue;
}

// This file's two-pass forward is the default.  SA_FORWARD_PATH=single_pass
// in the environment (read at every call) selects the single-pass forward
// of sa_fused_bf16.hip where it applies (a shared table, a non-empty batch);
// a refused cooperative launch falls back to the two-pass forward.  On
// MI355X the single-pass kernel is the slower of the two (its per-tile
// statistics exchange and barrier serialise the waves; the two-pass form
// spends 2 k d more matrix flops, which are not the bottleneck).
static bool single_pass_enabled() {
  const char* v = getenv("SA_FORWARD_PATH");
  return v != nullptr && strcmp(v, "single_pass") == 0;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st, Prof* prof) {
  if (a.T > 0 && a.pstride == 0 && single_pass_enabled()) {
    if (launch_fwd_fused_bf16(a, st, prof) == hipSuccess) return hipSuccess;
    (void)hipGetLastError();   // clear the error of the refused launch
  }
  switch (a.d) {
    case 32: return launch_fwd_bf16_t<32>(a, st, prof);
    case 64: return launch_fwd_bf16_t<64>(a, st, prof);
    case 128: return launch_fwd_bf16_t<128>(a, st, prof);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
