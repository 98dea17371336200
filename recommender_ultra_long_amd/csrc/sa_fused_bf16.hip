// sa_fused_bf16.hip — single-pass Sketch Attention forward, bf16 inputs, fp32
// accumulation: the affinities are computed once, the per-token softmax
// statistics over all k prototypes are exchanged between the workgroups that
// share a token segment, and the aggregation follows in the same pass.
//
// Method: SequenceO1 reading notes, section 3.1, Eq. (6)-(9); FlashSA
// paragraph of the paper's HTML page (affinities, per-token max and
// log-sum-exp, aggregation, fused and streamed, no k x n matrix in memory).
//
// Work partition as for the two-pass forward: grid (G segments, nchunks), a
// workgroup owns 256 prototypes (8 waves x 32) and one token segment, walked
// in 32-token tiles that never straddle two users.  Per tile:
//  1. Z = P_w X^T on the matrix cores (token per lane, the wave's 32
//     prototypes in registers), two tiles ahead of the aggregation;
//     in-lane max and sum of exp2 over the wave's prototypes; the 8 waves'
//     partial statistics are combined through LDS into the chunk's
//     log-sum-exp of every token (log2 units).
//  2. The chunk's values are published as 64-bit words (value | ready bit)
//     in a zeroed exchange array, [nchunks][T]; every word is written once
//     per call.  The words of the other chunks of the segment are read back,
//     and all chunks merge the nchunks values of a token in chunk order, so
//     every workgroup gets bitwise the same log-sum-exp.
//  3. A = E f with E = exp2(z alpha - m) kept from step 1 and the per-token
//     factor f = exp2(m - lse2); A (bf16) goes through a wave-private LDS
//     tile to the prototype-per-lane layout, and U^T += X^T A^T (X^T read
//     transposed from the LDS X tile).
// Matrix work: 4 k d flop per token (the two-pass forward issues 6 k d).
//
// The exchange.  Words are stored and loaded with relaxed atomics at agent
// scope: single-location coherence at agent scope is all the protocol needs,
// since a word carries its own ready bit (no other data is published through
// it, so no release / acquire pairing is required), and it holds whichever
// XCD the partners run on.  Only wave 7 publishes and reads words; waves
// 0-3 copy the X tiles global -> LDS with explicit vmcnt accounting, which
// the exchange's loads and stores would otherwise disturb.  A workgroup
// publishes tile t + 2 before it waits for tile t + 1, and tile t + 1 of
// every chunk was published a step earlier, so no workgroup waits for a
// partner that waits for it (the launch is cooperative: all workgroups are
// resident).  Each wait is bounded (200 ms by the 100 MHz real-time clock);
// past it the workgroup stops waiting, finishes with wrong numbers and sets
// the exchange status word, which sa_get_device_status reports.
#include <algorithm>

#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

namespace {

constexpr uint64_t kReady = (uint64_t)1 << 32;
constexpr uint64_t kWaitBudgetTicks = 20000000;   // 200 ms at 100 MHz

__device__ __forceinline__ void xchg_publish(uint64_t* p, float v) {
  __hip_atomic_store(p, kReady | (uint64_t)__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t xchg_read(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge of per-(token, group) statistics (m raw max, l = sum exp2((z - m)
// alpha)) into one; a group whose prototypes are all padding has m = -inf,
// l = 0.
__device__ __forceinline__ void merge_stats(float& m, float& l, float m2, float l2, float alpha) {
  const float M = fmaxf(m, m2);
  const float Ma = M == -INFINITY ? 0.f : M * alpha;
  const float a = m == -INFINITY ? 0.f : l * exp2_fast(fmaf(m, alpha, -Ma));
  const float b = m2 == -INFINITY ? 0.f : l2 * exp2_fast(fmaf(m2, alpha, -Ma));
  m = M;
  l = a + b;
}

}  // namespace

// grid = (G, nchunks), block = 512 (8 waves).  xchg: [nchunks][T] words,
// zero on entry.  status2: the exchange status word.
template <int D, bool MASS>
__global__ __launch_bounds__(512, 1) void sa_fused_bf16(
    const int64_t* __restrict__ offsets, int B, const bf16* __restrict__ X,
    const bf16* __restrict__ P, int k, int64_t T, int G, int nchunks, float alpha,
    uint64_t* __restrict__ xchg, float* __restrict__ lse_out, float* __restrict__ part,
    float* __restrict__ pmass, uint32_t* __restrict__ status2) {
  constexpr int NW = 8;
  constexpr int KS = D / 16;             // reduction steps of the affinity product
  constexpr int DB = D / 32;             // 32-row blocks of the transposed sketch
  constexpr int U = D / 8;               // 16-byte units per token row
  constexpr int KC = NW * 32;
  static_assert(KC == kChunkBf16, "one workgroup covers one prototype chunk");
  constexpr int TILE = 32;
  constexpr int NCW = 4;                 // waves that copy X tiles
  constexpr int UNITS = TILE * U;
  constexpr int UPW = UNITS / NCW;       // units copied by each copy wave
  static_assert(UNITS % NCW == 0 && (UPW <= 64 || UPW % 64 == 0), "");
  constexpr int XI = (UPW + 63) / 64;    // copy instructions per copy wave per tile
  constexpr int NBUF = 8;
  constexpr int AHEAD = 6;               // copy distance in tiles
  constexpr int LA = 2;                  // statistics look-ahead in tiles
  constexpr uint32_t XBYTES = TILE * D * 2;
  constexpr int XW = 7;                  // the exchange wave
  constexpr int NCMAX = 8;               // chunks for k <= 2048

  __shared__ __attribute__((aligned(16))) bf16 sX[NBUF][TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 sA[NW][TILE * 32];   // A tile, [token][proto]
  __shared__ __attribute__((aligned(16))) float2 sPart[2][NW][TILE];  // (m, l) per wave, token
  __shared__ __attribute__((aligned(16))) float sL[2][TILE];          // lse2 per token

  const int tid = threadIdx.x;
  // The wave index is uniform over the wave: said so, the branches on it and
  // the tile walkers they update stay scalar.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int s = blockIdx.x, chunk = blockIdx.y;
  const int pw0 = chunk * KC + wave * 32;        // first prototype of this wave
  const uint32_t sx0 = lds_addr((const SA_LDS void*)&sX[0][0]);
  const uint32_t sa0 = lds_addr((const SA_LDS void*)&sA[wave][0]);
  const SA_LDS char* lds = (const SA_LDS char*)0;
  SA_LDS char* ldsw = (SA_LDS char*)0;

  const int64_t lo = seg_lo(T, G, s), hi = seg_lo(T, G, s + 1);
  TileWalker<TILE> cw;                 // tile aggregated in this step (t)
  cw.start(offsets, B, lo, hi);
  if (!cw.valid) return;               // uniform over the segment's workgroups
  TileWalker<TILE> qw = cw;            // next tile to copy
  TileWalker<TILE> gw = cw;            // tile t + 2 (affinities and statistics)
  gw.advance();
  // Tile t + 1 (its statistics are read back): first row, rows, validity.
  int64_t n1_t0 = gw.valid ? gw.t0 : 0;
  int n1_nr = gw.valid ? (int)(gw.t1 - gw.t0) : 0;
  bool n1_valid = gw.valid;
  if (gw.valid) gw.advance();

  // Prototype rows as A operands of Z = P X^T: pa[ks] holds
  // P[pw0 + l32][16 ks + 8h .. +7].  Rows past k are zero, and their
  // affinities are masked to -inf below.
  bf16x8 pa[KS];
  {
    const int row = pw0 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      pa[ks] = row < k ? *(const bf16x8*)(P + (int64_t)row * D + 16 * ks + 8 * h) : bf16x8{};
  }
  // Register i of Z holds prototype pw0 + crow(i, h); padding mask.
  uint32_t pmask = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (pw0 + crow(i, h) >= k) pmask |= 1u << i;

  // Copy geometry of the copy waves: instruction j moves units
  // v0 .. v0 + 63 of the tile, v0 = wave UPW + 64 j.
  int crow_[XI];
  uint32_t ccol[XI];
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int v = wave * UPW + j * 64 + lane;
    crow_[j] = v / U;
    ccol[j] = (uint32_t)(((v % U) ^ xswz<D>(v / U)) * 16);
  }
  // Copy the tile of qw into buffer b and advance qw.  Copy waves issue
  // exactly XI loads per tile, also past the end of the stream (row 0 of X),
  // so that their vmcnt counts are the same every time.
  auto copy_next = [&](uint32_t b) {
    if (wave >= NCW) return;
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
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(pa[ks]));
  wait_vmcnt<0>();
  __syncthreads();

  // LDS byte offsets within an X tile buffer (loop invariant): boff[ks] for
  // the B operand of Z (token row l32, unit 2 ks + h); toff for the
  // transpose reads of X^T (rows 4h + tr_r + 8e + 16 kb, 4-column piece of
  // d block db), as in the two-pass aggregation.
  const int tr_r = (lane & 15) >> 2, tr_c = lane & 3, tr_half = (lane >> 4) & 1;
  uint32_t boff[KS], toff[DB][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) boff[ks] = (uint32_t)xoff<D>(l32, 2 * ks + h) * 2;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      toff[db][e] = (uint32_t)(xoff<D>(4 * h + tr_r + 8 * e, 4 * db + 2 * tr_half + (tr_c >> 1)) +
                               (tr_c & 1) * 4) * 2;
  // The A tile in LDS: row = token (64 bytes), 16-byte unit q (prototypes
  // 8q .. 8q+7) stored at unit q ^ ((row >> 2) & 3).
  //  aw[g]: this lane's write of prototypes 8g + 4h .. +3 of its token;
  //  ar[kb][e]: transpose read of tokens 16 kb + 8 e + 4h + tr_r, prototypes
  //  16 tr_half + 4 tr_c .. +3 (so lane l gets prototype l32 of 4 tokens).
  auto aswz = [](int row, int q) { return (q ^ ((row >> 2) & 3)); };
  uint32_t aw[4], ar[2][2];
#pragma unroll
  for (int g = 0; g < 4; ++g) aw[g] = (uint32_t)(l32 * 64 + aswz(l32, g) * 16 + 8 * h);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = 16 * kb + 8 * e + 4 * h + tr_r;
      const int col = 16 * tr_half + 4 * tr_c;
      ar[kb][e] = (uint32_t)(row * 64 + aswz(row, col >> 3) * 16 + (col & 7) * 2);
    }

  // Affinities and partial statistics of one tile: z = Z (token l32,
  // prototypes crow(i, h)), E = exp2(z alpha - m alpha) with m this half's
  // maximum; the wave's (max, sum) over its 32 prototypes goes to
  // sPart[par][wave][token].
  auto affinities = [&](uint32_t buf, f32x16& E, float& m, int par) {
    const SA_LDS char* xs = lds + sx0 + buf * XBYTES;
    f32x16 z = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      z = mfma32(pa[ks], *(const SA_LDS bf16x8*)(xs + boff[ks]), z);
    if (pmask != 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (pmask & (1u << i)) z[i] = -INFINITY;
    }
    float t0 = fmaxf(fmaxf(z[0], z[1]), z[2]), t1 = fmaxf(fmaxf(z[3], z[4]), z[5]);
    float t2 = fmaxf(fmaxf(z[6], z[7]), z[8]), t3 = fmaxf(fmaxf(z[9], z[10]), z[11]);
    float t4 = fmaxf(fmaxf(z[12], z[13]), fmaxf(z[14], z[15]));
    m = fmaxf(fmaxf(fmaxf(t0, t1), t2), fmaxf(t3, t4));
    const float ma = m == -INFINITY ? 0.f : m * alpha;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      E[i] = exp2_fast(fmaf(z[i], alpha, -ma));
      E[i + 1] = exp2_fast(fmaf(z[i + 1], alpha, -ma));
      E[i + 2] = exp2_fast(fmaf(z[i + 2], alpha, -ma));
      E[i + 3] = exp2_fast(fmaf(z[i + 3], alpha, -ma));
      s0 += E[i];
      s1 += E[i + 1];
      s2 += E[i + 2];
      s3 += E[i + 3];
    }
    float mw = m, lw = (s0 + s1) + (s2 + s3);
    merge_stats(mw, lw, shfl_xor32(m), shfl_xor32(lw), alpha);
    if (h == 0) sPart[par][wave][l32] = make_float2(mw, lw);
  };

  // Exchange wave: combine the 8 waves' partials of a tile (sPart[par]) into
  // this chunk's log2-sum-exp per token and publish it (rows < nr).
  auto publish = [&](int par, int64_t t0, int nr) {
    float m = -INFINITY, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float2 v = sPart[par][4 * h + w][l32];
      merge_stats(m, l, v.x, v.y, alpha);
    }
    merge_stats(m, l, shfl_xor32(m), shfl_xor32(l), alpha);
    if (h == 0 && l32 < nr) xchg_publish(xchg + (int64_t)chunk * T + t0 + l32, m * alpha + __log2f(l));
  };

  bool failed = false;
  // Exchange wave: the words of a tile that this lane reads (chunks h,
  // h + 2, ... of token l32), issued early so that their latency overlaps
  // other work; a word not read stays 0.
  auto poll_issue = [&](int64_t t0, int nr, uint64_t (&w)[NCMAX / 2]) {
#pragma unroll
    for (int j = 0; j < NCMAX / 2; ++j) {
      const int c = h + 2 * j;
      w[j] = (l32 < nr && c < nchunks) ? xchg_read(xchg + (int64_t)c * T + t0 + l32) : 0;
    }
  };
  // Exchange wave: wait until every chunk's value for the tokens of a tile
  // is there (re-reading the words that were not ready), merge them in chunk
  // order into lse2 (log2 units), store lse2 in sL[par] (+inf for rows past
  // nr) and, in chunk 0, the natural-log lse.
  auto gather = [&](int par, int64_t t0, int nr, uint64_t (&w)[NCMAX / 2]) {
    float v[NCMAX / 2];
    const bool row = l32 < nr;
    uint64_t spin_start = 0;
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int j = 0; j < NCMAX / 2; ++j) {
        const int c = h + 2 * j;
        if (row && c < nchunks && !(w[j] & kReady)) {
          w[j] = xchg_read(xchg + (int64_t)c * T + t0 + l32);
          ok = ok && (w[j] & kReady) != 0;
        }
      }
      if (__all(ok) || failed) break;
      const uint64_t now = __builtin_amdgcn_s_memrealtime();
      if (spin_start == 0) spin_start = now;
      else if (now - spin_start > kWaitBudgetTicks) {
        failed = true;
        if (lane == 0) *status2 = kStatusExchangeTimeout;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int j = 0; j < NCMAX / 2; ++j) v[j] = __uint_as_float((uint32_t)w[j]);
    // Every chunk's value in every lane (chunk c was read by the half
    // c % 2, slot c / 2), then the merge in chunk order.
    float o[NCMAX / 2];
#pragma unroll
    for (int j = 0; j < NCMAX / 2; ++j) o[j] = shfl_xor32(v[j]);
    auto val = [&](int c) { return (c & 1) == h ? v[c >> 1] : o[c >> 1]; };
    float M = val(0);
#pragma unroll
    for (int c = 1; c < NCMAX; ++c)
      if (c < nchunks) M = fmaxf(M, val(c));
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < NCMAX; ++c)
      if (c < nchunks) sum += exp2_fast(val(c) - M);
    const float l2 = row ? M + __log2f(sum) : INFINITY;
    if (h == 0) {
      sL[par][l32] = l2;
      if (chunk == 0 && row) lse_out[t0 + l32] = l2 * kLn2;
    }
  };

  // Three sets of affinities in flight: tile t (aggregated now), t + 1 and
  // t + 2 (its statistics are being exchanged).  The step body is unrolled
  // three times so that each set keeps its registers.
  f32x16 E0, E1, E2;
  float m0 = -INFINITY, m1 = -INFINITY, m2 = -INFINITY;

  // Prologue: statistics of tiles 0 and 1, published; tile 0 read back.
  affinities(0, E0, m0, 0);
  if (n1_valid) affinities(1, E1, m1, 1);
  __syncthreads();
  if (wave == XW) {
    publish(0, cw.t0, (int)(cw.t1 - cw.t0));
    if (n1_valid) publish(1, n1_t0, n1_nr);
    uint64_t w[NCMAX / 2];
    poll_issue(cw.t0, (int)(cw.t1 - cw.t0), w);
    gather(0, cw.t0, (int)(cw.t1 - cw.t0), w);
  }
  __syncthreads();

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float mass = 0.f;
  uint32_t t = 0;   // tile counter of the segment

  // One step: aggregate tile t (Ec, mc) and compute tile t + 2 into (En, mn).
  // Returns false after the segment's last tile.
  auto step = [&](f32x16& Ec, float& mc, f32x16& En, float& mn) -> bool {
    const uint32_t buf = t & (NBUF - 1);
    // Tile t + 1's words were published a step ago: read them now, use them
    // after this step's affinities.
    uint64_t w1[NCMAX / 2];
    if (wave == XW && n1_valid) poll_issue(n1_t0, n1_nr, w1);
    copy_next((t + AHEAD) & (NBUF - 1));
    const int par = (int)(t & 1);
    if (gw.valid) affinities((t + LA) & (NBUF - 1), En, mn, par);
    // Tiles up to t + 3 must be complete before the barrier; t + 4 .. t + 6
    // may be in flight (copy waves only).
    if (wave < NCW) wait_vmcnt<(AHEAD - 3) * XI>();
    barrier_lds();
    if (wave == XW) {
      if (gw.valid) publish(par, gw.t0, (int)(gw.t1 - gw.t0));
      if (n1_valid) gather(par ^ 1, n1_t0, n1_nr, w1);
    }
    // Weights of tile t: A = E f, f = exp2(m alpha - lse2) per token.
    const float l2 = sL[par][l32];
    const float f = mc == -INFINITY ? 0.f : exp2_fast(fmaf(mc, alpha, -l2));
    const uint32_t sab = sa0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = (bf16)(Ec[4 * g + r] * f);
      *(SA_LDS bf16x4*)(ldsw + sab + aw[g]) = w;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the A tile is written
    bf16x8 abf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      abf[kb] = concat4(lds_read_tr16((const SA_LDS bf16*)(lds + sab + ar[kb][0])),
                        lds_read_tr16((const SA_LDS bf16*)(lds + sab + ar[kb][1])));
    if (MASS) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) mass += (float)abf[kb][j];
    }
    // U^T (d x prototypes) += X^T (d x tokens) A^T (tokens x prototypes).
    const SA_LDS char* xs = lds + sx0 + buf * XBYTES;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 xt = concat4(lds_read_tr16((const SA_LDS bf16*)(xs + toff[db][0] + kb * 32 * D)),
                                  lds_read_tr16((const SA_LDS bf16*)(xs + toff[db][1] + kb * 32 * D)));
        acc[db] = mfma32(xt, abf[kb], acc[db]);
      }
    }
    const bool last = cw.last_in_piece();
    const int user = cw.user;
    cw.advance();
    n1_valid = gw.valid;
    n1_t0 = gw.valid ? gw.t0 : 0;
    n1_nr = gw.valid ? (int)(gw.t1 - gw.t0) : 0;
    if (gw.valid) gw.advance();
    ++t;
    if (last) {
      // Flush the piece: acc[db] register i holds
      // U[proto = pw0 + l32][d = 32 db + crow(i, h)].
      const int64_t slot = (int64_t)s + user;
      const int proto = pw0 + l32;
      const float mo = MASS ? shfl_xor32(mass) : 0.f;
      if (proto < k) {
        float* dst = part + (slot * k + proto) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 v = {acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
            *(f32x4*)(dst + 32 * db + 8 * g + 4 * h) = v;
          }
        if (MASS && h == 0) pmass[slot * k + proto] = mass + mo;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
      mass = 0.f;
      // The stores stay in flight: they only make later vmcnt waits of the
      // copy waves wait for more than they need, never for less.
    }
    return cw.valid;
  };

  while (step(E0, m0, E2, m2) && step(E1, m1, E0, m0) && step(E2, m2, E1, m1)) {
  }
  wait_vmcnt<0>();   // no copy or store left in flight at exit
}

// Clears the exchange words and the exchange status word.
__global__ __launch_bounds__(256) void sa_fused_clear(uint64_t* __restrict__ w, int64_t n,
                                                      uint32_t* __restrict__ status2) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 2;
  const int64_t stride = (int64_t)gridDim.x * 512;
  for (int64_t i = i0; i < n; i += stride) {
    if (i + 1 < n) *(ulonglong2*)(w + i) = ulonglong2{0ull, 0ull};
    else w[i] = 0ull;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *status2 = kStatusOk;
}

template <int D>
static hipError_t launch_fused_t(const FwdArgs& a, hipStream_t st, Prof* prof) {
  const float scale = 1.0f / sqrtf((float)D);
  const float alpha = scale * kLog2e;
  const int64_t n = (int64_t)a.nchunks * a.T;
  const unsigned cb = (unsigned)std::min<int64_t>((n + 511) / 512, 2048);
  prof_begin(prof, "sa_fused_clear", st);
  hipLaunchKernelGGL(sa_fused_clear, dim3(cb > 0 ? cb : 1), dim3(256), 0, st, a.xchg, n,
                     a.status + 1);
  hipError_t e = hipGetLastError();
  prof_end(prof, st);
  if (e != hipSuccess) return e;
  const bool ms = a.mass_norm || a.mass != nullptr;
  void* args[] = {(void*)&a.offsets, (void*)&a.B,     (void*)&a.X,      (void*)&a.P,
                  (void*)&a.k,       (void*)&a.T,     (void*)&a.G,      (void*)&a.nchunks,
                  (void*)&alpha,     (void*)&a.xchg,  (void*)&a.lse,    (void*)&a.part,
                  (void*)&a.pmass,   nullptr};
  uint32_t* s2 = a.status + 1;
  args[13] = (void*)&s2;
  prof_begin(prof, "sa_fused_bf16", st);
  const void* fn = ms ? (const void*)sa_fused_bf16<D, true> : (const void*)sa_fused_bf16<D, false>;
  e = hipLaunchCooperativeKernel(fn, dim3(a.G, a.nchunks), dim3(512), args, 0, st);
  prof_end(prof, st);
  if (e != hipSuccess) return e;
  return launch_reduce(a, st, prof, true);
}

// The single-pass forward: the clear, the fused kernel (a cooperative launch)
// and the reduce.  Returns hipErrorCooperativeLaunchTooLarge (or another
// error) without launching the fused kernel when the grid cannot be
// resident at once; the caller then runs the two-pass forward.
hipError_t launch_fwd_fused_bf16(const FwdArgs& a, hipStream_t st, Prof* prof) {
  switch (a.d) {
    case 32: return launch_fused_t<32>(a, st, prof);
    case 64: return launch_fused_t<64>(a, st, prof);
    case 128: return launch_fused_t<128>(a, st, prof);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
