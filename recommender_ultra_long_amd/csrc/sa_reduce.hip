// sa_reduce.hip — deterministic split-n reduction of the forward's partial
// sketches, mass normalisation, and the device-side offsets check.
//
// Each user's sketch is the sum of the partials of the pieces (segment s,
// user u) that cover its tokens.  The pieces of one user are split over the
// waves that share an output slice by a fixed rule (wave sub takes pieces
// sub, sub + WPS, ...) and the wave sums are added in wave order, so the
// result does not depend on scheduling.  Mass normalisation divides row j by
// the prototype mass mu_j = sum_i A[j,i] (a zero mass gives a zero row).  A
// user with one piece whose row the aggregation pass already wrote (skip_single)
// is left alone; an empty user gets zero rows here.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

// Lane l's value of a 64-bit per-lane variable (l uniform).
__device__ __forceinline__ int64_t lane64(int64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)(uint64_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Block (y, b) of grid (nsy, nub), 256 threads = 4 waves, reduces output
// group y (256 * 4 / WPS consecutive elements of S[u]) for the users
// u = b, b + nub, b + 2 nub, ...: the lanes of each wave read the offsets of
// 64 of these users at once and vote which of them need the reduction, and
// the block then takes those users one by one.  nub is capped, so that a
// batch of many short users launches neither a workgroup per (user, group)
// nor a serial offsets read per user.  WPS waves share one 256-element slice
// of S[u] (lane -> 4 consecutive outputs): wave sub of the slice adds pieces
// sub, sub + WPS, ... of user u in increasing order, and the WPS sums are
// added in wave order.  WPS = 4 for users with many pieces (one long user), 1
// when most users have one or two (many short users: no idle waves).  Block
// (0, 0) also checks all offsets and writes the status word.  With
// skip_single, a non-empty user whose tokens lie in one segment is skipped:
// the aggregation pass wrote its row of S (and of mass) directly.
template <int WPS>
__global__ __launch_bounds__(256) void sa_reduce_kernel(
    const int64_t* __restrict__ offsets, int B, int k, int d, int64_t T, int G,
    const float* __restrict__ part, const float* __restrict__ pmass, int use_mass,
    float* __restrict__ S, float* __restrict__ mass, int mass_norm, float out_scale,
    uint32_t* __restrict__ status, int keep2, int skip_single) {
  constexpr int SPB = 4 / WPS;                       // slices per block
  __shared__ f32x4 red[4][64];
  __shared__ float redm[4][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = wave % WPS;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    check_offsets_block(offsets, B, T, status, kStatusOk, kStatusBadOffsets, keep2 != 0);
  const int64_t kd = (int64_t)k * d;
  const int64_t y = blockIdx.x;
  // The vote is the same in every wave (it depends on the lane only), so every
  // branch below is uniform over the block and every wave reaches the same
  // barriers.
  const int64_t nub = gridDim.y;
  for (int64_t c0 = blockIdx.y; c0 < B; c0 += 64 * nub) {
    const int64_t ul = c0 + lane * nub;
    int64_t llo = 0, lhi = 0;
    int ls0 = 0, ls1 = 0;
    bool need = false;
    if (ul < B) {
      llo = clamp64(offsets[ul], 0, T);
      lhi = clamp64(offsets[ul + 1], llo, T);
      if (lhi > llo) { ls0 = seg_of(T, G, llo); ls1 = seg_of(T, G, lhi - 1); }
      need = !(skip_single && lhi > llo && ls0 == ls1);
    }
    uint64_t todo = __ballot(need);
    while (todo != 0) {
      const int l = __builtin_ctzll(todo);
      todo &= todo - 1;
      const int u = (int)(c0 + l * nub);
      const int64_t lo = lane64(llo, l), hi = lane64(lhi, l);
      const int s0 = __builtin_amdgcn_readlane(ls0, l), s1 = __builtin_amdgcn_readlane(ls1, l);
      const int64_t e = ((y * SPB + wave / WPS) * 64 + lane) * 4;
      const bool live = e < kd;
      const int j = live ? (int)(e / d) : 0;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      float mu = 0.f;
      if (hi > lo && live) {
        const int n = s1 - s0 + 1;                     // pieces of user u
        const float* pp = part + ((int64_t)s0 + u) * kd + e;
        const float* pm = use_mass ? pmass + ((int64_t)s0 + u) * k + j : nullptr;
        // Eight pieces in flight at a time; the masses in the same rounds.
        int q = sub;
        if (use_mass) {
          for (; q + 7 * WPS < n; q += 8 * WPS) {
            f32x4 v[8];
            float m8[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              v[r] = *(const f32x4*)(pp + (int64_t)(q + WPS * r) * kd);
              m8[r] = pm[(int64_t)(q + WPS * r) * k];
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              acc += v[r];
              mu += m8[r];
            }
          }
          for (; q < n; q += WPS) {
            acc += *(const f32x4*)(pp + (int64_t)q * kd);
            mu += pm[(int64_t)q * k];
          }
        } else {
          for (; q + 7 * WPS < n; q += 8 * WPS) {
            f32x4 v[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) v[r] = *(const f32x4*)(pp + (int64_t)(q + WPS * r) * kd);
#pragma unroll
            for (int r = 0; r < 8; ++r) acc += v[r];
          }
          for (; q < n; q += WPS) acc += *(const f32x4*)(pp + (int64_t)q * kd);
        }
      }
      if constexpr (WPS > 1) {
        red[wave][lane] = acc;
        redm[wave][lane] = mu;
        __syncthreads();
        if (sub == 0) {
          acc = red[wave][lane];
          mu = redm[wave][lane];
#pragma unroll
          for (int w = 1; w < WPS; ++w) {
            acc += red[wave + w][lane];
            mu += redm[wave + w][lane];
          }
        }
        __syncthreads();   // red is read before the next user writes it
        if (sub != 0) continue;
      }
      if (!live) continue;
      if (mass_norm) {
        const float inv = mu > 0.f ? 1.0f / mu : 0.f;
        acc = mu > 0.f ? acc * inv : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (out_scale != 1.0f) acc = acc * out_scale;
      *(f32x4*)(S + (int64_t)u * kd + e) = acc;
      if (mass != nullptr && (e % d) == 0) mass[(int64_t)u * k + j] = mu;
    }
  }
}

// Upper bound on the reduction's grid: eight 256-thread blocks per compute
// unit, enough to keep every CU busy; a larger batch loops over its users.
static constexpr int64_t kReduceBlocks = 2048;

// Waves per slice from the average number of pieces per user (the pieces of
// all users together are at most G + B - 1).
static int reduce_wps(int B, int G) {
  const double avg = (double)(G + B - 1) / (double)(B > 0 ? B : 1);
  return avg <= 2.0 ? 1 : (avg <= 8.0 ? 2 : 4);
}

static hipError_t launch_reduce_kernel(const int64_t* offsets, int B, int k, int d, int64_t T,
                                       int G, const float* part, const float* pmass,
                                       int use_mass, float* S, float* mass, int mass_norm,
                                       float out_scale, uint32_t* status, int keep2,
                                       int skip_single, hipStream_t st) {
  const int64_t kd = (int64_t)k * d;
  const int wps = reduce_wps(B, G);
  const int64_t per_block = 256 * (4 / wps);         // outputs per block
  const int64_t nsy = (kd + per_block - 1) / per_block;   // output groups per user
  int64_t nub = kReduceBlocks / nsy;                 // users taken at once
  nub = nub < 1 ? 1 : (nub > B ? B : nub);
  const dim3 grid((unsigned)nsy, (unsigned)nub);
  switch (wps) {
    case 1:
      hipLaunchKernelGGL(sa_reduce_kernel<1>, grid, dim3(256), 0, st, offsets, B, k, d, T, G,
                         part, pmass, use_mass, S, mass, mass_norm, out_scale, status, keep2, skip_single);
      break;
    case 2:
      hipLaunchKernelGGL(sa_reduce_kernel<2>, grid, dim3(256), 0, st, offsets, B, k, d, T, G,
                         part, pmass, use_mass, S, mass, mass_norm, out_scale, status, keep2, skip_single);
      break;
    default:
      hipLaunchKernelGGL(sa_reduce_kernel<4>, grid, dim3(256), 0, st, offsets, B, k, d, T, G,
                         part, pmass, use_mass, S, mass, mass_norm, out_scale, status, keep2, skip_single);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const FwdArgs& a, hipStream_t st, Prof* prof, bool keep_exchange_status,
                         bool skip_single) {
  const int use_mass = (a.mass_norm || a.mass != nullptr) ? 1 : 0;
  prof_begin(prof, "sa_reduce", st);
  const hipError_t e = launch_reduce_kernel(a.offsets, a.B, a.k, a.d, a.T, a.G, a.part, a.pmass,
                                            use_mass, a.S, a.mass, a.mass_norm, 1.0f, a.status,
                                            keep_exchange_status ? 1 : 0, skip_single ? 1 : 0, st);
  prof_end(prof, st);
  return e;
}

hipError_t launch_piece_sum(const int64_t* offsets, int B, int k, int d, int64_t T, int G,
                            const float* parts, float scale, float* out, uint32_t* status,
                            hipStream_t st, Prof* prof) {
  prof_begin(prof, "sa_reduce", st);
  const hipError_t e = launch_reduce_kernel(offsets, B, k, d, T, G, parts, (const float*)nullptr,
                                            0, out, (float*)nullptr, 0, scale, status, 0, 0, st);
  prof_end(prof, st);
  return e;
}

}  // namespace sa
