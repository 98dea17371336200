// sa_reduce.hip — deterministic split-n reduction of the forward's partial
// sketches, mass normalisation, and the device-side offsets check.
//
// Each user's sketch is the sum of the partials of the pieces (segment s,
// user u) that cover its tokens.  The pieces of one user are split over the
// four waves of a block by a fixed rule (wave w takes pieces w, w+4, ...) and
// the four wave sums are added in wave order, so the result does not depend
// on scheduling.  Mass normalisation divides row j by the prototype mass
// mu_j = sum_i A[j,i] (a zero mass gives a zero row).
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

// grid = (B, ceil(k d / 256)); block 256 = 4 waves; lane -> 4 consecutive
// outputs of the block's 256-element slice of S[u].  Block (0, 0) also checks
// all offsets and writes the status word.
__global__ __launch_bounds__(256) void sa_reduce_kernel(
    const int64_t* __restrict__ offsets, int B, int k, int d, int64_t T, int G,
    const float* __restrict__ part, const float* __restrict__ pmass, int use_mass,
    float* __restrict__ S, float* __restrict__ mass, int mass_norm, float out_scale,
    uint32_t* __restrict__ status, int keep2) {
  __shared__ f32x4 red[4][64];
  __shared__ float redm[4][64];
  const int u = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (blockIdx.y == 0 && u == 0)
    check_offsets_block(offsets, B, T, status, kStatusOk, kStatusBadOffsets, keep2 != 0);
  const int64_t kd = (int64_t)k * d;
  const int64_t e = ((int64_t)blockIdx.y * 64 + lane) * 4;
  const bool live = e < kd;
  const int j = live ? (int)(e / d) : 0;
  const int64_t lo = clamp64(uload64(offsets + u), 0, T);
  const int64_t hi = clamp64(uload64(offsets + u + 1), lo, T);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float mu = 0.f;
  if (hi > lo && live) {
    const int s0 = seg_of(T, G, lo), s1 = seg_of(T, G, hi - 1);
    const int n = s1 - s0 + 1;                       // pieces of user u
    const float* pp = part + ((int64_t)s0 + u) * kd + e;
    // Wave w adds pieces w, w + 4, ... in increasing order; eight loads are
    // in flight at a time.
    int q = wave;
    for (; q + 28 < n; q += 32) {
      f32x4 v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = *(const f32x4*)(pp + (int64_t)(q + 4 * r) * kd);
#pragma unroll
      for (int r = 0; r < 8; ++r) acc += v[r];
    }
    for (; q < n; q += 4) acc += *(const f32x4*)(pp + (int64_t)q * kd);
    if (use_mass) {
      const float* pm = pmass + ((int64_t)s0 + u) * k + j;
      int r = wave;
      for (; r + 28 < n; r += 32) {
        float m8[8];
#pragma unroll
        for (int q8 = 0; q8 < 8; ++q8) m8[q8] = pm[(int64_t)(r + 4 * q8) * k];
#pragma unroll
        for (int q8 = 0; q8 < 8; ++q8) mu += m8[q8];
      }
      for (; r < n; r += 4) mu += pm[(int64_t)r * k];
    }
  }
  red[wave][lane] = acc;
  redm[wave][lane] = mu;
  __syncthreads();
  if (wave != 0 || !live) return;
  acc = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
  mu = redm[0][lane] + redm[1][lane] + redm[2][lane] + redm[3][lane];
  if (mass_norm) {
    const float inv = mu > 0.f ? 1.0f / mu : 0.f;
    acc = mu > 0.f ? acc * inv : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (out_scale != 1.0f) acc = acc * out_scale;
  *(f32x4*)(S + (int64_t)u * kd + e) = acc;
  if (mass != nullptr && (e % d) == 0) mass[(int64_t)u * k + j] = mu;
}

hipError_t launch_reduce(const FwdArgs& a, hipStream_t st, Prof* prof, bool keep_exchange_status) {
  const int64_t kd = (int64_t)a.k * a.d;
  const unsigned gy = (unsigned)((kd + 255) / 256);
  const int use_mass = (a.mass_norm || a.mass != nullptr) ? 1 : 0;
  prof_begin(prof, "sa_reduce", st);
  hipLaunchKernelGGL(sa_reduce_kernel, dim3(a.B, gy), dim3(256), 0, st, a.offsets, a.B, a.k, a.d,
                     a.T, a.G, a.part, a.pmass, use_mass, a.S, a.mass, a.mass_norm, 1.0f,
                     a.status, keep_exchange_status ? 1 : 0);
  const hipError_t e = hipGetLastError();
  prof_end(prof, st);
  return e;
}

hipError_t launch_piece_sum(const int64_t* offsets, int B, int k, int d, int64_t T, int G,
                            const float* parts, float scale, float* out, uint32_t* status,
                            hipStream_t st, Prof* prof) {
  const int64_t kd = (int64_t)k * d;
  const unsigned gy = (unsigned)((kd + 255) / 256);
  prof_begin(prof, "sa_reduce", st);
  hipLaunchKernelGGL(sa_reduce_kernel, dim3(B, gy), dim3(256), 0, st, offsets, B, k, d, T, G,
                     parts, (const float*)nullptr, 0, out, (float*)nullptr, 0, scale, status, 0);
  const hipError_t e = hipGetLastError();
  prof_end(prof, st);
  return e;
}

}  // namespace sa
