// sa_reduce.hip — deterministic split-n reduction of the forward's partial
// sketches, mass normalisation, and the device-side offsets check.
//
// Each user's sketch is the sum of the partials of the pieces (segment s,
// user u) that cover its tokens, added in increasing segment order, so the
// result does not depend on scheduling.  Mass normalisation divides row j by
// the prototype mass mu_j = sum_i A[j,i] (a zero mass gives a zero row).
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

// grid = (B, ceil(k d / 1024)); block 256; thread -> 4 consecutive outputs.
// Block (0, 0) additionally checks all offsets and writes the status word.
__global__ __launch_bounds__(256) void sa_reduce_kernel(
    const int64_t* __restrict__ offsets, int B, int k, int d, int64_t T, int G,
    const float* __restrict__ part, const float* __restrict__ pmass, float* __restrict__ S,
    float* __restrict__ mass, int mass_norm, uint32_t* __restrict__ status) {
  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  if (blockIdx.y == 0 && u == 0) check_offsets_block(offsets, B, T, status, kStatusOk, kStatusBadOffsets);
  const int64_t kd = (int64_t)k * d;
  const int64_t e = ((int64_t)blockIdx.y * 256 + tid) * 4;
  if (e >= kd) return;
  const int j = (int)(e / d);
  const int64_t lo = clamp64(offsets[u], 0, T), hi = clamp64(offsets[u + 1], lo, T);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float mu = 0.f;
  if (hi > lo) {
    const int s0 = seg_of(T, G, lo), s1 = seg_of(T, G, hi - 1);
    for (int s = s0; s <= s1; ++s) {
      const int64_t slot = (int64_t)s + u;
      acc += *(const f32x4*)(part + slot * kd + e);
      mu += pmass[slot * k + j];
    }
  }
  if (mass_norm) {
    const float inv = mu > 0.f ? 1.0f / mu : 0.f;
    acc *= inv;
    if (!(mu > 0.f)) acc = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  *(f32x4*)(S + (int64_t)u * kd + e) = acc;
  if (mass != nullptr && (e % d) == 0) mass[(int64_t)u * k + j] = mu;
}

hipError_t launch_reduce(const FwdArgs& a, hipStream_t st, Prof* prof) {
  const int64_t kd = (int64_t)a.k * a.d;
  const unsigned gy = (unsigned)((kd / 4 + 255) / 256);
  prof_begin(prof, "sa_reduce", st);
  hipLaunchKernelGGL(sa_reduce_kernel, dim3(a.B, gy), dim3(256), 0, st, a.offsets, a.B, a.k, a.d,
                     a.T, a.G, a.part, a.pmass, a.S, a.mass, a.mass_norm, a.status);
  const hipError_t e = hipGetLastError();
  prof_end(prof, st);
  return e;
}

}  // namespace sa
