// sa_kernels.h — internal interface between the C-ABI layer (sa_api.cpp) and
// the kernel launchers.  Not installed; the public interface is include/sa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

// Work partition constants (MI355X: 256 compute units, one aggregation
// workgroup per unit).
constexpr int kTargetWorkgroups = 256;
constexpr int kChunkBf16 = 256;   // prototypes per bf16 aggregation workgroup
constexpr int kChunkF32 = 64;     // prototypes per fp32 aggregation workgroup

// Device status word values written into the first bytes of the workspace.
constexpr uint32_t kStatusOk = 0u;
constexpr uint32_t kStatusBadOffsets = 1u;

struct Plan {
  int B, k, d;
  int64_t T;
  int dtype;            // 0 = fp32, 1 = bf16
  bool mass_norm;
  int chunk;            // prototypes per aggregation workgroup
  int nchunks;          // ceil(k / chunk)
  int G;                // token segments
  int64_t nslots;       // G + B - 1 partial slots
  // forward workspace layout (byte offsets)
  size_t off_status, off_lse, off_part, off_pmass, fwd_bytes;
  // backward workspace layout (byte offsets)
  size_t off_G, off_cv, off_g, off_delta, off_dxp, off_dpp, off_blse, bwd_bytes;
};

// Fills the plan; returns false for an unsupported problem.
bool make_plan(int B, int k, int d, int64_t T, int dtype, bool mass_norm, Plan* p);

struct FwdArgs {
  const int64_t* offsets;
  int B, k, d;
  int64_t T;
  const void* X;
  const void* P;
  float* lse;          // [T] (caller's buffer or workspace)
  float* S;            // [B, k, d]
  float* mass;         // [B, k] or nullptr
  float* part;         // [nslots, k, d]
  float* pmass;        // [nslots, k]
  uint32_t* status;    // device status word
  int G, nchunks;
  int mass_norm;
};

struct BwdArgs {
  const int64_t* offsets;
  int B, k, d;
  int64_t T;
  const void* X;
  const void* P;
  const float* dS;     // [B, k, d]
  const float* lse;    // [T]
  float* lse_ws;       // [T] workspace for a recomputed lse
  const float* S;      // [B, k, d] (mass norm only)
  const float* mass;   // [B, k]    (mass norm only)
  float* dX;           // [T, d]
  float* dP;           // [k, d]
  void* Gq;            // [B, k, d] G in the input dtype
  float* cv;           // [B, k]
  float* g;            // [T, d]
  float* delta;        // [T]
  float* dxp;          // [nchunks, T, d]
  float* dpp;          // [G, k, d]
  uint32_t* status;
  int G, nchunks;
  int mass_norm;
  int recompute_lse;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st);
hipError_t launch_reduce(const FwdArgs& a, hipStream_t st);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t st);

}  // namespace sa
