// sa_api.cpp — the C-ABI of include/sa.h: validation, work plan, workspace
// layout and kernel dispatch.  Host code only; kernels live in the .hip files.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "sa.h"
#include "sa_kernels.h"

namespace sa {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool make_plan(int B, int k, int d, int64_t T, int dtype, bool mass_norm, bool per_user,
               Plan* p) {
  if (B < 1 || k < 1 || k > 2048 || !(d == 32 || d == 64 || d == 128)) return false;
  if (T < 0 || T >= ((int64_t)1 << 36)) return false;
  if (dtype != 0 && dtype != 1) return false;
  memset(p, 0, sizeof(*p));
  p->B = B; p->k = k; p->d = d; p->T = T; p->dtype = dtype; p->mass_norm = mass_norm;
  p->per_user = per_user;
  // Segments: about one prototype-stationary workgroup per compute unit, and
  // never more segments than tokens, so that every segment is non-empty.
  auto segments = [T](int nchunks) {
    int G = kTargetWorkgroups / nchunks;
    if (G < 1) G = 1;
    if ((int64_t)G > T) G = (int)(T > 0 ? T : 1);
    return G;
  };
  p->chunk = dtype == 1 ? kChunkBf16 : kChunkF32;
  p->nchunks = (k + p->chunk - 1) / p->chunk;
  p->G = segments(p->nchunks);
  p->nslots = (int64_t)p->G + B - 1;
  p->bchunk = dtype == 1 ? kChunkBf16 : kChunkF32Bwd;
  p->bnchunks = (k + p->bchunk - 1) / p->bchunk;
  p->Gb = segments(p->bnchunks);
  // dP partials: one per segment (shared P, summed over users), or one per
  // (segment, user) piece with per-user tables.
  p->bslots = per_user ? (int64_t)p->Gb + B - 1 : (int64_t)p->Gb;

  const size_t Tn = (size_t)T;
  size_t off = 0;
  p->off_status = off; off += 256;
  p->off_lse = off; off = align256(off + Tn * 4);
  p->off_lse2 = off; off = align256(off + (Tn + 1) * 4);
  p->off_part = off; off = align256(off + (size_t)p->nslots * k * d * 4);
  p->off_pmass = off; off = align256(off + (size_t)p->nslots * k * 4);
  p->off_pl = off; off = align256(off + (size_t)p->nslots * k * 4);
  p->off_tlse = off; off = align256(off + (size_t)B * k * 4);
  // exchange words of the single-pass forward: one per (chunk, token)
  p->off_xchg = off; off = align256(off + (dtype == 1 ? (size_t)p->nchunks * Tn * 8 : 0));
  p->fwd_bytes = off;

  const size_t esz = dtype == 1 ? 2 : 4;
  off = 256;   // status word shared with the forward layout
  p->kp = dtype == 1 ? (k + kBwdxChunkBf16 - 1) / kBwdxChunkBf16 * kBwdxChunkBf16 : k;
  const size_t kp = (size_t)p->kp;
  p->off_G = off; off = align256(off + (size_t)B * kp * d * esz);
  p->off_cv = off; off = align256(off + (size_t)B * kp * 4);
  p->off_cvs = off; off = align256(off + (size_t)B * kp * 4);
  p->off_Pq = off; off = align256(off + (per_user ? (size_t)B : 1u) * kp * d * 2);
  p->off_delta = off; off = align256(off + Tn * 4);
  p->off_dpp = off; off = align256(off + (size_t)p->bslots * k * d * 4);
  p->off_blse = off; off = align256(off + Tn * 4);
  p->off_blse2 = off; off = align256(off + (Tn + 1) * 4);
  p->off_tlse2 = off; off = align256(off + (size_t)B * kp * 4);
  // c dZ (bf16) per token and prototype, written by the dX pass and read by
  // the dP pass: 2 KiB per (32-token tile, 32-prototype tile) for
  // bnchunks x 256 prototypes, and one scratch token tile at the end.
  p->off_dz = off;
  if (dtype == 1)
    off = align256(off + ((Tn + 31) / 32 + 1) * (size_t)p->bnchunks * (kChunkBf16 / 32) * 2048);
  p->bwd_bytes = off;
  return true;
}

FwdArgs fwd_args(const Plan& p, char* w, const int64_t* offsets, const void* X, const void* P,
                 int64_t pstride, float* S, float* lse, float* mass) {
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.offsets = offsets;
  a.B = p.B; a.k = p.k; a.d = p.d; a.T = p.T;
  a.X = X; a.P = P; a.pstride = pstride;
  a.lse = lse ? lse : (float*)(w + p.off_lse);
  a.lse2 = (float*)(w + p.off_lse2);
  a.S = S; a.mass = mass;
  a.part = (float*)(w + p.off_part);
  a.pmass = (float*)(w + p.off_pmass);
  a.pl = (float*)(w + p.off_pl);
  a.status = (uint32_t*)(w + p.off_status);
  a.xchg = (uint64_t*)(w + p.off_xchg);
  a.G = p.G; a.nchunks = p.nchunks;
  a.mass_norm = p.mass_norm ? 1 : 0;
  return a;
}

BwdArgs bwd_args(const Plan& p, char* w, const int64_t* offsets, const void* X, const void* P,
                 int64_t pstride, const float* dS, const float* lse, const float* S,
                 const float* mass, float* dX, float* dP) {
  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.offsets = offsets;
  a.B = p.B; a.k = p.k; a.d = p.d; a.T = p.T;
  a.X = X; a.P = P; a.pstride = pstride; a.dS = dS;
  a.lse_ws = (float*)(w + p.off_blse);
  a.lse2 = (float*)(w + p.off_blse2);
  a.recompute_lse = lse == nullptr ? 1 : 0;
  a.lse = lse ? lse : a.lse_ws;
  a.S = S; a.mass = mass;
  a.dX = dX; a.dP = dP; a.acc_dx = 0;
  a.Gq = (void*)(w + p.off_G);
  a.cv = (float*)(w + p.off_cv);
  a.cvs = (float*)(w + p.off_cvs);
  a.Pq = (void*)(w + p.off_Pq);
  a.kp = p.kp;
  a.delta = (float*)(w + p.off_delta);
  a.dpp = (float*)(w + p.off_dpp);
  a.status = (uint32_t*)(w + p.off_status);
  a.Gb = p.Gb; a.bnchunks = p.bnchunks; a.bslots = p.bslots;
  a.mass_norm = p.mass_norm ? 1 : 0;
  a.tokwise = 0;
  a.tlse2 = (float*)(w + p.off_tlse2);
  a.dz = (void*)(w + p.off_dz);
  a.kz = p.bnchunks * kChunkBf16;
  return a;
}

}  // namespace sa

using namespace sa;

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

extern "C" {

int sa_version(void) { return 10000; }

const char* sa_status_string(sa_status s) {
  switch (s) {
    case SA_OK: return "SA_OK";
    case SA_ERR_NULL_ARG: return "SA_ERR_NULL_ARG: a required pointer is NULL";
    case SA_ERR_BAD_SHAPE: return "SA_ERR_BAD_SHAPE: batch, k, d or total_tokens out of range";
    case SA_ERR_BAD_DTYPE: return "SA_ERR_BAD_DTYPE: dtype must be SA_F32 or SA_BF16";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED: unsupported flags or operation";
    case SA_ERR_WORKSPACE_TOO_SMALL: return "SA_ERR_WORKSPACE_TOO_SMALL: workspace smaller than sa_workspace_size()";
    case SA_ERR_BAD_OFFSETS: return "SA_ERR_BAD_OFFSETS: offsets not 0-based, non-decreasing and ending at total_tokens";
    case SA_ERR_MISALIGNED: return "SA_ERR_MISALIGNED: a pointer is not 16-byte aligned";
    case SA_ERR_HIP: return "SA_ERR_HIP: a HIP runtime call failed";
    case SA_ERR_DEVICE_TIMEOUT: return "SA_ERR_DEVICE_TIMEOUT: the single-pass forward's statistics exchange gave up waiting (results are wrong)";
  }
  return "SA_ERR_UNKNOWN";
}

sa_status sa_validate(const sa_problem* pr, const int64_t* offsets_host) {
  if (pr == nullptr) return SA_ERR_NULL_ARG;
  if (pr->dtype != SA_F32 && pr->dtype != SA_BF16) return SA_ERR_BAD_DTYPE;
  const uint32_t known = SA_FLAG_MASS_NORM | SA_FLAG_PER_USER_PROTOTYPES | SA_FLAG_TOKEN_WISE;
  if ((pr->flags & ~known) != 0u) return SA_ERR_UNSUPPORTED;
  // Token-wise weights already sum to one per prototype (no mass
  // normalisation), and that variant takes one shared table.
  if ((pr->flags & SA_FLAG_TOKEN_WISE) != 0u &&
      (pr->flags & (SA_FLAG_MASS_NORM | SA_FLAG_PER_USER_PROTOTYPES)) != 0u)
    return SA_ERR_UNSUPPORTED;
  if (pr->batch < 1 || pr->k < 1 || pr->k > 2048) return SA_ERR_BAD_SHAPE;
  if (!(pr->d == 32 || pr->d == 64 || pr->d == 128)) return SA_ERR_BAD_SHAPE;
  if (pr->total_tokens < 0 || pr->total_tokens >= ((int64_t)1 << 36)) return SA_ERR_BAD_SHAPE;
  if (offsets_host != nullptr) {
    if (offsets_host[0] != 0 || offsets_host[pr->batch] != pr->total_tokens) return SA_ERR_BAD_OFFSETS;
    for (int32_t u = 0; u < pr->batch; ++u)
      if (offsets_host[u + 1] < offsets_host[u]) return SA_ERR_BAD_OFFSETS;
  }
  return SA_OK;
}

size_t sa_workspace_size(const sa_problem* pr, int op) {
  if (sa_validate(pr, nullptr) != SA_OK) return 0;
  Plan p;
  if (!make_plan(pr->batch, pr->k, pr->d, pr->total_tokens, (int)pr->dtype,
                 (pr->flags & SA_FLAG_MASS_NORM) != 0u,
                 (pr->flags & SA_FLAG_PER_USER_PROTOTYPES) != 0u, &p))
    return 0;
  if (op == SA_OP_FORWARD) return p.fwd_bytes;
  if (op == SA_OP_BACKWARD) return p.bwd_bytes;
  return 0;
}

static sa_status forward_impl(const sa_problem* pr, const int64_t* offsets_dev, const void* X,
                              const void* P, float* S, float* lse, float* mass, void* ws,
                              size_t ws_bytes, void* stream, Prof* prof) {
  sa_status v = sa_validate(pr, nullptr);
  if (v != SA_OK) return v;
  if (offsets_dev == nullptr || P == nullptr || S == nullptr || ws == nullptr) return SA_ERR_NULL_ARG;
  if (X == nullptr && pr->total_tokens > 0) return SA_ERR_NULL_ARG;
  if (((uintptr_t)offsets_dev & 7u) != 0u) return SA_ERR_MISALIGNED;
  if ((X && !aligned16(X)) || !aligned16(P) || !aligned16(S) || !aligned16(ws) ||
      (lse && !aligned16(lse)) || (mass && !aligned16(mass)))
    return SA_ERR_MISALIGNED;
  Plan p;
  const bool mn = (pr->flags & SA_FLAG_MASS_NORM) != 0u;
  const bool pu = (pr->flags & SA_FLAG_PER_USER_PROTOTYPES) != 0u;
  if (!make_plan(pr->batch, pr->k, pr->d, pr->total_tokens, (int)pr->dtype, mn, pu, &p))
    return SA_ERR_BAD_SHAPE;
  if (ws_bytes < p.fwd_bytes) return SA_ERR_WORKSPACE_TOO_SMALL;

  hipStream_t st = (hipStream_t)stream;
  if ((pr->flags & SA_FLAG_TOKEN_WISE) != 0u) {
    if (mass != nullptr) return SA_ERR_UNSUPPORTED;   // every row of weights sums to one
    const FwdArgs a = fwd_args(p, (char*)ws, offsets_dev, X, P, 0, S,
                               lse ? lse : (float*)((char*)ws + p.off_tlse), nullptr);
    const hipError_t e = launch_tok_fwd(a, (int)pr->dtype, st, prof);
    return e == hipSuccess ? SA_OK : SA_ERR_HIP;
  }
  const FwdArgs a = fwd_args(p, (char*)ws, offsets_dev, X, P, pu ? (int64_t)p.k * p.d : 0, S,
                             lse, mass);
  hipError_t e = pr->dtype == SA_BF16 ? launch_fwd_bf16(a, st, prof) : launch_fwd_f32(a, st, prof);
  return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

static sa_status backward_impl(const sa_problem* pr, const int64_t* offsets_dev, const void* X,
                               const void* P, const float* dS, const float* lse, const float* S,
                               const float* mass, float* dX, float* dP, void* ws, size_t ws_bytes,
                               void* stream, Prof* prof) {
  sa_status v = sa_validate(pr, nullptr);
  if (v != SA_OK) return v;
  const bool mn = (pr->flags & SA_FLAG_MASS_NORM) != 0u;
  if (offsets_dev == nullptr || P == nullptr || dS == nullptr || dP == nullptr || ws == nullptr)
    return SA_ERR_NULL_ARG;
  if ((X == nullptr || dX == nullptr) && pr->total_tokens > 0) return SA_ERR_NULL_ARG;
  if (mn && (S == nullptr || mass == nullptr)) return SA_ERR_NULL_ARG;
  if (((uintptr_t)offsets_dev & 7u) != 0u) return SA_ERR_MISALIGNED;
  if ((X && !aligned16(X)) || !aligned16(P) || !aligned16(dS) || !aligned16(dP) ||
      (dX && !aligned16(dX)) || !aligned16(ws) || (lse && !aligned16(lse)) ||
      (S && !aligned16(S)) || (mass && !aligned16(mass)))
    return SA_ERR_MISALIGNED;
  Plan p;
  const bool pu = (pr->flags & SA_FLAG_PER_USER_PROTOTYPES) != 0u;
  if (!make_plan(pr->batch, pr->k, pr->d, pr->total_tokens, (int)pr->dtype, mn, pu, &p))
    return SA_ERR_BAD_SHAPE;
  if (ws_bytes < p.bwd_bytes) return SA_ERR_WORKSPACE_TOO_SMALL;

  const bool tw = (pr->flags & SA_FLAG_TOKEN_WISE) != 0u;
  if (tw && (S == nullptr || lse == nullptr)) return SA_ERR_NULL_ARG;   // D_j = dS_j . S_j
  BwdArgs a = bwd_args(p, (char*)ws, offsets_dev, X, P, pu ? (int64_t)p.k * p.d : 0, dS, lse, S,
                       mass, dX, dP);
  a.tokwise = tw ? 1 : 0;
  hipError_t e = launch_bwd(a, (int)pr->dtype, (hipStream_t)stream, prof);
  return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

static sa_status profile_setup(sa_profile* prof, Prof* p) {
  if (prof == nullptr) return SA_ERR_NULL_ARG;
  for (int i = 0; i < 2 * SA_PROFILE_MAX_KERNELS; ++i)
    if (prof->events[i] == nullptr) return SA_ERR_NULL_ARG;
  p->ev = (hipEvent_t*)prof->events;
  p->cap = SA_PROFILE_MAX_KERNELS;
  p->n = 0;
  p->names = prof->names;
  prof->n_kernels = 0;
  return SA_OK;
}

sa_status sa_forward(const sa_problem* pr, const int64_t* offsets_dev, const void* X,
                     const void* P, float* S, float* lse, float* mass, void* ws,
                     size_t ws_bytes, void* stream) {
  return forward_impl(pr, offsets_dev, X, P, S, lse, mass, ws, ws_bytes, stream, nullptr);
}

sa_status sa_backward(const sa_problem* pr, const int64_t* offsets_dev, const void* X,
                      const void* P, const float* dS, const float* lse, const float* S,
                      const float* mass, float* dX, float* dP, void* ws, size_t ws_bytes,
                      void* stream) {
  return backward_impl(pr, offsets_dev, X, P, dS, lse, S, mass, dX, dP, ws, ws_bytes, stream,
                       nullptr);
}

sa_status sa_forward_profiled(const sa_problem* pr, const int64_t* offsets_dev, const void* X,
                              const void* P, float* S, float* lse, float* mass, void* ws,
                              size_t ws_bytes, void* stream, sa_profile* prof) {
  Prof p;
  sa_status v = profile_setup(prof, &p);
  if (v != SA_OK) return v;
  v = forward_impl(pr, offsets_dev, X, P, S, lse, mass, ws, ws_bytes, stream, &p);
  prof->n_kernels = p.n;
  return v;
}

sa_status sa_backward_profiled(const sa_problem* pr, const int64_t* offsets_dev, const void* X,
                               const void* P, const float* dS, const float* lse, const float* S,
                               const float* mass, float* dX, float* dP, void* ws,
                               size_t ws_bytes, void* stream, sa_profile* prof) {
  Prof p;
  sa_status v = profile_setup(prof, &p);
  if (v != SA_OK) return v;
  v = backward_impl(pr, offsets_dev, X, P, dS, lse, S, mass, dX, dP, ws, ws_bytes, stream, &p);
  prof->n_kernels = p.n;
  return v;
}

static bool fold_shape_ok(int rows, int d) {
  return rows >= 1 && rows <= (1 << 24) && (d == 32 || d == 64 || d == 128);
}

static sa_status fold_check(int k, int d, sa_dtype dtype) {
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_BAD_DTYPE;
  if (!fold_shape_ok(k, d)) return SA_ERR_BAD_SHAPE;
  return SA_OK;
}

size_t sa_fold_workspace_size(int k, int d) {
  if (!fold_shape_ok(k, d)) return 0;
  return fold_workspace_bytes(k, d);
}

sa_status sa_fold_prototypes(int k, int d, sa_dtype dtype, const void* P, const float* Wq,
                             const float* Wk, void* P_eff, void* stream) {
  const sa_status v = fold_check(k, d, dtype);
  if (v != SA_OK) return v;
  if (P == nullptr || Wq == nullptr || Wk == nullptr || P_eff == nullptr) return SA_ERR_NULL_ARG;
  if (!aligned16(P) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(P_eff))
    return SA_ERR_MISALIGNED;
  const hipError_t e = launch_fold(k, d, (int)dtype, P, Wq, Wk, P_eff, (hipStream_t)stream);
  return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

sa_status sa_fold_prototypes_backward(int k, int d, sa_dtype dtype, const void* P,
                                      const float* Wq, const float* Wk, const float* dP_eff,
                                      float* dP, float* dWq, float* dWk, void* ws,
                                      size_t ws_bytes, void* stream) {
  const sa_status v = fold_check(k, d, dtype);
  if (v != SA_OK) return v;
  if (P == nullptr || Wq == nullptr || Wk == nullptr || dP_eff == nullptr || dP == nullptr ||
      dWq == nullptr || dWk == nullptr || ws == nullptr)
    return SA_ERR_NULL_ARG;
  if (!aligned16(P) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(dP_eff) || !aligned16(dP) ||
      !aligned16(dWq) || !aligned16(dWk) || !aligned16(ws))
    return SA_ERR_MISALIGNED;
  if (ws_bytes < sa_fold_workspace_size(k, d)) return SA_ERR_WORKSPACE_TOO_SMALL;
  const hipError_t e = launch_fold_backward(k, d, (int)dtype, P, Wq, Wk, dP_eff, dP, dWq, dWk,
                                            (float*)ws, (hipStream_t)stream);
  return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // extern "C"

// Workspace of sa_forward_noalloc: one array per GPU, placed by the loader
// with the code object.  On the host, `scratch` only names the symbol; its
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[SA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, or null

// The device address of `scratch` on the current device (looked up on the
// first call for that device), or null if the lookup fails.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

sa_status sa_forward_noalloc(const sa_problem* pr, const int64_t* offsets_dev, const void* X,
                             const void* P, float* S, float* lse, float* mass, void* stream) {
  const sa_status v = sa_validate(pr, nullptr);
  if (v != SA_OK) return v;
  if (sa_workspace_size(pr, SA_OP_FORWARD) > SA_NOALLOC_SCRATCH_BYTES)
    return SA_ERR_WORKSPACE_TOO_SMALL;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return SA_ERR_HIP;
  return forward_impl(pr, offsets_dev, X, P, S, lse, mass, ws, SA_NOALLOC_SCRATCH_BYTES, stream,
                      nullptr);
}

sa_status sa_get_device_status(const void* ws, void* stream) {
  if (ws == nullptr) return SA_ERR_NULL_ARG;
  hipStream_t st = (hipStream_t)stream;
  uint32_t word[2] = {0u, 0u};
  if (hipMemcpyAsync(word, ws, sizeof(word), hipMemcpyDeviceToHost, st) != hipSuccess)
    return SA_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return SA_ERR_HIP;
  if (word[0] != kStatusOk) return SA_ERR_BAD_OFFSETS;
  return word[1] == kStatusExchangeTimeout ? SA_ERR_DEVICE_TIMEOUT : SA_OK;
}

}  // extern "C"
