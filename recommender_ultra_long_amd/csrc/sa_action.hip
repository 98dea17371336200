// sa_action.hip — the action-side SwiGLU fusion that builds the history rows
// (SequenceO1 reading notes, section 3.6, Eq. (20)):
//     x_i = e_i + (silu(v_i W1) * (v_i W3)) W2,   v_i = [e_i; a_{t_i}],
// e_i the item embedding, a_t row t of the action table A (one row per
// action type), W1, W3 in R^{2d x 2d}, W2 in R^{2d x d} (hidden width H = 2d).
//
// The action half of the first products depends only on the type, so
//     v W1 = e W1e + T1[t],   T1 = A W1a   (W1 = [W1e; W1a]),
// and the per-type rows T1, T3 (n_types x H, computed once per call) replace
// the second half of the product: each event costs 12 d^2 flops instead of 20.
//
// sa_action_prep:   W1e^T, W3e^T, W2^T in bf16 (matrix-core operands) and
//                   T1, T3 in fp32.
// sa_action_fwd<D>: persistent workgroups over 32-event tiles, 4 waves, all
//                   products on the matrix cores (bf16 in, fp32 accumulate),
//                   computed transposed so that each product's result feeds
//                   the next without a relayout:
//                     U^T = W1e^T e^T   (weights as A operands, kept in
//                                        registers; events as B operands)
//                     G   = silu(U1^T + T1) * (U3^T + T3)   -> LDS [event][H]
//                     x^T = W2^T G^T    (W2^T from LDS, G^T read back as
//                                        B operands), + e, stored in the
//                                        history's dtype.
//                   Wave w computes hidden rows [w H/4, (w+1) H/4) of U and
//                   output rows [32 w, 32 w + 32) of x.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {

constexpr int kActionMaxTypes = 16;

// Block b < nw: element i = b 256 + t of the transposed bf16 weights;
// blocks from nw: T1 / T3 entries.
//   W1eT[h][c] = W1[c][h], W3eT likewise (c < D, h < H); W2T[o][h] = W2[h][o];
//   T1[t][h] = sum_c A[t][c] W1[D + c][h], T3 likewise.
template <int D>
__global__ __launch_bounds__(256) void sa_action_prep(const float* __restrict__ A, int n_types,
                                                      const float* __restrict__ W1,
                                                      const float* __restrict__ W3,
                                                      const float* __restrict__ W2,
                                                      bf16* __restrict__ W1eT, bf16* __restrict__ W3eT,
                                                      bf16* __restrict__ W2T, float* __restrict__ T1,
                                                      float* __restrict__ T3, int nw) {
  constexpr int H = 2 * D;
  if ((int)blockIdx.x < nw) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < H * D) {
      const int h = i / D, c = i % D;            // W1eT / W3eT entry (h, c)
      W1eT[i] = (bf16)W1[c * H + h];
      W3eT[i] = (bf16)W3[c * H + h];
      const int o = i / H, hh = i % H;           // W2T entry (o, hh)
      W2T[i] = (bf16)W2[hh * D + o];
    }
    return;
  }
  const int i = (blockIdx.x - nw) * 256 + threadIdx.x;
  if (i >= n_types * H) return;
  const int t = i / H, h = i % H;
  float s1 = 0.f, s3 = 0.f;
  for (int c = 0; c < D; ++c) {
    const float a = A[t * D + c];
    s1 = fmaf(a, W1[(D + c) * H + h], s1);
    s3 = fmaf(a, W3[(D + c) * H + h], s3);
  }
  T1[i] = s1;
  T3[i] = s3;
}

template <typename ET>
__device__ __forceinline__ bf16x8 load8_bf16(const ET* p) {
  if constexpr (sizeof(ET) == 2) {
    return *(const bf16x8*)p;
  } else {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
    bf16x8 r;
    r[0] = (bf16)a[0]; r[1] = (bf16)a[1]; r[2] = (bf16)a[2]; r[3] = (bf16)a[3];
    r[4] = (bf16)b[0]; r[5] = (bf16)b[1]; r[6] = (bf16)b[2]; r[7] = (bf16)b[3];
    return r;
  }
}

// Four consecutive values of an fp32 or bf16 row (one 16- or 8-byte access).
__device__ __forceinline__ f32x4 ld4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 ld4(const bf16* p) {
  const bf16x4 v = *(const bf16x4*)p;
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ void st4(float* p, f32x4 v) { *(f32x4*)p = v; }
__device__ __forceinline__ void st4(bf16* p, f32x4 v) {
  bf16x4 b;
  b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
  *(bf16x4*)p = b;
}

// grid: persistent, ntiles = ceil(T / 32) tiles of 32 events; block 256.
template <int D, typename ET>
__global__ __launch_bounds__(256, 1) void sa_action_fwd(const ET* __restrict__ e,
                                                        const int32_t* __restrict__ types,
                                                        int n_types, int64_t T,
                                                        const bf16* __restrict__ W1eT,
                                                        const bf16* __restrict__ W3eT,
                                                        const bf16* __restrict__ W2T,
                                                        const float* __restrict__ T1,
                                                        const float* __restrict__ T3,
                                                        ET* __restrict__ x) {
  constexpr int H = 2 * D;
  constexpr int KS = D / 16;               // K steps of the first products (over d)
  constexpr int KH = H / 16;               // K steps of the second product (over H)
  constexpr int MT = H / 32;               // 32-row hidden tiles (2, 4, 8)
  constexpr int NW = 4;
  constexpr int TPW = MT / NW > 0 ? MT / NW : 1;   // hidden tiles per wave
  constexpr int OT = D / 32;               // 32-row output tiles (1, 2, 4)
  constexpr int GROW = H + 8;              // bf16 per LDS row of G and W2^T (16-byte pad:
                                           // rows of 32 lanes fall on distinct banks)
  __shared__ __attribute__((aligned(16))) bf16 sW2[D * GROW];       // W2^T [out][H]
  __shared__ __attribute__((aligned(16))) bf16 sG[32 * GROW];       // G [event][H]
  __shared__ __attribute__((aligned(16))) float sT1[kActionMaxTypes * H];
  __shared__ __attribute__((aligned(16))) float sT3[kActionMaxTypes * H];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  for (int i = tid; i < D * H / 8; i += 256) {
    const int row = i / (H / 8), c8 = i % (H / 8);
    *(bf16x8*)(sW2 + row * GROW + 8 * c8) = ((const bf16x8*)W2T)[i];
  }
  for (int i = tid; i < n_types * H; i += 256) {
    sT1[i] = T1[i];
    sT3[i] = T3[i];
  }
  // This wave's hidden tiles (waves past MT have none when H < 128).
  const bool has_hidden = wave * TPW < MT;
  bf16x8 w1[TPW][KS], w3[TPW][KS];
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int row = (wave * TPW + m) * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      w1[m][ks] = has_hidden ? *(const bf16x8*)(W1eT + row * D + 16 * ks + 8 * h) : bf16x8{};
      w3[m][ks] = has_hidden ? *(const bf16x8*)(W3eT + row * D + 16 * ks + 8 * h) : bf16x8{};
    }
  }
  __syncthreads();

  const int64_t ntiles = (T + 31) / 32;
  // The next tile's event rows and type are loaded one tile ahead, and this
  // tile's residual rows at its start, so that the loads overlap the products
  // (one workgroup per CU: nothing else hides their latency).
  auto load_rows = [&](int64_t tl, bf16x8* eb, int& ty) {
    const int64_t ev = tl * 32 + l32;
    const bool valid = tl < ntiles && ev < T;
    ty = valid ? types[ev] : 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      eb[ks] = valid ? load8_bf16(e + ev * D + 16 * ks + 8 * h) : bf16x8{};
  };
  bf16x8 ebn[KS];
  int tyn;
  load_rows(blockIdx.x, ebn, tyn);
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t ev = tile * 32 + l32;            // this lane's event
    const bool valid = ev < T;
    const int ty = tyn;
    const int tcl = ty < 0 ? 0 : (ty >= n_types ? n_types - 1 : ty);   // clamped type
    // e^T as B operands: eb[ks] = e[ev][16 ks + 8h .. +7].
    bf16x8 eb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) eb[ks] = ebn[ks];
    // Residual: columns 32 wave + 8 g4 + 4h .. +3 of this lane's event (one
    // 4-element load each).
    f32x4 res[4];
    if (wave < OT) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        res[g4] = ld4(e + (valid ? ev : 0) * D + 32 * wave + 8 * g4 + 4 * h);
    }
    load_rows(tile + gridDim.x, ebn, tyn);
    if (has_hidden) {
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        // Register i: hidden row hb + crow(i, h), this lane's event.  The
        // products start from the event type's rows of T1 and T3 (4
        // consecutive hidden rows per register group).
        const int hb = (wave * TPW + m) * 32;
        f32x16 u1, u3;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int hr = tcl * H + hb + 8 * g4 + 4 * h;
          const f32x4 t1 = *(const f32x4*)&sT1[hr], t3 = *(const f32x4*)&sT3[hr];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            u1[4 * g4 + r] = t1[r];
            u3[4 * g4 + r] = t3[r];
          }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u1 = mfma32(w1[m][ks], eb[ks], u1);
          u3 = mfma32(w3[m][ks], eb[ks], u3);
        }
        // silu(a1) a3 = a1 a3 / (1 + exp(-a1)), with the hardware reciprocal
        // (the result is rounded to bf16).
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16 gv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * g4 + r;
            const float a1 = u1[i], a3 = u3[i];
            const float den = 1.0f + exp2_fast(a1 * -kLog2e);
            gv[r] = (bf16)(a1 * a3 * __builtin_amdgcn_rcpf(den));
          }
          bf16* dst = sG + l32 * GROW + hb + 8 * g4 + 4 * h;
          *(uint2*)dst = *(const uint2*)gv;
        }
      }
    }
    __syncthreads();
    // x^T rows [32 wave, +32): A = W2^T rows from LDS, B = G^T from LDS.
    if (wave < OT) {
      f32x16 xo = f32x16{};
#pragma unroll
      for (int kb = 0; kb < KH; ++kb) {
        const bf16x8 a = *(const bf16x8*)(sW2 + (32 * wave + l32) * GROW + 16 * kb + 8 * h);
        const bf16x8 b = *(const bf16x8*)(sG + l32 * GROW + 16 * kb + 8 * h);
        xo = mfma32(a, b, xo);
      }
      // Register i: output column 32 wave + crow(i, h) of this lane's event.
      if (valid) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int c = 32 * wave + 8 * g4 + 4 * h;
          const f32x4 v = {res[g4][0] + xo[4 * g4], res[g4][1] + xo[4 * g4 + 1],
                           res[g4][2] + xo[4 * g4 + 2], res[g4][3] + xo[4 * g4 + 3]};
          st4(x + ev * D + c, v);
        }
      }
    }
    __syncthreads();   // sG is rewritten by the next tile
  }
}

hipError_t launch_action_fwd(int d, int dtype, int64_t T, int n_types, const void* e,
                             const int32_t* types, const float* A, const float* W1,
                             const float* W3, const float* W2, void* prep, void* x,
                             hipStream_t st) {
  if (n_types < 1 || n_types > kActionMaxTypes) return hipErrorInvalidValue;
  const int H = 2 * d;
  bf16* W1eT = (bf16*)prep;
  bf16* W3eT = W1eT + H * d;
  bf16* W2T = W3eT + H * d;
  float* T1 = (float*)(W2T + H * d);
  float* T3 = T1 + kActionMaxTypes * H;
  const int nw = (H * d + 255) / 256;
  const int nt = (n_types * H + 255) / 256;
  const int64_t ntiles = (T + 31) / 32;
  const unsigned grid = (unsigned)(ntiles < 512 ? (ntiles > 0 ? ntiles : 1) : 512);
#define SA_ACTION_CASE(DD)                                                                       \
  case DD:                                                                                      \
    hipLaunchKernelGGL(sa_action_prep<DD>, dim3(nw + nt), dim3(256), 0, st, A, n_types, W1, W3, \
                       W2, W1eT, W3eT, W2T, T1, T3, nw);                                         \
    if (T <= 0) break;                                                                          \
    if (dtype == 1)                                                                             \
      hipLaunchKernelGGL((sa_action_fwd<DD, bf16>), dim3(grid), dim3(256), 0, st,                \
                         (const bf16*)e, types, n_types, T, W1eT, W3eT, W2T, T1, T3, (bf16*)x);  \
    else                                                                                        \
      hipLaunchKernelGGL((sa_action_fwd<DD, float>), dim3(grid), dim3(256), 0, st,               \
                         (const float*)e, types, n_types, T, W1eT, W3eT, W2T, T1, T3,            \
                         (float*)x);                                                             \
    break;
  switch (d) {
    SA_ACTION_CASE(32)
    SA_ACTION_CASE(64)
    SA_ACTION_CASE(128)
    default: return hipErrorInvalidValue;
  }
#undef SA_ACTION_CASE
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Helpers of the backward and of the fp32 path (the products themselves run
// in sa_gemm_mx, or in sa_gemm_f32 for fp32 histories).
// V = [e; A[t]] as fp32 rows of width 2D (the fp32 path's hidden layer).
template <typename ET>
__global__ __launch_bounds__(256) void sa_action_build_v(const ET* __restrict__ e,
                                                         const int32_t* __restrict__ types,
                                                         int n_types, const float* __restrict__ A,
                                                         int d, int64_t T, float* __restrict__ V) {
  // Thread -> 4 consecutive columns of one row of V = [e | A[type]] (d % 4 == 0).
  const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int qpr = d / 2;                         // float4 per row of V (2d / 4)
  if (i4 >= T * qpr) return;
  const int64_t ev = i4 / qpr;
  const int c = (int)(i4 % qpr) * 4;
  f32x4 v;
  if (c < d) {
    const ET* src = e + ev * d + c;
    v = f32x4{(float)src[0], (float)src[1], (float)src[2], (float)src[3]};
  } else {
    int t = types[ev];
    t = t < 0 ? 0 : (t >= n_types ? n_types - 1 : t);
    v = *(const f32x4*)(A + t * d + (c - d));
  }
  *(f32x4*)(V + ev * 2 * d + c) = v;
}

// ----------------------------------------------------------------------------
// Backward helpers without the materialised history rows.  With
// V = [e | A[type]], the products over V split into e W?e plus the per-type
// rows T? = A W?a, and every sum over the action half of V becomes a sum over
// the events of each type (rank n_types).

__device__ __forceinline__ float act_logistic(float u) {
  return __builtin_amdgcn_rcpf(1.0f + exp2_fast(u * -kLog2e));
}


// a1 = U1' + T1[type], a3 = U3' + T3[type] (4 columns per thread, H columns
// per row).  fwd: G = silu(a1) a3.  bwd: dU1 = dG a3 s (1 + a1 (1 - s)),
// dU3 = dG a1 s, s = logistic(a1).
template <bool BWD, typename IT>
__global__ __launch_bounds__(256) void sa_action_swiglu_t(const IT* __restrict__ dG,
                                                          const IT* __restrict__ U1,
                                                          const IT* __restrict__ U3,
                                                          const int32_t* __restrict__ types,
                                                          const float* __restrict__ T1,
                                                          const float* __restrict__ T3,
                                                          int n_types, int H, int64_t n4,
                                                          IT* __restrict__ out1,
                                                          IT* __restrict__ out3) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const int q = H / 4;
  const int64_t ev = i / q;
  const int c = (int)(i % q) * 4;
  int t = types[ev];
  t = t < 0 ? 0 : (t >= n_types ? n_types - 1 : t);
  const f32x4 a1 = ld4(U1 + 4 * i) + *(const f32x4*)(T1 + t * H + c);
  const f32x4 a3 = ld4(U3 + 4 * i) + *(const f32x4*)(T3 + t * H + c);
  f32x4 s;
#pragma unroll
  for (int r = 0; r < 4; ++r) s[r] = act_logistic(a1[r]);
  if (!BWD) {
    st4(out1 + 4 * i, a1 * s * a3);
  } else {
    const f32x4 g = ld4(dG + 4 * i);
    st4(out1 + 4 * i, g * a3 * s * (1.0f + a1 * (1.0f - s)));
    st4(out3 + 4 * i, g * a1 * s);
  }
}

// Per-type sums of the rows of X [T, ncol] (ncol in {64, 128, 256, 512,
// 1024}): this block's events, part[(blk n_types + t) ncol + c].  Sub-rows of
// ncol / 4 threads take events e0 + r, e0 + r + SR, ... in order into their
// own LDS accumulators, added in sub-row order (deterministic).
template <typename IT>
__global__ __launch_bounds__(256) void sa_action_type_sums(const IT* __restrict__ X,
                                                           const int32_t* __restrict__ types,
                                                           int n_types, int ncol, int64_t T,
                                                           int64_t epb, float* __restrict__ part) {
  __shared__ f32x4 acc[256 * kActionMaxTypes];   // [sub-row][type][quad]
  const int qpr = ncol / 4, sr_n = 256 / qpr;
  const int tid = threadIdx.x, q = tid % qpr, sr = tid / qpr;
  const int64_t e0 = (int64_t)blockIdx.x * epb;
  const int64_t e1 = e0 + epb < T ? e0 + epb : T;
  f32x4* mine = acc + sr * n_types * qpr + q;
  for (int t = 0; t < n_types; ++t) mine[t * qpr] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto clampt = [&](int t) { return t < 0 ? 0 : (t >= n_types ? n_types - 1 : t); };
  int64_t ev = e0 + sr;
  for (; ev + 3 * sr_n < e1; ev += 4 * sr_n) {   // four events' loads in flight
    f32x4 g[4];
    int t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      g[j] = ld4(X + (ev + j * sr_n) * ncol + 4 * q);
      t[j] = types[ev + j * sr_n];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) mine[clampt(t[j]) * qpr] += g[j];
  }
  for (; ev < e1; ev += sr_n) mine[clampt(types[ev]) * qpr] += ld4(X + ev * ncol + 4 * q);
  __syncthreads();
  for (int o = tid; o < n_types * qpr; o += 256) {
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < sr_n; ++r) sum += acc[r * n_types * qpr + o];
    *(f32x4*)(part + (int64_t)blockIdx.x * n_types * ncol + 4 * (int64_t)o) = sum;
  }
}

// The rank-n_types products of the backward, one thread per output:
//   mode 0: T1 = A W1a, T3 = A W3a                       ([n_types, H] each)
//   mode 1: dA = S1 W1a^T + S3 W3a^T                      ([n_types, d])
//           dW1[d + c][h] = sum_t A[t][c] S1[t][h], dW3 likewise ([d, H] each)
// with W1a, W3a the rows d .. 2d - 1 of W1, W3 ([2d, H]).
__global__ __launch_bounds__(256) void sa_action_small(int mode, int d, int n_types,
                                                       const float* __restrict__ A,
                                                       const float* __restrict__ W1,
                                                       const float* __restrict__ W3,
                                                       const float* __restrict__ S1,
                                                       const float* __restrict__ S3,
                                                       float* __restrict__ T1,
                                                       float* __restrict__ T3,
                                                       float* __restrict__ dA,
                                                       float* __restrict__ dW1,
                                                       float* __restrict__ dW3) {
  const int H = 2 * d;
  const float* W1a = W1 + (int64_t)d * H;
  const float* W3a = W3 + (int64_t)d * H;
  int i = blockIdx.x * 256 + threadIdx.x;
  if (mode == 0) {
    if (i >= n_types * H) return;
    const int t = i / H, h = i % H;
    // d is a multiple of 8: eight terms' loads in flight, eight partial sums.
    float s1[8] = {}, s3[8] = {};
    for (int c = 0; c < d; c += 8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = A[t * d + c + j];
        s1[j] = fmaf(a, W1a[(c + j) * H + h], s1[j]);
        s3[j] = fmaf(a, W3a[(c + j) * H + h], s3[j]);
      }
    }
    T1[i] = ((s1[0] + s1[1]) + (s1[2] + s1[3])) + ((s1[4] + s1[5]) + (s1[6] + s1[7]));
    T3[i] = ((s3[0] + s3[1]) + (s3[2] + s3[3])) + ((s3[4] + s3[5]) + (s3[6] + s3[7]));
    return;
  }
  if (i < n_types * d) {
    const int t = i / d, c = i % d;
    const f32x4* s1r = (const f32x4*)(S1 + t * H);
    const f32x4* s3r = (const f32x4*)(S3 + t * H);
    const f32x4* w1r = (const f32x4*)(W1a + (int64_t)c * H);
    const f32x4* w3r = (const f32x4*)(W3a + (int64_t)c * H);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int h4 = 0; h4 < H / 4; ++h4) s += s1r[h4] * w1r[h4] + s3r[h4] * w3r[h4];
    dA[i] = (s[0] + s[1]) + (s[2] + s[3]);
    return;
  }
  i -= n_types * d;
  if (i >= d * H) return;
  const int c = i / H, h = i % H;
  float s1 = 0.f, s3 = 0.f;
  for (int t = 0; t < n_types; ++t) {
    const float a = A[t * d + c];
    s1 = fmaf(a, S1[t * H + h], s1);
    s3 = fmaf(a, S3[t * H + h], s3);
  }
  dW1[(int64_t)d * H + i] = s1;
  dW3[(int64_t)d * H + i] = s3;
}

hipError_t launch_action_small(int mode, int d, int n_types, const float* A, const float* W1,
                               const float* W3, const float* S1, const float* S3, float* T1,
                               float* T3, float* dA, float* dW1, float* dW3, hipStream_t st) {
  const int H = 2 * d;
  const int n = mode == 0 ? n_types * H : n_types * d + d * H;
  hipLaunchKernelGGL(sa_action_small, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, mode, d,
                     n_types, A, W1, W3, S1, S3, T1, T3, dA, dW1, dW3);
  return hipGetLastError();
}

hipError_t launch_action_swiglu(bool bwd, bool bf16_io, const void* dG, const void* U1,
                                const void* U3, const int32_t* types, const float* T1,
                                const float* T3, int n_types, int H, int64_t T, void* out1,
                                void* out3, hipStream_t st) {
  const int64_t n4 = T * (H / 4);
  if (n4 <= 0) return hipSuccess;
  const unsigned nb = (unsigned)((n4 + 255) / 256);
#define SA_SWIGLU(B_, IT_)                                                                       \
  hipLaunchKernelGGL((sa_action_swiglu_t<B_, IT_>), dim3(nb), dim3(256), 0, st, (const IT_*)dG, \
                     (const IT_*)U1, (const IT_*)U3, types, T1, T3, n_types, H, n4, (IT_*)out1,  \
                     (IT_*)out3)
  if (bf16_io) {
    if (bwd) SA_SWIGLU(true, bf16);
    else SA_SWIGLU(false, bf16);
  } else {
    if (bwd) SA_SWIGLU(true, float);
    else SA_SWIGLU(false, float);
  }
#undef SA_SWIGLU
  return hipGetLastError();
}

hipError_t launch_action_type_sums(bool bf16_in, const void* X, const int32_t* types, int n_types,
                                   int ncol, int64_t T, float* part, int nblk, hipStream_t st) {
  if (n_types < 1 || n_types > kActionMaxTypes || ncol % 4 != 0 || ncol > 1024 ||
      256 % (ncol / 4) != 0)
    return hipErrorInvalidValue;
  const int64_t epb = (T + nblk - 1) / nblk;
  if (bf16_in)
    hipLaunchKernelGGL(sa_action_type_sums<bf16>, dim3(nblk), dim3(256), 0, st, (const bf16*)X,
                       types, n_types, ncol, T, epb > 0 ? epb : 1, part);
  else
    hipLaunchKernelGGL(sa_action_type_sums<float>, dim3(nblk), dim3(256), 0, st, (const float*)X,
                       types, n_types, ncol, T, epb > 0 ? epb : 1, part);
  return hipGetLastError();
}

hipError_t launch_action_build_v(int d, int dtype, int64_t T, int n_types, const void* e,
                                 const int32_t* types, const float* A, float* V, hipStream_t st) {
  const int64_t n = T * (d / 2);                  // float4 of V
  if (n <= 0) return hipSuccess;
  const unsigned nb = (unsigned)((n + 255) / 256);
  if (dtype == 1)
    hipLaunchKernelGGL(sa_action_build_v<bf16>, dim3(nb), dim3(256), 0, st, (const bf16*)e, types,
                       n_types, A, d, T, V);
  else
    hipLaunchKernelGGL(sa_action_build_v<float>, dim3(nb), dim3(256), 0, st, (const float*)e,
                       types, n_types, A, d, T, V);
  return hipGetLastError();
}

size_t action_prep_bytes(int d) {
  const size_t H = 2 * (size_t)d;
  return 3 * H * d * 2 + 2 * (size_t)kActionMaxTypes * H * 4;
}

}  // namespace sa
