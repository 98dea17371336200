// sa_device.h — device-side building blocks shared by the Sketch Attention
// kernels: vector types, matrix-core wrappers, the CSR segment walker and the
// work partition.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define SA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_mfma_f32_32x32x16_bf16.  Operand layout (lane l, half h = l / 32):
//   A (32 x 16, M x K): lane l holds A[l % 32][8h .. 8h+7]
//   B (16 x 32, K x N): lane l holds B[8h .. 8h+7][l % 32]
//   C (32 x 32):        lane l, register i holds
//                       C[8 (i / 4) + 4h + (i % 4)][l % 32]
// Only the pairing of A's and B's K slots matters for a product, so any
// consistent assignment of the reduction index to (h, slot) is valid.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32 x 32 C tile held by register i of a lane in half h.
__device__ __forceinline__ constexpr int crow(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane 4r + c points at 4 consecutive 16-bit elements: row r, columns
// 4c .. 4c+3 of a 4 x 16 block.  Lane j of the group receives column j of
// rows 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const SA_LDS bf16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS i16x4*)p);
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 concat4(bf16x4 a, bf16x4 b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Direct global -> LDS copies (global_load_lds_dword{,x4}).  lds_copy16:
// lane i copies the 16 bytes at sbase + voff_i to LDS byte address
// lds + 16 i; sbase and lds must be the same for every lane of the wave.
// Written as assembly so that the compiler does not turn every later LDS read
// into a wait for all copies in flight: the caller orders them with explicit
// vmcnt waits.  The instructions write no register.  Every call sets M0, and
// no compiler-generated code in these kernels keeps a value in M0.  An LDS DMA
// reads M0 one wait state after an SALU write to it at the earliest (the
// compiler's own global_load_lds code keeps that gap), hence the s_nop 0:
// without it the copy can take the previous M0 and write another LDS address.
__device__ __forceinline__ uint32_t lds_addr(const SA_LDS void* p) {
  return (uint32_t)(uintptr_t)p;
}
__device__ __forceinline__ void lds_copy16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
// Lane i copies the 4 bytes at its own address src_i to LDS byte address
// lds + 4 i.
__device__ __forceinline__ void lds_copy4v(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight.
// Also a compiler memory barrier, so no LDS access moves across it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait for all vector-memory operations of this wave, written so that the
// compiler sees the wait (s_waitcnt vmcnt(0), expcnt and lgkmcnt untouched).
// Its own earlier loads and stores then count as complete, and it adds no wait
// for them inside a following loop, where such a wait would also hold up every
// copy in flight on every trip.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0xF70); }
// Workgroup barrier after this wave's LDS reads and writes have completed.
// Unlike __syncthreads() it does not wait for global loads (or the direct
// global -> LDS copies) still in flight.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float shfl_xor32(float v) { return __shfl_xor(v, 32, 64); }

// ---------------------------------------------------------------------------
// Work partition of the concatenated token axis.
//
// The T tokens are cut into G contiguous segments of (almost) equal size,
// segment s = [floor(T s / G), floor(T (s+1) / G)).  With G <= T every segment
// is non-empty.  The part of segment s that belongs to user u is a "piece";
// its partial result lives in slot s + u, which is unique because pieces
// appear in increasing (s, u) order and consecutive pieces raise s + u by at
// least one.  The slot count is therefore G + B - 1.
__device__ __forceinline__ int64_t seg_lo(int64_t T, int G, int s) {
  // floor(T s / G) without a 64-bit integer division: T s < 2^44 is exact in
  // double, and the integer check makes the rounded quotient exact.
  const int64_t x = T * (int64_t)s;
  int64_t q = (int64_t)((double)x / (double)G);
  if (q * G > x) --q;
  else if ((q + 1) * G <= x) ++q;
  return q;
}

// Largest s with seg_lo(s) <= t (the segment holding token t).
__device__ __forceinline__ int seg_of(int64_t T, int G, int64_t t) {
  int s = (int)((double)t * (double)G / (double)T);
  if (s > G - 1) s = G - 1;
  if (s < 0) s = 0;
  while (s + 1 < G && seg_lo(T, G, s + 1) <= t) ++s;
  while (s > 0 && seg_lo(T, G, s) > t) --s;
  return s;
}

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// Load of a value that is the same for every lane (offsets, which no kernel
// writes), as a scalar load: it is waited for with lgkmcnt, so its wait does
// not also wait for the vector loads and direct-to-LDS copies in flight, as a
// vector load's vmcnt wait would.
__device__ __forceinline__ int64_t uload64(const int64_t* p) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  typedef const __attribute__((address_space(4))) int64_t* const_i64_ptr;
  return *(const_i64_ptr)(((uint64_t)hi << 32) | lo);
}

// First user whose row range ends after token t (offsets[u+1] > t).
// Offsets are read as they are and every result is clamped, so corrupt
// offsets cannot cause an out-of-range user index.
__device__ __forceinline__ int first_user_after(const int64_t* offsets, int B, int64_t t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (uload64(offsets + mid + 1) <= t) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Block-wide check of the CSR offsets (offsets[0] = 0, non-decreasing,
// offsets[B] = T); thread 0 writes the status word and, unless keep2, clears
// the second status word (the single-pass forward's exchange status, which
// its reduce keeps).  Every thread of the block must call it.
__device__ __forceinline__ void check_offsets_block(const int64_t* offsets, int B, int64_t T,
                                                    uint32_t* status, uint32_t ok, uint32_t bad_code,
                                                    bool keep2 = false) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = (offsets[0] != 0 || offsets[B] != T) ? 1 : 0;
  __syncthreads();
  for (int i = threadIdx.x; i < B; i += blockDim.x)
    if (offsets[i + 1] < offsets[i]) bad = 1;
  __syncthreads();
  if (threadIdx.x == 0) {
    *status = bad ? bad_code : ok;
    if (!keep2) status[1] = ok;
  }
}

// LDS layout of a 32-token x D tile without padding: row r holds D/8 units of
// 16 bytes, unit u stored at position u ^ xswz(r).  The swizzle makes both
// access patterns bank-conflict free:
//  - 16 lanes reading one unit of 16 consecutive rows (the affinity product's
//    A operand), and
//  - 32 lanes transpose-reading 4 consecutive rows x one 32-column block (the
//    aggregation product's A operand).
template <int D>
__device__ __forceinline__ int xswz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return (r >> 2) & 3;
}

template <int D>
__device__ __forceinline__ int xoff(int r, int u) { return r * D + ((u ^ xswz<D>(r)) << 3); }

// Walks the pieces of one segment in token order, in tiles of TILE tokens.
// A tile never straddles two users.
template <int TILE>
struct TileWalker {
  const int64_t* offsets;
  int B;
  int64_t seg_begin, seg_end;
  // current tile
  int user;
  int64_t t0, t1;          // tile rows [t0, t1)
  int64_t piece_end;       // end of the current piece
  bool valid;

  __device__ void start(const int64_t* off, int nb, int64_t lo, int64_t hi) {
    offsets = off; B = nb; seg_begin = lo; seg_end = hi;
    valid = lo < hi;
    if (!valid) return;
    user = first_user_after(off, nb, lo);
    t0 = lo;
    piece_end = clamp64(uload64(off + user + 1), t0, hi);
    if (piece_end <= t0) piece_end = hi;   // only with corrupt offsets
    t1 = t0 + TILE < piece_end ? t0 + TILE : piece_end;
  }
  __device__ bool last_in_piece() const { return t1 >= piece_end; }
  __device__ void advance() {
    if (t1 < piece_end) {
      t0 = t1;
    } else {
      if (piece_end >= seg_end) { valid = false; return; }
      t0 = piece_end;
      // next user with a non-empty range starting at t0
      int u = user + 1;
      while (u < B - 1 && uload64(offsets + u + 1) <= t0) ++u;
      if (u > B - 1) u = B - 1;
      user = u;
      piece_end = clamp64(uload64(offsets + u + 1), t0, seg_end);
      if (piece_end <= t0) piece_end = seg_end;   // only with corrupt offsets
    }
    t1 = t0 + TILE < piece_end ? t0 + TILE : piece_end;
  }
};

}  // namespace sa
