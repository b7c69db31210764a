// Device-side helpers shared by the gfx950 kernels of the NSA / MoBA forward library.
//
// Matrix-core conventions (v_mfma_f32_16x16x32_bf16, wave64), used by every kernel:
//   A operand (16 x 32, M x K): lane L holds A[L % 16][8 * (L / 16) + e], e = 0..7
//   B operand (32 x 16, K x N): lane L holds B[8 * (L / 16) + e][L % 16], e = 0..7
//   C/D       (16 x 16)       : lane L holds C[4 * (L / 16) + i][L % 16], i = 0..3
// The K index seen by one lane is a contiguous run of 8, so both operands are loaded with one
// 16-byte read when the reduction dimension is the contiguous one in memory.
//
// Attention tiles are computed transposed (S^T = K Q^T, O^T = V^T P^T) so that the
// accumulator of a lane always belongs to ONE query row (L % 16): the softmax statistics of a
// row live in the lanes that own the row, and P^T is already in B-operand layout.  To make
// the P^T fragment's keys contiguous, the two 16-key S^T sub-tiles of a 32-key chunk read
// their K rows in the order  sub-tile s, C-row 4g+i  <->  key 8g + 4s + i.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load8(const u16* p) {  // 16-byte aligned
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ void store8(u16* p, const bf16x8& v) {
  *reinterpret_cast<bf16x8*>(p) = v;
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.0f;
  return z;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_to_f32(u16 b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return *reinterpret_cast<u16*>(&h);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Max over the four lanes that hold one C-layout column (lanes L, L^16, L^32, L^48).
__device__ __forceinline__ float col_max4(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float col_sum4(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Sum over aligned groups of GS consecutive lanes inside each 16-lane row (GS = 1..16).
template <int GS>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < GS; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// Workgroup barrier that orders LDS only: unlike __syncthreads it does not wait for global
// loads in flight, so prefetches issued before it stay outstanding.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int GS>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = 1; o < GS; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Key offset (inside a 32-key chunk) of C-row r of sub-tile s, per the ordering above.
__device__ __forceinline__ int perm_key(int r, int s) { return 8 * (r >> 2) + 4 * s + (r & 3); }

// bf16 padding of LDS rows (16 bytes) against bank conflicts.
constexpr int KPAD = 8;

// Compressed tokens visible to query position t: token i covers [i*d, i*d + l) and is
// visible once its whole span is in the past.
__device__ __forceinline__ int n_visible(int t, int l, int d, int ncmp) {
  if (t < l - 1) return 0;
  const int n = (t - l + 1) / d + 1;
  return n < ncmp ? n : ncmp;
}

__device__ __forceinline__ uint64_t u64_max(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Ranking key of a non-negative score: larger score first, then lower index.
__device__ __forceinline__ uint64_t rank_key(float score, int j) {
  return (static_cast<uint64_t>(__float_as_uint(score)) << 32) | (0xFFFFFFFFu - (uint32_t)j);
}
__device__ __forceinline__ int rank_key_index(uint64_t key) {
  return (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o);
  uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = u64_max(v, shfl_xor_u64(v, o));
  return v;
}

}  // namespace nsa
