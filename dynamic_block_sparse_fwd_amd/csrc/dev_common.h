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
typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
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

// Cross-lane exchanges done in the VALU, without the LDS round trip of a bpermute shuffle.
// DPP inside 16-lane rows: quad_perm [1,0,3,2] reads lane ^ 1, [2,3,0,1] lane ^ 2,
// row_half_mirror lane 7 - i of its 8-lane half, row_mirror lane 15 - i of its row.  Once a
// value is uniform over aligned groups of 4 (8), the half mirror (mirror) reads the partner
// group exactly as lane ^ 4 (lane ^ 8) would.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
// Partner read for step o = 1, 2, 4, 8 of a butterfly over aligned lane groups.
template <int O>
__device__ __forceinline__ float xor_lane_f(float v) {
  static_assert(O == 1 || O == 2 || O == 4 || O == 8, "DPP butterfly step");
  return dpp_f<O == 1 ? kDppXor1 : O == 2 ? kDppXor2 : O == 4 ? kDppHalfMirror : kDppMirror>(v);
}
template <int O>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v) {
  return dpp_u32<O == 1 ? kDppXor1 : O == 2 ? kDppXor2 : O == 4 ? kDppHalfMirror : kDppMirror>(v);
}

// gfx950 row swaps, both operands the same value: .x gets the even (lower) row or half of each
// pair, .y the odd (upper) one, in every lane of the pair.  x + y and max(x, y) therefore equal
// v + v[lane ^ 16] (swap16) or v + v[lane ^ 32] (swap32) exactly.
struct U32Pair { uint32_t x, y; };
__device__ __forceinline__ U32Pair swap16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return {r[0], r[1]};
}
__device__ __forceinline__ U32Pair swap32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return {r[0], r[1]};
}

// Max / sum over the four lanes that hold one C-layout column (lanes L, L^16, L^32, L^48).
__device__ __forceinline__ float col_max4(float v) {
  U32Pair p = swap16(__float_as_uint(v));
  v = fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
  p = swap32(__float_as_uint(v));
  return fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
}
__device__ __forceinline__ float col_sum4(float v) {
  U32Pair p = swap16(__float_as_uint(v));
  v = __uint_as_float(p.x) + __uint_as_float(p.y);
  p = swap32(__float_as_uint(v));
  return __uint_as_float(p.x) + __uint_as_float(p.y);
}

// Sum / max over aligned groups of GS consecutive lanes inside each 16-lane row (GS = 1, 2, 4,
// 8 or 16).
template <int GS>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(GS == 1 || GS == 2 || GS == 4 || GS == 8 || GS == 16, "group size");
  if constexpr (GS > 1) v += xor_lane_f<1>(v);
  if constexpr (GS > 2) v += xor_lane_f<2>(v);
  if constexpr (GS > 4) v += xor_lane_f<4>(v);
  if constexpr (GS > 8) v += xor_lane_f<8>(v);
  return v;
}
template <int GS>
__device__ __forceinline__ float group_max(float v) {
  static_assert(GS == 1 || GS == 2 || GS == 4 || GS == 8 || GS == 16, "group size");
  if constexpr (GS > 1) v = fmaxf(v, xor_lane_f<1>(v));
  if constexpr (GS > 2) v = fmaxf(v, xor_lane_f<2>(v));
  if constexpr (GS > 4) v = fmaxf(v, xor_lane_f<4>(v));
  if constexpr (GS > 8) v = fmaxf(v, xor_lane_f<8>(v));
  return v;
}

// Max / sum over the whole wave (rows, then across the four rows), returned in every lane; the
// order of the additions is fixed, so the result is the same on every call.
__device__ __forceinline__ float wave_max_f(float v) { return col_max4(group_max<16>(v)); }
__device__ __forceinline__ float wave_sum_f(float v) { return col_sum4(group_sum<16>(v)); }

// Unsigned max over the whole wave, returned in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, xor_lane_u32<1>(v));
  v = max(v, xor_lane_u32<2>(v));
  v = max(v, xor_lane_u32<4>(v));
  v = max(v, xor_lane_u32<8>(v));
  U32Pair p = swap16(v);
  v = max(p.x, p.y);
  p = swap32(v);
  return max(p.x, p.y);
}

// Lazy online-softmax rescaling: headroom of a row's reference max, in log2 units.  The
// reference moves (and the accumulators are rescaled) only when a score exceeds it by more than
// this, so probabilities fed to the matrix core stay below 2^8 (bf16 keeps its relative
// precision there) and most tiles skip the rescale.
constexpr float kLazyLog2 = 8.f;

// Workgroup barrier that orders LDS only: unlike __syncthreads it does not wait for global
// loads in flight, so prefetches issued before it stay outstanding.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

// Max of 64-bit keys over the whole (fully active) wave: high words first; the low word is read
// from the one lane holding the top high word, or reduced over the lanes that tie on it.
// Returned in every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = static_cast<uint32_t>(v >> 32);
  const uint32_t top = wave_max_u32(hi);
  const uint64_t eq = __ballot(hi == top);
  uint32_t lo;
  if (__popcll(eq) == 1)  // uniform
    lo = (uint32_t)__builtin_amdgcn_readlane((int)static_cast<uint32_t>(v),
                                             (int)__builtin_ctzll(eq));
  else
    lo = wave_max_u32(hi == top ? static_cast<uint32_t>(v) : 0u);
  return (static_cast<uint64_t>(top) << 32) | lo;
}

// Max of v over lanes L, L^16, L^32, L^48 (one C-layout column), for 64-bit keys.
__device__ __forceinline__ uint64_t col_max4_u64(uint64_t v) {
#pragma unroll
  for (int step = 0; step < 2; ++step) {
    const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
    const U32Pair pl = step == 0 ? swap16(lo) : swap32(lo);
    const U32Pair ph = step == 0 ? swap16(hi) : swap32(hi);
    v = u64_max((static_cast<uint64_t>(ph.x) << 32) | pl.x,
                (static_cast<uint64_t>(ph.y) << 32) | pl.y);
  }
  return v;
}

// Top-k by (key desc) of keyof(first) .. keyof(last - 1), 64-bit keys (score bits << 32 |
// ~index, 0 = none).  Every lane keeps its four best candidates; the wave repeatedly takes the
// best head, and a lane that runs out rescans below its last popped key (unless it never had
// more than four).  Lane e < k receives
// the e-th winner's key (0 when there are fewer than k candidates).
template <class KeyOf>
__device__ uint64_t wave_topk(KeyOf keyof, int first, int last, int k, int lane) {
  uint64_t c[4] = {0, 0, 0, 0};
  auto insert = [&](uint64_t key) {
    if (key <= c[3]) return;
    if (key > c[0]) { c[3] = c[2]; c[2] = c[1]; c[1] = c[0]; c[0] = key; }
    else if (key > c[1]) { c[3] = c[2]; c[2] = c[1]; c[1] = key; }
    else if (key > c[2]) { c[3] = c[2]; c[2] = key; }
    else c[3] = key;
  };
  int n = 0;
  for (int j = first + lane; j < last; j += 64, ++n) insert(keyof(j));
  uint64_t mine = 0;
  for (int it = 0; it < k; ++it) {
    const uint64_t best = wave_max_u64(c[0]);
    if (lane == it) mine = best;
    if (c[0] == best && best != 0) {
      c[0] = c[1]; c[1] = c[2]; c[2] = c[3]; c[3] = 0;
      if (c[0] == 0 && n > 4) {  // cache exhausted: rescan strictly below the popped key
        for (int j = first + lane; j < last; j += 64) {
          const uint64_t key = keyof(j);
          if (key < best) insert(key);
        }
      }
    }
  }
  return mine;
}

// Adaptive top-p cut of a ranked free list held one key per lane (lane e < k: the e-th best free
// block's rank key, 0 = none).  Lane e keeps its key while the importance chosen before it --
// the forced blocks' total, then the better free blocks added in rank order -- is below target,
// and gets 0 otherwise; the kept lanes are a prefix.  Called by the whole wave.
__device__ __forceinline__ uint64_t top_p_cut(uint64_t key, int k, float forced, float target,
                                              int lane) {
  const int sbits = (int)(uint32_t)(key >> 32);  // the score's bits (rank_key's high word)
  float before = forced;
  for (int o = 0; o < k; ++o) {
    const float s = __int_as_float(__builtin_amdgcn_readlane(sbits, o));
    if (o < lane) before += s;
  }
  return before < target ? key : 0;
}

}  // namespace nsa
