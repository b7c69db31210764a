// Attention tile building blocks shared by the prefill and MoBA kernels: 64-key K/V tiles
// staged in LDS, S^T = K Q^T sub-tiles and O^T += V^T P^T chunks (layouts in dev_common.h).
//
// LDS tiles are unpadded and XOR-swizzled in 16-byte chunks so that the 16-byte operand reads
// of a wave are free of bank conflicts:
//   K tile  Ks[64][D]: chunk c of key row r is stored at chunk c ^ k_swz(r), where k_swz(r) is
//           the lane index (lane & 15) that reads row r (4 bits for the 16 chunks of a D = 128
//           row, 3 bits for D = 64);
//   V tile  Vs[D][64]: chunk c of feature row r is stored at chunk c ^ (r & 7).
// With the sub-tile row order of dev_common.h a read of logical K chunk c by lane L is at
// physical chunk c ^ (L & 15) (D = 128), a V read at c ^ (L & 7).  (A 3-bit K swizzle at
// D = 128 left lanes L and L + 8 on the same banks: the counters showed as many conflict cycles
// as LDS instructions.)
#pragma once
#include "dev_common.h"

namespace nsa {

// Swizzle of K row r: the lane index r16 that reads the row (see perm_key), 4 bits wide when a
// row has 16 chunks (D = 128), 3 bits otherwise.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D >= 128 ? ((r & 3) | ((r & 24) >> 1)) : ((r & 3) | ((r & 8) >> 1));
}

// Global -> register staging of one 64 x D K tile (row-major source) and one D x 64 V tile
// (keys contiguous, row pitch `pitch`), NT threads; then register -> LDS with the swizzle.
template <int D, int NT>
struct KTileRegs {
  static_assert((64 * D / 8) % NT == 0, "K tile chunks must split evenly over the threads");
  static constexpr int N = 64 * D / 8 / NT;
  u32x4 r[N];
  // rows row0 .. row0+63 of src (row_limit >= row0 clamps the tail); a uniform base pointer and
  // a 32-bit lane offset keep the address arithmetic scalar
  __device__ __forceinline__ void load(const u16* src, long row0, int row_limit) {
    const u16* base = src + row0 * D;
    const int lim = row_limit - (int)row0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + i * NT;
      const int rr = c / (D / 8), o = c % (D / 8);
      const int row = rr < lim ? rr : lim;
      r[i] = *reinterpret_cast<const u32x4*>(base + (uint32_t)(row * D + o * 8));
    }
  }
  __device__ __forceinline__ void store(u16 (*Ks)[D]) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + i * NT;
      const int rr = c / (D / 8), o = c % (D / 8);
      *reinterpret_cast<u32x4*>(&Ks[rr][(o ^ k_swz<D>(rr)) * 8]) = r[i];
    }
  }
};

template <int D, int NT>
struct VTileRegs {
  static_assert((D * 8) % NT == 0, "V tile chunks must split evenly over the threads");
  static constexpr int N = D * 8 / NT;
  u32x4 r[N];
  __device__ __forceinline__ void load(const u16* src, long pitch, long col0) {
    const u16* base = src + col0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + i * NT;
      const int rr = c >> 3, o = c & 7;
      r[i] = *reinterpret_cast<const u32x4*>(base + (uint32_t)(rr * (int)pitch + o * 8));
    }
  }
  __device__ __forceinline__ void store(u16 (*Vs)[64]) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + i * NT;
      const int rr = c >> 3, o = c & 7;
      *reinterpret_cast<u32x4*>(&Vs[rr][(o ^ (rr & 7)) * 8]) = r[i];
    }
  }
};

// Direct (unpipelined) tile copies.
template <int D, int NT>
__device__ __forceinline__ void load_rows_tile(u16 (*dst)[D], const u16* src, long row0,
                                               int row_limit) {
  KTileRegs<D, NT> t;
  t.load(src, row0, row_limit);
  t.store(dst);
}

template <int D, int NT>
__device__ __forceinline__ void load_cols_tile(u16 (*dst)[64], const u16* src, long pitch,
                                               long col0) {
  VTileRegs<D, NT> t;
  t.load(src, pitch, col0);
  t.store(dst);
}

// The D/32 A-operand fragments of the K rows this lane reads for sub-tile (kc, s).
template <int D>
__device__ __forceinline__ void k_frags(const u16 (*Ks)[D], int kc, int s, int g4, int r16,
                                        bf16x8* kf) {
  const u16* krow = Ks[32 * kc + perm_key(r16, s)];
  const int x = D >= 128 ? r16 : (r16 & 7);
#pragma unroll
  for (int c = 0; c < D / 32; ++c) kf[c] = load8(krow + (((4 * c + g4) ^ x) * 8));
}

// S^T sub-tile: 16 keys (chunk kc, sub-tile s of the LDS tile) x 16 query rows.
template <int D>
__device__ __forceinline__ f32x4 score_subtile(const u16 (*Ks)[D], const bf16x8* qf, int kc,
                                               int s, int g4, int r16) {
  bf16x8 kf[D / 32];
  k_frags<D>(Ks, kc, s, g4, r16, kf);
  f32x4 acc = zero4();
#pragma unroll
  for (int c = 0; c < D / 32; ++c) acc = mfma16x16x32(kf[c], qf[c], acc);
  return acc;
}

// O^T += V^T P^T for one 32-key chunk; pb holds this lane's row probabilities for keys
// 32*kc + 8*g4 .. +7.
template <int D>
__device__ __forceinline__ void pv_chunk(const u16 (*Vs)[64], const bf16x8& pb, int kc, int g4,
                                         int r16, f32x4* O) {
  const int ch = ((4 * kc + g4) ^ (r16 & 7)) * 8;
#pragma unroll
  for (int n = 0; n < D / 16; ++n) O[n] = mfma16x16x32(load8(&Vs[16 * n + r16][ch]), pb, O[n]);
}

// S^T for RTW row tiles against the 64-key LDS tile: each K fragment is read from LDS once
// and multiplies every row tile (LDS bandwidth, not the matrix core, is the scarcer resource
// when each fragment feeds one MFMA).  raw[rt][kc*8 + s*4 + i] = score of key
// 32*kc + 8*g4 + 4*s + i for row tile rt.
template <int D, int RTW>
__device__ __forceinline__ void score_tiles(const u16 (*Ks)[D], const bf16x8 (*qf)[D / 32],
                                            int g4, int r16, float (*raw)[16]) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 kf[D / 32];
      k_frags<D>(Ks, kc, s, g4, r16, kf);
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int c = 0; c < D / 32; ++c) acc = mfma16x16x32(kf[c], qf[rt][c], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[rt][kc * 8 + s * 4 + i] = acc[i];
      }
    }
}

// O^T += V^T P^T for RTW row tiles: each V fragment is read from LDS once.  pb[rt][kc] holds
// row tile rt's probabilities of keys 32*kc + 8*g4 .. +7.
template <int D, int RTW>
__device__ __forceinline__ void pv_tiles(const u16 (*Vs)[64], const bf16x8 (*pb)[2], int g4,
                                         int r16, f32x4 (*O)[D / 16]) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const int ch = ((4 * kc + g4) ^ (r16 & 7)) * 8;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      const bf16x8 vf = load8(&Vs[16 * n + r16][ch]);
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) O[rt][n] = mfma16x16x32(vf, pb[rt][kc], O[rt][n]);
    }
  }
}

// Sum over the 16 lanes of a DPP row (row rotations 8, 4, 2, 1); every lane ends with a sum,
// lane 0 of the row with a fixed association.  A rotation never leaves the row, so bound_ctrl
// is moot and set, which lets the compiler fold each move into the add (v_add_f32_dpp).
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xF, 0xF, true));
  return v;
}

}  // namespace nsa
