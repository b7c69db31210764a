// Attention tile building blocks shared by the prefill and MoBA kernels: 64-key K/V tiles
// staged in LDS, S^T = K Q^T sub-tiles and O^T += V^T P^T chunks (layouts in dev_common.h).
#pragma once
#include "dev_common.h"

namespace nsa {

// Cooperative copy of a 64-row x D tile (row-major, 16-byte rows chunks) into LDS [64][D+KPAD].
template <int D, int NT>
__device__ __forceinline__ void load_rows_tile(u16 (*dst)[D + KPAD], const u16* src, long row0,
                                               int row_limit) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  for (int c = threadIdx.x; c < 64 * CH; c += NT) {
    const int r = c / CH, o = (c % CH) * 8;
    long row = row0 + r;
    if (row > row_limit) row = row_limit;
    store8(&dst[r][o], load8(src + row * D + o));
  }
}

// Cooperative copy of a D x 64 tile of a transposed tensor (keys contiguous, row pitch `pitch`).
template <int D, int NT>
__device__ __forceinline__ void load_cols_tile(u16 (*dst)[64 + KPAD], const u16* src, long pitch,
                                               long col0) {
  for (int c = threadIdx.x; c < D * 8; c += NT) {
    const int r = c >> 3, o = (c & 7) * 8;
    store8(&dst[r][o], load8(src + r * pitch + col0 + o));
  }
}

// S^T sub-tile: 16 keys (chunk kc, sub-tile s of the LDS tile) x 16 query rows.
template <int D>
__device__ __forceinline__ f32x4 score_subtile(const u16 (*Ks)[D + KPAD], const bf16x8* qf,
                                               int kc, int s, int g4, int r16) {
  f32x4 acc = zero4();
  const u16* krow = Ks[32 * kc + perm_key(r16, s)];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) acc = mfma16x16x32(load8(krow + 32 * c + 8 * g4), qf[c], acc);
  return acc;
}

// O^T += V^T P^T for one 32-key chunk; pb holds this lane's row probabilities for keys
// 32*kc + 8*g4 .. +7.
template <int D>
__device__ __forceinline__ void pv_chunk(const u16 (*Vs)[64 + KPAD], const bf16x8& pb, int kc,
                                         int g4, int r16, f32x4* O) {
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
    O[n] = mfma16x16x32(load8(&Vs[16 * n + r16][32 * kc + 8 * g4]), pb, O[n]);
}

}  // namespace nsa
