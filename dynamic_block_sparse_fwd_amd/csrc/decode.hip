// NSA decode: one new query per sequence against a KV cache ("Native Sparse Attention"
// article: decode loads only the compressed, the selected and the window KV, saving HBM
// bandwidth; podcast notes EP94 section 6: one shared selection per GQA group, so one KV read
// serves the group's heads).  Every phase streams HBM; the matrix core does the contractions
// with the group's heads as the 16 MFMA rows.
//
//   dec_cmp_kernel     split-K over the compressed cache: per 256-token chunk, per head,
//                      (max, sum, unnormalised output) and per-block probability mass
//   dec_scores_kernel  per-head log-sum-exp, then group block scores for a slice of blocks
//   dec_select_kernel  top-n with forced block 0 + local blocks (one wave)
//   dec_tiles_kernel   selected blocks and window as one de-duplicated list of 64-token
//                      tiles; each tile is read once and feeds whichever branches use it
//   dec_combine_kernel merges all partials and applies the gate
#include "dev_common.h"
#include "kernels.h"

namespace nsa {

constexpr int CHUNK = 256;  // compressed tokens per dec_cmp workgroup (4 waves x 64)

// Loads this wave's 64-key tile of a [rows, D] bf16 matrix (rows clamped to `last`) into LDS
// transposed, Vt[d][key], four keys per 8-byte store.
template <int D>
__device__ __forceinline__ void stage_vt(u16 (*Vt)[64 + KPAD], const u16* src, int k0, int last,
                                         int lane) {
  constexpr int DC = D / 8;
  for (int it = lane; it < 16 * DC; it += 64) {
    const int kq = it / DC, dc = it % DC;
    uint32_t v[4][4];  // four keys x 8 features, as 32-bit words (2 features each)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int row = k0 + 4 * kq + r;
      row = row < last ? row : last;
      const uint4 w = *reinterpret_cast<const uint4*>(src + (long)row * D + 8 * dc);
      v[r][0] = w.x; v[r][1] = w.y; v[r][2] = w.z; v[r][3] = w.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t h0 = (v[0][e >> 1] >> sh) & 0xFFFFu, h1 = (v[1][e >> 1] >> sh) & 0xFFFFu;
      const uint32_t h2 = (v[2][e >> 1] >> sh) & 0xFFFFu, h3 = (v[3][e >> 1] >> sh) & 0xFFFFu;
      uint2 pk;
      pk.x = h0 | (h1 << 16);
      pk.y = h2 | (h3 << 16);
      *reinterpret_cast<uint2*>(&Vt[8 * dc + e][4 * kq]) = pk;
    }
  }
}

// S^T for a 64-key tile whose K rows are read straight from global memory (16-byte loads);
// z[kc*8 + s*4 + i] belongs to key k0 + 32*kc + 8*g4 + 4*s + i.
template <int D>
__device__ __forceinline__ void tile_scores(const u16* kb, int k0, int last, const bf16x8* qf,
                                            int g4, int r16, f32x4* acc) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      int row = k0 + 32 * kc + perm_key(r16, s);
      row = row < last ? row : last;
      const u16* kp = kb + (long)row * D + 8 * g4;
      f32x4 a = zero4();
#pragma unroll
      for (int c = 0; c < D / 32; ++c) a = mfma16x16x32(load8(kp + 32 * c), qf[c], a);
      acc[kc * 2 + s] = a;
    }
}

template <int D>
__device__ __forceinline__ void load_q_decode(const DecodeArgs& a, int b, int kvh, int lane,
                                              bf16x8* qf) {
  const int g4 = lane >> 4, r16 = lane & 15;
  const bool hlive = r16 < a.G;
  const u16* qp = a.q + ((long)b * a.Hkv * a.G + kvh * a.G + (hlive ? r16 : 0)) * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) qf[c] = hlive ? load8(qp + 32 * c + 8 * g4) : zero8();
}

// ------------------------------------------------------------------ phase 1: compressed stream

template <int D>
__global__ __launch_bounds__(256) void dec_cmp_kernel(DecodeArgs a) {
  __shared__ u16 Vt[4][D][64 + KPAD];
  __shared__ float Pw[4][16][64];
  __shared__ float Wm[4][16], Wl[4][16];
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int t = a.seqlens[b] - 1;
  const int nvis = n_visible(t, a.l, a.d, a.ncmp);
  const int c0 = chunk * CHUNK;
  if (c0 >= nvis) return;  // uniform across the workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const long bkv = (long)b * a.Hkv + kvh;
  const int k0 = c0 + 64 * wave;
  const u16* kcb = a.kc + bkv * a.ncmp * D;
  const u16* vcb = a.vc + bkv * a.ncmp * D;

  bf16x8 qf[D / 32];
  load_q_decode<D>(a, b, kvh, lane, qf);
  f32x4 acc[4];
  tile_scores<D>(kcb, k0, nvis - 1, qf, g4, r16, acc);
  stage_vt<D>(Vt[wave], vcb, k0, nvis - 1, lane);

  float z[16];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = k0 + 32 * (q4 >> 1) + 8 * g4 + 4 * (q4 & 1) + i;
      z[q4 * 4 + i] = key < nvis ? acc[q4][i] * a.scale_log2 : kNegInf;
    }
  float tm = z[0];
#pragma unroll
  for (int e = 1; e < 16; ++e) tm = fmaxf(tm, z[e]);
  tm = col_max4(tm);
  const float ms = tm == kNegInf ? 0.f : tm;
  float p[16], ls = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) { p[e] = fast_exp2(z[e] - ms); ls += p[e]; }
  ls = col_sum4(ls);
  __syncthreads();  // Vt staged by the whole wave

  constexpr int DT = D / 16;
  f32x4 O[DT];
#pragma unroll
  for (int n = 0; n < DT; ++n) O[n] = zero4();
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = (__bf16)p[kc * 8 + e];
#pragma unroll
    for (int n = 0; n < DT; ++n)
      O[n] = mfma16x16x32(load8(&Vt[wave][16 * n + r16][32 * kc + 8 * g4]), pb, O[n]);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) Pw[wave][r16][32 * (e >> 3) + 8 * g4 + (e & 7)] = p[e];
  if (g4 == 0) { Wm[wave][r16] = tm; Wl[wave][r16] = ls; }
  __syncthreads();

  // merge the four tiles: chunk max, rescaled sums and outputs
  float sc[4];
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, Wm[w][r16]);
#pragma unroll
  for (int w = 0; w < 4; ++w) sc[w] = Wm[w][r16] == kNegInf ? 0.f : fast_exp2(Wm[w][r16] - M);
  const long cidx = bkv * a.NCH + chunk;
  // each wave adds its scaled output into LDS (reusing Vt storage as [16][D] fp32)
  float* Ob = reinterpret_cast<float*>(&Vt[0][0][0]);
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * D; e += 256) Ob[e] = 0.f;
  __syncthreads();
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int n = 0; n < DT; ++n)
#pragma unroll
        for (int e = 0; e < 4; ++e) Ob[r16 * D + 16 * n + 4 * g4 + e] += sc[w] * O[n][e];
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < 16 * D; e += 256) a.co[cidx * 16 * D + e] = Ob[e];
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) L += Wl[w][h] * (Wm[w][h] == kNegInf ? 0.f : fast_exp2(Wm[w][h] - M));
    a.cm[cidx * 16 + h] = M;
    a.cl[cidx * 16 + h] = L;
  }
  // per-head block mass (relative to the chunk max) of the blocks this chunk touches
  const int jb0 = (c0 * a.d) / a.beta;
  for (int pr = threadIdx.x; pr < 16 * a.NBC; pr += 256) {
    const int h = pr / a.NBC, j = jb0 + pr % a.NBC;
    float Mh = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mh = fmaxf(Mh, Wm[w][h]);
    const int bs = j * a.beta, be = bs + a.beta;
    int ilo = bs - a.l + 1 <= 0 ? 0 : (bs - a.l + 1 + a.d - 1) / a.d;
    if (ilo < c0) ilo = c0;
    int ihi = (be - 1) / a.d;
    if (ihi > c0 + CHUNK - 1) ihi = c0 + CHUNK - 1;
    if (ihi > nvis - 1) ihi = nvis - 1;
    float sv = 0.f;
    for (int i = ilo; i <= ihi; ++i) {
      const int w = (i - c0) >> 6;
      const float f = Wm[w][h] == kNegInf ? 0.f : fast_exp2(Wm[w][h] - Mh);
      const int s0 = i * a.d, s1 = s0 + a.l;
      const int ov = (s1 < be ? s1 : be) - (s0 > bs ? s0 : bs);
      if (ov > 0) sv += Pw[w][h][(i - c0) & 63] * f * ((float)ov / (float)a.l);
    }
    a.cb[cidx * 16 * a.NBC + pr] = sv;
  }
}

// ------------------------------------------------------------------ phase 2: block scores

__global__ __launch_bounds__(256) void dec_scores_kernel(DecodeArgs a) {
  __shared__ float lse[16];
  const int slice = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const long bkv = (long)b * a.Hkv + kvh;
  const int t = a.seqlens[b] - 1;
  const int nvis = n_visible(t, a.l, a.d, a.ncmp);
  const int nch = (nvis + CHUNK - 1) / CHUNK;
  const int nb = t / a.beta + 1;
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    float M = kNegInf;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, a.cm[(bkv * a.NCH + c) * 16 + h]);
    float L = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float mc = a.cm[(bkv * a.NCH + c) * 16 + h];
      if (mc != kNegInf) L += a.cl[(bkv * a.NCH + c) * 16 + h] * fast_exp2(mc - M);
    }
    const float v = (M == kNegInf) ? __builtin_inff() : M + __log2f(L);
    lse[h] = v;
    if (slice == 0) a.lse[bkv * 16 + h] = v;
  }
  __syncthreads();
  const int per = (nb + gridDim.x - 1) / gridDim.x;
  const int j0 = slice * per, j1 = (j0 + per < nb) ? j0 + per : nb;
  for (int j = j0 + threadIdx.x; j < j1; j += blockDim.x) {
    const int bs = j * a.beta, be = bs + a.beta;
    int ilo = bs - a.l + 1 <= 0 ? 0 : (bs - a.l + 1 + a.d - 1) / a.d;
    int ihi = (be - 1) / a.d;
    if (ihi > nvis - 1) ihi = nvis - 1;
    float S = 0.f;
    if (ilo <= ihi) {
      const int clo = ilo / CHUNK, chi = ihi / CHUNK;
      for (int h = 0; h < a.G; ++h) {
        for (int c = clo; c <= chi; ++c) {
          const long cidx = bkv * a.NCH + c;
          const float mc = a.cm[cidx * 16 + h];
          const int jb0 = (c * CHUNK * a.d) / a.beta;
          if (mc != kNegInf)
            S += a.cb[(cidx * 16 + h) * a.NBC + (j - jb0)] * fast_exp2(mc - lse[h]);
        }
      }
    }
    a.S[bkv * a.nblk + j] = S;
  }
}

// ------------------------------------------------------------------ phase 3: selection

// Top-k of S[first, last) by (score desc, index asc) for non-negative scores.  Every lane keeps
// its four best candidates; the wave repeatedly takes the best head, and a lane that runs out
// rescans below its last popped key.  Lane e < k receives the e-th winner.
__device__ int wave_topk(const float* S, int first, int last, int k, int lane) {
  uint64_t c[4] = {0, 0, 0, 0};
  auto insert = [&](uint64_t key) {
    if (key <= c[3]) return;
    if (key > c[0]) { c[3] = c[2]; c[2] = c[1]; c[1] = c[0]; c[0] = key; }
    else if (key > c[1]) { c[3] = c[2]; c[2] = c[1]; c[1] = key; }
    else if (key > c[2]) { c[3] = c[2]; c[2] = key; }
    else c[3] = key;
  };
  for (int j = first + lane; j < last; j += 64) insert(rank_key(S[j], j));
  int mine = -1;
  for (int it = 0; it < k; ++it) {
    const uint64_t best = wave_max_u64(c[0]);
    if (lane == it) mine = rank_key_index(best);
    if (c[0] == best && best != 0) {
      c[0] = c[1]; c[1] = c[2]; c[2] = c[3]; c[3] = 0;
      if (c[0] == 0) {  // cache exhausted: rescan strictly below the popped key
        for (int j = first + lane; j < last; j += 64) {
          const uint64_t key = rank_key(S[j], j);
          if (key < best) insert(key);
        }
      }
    }
  }
  return mine;
}

__global__ __launch_bounds__(64) void dec_select_kernel(DecodeArgs a) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const long bkv = (long)b * a.Hkv + kvh;
  const int t = a.seqlens[b] - 1;
  const int bcur = t / a.beta, nb = bcur + 1;
  int32_t* orow = a.idx + bkv * a.top_n;
  if (nb <= a.top_n) {
    for (int e = lane; e < a.top_n; e += 64) orow[e] = e < nb ? e : -1;
    return;
  }
  const int flo = bcur - a.n_local + 1;
  const int kfree = a.top_n - 1 - a.n_local;
  int el = wave_topk(a.S + bkv * a.nblk, 1, flo, kfree, lane);
  if (lane == kfree) el = 0;
  if (lane > kfree && lane < a.top_n) el = flo + (lane - kfree - 1);
  int rank = 0;
  for (int o = 0; o < a.top_n; ++o) rank += (__shfl(el, o) < el) ? 1 : 0;
  if (lane < a.top_n) orow[rank] = el;
}

// ------------------------------------------------------------------ phase 4: selected + window

// Tile list of one (sequence, group): selected-block tiles and window tiles, ascending, each
// tile once.  Returns the count; tiles[] gets the tile numbers (64 tokens each).
__device__ int tile_list(const DecodeArgs& a, const int32_t* irow, int t, int* tiles) {
  const int w0 = t - a.window + 1 > 0 ? t - a.window + 1 : 0;
  const int wt0 = w0 / 64, wt1 = t / 64;
  const int per = a.beta / 64;
  int n = 0, wnext = wt0;
  for (int e = 0; e < a.top_n; ++e) {
    const int j = irow[e];
    if (j < 0) break;
    for (int u = 0; u < per; ++u) {
      const int tile = j * per + u;
      if (tile * 64 > t) break;
      while (wnext <= wt1 && wnext < tile) tiles[n++] = wnext++;
      if (wnext == tile) ++wnext;
      tiles[n++] = tile;
    }
  }
  while (wnext <= wt1) tiles[n++] = wnext++;
  return n;
}

template <int D>
__global__ __launch_bounds__(256) void dec_tiles_kernel(DecodeArgs a) {
  __shared__ u16 Vt[4][D][64 + KPAD];
  __shared__ int tiles[160];
  __shared__ int ntiles;
  __shared__ float Wm[2][4][16], Wl[2][4][16];
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const long bkv = (long)b * a.Hkv + kvh;
  const int t = a.seqlens[b] - 1;
  const int32_t* irow = a.idx + bkv * a.top_n;
  if (threadIdx.x == 0) ntiles = tile_list(a, irow, t, tiles);
  __syncthreads();
  const int my = split * 4 + wave;
  const bool have = my < ntiles;
  const int tile = have ? tiles[my] : 0;
  const int k0 = tile * 64;
  // branch membership of this tile
  const int jblk = k0 / a.beta;
  bool in_slc = false;
  for (int e = 0; e < a.top_n; ++e) in_slc |= (irow[e] == jblk);
  const int w0 = t - a.window + 1;
  const bool in_win = have && (k0 + 63 >= w0);
  in_slc = in_slc && have;

  const u16* kb = a.kcache + bkv * (long)a.L * D;
  const u16* vb = a.vcache + bkv * (long)a.L * D;
  bf16x8 qf[D / 32];
  load_q_decode<D>(a, b, kvh, lane, qf);
  f32x4 acc[4];
  tile_scores<D>(kb, k0, t, qf, g4, r16, acc);
  stage_vt<D>(Vt[wave], vb, k0, t, lane);
  __syncthreads();

  constexpr int DT = D / 16;
  f32x4 O[2][DT];
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    float z[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 32 * (q4 >> 1) + 8 * g4 + 4 * (q4 & 1) + i;
        const bool ok = br == 0 ? (in_slc && key <= t) : (in_win && key <= t && key >= w0);
        z[q4 * 4 + i] = ok ? acc[q4][i] * a.scale_log2 : kNegInf;
      }
    float tm = z[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) tm = fmaxf(tm, z[e]);
    tm = col_max4(tm);
    const float ms = tm == kNegInf ? 0.f : tm;
    float p[16], ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) { p[e] = fast_exp2(z[e] - ms); ls += p[e]; }
    ls = col_sum4(ls);
#pragma unroll
    for (int n = 0; n < DT; ++n) O[br][n] = zero4();
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)p[kc * 8 + e];
#pragma unroll
      for (int n = 0; n < DT; ++n)
        O[br][n] = mfma16x16x32(load8(&Vt[wave][16 * n + r16][32 * kc + 8 * g4]), pb, O[br][n]);
    }
    if (g4 == 0) { Wm[br][wave][r16] = tm; Wl[br][wave][r16] = ls; }
  }
  __syncthreads();
  // merge the four waves per branch into one partial of this split
  float* Ob = reinterpret_cast<float*>(&Vt[0][0][0]);  // [2][16][D] fp32
  for (int e = threadIdx.x; e < 2 * 16 * D; e += 256) Ob[e] = 0.f;
  __syncthreads();
  const long sidx = bkv * a.NSPLIT + split;
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int br = 0; br < 2; ++br) {
        float M = kNegInf;
#pragma unroll
        for (int v = 0; v < 4; ++v) M = fmaxf(M, Wm[br][v][r16]);
        const float f = Wm[br][w][r16] == kNegInf ? 0.f : fast_exp2(Wm[br][w][r16] - M);
#pragma unroll
        for (int n = 0; n < DT; ++n)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Ob[(br * 16 + r16) * D + 16 * n + 4 * g4 + e] += f * O[br][n][e];
      }
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < 2 * 16 * D; e += 256) a.po[sidx * 2 * 16 * D + e] = Ob[e];
  if (threadIdx.x < 32) {
    const int br = threadIdx.x >> 4, h = threadIdx.x & 15;
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < 4; ++v) M = fmaxf(M, Wm[br][v][h]);
    float L = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      L += Wm[br][v][h] == kNegInf ? 0.f : Wl[br][v][h] * fast_exp2(Wm[br][v][h] - M);
    a.pm[(sidx * 2 + br) * 16 + h] = M;
    a.pl[(sidx * 2 + br) * 16 + h] = L;
  }
}

// ------------------------------------------------------------------ phase 5: merge + gate

__global__ __launch_bounds__(256) void dec_combine_kernel(DecodeArgs a) {
  const int kvh = blockIdx.y, b = blockIdx.z;
  const long bkv = (long)b * a.Hkv + kvh;
  const int pair = blockIdx.x * 256 + threadIdx.x;
  const int h = pair / a.D, dd = pair % a.D;
  if (h >= a.G) return;
  const int t = a.seqlens[b] - 1;
  const int nvis = n_visible(t, a.l, a.d, a.ncmp);
  const int nch = (nvis + CHUNK - 1) / CHUNK;
  float ocmp = 0.f;
  const float lse = a.lse[bkv * 16 + h];
  for (int c = 0; c < nch; ++c) {
    const long cidx = bkv * a.NCH + c;
    const float mc = a.cm[cidx * 16 + h];
    if (mc != kNegInf) ocmp += a.co[(cidx * 16 + h) * a.D + dd] * fast_exp2(mc - lse);
  }
  float ob[2];
  for (int br = 0; br < 2; ++br) {
    float M = kNegInf;
    for (int s = 0; s < a.NSPLIT; ++s) M = fmaxf(M, a.pm[((bkv * a.NSPLIT + s) * 2 + br) * 16 + h]);
    float L = 0.f, o = 0.f;
    for (int s = 0; s < a.NSPLIT; ++s) {
      const long sidx = bkv * a.NSPLIT + s;
      const float m = a.pm[(sidx * 2 + br) * 16 + h];
      if (m == kNegInf) continue;
      const float f = fast_exp2(m - M);
      L += a.pl[(sidx * 2 + br) * 16 + h] * f;
      o += a.po[((sidx * 2 + br) * 16 + h) * a.D + dd] * f;
    }
    ob[br] = L > 0.f ? o / L : 0.f;
  }
  const int head = kvh * a.G + h;
  const float* g = a.gate + ((long)b * a.Hkv * a.G + head) * 3;
  a.out[((long)b * a.Hkv * a.G + head) * a.D + dd] = g[0] * ocmp + g[1] * ob[0] + g[2] * ob[1];
}

// ------------------------------------------------------------------ launcher

void launch_decode(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  auto mark = [&](int i) {
    if (ev != nullptr) (void)hipEventRecord(ev[i], s);
  };
  const dim3 g1(a.NCH, a.Hkv, a.B);
  mark(0);
  if (a.NCH > 0) {
    if (a.D == 128) dec_cmp_kernel<128><<<g1, 256, 0, s>>>(a);
    else dec_cmp_kernel<64><<<g1, 256, 0, s>>>(a);
  }
  mark(1);
  dec_scores_kernel<<<dim3(a.NSLICE, a.Hkv, a.B), 256, 0, s>>>(a);
  mark(2);
  dec_select_kernel<<<dim3(a.Hkv, a.B), 64, 0, s>>>(a);
  mark(3);
  const dim3 g4(a.NSPLIT, a.Hkv, a.B);
  if (a.D == 128) dec_tiles_kernel<128><<<g4, 256, 0, s>>>(a);
  else dec_tiles_kernel<64><<<g4, 256, 0, s>>>(a);
  mark(4);
  dec_combine_kernel<<<dim3((16 * a.D + 255) / 256, a.Hkv, a.B), 256, 0, s>>>(a);
  mark(5);
}

}  // namespace nsa
