// NSA decode: one new query per sequence against a KV cache ("Native Sparse Attention"
// article: decode loads only the compressed, the selected and the window KV, saving HBM
// bandwidth; podcast notes EP94 section 6: one shared selection per GQA group, so one KV read
// serves the group's heads).  Every phase streams HBM; the matrix core does the contractions
// with the group's heads as the 16 MFMA rows.
//
//   dec_cmp_kernel     split-K over the compressed cache: each wave streams TPW 64-token tiles
//                      with register prefetch and an online softmax; per 1024-token chunk, per
//                      head, (max, sum, unnormalised output); per tile, the probability mass of
//                      every selection block it touches, relative to a per-tile reference
//   dec_select_kernel  per (sequence, group): per-head log-sum-exp, every group block score,
//                      the top-n (forced block 0 + local blocks) and the list of selected and
//                      window tiles, each tile once
//   dec_tiles_kernel   one wave per listed tile: the tile is read once and feeds whichever of
//                      the selected and window branches use it
//   dec_combine_kernel normalises the compressed output, merges all partials, applies the gate
#include "attn_tile.h"
#include "dev_common.h"
#include "kernels.h"

namespace nsa {

constexpr int TPW = 4;               // 64-token tiles per wave in dec_cmp
constexpr int CHUNK = 4 * TPW * 64;  // compressed tokens per dec_cmp workgroup
constexpr int kMaxTiles = 160;       // selected + window tiles per group
constexpr int kMaxSplits = 64;       // splits of that list (8 tiles each)

// One 64-key tile of a [rows, D] K/V cache pair in registers: K in MFMA A-operand order, V in
// the gather order of the transposing LDS store.  Rows past `last` are clamped to it.
template <int D>
struct DecTile {
  static constexpr int NK = D / 8, NV = D / 8, DC = D / 8;
  u32x4 k[NK], v[NV];

  __device__ __forceinline__ void load(const u16* kb, const u16* vb, int k0, int last,
                                       int lane) {
    load_k(kb, k0, last, lane);
    load_v(vb, k0, last, lane);
  }

  __device__ __forceinline__ void load_k(const u16* kb, int k0, int last, int lane) {
    const int g4 = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        int row = k0 + 32 * kc + perm_key(r16, s);
        row = row < last ? row : last;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
          k[(kc * 2 + s) * (D / 32) + c] = *reinterpret_cast<const u32x4*>(
              kb + ((uint32_t)row * D + 8 * g4 + 32 * c));
      }
  }

  __device__ __forceinline__ void load_v(const u16* vb, int k0, int last, int lane) {
#pragma unroll
    for (int it = 0; it < DC / 4; ++it) {
      const int x = it * 64 + lane, kq = x & 15, dc = x >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int row = k0 + 4 * kq + r;
        row = row < last ? row : last;
        v[it * 4 + r] = *reinterpret_cast<const u32x4*>(vb + ((uint32_t)row * D + 8 * dc));
      }
    }
  }

  // S^T = K Q^T; acc[kc*2 + s][i] belongs to key 32*kc + 8*g4 + 4*s + i of the tile.
  __device__ __forceinline__ void scores(const bf16x8* qf, f32x4* acc) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 a = zero4();
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        a = mfma16x16x32(__builtin_bit_cast(bf16x8, k[q * (D / 32) + c]), qf[c], a);
      acc[q] = a;
    }
  }

  // V^T into LDS, Vt[d][key], in the V-tile swizzle of attn_tile.h (8-key chunk c of feature
  // row d at chunk c ^ (d & 7)), four keys per 8-byte store.  The 16 lanes of a row hold 16
  // key quads of one feature octet, so each store instruction covers whole LDS rows.
  __device__ __forceinline__ void stage(u16 (*Vt)[64], int lane) const {
#pragma unroll
    for (int it = 0; it < DC / 4; ++it) {
      const int x = it * 64 + lane, kq = x & 15, dc = x >> 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16, d = 8 * dc + e;
        const uint32_t h0 = (v[it * 4 + 0][e >> 1] >> sh) & 0xFFFFu;
        const uint32_t h1 = (v[it * 4 + 1][e >> 1] >> sh) & 0xFFFFu;
        const uint32_t h2 = (v[it * 4 + 2][e >> 1] >> sh) & 0xFFFFu;
        const uint32_t h3 = (v[it * 4 + 3][e >> 1] >> sh) & 0xFFFFu;
        uint2 pk;
        pk.x = h0 | (h1 << 16);
        pk.y = h2 | (h3 << 16);
        *reinterpret_cast<uint2*>(&Vt[d][(((kq >> 1) ^ (d & 7)) * 8) + (kq & 1) * 4]) = pk;
      }
    }
  }
};

// One 64-token tile of the compressed caches in registers: K rows in MFMA A-operand order
// (rows past `last` clamp to it) and V^T fragments read straight from the tiled feature-major
// value cache (one contiguous [D][64] block per tile) as the A operand of O^T += V^T P^T, so no
// LDS staging is needed.
template <int D>
struct CmpTile {
  static constexpr int DT = D / 16;
  u32x4 k[D / 8], vt[2 * DT];

  __device__ __forceinline__ void load_k(const u16* kb, int k0, int last, int lane) {
    const int g4 = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        int row = k0 + 32 * kc + perm_key(r16, s);
        row = row < last ? row : last;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
          k[(kc * 2 + s) * (D / 32) + c] = *reinterpret_cast<const u32x4*>(
              kb + ((uint32_t)row * D + 8 * g4 + 32 * c));
      }
  }

  // Lane (g4, r16) of fragment (kc, n) holds V^T[16n + r16][k0 + 32kc + 8g4 .. + 7].  `k0`
  // clamps to `last0`, the last visible tile, so a prefetch past the end stays in bounds.
  __device__ __forceinline__ void load_vt(const u16* vtb, int k0, int last0, int lane) {
    const int g4 = lane >> 4, r16 = lane & 15;
    k0 = k0 < last0 ? k0 : last0;
    const u16* tb = vtb + (uint32_t)k0 * D;  // tile k0 / 64 starts at (k0 / 64) * D * 64
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int n = 0; n < DT; ++n)
        vt[kc * DT + n] = *reinterpret_cast<const u32x4*>(
            tb + ((16 * n + r16) * 64 + 32 * kc + 8 * g4));
  }

  // Zero the V^T columns from `nvis` on: the cache past the visible tokens is arbitrary, and a
  // zero probability times a NaN is still NaN.
  __device__ __forceinline__ void mask_tail(int k0, int nvis, int lane) {
    const int g4 = lane >> 4;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int lim = nvis - (k0 + 32 * kc + 8 * g4);  // valid columns among this lane's 8
      uint32_t m[4];
#pragma unroll
      for (int w = 0; w < 4; ++w)
        m[w] = (2 * w < lim ? 0xFFFFu : 0u) | (2 * w + 1 < lim ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int n = 0; n < DT; ++n)
#pragma unroll
        for (int w = 0; w < 4; ++w) vt[kc * DT + n][w] &= m[w];
    }
  }

  // S^T = K Q^T; acc[kc*2 + s][i] belongs to key 32*kc + 8*g4 + 4*s + i of the tile.
  __device__ __forceinline__ void scores(const bf16x8* qf, f32x4* acc) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 a = zero4();
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        a = mfma16x16x32(__builtin_bit_cast(bf16x8, k[q * (D / 32) + c]), qf[c], a);
      acc[q] = a;
    }
  }

  // O^T += V^T P^T; p[kc*8 + e] is the probability of key 32kc + 8g4 + e.
  __device__ __forceinline__ void pv(const float* p, f32x4* O) const {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)p[kc * 8 + e];
#pragma unroll
      for (int n = 0; n < DT; ++n)
        O[n] = mfma16x16x32(__builtin_bit_cast(bf16x8, vt[kc * DT + n]), pb, O[n]);
    }
  }
};

template <int D>
__device__ __forceinline__ void load_q_decode(const DecodeArgs& a, int b, int kvh, int lane,
                                              bf16x8* qf) {
  const int g4 = lane >> 4, r16 = lane & 15;
  const bool hlive = r16 < a.G;
  const u16* qp = a.q + ((long)b * a.Hkv * a.G + kvh * a.G + (hlive ? r16 : 0)) * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) qf[c] = hlive ? load8(qp + 32 * c + 8 * g4) : zero8();
}

// Key (tile-relative) of this lane's score e = 4*q4 + i.
__device__ __forceinline__ int lane_key(int q4, int i, int g4) {
  return 32 * (q4 >> 1) + 8 * g4 + 4 * (q4 & 1) + i;
}

// O^T += V^T P^T over one 64-key tile staged in Vt (16 probabilities per lane).
template <int D>
__device__ __forceinline__ void tile_pv(const u16 (*Vt)[64], const float* p, int g4, int r16,
                                        f32x4* O) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = (__bf16)p[kc * 8 + e];
    pv_chunk<D>(Vt, pb, kc, g4, r16, O);
  }
}

// First and last compressed token whose span [i*d, i*d + l) overlaps block j.
__device__ __forceinline__ int block_tok_lo(int j, int beta, int l, int d) {
  const int x = j * beta - l + 1;
  return x <= 0 ? 0 : (x + d - 1) / d;
}
__device__ __forceinline__ int block_tok_hi(int j, int beta, int d) {
  return ((j + 1) * beta - 1) / d;
}

// ------------------------------------------------------------------ phase 1: compressed stream

// FAST: sel_block = 4 * stride and cmp_len = 2 * stride, where block j receives
// p(4j-1)/2 + p(4j) + p(4j+1) + p(4j+2) + p(4j+3)/2: the lane holding keys 4jl..4jl+3 of a
// tile forms the block's core, and the half-token carries cross lanes by shuffles.
template <int D, bool FAST>
__global__ __launch_bounds__(256, FAST ? 2 : 1) void dec_cmp_kernel(DecodeArgs a) {
  constexpr int DT = D / 16, OP = D + 4;
  __shared__ __align__(16) float Ob[4 * 16 * OP];
  __shared__ float Wm[4][16], Wl[4][16];
  __shared__ float Pw[FAST ? 1 : 4][FAST ? 1 : 16][64];
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int t = a.seqlens[b] - 1;
  const int nvis = n_visible(t, a.l, a.d, a.ncmp);
  const int c0 = chunk * CHUNK;
  const long bkv = (long)b * a.Hkv + kvh;
  if (c0 >= nvis) return;  // uniform across the workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const u16* kcb = a.kc + bkv * a.ncmp * D;
  const u16* vtb = a.vct + bkv * (long)a.NT * D * 64;
  const int last0 = (nvis - 1) & ~63;  // first key of the last visible tile
  const float sl = a.scale_log2;

  bf16x8 qf[D / 32];
  load_q_decode<D>(a, b, kvh, lane, qf);
  float m_run = kNegInf, l_run = 0.f;
  f32x4 O[DT];
#pragma unroll
  for (int n = 0; n < DT; ++n) O[n] = zero4();

  // wave w takes tiles c0/64 + w, + 4, + 8, ... (the four waves read adjacent tiles together)
  const int tile0 = (c0 >> 6) + wave;
  CmpTile<D> cur;
  if (tile0 * 64 < nvis) {
    cur.load_k(kcb, tile0 * 64, nvis - 1, lane);
    cur.load_vt(vtb, tile0 * 64, last0, lane);
  }
#pragma unroll
  for (int it = 0; it < TPW; ++it) {
    const int tile = tile0 + 4 * it;
    const int k0 = tile * 64;
    if (k0 >= nvis) break;  // wave-uniform
    f32x4 acc[4];
    cur.scores(qf, acc);
    // the loop is unrolled, so this condition is resolved at compile time: a load under a
    // run-time branch would make the join wait for every load in flight (rows past the last
    // visible one clamp to it)
    if (it + 1 < TPW) cur.load_k(kcb, k0 + 256, nvis - 1, lane);

    float p[16];
    float tm = kNegInf;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = k0 + lane_key(q4, i, g4) < nvis ? acc[q4][i] : kNegInf;
        p[q4 * 4 + i] = r;
        tm = fmaxf(tm, r);
      }
    tm = col_max4(tm);
    const float m_new = fmaxf(m_run, tm);  // finite: the tile holds a visible key
    const float ms = m_new * sl;
    const float alpha = fast_exp2(fmaf(m_run, sl, -ms));
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = fast_exp2(fmaf(p[e], sl, -ms));
      ls += p[e];
    }
    ls = col_sum4(ls);
    l_run = fmaf(l_run, alpha, ls);
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < DT; ++n) O[n] *= alpha;
    if (k0 + 64 > nvis) cur.mask_tail(k0, nvis, lane);  // wave-uniform; no load inside
    cur.pv(p, O);
    if (it + 1 < TPW) cur.load_vt(vtb, k0 + 256, last0, lane);

    // block masses of this tile, relative to exp2(ms)
    const long tix = bkv * a.NT + tile;
    if (g4 == 0) a.tref[tix * 16 + r16] = ms;
    float* cbt = a.cb + tix * a.NBT * 16;
    if constexpr (FAST) {
      float core[2][2], cout[2][2];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const float* q = p + 8 * kc + 4 * s;
          core[kc][s] = (q[0] + q[1]) + q[2] + 0.5f * q[3];
          cout[kc][s] = 0.5f * q[3];
        }
      // lane (g4, kc, s) holds block 8kc + 2g4 + s; its carry-in comes from block - 1
      const int src = (lane + 48) & 63;
      const float y = __shfl(cout[0][1], src), z = __shfl(cout[1][1], src);
      cbt[(2 * g4) * 16 + r16] = core[0][0] + (g4 > 0 ? y : 0.f);
      cbt[(2 * g4 + 1) * 16 + r16] = core[0][1] + cout[0][0];
      cbt[(8 + 2 * g4) * 16 + r16] = core[1][0] + (g4 > 0 ? z : y);
      cbt[(9 + 2 * g4) * 16 + r16] = core[1][1] + cout[1][0];
      if (g4 == 3) cbt[16 * 16 + r16] = cout[1][1];  // into the next tile's first block
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) Pw[wave][r16][32 * (e >> 3) + 8 * g4 + (e & 7)] = p[e];
      __asm__ volatile("" ::: "memory");
      const int jb0 = (k0 * a.d) / a.beta;
      for (int pr = lane; pr < 16 * a.NBT; pr += 64) {
        const int h = pr & 15, jj = pr >> 4;
        const int j = jb0 + jj;
        const int bs = j * a.beta, be = bs + a.beta;
        int ilo = block_tok_lo(j, a.beta, a.l, a.d), ihi = block_tok_hi(j, a.beta, a.d);
        ilo = ilo > k0 ? ilo : k0;
        ihi = ihi < k0 + 63 ? ihi : k0 + 63;
        ihi = ihi < nvis - 1 ? ihi : nvis - 1;
        float sv = 0.f;
        for (int i = ilo; i <= ihi; ++i) {
          const int s0 = i * a.d, s1 = s0 + a.l;
          const int ov = (s1 < be ? s1 : be) - (s0 > bs ? s0 : bs);
          sv += Pw[wave][h][i - k0] * ((float)ov / (float)a.l);
        }
        cbt[pr] = sv;
      }
      __asm__ volatile("" ::: "memory");  // Pw reads stay before the next tile's writes
    }
  }

  // merge the four waves: outputs rescaled to the chunk max, summed through LDS
  if (g4 == 0) { Wm[wave][r16] = m_run; Wl[wave][r16] = l_run; }
  __syncthreads();  // statistics posted
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, Wm[w][r16]);
  const float sc = fast_exp2((Wm[wave][r16] - M) * sl);
#pragma unroll
  for (int n = 0; n < DT; ++n)
    *reinterpret_cast<f32x4*>(&Ob[(wave * 16 + r16) * OP + 16 * n + 4 * g4]) = sc * O[n];
  __syncthreads();
  const long cidx = bkv * a.NCH + chunk;
  for (int e = threadIdx.x; e < 16 * D; e += 256) {
    const int o = (e / D) * OP + e % D;
    a.co[cidx * 16 * D + e] = (Ob[o] + Ob[16 * OP + o]) + (Ob[32 * OP + o] + Ob[48 * OP + o]);
  }
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    float Mh = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mh = fmaxf(Mh, Wm[w][h]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) L += Wl[w][h] * fast_exp2((Wm[w][h] - Mh) * sl);
    a.cm[cidx * 16 + h] = Mh * sl;
    a.cl[cidx * 16 + h] = L;
  }
}

// ------------------------------------------------------------------ phase 2: scores + selection

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

// Masses and tile references of block j for heads 4*hq .. 4*hq + 3 over the (at most) first
// two tiles it touches.  Every index is clamped so the loads are unconditional (no branch
// around them); `ntile` is the number of tiles the block really touches (0 when none of its
// compressed tokens is visible).
struct BlockMass {
  f32x4 m0, r0, m1, r1;
  int ta, ntile;
};

__device__ __forceinline__ BlockMass fetch_block(const DecodeArgs& a, long bkv, int j, int nvis,
                                                 int hq) {
  const int lo = block_tok_lo(j, a.beta, a.l, a.d);
  int hi = block_tok_hi(j, a.beta, a.d);
  hi = hi < nvis - 1 ? hi : nvis - 1;
  const int ta = (lo < nvis - 1 ? lo : nvis - 1) / 64;
  const int tb = hi / 64 > ta ? ta + 1 : ta;
  auto entry = [&](int T) {
    int jj = j - (T * 64 * a.d) / a.beta;
    jj = jj < 0 ? 0 : (jj < a.NBT ? jj : a.NBT - 1);
    return ((bkv * a.NT + T) * a.NBT + jj) * 16 + 4 * hq;
  };
  BlockMass r;
  r.m0 = *reinterpret_cast<const f32x4*>(a.cb + entry(ta));
  r.r0 = *reinterpret_cast<const f32x4*>(a.tref + (bkv * a.NT + ta) * 16 + 4 * hq);
  r.m1 = *reinterpret_cast<const f32x4*>(a.cb + entry(tb));
  r.r1 = *reinterpret_cast<const f32x4*>(a.tref + (bkv * a.NT + tb) * 16 + 4 * hq);
  r.ta = ta;
  r.ntile = lo <= hi ? hi / 64 - lo / 64 + 1 : 0;
  return r;
}

// Group score share of one tile: masses times exp2(tref - lse), the per-head normalisation of
// the compressed softmax.
__device__ __forceinline__ float mass_score(const f32x4& m, const f32x4& r, const float* wl) {
  return (m[0] * fast_exp2(r[0] - wl[0]) + m[1] * fast_exp2(r[1] - wl[1])) +
         (m[2] * fast_exp2(r[2] - wl[2]) + m[3] * fast_exp2(r[3] - wl[3]));
}

constexpr int kSelThreads = 1024;
constexpr int kSelLanes = kSelThreads / 4;  // blocks per pass (four lanes per block)
constexpr int kSelUnroll = 4;              // passes whose loads are in flight together

// One workgroup per (sequence, group): per-head log-sum-exp of the compressed softmax, every
// group block score (four lanes per block, four heads each), the top-n with forced block 0 +
// local blocks, and the group's tile list: tl[e] = tile | (1 << 30) for a tile of a selected
// block, then the window tiles outside the selected blocks.
__global__ __launch_bounds__(kSelThreads) void dec_select_kernel(DecodeArgs a) {
  extern __shared__ float sh[];  // cm[NCH * 16] | cl[NCH * 16] | S[nblk]
  __shared__ float lse[16];
  __shared__ int sidx[64];
  const int kvh = blockIdx.x, b = blockIdx.y;
  const long bkv = (long)b * a.Hkv + kvh;
  const int t = a.seqlens[b] - 1;
  const int nb = t / a.beta + 1;
  const int nvis = n_visible(t, a.l, a.d, a.ncmp);
  const int nch = (nvis + CHUNK - 1) / CHUNK;
  const bool all = nb <= a.top_n;            // uniform: every block is selected
  const bool scored = !all && nvis > 0;      // uniform
  const int hq = threadIdx.x & 3, jq = threadIdx.x >> 2;
  float* scm = sh;
  float* scl = sh + a.NCH * 16;
  float* Ss = sh + 2 * a.NCH * 16;

  // Chunk statistics first, then the first pass of block masses: the wait for the former
  // (vmcnt retires in order) leaves the latter in flight while the lse is formed.  The loads
  // are unconditional, every index clamped into the workspace (which is never empty); values
  // of a missing chunk or tile are never used.
  const bool many = nch * 16 > kSelThreads;  // uniform: beyond 64 chunks, a plain loop
  if (many)
    for (int e = threadIdx.x; e < nch * 16; e += kSelThreads) {
      scm[e] = a.cm[bkv * a.NCH * 16 + e];
      scl[e] = a.cl[bkv * a.NCH * 16 + e];
    }
  const int ce = threadIdx.x < nch * 16 ? threadIdx.x : 0;
  const float cmv = a.cm[bkv * a.NCH * 16 + ce], clv = a.cl[bkv * a.NCH * 16 + ce];
  BlockMass bm[kSelUnroll];
#pragma unroll
  for (int u = 0; u < kSelUnroll; ++u) {
    const int j = jq + kSelLanes * u;
    bm[u] = fetch_block(a, bkv, j < nb ? j : nb - 1, nvis, hq);
  }
  if (!many && threadIdx.x < nch * 16) {
    scm[threadIdx.x] = cmv;
    scl[threadIdx.x] = clv;
  }
  lds_barrier();
  if (threadIdx.x < 256) {  // 16 lanes per head
    const int h = threadIdx.x >> 4, sub = threadIdx.x & 15;
    float M = kNegInf;
    for (int c = sub; c < nch; c += 16) M = fmaxf(M, scm[c * 16 + h]);
    M = group_max<16>(M);
    float L = 0.f;
    for (int c = sub; c < nch; c += 16) L += scl[c * 16 + h] * fast_exp2(scm[c * 16 + h] - M);
    L = group_sum<16>(L);
    if (sub == 0) {
      // heads past G get +inf: their weights vanish
      const float v = (M == kNegInf || h >= a.G) ? __builtin_inff() : M + __log2f(L);
      lse[h] = v;
      a.lse[bkv * 16 + h] = v;
    }
  }
  lds_barrier();
  if (scored) {
    float wl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) wl[k] = lse[4 * hq + k];
    for (int j0 = jq;; j0 += kSelLanes * kSelUnroll) {
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u) {
        const int j = j0 + kSelLanes * u;
        float S = 0.f;
        if (bm[u].ntile >= 1) S = mass_score(bm[u].m0, bm[u].r0, wl);
        if (bm[u].ntile >= 2) S += mass_score(bm[u].m1, bm[u].r1, wl);
        for (int T = bm[u].ta + 2; T < bm[u].ta + bm[u].ntile; ++T) {  // wide blocks only
          const int jj = j - (T * 64 * a.d) / a.beta;
          const f32x4 m = *reinterpret_cast<const f32x4*>(
              a.cb + ((bkv * a.NT + T) * a.NBT + jj) * 16 + 4 * hq);
          const f32x4 r =
              *reinterpret_cast<const f32x4*>(a.tref + (bkv * a.NT + T) * 16 + 4 * hq);
          S += mass_score(m, r, wl);
        }
        S = group_sum<4>(S);
        if (hq == 0 && j < nb) Ss[j] = S;
      }
      const int jn = j0 + kSelLanes * kSelUnroll;
      if (jn - jq >= nb) break;  // uniform
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u) {
        const int j = jn + kSelLanes * u;
        bm[u] = fetch_block(a, bkv, j < nb ? j : nb - 1, nvis, hq);
      }
    }
  } else if (!all) {
    for (int j = threadIdx.x; j < nb; j += kSelThreads) Ss[j] = 0.f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int bcur = nb - 1;
  const int flo = bcur - a.n_local + 1;
  const int kfree = a.top_n - 1 - a.n_local;
  if (threadIdx.x < 64) {
    int32_t* orow = a.idx + bkv * a.top_n;
    if (all) {
      if (lane < a.top_n) {
        const int el = lane < nb ? lane : -1;
        orow[lane] = el;
        sidx[lane] = el;
      }
    } else {
      int el = wave_topk(Ss, 1, flo, kfree, lane);
      if (lane == kfree) el = 0;
      if (lane > kfree && lane < a.top_n) el = flo + (lane - kfree - 1);
      int rank = 0;
      for (int o = 0; o < a.top_n; ++o)  // the whole wave is active here
        rank += (__builtin_amdgcn_readlane(el, o) < el) ? 1 : 0;
      if (lane < a.top_n) {
        orow[rank] = el;
        sidx[rank] = el;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int per = a.beta / 64;
    const int w0 = t - a.window + 1 > 0 ? t - a.window + 1 : 0;
    const int wt0 = w0 / 64, wt1 = t / 64;
    const int nsel = a.top_n * per, ncand = nsel + (wt1 - wt0 + 1);
    int base = 0;
    for (int i0 = 0; i0 < ncand; i0 += 64) {
      const int i = i0 + lane;
      int code = -1;
      if (i < nsel) {
        const int jb = sidx[i / per], tile = jb * per + i % per;
        if (jb >= 0 && tile * 64 <= t) code = tile | (1 << 30);
      } else if (i < ncand) {
        const int tile = wt0 + (i - nsel), jw = tile / per;
        bool in = false;
        for (int e = 0; e < a.top_n; ++e) in |= sidx[e] == jw;
        if (!in) code = tile;
      }
      const uint64_t m = __ballot(code >= 0);
      const int pos = base + (int)__popcll(m & ((1ull << lane) - 1ull));
      if (code >= 0) a.tl[bkv * kMaxTiles + pos] = code;
      base += (int)__popcll(m);
    }
    if (lane == 0) a.tn[bkv] = base;
  }
}

// ------------------------------------------------------------------ phase 3: selected + window

// Two listed tiles per wave (the second in flight while the first computes), eight per
// workgroup, merged into one partial per branch; the first four tiles of a split go to the four
// waves, then the next four.
constexpr int kTilesPerWave = 2;

template <int D>
__global__ __launch_bounds__(256, 2) void dec_tiles_kernel(DecodeArgs a) {
  constexpr int DT = D / 16, OP = D + 4;
  constexpr int VT_U16 = 4 * D * 64, OB_U16 = 4 * 2 * 16 * OP * 2;
  __shared__ __align__(16) u16 smem[VT_U16 > OB_U16 ? VT_U16 : OB_U16];
  __shared__ float Wm[2][4][16], Wl[2][4][16];
  u16(*Vt)[D][64] = reinterpret_cast<u16(*)[D][64]>(smem);
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const long bkv = (long)b * a.Hkv + kvh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tn = a.tn[bkv];
  int code_raw[kTilesPerWave];
#pragma unroll
  for (int u = 0; u < kTilesPerWave; ++u) {
    const int my = split * 4 * kTilesPerWave + 4 * u + wave;
    code_raw[u] = a.tl[bkv * kMaxTiles + (my < kMaxTiles ? my : 0)];
  }
  if (split * 4 * kTilesPerWave >= tn) return;  // uniform
  const int g4 = lane >> 4, r16 = lane & 15;
  const int t = a.seqlens[b] - 1;
  const float sl = a.scale_log2;
  const int w0 = t - a.window + 1;
  const u16* kcb = a.kcache + bkv * (long)a.L * D;
  const u16* vcb = a.vcache + bkv * (long)a.L * D;

  bf16x8 qf[D / 32];
  load_q_decode<D>(a, b, kvh, lane, qf);
  float mrun[2] = {kNegInf, kNegInf}, lrun[2] = {0.f, 0.f};
  f32x4 O[2][DT];
#pragma unroll
  for (int br = 0; br < 2; ++br)
#pragma unroll
    for (int n = 0; n < DT; ++n) O[br][n] = zero4();

  auto tile_of = [&](int u, bool* have, bool* in_slc, bool* in_win) {
    const int my = split * 4 * kTilesPerWave + 4 * u + wave;
    *have = my < tn;
    const int code = *have ? code_raw[u] : 0;
    const int k0 = (code & 0x3FFFFFFF) * 64;
    *in_slc = *have && ((code >> 30) & 1);
    *in_win = *have && (k0 + 63 >= w0);
    return k0;
  };
  DecTile<D> kv;
  bool have0, slc0, win0;
  int k0 = tile_of(0, &have0, &slc0, &win0);
  kv.load(kcb, vcb, k0, t, lane);
#pragma unroll
  for (int u = 0; u < kTilesPerWave; ++u) {
    bool have, in_slc, in_win;
    k0 = tile_of(u, &have, &in_slc, &in_win);
    f32x4 acc[4];
    kv.scores(qf, acc);
    __asm__ volatile("" ::: "memory");  // the previous tile's Vt reads stay before these writes
    kv.stage(Vt[wave], lane);
    __asm__ volatile("" ::: "memory");  // Vt[wave] is this wave's own: LDS keeps its order
    bool h1, s1, w1;
    const int k1 = u + 1 < kTilesPerWave ? tile_of(u + 1, &h1, &s1, &w1) : 0;
    // the next tile's K is in flight during this tile's softmax and P V, its V after them
    // (compile-time conditions: the loop is unrolled)
    if (u + 1 < kTilesPerWave) kv.load_k(kcb, k1, t, lane);
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      float p[16];
      float tm = kNegInf;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + lane_key(q4, i, g4);
          const bool ok = br == 0 ? (in_slc && key <= t) : (in_win && key <= t && key >= w0);
          const float r = ok ? acc[q4][i] : kNegInf;
          p[q4 * 4 + i] = r;
          tm = fmaxf(tm, r);
        }
      tm = col_max4(tm);
      const float mn = fmaxf(mrun[br], tm);
      const float ms = mn == kNegInf ? 0.f : mn * sl;
      const float alpha = fast_exp2(fmaf(mrun[br], sl, -ms));
      mrun[br] = mn;
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = fast_exp2(fmaf(p[e], sl, -ms));
        ls += p[e];
      }
      lrun[br] = fmaf(lrun[br], alpha, col_sum4(ls));
#pragma unroll
      for (int n = 0; n < DT; ++n) O[br][n] *= alpha;
      tile_pv<D>(Vt[wave], p, g4, r16, O[br]);
    }
    if (u + 1 < kTilesPerWave) kv.load_v(vcb, k1, t, lane);
  }
  if (g4 == 0) {
#pragma unroll
    for (int br = 0; br < 2; ++br) { Wm[br][wave][r16] = mrun[br]; Wl[br][wave][r16] = lrun[br]; }
  }
  __syncthreads();  // Vt reads done; maxima posted
  // merge the four waves per branch into this split's partial, summed through LDS
  float* Ob = reinterpret_cast<float*>(smem);  // [4][2][16][OP] fp32
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, Wm[br][w][r16]);
    const float f =
        Wm[br][wave][r16] == kNegInf ? 0.f : fast_exp2((Wm[br][wave][r16] - M) * sl);
#pragma unroll
    for (int n = 0; n < DT; ++n)
      *reinterpret_cast<f32x4*>(&Ob[((wave * 2 + br) * 16 + r16) * OP + 16 * n + 4 * g4]) =
          f * O[br][n];
  }
  __syncthreads();
  const long sidx = bkv * a.NSPLIT + split;
  for (int e = threadIdx.x; e < 2 * 16 * D; e += 256) {
    const int br = e / (16 * D), rest = e % (16 * D);
    const int o = (br * 16 + rest / D) * OP + rest % D;
    a.po[sidx * 2 * 16 * D + e] =
        (Ob[o] + Ob[2 * 16 * OP + o]) + (Ob[4 * 16 * OP + o] + Ob[6 * 16 * OP + o]);
  }
  if (threadIdx.x < 32) {
    const int br = threadIdx.x >> 4, h = threadIdx.x & 15;
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < 4; ++v) M = fmaxf(M, Wm[br][v][h]);
    float L = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (Wm[br][v][h] != kNegInf) L += Wl[br][v][h] * fast_exp2((Wm[br][v][h] - M) * sl);
    a.pm[(sidx * 2 + br) * 16 + h] = M == kNegInf ? kNegInf : M * sl;
    a.pl[(sidx * 2 + br) * 16 + h] = L;
  }
}

// ------------------------------------------------------------------ phase 4: merge + gate

// 256 (head, feature) outputs of one (sequence, group) per workgroup: the compressed output
// normalised by the lse, the selected and window partials merged, then the gate.
__global__ __launch_bounds__(256) void dec_combine_kernel(DecodeArgs a) {
  extern __shared__ float wc[];  // [nch][16] chunk weights exp2(cm - lse)
  __shared__ float pm[2][kMaxSplits][16], pl[2][kMaxSplits][16];
  const int kvh = blockIdx.y, b = blockIdx.z;
  const long bkv = (long)b * a.Hkv + kvh;
  const int t = a.seqlens[b] - 1;
  const int nvis = n_visible(t, a.l, a.d, a.ncmp);
  const int nch = (nvis + CHUNK - 1) / CHUNK;
  const int nsp = (a.tn[bkv] + 4 * kTilesPerWave - 1) / (4 * kTilesPerWave);
  for (int e = threadIdx.x; e < nsp * 32; e += 256) {
    const int s = e >> 5, br = (e >> 4) & 1, h = e & 15;
    pm[br][s][h] = a.pm[(bkv * a.NSPLIT + s) * 32 + (e & 31)];
    pl[br][s][h] = a.pl[(bkv * a.NSPLIT + s) * 32 + (e & 31)];
  }
  for (int e = threadIdx.x; e < nch * 16; e += 256)
    wc[e] = fast_exp2(a.cm[bkv * a.NCH * 16 + e] - a.lse[bkv * 16 + (e & 15)]);
  __syncthreads();
  const int pair = blockIdx.x * 256 + threadIdx.x;
  const int h = pair / a.D, dd = pair % a.D;
  if (h >= a.G) return;
  float ocmp = 0.f;
  const float* cop = a.co + bkv * a.NCH * 16 * a.D + pair;
#pragma unroll 4
  for (int c = 0; c < nch; ++c) ocmp += cop[(long)c * 16 * a.D] * wc[c * 16 + h];
  float ob[2];
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    float M = kNegInf;
    for (int s = 0; s < nsp; ++s) M = fmaxf(M, pm[br][s][h]);
    float L = 0.f, o = 0.f;
#pragma unroll 4
    for (int s = 0; s < nsp; ++s) {
      const float m = pm[br][s][h];
      const float f = m == kNegInf ? 0.f : fast_exp2(m - M);
      L += pl[br][s][h] * f;
      o += a.po[((bkv * a.NSPLIT + s) * 2 + br) * 16 * a.D + pair] * f;
    }
    ob[br] = L > 0.f ? o / L : 0.f;
  }
  const int head = kvh * a.G + h;
  const float* g = a.gate + ((long)b * a.Hkv * a.G + head) * 3;
  a.out[((long)b * a.Hkv * a.G + head) * a.D + dd] = g[0] * ocmp + g[1] * ob[0] + g[2] * ob[1];
}

// ------------------------------------------------------------------ launcher

int decode_chunk_tokens() { return CHUNK; }
int decode_max_splits() { return kMaxSplits; }
int decode_tiles_per_split() { return 4 * kTilesPerWave; }
int decode_max_tile_list() { return kMaxTiles; }
size_t decode_select_lds_bytes(int nch, int nblk) {
  return (size_t)(2 * nch * 16 + nblk) * sizeof(float);
}

void launch_decode(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  auto mark = [&](int i) {
    if (ev != nullptr) (void)hipEventRecord(ev[i], s);
  };
  const bool fast = a.beta == 4 * a.d && a.l == 2 * a.d && a.NBT >= 17;
  const size_t sel_lds = decode_select_lds_bytes(a.NCH, a.nblk);
  if (sel_lds > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dec_select_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sel_lds);
  mark(0);
  if (a.NCH > 0) {
    const dim3 g1(a.NCH, a.Hkv, a.B);
    if (a.D == 128) {
      if (fast) dec_cmp_kernel<128, true><<<g1, 256, 0, s>>>(a);
      else dec_cmp_kernel<128, false><<<g1, 256, 0, s>>>(a);
    } else {
      if (fast) dec_cmp_kernel<64, true><<<g1, 256, 0, s>>>(a);
      else dec_cmp_kernel<64, false><<<g1, 256, 0, s>>>(a);
    }
  }
  mark(1);
  dec_select_kernel<<<dim3(a.Hkv, a.B), kSelThreads, sel_lds, s>>>(a);
  mark(2);
  const dim3 g3(a.NSPLIT, a.Hkv, a.B);
  if (a.D == 128) dec_tiles_kernel<128><<<g3, 256, 0, s>>>(a);
  else dec_tiles_kernel<64><<<g3, 256, 0, s>>>(a);
  mark(3);
  dec_combine_kernel<<<dim3((16 * a.D + 255) / 256, a.Hkv, a.B), 256,
                       (size_t)a.NCH * 16 * sizeof(float), s>>>(a);
  mark(4);
}

}  // namespace nsa
