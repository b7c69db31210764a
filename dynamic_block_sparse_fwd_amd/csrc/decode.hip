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
//   dec_group_kernel   one workgroup per (sequence, group): per-head log-sum-exp, every group
//                      block score, the top-n (forced block 0 + local blocks), the list of
//                      selected and window tiles (each tile read once, feeding whichever branch
//                      uses it), the merge of all partials and the gate
#include "attn_tile.h"
#include "dev_common.h"
#include "kernels.h"

namespace nsa {

constexpr int TPW = 4;               // 64-token tiles per wave in dec_cmp
constexpr int CHUNK = 4 * TPW * 64;  // compressed tokens per dec_cmp workgroup
constexpr int kMaxTiles = 160;       // selected + window tiles per group

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

// ------------------------------------------------------------------ phase 2: one workgroup per group

// Masses of block j for heads 4*hq .. 4*hq + 3.  Every index is clamped so the loads are
// unconditional (no branch around them).
//  generic: the (at most) first two tiles the block touches, from tile ta; `ntile` is the
//    number of tiles it really touches (0 when none of its compressed tokens is visible);
//  FAST (sel_block = 4 * stride, cmp_len = 2 * stride): block j spans compressed tokens
//    4j - 1 .. 4j + 3, all in tile T = j / 16 except for j = 16 T, whose half-weight first token
//    is the previous tile's carry slot 16.  m0 = tile T's slot j - 16 T, m1 = tile T - 1's carry:
//    the 16 blocks of one wave instruction share that address, so it costs one 64-byte request.
struct BlockMass {
  f32x4 m0, m1;
  int ta, tb, ntile;  // generic: first tile, -, tiles touched; FAST: tile of m0, tile of m1,
                      // (m0 used) | 2 (m1 used)
};

template <bool FAST>
__device__ __forceinline__ BlockMass fetch_block(const DecodeArgs& a, long bkv, int j, int nvis,
                                                 int hq) {
  BlockMass r;
  if constexpr (FAST) {
    const int T = j >> 4;
    const int tmax = a.NT > 0 ? a.NT - 1 : 0;
    const int Tm = T < tmax ? T : tmax, Tc = T > 0 ? (T - 1 < tmax ? T - 1 : tmax) : 0;
    const bool first = (j & 15) == 0;
    const bool main_ok = (first ? 4 * j : 4 * j - 1) <= nvis - 1;
    const bool carry_ok = first && j > 0 && 4 * j - 1 <= nvis - 1;
    r.m0 = *reinterpret_cast<const f32x4*>(a.cb + ((bkv * a.NT + Tm) * a.NBT + (j - 16 * T)) * 16 +
                                           4 * hq);
    r.m1 = *reinterpret_cast<const f32x4*>(a.cb + ((bkv * a.NT + Tc) * a.NBT + 16) * 16 + 4 * hq);
    r.ta = Tm;
    r.tb = Tc;
    r.ntile = (main_ok ? 1 : 0) | (carry_ok ? 2 : 0);
  } else {
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
    r.m0 = *reinterpret_cast<const f32x4*>(a.cb + entry(ta));
    r.m1 = *reinterpret_cast<const f32x4*>(a.cb + entry(tb));
    r.ta = ta;
    r.tb = tb;
    r.ntile = lo <= hi ? hi / 64 - lo / 64 + 1 : 0;
  }
  return r;
}

// Group score share of one tile: masses times w = exp2(tref - lse), the per-head normalisation
// of the compressed softmax (w per tile and head, computed once).
__device__ __forceinline__ float mass_score(const f32x4& m, const float* w) {
  return (m[0] * w[0] + m[1] * w[1]) + (m[2] * w[2] + m[3] * w[3]);
}

constexpr int kGrpWaves = 8;
constexpr int kGrpThreads = 64 * kGrpWaves;
constexpr int kGrpLanes = kGrpThreads / 4;  // blocks per pass (four lanes per block)
constexpr int kGrpUnroll = 8;               // passes whose loads are in flight together
constexpr int kCoRegs = 4;                  // compressed-output chunks prefetched in registers

// Dynamic LDS of dec_group_kernel: one region reused by the three phases (selection state,
// per-wave V^T tiles, per-wave partial outputs), then the compressed chunk weights.
struct GroupLds {
  size_t cm, cl, tr, S, keys, region, wc, total;
};
__host__ __device__ inline GroupLds group_lds(int D, int nch, int nt, int nblk) {
  auto up = [](size_t x) { return (x + 15) & ~(size_t)15; };
  GroupLds g{};
  size_t o = 0;
  g.cm = o;   o = up(o + (size_t)nch * 16 * 4);
  g.cl = o;   o = up(o + (size_t)nch * 16 * 4);
  g.tr = o;   o = up(o + (size_t)nt * 16 * 4);
  g.S = o;    o = up(o + (size_t)nblk * 4);
  g.keys = o; o = up(o + (size_t)kGrpWaves * 64 * 8);
  const size_t tiles = (size_t)kGrpWaves * D * 64 * 2;
  const size_t merge = (size_t)2 * kGrpWaves * 16 * (D + 4) * 4;
  g.region = o > tiles ? o : tiles;
  g.region = g.region > merge ? g.region : merge;
  g.wc = g.region;
  g.total = up(g.wc + (size_t)nch * 16 * 4);
  return g;
}

// One workgroup per (sequence, group), after the compressed stream:
//  1. the window's tiles (known before any selection) are requested at once, one per wave;
//  2. per-head log-sum-exp of the compressed softmax, every group block score (the tile masses
//     of the compressed stream rescaled by exp2(tref - lse), summed over the group's heads), the
//     top-n with block 0 and the local blocks forced (each wave ranks an eighth of the blocks,
//     one wave merges), the compressed output normalised and weighted;
//  3. the tile list: window tiles first, then selected tiles outside the window, each tile once
//     and marked with the branches it feeds; the waves take turns over it (the next tile's K in
//     flight during this tile's softmax and P V, its V after them);
//  4. the waves' partials merged per branch in LDS and the gate applied:
//     out = g0 * o_cmp + g1 * o_slc + g2 * o_win.
template <int D, bool FAST>
__global__ __launch_bounds__(kGrpThreads, 1) void dec_group_kernel(DecodeArgs a) {
  constexpr int DT = D / 16, OP = D + 4;
  extern __shared__ __align__(16) unsigned char gsm[];
  __shared__ float lse_s[16];
  __shared__ int sidx[64];
  __shared__ int tl_s[kMaxTiles];
  __shared__ int tn_s;
  __shared__ float Wm[2][kGrpWaves][16], Wl[2][kGrpWaves][16];
  __shared__ __align__(16) u16 Qs[16][D + 8];  // the group's queries (MFMA B operand rows)
  const GroupLds L = group_lds(D, a.NCH, a.NT, a.nblk);
  float* scm = reinterpret_cast<float*>(gsm + L.cm);
  float* scl = reinterpret_cast<float*>(gsm + L.cl);
  float* trs = reinterpret_cast<float*>(gsm + L.tr);
  float* Ss = reinterpret_cast<float*>(gsm + L.S);
  uint64_t* Kw = reinterpret_cast<uint64_t*>(gsm + L.keys);
  u16(*Vt)[D][64] = reinterpret_cast<u16(*)[D][64]>(gsm);
  float* Ob = reinterpret_cast<float*>(gsm);  // [2][waves][16][OP]
  float* wc = reinterpret_cast<float*>(gsm + L.wc);

  const int kvh = blockIdx.x, b = blockIdx.y;
  const long bkv = (long)b * a.Hkv + kvh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int g4 = lane >> 4, r16 = lane & 15;
  const int t = a.seqlens[b] - 1;
  const int nb = t / a.beta + 1;
  const int nvis = n_visible(t, a.l, a.d, a.ncmp);
  const int nch = (nvis + CHUNK - 1) / CHUNK;
  const int ntv = (nvis + 63) / 64;
  const bool top_p = a.top_p > 0.f;
  const bool all = nb <= a.top_n && !top_p;  // uniform: every block is selected
  const bool scored = !all && nvis > 0;  // uniform
  const float sl = a.scale_log2;
  const int w0 = t - a.window + 1;
  const int wt0 = (w0 > 0 ? w0 : 0) / 64, wt1 = t / 64, nwin = wt1 - wt0 + 1;
  const u16* kcb = a.kcache + bkv * (long)a.L * D;
  const u16* vcb = a.vcache + bkv * (long)a.L * D;

  // the group's queries, one 16-byte octet per thread (16 heads x D / 8 octets <= 512 threads),
  // stored to LDS with the first statistics: the waves re-read their fragments per tile
  // instead of holding them in registers
  const int qh = tid / (D / 8), qc = (tid % (D / 8)) * 8;
  const bool qlive = tid < 16 * (D / 8) && qh < a.G;
  const bf16x8 qv =
      load8(a.q + ((long)b * a.Hkv * a.G + kvh * a.G + (qlive ? qh : 0)) * D + (qlive ? qc : 0));

  // 2. selection.  Loads first (chunk statistics, tile references, compressed outputs of the
  // first chunks, the first block masses), then the LDS stores that wait for them.
  const int hq = tid & 3, jq = tid >> 2;
  const bool many = nch * 16 > kGrpThreads;  // uniform: beyond 32 chunks, a loop below
  const int ce = tid < nch * 16 ? tid : 0;
  const float cmv = a.cm[bkv * a.NCH * 16 + ce], clv = a.cl[bkv * a.NCH * 16 + ce];
  // tile references: one f32x4 per thread up to 128 tiles (clamped, stored below), a loop beyond
  const bool tr_loop = ntv * 4 > kGrpThreads;  // uniform
  const f32x4 trv = *reinterpret_cast<const f32x4*>(
      a.tref + bkv * a.NT * 16 + 4 * (tid < ntv * 4 ? tid : 0));
  // the loads above are waited for first: keep them ahead of the prefetches below (the counter
  // of loads in flight retires in order, so waiting for a later load waits for every earlier one)
  __asm__ volatile("" ::: "memory");
  BlockMass bm[kGrpUnroll];
#pragma unroll
  for (int u = 0; u < kGrpUnroll; ++u) {
    const int j = jq + kGrpLanes * u;
    bm[u] = fetch_block<FAST>(a, bkv, j < nb ? j : nb - 1, nvis, hq);
  }
  __asm__ volatile("" ::: "memory");
  if (!many && tid < nch * 16) {
    scm[tid] = cmv;
    scl[tid] = clv;
  }
  if (tid < 16 * (D / 8)) *reinterpret_cast<bf16x8*>(&Qs[qh][qc]) = qlive ? qv : zero8();
  if (many)
    for (int e = tid; e < nch * 16; e += kGrpThreads) {
      scm[e] = a.cm[bkv * a.NCH * 16 + e];
      scl[e] = a.cl[bkv * a.NCH * 16 + e];
    }
  if (tr_loop) {
    for (int e = tid; e < ntv * 4; e += kGrpThreads)
      *reinterpret_cast<f32x4*>(trs + 4 * e) =
          *reinterpret_cast<const f32x4*>(a.tref + bkv * a.NT * 16 + 4 * e);
  } else if (tid < ntv * 4) {
    *reinterpret_cast<f32x4*>(trs + 4 * tid) = trv;
  }
  lds_barrier();
  if (tid < 256) {  // 16 lanes per head
    const int h = tid >> 4, sub = tid & 15;
    float M = kNegInf;
    for (int c = sub; c < nch; c += 16) M = fmaxf(M, scm[c * 16 + h]);
    M = group_max<16>(M);
    float Ls = 0.f;
    for (int c = sub; c < nch; c += 16) Ls += scl[c * 16 + h] * fast_exp2(scm[c * 16 + h] - M);
    Ls = group_sum<16>(Ls);
    // heads past G get +inf: their weights vanish
    if (sub == 0) lse_s[h] = (M == kNegInf || h >= a.G) ? __builtin_inff() : M + __log2f(Ls);
  }
  lds_barrier();
  // chunk weights exp2(cm - lse); tile weights exp2(tref - lse) in place of the references
  for (int e = tid; e < nch * 16; e += kGrpThreads) wc[e] = fast_exp2(scm[e] - lse_s[e & 15]);
  for (int e = tid; e < ntv * 16; e += kGrpThreads) trs[e] = fast_exp2(trs[e] - lse_s[e & 15]);
  lds_barrier();
  if (scored) {
    for (int j0 = jq;; j0 += kGrpLanes * kGrpUnroll) {
#pragma unroll
      for (int u = 0; u < kGrpUnroll; ++u) {
        const int j = j0 + kGrpLanes * u;
        float S = 0.f;
        if constexpr (FAST) {
          // main + carry equals the generic carry + main bit for bit (one commutative add)
          if (bm[u].ntile & 1) S = mass_score(bm[u].m0, trs + bm[u].ta * 16 + 4 * hq);
          if (bm[u].ntile & 2) S += mass_score(bm[u].m1, trs + bm[u].tb * 16 + 4 * hq);
        } else {
          if (bm[u].ntile >= 1) S = mass_score(bm[u].m0, trs + bm[u].ta * 16 + 4 * hq);
          if (bm[u].ntile >= 2) S += mass_score(bm[u].m1, trs + (bm[u].ta + 1) * 16 + 4 * hq);
          for (int T = bm[u].ta + 2; T < bm[u].ta + bm[u].ntile; ++T) {  // wide blocks only
            const int jj = j - (T * 64 * a.d) / a.beta;
            const f32x4 m = *reinterpret_cast<const f32x4*>(
                a.cb + ((bkv * a.NT + T) * a.NBT + jj) * 16 + 4 * hq);
            S += mass_score(m, trs + T * 16 + 4 * hq);
          }
        }
        S = group_sum<4>(S);
        if (hq == 0 && j < nb) Ss[j] = S;
      }
      const int jn = j0 + kGrpLanes * kGrpUnroll;
      if (jn - jq >= nb) break;  // uniform
#pragma unroll
      for (int u = 0; u < kGrpUnroll; ++u) {
        const int j = jn + kGrpLanes * u;
        bm[u] = fetch_block<FAST>(a, bkv, j < nb ? j : nb - 1, nvis, hq);
      }
    }
  } else if (!all) {
    for (int j = tid; j < nb; j += kGrpThreads) Ss[j] = 0.f;
  }
  // compressed outputs of the first chunks for this thread's output pairs p = tid + 512 i
  // (head p / D, feature p % D), in flight during the top-n.  (The window's K/V tiles are not
  // requested here: with every group doing so at once, a wave stalls issuing them while memory
  // is busy, and the whole workgroup waits for it at the next barrier.)
  constexpr int PPT = 16 * D / kGrpThreads;
  float cov[PPT][kCoRegs];
#pragma unroll
  for (int i = 0; i < PPT; ++i)
#pragma unroll
    for (int c = 0; c < kCoRegs; ++c) {
      const int cc = c < a.NCH ? c : 0;
      cov[i][c] = a.co[(bkv * a.NCH + cc) * 16 * D + tid + kGrpThreads * i];
    }
  lds_barrier();  // scores and chunk weights in LDS (the loads stay in flight)
  const int bcur = nb - 1;
  const int flo = bcur - a.n_local + 1 > 1 ? bcur - a.n_local + 1 : 1;  // forced: 0, flo..bcur
  const int kfree = a.top_n - 1 - a.n_local;
  // top-n in two levels: waves 0-3 (one per SIMD) each rank a quarter of the free blocks
  // 1 .. flo-1, then wave 0 ranks their 4 * kfree winners
  constexpr int kRankWaves = 4;
  if (!all && wave < kRankWaves) {  // uniform
    const int span = (flo - 1 + kRankWaves - 1) / kRankWaves;
    const int lo = 1 + wave * span;
    const int hi = lo + span < flo ? lo + span : flo;
    const uint64_t key =
        wave_topk([&](int j) { return rank_key(Ss[j], j); }, lo, hi, kfree, lane);
    if (lane < kfree) Kw[wave * kfree + lane] = key;
  }
  lds_barrier();
  if (wave == 0) {
    int32_t* orow = a.idx + bkv * a.top_n;
    if (all) {
      if (lane < a.top_n) {
        const int el = lane < nb ? lane : -1;
        orow[lane] = el;
        sidx[lane] = el;
      }
    } else {
      uint64_t key =
          wave_topk([&](int i) { return Kw[i]; }, 0, kRankWaves * kfree, kfree, lane);
      if (top_p) {
        float forced = Ss[0];
        for (int j = flo; j <= bcur; ++j) forced += Ss[j];
        key = top_p_cut(key, kfree, forced, nvis > 0 ? a.top_p * (float)a.G : 0.f, lane);
      }
      int el = key != 0 ? rank_key_index(key) : 0x7FFFFFFF;
      if (lane == kfree) el = 0;
      if (lane > kfree && lane <= kfree + bcur - flo + 1) el = flo + (lane - kfree - 1);
      int rank = 0;
      for (int o = 0; o < a.top_n; ++o)  // the whole wave is active here
        rank += (__builtin_amdgcn_readlane(el, o) < el) ? 1 : 0;
      const bool valid = lane < a.top_n && el != 0x7FFFFFFF;
      const int nsel = (int)__popcll(__ballot(valid));
      if (valid) {
        orow[rank] = el;
        sidx[rank] = el;
      }
      if (lane >= nsel && lane < a.top_n) {
        orow[lane] = -1;
        sidx[lane] = -1;
      }
    }
    __asm__ volatile("" ::: "memory");  // sidx written by this wave before its reads
    // 3. tile list: the window tiles, flagged when their block is selected, then the tiles of
    // selected blocks outside the window, at or before t
    const int per = a.beta / 64;
    for (int i = lane; i < nwin; i += 64) {
      const int tile = wt0 + i, jw = tile / per;
      bool in = false;
      for (int e = 0; e < a.top_n; ++e) in |= sidx[e] == jw;
      tl_s[i] = tile | (in ? 1 << 30 : 0);
    }
    const int nsel = a.top_n * per;
    int base = nwin;
    for (int i0 = 0; i0 < nsel; i0 += 64) {
      const int i = i0 + lane;
      int code = -1;
      if (i < nsel) {
        const int jb = sidx[i / per], tile = jb * per + i % per;
        if (jb >= 0 && tile * 64 <= t && (tile < wt0 || tile > wt1)) code = tile | (1 << 30);
      }
      const uint64_t m = __ballot(code >= 0);
      const int pos = base + (int)__popcll(m & ((1ull << lane) - 1ull));
      if (code >= 0) tl_s[pos] = code;
      base += (int)__popcll(m);
    }
    if (lane == 0) tn_s = base;
  }
  lds_barrier();  // tile list ready; the selection state in the shared region is dead
  // compressed output of this thread's pairs: sum over chunks of co * exp2(cm - lse)
  float ocmp[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int h = (tid + kGrpThreads * i) / D;
    float o = 0.f;
#pragma unroll
    for (int c = 0; c < kCoRegs; ++c) o += c < nch ? cov[i][c] * wc[c * 16 + h] : 0.f;
    for (int c = kCoRegs; c < nch; ++c)  // long contexts only
      o += a.co[(bkv * a.NCH + c) * 16 * D + tid + kGrpThreads * i] * wc[c * 16 + h];
    ocmp[i] = o;
  }

  // 3. the tiles: wave w takes list entries w, w + 8, ... (a fixed assignment: the same wave
  // sums the same tiles in the same order on every call, so the output is reproducible bit for
  // bit; handing entries to whichever wave asks first balanced slow loads for 1.3 us less)
  const int tn = __builtin_amdgcn_readfirstlane(tn_s);
  float mrun[2] = {kNegInf, kNegInf}, lrun[2] = {0.f, 0.f};
  f32x4 O[2][DT];
#pragma unroll
  for (int br = 0; br < 2; ++br)
#pragma unroll
    for (int n = 0; n < DT; ++n) O[br][n] = zero4();
  if (wave < tn) {  // uniform per wave
    int e = wave;
    DecTile<D> kv;
    kv.load(kcb, vcb, (tl_s[e] & 0x3FFFFFFF) * 64, t, lane);
    for (;;) {
      const int code = __builtin_amdgcn_readfirstlane(tl_s[e]);
      const int k0 = (code & 0x3FFFFFFF) * 64;
      const bool in_slc = (code >> 30) & 1, in_win = k0 + 63 >= w0;
      // the next tile; after the last one every row of the "next" load is row t (one line)
      const int en = e + kGrpWaves;  // static round robin: the same wave sums the same tiles
      const bool more = en < tn;
      const int k1 =
          more ? (__builtin_amdgcn_readfirstlane(tl_s[en]) & 0x3FFFFFFF) * 64 : t;
      const int last1 = more ? t : k1;
      f32x4 acc[4];
      {
        bf16x8 qf[D / 32];
#pragma unroll
        for (int c = 0; c < D / 32; ++c) qf[c] = load8(&Qs[r16][32 * c + 8 * g4]);
        kv.scores(qf, acc);
      }
      __asm__ volatile("" ::: "memory");  // the previous tile's Vt reads stay before these writes
      kv.stage(Vt[wave], lane);
      __asm__ volatile("" ::: "memory");  // Vt[wave] is this wave's own: LDS keeps its order
      kv.load_k(kcb, k1, last1, lane);
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
        for (int q = 0; q < 16; ++q) {
          p[q] = fast_exp2(fmaf(p[q], sl, -ms));
          ls += p[q];
        }
        lrun[br] = fmaf(lrun[br], alpha, col_sum4(ls));
#pragma unroll
        for (int n = 0; n < DT; ++n) O[br][n] *= alpha;
        tile_pv<D>(Vt[wave], p, g4, r16, O[br]);
      }
      kv.load_v(vcb, k1, last1, lane);
      if (!more) break;
      e = en;
    }
  }
  if (g4 == 0) {
#pragma unroll
    for (int br = 0; br < 2; ++br) { Wm[br][wave][r16] = mrun[br]; Wl[br][wave][r16] = lrun[br]; }
  }
  __syncthreads();  // Vt reads done; maxima posted
  // 4. partials rescaled to the workgroup maximum of each branch, summed through LDS
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kGrpWaves; ++w) M = fmaxf(M, Wm[br][w][r16]);
    const float f =
        Wm[br][wave][r16] == kNegInf ? 0.f : fast_exp2((Wm[br][wave][r16] - M) * sl);
#pragma unroll
    for (int n = 0; n < DT; ++n)
      *reinterpret_cast<f32x4*>(&Ob[((br * kGrpWaves + wave) * 16 + r16) * OP + 16 * n + 4 * g4]) =
          f * O[br][n];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int pr = tid + kGrpThreads * i;
    const int h = pr / D, dd = pr % D;
    if (h >= a.G) continue;
    float ob[2];
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kGrpWaves; ++w) M = fmaxf(M, Wm[br][w][h]);
      float Lb = 0.f, o = 0.f;
#pragma unroll
      for (int w = 0; w < kGrpWaves; ++w) {
        if (Wm[br][w][h] != kNegInf) Lb += Wl[br][w][h] * fast_exp2((Wm[br][w][h] - M) * sl);
        o += Ob[((br * kGrpWaves + w) * 16 + h) * OP + dd];
      }
      ob[br] = Lb > 0.f ? o / Lb : 0.f;
    }
    const long head = (long)b * a.Hkv * a.G + kvh * a.G + h;
    const float* g = a.gate + head * 3;
    a.out[head * D + dd] = g[0] * ocmp[i] + g[1] * ob[0] + g[2] * ob[1];
  }
}

// ------------------------------------------------------------------ launcher

int decode_chunk_tokens() { return CHUNK; }
int decode_max_tile_list() { return kMaxTiles; }
size_t decode_group_lds_bytes(int D, int nch, int nt, int nblk) {
  return group_lds(D, nch, nt, nblk).total;
}

void launch_decode(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  auto mark = [&](int i) {
    if (ev != nullptr) (void)hipEventRecord(ev[i], s);
  };
  const bool fast = a.beta == 4 * a.d && a.l == 2 * a.d && a.NBT >= 17;
  const size_t lds = decode_group_lds_bytes(a.D, a.NCH, a.NT, a.nblk);
  const void* gk =
      a.D == 128 ? (fast ? reinterpret_cast<const void*>(dec_group_kernel<128, true>)
                         : reinterpret_cast<const void*>(dec_group_kernel<128, false>))
                 : (fast ? reinterpret_cast<const void*>(dec_group_kernel<64, true>)
                         : reinterpret_cast<const void*>(dec_group_kernel<64, false>));
  // opt in to the accepted maximum (not this launch's size: concurrent calls on other host
  // threads may need more); the attribute is per device, so it is set on every launch
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(gk, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kMaxDecodeDynLds);
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
  const dim3 g2(a.Hkv, a.B);
  if (a.D == 128) {
    if (fast) dec_group_kernel<128, true><<<g2, kGrpThreads, lds, s>>>(a);
    else dec_group_kernel<128, false><<<g2, kGrpThreads, lds, s>>>(a);
  } else {
    if (fast) dec_group_kernel<64, true><<<g2, kGrpThreads, lds, s>>>(a);
    else dec_group_kernel<64, false><<<g2, kGrpThreads, lds, s>>>(a);
  }
  mark(2);
}

}  // namespace nsa
