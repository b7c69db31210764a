// NSA decode: one new query per sequence against a KV cache ("Native Sparse Attention"
// article: decode loads only the compressed, the selected and the window KV, saving HBM
// bandwidth; podcast notes EP94 section 6: one shared selection per GQA group, so one KV read
// serves the group's heads).  Every phase streams HBM; the matrix core does the contractions
// with the group's heads as the 16 MFMA rows.  Four launches:
//
//   dec_cmp_kernel     split-K over the compressed cache: each wave streams TPW 64-token tiles
//                      with register prefetch and an online softmax; per 1024-token chunk, per
//                      head, (max, sum, unnormalised output); per tile, the probability mass of
//                      every selection block it touches, relative to a per-tile reference
//   dec_select_kernel  per 256-block slice of a group (so a long sequence spreads its selection
//                      over many workgroups): the per-head log-sum-exp, the group block scores,
//                      the slice's best free blocks, and the normalised compressed output of a
//                      share of the heads
//   dec_tiles_kernel   NG workgroups per group: NGW of them take the window's and the forced
//                      blocks' tiles (known before the selection) at once, the others merge the
//                      slices' candidates into the top-n (forced blocks added, ascending,
//                      written out) and take the other selected blocks' tiles; tiles dealt out
//                      over the waves of each kind; per branch one partial record per
//                      workgroup
//   dec_merge_kernel   per group (over four workgroups): the records merged in workgroup order,
//                      and the gate
// Tile work is assigned in a fixed order and every sum runs in a fixed order, so the output is
// the same bit for bit on every call.
#include "attn_tile.h"
#include "dev_common.h"
#include "kernels.h"

namespace nsa {

constexpr int TPW = 4;               // 64-token tiles per wave in dec_cmp
constexpr int CHUNK = 4 * TPW * 64;  // compressed tokens per dec_cmp workgroup

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
        // the e-th features of keys 4 kq .. 4 kq + 3 paired by byte permutes: bytes 0,1 (even
        // e) or 2,3 (odd e) of the lower key's word, then the same of the upper key's
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u, d = 8 * dc + e;
        uint2 pk;
        pk.x = __builtin_amdgcn_perm(v[it * 4 + 1][e >> 1], v[it * 4 + 0][e >> 1], sel);
        pk.y = __builtin_amdgcn_perm(v[it * 4 + 3][e >> 1], v[it * 4 + 2][e >> 1], sel);
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

// ------------------------------------------------------------------ block masses

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


constexpr int kSelThreads = 256;             // one selection slice
constexpr int kSelWaves = kSelThreads / 64;  // tile slots of a tile worker
constexpr int kSliceTiles = 64;              // tile weights a selection slice holds
constexpr uint32_t kCodeSlc = 1u << 30, kCodeWin = 1u << 29, kCodeTile = (1u << 29) - 1;

int decode_slice_blocks(int l, int d, int beta) {
  // the blocks j0 .. j0 + sb - 1 touch compressed tokens (j0 beta - l + 1) / d .. ((j0 + sb)
  // beta - 1) / d: at most (sb beta + l) / d + 1 tokens, i.e. that / 64 + 2 tiles
  int sb = 256;
  while (sb > 1 && ((long)sb * beta + l) / d + 1 > (long)(kSliceTiles - 2) * 64) sb /= 2;
  return sb;
}

// Per-sequence selection geometry of one decode query.
struct DecRow {
  int t, nb, nvis, nch, bcur, flo, kfree, wt0, wt1, w0;
  bool top_p, all;
};

__device__ __forceinline__ DecRow dec_row(const DecodeArgs& a, int b) {
  DecRow r;
  r.t = a.seqlens[b] - 1;
  r.nb = r.t / a.beta + 1;
  r.nvis = n_visible(r.t, a.l, a.d, a.ncmp);
  r.nch = (r.nvis + CHUNK - 1) / CHUNK;
  r.top_p = a.top_p > 0.f;
  r.all = r.nb <= a.top_n && !r.top_p;  // every block is selected
  r.bcur = r.nb - 1;
  r.flo = r.bcur - a.n_local + 1 > 1 ? r.bcur - a.n_local + 1 : 1;  // forced: 0, flo .. bcur
  r.kfree = a.top_n - 1 - a.n_local;
  r.w0 = r.t - a.window + 1;
  r.wt0 = (r.w0 > 0 ? r.w0 : 0) / 64;
  r.wt1 = r.t / 64;
  return r;
}

// The group's queries (rows of the MFMA B operand) into LDS, one 16-byte octet per thread;
// rows past G are zero.
template <int D>
__device__ __forceinline__ void stage_queries(const DecodeArgs& a, int b, int kvh,
                                              u16 (*Qs)[D + 8]) {
  for (int e = threadIdx.x; e < 16 * (D / 8); e += kSelThreads) {
    const int qh = e / (D / 8), qc = (e % (D / 8)) * 8;
    *reinterpret_cast<bf16x8*>(&Qs[qh][qc]) =
        qh < a.G ? load8(a.q + ((long)b * a.Hkv * a.G + kvh * a.G + qh) * D + qc) : zero8();
  }
}

// Running softmax state of one wave over its tiles, for NBR branches.
template <int D, int NBR>
struct WaveSoftmax {
  float m[NBR], l[NBR];
  f32x4 O[NBR][D / 16];
};

// One wave's pass over the tile list entries first, first + stride, ... (< n): each tile's K
// and V read once, feeding every branch whose mask its code allows (branch 0: selected keys
// <= t; branch 1: window keys w0 .. t); the next tile's K in flight during this tile's softmax
// and P V, its V after them.  Codes: tile index | kCodeSlc | kCodeWin.
template <int D, int NBR>
__device__ void wave_tiles(const DecodeArgs& a, long bkv, const DecRow& r, const int* list,
                           int n, int first, int stride, const u16 (*Qs)[D + 8],
                           u16 (*Vt)[64], WaveSoftmax<D, NBR>& st) {
  constexpr int DT = D / 16;
  const int lane = threadIdx.x & 63, g4 = lane >> 4, r16 = lane & 15;
  const float sl = a.scale_log2;
  const u16* kcb = a.kcache + bkv * (long)a.L * D;
  const u16* vcb = a.vcache + bkv * (long)a.L * D;
#pragma unroll
  for (int br = 0; br < NBR; ++br) {
    st.m[br] = kNegInf;
    st.l[br] = 0.f;
#pragma unroll
    for (int n2 = 0; n2 < DT; ++n2) st.O[br][n2] = zero4();
  }
  if (first >= n) return;  // uniform per wave
  int e = first;
  DecTile<D> kv;
  kv.load(kcb, vcb, (int)(list[e] & kCodeTile) * 64, r.t, lane);
  for (;;) {
    const uint32_t code = (uint32_t)__builtin_amdgcn_readfirstlane(list[e]);
    const int k0 = (int)(code & kCodeTile) * 64;
    const bool in_slc = code & kCodeSlc, in_win = code & kCodeWin;
    const int en = e + stride;
    const bool more = en < n;
    // after the last tile every row of the "next" load is row t (one line, in bounds)
    const int k1 = more ? (int)((uint32_t)__builtin_amdgcn_readfirstlane(list[en]) & kCodeTile) * 64
                        : r.t;
    const int last1 = more ? r.t : k1;
    f32x4 acc[4];
    {
      bf16x8 qf[D / 32];
#pragma unroll
      for (int c = 0; c < D / 32; ++c) qf[c] = load8(&Qs[r16][32 * c + 8 * g4]);
      kv.scores(qf, acc);
    }
    __asm__ volatile("" ::: "memory");  // the previous tile's Vt reads stay before these writes
    kv.stage(Vt, lane);
    __asm__ volatile("" ::: "memory");  // Vt is this wave's own: LDS keeps its order
    kv.load_k(kcb, k1, last1, lane);
#pragma unroll
    for (int br = 0; br < NBR; ++br) {
      // a branch the tile does not feed (uniform) would only add masked zeros: skipped
      if (!(br == 0 ? in_slc : in_win)) continue;
      float p[16];
      float tm = kNegInf;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + lane_key(q4, i, g4);
          const bool ok = br == 0 ? (in_slc && key <= r.t)
                                  : (in_win && key <= r.t && key >= r.w0);
          const float x = ok ? acc[q4][i] : kNegInf;
          p[q4 * 4 + i] = x;
          tm = fmaxf(tm, x);
        }
      tm = col_max4(tm);
      const float mn = fmaxf(st.m[br], tm);
      const float ms = mn == kNegInf ? 0.f : mn * sl;
      const float alpha = fast_exp2(fmaf(st.m[br], sl, -ms));
      st.m[br] = mn;
      float ls = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        p[q] = fast_exp2(fmaf(p[q], sl, -ms));
        ls += p[q];
      }
      st.l[br] = fmaf(st.l[br], alpha, col_sum4(ls));
#pragma unroll
      for (int n2 = 0; n2 < DT; ++n2) st.O[br][n2] *= alpha;
      tile_pv<D>(Vt, p, g4, r16, st.O[br]);
    }
    kv.load_v(vcb, k1, last1, lane);
    if (!more) break;
    e = en;
  }
}

// The four waves' states of branch br merged into one record (16 maxima in scaled log2 units,
// 16 sums, 16 x D outputs relative to the maxima), summed in wave order.  Reuses `region`
// (the waves' Vt tiles: every wave must be past its tile loop, which the first barrier
// ensures).
template <int D, int NBR>
__device__ void write_record(const WaveSoftmax<D, NBR>& st, int br, float sl, float* region,
                             float* rec) {
  constexpr int DT = D / 16, OP = D + 4;
  __shared__ float Wm[kSelWaves][16], Wl[kSelWaves][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  __syncthreads();  // region free (tile loops or an earlier branch's reads done)
  if (g4 == 0) {
    Wm[wave][r16] = st.m[br];
    Wl[wave][r16] = st.l[br];
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) M = fmaxf(M, Wm[w][r16]);
  const float f = st.m[br] == kNegInf ? 0.f : fast_exp2((st.m[br] - M) * sl);
#pragma unroll
  for (int n2 = 0; n2 < DT; ++n2)
    *reinterpret_cast<f32x4*>(&region[(wave * 16 + r16) * OP + 16 * n2 + 4 * g4]) =
        f * st.O[br][n2];
  __syncthreads();
  for (int e = tid; e < 16 * D; e += kSelThreads) {
    const int o = (e / D) * OP + e % D;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) v += region[w * 16 * OP + o];
    rec[32 + e] = v;
  }
  if (tid < 16) {
    float Mh = kNegInf;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) Mh = fmaxf(Mh, Wm[w][tid]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w)
      if (Wm[w][tid] != kNegInf) L += Wl[w][tid] * fast_exp2((Wm[w][tid] - Mh) * sl);
    rec[tid] = Mh == kNegInf ? kNegInf : Mh * sl;
    rec[16 + tid] = L;
  }
}

// Fixed tiles of one group: the window's tiles and the forced blocks' tiles (or, when every
// block fits in top_n, all tiles), known before the selection; flagged with the branches they
// feed.  Written to list by the first wave; returns the count (lane-uniform).
__device__ int fixed_tile_list(const DecodeArgs& a, const DecRow& r, int* list, int lane) {
  const int per = a.beta / 64;
  const int tl = r.t / 64;  // last tile at or before t
  if (r.all) {
    for (int i = lane; i <= tl; i += 64)
      list[i] = (int)(i | kCodeSlc | (i >= r.wt0 ? kCodeWin : 0u));
    return tl + 1;
  }
  const int nw = r.wt1 - r.wt0 + 1;
  for (int i = lane; i < nw; i += 64) {
    const int tile = r.wt0 + i, jb = tile / per;
    const bool forced = jb == 0 || (jb >= r.flo && jb <= r.bcur);
    list[i] = (int)(tile | kCodeWin | (forced ? kCodeSlc : 0u));
  }
  // forced blocks' tiles outside the window: block 0, then flo .. bcur
  const int nf = (1 + (r.bcur - r.flo + 1)) * per;
  int base = nw;
  for (int i0 = 0; i0 < nf; i0 += 64) {
    const int i = i0 + lane;
    int code = -1;
    if (i < nf) {
      const int jb = i < per ? 0 : r.flo + (i - per) / per;
      const int tile = jb * per + i % per;
      if (tile <= tl && (tile < r.wt0 || tile > r.wt1)) code = (int)(tile | kCodeSlc);
    }
    const uint64_t m = __ballot(code >= 0);
    const int pos = base + (int)__popcll(m & ((1ull << lane) - 1ull));
    if (code >= 0) list[pos] = code;
    base += (int)__popcll(m);
  }
  return base;
}

// ------------------------------------------------------------------ phase 1: compressed stream

// FAST: sel_block = 4 * stride and cmp_len = 2 * stride, where block j receives
// p(4j-1)/2 + p(4j) + p(4j+1) + p(4j+2) + p(4j+3)/2: the lane holding keys 4jl..4jl+3 of a
// tile forms the block's core, and the half-token carries cross lanes by shuffles.
// The compressed chunk of dec_cmp_kernel (see there).
template <int D, bool FAST>
__device__ __forceinline__ void cmp_chunk(const DecodeArgs& a, int b, int kvh, long bkv, int chunk,
                                          int nvis, float* Ob, float (*Wm)[16], float (*Wl)[16],
                                          float (*Pw)[FAST ? 1 : 16][64]) {
  constexpr int DT = D / 16, OP = D + 4;
  const int c0 = chunk * CHUNK;
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


// Workgroup `chunk` of a group streams the compressed tokens chunk * CHUNK .. + CHUNK - 1 that
// are visible.
template <int D, bool FAST>
__global__ __launch_bounds__(256, FAST ? 2 : 1) void dec_cmp_kernel(DecodeArgs a) {
  __shared__ __align__(16) float Ob[4 * 16 * (D + 4)];  // the waves' compressed partials
  __shared__ float Wm[4][16], Wl[4][16];
  __shared__ float Pw[FAST ? 1 : 4][FAST ? 1 : 16][64];
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int nvis = n_visible(a.seqlens[b] - 1, a.l, a.d, a.ncmp);
  const long bkv = (long)b * a.Hkv + kvh;
  if (chunk * CHUNK < nvis) cmp_chunk<D, FAST>(a, b, kvh, bkv, chunk, nvis, Ob, Wm, Wl, Pw);
}

// ------------------------------------------------------------------ phase 2: selection slices

constexpr int kLseRegs = 4;  // chunk statistics per thread held in registers (<= 64 chunks)

// One selection slice: the group block scores of blocks j0 .. j1-1 (the tile masses of the
// compressed stream rescaled by exp2(tref - lse), summed over the group's heads; four lanes per
// block, four heads each), written out, and the slice's best free blocks by (score desc, index
// asc).  Every load the slice needs (chunk statistics, tile references, block masses) is issued
// up front, before the per-head log-sum-exp they wait on is reduced.  Slice 0 also posts the
// log-sum-exp for the merge, and each running slice normalises the compressed output of its
// share of the heads (heads s, s + nrun, ...: the chunk partials of one head weighted by
// exp2(chunk max - lse)).  Runs before the selection of the group is known, so every slice
// of every group is independent.
template <int D, bool FAST>
__device__ void select_slice(const DecodeArgs& a, long bkv, int b, int s, unsigned char* smem) {
  const DecRow r = dec_row(a, b);
  const int j0 = s * a.SB;
  const bool ranks = !r.all && j0 < r.nb;  // uniform
  if (!ranks && s != 0) return;
  const int j1 = j0 + a.SB < r.nb ? j0 + a.SB : r.nb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* lse_s = reinterpret_cast<float*>(smem);  // [16]
  float* trs = lse_s + 16;                        // [kSliceTiles][16]
  float* Ss = trs + kSliceTiles * 16;             // [SB]
  f32x4* red = reinterpret_cast<f32x4*>(Ss + 256);  // [parts][span] compressed-output partials
  const bool scored = r.nvis > 0;
  const int ntv = (r.nvis + 63) / 64;
  // tiles the slice's blocks read: from the one holding block j0's first compressed token (or
  // the carry of the tile before) to the one holding block j1-1's last visible token
  int tlo, thi;
  if constexpr (FAST) {
    tlo = (j0 >> 4) > 0 ? (j0 >> 4) - 1 : 0;
    thi = (j1 - 1) >> 4;
  } else {
    tlo = block_tok_lo(j0, a.beta, a.l, a.d) / 64;
    thi = block_tok_hi(j1 - 1, a.beta, a.d) / 64;
  }
  thi = thi < ntv - 1 ? thi : ntv - 1;
  const int ntr = ranks && scored && thi >= tlo ? (thi - tlo + 1) * 16 : 0;
  // 1. loads: chunk statistics of head h = tid / 16 (chunks sub, sub + 16, ...), the slice's
  // tile references, its blocks' masses (every index clamped: no load under a branch)
  const int h = tid >> 4, sub = tid & 15;
  const long cbase = bkv * a.NCH * 16 + h;
  const int clast = r.nch > 0 ? r.nch - 1 : 0;
  float vm[kLseRegs], vl[kLseRegs];
#pragma unroll
  for (int i = 0; i < kLseRegs; ++i) {
    const int c = sub + 16 * i, cc = c < clast ? c : clast;
    vm[i] = a.cm[cbase + cc * 16];
    vl[i] = a.cl[cbase + cc * 16];
  }
  f32x4 trv[kSliceTiles * 16 / kSelThreads / 4];
#pragma unroll
  for (int i = 0; i < kSliceTiles * 16 / kSelThreads / 4; ++i) {
    const int e = 4 * (tid + kSelThreads * i);
    const int ee = e < ntr ? e : 0;
    trv[i] = *reinterpret_cast<const f32x4*>(a.tref + (bkv * a.NT + tlo) * 16 + ee);
  }
  const int hq = tid & 3;
  constexpr int kPass = 256 / (kSelThreads / 4);  // block passes of a 256-block slice
  BlockMass bm[kPass];
  if (ranks && scored) {
#pragma unroll
    for (int u = 0; u < kPass; ++u) {
      const int j = j0 + (tid >> 2) + (kSelThreads / 4) * u;
      bm[u] = fetch_block<FAST>(a, bkv, j < j1 ? j : j1 - 1, r.nvis, hq);
    }
  }
  // compressed output of this slice's heads: pair = (head of the slice, feature quad); with few
  // pairs the chunks are split over `parts` threads per pair, with many (one slice for every
  // head) the pairs take several passes.  The first batch of loads is issued now.
  const int nrun = ranks ? (r.nb + a.SB - 1) / a.SB : 1;
  const int hps = s < a.G ? (a.G - 1 - s) / nrun + 1 : 0;
  const int npair = hps * (D / 4);
  int parts = 1;
  while (parts < 8 && 2 * parts * npair <= kSelThreads) parts *= 2;
  const int npass = (npair + kSelThreads - 1) / kSelThreads;
  struct OcMap { int pair, part, oh, of; bool on; };
  auto oc_map = [&](int pass) {
    OcMap m;
    const int base = pass * kSelThreads;
    const int span = npair - base < kSelThreads ? npair - base : kSelThreads;
    m.pair = base + tid % span;
    m.part = tid / span;
    m.on = m.part < parts;
    m.oh = s + nrun * (m.pair / (D / 4));
    m.of = 4 * (m.pair % (D / 4));
    return m;
  };
  constexpr int kOcBatch = 8;
  f32x4 ocv[kOcBatch];
  float ocm[kOcBatch];
  auto oc_load = [&](const OcMap& m, int c0) {
#pragma unroll
    for (int u = 0; u < kOcBatch; ++u) {
      const int c = c0 + u * parts, cc = c < clast ? c : clast;
      const long ci = (bkv * a.NCH + cc) * 16 + m.oh;
      ocv[u] = *reinterpret_cast<const f32x4*>(a.co + ci * D + m.of);
      ocm[u] = c < r.nch ? a.cm[ci] : kNegInf;
    }
  };
  if (npass > 0) {
    const OcMap m = oc_map(0);
    if (m.on) oc_load(m, m.part);
  }
  // 2. per-head log-sum-exp2 (16 lanes per head); heads past G get +inf: their weights vanish
  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < kLseRegs; ++i)
    if (sub + 16 * i < r.nch) M = fmaxf(M, vm[i]);
  for (int c = sub + 16 * kLseRegs; c < r.nch; c += 16) M = fmaxf(M, a.cm[cbase + c * 16]);
  M = group_max<16>(M);
  float Ls = 0.f;
#pragma unroll
  for (int i = 0; i < kLseRegs; ++i)
    if (sub + 16 * i < r.nch) Ls += vl[i] * fast_exp2(vm[i] - M);
  for (int c = sub + 16 * kLseRegs; c < r.nch; c += 16)
    Ls += a.cl[cbase + c * 16] * fast_exp2(a.cm[cbase + c * 16] - M);
  Ls = group_sum<16>(Ls);
  const float lse = M == kNegInf ? __builtin_inff() : M + __log2f(Ls);
  if (sub == 0) lse_s[h] = lse;
  lds_barrier();
  // the compressed output of this slice's heads, summed over the parts in order
  for (int pass = 0; pass < npass; ++pass) {
    const OcMap m = oc_map(pass);
    if (m.on) {
      if (pass > 0) oc_load(m, m.part);
      const float lh = lse_s[m.oh];
      f32x4 o = zero4();
      for (int c0 = m.part;; c0 += kOcBatch * parts) {
#pragma unroll
        for (int u = 0; u < kOcBatch; ++u)  // a select: a chunk not written this call may hold NaN
          o += ocm[u] == kNegInf ? zero4() : ocv[u] * fast_exp2(ocm[u] - lh);
        if (c0 + kOcBatch * parts >= r.nch) break;
        oc_load(m, c0 + kOcBatch * parts);
      }
      red[tid] = o;  // tid = part * span + local pair
    }
    lds_barrier();
    if (m.on && m.part == 0) {
      const int span = npair - pass * kSelThreads < kSelThreads ? npair - pass * kSelThreads
                                                                  : kSelThreads;
      f32x4 o = red[tid];
      for (int q = 1; q < parts; ++q) o += red[q * span + tid];
      *reinterpret_cast<f32x4*>(a.ocmp + (bkv * 16 + m.oh) * D + m.of) = o;
    }
    lds_barrier();  // red is reused by the next pass
  }
  if (!ranks) return;  // slice 0 of a group whose blocks all fit: only the compressed output
  if (tid < 16 && tid >= a.G) lse_s[tid] = __builtin_inff();  // idle heads weigh nothing
  lds_barrier();
  // 3. tile weights exp2(tref - lse), then the block scores
#pragma unroll
  for (int i = 0; i < kSliceTiles * 16 / kSelThreads / 4; ++i) {
    const int e = 4 * (tid + kSelThreads * i);
    if (e < ntr) {
      f32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = fast_exp2(trv[i][q] - lse_s[(e + q) & 15]);
      *reinterpret_cast<f32x4*>(trs + e) = w;
    }
  }
  lds_barrier();
  if (scored) {
#pragma unroll
    for (int u = 0; u < kPass; ++u) {
      const int j = j0 + (tid >> 2) + (kSelThreads / 4) * u;
      float S = 0.f;
      if constexpr (FAST) {
        if (bm[u].ntile & 1) S = mass_score(bm[u].m0, trs + (bm[u].ta - tlo) * 16 + 4 * hq);
        if (bm[u].ntile & 2) S += mass_score(bm[u].m1, trs + (bm[u].tb - tlo) * 16 + 4 * hq);
      } else {
        if (bm[u].ntile >= 1) S = mass_score(bm[u].m0, trs + (bm[u].ta - tlo) * 16 + 4 * hq);
        if (bm[u].ntile >= 2) S += mass_score(bm[u].m1, trs + (bm[u].ta + 1 - tlo) * 16 + 4 * hq);
        for (int T = bm[u].ta + 2; T < bm[u].ta + bm[u].ntile; ++T) {  // wide blocks only
          const int jj = j - (T * 64 * a.d) / a.beta;
          const f32x4 m = *reinterpret_cast<const f32x4*>(
              a.cb + ((bkv * a.NT + T) * a.NBT + jj) * 16 + 4 * hq);
          S += mass_score(m, trs + (T - tlo) * 16 + 4 * hq);
        }
      }
      S = group_sum<4>(S);  // the four lanes of a block hold the same j
      if (hq == 0 && j < j1) Ss[j - j0] = S;
    }
  } else {
    for (int j = j0 + tid; j < j1; j += kSelThreads) Ss[j - j0] = 0.f;
  }
  lds_barrier();
  for (int j = j0 + tid; j < j1; j += kSelThreads) a.sS[bkv * a.NSL * a.SB + j] = Ss[j - j0];
  if (wave == 0) {
    const int lo = j0 > 1 ? j0 : 1;
    const int hi = j1 < r.flo ? j1 : r.flo;  // free blocks: 1 .. flo - 1
    const uint64_t key =
        wave_topk([&](int j) { return rank_key(Ss[j - j0], j); }, lo, hi, a.KF, lane);
    if (lane < a.KF) a.cand[(bkv * a.NSL + s) * a.KF + lane] = key;
  }
}

// Selection slices of every group (see select_slice).
template <int D, bool FAST>
__global__ __launch_bounds__(kSelThreads) void dec_select_kernel(DecodeArgs a) {
  __shared__ __align__(16) unsigned char smem[(16 + kSliceTiles * 16 + 256) * 4 +
                                               kSelThreads * 16];
  const int kvh = blockIdx.y, b = blockIdx.z;
  select_slice<D, FAST>(a, (long)b * a.Hkv + kvh, b, blockIdx.x, smem);
}

// ------------------------------------------------------------------ phase 3: tiles, then merge

constexpr int kTileWaves = kSelWaves;  // waves of a tile workgroup (write_record's count)
constexpr int kTileThreads = kSelThreads;

// The rest of a group's step, after the slices, spread over NG workgroups per group in two
// kinds.  The first NGW take the tiles known before the selection -- the window's, then the
// forced blocks' outside it (or every tile when all blocks fit) -- and start on them at once.
// The others merge the slices' candidates into the top-n (forced blocks added; the first of
// them writes the ascending row out) and take the other selected blocks' tiles, inside the
// window or not, for the selected branch only.  Within a kind, wave w of its workgroup g takes
// entries g W + w, g W + w + n W, ... (a fixed assignment, so the output is reproducible bit
// for bit); per branch the workgroup's waves are merged into one record (maxima, sums,
// outputs relative to the maxima).
template <int D>
__global__ __launch_bounds__(kTileThreads) void dec_tiles_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  u16(*Qs)[D + 8] = reinterpret_cast<u16(*)[D + 8]>(smem);
  int* list = reinterpret_cast<int*>(smem + 16 * (D + 8) * 2);
  unsigned char* region = smem + 16 * (D + 8) * 2 + kDecodeMaxList * 4;
  u16(*Vt)[D][64] = reinterpret_cast<u16(*)[D][64]>(region);
  __shared__ int sidx[64];
  __shared__ int n_s;
  const int ng = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const long bkv = (long)b * a.Hkv + kvh;
  const DecRow r = dec_row(a, b);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int e = tid; e < 16 * (D / 8); e += kTileThreads) {
    const int qh = e / (D / 8), qc = (e % (D / 8)) * 8;
    *reinterpret_cast<bf16x8*>(&Qs[qh][qc]) =
        qh < a.G ? load8(a.q + ((long)b * a.Hkv * a.G + kvh * a.G + qh) * D + qc) : zero8();
  }
  const bool fixed_kind = ng < a.NGW;  // uniform per workgroup
  if (fixed_kind) {
    // the window's and forced blocks' tiles (all tiles when every block fits)
    if (wave == 0) {
      const int nf = fixed_tile_list(a, r, list, lane);
      if (lane == 0) n_s = nf;
    }
    __syncthreads();
  } else {
    // the slices' candidates into LDS (the region the tiles use later), loads issued together
    uint64_t* ck = reinterpret_cast<uint64_t*>(region);
    const int nsl = (r.nb + a.SB - 1) / a.SB;
    if (!r.all) {
      const uint64_t* cb = a.cand + bkv * a.NSL * a.KF;
      for (int i = tid; i < nsl * a.KF; i += kTileThreads) ck[i] = cb[i];
    }
    __syncthreads();
    if (wave == 0) {
      const bool writer = ng == a.NGW;
      int32_t* orow = a.idx + bkv * a.top_n;
      int base = 0;
      if (r.all) {
        if (lane < a.top_n && writer) orow[lane] = lane < r.nb ? lane : -1;
      } else {
        uint64_t key = wave_topk([&](int i) { return ck[i]; }, 0, nsl * a.KF, r.kfree, lane);
        if (r.top_p) {
          const float* S = a.sS + bkv * a.NSL * a.SB;
          float forced = S[0];
          for (int j = r.flo; j <= r.bcur; ++j) forced += S[j];
          key = top_p_cut(key, r.kfree, forced, r.nvis > 0 ? a.top_p * (float)a.G : 0.f, lane);
        }
        int el = key != 0 ? rank_key_index(key) : 0x7FFFFFFF;
        if (lane >= r.kfree) el = 0x7FFFFFFF;
        if (lane == r.kfree) el = 0;
        if (lane > r.kfree && lane <= r.kfree + r.bcur - r.flo + 1) el = r.flo + (lane - r.kfree - 1);
        int rank = 0;
        for (int o = 0; o < a.top_n; ++o)  // the whole wave is active here
          rank += (__builtin_amdgcn_readlane(el, o) < el) ? 1 : 0;
        const bool valid = lane < a.top_n && el != 0x7FFFFFFF;
        const int nsel = (int)__popcll(__ballot(valid));
        if (valid) {
          if (writer) orow[rank] = el;
          sidx[rank] = el;
        }
        if (lane >= nsel && lane < a.top_n) {
          if (writer) orow[lane] = -1;
          sidx[lane] = -1;
        }
        __asm__ volatile("" ::: "memory");  // sidx written by this wave before its reads
        // the tiles of the selected blocks other than the forced ones, for the selected branch
        const int per = a.beta / 64, ns = a.top_n * per, tl = r.t / 64;
        for (int i0 = 0; i0 < ns; i0 += 64) {
          const int i = i0 + lane;
          int code = -1;
          if (i < ns) {
            const int jb = sidx[i / per], tile = jb * per + i % per;
            const bool forced = jb == 0 || (jb >= r.flo && jb <= r.bcur);
            if (jb >= 0 && !forced && tile <= tl) code = (int)(tile | kCodeSlc);
          }
          const uint64_t m = __ballot(code >= 0);
          const int pos = base + (int)__popcll(m & ((1ull << lane) - 1ull));
          if (code >= 0) list[pos] = code;
          base += (int)__popcll(m);
        }
      }
      if (lane == 0) n_s = base;
    }
    __syncthreads();  // the list is posted and the candidates' LDS is free for the tiles
  }
  const int n = __builtin_amdgcn_readfirstlane(n_s);
  const int g0 = fixed_kind ? ng : ng - a.NGW;                 // this workgroup's index in its kind
  const int gn = fixed_kind ? a.NGW : a.NG - a.NGW;           // workgroups of its kind
  WaveSoftmax<D, 2> st;
  wave_tiles<D, 2>(a, bkv, r, list, n, g0 * kTileWaves + wave, gn * kTileWaves, Qs, Vt[wave],
                   st);
  float* rec = a.grec + (bkv * a.NG + ng) * 2 * (32 + 16 * D);
  write_record<D, 2>(st, 0, a.scale_log2, reinterpret_cast<float*>(region), rec);
  write_record<D, 2>(st, 1, a.scale_log2, reinterpret_cast<float*>(region), rec + 32 + 16 * D);
}

// Per group: the NG tile workgroups' records of each branch merged in workgroup order, then
// the gate: out = g0 o_cmp + g1 o_slc + g2 o_win (o_cmp normalised by the selection slices).
// Every thread issues its loads of the records' outputs, the compressed output and the gates
// first; meanwhile threads 0..31 turn the records' maxima and sums into per-(branch, head)
// weights.  A group's (head, feature) outputs are split over kMergeSplit workgroups (each
// computes the weights itself), so that a small batch still spreads its merge over the GPU.
constexpr int kMergeMaxNG = 8;
constexpr int kMergeSplit = 4;

template <int D>
__global__ __launch_bounds__(256) void dec_merge_kernel(DecodeArgs a) {
  constexpr int RS = 32 + 16 * D;  // floats of one record
  constexpr int PW = 16 * D / kMergeSplit;  // (head, feature) pairs per workgroup
  constexpr int PT = PW / 256;               // ... per thread
  static_assert(PT * 256 * kMergeSplit == 16 * D, "pairs must split evenly");
  __shared__ float W[2][16][kMergeMaxNG];  // weight of record g relative to the common max, / L
  const int kvh = blockIdx.x, b = blockIdx.y, p0 = blockIdx.z * PW;
  const long bkv = (long)b * a.Hkv + kvh;
  const float* recs = a.grec + bkv * a.NG * 2 * RS;
  const int tid = threadIdx.x;
  // the compressed output and the gates do not depend on the weights: loaded first
  float oc[PT], g3[PT][3];
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    const int pr = p0 + tid + 256 * q, h = pr / D, dd = pr % D;
    const int hc = h < a.G ? h : 0;  // rows past G read head 0 (in bounds) and write nothing
    const long head = (long)b * a.Hkv * a.G + kvh * a.G + hc;
    oc[q] = a.ocmp[(bkv * 16 + h) * D + dd];
#pragma unroll
    for (int c = 0; c < 3; ++c) g3[q][c] = a.gate[head * 3 + c];
  }
  // the records' outputs do not depend on the weights either: in flight across the barrier
  float ro[kMergeMaxNG][2][PT];
#pragma unroll
  for (int g = 0; g < kMergeMaxNG; ++g) {
    const int gc = g < a.NG ? g : a.NG - 1;  // unconditional loads: the record index clamped
#pragma unroll
    for (int br = 0; br < 2; ++br)
#pragma unroll
      for (int q = 0; q < PT; ++q)
        ro[g][br][q] = recs[(gc * 2 + br) * RS + 32 + p0 + tid + 256 * q];
  }
  if (tid < 32) {
    const int br = tid >> 4, h = tid & 15;
    // every record's maximum and sum loaded unconditionally (record index clamped), together
    float m[kMergeMaxNG], sm[kMergeMaxNG];
#pragma unroll
    for (int g = 0; g < kMergeMaxNG; ++g) {
      const float* rg = recs + ((g < a.NG ? g : a.NG - 1) * 2 + br) * RS;
      m[g] = rg[h];
      sm[g] = rg[16 + h];
    }
    float M = kNegInf;
#pragma unroll
    for (int g = 0; g < kMergeMaxNG; ++g) {
      m[g] = g < a.NG ? m[g] : kNegInf;
      M = fmaxf(M, m[g]);
    }
    float L = 0.f, w[kMergeMaxNG];
#pragma unroll
    for (int g = 0; g < kMergeMaxNG; ++g) {
      w[g] = m[g] == kNegInf ? 0.f : fast_exp2(m[g] - M);
      L += g < a.NG ? w[g] * sm[g] : 0.f;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int g = 0; g < kMergeMaxNG; ++g) W[br][h][g] = w[g] * inv;
  }
  __syncthreads();
  float acc[PT][2];
#pragma unroll
  for (int q = 0; q < PT; ++q) acc[q][0] = acc[q][1] = 0.f;
#pragma unroll
  for (int g = 0; g < kMergeMaxNG; ++g) {
    if (g >= a.NG) break;  // uniform
#pragma unroll
    for (int br = 0; br < 2; ++br) {
#pragma unroll
      for (int q = 0; q < PT; ++q) {
        const int pr = p0 + tid + 256 * q, h = pr / D;
        acc[q][br] += W[br][h][g] * ro[g][br][q];
      }
    }
  }
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    const int pr = p0 + tid + 256 * q, h = pr / D, dd = pr % D;
    if (h >= a.G) continue;
    const long head = (long)b * a.Hkv * a.G + kvh * a.G + h;
    a.out[head * D + dd] = g3[q][0] * oc[q] + g3[q][1] * acc[q][0] + g3[q][2] * acc[q][1];
  }
}

// ------------------------------------------------------------------ launcher

int decode_chunk_tokens() { return CHUNK; }

// Dynamic LDS of a tile workgroup: the group's queries, its tile list, and one V^T tile per
// wave (the candidates before, the records' merge after reuse the tiles' space).
static size_t tile_lds(int D) {
  const size_t tiles = (size_t)kTileWaves * D * 64 * 2;
  const size_t merge = (size_t)kTileWaves * 16 * (D + 4) * 4;
  const size_t cand = (size_t)decode_max_candidates(D) * 8;
  size_t region = tiles > merge ? tiles : merge;
  region = region > cand ? region : cand;
  return (size_t)16 * (D + 8) * 2 + kDecodeMaxList * 4 + region;
}

template <int D, bool FAST>
static void launch_decode_t(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  auto mark = [&](int i) {
    if (ev != nullptr) (void)hipEventRecord(ev[i], s);
  };
  const size_t lds = tile_lds(D);
  // opt in to the dynamic LDS beyond 64 KB; the attribute is per device, so it is set on every
  // launch
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dec_tiles_kernel<D>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  mark(0);
  if (a.NCH > 0) dec_cmp_kernel<D, FAST><<<dim3(a.NCH, a.Hkv, a.B), 256, 0, s>>>(a);
  mark(1);
  dec_select_kernel<D, FAST><<<dim3(a.NSL, a.Hkv, a.B), kSelThreads, 0, s>>>(a);
  mark(2);
  dec_tiles_kernel<D><<<dim3(a.NG, a.Hkv, a.B), kTileThreads, lds, s>>>(a);
  mark(3);
  dec_merge_kernel<D><<<dim3(a.Hkv, a.B, kMergeSplit), 256, 0, s>>>(a);
  mark(4);
}

void launch_decode(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  const bool fast = a.beta == 4 * a.d && a.l == 2 * a.d && a.NBT >= 17;
  if (a.D == 128) {
    if (fast) launch_decode_t<128, true>(a, s, ev);
    else launch_decode_t<128, false>(a, s, ev);
  } else {
    if (fast) launch_decode_t<64, true>(a, s, ev);
    else launch_decode_t<64, false>(a, s, ev);
  }
}

}  // namespace nsa
