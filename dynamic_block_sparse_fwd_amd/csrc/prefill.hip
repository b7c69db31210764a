// NSA prefill kernels ("Zhang Xiaojun podcast EP94 notes", sections 5 and 6):
//   cmp_select_kernel: compressed attention + block importance + group top-n selection;
//   window_kernel:     sliding-window attention;
//   selected_kernel:   attention over the selected blocks, the group's heads stacked into the
//                      matrix-core M dimension (section 6: heads of a GQA group share one
//                      selection, so their queries form one tile against each block).
// The gate mix is folded into the three output writes: cmp stores g0*o_cmp, window and
// selected add g2*o_win and g1*o_slc.
#include "attn_tile.h"
#include "dev_common.h"
#include "kernels.h"

namespace nsa {

// Query tile geometry shared by the compressed and window kernels: TQ positions x G heads
// = ROWS matrix rows, 16 rows per MFMA tile, up to two tiles per wave.
template <int G>
struct QTile {
  static constexpr int TQ = (16 / G > 8) ? 16 / G : 8;
  static constexpr int ROWS = TQ * G;
  static constexpr int RT_ALL = ROWS / 16;
  static constexpr int NW = RT_ALL >= 2 ? RT_ALL / 2 : 1;
  static constexpr int RTW = RT_ALL / NW;
};

template <int D, int G>
__device__ __forceinline__ void load_q_frags(const PrefillArgs& a, int b, int kvh, int t0,
                                             int wave, int lane, bf16x8 (*qf)[D / 32],
                                             int* row_t, int* row_h) {
  using QT = QTile<G>;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int Hq = a.Hkv * G;
#pragma unroll
  for (int rt = 0; rt < QT::RTW; ++rt) {
    const int r = (wave * QT::RTW + rt) * 16 + r16;
    const int t = t0 + r / G, hh = r % G;
    row_t[rt] = t;
    row_h[rt] = kvh * G + hh;
    const bool live = t < a.T;
    const u16* qp = a.q + (prow(a, b, live ? t : a.q0) * Hq + kvh * G + hh) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qf[rt][c] = live ? load8(qp + 32 * c + 8 * g4) : zero8();
  }
}

// ------------------------------------------------------------------ compressed + selection

// Block importance, fast geometry (sel_block = 4 * stride, cmp_len = 2 * stride): block j
// receives p(4j-1)/2 + p(4j) + p(4j+1) + p(4j+2) + p(4j+3)/2.  A lane holds the 8 keys
// 8*g4 .. 8*g4+7 of a 32-key chunk, i.e. the "core" p(4j) + p(4j+1) + p(4j+2) + p(4j+3)/2 of
// two blocks and the half-key carries p(4j+3)/2 into the next block; cores and carries are
// summed over the group's heads, and every block is assembled as core + carry in the same
// order (exact ties stay exact).
template <int G>
__device__ __forceinline__ float head_sum(float v) {
  if constexpr (G >= 16) return row16_sum(v);
  else return group_sum<G>(v);
}

template <int D, int G, bool FAST>
__global__ __launch_bounds__(QTile<G>::NW * 64, G == 16 ? 2 : 1) void cmp_select_kernel(PrefillArgs a) {
  using QT = QTile<G>;
  constexpr int NT = QT::NW * 64, TQ = QT::TQ, RTW = QT::RTW, DT = D / 16;
  __shared__ u16 Ks[64][D];
  __shared__ u16 Vs[D][64];
  __shared__ float Mb[FAST ? 1 : TQ][64];   // generic path: group mass per (t, key)
  __shared__ float Cb[FAST ? TQ : 1][16];   // fast path: block cores of the tile
  __shared__ float Hb[FAST ? TQ : 1][17];   // fast path: half-key carries into blocks 0..16
  __shared__ float Pc[TQ];                  // fast path: carry into the tile's first block
  extern __shared__ float Sb[];             // [TQ][nblk] group block scores

  const int tile = gridDim.x - 1 - blockIdx.x;  // longest rows first
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int t0 = a.q0 + tile * TQ;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const long bkv = (long)b * a.Hkv + kvh;
  const int nblk = a.nblk;
  const float sl = a.scale_log2;

  bf16x8 qf[RTW][D / 32];
  int row_t[RTW], row_h[RTW], nvis[RTW];
  load_q_frags<D, G>(a, b, kvh, t0, wave, lane, qf, row_t, row_h);
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
    nvis[rt] = row_t[rt] < a.T ? n_visible(row_t[rt], a.l, a.d, a.ncmp) : 0;

  const int tlast = (t0 + TQ - 1 < a.T - 1) ? t0 + TQ - 1 : a.T - 1;
  const int nvis_max = n_visible(tlast, a.l, a.d, a.ncmp);
  // keys below nvis_lo are visible to every row of the tile (rows past T see none)
  const int nvis_lo = (t0 + TQ - 1 < a.T) ? n_visible(t0, a.l, a.d, a.ncmp) : 0;
  const int nkt = (nvis_max + 63) / 64;
  const u16* kc = a.kc + bkv * (long)a.NCP * D;
  const u16* vct = a.vct + bkv * (long)D * a.NCP;

  for (int e = threadIdx.x; e < TQ * nblk; e += NT) Sb[e] = 0.f;
  if (threadIdx.x < TQ) Pc[threadIdx.x] = 0.f;

  // Pass 1: per-row max and sum of exp2 (per lane; merged over the row's four lanes below).
  float mrun[RTW], lrun[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) { mrun[rt] = kNegInf; lrun[rt] = 0.f; }
  KTileRegs<D, NT> kr;
  VTileRegs<D, NT> vr;
  if (nkt > 0) kr.load(kc, 0, a.NCP - 1);
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    kr.store(Ks);
    __syncthreads();
    if (kt + 1 < nkt) kr.load(kc, (long)(kt + 1) * 64, a.NCP - 1);
    const bool full = (kt + 1) * 64 <= nvis_lo;
    float raw[RTW][16];
    score_tiles<D, RTW>(Ks, qf, g4, r16, raw);
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      if (!full) {  // a real (uniform) branch: full tiles skip the masking arithmetic
        __asm__ volatile("" ::: "memory");
        // key kt*64 + 32*(e>>3) + 8*g4 + (e&7) is visible iff its offset from the lane's first
        // key is below lim (one subtraction per lane, constant offsets per element)
        const int lim = nvis[rt] - (kt * 64 + 8 * g4);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          raw[rt][e] = 32 * (e >> 3) + (e & 7) < lim ? raw[rt][e] : kNegInf;
      }
      float tm = raw[rt][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) tm = fmaxf(tm, raw[rt][e]);
      const float mn = fmaxf(mrun[rt], tm);
      if (mn != kNegInf) {
        const float msl = mn * sl;
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += fast_exp2(fmaf(raw[rt][e], sl, -msl));
        lrun[rt] = lrun[rt] * fast_exp2(fmaf(mrun[rt], sl, -msl)) + sum;
        mrun[rt] = mn;
      }
    }
  }
  // Row log-sum-exp (scaled, log2 units): pass 2 computes the normalised probabilities
  // p = exp2(z - lse) directly, for the block importance (fp32) and the P V product (bf16).
  float rlse[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const float M = col_max4(mrun[rt]);
    const float part = (mrun[rt] == kNegInf) ? 0.f : lrun[rt] * fast_exp2((mrun[rt] - M) * sl);
    const float L = col_sum4(part);
    rlse[rt] = (M == kNegInf) ? 0.f : M * sl + __log2f(L);  // no visible key: p masked to 0
  }

  f32x4 O[RTW][DT];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int n = 0; n < DT; ++n) O[rt][n] = zero4();
  const int Hq = a.Hkv * G;
  // The epilogue multiplies O by ef = g0.  Fused, O first receives the window output times
  // g2 / ef, so that out = g0 * o_cmp + g2 * o_win is written once and never read; a row with
  // g0 = 0 keeps the window output as is (ef taken as 1) and drops p from the P V product
  // (ps = 0).
  float ps[RTW], ef[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int t = row_t[rt];
    const float g0 =
        t < a.T ? a.gate[(prow(a, b, t) * Hq + row_h[rt]) * 3 + 0] : 0.f;
    const bool zero = a.fuse_window && g0 == 0.f;
    ps[rt] = zero ? 0.f : 1.f;
    ef[rt] = zero ? 1.f : g0;
  }
  if (a.fuse_window) {  // uniform: sliding window over the raw K/V, same query tile
    const int tlast = (t0 + TQ - 1 < a.T - 1) ? t0 + TQ - 1 : a.T - 1;
    const int kstart = t0 - a.window + 1 > 0 ? t0 - a.window + 1 : 0;
    const int kw0 = kstart / 64, kw1 = tlast / 64;
    const bool alive = t0 + TQ - 1 < a.T;
    const u16* kb = a.k + bkv * (long)a.ldk * D;
    const u16* vtb = a.vt + bkv * (long)D * a.TP;
    float wm[RTW], wl[RTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) { wm[rt] = kNegInf; wl[rt] = 0.f; }
    kr.load(kb, (long)kw0 * 64, a.T - 1);
    vr.load(vtb, a.TP, (long)kw0 * 64);
    for (int kt = kw0; kt <= kw1; ++kt) {
      __syncthreads();
      kr.store(Ks);
      vr.store(Vs);
      __syncthreads();
      if (kt < kw1) {
        kr.load(kb, (long)(kt + 1) * 64, a.T - 1);
        vr.load(vtb, a.TP, (long)(kt + 1) * 64);
      }
      // keys of this tile are inside every row's window unless the tile touches either end
      const bool wfull = alive && kt * 64 >= tlast - a.window + 1 && kt * 64 + 63 <= t0;
      float raw[RTW][16];
      score_tiles<D, RTW>(Ks, qf, g4, r16, raw);
      bf16x8 pb[RTW][2];
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
        const int t = row_t[rt];
        const int lo = t - a.window + 1;
        if (!wfull) {
          __asm__ volatile("" ::: "memory");
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kt * 64 + 32 * (e >> 3) + 8 * g4 + (e & 7);
            raw[rt][e] = (key <= t && key >= lo && t < a.T) ? raw[rt][e] : kNegInf;
          }
        }
        float tm = raw[rt][0];
#pragma unroll
        for (int e = 1; e < 16; ++e) tm = fmaxf(tm, raw[rt][e]);
        tm = col_max4(tm);
        // lazy rescale: the reference moves only past kLazyLog2 of headroom (a row with no key
        // yet has reference -inf and moves on its first key)
        const bool move = tm * sl > wm[rt] * sl + kLazyLog2;
        if (__ballot(move) != 0) {  // uniform
          const float mn = move ? tm : wm[rt];
          const float alpha = move ? fast_exp2((wm[rt] - mn) * sl) : 1.f;
          wm[rt] = mn;
          wl[rt] *= alpha;
#pragma unroll
          for (int n = 0; n < DT; ++n) O[rt][n] *= alpha;
        }
        const float msl = (wm[rt] == kNegInf) ? 0.f : wm[rt] * sl;
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(fmaf(raw[rt][e], sl, -msl));
          sum += p;
          pb[rt][e >> 3][e & 7] = (__bf16)p;
        }
        wl[rt] += sum;
      }
      pv_tiles<D, RTW>(Vs, pb, g4, r16, O);
    }
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const float L = col_sum4(wl[rt]);
      const int t = row_t[rt];
      const float g2 =
          t < a.T ? a.gate[(prow(a, b, t) * Hq + row_h[rt]) * 3 + 2] : 0.f;
      const float f = L > 0.f ? g2 / (L * ef[rt]) : 0.f;
#pragma unroll
      for (int n = 0; n < DT; ++n) O[rt][n] *= f;
    }
  }

  bool ps_zero = false;
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) ps_zero |= ps[rt] == 0.f;
  ps_zero = __ballot(ps_zero) != 0;  // wave-uniform
  // Pass 2: normalised probabilities -> o_cmp and group block scores.
  const float inv_l = 1.0f / (float)a.l;
  if (nkt > 0) {
    kr.load(kc, 0, a.NCP - 1);
    vr.load(vct, a.NCP, 0);
  }
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    kr.store(Ks);
    vr.store(Vs);
    __syncthreads();
    if (kt + 1 < nkt) {
      kr.load(kc, (long)(kt + 1) * 64, a.NCP - 1);
      vr.load(vct, a.NCP, (long)(kt + 1) * 64);
    }
    const bool full = (kt + 1) * 64 <= nvis_lo;
    float raw[RTW][16];
    score_tiles<D, RTW>(Ks, qf, g4, r16, raw);
    bf16x8 pbt[RTW][2];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int r = (wave * RTW + rt) * 16 + r16;
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(raw[rt][kc2 * 8 + e], sl, -rlse[rt]));
        if (!full) {
          __asm__ volatile("" ::: "memory");
          const int lim = nvis[rt] - (kt * 64 + 32 * kc2 + 8 * g4);  // key offsets e < lim
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = e < lim ? pv[e] : 0.f;
        }
        if (ps_zero) {  // uniform: a row of this wave drops p' from P V (rare)
#pragma unroll
          for (int e = 0; e < 8; ++e) pbt[rt][kc2][e] = (__bf16)(pv[e] * ps[rt]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) pbt[rt][kc2][e] = (__bf16)pv[e];
        }
        if constexpr (FAST && G == 16) {
          const float cA = (pv[0] + pv[1]) + pv[2] + 0.5f * pv[3];
          const float cB = (pv[4] + pv[5]) + pv[6] + 0.5f * pv[7];
          const float h3 = 0.5f * pv[3];
          const float h7 = 0.5f * pv[7];
          // the four sums over the row's 16 lanes (the group's heads) at once: each step pairs
          // lanes that keep complementary halves of the values and adds what the partner sends;
          // lane r16 ends with the sum of value r16 / 4 (cA, cB, h3, h7), every block through
          // the same association
          const bool hi = r16 >= 8, b2 = (r16 & 4) != 0;
          float x = hi ? h3 : cA, u = hi ? h7 : cB;
          x += dpp_f<kDppMirror>(hi ? cA : h3);  // partner 15 - r16
          u += dpp_f<kDppMirror>(hi ? cB : h7);
          float v = b2 ? u : x;
          v += dpp_f<kDppHalfMirror>(b2 ? x : u);  // partner 7 - r16 of its half
          v += xor_lane_f<2>(v);
          v += xor_lane_f<1>(v);
          if ((r16 & 3) == 0) {
            const int tq = r / G, jl = 8 * kc2 + 2 * g4, which = r16 >> 2;
            float* dst = which < 2 ? &Cb[tq][jl + which] : &Hb[tq][jl + which - 1];
            *dst = v;
          }
        } else if constexpr (FAST) {
          const float cA = head_sum<G>((pv[0] + pv[1]) + pv[2] + 0.5f * pv[3]);
          const float cB = head_sum<G>((pv[4] + pv[5]) + pv[6] + 0.5f * pv[7]);
          const float h3 = head_sum<G>(0.5f * pv[3]);
          const float h7 = head_sum<G>(0.5f * pv[7]);
          if ((r16 % G) == 0) {
            const int tq = r / G, jl = 8 * kc2 + 2 * g4;
            Cb[tq][jl] = cA;
            Cb[tq][jl + 1] = cB;
            Hb[tq][jl + 1] = h3;
            Hb[tq][jl + 2] = h7;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float hs = head_sum<G>(pv[e]);
            if ((r16 % G) == 0) Mb[r / G][32 * kc2 + 8 * g4 + e] = hs;
          }
        }
      }
    }
    pv_tiles<D, RTW>(Vs, pbt, g4, r16, O);
    __syncthreads();
    if constexpr (FAST) {
      // blocks 16*kt .. 16*kt + 15 are complete: core + carry (the carry of the first block
      // comes from the previous tile)
      for (int pr = threadIdx.x; pr < TQ * 16; pr += NT) {
        const int tq = pr >> 4, jl = pr & 15, j = 16 * kt + jl;
        if (t0 + tq >= a.T || j >= nblk) continue;
        const float carry = jl == 0 ? Pc[tq] : Hb[tq][jl];
        Sb[tq * nblk + j] = Cb[tq][jl] + carry;
        if (jl == 0) Pc[tq] = Hb[tq][16];
      }
    } else {
      // compressed token i covers tokens [i*d, i*d + l); its mass is spread evenly over those
      // tokens and summed per block of `beta` tokens; terms are added one by one in key order
      const int k0 = kt * 64;
      const int jlo = (k0 * a.d) / a.beta;
      int jhi = ((k0 + 63) * a.d + a.l - 1) / a.beta;
      if (jhi > nblk - 1) jhi = nblk - 1;
      const int nj = jhi - jlo + 1;
      for (int pr = threadIdx.x; pr < TQ * nj; pr += NT) {
        const int tq = pr / nj, j = jlo + pr % nj;
        if (t0 + tq >= a.T) continue;
        const int bs = j * a.beta, be = bs + a.beta;
        int ilo = bs - a.l + 1 <= 0 ? 0 : (bs - a.l + 1 + a.d - 1) / a.d;
        if (ilo < k0) ilo = k0;
        int ihi = (be - 1) / a.d;
        if (ihi > k0 + 63) ihi = k0 + 63;
        float sv = Sb[tq * nblk + j];
        for (int i = ilo; i <= ihi; ++i) {
          const int s0 = i * a.d, s1 = s0 + a.l;
          const int ov = (s1 < be ? s1 : be) - (s0 > bs ? s0 : bs);
          if (ov > 0) sv += Mb[tq][i - k0] * ((float)ov * inv_l);
        }
        Sb[tq * nblk + j] = sv;
      }
    }
  }
  if constexpr (FAST) {
    __syncthreads();
    // the block after the last tile only has its carry
    if (threadIdx.x < TQ && t0 + (int)threadIdx.x < a.T && 16 * nkt < nblk && nkt > 0)
      Sb[threadIdx.x * nblk + 16 * nkt] = 0.f + Pc[threadIdx.x];
  }

  // epilogue: out = g0 * o_cmp (+ g2 * o_win fused).  Lane holds O^T[d = 16n + 4*g4 + e][row
  // r16].
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int t = row_t[rt];
    if (t < a.T) {
      const long rowoff = prow(a, b, t) * Hq + row_h[rt];
      const float g0 = ef[rt];
      float* op = a.out + rowoff * D;
#pragma unroll
      for (int n = 0; n < DT; ++n) {
        float4 v = make_float4(g0 * O[rt][n][0], g0 * O[rt][n][1], g0 * O[rt][n][2],
                               g0 * O[rt][n][3]);
        *reinterpret_cast<float4*>(op + 16 * n + 4 * g4) = v;
      }
    }
  }
  __syncthreads();

  // Selection: one wave per position.  Free candidates are ranked by a 64-bit key
  // (score bits << 32 | ~index): larger score first, then lower index.
  const bool top_p = a.top_p > 0.f;
  for (int tq = wave; tq < TQ; tq += QT::NW) {
    const int t = t0 + tq;
    if (t >= a.T) break;
    const int bcur = t / a.beta, nb = bcur + 1;
    int32_t* orow = a.idx + (prow(a, b, t) * a.Hkv + kvh) * a.top_n;
    if (nb <= a.top_n && !top_p) {
      for (int e = lane; e < a.top_n; e += 64) orow[e] = e < nb ? e : -1;
      continue;
    }
    // forced: block 0 and the local blocks flo..bcur; free candidates 1 .. flo-1
    const int flo = bcur - a.n_local + 1 > 1 ? bcur - a.n_local + 1 : 1;
    const int kfree = a.top_n - 1 - a.n_local;
    const float* srow = Sb + tq * nblk;
    // lane e < kfree receives the e-th winner among the free blocks (0 past the last one)
    uint64_t key = wave_topk([&](int j) { return rank_key(srow[j], j); }, 1, flo, kfree, lane);
    if (top_p) {
      float forced = srow[0];
      for (int j = flo; j <= bcur; ++j) forced += srow[j];
      const bool seen = t >= a.l - 1;  // a compressed token is visible: total importance G
      key = top_p_cut(key, kfree, forced, seen ? a.top_p * (float)a.G : 0.f, lane);
    }
    // the set: lanes 0..kfree-1 hold winners; next lanes hold block 0 and flo..bcur
    int el = key != 0 ? rank_key_index(key) : 0x7FFFFFFF;
    if (lane == kfree) el = 0;
    if (lane > kfree && lane <= kfree + bcur - flo + 1) el = flo + (lane - kfree - 1);
    int rank = 0;
    for (int o = 0; o < a.top_n; ++o) {
      const int other = __builtin_amdgcn_readlane(el, o);  // the whole wave is active here
      rank += (other < el) ? 1 : 0;
    }
    const bool valid = lane < a.top_n && el != 0x7FFFFFFF;
    const int nsel = (int)__popcll(__ballot(valid));
    if (valid) orow[rank] = el;
    if (lane >= nsel && lane < a.top_n) orow[lane] = -1;
  }
}

// ------------------------------------------------------------------ sliding window

template <int D, int G>
__global__ __launch_bounds__(QTile<G>::NW * 64) void window_kernel(PrefillArgs a) {
  using QT = QTile<G>;
  constexpr int NT = QT::NW * 64, TQ = QT::TQ, RTW = QT::RTW, DT = D / 16;
  __shared__ u16 Ks[64][D];
  __shared__ u16 Vs[D][64];

  const int tile = blockIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int t0 = a.q0 + tile * TQ;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const long bkv = (long)b * a.Hkv + kvh;
  const float sl = a.scale_log2;

  bf16x8 qf[RTW][D / 32];
  int row_t[RTW], row_h[RTW];
  load_q_frags<D, G>(a, b, kvh, t0, wave, lane, qf, row_t, row_h);

  const int tlast = (t0 + TQ - 1 < a.T - 1) ? t0 + TQ - 1 : a.T - 1;
  const int kstart = t0 - a.window + 1 > 0 ? t0 - a.window + 1 : 0;
  const int kt0 = kstart / 64, kt1 = tlast / 64;
  const bool alive = t0 + TQ - 1 < a.T;
  const u16* kb = a.k + bkv * (long)a.ldk * D;
  const u16* vtb = a.vt + bkv * (long)D * a.TP;

  float mrun[RTW], lrun[RTW];
  f32x4 O[RTW][DT];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    mrun[rt] = kNegInf;
    lrun[rt] = 0.f;
#pragma unroll
    for (int n = 0; n < DT; ++n) O[rt][n] = zero4();
  }

  KTileRegs<D, NT> kr;
  VTileRegs<D, NT> vr;
  kr.load(kb, (long)kt0 * 64, a.T - 1);
  vr.load(vtb, a.TP, (long)kt0 * 64);
  for (int kt = kt0; kt <= kt1; ++kt) {
    __syncthreads();
    kr.store(Ks);
    vr.store(Vs);
    __syncthreads();
    if (kt < kt1) {
      kr.load(kb, (long)(kt + 1) * 64, a.T - 1);
      vr.load(vtb, a.TP, (long)(kt + 1) * 64);
    }
    // keys of this tile are inside every row's window unless the tile touches either end
    const bool full = alive && kt * 64 >= tlast - a.window + 1 && kt * 64 + 63 <= t0;
    float raw[RTW][16];
    score_tiles<D, RTW>(Ks, qf, g4, r16, raw);
    bf16x8 pb[RTW][2];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int t = row_t[rt];
      const int lo = t - a.window + 1;
      if (!full) {
        __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kt * 64 + 32 * (e >> 3) + 8 * g4 + (e & 7);
          raw[rt][e] = (key <= t && key >= lo && t < a.T) ? raw[rt][e] : kNegInf;
        }
      }
      float tm = raw[rt][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) tm = fmaxf(tm, raw[rt][e]);
      tm = col_max4(tm);
      // lazy rescale: the reference moves only past kLazyLog2 of headroom
      const bool move = tm * sl > mrun[rt] * sl + kLazyLog2;
      if (__ballot(move) != 0) {  // uniform
        const float mn = move ? tm : mrun[rt];
        const float alpha = move ? fast_exp2((mrun[rt] - mn) * sl) : 1.f;
        mrun[rt] = mn;
        lrun[rt] *= alpha;
#pragma unroll
        for (int n = 0; n < DT; ++n) O[rt][n] *= alpha;
      }
      // A row with no visible key yet keeps m = -inf; exponentials then use 0 as reference
      // so every p is exactly 0 (no branch: the MFMAs below need the whole wave).
      const float msl = (mrun[rt] == kNegInf) ? 0.f : mrun[rt] * sl;
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(fmaf(raw[rt][e], sl, -msl));
        sum += p;
        pb[rt][e >> 3][e & 7] = (__bf16)p;
      }
      lrun[rt] += sum;
    }
    pv_tiles<D, RTW>(Vs, pb, g4, r16, O);
  }

  const int Hq = a.Hkv * G;
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const float L = col_sum4(lrun[rt]);
    const int t = row_t[rt];
    if (t < a.T) {
      const long rowoff = prow(a, b, t) * Hq + row_h[rt];
      const float gs = a.gate[rowoff * 3 + 2] / L;
      float* op = a.out + rowoff * D;
#pragma unroll
      for (int n = 0; n < DT; ++n) {
        float4* dst = reinterpret_cast<float4*>(op + 16 * n + 4 * g4);
        float4 v = *dst;
        v.x += gs * O[rt][n][0];
        v.y += gs * O[rt][n][1];
        v.z += gs * O[rt][n][2];
        v.w += gs * O[rt][n][3];
        *dst = v;
      }
    }
  }
}

// ------------------------------------------------------------------ selected blocks

// One wave per (position, KV group), eight consecutive positions of one group per workgroup:
// the group's heads form the 16 MFMA rows.  The forced blocks (block 0 and the local blocks,
// one 64-key tile each at the benchmark geometry) are common to the eight positions, so up to
// three of their tiles are staged in LDS once per workgroup; every other selected tile is
// gathered straight from global memory (16-byte loads), the next tile's K and V in flight
// while the current one computes.  A wave's tiles (in index-list order) are listed once, lane
// e holding the first key of tile e or -1 (padding, a block outside [0, nblk), a tile past t);
// tiles it shares with the workgroup are taken from LDS (as often as they occur), the rest
// are visited in order through the ballot mask.
// Workgroups are dealt to the 8 XCDs round-robin; the linear index is remapped so that XCD x
// runs a contiguous 1/8 of the (sequence, group, position) range: the waves that share an
// XCD's L2 then read the same group's K/V at nearby positions.
constexpr int kSelWaves = 8;   // positions per workgroup
constexpr int kSelShared = 3;  // tiles staged in LDS per workgroup

template <int D, int G>
__global__ __launch_bounds__(kSelWaves * 64, 1) void selected_kernel(PrefillArgs a) {
  constexpr int DT = D / 16, NK = D / 8, NV = D / 8, NT = kSelWaves * 64;
  __shared__ __align__(16) u16 Ksh[kSelShared][64][D];
  __shared__ __align__(16) u16 Vsh[kSelShared][D][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int ntb = (a.nq + kSelWaves - 1) / kSelWaves;
  const int per_xcd = gridDim.x / 8;  // the grid is padded to a multiple of 8
  const int w = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int stream = w / ntb;
  if (stream >= a.B * a.Hkv) return;  // uniform
  const int t0 = a.q0 + (w % ntb) * kSelWaves;
  const int t = t0 + wave;
  const bool act = t < a.T;
  const int kvh = stream % a.Hkv, b = stream / a.Hkv;
  const long bkv = (long)b * a.Hkv + kvh;
  const int Hq = a.Hkv * G;
  const bool hlive = r16 < G;
  const int head = kvh * G + (hlive ? r16 : 0);
  const float sl = a.scale_log2;
  const u16* kb = a.k + bkv * (long)a.ldk * D;
  const u16* vtb = a.vt + bkv * (long)D * a.TP;

  // The workgroup's shared tiles: tiles of the current block up to t0, of the other local
  // blocks, then block 0's first tile (uniform; t0 .. t0+7 share one block since the block
  // size is a multiple of 64 and t0 of 8).
  int sh[kSelShared];
  int nsh = 0;
  {
    const int bcur = t0 / a.beta, per = a.beta >> 6;
    for (int f = bcur; f >= 0 && f > bcur - a.n_local && nsh < kSelShared; --f)
      for (int u = 0; u < per && nsh < kSelShared; ++u)
        if (f * a.beta + 64 * u <= t0) sh[nsh++] = f * a.beta + 64 * u;
    if (nsh < kSelShared && bcur - a.n_local >= 0) sh[nsh++] = 0;
  }

  int my_key0 = -1;
  if (act) {
    const int per = a.beta >> 6;
    const int32_t* irow = a.idx + (prow(a, b, t) * a.Hkv + kvh) * a.top_n;
    if (lane < a.top_n * per) {
      const int j = irow[lane / per];
      const int k0 = j * a.beta + 64 * (lane % per);
      if (j >= 0 && j < a.nblk && k0 <= t) my_key0 = k0;
    }
  }
  uint64_t todo = __ballot(my_key0 >= 0);  // wave-uniform: gathered tiles still to visit
  int shcnt[kSelShared];
#pragma unroll
  for (int i = 0; i < kSelShared; ++i) {
    const uint64_t m = i < nsh ? __ballot(my_key0 == sh[i]) : 0ull;
    shcnt[i] = (int)__popcll(m);
    todo &= ~m;
  }
  const int ntile = (int)__popcll(todo);

  bf16x8 qf[D / 32];
  {
    const u16* qp = a.q + (prow(a, b, act ? t : a.q0) * Hq + head) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qf[c] = hlive ? load8(qp + 32 * c + 8 * g4) : zero8();
  }
  const int tmax = a.T - 1;
  u32x4 kr[NK], vr[NV];
  auto load_k = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int row = k0 + 32 * (q >> 1) + perm_key(r16, q & 1);
      row = row < tmax ? row : tmax;
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        kr[q * (D / 32) + c] =
            *reinterpret_cast<const u32x4*>(kb + ((uint32_t)row * D + 8 * g4 + 32 * c));
    }
  };
  auto load_v = [&](int k0) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int n = 0; n < DT; ++n)
        vr[kc * DT + n] = *reinterpret_cast<const u32x4*>(
            vtb + ((uint32_t)(16 * n + r16) * a.TP + k0 + 32 * kc + 8 * g4));
  };
  for (int i = 0; i < nsh; ++i) {  // uniform
    KTileRegs<D, NT> sk;
    VTileRegs<D, NT> sv;
    sk.load(kb, sh[i], tmax);
    sv.load(vtb, a.TP, sh[i]);
    sk.store(Ksh[i]);
    sv.store(Vsh[i]);
  }
  __syncthreads();
  if (!act) return;  // after the workgroup's only barrier
  // the first gathered tile's K is in flight while the shared tiles compute (its V follows:
  // both at once would not fit the register budget)
  int key0 = 0;
  if (ntile > 0) {
    key0 = __builtin_amdgcn_readlane(my_key0, __builtin_ctzll(todo));
    todo &= todo - 1;
  }
  load_k(key0);

  float mrun = kNegInf, lrun = 0.f;
  f32x4 O[DT];
#pragma unroll
  for (int n = 0; n < DT; ++n) O[n] = zero4();
  // masking, online softmax and the rescale of O; returns P^T fragments for the P V product
  auto softmax_step = [&](float* z, int k0, bf16x8* pb) {
    if (k0 + 63 > t) {  // the diagonal tile (uniform branch)
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + 32 * (q >> 1) + 8 * g4 + 4 * (q & 1) + e;
          z[q * 4 + e] = key <= t ? z[q * 4 + e] : kNegInf;
        }
    }
    float tm = z[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) tm = fmaxf(tm, z[e]);
    tm = col_max4(tm);  // finite: every tile used holds a key <= t
    const bool move = tm * sl > mrun * sl + kLazyLog2;
    if (__ballot(move) != 0) {  // uniform: lazy rescale
      const float mn = move ? tm : mrun;
      const float alpha = move ? fast_exp2((mrun - mn) * sl) : 1.f;
      mrun = mn;
      lrun *= alpha;
#pragma unroll
      for (int n = 0; n < DT; ++n) O[n] *= alpha;
    }
    const float msl = mrun * sl;
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = fast_exp2(fmaf(z[e], sl, -msl));
      sum += p;
      pb[e >> 3][e & 7] = (__bf16)p;
    }
    lrun += sum;
  };

  // shared tiles, from LDS
  for (int i = 0; i < nsh; ++i)
    for (int c = 0; c < shcnt[i]; ++c) {
      float z[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 acc = score_subtile<D>(Ksh[i], qf, q >> 1, q & 1, g4, r16);
#pragma unroll
        for (int e = 0; e < 4; ++e) z[q * 4 + e] = acc[e];
      }
      bf16x8 pb[2];
      softmax_step(z, sh[i], pb);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) pv_chunk<D>(Vsh[i], pb[kc], kc, g4, r16, O);
    }

  load_v(key0);

  // gathered tiles
  for (int it = 0; it < ntile; ++it) {
    // the last tile re-fetches itself: unconditional loads keep the wait counts exact (a load
    // under a branch makes the join wait for every load in flight)
    const int knext = todo ? __builtin_amdgcn_readlane(my_key0, __builtin_ctzll(todo)) : key0;
    todo &= todo - 1;
    float z[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 acc = zero4();
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        acc = mfma16x16x32(__builtin_bit_cast(bf16x8, kr[q * (D / 32) + c]), qf[c], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) z[q * 4 + e] = acc[e];
    }
    load_k(knext);
    bf16x8 pb[2];
    softmax_step(z, key0, pb);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int n = 0; n < DT; ++n)
        O[n] = mfma16x16x32(__builtin_bit_cast(bf16x8, vr[kc * DT + n]), pb[kc], O[n]);
    load_v(knext);
    key0 = knext;
  }

  const float L = col_sum4(lrun);
  if (hlive) {
    const long rowoff = prow(a, b, t) * Hq + head;
    const float gs = L > 0.f ? a.gate[rowoff * 3 + 1] / L : 0.f;
    float* op = a.out + rowoff * D;
#pragma unroll
    for (int n = 0; n < DT; ++n) {
      float4* dst = reinterpret_cast<float4*>(op + 16 * n + 4 * g4);
      float4 v = *dst;
      v.x += gs * O[n][0];
      v.y += gs * O[n][1];
      v.z += gs * O[n][2];
      v.w += gs * O[n][3];
      *dst = v;
    }
  }
}

// ------------------------------------------------------------------ launchers

template <int G>
static size_t cmp_lds(int nblk) {
  return (size_t)QTile<G>::TQ * nblk * sizeof(float);
}

size_t cmp_select_lds_bytes(int G, int nblk) {
  switch (G) {
    case 1: return cmp_lds<1>(nblk);
    case 2: return cmp_lds<2>(nblk);
    case 4: return cmp_lds<4>(nblk);
    case 8: return cmp_lds<8>(nblk);
    default: return cmp_lds<16>(nblk);
  }
}

template <int D, int G>
static void launch_prefill_all(const PrefillArgs& a, int which, hipStream_t s) {
  using QT = QTile<G>;
  const int ntile = (a.nq + QT::TQ - 1) / QT::TQ;
  if (which == 0) {
    const size_t lds = cmp_lds<G>(a.nblk);
    const bool fast = a.beta == 4 * a.d && a.l == 2 * a.d;
    // opt in to the largest dynamic LDS any launch may use (64 KB, the validated limit); the
    // attribute is per device, so it is set on every launch rather than once per process
    (void)hipFuncSetAttribute(fast ? reinterpret_cast<const void*>(&cmp_select_kernel<D, G, true>)
                                   : reinterpret_cast<const void*>(&cmp_select_kernel<D, G, false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024);
    if (fast)
      cmp_select_kernel<D, G, true><<<dim3(ntile, a.Hkv, a.B), QT::NW * 64, lds, s>>>(a);
    else
      cmp_select_kernel<D, G, false><<<dim3(ntile, a.Hkv, a.B), QT::NW * 64, lds, s>>>(a);
  } else if (which == 1) {
    window_kernel<D, G><<<dim3(ntile, a.Hkv, a.B), QT::NW * 64, 0, s>>>(a);
  } else {
    const long nwg = (long)((a.nq + kSelWaves - 1) / kSelWaves) * a.Hkv * a.B;
    selected_kernel<D, G><<<dim3((unsigned)((nwg + 7) / 8 * 8)), kSelWaves * 64, 0, s>>>(a);
  }
}

template <int D>
static void dispatch_g(const PrefillArgs& a, int which, hipStream_t s) {
  switch (a.G) {
    case 1: launch_prefill_all<D, 1>(a, which, s); break;
    case 2: launch_prefill_all<D, 2>(a, which, s); break;
    case 4: launch_prefill_all<D, 4>(a, which, s); break;
    case 8: launch_prefill_all<D, 8>(a, which, s); break;
    default: launch_prefill_all<D, 16>(a, which, s); break;
  }
}

static void dispatch(const PrefillArgs& a, int which, hipStream_t s) {
  if (a.D == 128) dispatch_g<128>(a, which, s);
  else dispatch_g<64>(a, which, s);
}

void launch_cmp_select(const PrefillArgs& a, hipStream_t s) { dispatch(a, 0, s); }
void launch_window(const PrefillArgs& a, hipStream_t s) { dispatch(a, 1, s); }
void launch_selected(const PrefillArgs& a, hipStream_t s) { dispatch(a, 2, s); }

}  // namespace nsa
