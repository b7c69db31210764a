// NSA prefill kernels ("Zhang Xiaojun podcast EP94 notes", sections 5 and 6):
//   kc_norm_kernel:    maxima of the compressed keys' squared norms (the score bound of the
//                      compressed attention's first pass);
//   cmp_select_kernel: compressed attention + block importance + group top-n selection;
//   window_kernel:     sliding-window attention (when run as a stage of its own).
// The selected-block branch is in selected.hip.  The gate mix is folded into the output
// writes: cmp stores g0*o_cmp (+ g2*o_win when the window runs inside it), the window and
// selected branches add g2*o_win and g1*o_slc.
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

// Shift a wave-wide 64-bit value up by one lane (lane e receives lane e - 1's; lane 0 its own).
__device__ __forceinline__ uint64_t shfl_up1_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)v, 1);
  const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(v >> 32), 1);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Streaming selection (sequences too long for a query tile's block scores to fit in LDS): a
// block's group score is final once the key-tile walk has passed its last compressed token, and
// is then offered at once to the position's running top list, kept sorted in LDS (list[e] =
// the e-th best free block's rank key so far, 0 = empty); the forced blocks' total is summed in
// block order for the top-p cut.  Called by a whole wave: block j in the lanes with `have`
// (ascending with the lane), score s.  Rank keys are unique, so the final list is the same
// set, in the same order, as a top-k over all scores at the end.
__device__ __forceinline__ void stream_offer(const PrefillArgs& a, int t, uint64_t* list,
                                             float* forced_sum, int j, bool have, float s,
                                             int lane) {
  const bool top_p = a.top_p > 0.f;
  const int bcur = t / a.beta;
  if (bcur + 1 <= a.top_n && !top_p) return;  // every visible block is chosen anyway
  const int flo = bcur - a.n_local + 1 > 1 ? bcur - a.n_local + 1 : 1;
  const int kfree = a.top_n - 1 - a.n_local;
  if (top_p) {
    uint64_t fm = __ballot(have && (j == 0 || (j >= flo && j <= bcur)));
    if (fm != 0) {  // uniform
      float f = *forced_sum;
      while (fm != 0) {
        const int src = (int)__builtin_ctzll(fm);
        fm &= fm - 1;
        f += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), src));
      }
      if (lane == 0) *forced_sum = f;
    }
  }
  if (kfree <= 0) return;
  const uint64_t key = have && j >= 1 && j < flo ? rank_key(s, j) : 0;
  uint64_t mine = lane < kfree ? list[lane] : 0;
  uint64_t thr = readlane_u64(mine, kfree - 1);
  uint64_t pass = __ballot(key > thr);
  if (pass == 0) return;  // uniform
  while (pass != 0) {
    const int src = (int)__builtin_ctzll(pass);
    pass &= pass - 1;
    const uint64_t x = readlane_u64(key, src);
    if (x <= thr) continue;  // uniform: an earlier insertion raised the bar
    const int pos = (int)__popcll(__ballot(lane < kfree && mine > x));
    const uint64_t up = shfl_up1_u64(mine);
    if (lane > pos && lane < kfree) mine = up;
    if (lane == pos) mine = x;
    thr = readlane_u64(mine, kfree - 1);
  }
  if (lane < kfree) list[lane] = mine;
}

// Ring of partially summed block scores (generic geometry, streaming selection): block j at
// slot j mod kRing.
constexpr int kRing = 128;

// Squared norms of the compressed keys of one (sequence, KV group) as running maxima within
// kNormRows-row chunks (kpmax) and per chunk (kcmax): one row per thread, the chunk's prefix a
// wave scan plus the maxima of the waves before.  Rows at or past ncmp count as zero.  The sums
// run in a fixed order, so a row's entry depends on the rows up to it only.
__global__ __launch_bounds__(kNormRows) void kc_norm_kernel(PrefillArgs a) {
  __shared__ float wmax[kNormRows / 64];
  const int c = blockIdx.x;
  const long bkv = (long)blockIdx.z * a.Hkv + blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = c * kNormRows + tid;
  float sq = 0.f;
  if (j < a.ncmp) {
    const u32x4* row = reinterpret_cast<const u32x4*>(a.kc + (bkv * a.NCP + j) * a.D);
    for (int e = 0; e < a.D / 8; ++e) {
      const u32x4 w = row[e];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float lo = __uint_as_float(w[h] << 16), hi = __uint_as_float(w[h] & 0xFFFF0000u);
        sq = fmaf(lo, lo, sq);
        sq = fmaf(hi, hi, sq);
      }
    }
  }
  float incl = sq;  // maximum over the wave's rows up to this one
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float u = __shfl_up(incl, o);
    if (lane >= o) incl = fmaxf(incl, u);
  }
  if (lane == 63) wmax[wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl = fmaxf(incl, wmax[w]);
  if (j < a.ncmp) a.kpmax[bkv * a.NCP + j] = incl;
  if (tid == 0) {
    float m = wmax[0];
    for (int w = 1; w < kNormRows / 64; ++w) m = fmaxf(m, wmax[w]);
    a.kcmax[bkv * a.NKB + c] = m;
  }
}

template <int D, int G, bool FAST, bool STREAM>
__global__ __launch_bounds__(QTile<G>::NW * 64, G == 16 ? 2 : 1) void cmp_select_kernel(PrefillArgs a) {
  using QT = QTile<G>;
  constexpr int NT = QT::NW * 64, TQ = QT::TQ, RTW = QT::RTW, DT = D / 16;
  __shared__ u16 Ks[64][D];
  __shared__ u16 Vs[D][64];
  __shared__ float Mb[FAST ? 1 : TQ][64];   // generic path: group mass per (t, key)
  __shared__ float Cb[FAST ? TQ : 1][16];   // fast path: block cores of the tile
  __shared__ float Hb[FAST ? TQ : 1][17];   // fast path: half-key carries into blocks 0..16
  __shared__ float Pc[TQ];                  // fast path: carry into the tile's first block
  // streaming selection: per position its running top list and forced total; generic path:
  // the ring of open block sums
  __shared__ uint64_t Lk[STREAM ? TQ : 1][64];
  __shared__ float Fm[STREAM ? TQ : 1];
  __shared__ float Sr[STREAM && !FAST ? TQ : 1][kRing];
  extern __shared__ float Sb[];             // [TQ][nblk] group block scores (not streaming)

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

  if constexpr (STREAM) {
    for (int e = threadIdx.x; e < TQ * 64; e += NT) Lk[e / 64][e % 64] = 0;
    if constexpr (!FAST)
      for (int e = threadIdx.x; e < TQ * kRing; e += NT) Sr[e / kRing][e % kRing] = 0.f;
    if (threadIdx.x < TQ) Fm[threadIdx.x] = 0.f;
  } else {
    for (int e = threadIdx.x; e < TQ * nblk; e += NT) Sb[e] = 0.f;
  }
  if (threadIdx.x < TQ) Pc[threadIdx.x] = 0.f;
  int jemit = 0;  // streaming, generic path: blocks below jemit are final and offered

  // Pass 1: the row log-sum-exp of the compressed scores.  Every scaled score z sl of a row is at
  // most U = |sl| |q| max |k_c| over the compressed keys the tile sees (Cauchy-Schwarz; the
  // factor 1 + 2^-10 covers the fp32 rounding of the norms and of the products' sums), so the
  // row sum of exp2(z sl - U) needs no running maximum.  A row whose sum falls below 2^-60 (a
  // bound loose by more than 60 in log2 units) or is not finite and at most 2^100 sends the
  // workgroup through the running-maximum form instead.  U depends only on the keys the tile sees, so a
  // chunked prefill takes the same path, bit for bit, as the whole sequence.
  float U[RTW];
  {
    float km = 0.f;
    if (nvis_max > 0) {  // uniform
      const int jl = nvis_max - 1, cl = jl / kNormRows;
      km = a.kpmax[bkv * a.NCP + jl];
      for (int i = lane; i < cl; i += 64) km = fmaxf(km, a.kcmax[bkv * a.NKB + i]);
      km = wave_max_f(km);
    }
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      float qn = 0.f;
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)qf[rt][c][e];
          qn = fmaf(x, x, qn);
        }
      U[rt] = fabsf(sl) * sqrtf(col_sum4(qn) * km) * (1.f + 0x1p-10f);
    }
  }
  float lsum[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) lsum[rt] = 0.f;
  KTileRegs<D, NT> kr;
  VTileRegs<D, NT> vr;
  // the compressed keys' scores of one 64-key tile (keys past a row's visible count at -inf)
  auto tile_scores = [&](int kt, float (*raw)[16]) {
    __syncthreads();
    kr.store(Ks);
    __syncthreads();
    if (kt + 1 < nkt) kr.load(kc, (long)(kt + 1) * 64, a.NCP - 1);
    const bool full = (kt + 1) * 64 <= nvis_lo;
    score_tiles<D, RTW>(Ks, qf, g4, r16, raw);
    if (!full) {  // a real (uniform) branch: full tiles skip the masking arithmetic
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
        __asm__ volatile("" ::: "memory");
        // key kt*64 + 32*(e>>3) + 8*g4 + (e&7) is visible iff its offset from the lane's first
        // key is below lim (one subtraction per lane, constant offsets per element)
        const int lim = nvis[rt] - (kt * 64 + 8 * g4);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          raw[rt][e] = 32 * (e >> 3) + (e & 7) < lim ? raw[rt][e] : kNegInf;
      }
    }
  };
  if (nkt > 0) kr.load(kc, 0, a.NCP - 1);
  for (int kt = 0; kt < nkt; ++kt) {
    float raw[RTW][16];
    tile_scores(kt, raw);
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += fast_exp2(fmaf(raw[rt][e], sl, -U[rt]));
      lsum[rt] += sum;
    }
  }
  // Row log-sum-exp (scaled, log2 units): pass 2 computes the normalised probabilities
  // p = exp2(z - lse) directly, for the block importance (fp32) and the P V product (bf16).
  float rlse[RTW];
  bool vis[RTW];  // the row sees a compressed key (else p is masked to 0)
  int loose = 0;
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const float L = col_sum4(lsum[rt]);
    vis[rt] = nvis[rt] > 0;
    rlse[rt] = vis[rt] ? U[rt] + __log2f(L) : 0.f;
    if (vis[rt] && !(L >= 0x1p-60f && L <= 0x1p100f)) loose = 1;  // also an overflowed sum
  }
  if (__syncthreads_or(loose)) {  // uniform: the running-maximum form (per lane, then per row)
    float mrun[RTW], lrun[RTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) { mrun[rt] = kNegInf; lrun[rt] = 0.f; }
    if (nkt > 0) kr.load(kc, 0, a.NCP - 1);
    for (int kt = 0; kt < nkt; ++kt) {
      float raw[RTW][16];
      tile_scores(kt, raw);
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
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
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const float M = col_max4(mrun[rt]);
      const float part = (mrun[rt] == kNegInf) ? 0.f : lrun[rt] * fast_exp2((mrun[rt] - M) * sl);
      const float L = col_sum4(part);
      vis[rt] = M != kNegInf;
      rlse[rt] = vis[rt] ? M * sl + __log2f(L) : 0.f;
    }
  }
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
    if (a.dlse != nullptr && g4 == 0 && row_t[rt] < a.T)  // diagnostics: natural-log lse
      a.dlse[prow(a, b, row_t[rt]) * (a.Hkv * G) + row_h[rt]] =
          vis[rt] ? rlse[rt] * 0.6931471805599453f : kNegInf;

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
    if constexpr (FAST && STREAM) {
      // blocks 16*kt .. 16*kt + 15 are complete (core + carry, as below): offered per position
      for (int tq = wave; tq < TQ; tq += QT::NW) {
        if (t0 + tq >= a.T) break;  // uniform
        const int j = 16 * kt + lane;
        const bool have = lane < 16 && j < nblk;
        float sv = 0.f;
        if (have) sv = Cb[tq][lane] + (lane == 0 ? Pc[tq] : Hb[tq][lane]);
        if (lane == 0) Pc[tq] = Hb[tq][16];
        stream_offer(a, t0 + tq, Lk[tq], &Fm[tq], j, have, sv, lane);
      }
    } else if constexpr (FAST) {
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
        float* slot = STREAM ? &Sr[tq][j & (kRing - 1)] : &Sb[tq * nblk + j];
        float sv = *slot;
        for (int i = ilo; i <= ihi; ++i) {
          const int s0 = i * a.d, s1 = s0 + a.l;
          const int ov = (s1 < be ? s1 : be) - (s0 > bs ? s0 : bs);
          if (ov > 0) sv += Mb[tq][i - k0] * ((float)ov * inv_l);
        }
        *slot = sv;
      }
      if constexpr (STREAM) {
        // no later tile adds to the blocks below the next tile's first block: offer them and
        // clear their slots
        int jend = (int)(((long)(kt + 1) * 64 * a.d) / a.beta);
        jend = jend < nblk ? jend : nblk;
        __syncthreads();
        for (int tq = wave; tq < TQ; tq += QT::NW) {
          if (t0 + tq >= a.T) break;  // uniform
          for (int j0 = jemit; j0 < jend; j0 += 64) {
            const int j = j0 + lane;
            const bool have = j < jend;
            float sv = 0.f;
            if (have) {
              sv = Sr[tq][j & (kRing - 1)];
              Sr[tq][j & (kRing - 1)] = 0.f;
            }
            stream_offer(a, t0 + tq, Lk[tq], &Fm[tq], j, have, sv, lane);
          }
        }
        jemit = jend > jemit ? jend : jemit;
      }
    }
  }
  if constexpr (STREAM) {
    __syncthreads();
    // the rest of the blocks up to the tile's last position's: the block after the last tile
    // has only its carry (fast path) or the ring's sum (generic path), the ones after it
    // nothing visible
    const int jfirst = FAST ? 16 * nkt : jemit;
    const int bmax = tlast / a.beta;
    for (int tq = wave; tq < TQ; tq += QT::NW) {
      if (t0 + tq >= a.T) break;  // uniform
      for (int j0 = jfirst; j0 <= bmax; j0 += 64) {
        const int j = j0 + lane;
        const bool have = j <= bmax && j < nblk;
        float sv = 0.f;
        if (have) {
          if constexpr (FAST) sv = (j == 16 * nkt && nkt > 0) ? 0.f + Pc[tq] : 0.f;
          else sv = Sr[tq][j & (kRing - 1)];
        }
        stream_offer(a, t0 + tq, Lk[tq], &Fm[tq], j, have, sv, lane);
      }
    }
  } else if constexpr (FAST) {
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
    if constexpr (!STREAM) {
      if (a.dscores != nullptr) {  // diagnostics: the group block scores, 0 past block bcur
        float* drow = a.dscores + (prow(a, b, t) * a.Hkv + kvh) * nblk;
        for (int j = lane; j < nblk; j += 64) drow[j] = j <= bcur ? Sb[tq * nblk + j] : 0.f;
      }
    }
    if (nb <= a.top_n && !top_p) {
      for (int e = lane; e < a.top_n; e += 64) orow[e] = e < nb ? e : -1;
      continue;
    }
    // forced: block 0 and the local blocks flo..bcur; free candidates 1 .. flo-1
    const int flo = bcur - a.n_local + 1 > 1 ? bcur - a.n_local + 1 : 1;
    const int kfree = a.top_n - 1 - a.n_local;
    // lane e < kfree receives the e-th winner among the free blocks (0 past the last one)
    uint64_t key;
    float forced = 0.f;
    if constexpr (STREAM) {
      key = lane < kfree ? Lk[tq][lane] : 0;
      forced = Fm[tq];
    } else {
      const float* srow = Sb + tq * nblk;
      key = wave_topk([&](int j) { return rank_key(srow[j], j); }, 1, flo, kfree, lane);
      if (top_p) {
        forced = srow[0];
        for (int j = flo; j <= bcur; ++j) forced += srow[j];
      }
    }
    if (top_p) {
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

bool cmp_select_streams(int G, int nblk) { return cmp_select_lds_bytes(G, nblk) > 64 * 1024; }

template <int D, int G>
static void launch_prefill_all(const PrefillArgs& a, int which, hipStream_t s) {
  using QT = QTile<G>;
  const int ntile = (a.nq + QT::TQ - 1) / QT::TQ;
  const bool fast = a.beta == 4 * a.d && a.l == 2 * a.d;
  if (which == 0 && cmp_select_streams(G, a.nblk)) {
    const dim3 grid(ntile, a.Hkv, a.B);
    if (fast) cmp_select_kernel<D, G, true, true><<<grid, QT::NW * 64, 0, s>>>(a);
    else cmp_select_kernel<D, G, false, true><<<grid, QT::NW * 64, 0, s>>>(a);
  } else if (which == 0) {
    const size_t lds = cmp_lds<G>(a.nblk);
    // opt in to the largest dynamic LDS any launch may use (64 KB, the validated limit); the
    // attribute is per device, so it is set on every launch rather than once per process
    (void)hipFuncSetAttribute(
        fast ? reinterpret_cast<const void*>(&cmp_select_kernel<D, G, true, false>)
             : reinterpret_cast<const void*>(&cmp_select_kernel<D, G, false, false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024);
    if (fast)
      cmp_select_kernel<D, G, true, false><<<dim3(ntile, a.Hkv, a.B), QT::NW * 64, lds, s>>>(a);
    else
      cmp_select_kernel<D, G, false, false><<<dim3(ntile, a.Hkv, a.B), QT::NW * 64, lds, s>>>(a);
  } else {
    window_kernel<D, G><<<dim3(ntile, a.Hkv, a.B), QT::NW * 64, 0, s>>>(a);
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

void launch_cmp_select(const PrefillArgs& a, hipStream_t s) {
  if (a.ncmp > 0) kc_norm_kernel<<<dim3(a.NKB, a.Hkv, a.B), kNormRows, 0, s>>>(a);
  dispatch(a, 0, s);
}
void launch_window(const PrefillArgs& a, hipStream_t s) { dispatch(a, 1, s); }

}  // namespace nsa
