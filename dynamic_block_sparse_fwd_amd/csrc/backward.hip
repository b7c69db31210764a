// Backward of the NSA prefill layer ("Zhang Xiaojun podcast EP94" notes, section 5: three
// attention branches mixed by a gate; the "Native Sparse Attention" article: the layer is
// trained end to end and its compressor is a learnable linear map).  The forward's block
// selection is an input: a discrete choice, it passes no gradient, and the bf16 rounding of a
// compressed token passes the gradient unchanged.
//
// A position's G query heads form one 16-row matrix-core tile (rows G .. 15 repeat head G - 1
// with a zero gate and zero transposed operands, and write nothing).  Per branch:
//   bwd_q_kernel / bwd_q_shared_kernel
//                  query-major, one wave per position, one online pass over the branch's
//                  64-key tiles: the log2-sum-exp2 of the scaled scores, <dO, o> and
//                  dq += scale * dS K (dS taken against the running mean of dP', corrected as
//                  the mean moves); the compressed and window passes stage each key tile in
//                  LDS once for 8 neighbouring positions;
//   bwd_kv_kernel  key-major, one workgroup per 64- or 128-key tile (a wave per 16 keys): over
//                  the positions that see the tile, two positions (32 rows) per step staged in
//                  LDS, dV += (g P)^T dO and dK += scale * dS^T q;
// the compressed branch's key gradients then go back through the compressor
// (bwd_cmp_dx_kernel: dK, dV; bwd_cmp_dw_kernel: dWk, dWv).  No floating-point atomics: every
// output element has one writer per launch and launches that add to the same output run in
// order.  The compressed and selected key-major passes split the positions into chunks that
// write fp32 partials of their own; a reduction adds the chunks in chunk order, so two calls on
// the same inputs give the same bits.  The selected pass takes a tile's positions, ascending,
// from a bitmap of the selection (bwd_selbits_kernel, built with an order-free atomic OR).  dO enters the matrix core in bf16; q and dO are also kept with
// the 16 rows of a (position, group) contiguous per feature (the B operand of the key-major
// products).
#include "attn_tile.h"
#include "kernels.h"

namespace nsa {

namespace {

constexpr int kBrCmp = 0, kBrSlc = 1, kBrWin = 2;  // also the gate columns
constexpr float kInf = __builtin_huge_valf();

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)v[i];
  return r;
}

// Key-set geometry of one branch for query position t.
template <int BR>
struct KeySet {
  int lo, hi;  // valid keys: lo <= key <= hi (compressed: token indices)
  __device__ __forceinline__ KeySet(const BwdArgs& a, int t) {
    if constexpr (BR == kBrCmp) {
      lo = 0;
      hi = n_visible(t, a.l, a.d, a.ncmp) - 1;
    } else if constexpr (BR == kBrSlc) {
      lo = 0;
      hi = t;
    } else {
      lo = t - a.window + 1 > 0 ? t - a.window + 1 : 0;
      hi = t;
    }
  }
  __device__ __forceinline__ bool valid(int key) const { return key >= lo && key <= hi; }
};

// One tile of the query-major online pass.  With e = exp2(s - m) against the running maximum m,
// l = sum e and c = sum e dP' / l, the running mean of dP' under p (it ends as <dO, o>):
//   Z = sum_k e_k (dP'_k - c) K_k,  Bk = sum_k e_k K_k,
// and when c moves from c0 to c1, Z += (c0 - c1) Bk keeps Z referred to the new mean; at the
// end dq = scale * g * Z / l = scale * sum_k g p_k (dP'_k - <dO, o>) K_k.  The operand rounded
// to bf16 for the matrix core is e (dP' - c), small where dP' is near its mean, as in the
// two-pass form dS = p (dP' - <dO, o>); Bk's own rounding enters only through the moves of c.
// raw: scaled scores (log2 units, -inf where masked), dp: dP' of the tile's 16 keys per lane
// (key 32 kc + 8 g4 + i of row r16); kfrag(kc, n) gives the A operand K^T[16 n + r16][32 kc +
// 8 g4 ..].
struct OnlineDq {
  float m = -kInf, lsum = 0.f, acc = 0.f, c = 0.f;
  template <int DT, class KF>
  __device__ __forceinline__ void step(float* raw, const float* dp, f32x4* Z, f32x4* Bk,
                                       KF kfrag) {
    float mx = raw[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, raw[i]);
    mx = col_max4(mx);
    const float mn = fmaxf(m, mx);
    if (mn == -kInf) return;  // nothing visible yet (the same for every head)
    const float sc = exp2f(m - mn);
    if (__ballot(sc != 1.f) != 0) {  // uniform: some head's maximum moved
#pragma unroll
      for (int n = 0; n < DT; ++n) { Z[n] *= sc; Bk[n] *= sc; }
    }
    float ls = 0.f, as = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      raw[i] = exp2f(raw[i] - mn);  // e from here on
      ls += raw[i];
      as += raw[i] * dp[i];
    }
    lsum = lsum * sc + col_sum4(ls);
    acc = acc * sc + col_sum4(as);
    m = mn;
    const float cn = acc / lsum;  // lsum >= 1: the maximum's own term
    const float dc = c - cn;
    c = cn;
    if (__ballot(dc != 0.f) != 0) {  // uniform
#pragma unroll
      for (int n = 0; n < DT; ++n) Z[n] += dc * Bk[n];
    }
    bf16x8 xb[2], eb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      xb[i >> 3][i & 7] = (__bf16)(raw[i] * (dp[i] - cn));
      eb[i >> 3][i & 7] = (__bf16)raw[i];
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int n = 0; n < DT; ++n) {
        const bf16x8 kf = kfrag(kc, n);
        Z[n] = mfma16x16x32(kf, xb[kc], Z[n]);
        Bk[n] = mfma16x16x32(kf, eb[kc], Bk[n]);
      }
  }
};

}  // namespace

// dO -> bf16 rows; q and dO with the G heads of a (position, group) contiguous per feature,
// zero in the 16 - G pad rows.
// The selection as a bitmap: bit t of row (sequence, group, block j) is set when position t's
// index row holds j (repeats, holes and blocks out of range ignored).  OR is order-free, so the
// bitmap is the same on every call; the selected key-major pass reads its positions from it.
__global__ __launch_bounds__(256) void bwd_selbits_kernel(BwdArgs a) {
  const long id = (long)blockIdx.x * 256 + threadIdx.x;  // (b * T + t) * Hkv + g
  if (id >= (long)a.B * a.T * a.Hkv) return;
  const int g = (int)(id % a.Hkv);
  const long bt = id / a.Hkv;
  const int t = (int)(bt % a.T), b = (int)(bt / a.T);
  const int32_t* ir = a.idx + id * a.top_n;
  uint32_t* rows = a.selbits + ((long)b * a.Hkv + g) * a.nblk * a.SW + (t >> 5);
  for (int e = 0; e < a.top_n; ++e) {
    const int j = ir[e];
    if (j >= 0 && j < a.nblk) atomicOr(&rows[(long)j * a.SW], 1u << (t & 31));
  }
}

__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  const long n = (long)a.B * a.T * a.Hkv * a.D;
  if (e >= n) return;
  const int D = a.D;
  const int dd = (int)(e % D);
  const long r = e / D;  // (b, t, g)
  const int G = a.G;
  const long row0 = r * G;  // first head row of [B, T, Hq] (Hq = G Hkv)
  u16 qh[16], dh[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    dh[h] = 0;
    qh[h] = 0;
    if (h < G) {
      dh[h] = f32_to_bf16(a.dout[(row0 + h) * D + dd]);
      qh[h] = a.q[(row0 + h) * D + dd];
      a.dob[(row0 + h) * D + dd] = dh[h];
    }
  }
  u16* dt = a.dot + (r * D + dd) * 16;
  u16* qt = a.qt + (r * D + dd) * 16;
#pragma unroll
  for (int h = 0; h < 16; h += 8) {
    u32x4 w1, w2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w1[i] = (uint32_t)dh[h + 2 * i] | ((uint32_t)dh[h + 2 * i + 1] << 16);
      w2[i] = (uint32_t)qh[h + 2 * i] | ((uint32_t)qh[h + 2 * i + 1] << 16);
    }
    *reinterpret_cast<u32x4*>(dt + h) = w1;
    *reinterpret_cast<u32x4*>(qt + h) = w2;
  }
}

// Query-major pass of branch BR: lse, <dO, o> and dq per (position, head), one pass.
template <int D, int BR>
__global__ __launch_bounds__(256, 2) void bwd_q_kernel(BwdArgs a) {
  constexpr int DC = D / 32, DT = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int t = blockIdx.x * 4 + wave, g = blockIdx.y, b = blockIdx.z;
  if (t >= a.T) return;  // uniform per wave; no barrier in this kernel
  const int Hq = a.Hkv * a.G;
  const long bg = (long)b * a.Hkv + g;
  const bool head = r16 < a.G;  // rows G .. 15 repeat head G - 1 and write nothing
  const long myrow = ((long)b * a.T + t) * Hq + g * a.G + (head ? r16 : a.G - 1);
  bf16x8 qf[DC], df[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    qf[c] = load8(a.q + myrow * D + 32 * c + 8 * g4);
    df[c] = load8(a.dob + myrow * D + 32 * c + 8 * g4);
  }
  const float gt = a.gate[myrow * 3 + BR];
  const float sl = a.scale_log2;
  const KeySet<BR> ks(a, t);

  const u16* krows;
  const u16* vrows;
  const u16* kcols;
  int pitch, klim;
  if constexpr (BR == kBrCmp) {
    krows = a.kc + bg * (long)a.NCP * D;
    vrows = a.vc + bg * (long)a.NCP * D;
    kcols = a.kct + bg * (long)D * a.NCP;
    pitch = a.NCP;
    klim = a.NCP - 1;
  } else {
    krows = a.k + bg * (long)a.T * D;
    vrows = a.v + bg * (long)a.T * D;
    kcols = a.kt + bg * (long)D * a.TP;
    pitch = a.TP;
    klim = a.T - 1;
  }
  // tiles: base key of tile e, or -1 to skip (uniform over the wave)
  const int per = a.beta / 64;
  int ntiles;
  if constexpr (BR == kBrCmp) ntiles = (ks.hi + 1 + 63) / 64;
  else if constexpr (BR == kBrSlc) ntiles = a.top_n * per;
  else ntiles = t / 64 - ks.lo / 64 + 1;
  const int32_t* irow = a.idx + (((long)b * a.T + t) * a.Hkv + g) * a.top_n;
  auto tile_base = [&](int e) -> int {
    if constexpr (BR == kBrCmp) return 64 * e;
    else if constexpr (BR == kBrSlc) {
      const int j = irow[e / per];
      const int base = j * a.beta + 64 * (e % per);
      return (j >= 0 && j < a.nblk && base <= t) ? base : -1;
    } else return (ks.lo / 64 + e) * 64;
  };
  // S^T and dP'^T = V dO^T of one tile: raw[kc*8 + s*4 + i] / dp[..] belong to key
  // base + 32 kc + 8 g4 + 4 s + i and query row (head) r16
  auto tile = [&](int base, float* raw, float* dp) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        int key = base + 32 * kc + perm_key(r16, s);
        key = key < klim ? key : klim;
        f32x4 as = zero4(), ap = zero4();
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          as = mfma16x16x32(load8(krows + (long)key * D + 32 * c + 8 * g4), qf[c], as);
          ap = mfma16x16x32(load8(vrows + (long)key * D + 32 * c + 8 * g4), df[c], ap);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = base + 32 * kc + 8 * g4 + 4 * s + i;
          raw[kc * 8 + s * 4 + i] = ks.valid(kk) ? as[i] * sl : -kInf;
          dp[kc * 8 + s * 4 + i] = ap[i];
        }
      }
  };

  f32x4 Z[DT], Bk[DT];
#pragma unroll
  for (int n = 0; n < DT; ++n) { Z[n] = zero4(); Bk[n] = zero4(); }
  OnlineDq st;
  for (int e = 0; e < ntiles; ++e) {
    const int base = tile_base(e);
    if (base < 0) continue;
    float raw[16], dp[16];
    tile(base, raw, dp);
    st.step<DT>(raw, dp, Z, Bk, [&](int kc, int n) {
      return load8(kcols + (long)(16 * n + r16) * pitch + base + 32 * kc + 8 * g4);
    });
  }
  const bool any = st.lsum > 0.f;
  const float lse2 = any ? st.m + __log2f(st.lsum) : kInf;  // no key: every p is 0
  const float dl = any ? st.c : 0.f;
  if (g4 == 0 && head) {
    const long o = (long)BR * a.B * a.T * Hq + myrow;
    a.lse[o] = lse2;
    a.dlt[o] = dl;
    a.dgate[myrow * 3 + BR] = dl;
  }
  const float f = any ? a.scale * gt / st.lsum : 0.f;
  f32x4 dq[DT];
#pragma unroll
  for (int n = 0; n < DT; ++n) dq[n] = Z[n] * f;
  if (!head) return;
  // lane holds dq^T[feature 16 n + 4 g4 + i][head r16]
  float* dqp = a.dq + myrow * D;
#pragma unroll
  for (int n = 0; n < DT; ++n) {
    float4 v = make_float4(dq[n][0], dq[n][1], dq[n][2], dq[n][3]);
    float4* dst = reinterpret_cast<float4*>(dqp + 16 * n + 4 * g4);
    if constexpr (BR != kBrCmp) {
      const float4 o = *dst;
      v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
    }
    *dst = v;
  }
}

// Query-major pass of the compressed or window branch with the workgroup's NW positions
// (consecutive, one per wave) sharing every key tile: K and V rows and the transposed keys are
// staged once in LDS (the swizzled tile layouts of the forward), the next tile's loads in flight
// during the current one.  Neighbouring positions' key sets differ by a few tokens at either
// end, so the workgroup walks the union of their tiles and each wave masks its own keys.
template <int D, int BR, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_q_shared_kernel(BwdArgs a) {
  static_assert(BR != kBrSlc, "the selected branch's key sets differ per position");
  constexpr int DC = D / 32, DT = D / 16, NT = NW * 64;
  __shared__ __align__(16) u16 Ks[64][D];
  __shared__ __align__(16) u16 Vr[64][D];
  __shared__ __align__(16) u16 Kt[D][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int tfirst = blockIdx.x * NW, g = blockIdx.y, b = blockIdx.z;
  const int t = tfirst + wave;
  const bool live = t < a.T;  // dead waves still pass the barriers
  const int tq = live ? t : a.T - 1;
  const int tlastw = tfirst + NW - 1 < a.T - 1 ? tfirst + NW - 1 : a.T - 1;
  const int Hq = a.Hkv * a.G;
  const long bg = (long)b * a.Hkv + g;
  const bool head = r16 < a.G;  // rows G .. 15 repeat head G - 1 and write nothing
  const long myrow = ((long)b * a.T + tq) * Hq + g * a.G + (head ? r16 : a.G - 1);
  bf16x8 qf[DC], df[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    qf[c] = load8(a.q + myrow * D + 32 * c + 8 * g4);
    df[c] = load8(a.dob + myrow * D + 32 * c + 8 * g4);
  }
  const float gt = a.gate[myrow * 3 + BR];
  const float sl = a.scale_log2;
  const KeySet<BR> ks(a, tq);

  const u16* krows;
  const u16* vrows;
  const u16* kcols;
  int pitch, klim, kt0, kt1;
  if constexpr (BR == kBrCmp) {
    krows = a.kc + bg * (long)a.NCP * D;
    vrows = a.vc + bg * (long)a.NCP * D;
    kcols = a.kct + bg * (long)D * a.NCP;
    pitch = a.NCP;
    klim = a.NCP - 1;
    kt0 = 0;
    kt1 = (n_visible(tlastw, a.l, a.d, a.ncmp) + 63) / 64 - 1;
  } else {
    krows = a.k + bg * (long)a.T * D;
    vrows = a.v + bg * (long)a.T * D;
    kcols = a.kt + bg * (long)D * a.TP;
    pitch = a.TP;
    klim = a.T - 1;
    kt0 = (tfirst - a.window + 1 > 0 ? tfirst - a.window + 1 : 0) / 64;
    kt1 = tlastw / 64;
  }
  // scores and dP'^T of the staged tile: raw[kc*8 + s*4 + i] / dp[..] belong to key
  // base + 32 kc + 8 g4 + 4 s + i and query row (head) r16
  auto tile = [&](int base, float* raw, float* dp) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 kf[DC], vf[DC];
        k_frags<D>(Ks, kc, s, g4, r16, kf);
        k_frags<D>(Vr, kc, s, g4, r16, vf);
        f32x4 as = zero4(), ap = zero4();
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          as = mfma16x16x32(kf[c], qf[c], as);
          ap = mfma16x16x32(vf[c], df[c], ap);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = base + 32 * kc + 8 * g4 + 4 * s + i;
          raw[kc * 8 + s * 4 + i] = live && ks.valid(kk) ? as[i] * sl : -kInf;
          dp[kc * 8 + s * 4 + i] = ap[i];
        }
      }
  };

  // one online pass (OnlineDq): the three tiles of each step staged once
  f32x4 Z[DT], Bk[DT];
#pragma unroll
  for (int n = 0; n < DT; ++n) { Z[n] = zero4(); Bk[n] = zero4(); }
  OnlineDq st;
  {
    KTileRegs<D, NT> kr, vr;
    VTileRegs<D, NT> tr;
    if (kt0 <= kt1) {
      kr.load(krows, (long)kt0 * 64, klim);
      vr.load(vrows, (long)kt0 * 64, klim);
      tr.load(kcols, pitch, (long)kt0 * 64);
    }
    for (int kt = kt0; kt <= kt1; ++kt) {
      kr.store(Ks);
      vr.store(Vr);
      tr.store(Kt);
      lds_barrier();
      if (kt < kt1) {
        kr.load(krows, (long)(kt + 1) * 64, klim);
        vr.load(vrows, (long)(kt + 1) * 64, klim);
        tr.load(kcols, pitch, (long)(kt + 1) * 64);
      }
      float raw[16], dp[16];
      tile(kt * 64, raw, dp);
      st.step<DT>(raw, dp, Z, Bk, [&](int kc, int n) {
        return load8(&Kt[16 * n + r16][((4 * kc + g4) ^ (r16 & 7)) * 8]);
      });
      lds_barrier();
    }
  }
  const bool any = st.lsum > 0.f;
  const float lse2 = any ? st.m + __log2f(st.lsum) : kInf;
  const float dl = any ? st.c : 0.f;
  if (live && head && g4 == 0) {
    const long o = (long)BR * a.B * a.T * Hq + myrow;
    a.lse[o] = lse2;
    a.dlt[o] = dl;
    a.dgate[myrow * 3 + BR] = dl;
  }
  const float f = any ? a.scale * gt / st.lsum : 0.f;
  f32x4 dq[DT];
#pragma unroll
  for (int n = 0; n < DT; ++n) dq[n] = Z[n] * f;
  if (!live || !head) return;
  float* dqp = a.dq + myrow * D;
#pragma unroll
  for (int n = 0; n < DT; ++n) {
    float4 v = make_float4(dq[n][0], dq[n][1], dq[n][2], dq[n][3]);
    float4* dst = reinterpret_cast<float4*>(dqp + 16 * n + 4 * g4);
    if constexpr (BR != kBrCmp) {
      const float4 o = *dst;
      v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
    }
    *dst = v;
  }
}

// LDS copy of one position pair's operands for the key-major pass (rows 0-15: position ta's
// heads, 16-31: tb's).  q and dO rows are chunk-swizzled (chunk c of row r at c ^ pair_swz(r):
// the 16 rows one operand read touches land on 16 distinct chunks); the heads-contiguous
// copies have a 40-element pitch (80 bytes: 16 consecutive features on distinct banks).
template <int D>
struct PairStage {
  u16 qr[32][D];
  u16 dr[32][D];
  u16 qt[D][40];
  u16 dt[D][40];
  float lse[32], dlt[32], gt[32];
};

template <int D>
__device__ __forceinline__ int pair_swz(int r) {
  return ((r & 3) | ((r >> 3) << 2)) & (D / 8 - 1);
}

// Key-major pass of branch BR over one 64-key tile: dK and dV of its keys.  The workgroup
// stages each position pair's q, dO (both layouts) and row statistics in LDS once for its four
// waves, the next pair's global loads in flight while the current one is computed.
template <int D, int BR, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_kv_kernel(BwdArgs a) {
  static_assert(BR != kBrSlc || NW == 4, "a selected tile is one 64-key piece of one block");
  constexpr int DC = D / 32, DT = D / 16, NT = NW * 64;
  constexpr int NCH = 16 * D / NT;  // 16-byte chunks per thread per pair (4 arrays of 4D)
  __shared__ PairStage<D> st;
  __shared__ int plist[BR == kBrSlc ? 64 * 32 : 1];
  __shared__ int ptot;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int kb = blockIdx.x * 16 * NW;
  const long bg = blockIdx.y;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int Hq = a.Hkv * a.G;
  const float sl = a.scale_log2;
  const u16* krows;
  const u16* vrows;
  int klim;
  if constexpr (BR == kBrCmp) {
    krows = a.kc + bg * (long)a.NCP * D;
    vrows = a.vc + bg * (long)a.NCP * D;
    klim = a.NCP - 1;
  } else {
    krows = a.k + bg * (long)a.T * D;
    vrows = a.v + bg * (long)a.T * D;
    klim = a.T - 1;
  }
  // B operands of S = Q K^T and dP' = dO V^T: key kb + 16 wave + r16, features 32 c + 8 g4 ..
  const int mykey = kb + 16 * wave + r16;
  const int kr = mykey < klim ? mykey : klim;
  bf16x8 kf[DC], vf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    kf[c] = load8(krows + (long)kr * D + 32 * c + 8 * g4);
    vf[c] = load8(vrows + (long)kr * D + 32 * c + 8 * g4);
  }
  f32x4 dK[DT], dV[DT];
#pragma unroll
  for (int n = 0; n < DT; ++n) { dK[n] = zero4(); dV[n] = zero4(); }
  const long bto = (long)BR * a.B * a.T * Hq;

  // global -> registers for the pair (ta, tb); tb < 0: rows 16-31 repeat ta's (masked later)
  u32x4 pre[NCH];
  float pst = 0.f;
  auto fetch = [&](int ta, int tb) {
    const int tb2 = tb >= 0 ? tb : ta;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + NT * i;
      const int region = c / (4 * D), w = c % (4 * D);
      const u16* src;
      if (region < 2) {
        const int row = w / (D / 8), ch = w % (D / 8);
        const int pos = row < 16 ? ta : tb2;
        const int h = (row & 15) < a.G ? (row & 15) : a.G - 1;
        const long qrow = ((long)b * a.T + pos) * Hq + g * a.G + h;
        src = (region == 0 ? a.q : a.dob) + qrow * D + 8 * ch;
      } else {
        const int f = w / 4, part = w % 4;
        const int pos = (part >> 1) ? tb2 : ta;
        src = (region == 2 ? a.qt : a.dot) + ((((long)b * a.T + pos) * a.Hkv + g) * D + f) * 16 +
              8 * (part & 1);
      }
      pre[i] = *reinterpret_cast<const u32x4*>(src);
    }
    if (tid < 96) {
      const int kind = tid / 32, row = tid % 32;
      const int pos = row < 16 ? ta : tb2;
      const bool hd = (row & 15) < a.G;  // pad rows: a zero gate cancels every term
      const long hrow = ((long)b * a.T + pos) * Hq + g * a.G + (hd ? (row & 15) : a.G - 1);
      pst = kind == 0 ? a.lse[bto + hrow] : kind == 1 ? a.dlt[bto + hrow]
                      : hd ? a.gate[hrow * 3 + BR] : 0.f;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + NT * i;
      const int region = c / (4 * D), w = c % (4 * D);
      u16* dst;
      if (region < 2) {
        const int row = w / (D / 8), ch = w % (D / 8);
        dst = (region == 0 ? &st.qr[row][0] : &st.dr[row][0]) + 8 * (ch ^ pair_swz<D>(row));
      } else {
        const int f = w / 4, part = w % 4;
        dst = (region == 2 ? &st.qt[f][0] : &st.dt[f][0]) + 8 * part;
      }
      *reinterpret_cast<u32x4*>(dst) = pre[i];
    }
    if (tid < 96) {
      const int kind = tid / 32, row = tid % 32;
      (kind == 0 ? st.lse : kind == 1 ? st.dlt : st.gt)[row] = pst;
    }
  };
  // one pair from the staged operands
  auto compute = [&](int ta, int tb) {
    bf16x8 qa[2][DC], da[2][DC];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int row = perm_key(r16, s), sw = pair_swz<D>(row);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        qa[s][c] = load8(&st.qr[row][8 * ((4 * c + g4) ^ sw)]);
        da[s][c] = load8(&st.dr[row][8 * ((4 * c + g4) ^ sw)]);
      }
    }
    // this lane's rows: 8 g4 + j (j = 4 s + i), all of position p
    const int p = g4 < 2 ? ta : tb;
    bool ok = p >= 0;
    if (ok) {
      const KeySet<BR> ks(a, p);
      ok = ks.valid(mykey);
    }
    float gp[8], ds[8];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      f32x4 as = zero4(), ap = zero4();
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        as = mfma16x16x32(qa[s][c], kf[c], as);
        ap = mfma16x16x32(da[s][c], vf[c], ap);
      }
      // C[m = 4 g4 + i][n = key r16]: row perm_key(4 g4 + i, s) = 8 g4 + 4 s + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * s + i, row = 8 * g4 + j;
        const float gt = st.gt[row];
        const float pv = ok ? exp2f(as[i] * sl - st.lse[row]) : 0.f;
        gp[j] = gt * pv;
        ds[j] = gt * pv * (ap[i] - st.dlt[row]);
      }
    }
    // A = (gP)^T and dS^T: key r16, rows 8 g4 .. 8 g4 + 7; B = dO^T, q^T of those rows
    const bf16x8 ap8 = pack8(gp), as8 = pack8(ds);
#pragma unroll
    for (int n = 0; n < DT; ++n) {
      dV[n] = mfma16x16x32(ap8, load8(&st.dt[16 * n + r16][8 * g4]), dV[n]);
      dK[n] = mfma16x16x32(as8, load8(&st.qt[16 * n + r16][8 * g4]), dK[n]);
    }
  };
  // the pairs pair(0 .. np-1), software-pipelined through the LDS stage
  auto run = [&](int np, auto pair) {
    if (np <= 0) return;
    int ta, tb;
    pair(0, ta, tb);
    fetch(ta, tb);
    for (int e = 0; e < np; ++e) {
      stash();
      lds_barrier();
      const int ca = ta, cb = tb;
      if (e + 1 < np) {
        pair(e + 1, ta, tb);
        fetch(ta, tb);  // in flight during this pair's products
      }
      compute(ca, cb);
      lds_barrier();  // the stage is rewritten next
    }
  };

  if constexpr (BR == kBrWin) {
    const int klast = kb + 16 * NW - 1;
    const int t0 = kb, t1 = klast + a.window - 1 < a.T - 1 ? klast + a.window - 1 : a.T - 1;
    run((t1 - t0 + 2) / 2, [&](int e, int& x, int& y) {
      x = t0 + 2 * e;
      y = x + 1 <= t1 ? x + 1 : -1;
    });
  } else if constexpr (BR == kBrCmp) {
    const int tlo = kb * a.d + a.l - 1;  // first position that sees compressed token kb
    int t0 = blockIdx.z * a.PC, t1 = t0 + a.PC - 1;
    t0 = t0 > tlo ? t0 : tlo;
    t1 = t1 < a.T - 1 ? t1 : a.T - 1;
    run((t1 - t0 + 2) / 2, [&](int e, int& x, int& y) {
      x = t0 + 2 * e;
      y = x + 1 <= t1 ? x + 1 : -1;
    });
  } else {
    // positions of chunk blockIdx.z at or after kb whose group selected the block of this tile
    // (block 0 is selected by every position: without the chunks its tile alone would walk the
    // whole sequence), read from the selection bitmap 64 words (2048 positions) at a time: the
    // first wave turns its words into the ascending list of their set bits
    const int jb = kb / a.beta;
    const int c_lo = (int)blockIdx.z * a.PC > kb ? (int)blockIdx.z * a.PC : kb;
    const int c_hi = ((int)blockIdx.z + 1) * a.PC < a.T ? ((int)blockIdx.z + 1) * a.PC : a.T;
    if (c_lo >= c_hi) return;  // uniform: no position of this chunk sees the tile
    // c_lo is a multiple of 64 (PC and kb are), so every word starts inside the chunk
    const uint32_t* bits = a.selbits + ((long)bg * a.nblk + jb) * a.SW;
    for (int p0 = c_lo; p0 < c_hi; p0 += 64 * 32) {
      if (wave == 0) {
        const int p = p0 + 32 * lane;  // this lane's word covers positions p .. p + 31
        uint32_t word = p < c_hi ? bits[p >> 5] : 0u;
        const int keep = c_hi - p;  // positions of the word inside the chunk
        if (keep < 32) word &= keep > 0 ? (1u << keep) - 1u : 0u;
        const int n = __popc(word);
        int incl = n;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int u = __shfl_up(incl, o);
          incl += lane >= o ? u : 0;
        }
        int at = incl - n;
        while (word != 0u) {
          plist[at++] = p + (__ffs(word) - 1);
          word &= word - 1u;
        }
        if (lane == 63) ptot = incl;
      }
      __syncthreads();
      const int tot = ptot;
      run((tot + 1) / 2, [&](int e, int& x, int& y) {
        x = plist[2 * e];
        y = 2 * e + 1 < tot ? plist[2 * e + 1] : -1;
      });
      __syncthreads();  // plist and ptot are rewritten by the next round
    }
  }

  // lane holds dK[key kb + 16 wave + 4 g4 + i][feature 16 n + r16]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = kb + 16 * wave + 4 * g4 + i;
    if constexpr (BR == kBrCmp) {
      if (key >= a.NCP) continue;  // NCP is a multiple of 64, the workgroup may span 128
      const long o = (((long)blockIdx.z * a.B * a.Hkv + bg) * a.NCP + key) * D;
#pragma unroll
      for (int n = 0; n < DT; ++n) {
        a.pk[o + 16 * n + r16] = a.scale * dK[n][i];
        a.pv[o + 16 * n + r16] = dV[n][i];
      }
    } else {
      if (key >= a.T) continue;
      // selected: the chunk's own partial (every chunk that reaches the tile writes one, zero
      // when none of its positions chose the block)
      const long o = BR == kBrSlc ? (((long)blockIdx.z * a.B * a.Hkv + bg) * a.T + key) * D
                                  : (bg * a.T + key) * D;
      float* dk = BR == kBrSlc ? a.psk : a.dk;
      float* dv = BR == kBrSlc ? a.psv : a.dv;
#pragma unroll
      for (int n = 0; n < DT; ++n) {
        dk[o + 16 * n + r16] = a.scale * dK[n][i];
        dv[o + 16 * n + r16] = dV[n][i];
      }
    }
  }
}

// dK, dV += the selected branch's position-chunk partials, in chunk order from the first chunk
// that reaches the key's 64-key tile (the chunks that wrote one).
__global__ __launch_bounds__(256) void bwd_slc_reduce_kernel(BwdArgs a) {
  const long n = (long)a.B * a.Hkv * a.T * a.D;
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const int key = (int)((e / a.D) % a.T);
  float sk = 0.f, sv = 0.f;
  for (int z = (key & ~63) / a.PC; z < a.NPC; ++z) {
    sk += a.psk[(long)z * n + e];
    sv += a.psv[(long)z * n + e];
  }
  a.dk[e] += sk;
  a.dv[e] += sv;
}

// dKc, dVc = sum of the position-chunk partials (chunk order).
__global__ __launch_bounds__(256) void bwd_cmp_reduce_kernel(BwdArgs a) {
  const long n = (long)a.B * a.Hkv * a.NCP * a.D;
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float sk = 0.f, sv = 0.f;
  for (int z = 0; z < a.NPC; ++z) {
    sk += a.pk[(long)z * n + e];
    sv += a.pv[(long)z * n + e];
  }
  a.dkc[e] = sk;
  a.dvc[e] = sv;
}

// dK[s] += sum over the compressed tokens i covering s of dKc[i] W[s - i d]^T (same for V), as
// one matrix-core GEMM per residue r = s mod d: token s = u d + r receives
// sum_q dKc[u - q] W[r + q d]^T over q = 0 .. ceil(l / d) - 1 (terms with u - q outside
// [0, n_cmp) or r + q d >= l drop out), so every output row has one writer.  The fp32 dKc
// enters the matrix core as a bf16 pair (hi + lo, 2^-17 relative), the weight exactly.
// Workgroup: 64 values of u x D features of one (sequence-head, residue) for keys (z = 0) or
// values (z = 1); wave w owns features [w D/4, (w+1) D/4).
template <int D>
__global__ __launch_bounds__(256) void bwd_cmp_dx_kernel(BwdArgs a) {
  constexpr int CT = D / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int u0 = blockIdx.x * 64;
  const int r = (int)(blockIdx.y % a.d);
  const long bg = blockIdx.y / a.d;
  const int kv = blockIdx.z;
  const float* dxc = (kv ? a.dvc : a.dkc) + bg * (long)a.NCP * D;
  const u16* w = kv ? a.wv : a.wk;
  float* dx = (kv ? a.dv : a.dk) + bg * (long)a.T * D;
  f32x4 acc[CT][4];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int it = 0; it < 4; ++it) acc[ct][it] = zero4();
  for (int q = 0; r + q * a.d < a.l; ++q) {
    const int j = r + q * a.d;
    for (int kk = 0; kk < D / 32; ++kk) {
      bf16x8 bw[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        bw[ct] = load8(w + ((long)j * D + wave * (D / 4) + ct * 16 + r16) * D + 32 * kk + 8 * g4);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int i = u0 + it * 16 + r16 - q;
        bf16x8 hi, lo;
        if (i >= 0 && i < a.ncmp) {
          const float4* src = reinterpret_cast<const float4*>(dxc + (long)i * D + 32 * kk + 8 * g4);
          const float4 x0 = src[0], x1 = src[1];
          const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            hi[e] = (__bf16)xv[e];
            lo[e] = (__bf16)(xv[e] - (float)hi[e]);
          }
        } else {
          hi = zero8();
          lo = zero8();
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          acc[ct][it] = mfma16x16x32(hi, bw[ct], acc[ct][it]);
          acc[ct][it] = mfma16x16x32(lo, bw[ct], acc[ct][it]);
        }
      }
    }
  }
  // lane holds C[u = u0 + it*16 + 4*g4 + e][feature wave*D/4 + ct*16 + r16]
#pragma unroll
  for (int it = 0; it < 4; ++it)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const long s = (long)(u0 + it * 16 + 4 * g4 + e) * a.d + r;
      if (s >= a.T) continue;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) dx[s * D + wave * (D / 4) + ct * 16 + r16] += acc[ct][it][e];
    }
}

// dW[j][e][c] = sum over (sequence-head, token i) of x[i d + j][e] dXc[i][c]: 64 x 64 output
// tiles, 16 reduction rows per step through LDS, 4 x 4 outputs per thread (fp32).
template <int D>
__global__ __launch_bounds__(256) void bwd_cmp_dw_kernel(BwdArgs a) {
  __shared__ float As[16][64];
  __shared__ float Bs[16][64];
  const int c0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int j = blockIdx.z % a.l, kv = blockIdx.z / a.l;
  const u16* x = kv ? a.v : a.k;
  const float* dxc = kv ? a.dvc : a.dkc;
  float* dw = kv ? a.dwv : a.dwk;
  const int tid = threadIdx.x;
  const int te = (tid / 16) * 4, tc = (tid % 16) * 4;
  float acc[4][4] = {};
  const long N = (long)a.B * a.Hkv * a.ncmp;
  for (long n0 = 0; n0 < N; n0 += 16) {
    for (int q = tid; q < 16 * 64; q += 256) {
      const int rr = q / 64, cc = q % 64;
      const long nn = n0 + rr;
      float av = 0.f, bv = 0.f;
      if (nn < N) {
        const long bg = nn / a.ncmp;
        const int i = (int)(nn % a.ncmp);
        const u16 xb = x[(bg * a.T + (long)i * a.d + j) * D + e0 + cc];
        av = __uint_as_float((uint32_t)xb << 16);
        bv = dxc[(bg * a.NCP + i) * D + c0 + cc];
      }
      As[rr][cc] = av;
      Bs[rr][cc] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float av[4], bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { av[u] = As[rr][te + u]; bv[u] = Bs[rr][tc + u]; }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] = fmaf(av[u], bv[w], acc[u][w]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
    *reinterpret_cast<float4*>(dw + ((long)j * D + e0 + te + u) * D + c0 + tc) =
        make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
}

template <int D>
static void launch_bwd_d(const BwdArgs& a, hipStream_t s, hipEvent_t* ev) {
  auto mark = [&](int i) {
    if (ev != nullptr) (void)hipEventRecord(ev[i], s);
  };
  const long nprep = (long)a.B * a.T * a.Hkv * D;
  bwd_prep_kernel<<<(unsigned)((nprep + 255) / 256), 256, 0, s>>>(a);
  launch_fill_zero(reinterpret_cast<float*>(a.selbits), (size_t)a.B * a.Hkv * a.nblk * a.SW, s);
  const long nsel = (long)a.B * a.T * a.Hkv;
  bwd_selbits_kernel<<<(unsigned)((nsel + 255) / 256), 256, 0, s>>>(a);
  mark(2);
  const dim3 gq((a.T + 3) / 4, a.Hkv, a.B);
  const dim3 gq8((a.T + 7) / 8, a.Hkv, a.B);
  bwd_q_shared_kernel<D, kBrCmp, 8><<<gq8, 512, 0, s>>>(a);
  bwd_q_kernel<D, kBrSlc><<<gq, 256, 0, s>>>(a);
  bwd_q_shared_kernel<D, kBrWin, 8><<<gq8, 512, 0, s>>>(a);
  mark(3);
  const int nkt = (a.T + 63) / 64;
  bwd_kv_kernel<D, kBrWin, 8><<<dim3((a.T + 127) / 128, a.B * a.Hkv, 1), 512, 0, s>>>(a);
  bwd_kv_kernel<D, kBrSlc, 4><<<dim3(nkt, a.B * a.Hkv, a.NPC), 256, 0, s>>>(a);
  const long nk = (long)a.B * a.Hkv * a.T * D;
  bwd_slc_reduce_kernel<<<(unsigned)((nk + 255) / 256), 256, 0, s>>>(a);
  if (a.ncmp > 0)
    // 64 compressed keys per workgroup (two workgroups per CU); the window pass keeps 128
    bwd_kv_kernel<D, kBrCmp, 4><<<dim3((a.NCP + 63) / 64, a.B * a.Hkv, a.NPC), 256, 0, s>>>(a);
  mark(4);
  if (a.ncmp > 0) {
    const long nr = (long)a.B * a.Hkv * a.NCP * D;
    bwd_cmp_reduce_kernel<<<(unsigned)((nr + 255) / 256), 256, 0, s>>>(a);
    const int nu = (a.T + a.d - 1) / a.d;  // token s = u d + r for u < nu
    bwd_cmp_dx_kernel<D><<<dim3((nu + 63) / 64, a.B * a.Hkv * a.d, 2), 256, 0, s>>>(a);
    bwd_cmp_dw_kernel<D><<<dim3(D / 64, D / 64, 2 * a.l), 256, 0, s>>>(a);
  } else {
    launch_fill_zero(a.dwk, (size_t)a.l * D * D, s);
    launch_fill_zero(a.dwv, (size_t)a.l * D * D, s);
  }
  mark(5);
}

void launch_backward(const BwdArgs& a, hipStream_t s, hipEvent_t* ev) {
  if (a.D == 128) launch_bwd_d<128>(a, s, ev);
  else launch_bwd_d<64>(a, s, ev);
}

}  // namespace nsa
