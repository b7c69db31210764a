// MoBA forward ("Zhang Xiaojun podcast EP94 notes", sections 9-10; podcast transcript "Late
// Talk #103"): per head, block keys are the mean of each block's keys (no parameters), each
// query keeps its top-k past blocks by q . kbar plus its own block, and attends causally over
// their union with one softmax.
//
// The notes describe the implementation as: for every KV block, gather the queries that chose
// it into a contiguous tile and run dense attention on it.  Here that is one block-major
// kernel (gathered query rows x one block's keys, partial max/sum/output per query and slot)
// and one query-major kernel that attends the causal own block and merges the partials.
//
//   moba_zero_kernel   clears per-block counters
//   moba_pool_kernel   kbar = mean of block keys, kept as bf16 hi + lo (kbar ~ hi + lo)
//   moba_gate_kernel   scores q . kbar on the matrix core (hi and lo), top-k per query,
//                      ascending index list, per-block query counts
//   moba_scan_kernel   offsets of the per-block query lists and of their 128-row tiles
//   moba_fill_kernel   places every (query, slot) into its block's list
//   moba_block_kernel  gathered queries x block keys -> partial (max, sum, output)
//   moba_own_kernel    own block (causal) + merge of the partials -> out
#include "attn_tile.h"
#include "dev_common.h"
#include "kernels.h"

namespace nsa {

constexpr int MOBA_ROWS = 128;  // gathered queries per block-major tile
constexpr int MOBA_KMAX = 8;    // largest top_k kept in registers

__global__ void moba_zero_kernel(int32_t* a, int32_t* b, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) { a[i] = 0; b[i] = 0; }
}

template <int D>
__global__ __launch_bounds__(256) void moba_pool_kernel(MobaArgs a) {
  constexpr int NP = 256 / D;
  __shared__ float part[NP][D];
  const int j = blockIdx.x;
  const long bh = blockIdx.y;
  const int d = threadIdx.x % D, p = threadIdx.x / D;
  const int per = a.block / NP;
  const u16* src = a.k + (bh * a.T + (long)j * a.block + p * per) * D + d;
  float s = 0.f;
  for (int r = 0; r < per; ++r) s += bf16_to_f32(src[(long)r * D]);
  part[p][d] = s;
  __syncthreads();
  if (threadIdx.x < D) {
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < NP; ++q) tot += part[q][d];
    const float kbar = tot / (float)a.block;
    const u16 hi = f32_to_bf16(kbar);
    const u16 lo = f32_to_bf16(kbar - bf16_to_f32(hi));
    const long o = (bh * a.nb + j) * D + d;
    a.kb_hi[o] = hi;
    a.kb_lo[o] = lo;
  }
}

// Order-preserving ranking key of a signed score: larger score first, then lower index.
__device__ __forceinline__ uint64_t signed_rank_key(float s, int j) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(o) << 32) | (0xFFFFFFFFu - (uint32_t)j);
}

template <int D>
__global__ __launch_bounds__(256) void moba_gate_kernel(MobaArgs a) {
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int t0 = tile * 64;
  const int bq = t0 / a.block;  // every query of the tile sits in this block
  const int t = t0 + 16 * wave + r16;
  const long bh = (long)b * a.H + h;
  const int K = a.top_k;
  const int nsel = bq < K ? bq : K;
  int chosen[MOBA_KMAX];
#pragma unroll
  for (int s = 0; s < MOBA_KMAX; ++s) chosen[s] = s;  // the b <= top_k case: blocks 0..b-1
  if (bq > K) {
    bf16x8 qf[D / 32];
    const u16* qp = a.q + (((long)b * a.T + t) * a.H + h) * D + 8 * g4;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qf[c] = load8(qp + 32 * c);
    uint64_t cand[MOBA_KMAX];
#pragma unroll
    for (int s = 0; s < MOBA_KMAX; ++s) cand[s] = 0;
    const u16* hib = a.kb_hi + bh * a.nb * D + 8 * g4;
    const u16* lob = a.kb_lo + bh * a.nb * D + 8 * g4;
    for (int jt = 0; jt * 16 < bq; ++jt) {
      int jr = jt * 16 + r16;
      jr = jr < bq ? jr : bq - 1;
      f32x4 acc = zero4();
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        acc = mfma16x16x32(load8(hib + (long)jr * D + 32 * c), qf[c], acc);
        acc = mfma16x16x32(load8(lob + (long)jr * D + 32 * c), qf[c], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = jt * 16 + 4 * g4 + i;
        uint64_t key = j < bq ? signed_rank_key(acc[i], j) : 0;
#pragma unroll
        for (int s = 0; s < MOBA_KMAX; ++s) {
          const uint64_t c0 = cand[s];
          const bool gt = key > c0;
          cand[s] = gt ? key : c0;
          key = gt ? c0 : key;
        }
      }
    }
    // merge the four lanes that hold this query's candidates
#pragma unroll
    for (int s = 0; s < MOBA_KMAX; ++s) {
      if (s < K) {
        uint64_t m = cand[0];
        m = u64_max(m, shfl_xor_u64(m, 16));
        m = u64_max(m, shfl_xor_u64(m, 32));
        if (cand[0] == m) {
#pragma unroll
          for (int q = 0; q + 1 < MOBA_KMAX; ++q) cand[q] = cand[q + 1];
          cand[MOBA_KMAX - 1] = 0;
        }
        chosen[s] = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFu));
      }
    }
    // ascending order of the K chosen blocks
#pragma unroll
    for (int x = 0; x < MOBA_KMAX; ++x)
#pragma unroll
      for (int y = 0; y + 1 < MOBA_KMAX; ++y)
        if (y + 1 < K && chosen[y] > chosen[y + 1]) {
          const int tmp = chosen[y];
          chosen[y] = chosen[y + 1];
          chosen[y + 1] = tmp;
        }
  }
  if (g4 == 0) {
    int32_t* orow = a.idx + (((long)b * a.T + t) * a.H + h) * (K + 1);
#pragma unroll
    for (int s = 0; s < MOBA_KMAX; ++s)
      if (s < nsel) {
        orow[s] = chosen[s];
        atomicAdd(&a.count[bh * a.nb + chosen[s]], 1);
      }
    orow[nsel] = bq;
    for (int s = nsel + 1; s <= K; ++s) orow[s] = -1;
  }
}

// Exclusive prefix sums of the list lengths and of their 128-row tile counts (one workgroup).
__global__ __launch_bounds__(1024) void moba_scan_kernel(MobaArgs a) {
  __shared__ int sc[1024], st[1024];
  const int n = a.B * a.H * a.nb;
  const int per = (n + 1023) / 1024;
  const int lo = threadIdx.x * per, hi = lo + per < n ? lo + per : n;
  int c = 0, tl = 0;
  for (int e = lo; e < hi; ++e) {
    const int v = a.count[e];
    c += v;
    tl += (v + MOBA_ROWS - 1) / MOBA_ROWS;
  }
  sc[threadIdx.x] = c;
  st[threadIdx.x] = tl;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int vc = threadIdx.x >= o ? sc[threadIdx.x - o] : 0;
    const int vt = threadIdx.x >= o ? st[threadIdx.x - o] : 0;
    __syncthreads();
    sc[threadIdx.x] += vc;
    st[threadIdx.x] += vt;
    __syncthreads();
  }
  int co = sc[threadIdx.x] - c, to = st[threadIdx.x] - tl;  // exclusive
  for (int e = lo; e < hi; ++e) {
    const int v = a.count[e];
    a.offset[e] = co;
    a.tstart[e] = to;
    co += v;
    to += (v + MOBA_ROWS - 1) / MOBA_ROWS;
  }
  if (threadIdx.x == 1023) a.ntiles[0] = st[1023];
}

__global__ __launch_bounds__(256) void moba_fill_kernel(MobaArgs a) {
  const long row = (long)blockIdx.x * 256 + threadIdx.x;  // (b, t, h)
  if (row >= (long)a.B * a.T * a.H) return;
  const int h = (int)(row % a.H);
  const long bt = row / a.H;
  const int t = (int)(bt % a.T), b = (int)(bt / a.T);
  const int bq = t / a.block;
  const int nsel = bq < a.top_k ? bq : a.top_k;
  const long bh = (long)b * a.H + h;
  const int32_t* irow = a.idx + row * (a.top_k + 1);
  for (int s = 0; s < nsel; ++s) {
    const int j = irow[s];
    const long e = bh * a.nb + j;
    const int pos = a.offset[e] + atomicAdd(&a.cursor[e], 1);
    a.list[pos] = (t << 4) | s;
  }
}

template <int D>
__global__ __launch_bounds__(256) void moba_block_kernel(MobaArgs a) {
  constexpr int RTW = 2, DT = D / 16;
  __shared__ u16 Ks[64][D];
  __shared__ u16 Vs[D][64];
  __shared__ int ent;
  const int tile = blockIdx.x;
  if (tile >= a.ntiles[0]) return;
  const int n = a.B * a.H * a.nb;
  if (threadIdx.x == 0) {  // last list whose first tile is <= this tile
    int lo = 0, hi = n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tstart[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    ent = lo;
  }
  __syncthreads();
  const int e = ent;
  const long bh = e / a.nb;
  const int j = e % a.nb;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int kt_in = tile - a.tstart[e];
  const int base = a.offset[e] + kt_in * MOBA_ROWS;
  const int rem = a.count[e] - kt_in * MOBA_ROWS;
  const int cnt = rem < MOBA_ROWS ? rem : MOBA_ROWS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;

  bf16x8 qf[RTW][D / 32];
  int rt_t[RTW], rt_s[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int r = (wave * RTW + rt) * 16 + r16;
    const int en = r < cnt ? a.list[base + r] : -1;
    rt_t[rt] = en >= 0 ? (en >> 4) : -1;
    rt_s[rt] = en >= 0 ? (en & 15) : 0;
    const u16* qp = a.q + (((long)b * a.T + (en >= 0 ? rt_t[rt] : 0)) * a.H + h) * D + 8 * g4;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qf[rt][c] = en >= 0 ? load8(qp + 32 * c) : zero8();
  }
  const u16* kb = a.k + bh * (long)a.T * D;
  const u16* vtb = a.vt + bh * (long)D * a.T;
  float mrun[RTW], lrun[RTW];
  f32x4 O[RTW][DT];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    mrun[rt] = kNegInf;
    lrun[rt] = 0.f;
#pragma unroll
    for (int nn = 0; nn < DT; ++nn) O[rt][nn] = zero4();
  }
  const long key0 = (long)j * a.block;
  for (int kt = 0; kt < a.block / 64; ++kt) {
    __syncthreads();
    load_rows_tile<D, 256>(Ks, kb, key0 + kt * 64, a.T - 1);
    load_cols_tile<D, 256>(Vs, vtb, a.T, key0 + kt * 64);
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      float z[16];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const f32x4 acc = score_subtile<D>(Ks, qf[rt], kc, s, g4, r16);
#pragma unroll
          for (int i = 0; i < 4; ++i) z[kc * 8 + s * 4 + i] = acc[i] * a.scale_log2;
        }
      float tm = z[0];
#pragma unroll
      for (int q = 1; q < 16; ++q) tm = fmaxf(tm, z[q]);
      tm = col_max4(tm);
      const float mn = fmaxf(mrun[rt], tm);
      const float alpha = fast_exp2(mrun[rt] - mn);
      mrun[rt] = mn;
      float p[16], sum = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) { p[q] = fast_exp2(z[q] - mn); sum += p[q]; }
      lrun[rt] = lrun[rt] * alpha + sum;
#pragma unroll
      for (int nn = 0; nn < DT; ++nn) O[rt][nn] *= alpha;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        bf16x8 pb;
#pragma unroll
        for (int q = 0; q < 8; ++q) pb[q] = (__bf16)p[kc * 8 + q];
        pv_chunk<D>(Vs, pb, kc, g4, r16, O[rt]);
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const float L = col_sum4(lrun[rt]);
    if (rt_t[rt] >= 0) {
      const long slot = (((long)b * a.T + rt_t[rt]) * a.H + h) * a.top_k + rt_s[rt];
      float* op = a.po + slot * D;
#pragma unroll
      for (int nn = 0; nn < DT; ++nn)
        *reinterpret_cast<float4*>(op + 16 * nn + 4 * g4) =
            make_float4(O[rt][nn][0], O[rt][nn][1], O[rt][nn][2], O[rt][nn][3]);
      if (g4 == 0) {
        a.pml[slot * 2 + 0] = mrun[rt];
        a.pml[slot * 2 + 1] = L;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(128) void moba_own_kernel(MobaArgs a) {
  constexpr int RTW = 2, DT = D / 16;
  __shared__ u16 Ks[64][D];
  __shared__ u16 Vs[D][64];
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int t0 = tile * 64;
  const int bq = t0 / a.block;
  const long bh = (long)b * a.H + h;
  bf16x8 qf[RTW][D / 32];
  int row_t[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    row_t[rt] = t0 + (wave * RTW + rt) * 16 + r16;
    const u16* qp = a.q + (((long)b * a.T + row_t[rt]) * a.H + h) * D + 8 * g4;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qf[rt][c] = load8(qp + 32 * c);
  }
  const u16* kb = a.k + bh * (long)a.T * D;
  const u16* vtb = a.vt + bh * (long)D * a.T;
  float mrun[RTW], lrun[RTW];
  f32x4 O[RTW][DT];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    mrun[rt] = kNegInf;
    lrun[rt] = 0.f;
#pragma unroll
    for (int nn = 0; nn < DT; ++nn) O[rt][nn] = zero4();
  }
  const int kt0 = (bq * a.block) / 64, kt1 = (t0 + 63) / 64;
  for (int kt = kt0; kt <= kt1; ++kt) {
    __syncthreads();
    load_rows_tile<D, 128>(Ks, kb, (long)kt * 64, a.T - 1);
    load_cols_tile<D, 128>(Vs, vtb, a.T, (long)kt * 64);
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      float z[16];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const f32x4 acc = score_subtile<D>(Ks, qf[rt], kc, s, g4, r16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kt * 64 + 32 * kc + 8 * g4 + 4 * s + i;
            z[kc * 8 + s * 4 + i] = key <= row_t[rt] ? acc[i] * a.scale_log2 : kNegInf;
          }
        }
      float tm = z[0];
#pragma unroll
      for (int q = 1; q < 16; ++q) tm = fmaxf(tm, z[q]);
      tm = col_max4(tm);
      const float mn = fmaxf(mrun[rt], tm);
      const float ms = mn == kNegInf ? 0.f : mn;
      const float alpha = fast_exp2(mrun[rt] - ms);
      mrun[rt] = mn;
      float p[16], sum = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) { p[q] = fast_exp2(z[q] - ms); sum += p[q]; }
      lrun[rt] = lrun[rt] * alpha + sum;
#pragma unroll
      for (int nn = 0; nn < DT; ++nn) O[rt][nn] *= alpha;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        bf16x8 pb;
#pragma unroll
        for (int q = 0; q < 8; ++q) pb[q] = (__bf16)p[kc * 8 + q];
        pv_chunk<D>(Vs, pb, kc, g4, r16, O[rt]);
      }
    }
  }
  const int nsel = bq < a.top_k ? bq : a.top_k;
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int t = row_t[rt];
    const long row = ((long)b * a.T + t) * a.H + h;
    float M = mrun[rt];
    for (int s = 0; s < nsel; ++s) M = fmaxf(M, a.pml[(row * a.top_k + s) * 2]);
    const float fo = fast_exp2(mrun[rt] - M);
    float L = col_sum4(lrun[rt]) * fo;
    float4 acc[DT];
#pragma unroll
    for (int nn = 0; nn < DT; ++nn)
      acc[nn] = make_float4(O[rt][nn][0] * fo, O[rt][nn][1] * fo, O[rt][nn][2] * fo,
                            O[rt][nn][3] * fo);
    for (int s = 0; s < nsel; ++s) {
      const long slot = row * a.top_k + s;
      const float f = fast_exp2(a.pml[slot * 2] - M);
      L += a.pml[slot * 2 + 1] * f;
      const float* op = a.po + slot * D;
#pragma unroll
      for (int nn = 0; nn < DT; ++nn) {
        const float4 v = *reinterpret_cast<const float4*>(op + 16 * nn + 4 * g4);
        acc[nn].x += f * v.x;
        acc[nn].y += f * v.y;
        acc[nn].z += f * v.z;
        acc[nn].w += f * v.w;
      }
    }
    const float inv = 1.0f / L;
    float* dst = a.out + row * D;
#pragma unroll
    for (int nn = 0; nn < DT; ++nn)
      *reinterpret_cast<float4*>(dst + 16 * nn + 4 * g4) =
          make_float4(acc[nn].x * inv, acc[nn].y * inv, acc[nn].z * inv, acc[nn].w * inv);
  }
}

void launch_moba(const MobaArgs& a, hipStream_t s, hipEvent_t* ev) {
  auto mark = [&](int i) {
    if (ev != nullptr) (void)hipEventRecord(ev[i], s);
  };
  const int n = a.B * a.H * a.nb;
  moba_zero_kernel<<<(n + 255) / 256, 256, 0, s>>>(a.count, a.cursor, n);
  const long rows = (long)a.B * a.T * a.H;
  const dim3 gp(a.nb, a.B * a.H), gq(a.T / 64, a.H, a.B);
  if (a.D == 128) {
    moba_pool_kernel<128><<<gp, 256, 0, s>>>(a);
    moba_gate_kernel<128><<<gq, 256, 0, s>>>(a);
  } else {
    moba_pool_kernel<64><<<gp, 256, 0, s>>>(a);
    moba_gate_kernel<64><<<gq, 256, 0, s>>>(a);
  }
  mark(1);
  moba_scan_kernel<<<1, 1024, 0, s>>>(a);
  moba_fill_kernel<<<(int)((rows + 255) / 256), 256, 0, s>>>(a);
  mark(2);
  if (a.max_tiles > 0) {
    if (a.D == 128) moba_block_kernel<128><<<a.max_tiles, 256, 0, s>>>(a);
    else moba_block_kernel<64><<<a.max_tiles, 256, 0, s>>>(a);
  }
  mark(3);
  if (a.D == 128) moba_own_kernel<128><<<gq, 128, 0, s>>>(a);
  else moba_own_kernel<64><<<gq, 128, 0, s>>>(a);
  mark(4);
}

}  // namespace nsa
