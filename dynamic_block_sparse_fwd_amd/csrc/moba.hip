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
//   moba_pool_kernel   kbar = mean of block keys, kept as bf16 hi + lo (kbar ~ hi + lo)
//   moba_gate_kernel   scores q . kbar on the matrix core (hi and lo), top-k per query,
//                      ascending index list
//   moba_count_kernel  per-block query counts and each entry's rank in its block's list
//   moba_scan_kernel   offsets of the per-block query lists and of their 128-row tiles
//   moba_fill_kernel   places every (query, slot) into its block's list (no atomics)
//   moba_block_kernel  gathered queries x block keys -> partial (max, sum, output)
//   moba_own_kernel    own block (causal) + merge of the partials -> out
#include "attn_tile.h"
#include "dev_common.h"
#include "kernels.h"

namespace nsa {

constexpr int MOBA_ROWS = 128;  // gathered queries per block-major tile

// A call runs its heads in chunks (a.H heads from a.h0 of a.Hs).  q, k, out and the index
// list are addressed with the caller's head count; the workspace arrays hold the chunk's heads.
__device__ __forceinline__ long moba_gbh(const MobaArgs& a, int b, int h) {
  return (long)b * a.Hs + a.h0 + h;  // (sequence, head) of the caller's k
}
__device__ __forceinline__ long moba_grow(const MobaArgs& a, int b, long t, int h) {
  return ((long)b * a.T + t) * a.Hs + a.h0 + h;  // row of the caller's q, out, index list
}

// kbar of one block: 16-byte loads, each thread sums 8 features over a stride of rows; the
// row groups are then added in a fixed order (fp32), and kbar is split into bf16 hi + lo.
template <int D>
__global__ __launch_bounds__(256) void moba_pool_kernel(MobaArgs a) {
  constexpr int DC = D / 8, NP = 256 / DC;
  __shared__ float part[NP][D];
  const int j = blockIdx.x;
  const long bh = blockIdx.y;
  const int dc = threadIdx.x % DC, p = threadIdx.x / DC;
  const long gbh = moba_gbh(a, (int)(bh / a.H), (int)(bh % a.H));
  const u16* src = a.k + (gbh * a.T + (long)j * a.block) * D + 8 * dc;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int r = p; r < a.block; r += NP) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(src + (long)r * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[2 * e] += __uint_as_float(w[e] << 16);
      s[2 * e + 1] += __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[p][8 * dc + e] = s[e];
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
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

// Order-preserving ranking key of a signed score: larger score first, then lower index
// (-0 and +0 compare equal, as in the scores' arithmetic).
__device__ __forceinline__ uint64_t signed_rank_key(float s, int j) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(o) << 32) | (0xFFFFFFFFu - (uint32_t)j);
}

// The KS best (score, block) pairs seen by one lane for one query, largest first.  Candidates
// arrive in increasing block order and displace only on a strictly larger score, so of two
// equal scores the lower block stays ahead.
template <int KS>
struct TopList {
  float v[KS];
  int j[KS];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int s = 0; s < KS; ++s) { v[s] = kNegInf; j[s] = 0; }
  }
  __device__ __forceinline__ void insert(float x, int jj) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bool gt = x > v[s];
      const float tv = v[s];
      const int tj = j[s];
      v[s] = gt ? x : tv;
      j[s] = gt ? jj : tj;
      x = gt ? tv : x;
      jj = gt ? tj : jj;
    }
  }
  __device__ __forceinline__ void pop() {
#pragma unroll
    for (int s = 0; s + 1 < KS; ++s) { v[s] = v[s + 1]; j[s] = j[s + 1]; }
    v[KS - 1] = kNegInf;
  }
};

// One workgroup scores 256 consecutive queries (4 waves x four 16-query sub-tiles) against every
// past block key on the matrix core; three workgroups share a CU, so one waiting at its per-tile
// barrier leaves the matrix cores to the others.  Each 16-block tile of kbar (bf16 hi and lo
// parts, two 16-byte pieces per thread) is staged in LDS once for the four waves
// (double-buffered, one barrier per tile; its rows
// chunk-swizzled so the 16 rows one operand read touches fall on distinct banks) and multiplies
// all of a wave's sub-tiles, as four independent accumulation chains; three tiles' loads are in
// flight.  Every lane keeps the top KS of its four blocks per tile for its queries; the four
// lanes of a query then merge.  The ascending index list is written.  An insert that does not
// beat the list's last entry changes nothing, so inserts run only where some lane of the wave
// needs one: with few blocks nearly every sub-tile has such a lane (one test per sub-tile, then
// its four inserts); with many (LATE) a lane's list rarely moves after the first tiles (one test
// per score).  Either way a lane inserts its scores in block order, so the lists are the same.
constexpr int kGateWaves = 4;
constexpr int kGateLateBlocks = 2048;  // blocks per head from which the gate tests per score

template <int D>
__device__ __forceinline__ int gate_swz(int row) { return row & (D / 8 - 1); }

template <int D, int KS, bool LATE>
__global__ __launch_bounds__(kGateWaves * 64, 3) void moba_gate_kernel(MobaArgs a) {
  constexpr int NU = 4, DC = D / 8;
  __shared__ __align__(16) u16 kbs[2][2][16][D];  // [buffer][hi, lo][block of the tile][feature]
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int tw = blockIdx.x * kGateWaves * 64;  // the workgroup's first query
  const int t0 = tw + wave * 64;
  const bool live = t0 < a.T;  // dead waves still pass the barriers
  const int bq = live ? t0 / a.block : 0;  // the wave's 64 queries share one block
  const int tlast = (tw + kGateWaves * 64 < a.T ? tw + kGateWaves * 64 : a.T) - 1;
  const int bq_max = tlast / a.block;  // the largest bq of the workgroup
  const long bh = (long)b * a.H + h;
  const int K = a.top_k;
  const int nsel = bq < K ? bq : K;
  const bool scoring = live && K > 0 && bq > K;  // uniform per wave
  int chosen[NU][KS];
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int s = 0; s < KS; ++s) chosen[u][s] = s;  // bq <= top_k: blocks 0 .. bq-1
  if (K > 0 && bq_max > K) {  // uniform per workgroup
    bf16x8 qf[NU][D / 32];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int tq = scoring ? t0 + 16 * u + r16 : 0;
      const u16* qp = a.q + moba_grow(a, b, tq, h) * D + 8 * g4;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) qf[u][c] = load8(qp + 32 * c);
    }
    // staging: thread -> (hi/lo part, row, 16-byte chunk); 4 D threads stage a tile (past the
    // last block the last one is loaded again, so the loads are unconditional)
    constexpr int NTH = kGateWaves * 64, NST = (4 * D + NTH - 1) / NTH;
    const bool stager = tid < 4 * D;
    int spart[NST], srow[NST], sch[NST];
    const u16* sbase[NST];
#pragma unroll
    for (int k = 0; k < NST; ++k) {
      const int c = tid + NTH * k;
      spart[k] = c / (16 * DC); srow[k] = (c / DC) % 16; sch[k] = c % DC;
      sbase[k] = (spart[k] ? a.kb_lo : a.kb_hi) + bh * a.nb * D + 8 * sch[k];
    }
    auto fetch = [&](int jt, int k) -> u32x4 {
      int jr = jt * 16 + srow[k];
      jr = jr < bq_max ? jr : bq_max - 1;
      return *reinterpret_cast<const u32x4*>(sbase[k] + (long)jr * D);
    };
    const int nt = (bq_max + 15) / 16;
    // one sweep over the tiles: visit(jt, x) receives, per sub-tile u, the scores x[u][i] of
    // block jt * 16 + 4 g4 + i for this lane's query (-inf past the wave's own past blocks)
    auto sweep = [&](auto visit) {
      // three tiles' loads in flight (an L2 round trip outlasts one tile's products)
      const u32x4 z4 = {0u, 0u, 0u, 0u};
      u32x4 p0[NST], p1[NST], p2[NST];
#pragma unroll
      for (int k = 0; k < NST; ++k) {
        p0[k] = stager ? fetch(0, k) : z4;
        p1[k] = stager ? fetch(1, k) : z4;
        p2[k] = stager ? fetch(2, k) : z4;
      }
      for (int jt = 0; jt < nt; ++jt) {
        const int buf = jt & 1;
        if (stager) {
#pragma unroll
          for (int k = 0; k < NST; ++k)
            *reinterpret_cast<u32x4*>(
                &kbs[buf][spart[k]][srow[k]][8 * (sch[k] ^ gate_swz<D>(srow[k]))]) = p0[k];
        }
        __syncthreads();  // tile jt staged; tile jt - 1's buffer is free again
#pragma unroll
        for (int k = 0; k < NST; ++k) {
          p0[k] = p1[k];
          p1[k] = p2[k];
          if (stager) p2[k] = fetch(jt + 3, k);
        }
        if (scoring && jt * 16 < bq) {  // uniform per wave
          bf16x8 kh[D / 32], kl[D / 32];
#pragma unroll
          for (int c = 0; c < D / 32; ++c) {
            const int ch = 8 * ((4 * c + g4) ^ gate_swz<D>(r16));
            kh[c] = load8(&kbs[buf][0][r16][ch]);
            kl[c] = load8(&kbs[buf][1][r16][ch]);
          }
          f32x4 acc[NU];
#pragma unroll
          for (int u = 0; u < NU; ++u) acc[u] = zero4();
#pragma unroll
          for (int c = 0; c < D / 32; ++c)
#pragma unroll
            for (int u = 0; u < NU; ++u) {
              acc[u] = mfma16x16x32(kh[c], qf[u][c], acc[u]);
              acc[u] = mfma16x16x32(kl[c], qf[u][c], acc[u]);
            }
          float x[NU][4];
#pragma unroll
          for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              x[u][i] = jt * 16 + 4 * g4 + i < bq ? acc[u][i] : kNegInf;
          visit(jt, x);
        }
      }
    };
    TopList<KS> lst[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) lst[u].init();
    sweep([&](int jt, float (&x)[NU][4]) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        if constexpr (LATE) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (__ballot(x[u][i] > lst[u].v[KS - 1]) != 0)  // uniform
              lst[u].insert(x[u][i], jt * 16 + 4 * g4 + i);
        } else {
          const float mx = fmaxf(fmaxf(x[u][0], x[u][1]), fmaxf(x[u][2], x[u][3]));
          if (__ballot(mx > lst[u].v[KS - 1]) != 0) {  // uniform
#pragma unroll
            for (int i = 0; i < 4; ++i) lst[u].insert(x[u][i], jt * 16 + 4 * g4 + i);
          }
        }
      }
    });
    if (scoring) {
      // merge the four lanes (L, L^16, L^32, L^48) that hold one query's candidates
#pragma unroll
      for (int u = 0; u < NU; ++u) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if (s < K) {
            const uint64_t mine =
                lst[u].v[0] == kNegInf ? 0 : signed_rank_key(lst[u].v[0], lst[u].j[0]);
            const uint64_t m = col_max4_u64(mine);
            if (mine == m) lst[u].pop();
            chosen[u][s] = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFu));
          }
        }
        // ascending order of the K chosen blocks
#pragma unroll
        for (int x = 0; x < KS; ++x)
#pragma unroll
          for (int y = 0; y + 1 < KS; ++y)
            if (y + 1 < K && chosen[u][y] > chosen[u][y + 1]) {
              const int tmp = chosen[u][y];
              chosen[u][y] = chosen[u][y + 1];
              chosen[u][y + 1] = tmp;
            }
      }
    }
  }
  if (!live) return;  // after the workgroup's last barrier
  if (g4 == 0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      int32_t* orow = a.idx + moba_grow(a, b, t0 + 16 * u + r16, h) * (K + 1);
#pragma unroll
      for (int s = 0; s < KS; ++s)
        if (s < nsel) orow[s] = chosen[u][s];
      orow[nsel] = bq;
      for (int s = nsel + 1; s <= K; ++s) orow[s] = -1;
    }
  }
}

// Per (sequence, head, T-chunk, range of kMobaCountBlocks blocks): how many of the chunk's
// queries chose each block of the range, and every such (query, slot)'s rank among them,
// counted with LDS atomics (no global atomics).  Each thread takes kCountRows rows per pass
// with every index load issued before the atomics.
constexpr int kCountThreads = 1024, kCountRows = 8;

template <int KS>
__global__ __launch_bounds__(kCountThreads) void moba_count_kernel(MobaArgs a) {
  extern __shared__ int cnt[];  // [blocks of the range]
  const int nr = (a.nb + kMobaCountBlocks - 1) / kMobaCountBlocks;
  const int chunk = blockIdx.x, h = (int)blockIdx.y / nr, b = blockIdx.z;
  const int jlo = ((int)blockIdx.y % nr) * kMobaCountBlocks;
  const int jhi = jlo + kMobaCountBlocks < a.nb ? jlo + kMobaCountBlocks : a.nb;
  const long bh = (long)b * a.H + h;
  const int K = a.top_k;
  const int slast = K > 0 ? K - 1 : 0;
  const int cl = (a.T + kMobaChunks - 1) / kMobaChunks;
  const int tbeg = chunk * cl, tend = tbeg + cl < a.T ? tbeg + cl : a.T;
  for (int j = threadIdx.x; j < jhi - jlo; j += kCountThreads) cnt[j] = 0;
  __syncthreads();
  for (int t0 = tbeg + threadIdx.x; t0 < tend; t0 += kCountThreads * kCountRows) {
    int jb[kCountRows][KS];
#pragma unroll
    for (int u = 0; u < kCountRows; ++u) {
      int t = t0 + u * kCountThreads;
      t = t < tend ? t : tend - 1;
      const int32_t* orow = a.idx + moba_grow(a, b, t, h) * (K + 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) jb[u][s] = orow[s < slast ? s : slast];
    }
#pragma unroll
    for (int u = 0; u < kCountRows; ++u) {
      const int t = t0 + u * kCountThreads;
      const int bq = t / a.block;
      const int nsel = t < tend ? (bq < K ? bq : K) : 0;
      const long rrow = bh * a.T + t;  // rank rows are head-major: the stores are contiguous
#pragma unroll
      for (int s = 0; s < KS; ++s)
        if (s < nsel && jb[u][s] >= jlo && jb[u][s] < jhi)
          a.rank[rrow * K + s] = atomicAdd(&cnt[jb[u][s] - jlo], 1);
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j < jhi - jlo; j += kCountThreads)
    a.count[(bh * a.nb + jlo + j) * kMobaChunks + chunk] = cnt[j];
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int moba_wave_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    v += lane >= o ? u : 0;
  }
  return v;
}

// Exclusive prefix sums of the list lengths and of their 128-row tile counts (one workgroup);
// each list's chunk counts become the chunk offsets inside the list, and every tile records
// its list.  1024 consecutive lists per step, one per thread (its kMobaChunks counts in two
// 16-byte loads), each step's sums scanned over the waves and added to the running totals of
// the steps before; the next step's counts are loaded during this one.
__global__ __launch_bounds__(1024) void moba_scan_kernel(MobaArgs a) {
  static_assert(kMobaChunks == 8, "a list's chunk counts are two 16-byte loads");
  __shared__ int wc[16], wt[16];
  __shared__ int carry_c, carry_t;
  const long n = (long)a.B * a.H * a.nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n == 0) {  // no lists (T < block)
    if (tid == 0) {
      a.ntiles[0] = 0;
      a.offset[0] = 0;
    }
    return;
  }
  int4* cnt4 = reinterpret_cast<int4*>(a.count);  // list e: cnt4[2 e], cnt4[2 e + 1]
  if (tid == 0) {
    carry_c = 0;
    carry_t = 0;
  }
  const long e0 = tid < n ? tid : n - 1;  // every load unconditional (index clamped)
  int4 n0 = cnt4[2 * e0], n1 = cnt4[2 * e0 + 1];
  for (long base = 0; base < n; base += 1024) {
    const long e = base + tid;
    const bool live = e < n;
    const int4 c0 = n0, c1 = n1;
    const long en = base + 1024 + tid < n ? base + 1024 + tid : n - 1;
    n0 = cnt4[2 * en];
    n1 = cnt4[2 * en + 1];
    const int v[kMobaChunks] = {live ? c0.x : 0, live ? c0.y : 0, live ? c0.z : 0,
                                live ? c0.w : 0, live ? c1.x : 0, live ? c1.y : 0,
                                live ? c1.z : 0, live ? c1.w : 0};
    int r[kMobaChunks], sv = 0;
#pragma unroll
    for (int c = 0; c < kMobaChunks; ++c) {
      r[c] = sv;
      sv += v[c];
    }
    const int nt = (sv + MOBA_ROWS - 1) / MOBA_ROWS;
    const int ic = moba_wave_scan(sv, lane), it = moba_wave_scan(nt, lane);
    if (lane == 63) {
      wc[wave] = ic;
      wt[wave] = it;
    }
    __syncthreads();  // the wave totals (and the carries of the step before) are posted
    int co = carry_c + ic - sv, to = carry_t + it - nt;  // exclusive
    for (int w = 0; w < wave; ++w) {
      co += wc[w];
      to += wt[w];
    }
    if (live) {
      cnt4[2 * e] = int4{r[0], r[1], r[2], r[3]};
      cnt4[2 * e + 1] = int4{r[4], r[5], r[6], r[7]};
      a.offset[e] = co;
      a.tstart[e] = to;
      for (int k = 0; k < nt; ++k) a.tile_entry[to + k] = (int)e;
    }
    __syncthreads();  // every thread has read wc, wt and the carries
    if (tid == 1023) {  // its inclusive sums close the step (0 past the end)
      carry_c = co + sv;
      carry_t = to + nt;
    }
  }
  __syncthreads();
  if (tid == 0) {
    a.ntiles[0] = carry_t;
    a.offset[n] = carry_c;  // end of the last list
  }
}

// Places every (query, slot) at its block's list offset + its chunk's offset in the list + its
// rank among the chunk's queries.  KS >= top_k slots per row: the row's block indices are
// loaded together, then every slot's offset, chunk offset and rank together (indices clamped
// into range, so no load waits behind a per-slot condition); only the stores are conditional.
template <int KS>
__global__ __launch_bounds__(256) void moba_fill_kernel(MobaArgs a) {
  // (b, h, t), t fastest: a wave's rows share a head, so their ranks are contiguous and their
  // entries of one block land close together in its list
  const long row = (long)blockIdx.x * 256 + threadIdx.x;
  if (row >= (long)a.B * a.H * a.T || a.nb == 0) return;  // nb = 0: no query selects a block
  const int t = (int)(row % a.T);
  const long bh = row / a.T;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int K = a.top_k, slast = K > 0 ? K - 1 : 0;
  const int bq = t / a.block;
  const int nsel = bq < K ? bq : K;
  const int chunk = t / ((a.T + kMobaChunks - 1) / kMobaChunks);
  const int32_t* irow = a.idx + moba_grow(a, b, t, h) * (K + 1);  // K + 1 entries
  int jb[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int v = irow[s < K ? s : K];
    jb[s] = v < 0 ? 0 : (v < a.nb ? v : a.nb - 1);
  }
  int off[KS], cnt[KS], rk[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const long e = bh * a.nb + jb[s];
    off[s] = a.offset[e];
    cnt[s] = a.count[e * kMobaChunks + chunk];
    rk[s] = a.rank[row * K + (s < slast ? s : slast)];  // K = 0: the spare slot 0
  }
#pragma unroll
  for (int s = 0; s < KS; ++s)
    if (s < nsel) a.list[off[s] + cnt[s] + rk[s]] = (t << 4) | s;
}

template <int D>
__global__ __launch_bounds__(256) void moba_block_kernel(MobaArgs a) {
  constexpr int RTW = 2, DT = D / 16;
  __shared__ u16 Ks[64][D];
  __shared__ u16 Vs[D][64];
  // XCD-contiguous order: workgroup i runs on XCD i % 8, so logical tiles are dealt out in eight
  // contiguous runs, one per XCD; the tiles of one (head, block) then share that XCD's L2 for
  // the block's K/V
  const int ntiles = a.ntiles[0];
  const int per = (ntiles + 7) / 8;
  const int tile = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if ((int)(blockIdx.x / 8) >= per || tile >= ntiles) return;
  const int e = a.tile_entry[tile];
  const long bh = e / a.nb;
  const int j = e % a.nb;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int kt_in = tile - a.tstart[e];
  const int base = a.offset[e] + kt_in * MOBA_ROWS;
  const int rem = a.offset[e + 1] - base;
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
    const u16* qp = a.q + moba_grow(a, b, en >= 0 ? rt_t[rt] : 0, h) * D + 8 * g4;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qf[rt][c] = en >= 0 ? load8(qp + 32 * c) : zero8();
  }
  const u16* kb = a.k + moba_gbh(a, b, h) * (long)a.T * D;
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
  const int nkt = a.block / 64;
  KTileRegs<D, 256> kr;
  VTileRegs<D, 256> vr;
  kr.load(kb, key0, a.T - 1);
  vr.load(vtb, a.T, key0);
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    kr.store(Ks);
    vr.store(Vs);
    __syncthreads();
    {  // next tile in flight while this one computes (the last re-fetches itself: no branch)
      const long nxt = key0 + 64L * (kt + 1 < nkt ? kt + 1 : kt);
      kr.load(kb, nxt, a.T - 1);
      vr.load(vtb, a.T, nxt);
    }
    float z[RTW][16];
    score_tiles<D, RTW>(Ks, qf, g4, r16, z);
    bf16x8 pb[RTW][2];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      float tm = z[rt][0];
#pragma unroll
      for (int q = 1; q < 16; ++q) tm = fmaxf(tm, z[rt][q]);
      tm = col_max4(tm);
      // The reference max moves only when a score exceeds it by more than kLazyLog2 (log2
      // units): probabilities then stay below 2^kLazyLog2, and the rescale of O (a multiply
      // per accumulator) is skipped by the whole wave in the usual case.
      const bool move = tm * a.scale_log2 > mrun[rt] * a.scale_log2 + kLazyLog2;
      if (__ballot(move) != 0) {  // uniform
        const float mn = move ? tm : mrun[rt];
        const float alpha = move ? fast_exp2((mrun[rt] - mn) * a.scale_log2) : 1.f;
        mrun[rt] = mn;
        lrun[rt] *= alpha;
#pragma unroll
        for (int nn = 0; nn < DT; ++nn) O[rt][nn] *= alpha;
      }
      const float msl = mrun[rt] * a.scale_log2;
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float p = fast_exp2(fmaf(z[rt][q], a.scale_log2, -msl));
        sum += p;
        pb[rt][q >> 3][q & 7] = (__bf16)p;
      }
      lrun[rt] += sum;
    }
    pv_tiles<D, RTW>(Vs, pb, g4, r16, O);
  }
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const float L = col_sum4(lrun[rt]);
    // stored normalised by the partial's own sum (a convex combination of value rows) and by
    // the power of two at or above its largest magnitude, so fp16 keeps any bf16 value range
    // (|v| up to 3e38, or far below fp16's normal range) at full relative precision
    float mx = 0.f;
#pragma unroll
    for (int nn = 0; nn < DT; ++nn)
#pragma unroll
      for (int q = 0; q < 4; ++q) mx = fmaxf(mx, fabsf(O[rt][nn][q]));
    const float inv = 1.0f / L;  // a chosen past block always has visible keys: L > 0
    int ex = 0;
    (void)frexpf(col_max4(mx) * inv, &ex);  // = f 2^ex, f in [0.5, 1); 0 gives ex = 0
    ex = ex < -126 ? -126 : (ex > 127 ? 127 : ex);  // scale and 1 / scale both finite
    const float w = inv * ldexpf(1.f, -ex);          // exact power-of-two factor
    if (rt_t[rt] >= 0) {
      const long slot = (((long)b * a.T + rt_t[rt]) * a.H + h) * a.top_k + rt_s[rt];
      // the lane's output quads of column tiles 2 p and 2 p + 1 in one 16-byte piece at
      // 32 p + 8 g4 of the slot (moba_own_kernel reads them back whole)
      _Float16* op = a.po + slot * D;
#pragma unroll
      for (int p2 = 0; p2 < DT / 2; ++p2) {
        h16x8 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = (_Float16)(O[rt][2 * p2][q] * w);
          v[4 + q] = (_Float16)(O[rt][2 * p2 + 1][q] * w);
        }
        *reinterpret_cast<h16x8*>(op + 32 * p2 + 8 * g4) = v;
      }
      if (g4 == 0)
        *reinterpret_cast<f32x4*>(a.pml + slot * 4) =
            f32x4{mrun[rt] * a.scale_log2, L, ldexpf(1.f, ex), 0.f};
    }
  }
}

// Own block (causal) of 64 queries, then the merge with the KS partials of their chosen blocks
// (slots past the row's count are masked by selects, never multiplied in).
template <int D, int KS>
__global__ __launch_bounds__(256) void moba_own_kernel(MobaArgs a) {
  constexpr int RTW = 1, DT = D / 16;
  __shared__ u16 Ks[64][D];
  __shared__ u16 Vs[D][64];
  // XCD-contiguous order (workgroup i runs on XCD i % 8): the 64-query tiles of one own block
  // run on one XCD and share its L2 for the block's K/V
  const int ntq = a.T / 64, n = ntq * a.H * a.B;
  const int per = (n + 7) / 8;
  const int lin = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if ((int)(blockIdx.x / 8) >= per || lin >= n) return;
  const int tile = lin % ntq, h = (lin / ntq) % a.H, b = lin / (ntq * a.H);
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
    const u16* qp = a.q + moba_grow(a, b, row_t[rt], h) * D + 8 * g4;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qf[rt][c] = load8(qp + 32 * c);
  }
  const u16* kb = a.k + moba_gbh(a, b, h) * (long)a.T * D;
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
  KTileRegs<D, 256> kr;
  VTileRegs<D, 256> vr;
  kr.load(kb, (long)kt0 * 64, a.T - 1);
  vr.load(vtb, a.T, (long)kt0 * 64);
  for (int kt = kt0; kt <= kt1; ++kt) {
    __syncthreads();
    kr.store(Ks);
    vr.store(Vs);
    __syncthreads();
    {
      const long nxt = 64L * (kt < kt1 ? kt + 1 : kt);
      kr.load(kb, nxt, a.T - 1);
      vr.load(vtb, a.T, nxt);
    }
    const bool diag = kt == kt1;  // uniform: only the last tile needs the causal mask
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
      if (diag) {
        __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kt * 64 + 32 * (e >> 3) + 8 * g4 + 4 * ((e >> 2) & 1) + (e & 3);
          z[e] = key <= row_t[rt] ? z[e] : kNegInf;
        }
      }
      float tm = z[0];
#pragma unroll
      for (int q = 1; q < 16; ++q) tm = fmaxf(tm, z[q]);
      tm = col_max4(tm);  // finite: every row sees a key of every tile it reaches
      const bool move = tm > mrun[rt] + kLazyLog2;  // lazy rescale, as in the block kernel
      if (__ballot(move) != 0) {  // uniform
        const float mn = move ? tm : mrun[rt];
        const float alpha = move ? fast_exp2(mrun[rt] - mn) : 1.f;
        mrun[rt] = mn;
        lrun[rt] *= alpha;
#pragma unroll
        for (int nn = 0; nn < DT; ++nn) O[rt][nn] *= alpha;
      }
      const float mn = mrun[rt];
      float p[16], sum = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) { p[q] = fast_exp2(z[q] - mn); sum += p[q]; }
      lrun[rt] += sum;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        bf16x8 pb;
#pragma unroll
        for (int q = 0; q < 8; ++q) pb[q] = (__bf16)p[kc * 8 + q];
        pv_chunk<D>(Vs, pb, kc, g4, r16, O[rt]);
      }
    }
  }
  const int K = a.top_k;
  const int nsel = bq < K ? bq : K;
  const int slast = K > 0 ? K - 1 : 0;
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const long row = ((long)b * a.T + row_t[rt]) * a.H + h;
    float pm[KS], pl[KS], ps[KS];
    float4 pv[KS][DT];
#pragma unroll
    for (int s = 0; s < KS; ++s) {  // every load unconditional (slot index clamped)
      const long slot = row * K + (s < slast ? s : slast);
      const f32x4 st = *reinterpret_cast<const f32x4*>(a.pml + slot * 4);
      pm[s] = st[0];
      pl[s] = st[1];
      ps[s] = st[2];
      const _Float16* op = a.po + slot * D;
#pragma unroll
      for (int p2 = 0; p2 < DT / 2; ++p2) {
        const h16x8 v = *reinterpret_cast<const h16x8*>(op + 32 * p2 + 8 * g4);
        pv[s][2 * p2] = make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
        pv[s][2 * p2 + 1] = make_float4((float)v[4], (float)v[5], (float)v[6], (float)v[7]);
      }
    }
    float M = mrun[rt];
#pragma unroll
    for (int s = 0; s < KS; ++s) M = s < nsel ? fmaxf(M, pm[s]) : M;
    const float fo = fast_exp2(mrun[rt] - M);
    float L = col_sum4(lrun[rt]) * fo;
    float4 acc[DT];
#pragma unroll
    for (int nn = 0; nn < DT; ++nn)
      acc[nn] = make_float4(O[rt][nn][0] * fo, O[rt][nn][1] * fo, O[rt][nn][2] * fo,
                            O[rt][nn][3] * fo);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bool ok = s < nsel;
      // the partials are normalised: weight = their sum relative to the common max (times the
      // power-of-two scale of the stored outputs)
      const float f = ok ? pl[s] * fast_exp2(pm[s] - M) : 0.f;
      const float fo = f * (ok ? ps[s] : 0.f);
      L += f;
#pragma unroll
      for (int nn = 0; nn < DT; ++nn) {
        acc[nn].x += ok ? fo * pv[s][nn].x : 0.f;
        acc[nn].y += ok ? fo * pv[s][nn].y : 0.f;
        acc[nn].z += ok ? fo * pv[s][nn].z : 0.f;
        acc[nn].w += ok ? fo * pv[s][nn].w : 0.f;
      }
    }
    const float inv = 1.0f / L;
    float* dst = a.out + moba_grow(a, b, row_t[rt], h) * D;
#pragma unroll
    for (int nn = 0; nn < DT; ++nn)
      *reinterpret_cast<float4*>(dst + 16 * nn + 4 * g4) =
          make_float4(acc[nn].x * inv, acc[nn].y * inv, acc[nn].z * inv, acc[nn].w * inv);
  }
}

template <int D, int KS>
static void launch_moba_k(const MobaArgs& a, hipStream_t s, hipEvent_t* ev) {
  auto mark = [&](int i) {
    if (ev != nullptr) (void)hipEventRecord(ev[i], s);
  };
  const long rows = (long)a.B * a.T * a.H;
  const dim3 gp(a.nb, a.B * a.H), gg((a.T + kGateWaves * 64 - 1) / (kGateWaves * 64), a.H, a.B);
  moba_pool_kernel<D><<<gp, 256, 0, s>>>(a);
  if (a.nb > kGateLateBlocks) moba_gate_kernel<D, KS, true><<<gg, kGateWaves * 64, 0, s>>>(a);
  else moba_gate_kernel<D, KS, false><<<gg, kGateWaves * 64, 0, s>>>(a);
  mark(1);
  const int nr = (a.nb + kMobaCountBlocks - 1) / kMobaCountBlocks;
  const int cblk = a.nb < kMobaCountBlocks ? a.nb : kMobaCountBlocks;
  moba_count_kernel<KS><<<dim3(kMobaChunks, a.H * nr, a.B), kCountThreads,
                          (size_t)cblk * sizeof(int), s>>>(a);
  moba_scan_kernel<<<1, 1024, 0, s>>>(a);
  moba_fill_kernel<KS><<<(int)((rows + 255) / 256), 256, 0, s>>>(a);
  mark(2);
  if (a.max_tiles > 0) moba_block_kernel<D><<<(a.max_tiles + 7) / 8 * 8, 256, 0, s>>>(a);
  mark(3);
  moba_own_kernel<D, KS><<<(int)((rows / 64 + 7) / 8 * 8), 256, 0, s>>>(a);
  mark(4);
}

template <int D>
static void launch_moba_d(const MobaArgs& a, hipStream_t s, hipEvent_t* ev) {
  if (a.top_k <= 1) launch_moba_k<D, 1>(a, s, ev);
  else if (a.top_k == 2) launch_moba_k<D, 2>(a, s, ev);
  else if (a.top_k == 3) launch_moba_k<D, 3>(a, s, ev);
  else if (a.top_k == 4) launch_moba_k<D, 4>(a, s, ev);
  else launch_moba_k<D, 8>(a, s, ev);
}

void launch_moba(const MobaArgs& a, hipStream_t s, hipEvent_t* ev) {
  if (a.D == 128) launch_moba_d<128>(a, s, ev);
  else launch_moba_d<64>(a, s, ev);
}

}  // namespace nsa
