// Selected-block branch of the NSA prefill ("Zhang Xiaojun podcast EP94 notes", sections 5-6:
// each position attends over the tokens of its top-n blocks, the group's heads stacked into the
// matrix-core M dimension because they share one selection).
//
// With independent selections, neighbouring positions share only the forced blocks (block 0 and
// the local blocks), while every other chosen block is picked by hundreds of positions spread
// over the sequence.  So the branch runs in two parts:
//   block-major   per (T-chunk, sequence-group, 64-key tile), the list of (position, slot)
//                 entries that chose the tile (slc_count / slc_scan / slc_fill); one workgroup
//                 per kSlcRows entries stages the tile's K and V^T in LDS once and writes each
//                 entry's partial softmax (own max and sum, output normalised by the sum and by
//                 a power-of-two scale, in fp16) -- slc_block_kernel
//   position-major one wave per position, 16 positions per workgroup: the shared tiles (the
//                 forced blocks) from LDS, then the position's partials merged in slot order;
//                 out += g1 * o_slc -- selected_kernel
// Lists are built chunk-major (all entries of positions in T-chunk 0 first), so the queries one
// wave of work tiles reads stay a cache-sized slice of q.
#include "attn_tile.h"
#include "dev_common.h"
#include "kernels.h"

namespace nsa {

constexpr int kSelWaves = 16;  // positions per workgroup of the position-major kernel
constexpr int kSelShared = 3;  // tiles staged in LDS per workgroup

// The tiles the workgroup of positions t0 .. t0 + kSelWaves - 1 shares: the current block's
// tiles up to t0, the other local blocks' tiles, then block 0's first tile, at most kSelShared
// of them (block size a multiple of 64 and t0 of kSelWaves, so the positions share one block).
// In closed form, three scalars: no indexed array (it would live in scratch memory).
struct SelShared {
  int k0, k1, k2, n;
  __device__ __forceinline__ int key(int i) const { return i == 0 ? k0 : (i == 1 ? k1 : k2); }
};

__device__ __forceinline__ SelShared sel_shared(const PrefillArgs& a, int t0) {
  const int bcur = t0 / a.beta, per = a.beta >> 6;
  // candidates in order: bcur's tiles at or before t0, the tiles of blocks bcur-1 .. down to
  // max(0, bcur - n_local + 1), block 0's first tile when block 0 is not itself local
  const int ncur = a.n_local >= 1 ? min(per, (t0 - bcur * a.beta) / 64 + 1) : 0;
  const int nloc = a.n_local >= 1 ? min(bcur, a.n_local - 1) * per : 0;
  const int nzero = bcur - a.n_local >= 0 ? 1 : 0;
  auto cand = [&](int i) {
    if (i < ncur) return bcur * a.beta + 64 * i;
    const int i2 = i - ncur;
    if (i2 < nloc) return (bcur - 1 - i2 / per) * a.beta + 64 * (i2 % per);
    return 0;
  };
  SelShared s;
  s.n = min(kSelShared, ncur + nloc + nzero);
  s.k0 = s.n > 0 ? cand(0) : -1;
  s.k1 = s.n > 1 ? cand(1) : -1;
  s.k2 = s.n > 2 ? cand(2) : -1;
  return s;
}

// Lane e < top_n * per: first key of the e-th selected 64-key tile of position t (block
// idx[e / per], sub-tile e % per), or -1 for padding, a block outside [0, nblk) or a tile past t.
__device__ __forceinline__ int sel_tile_key(const PrefillArgs& a, int b, int kvh, int t,
                                            int lane) {
  const int per = a.beta >> 6;
  int k0 = -1;
  if (lane < a.top_n * per) {
    const int j = a.idx[(prow(a, b, t) * a.Hkv + kvh) * a.top_n + lane / per];
    const int kk = j * a.beta + 64 * (lane % per);
    if (j >= 0 && j < a.nblk && kk <= t) k0 = kk;
  }
  return k0;
}

// Lane e < top_n * per of a position's index row: its block slot e / per and its sub-tile
// e % per, the same for every position (computed once per lane).
struct LaneTile {
  int slot, sub;
  bool on;
};

__device__ __forceinline__ LaneTile lane_tile(const PrefillArgs& a, int lane) {
  const int per = a.beta >> 6;
  return LaneTile{lane / per, lane % per, lane < a.top_n * per};
}

// The lane's tile key of position t, given the block j its index row holds in the lane's slot
// (as sel_tile_key), if it is not one of the tiles `sh` shared by t's workgroup of the
// position-major kernel, else -1.
__device__ __forceinline__ int free_tile_key(const PrefillArgs& a, int j, int t,
                                             const LaneTile& lt, const SelShared& sh) {
  int k0 = -1;
  if (lt.on) {
    const int kk = j * a.beta + 64 * lt.sub;
    if (j >= 0 && j < a.nblk && kk <= t) k0 = kk;
  }
#pragma unroll
  for (int i = 0; i < kSelShared; ++i)
    if (i < sh.n && k0 == sh.key(i)) k0 = -1;
  return k0;
}

__device__ __forceinline__ int lanes_below(uint64_t m, int lane) {
  return (int)__popcll(m & ((1ull << lane) - 1ull));
}

// ------------------------------------------------------------------ lists

constexpr int kSlcCountThreads = 1024;

// Per (T-chunk, group, sequence): the free tiles of every position are listed (their rank among
// the row's free tiles is the slot fs); every entry's rank among the chunk's entries of its key
// tile comes from LDS counters (no global atomics), the counts per key tile are written out.
// A wave takes the kSelWaves positions that share one workgroup of the position-major kernel
// at a time: their shared tiles (scalar arithmetic with divisions) are found once, and their
// index loads are in flight together.
__global__ __launch_bounds__(kSlcCountThreads) void slc_count_kernel(PrefillArgs a) {
  extern __shared__ int cnt[];  // [NTK]
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const long bkv = (long)b * a.Hkv + kvh;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // positions: uniform
  const LaneTile lt = lane_tile(a, lane);
  const int cl = (a.nq + a.SC - 1) / a.SC;
  const int r0 = c * cl, r1 = r0 + cl < a.nq ? r0 + cl : a.nq;
  for (int i = threadIdx.x; i < a.NTK; i += kSlcCountThreads) cnt[i] = 0;
  __syncthreads();
  constexpr int W = kSlcCountThreads / 64, U = kSelWaves;
  // position groups (rows r = U g .. U g + U - 1, relative to q0) overlapping [r0, r1)
  // consecutive positions: index rows si ints apart, entry rows ss apart
  const int si = a.Hkv * a.top_n, ss = a.Hkv * a.FS;
  for (int g = r0 / U + wave; g * U < r1; g += W) {  // wave-uniform
    const int rg = g * U;
    const SelShared sh = sel_shared(a, a.q0 + rg);
    const int32_t* irow = a.idx + (prow(a, b, a.q0 + rg) * a.Hkv + kvh) * a.top_n;
    const long sbase = (((long)b * a.nq + rg) * a.Hkv + kvh) * a.FS;
    // the U index loads unconditional (rows outside [r0, r1) clamped into it, lanes past the
    // row's slots at slot 0) and issued together before any of them is used
    int jv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int r = rg + u;
      r = r < r0 ? r0 : (r < r1 ? r : r1 - 1);
      jv[u] = irow[(r - rg) * si + (lt.on ? lt.slot : 0)];
    }
    __builtin_amdgcn_sched_barrier(0);
    int k0[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rg + u;
      k0[u] = r >= r0 && r < r1 ? free_tile_key(a, jv[u], a.q0 + r, lt, sh) : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rg + u;
      if (r < r0 || r >= r1) continue;  // uniform
      const uint64_t m = __ballot(k0[u] >= 0);
      const int nfree = (int)__popcll(m);
      int32_t* rk = a.s_rank + sbase + u * ss;
      int32_t* kt = a.s_kt + sbase + u * ss;
      if (k0[u] >= 0) {
        const int fs = lanes_below(m, lane);
        rk[fs] = atomicAdd(&cnt[k0[u] >> 6], 1);
        kt[fs] = k0[u] >> 6;
      }
      if (lane >= nfree && lane < a.FS) kt[lane] = -1;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < a.NTK; i += kSlcCountThreads)
    a.s_count[((long)c * a.B * a.Hkv + bkv) * a.NTK + i] = cnt[i];
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    v += lane >= o ? u : 0;
  }
  return v;
}

// Exclusive prefix sums of the sub-list lengths and of their kSlcRows-entry tile counts (one
// workgroup, sub-lists in (chunk, sequence-group, key tile) order), and the sub-list of every
// work tile.  4096 consecutive sub-lists per step, four per thread (one 16-byte load; the count
// is a multiple of the T-chunk count, itself a multiple of 4), each step's sums scanned over the
// waves and added to the running totals of the steps before; the next step's counts are loaded
// during this one.
__global__ __launch_bounds__(1024) void slc_scan_kernel(PrefillArgs a) {
  static_assert(kSlcChunks % 4 == 0, "four sub-lists per thread");
  __shared__ int wc[16], wt[16];
  __shared__ int carry_c, carry_t;
  const long n = (long)a.SC * a.B * a.Hkv * a.NTK;
  const long n4 = n / 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int4* cnt4 = reinterpret_cast<const int4*>(a.s_count);
  if (tid == 0) {
    carry_c = 0;
    carry_t = 0;
  }
  int4 v_next = cnt4[tid < n4 ? tid : n4 - 1];  // every load unconditional (index clamped)
  for (long base = 0; base < n4; base += 1024) {
    const long q = base + tid;  // this thread's sub-lists 4 q .. 4 q + 3
    const bool live = q < n4;
    const int4 v4 = v_next;
    const long qn = base + 1024 + tid;
    v_next = cnt4[qn < n4 ? qn : n4 - 1];
    const int v[4] = {live ? v4.x : 0, live ? v4.y : 0, live ? v4.z : 0, live ? v4.w : 0};
    int nt[4], sv = 0, st = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nt[i] = (v[i] + kSlcRows - 1) / kSlcRows;
      sv += v[i];
      st += nt[i];
    }
    const int ic = wave_incl_scan(sv, lane), it = wave_incl_scan(st, lane);
    if (lane == 63) {
      wc[wave] = ic;
      wt[wave] = it;
    }
    __syncthreads();  // the wave totals (and the carries of the step before) are posted
    int co = carry_c + ic - sv, to = carry_t + it - st;  // exclusive
    for (int w = 0; w < wave; ++w) {
      co += wc[w];
      to += wt[w];
    }
    if (live) {
      const int4 o4 = {co, co + v[0], co + v[0] + v[1], co + v[0] + v[1] + v[2]};
      const int4 t4 = {to, to + nt[0], to + nt[0] + nt[1], to + nt[0] + nt[1] + nt[2]};
      reinterpret_cast<int4*>(a.s_offset)[q] = o4;
      reinterpret_cast<int4*>(a.s_tstart)[q] = t4;
      int tt = to;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        for (int k = 0; k < nt[i]; ++k) a.s_tile_entry[tt++] = (int)(4 * q + i);
    }
    __syncthreads();  // every thread has read wc, wt and the carries
    if (tid == 1023) {  // its inclusive sums close the step (0 past the end)
      carry_c = co + sv;
      carry_t = to + st;
    }
  }
  __syncthreads();
  if (tid == 0) {
    a.s_ntiles[0] = carry_t;
    a.s_offset[n] = carry_c;
  }
}

// Every entry at its sub-list's offset + its rank.
__global__ __launch_bounds__(256) void slc_fill_kernel(PrefillArgs a) {
  const long id = (long)blockIdx.x * 256 + threadIdx.x;  // ((b * nq + r) * Hkv + kvh) * FS + fs
  if (id >= (long)a.B * a.nq * a.Hkv * a.FS) return;
  const int kt = a.s_kt[id];
  if (kt < 0) return;
  const int fs = (int)(id % a.FS);
  const long rg = id / a.FS;
  const int kvh = (int)(rg % a.Hkv);
  const long row = rg / a.Hkv;
  const int b = (int)(row / a.nq), r = (int)(row % a.nq);
  const int c = r / ((a.nq + a.SC - 1) / a.SC);
  const long e = ((long)c * a.B * a.Hkv + (long)b * a.Hkv + kvh) * a.NTK + kt;
  a.s_list[a.s_offset[e] + a.s_rank[id]] = (int)(row << 6) | fs;
}

// ------------------------------------------------------------------ block-major attention

// One work tile: up to kSlcRows entries of one key tile; the tile's K and V^T staged in LDS once,
// each wave takes the entry pairs (2 w, 2 w + 1), (2 w + 8, 2 w + 9), ... (one position = the
// group's 16 heads = one MFMA row tile; two positions share every K and V fragment read from
// LDS): S^T = K Q^T, the tile's own softmax, O^T = V^T P^T, and the partial written as
// fp16(O / (sum * scale)) with scale the power of two at or above max |O / sum| of the head (so
// any bf16 value range survives), plus (max in log2 units, sum, scale).
template <int D, int G>
__global__ __launch_bounds__(256) void slc_block_kernel(PrefillArgs a) {
  constexpr int DT = D / 16, RT = 2;
  __shared__ __align__(16) u16 Ks[64][D];
  __shared__ __align__(16) u16 Vs[D][64];
  const int tile = blockIdx.x;
  if (tile >= a.s_ntiles[0]) return;  // uniform
  const int e = a.s_tile_entry[tile];
  const int kt = e % a.NTK;
  const long bkv = (e / a.NTK) % ((long)a.B * a.Hkv);
  const int b = (int)(bkv / a.Hkv), kvh = (int)(bkv % a.Hkv);
  const int base = a.s_offset[e] + (tile - a.s_tstart[e]) * kSlcRows;
  const int rem = a.s_offset[e + 1] - base;
  const int cnt = rem < kSlcRows ? rem : kSlcRows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int Hq = a.Hkv * G;
  const bool hlive = r16 < G;
  const float sl = a.scale_log2;
  load_rows_tile<D, 256>(Ks, a.k + bkv * (long)a.ldk * D, (long)kt * 64, a.T - 1);
  load_cols_tile<D, 256>(Vs, a.vt + bkv * (long)D * a.TP, a.TP, (long)kt * 64);
  // entry i's code and queries (an index past the tile re-reads its last entry: unconditional
  // loads keep the wait counts exact); the next pair is loaded while the current one computes
  auto entry_q = [&](int i, int& en, bf16x8* qf) {
    en = a.s_list[base + (i < cnt ? i : cnt - 1)];
    const int t = a.q0 + (int)((en >> 6) % a.nq);
    const u16* qp = a.q + (prow(a, b, t) * Hq + kvh * G + (hlive ? r16 : 0)) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qf[c] = hlive ? load8(qp + 32 * c + 8 * g4) : zero8();
  };
  int en_n[RT];
  bf16x8 qn[RT][D / 32];
  const int i0 = 2 * wave;
#pragma unroll
  for (int r = 0; r < RT; ++r) entry_q(i0 + r, en_n[r], qn[r]);
  __syncthreads();
  for (int i = i0; i < cnt; i += 2 * 4) {  // wave-uniform
    int en[RT];
    bf16x8 qf[RT][D / 32];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      en[r] = en_n[r];
#pragma unroll
      for (int c = 0; c < D / 32; ++c) qf[r][c] = qn[r][c];
    }
    const int inext = i + 8 < cnt ? i + 8 : i;
#pragma unroll
    for (int r = 0; r < RT; ++r) entry_q(inext + r, en_n[r], qn[r]);
    float z[RT][16];
    score_tiles<D, RT>(Ks, qf, g4, r16, z);
    bf16x8 pb[RT][2];
    float msl[RT], L[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int t = a.q0 + (int)((en[r] >> 6) % a.nq);
      if (kt * 64 + 63 > t) {  // the diagonal tile (uniform branch)
        __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int key = kt * 64 + 32 * (q >> 3) + 8 * g4 + (q & 7);
          z[r][q] = key <= t ? z[r][q] : kNegInf;
        }
      }
      float tm = z[r][0];
#pragma unroll
      for (int q = 1; q < 16; ++q) tm = fmaxf(tm, z[r][q]);
      tm = col_max4(tm);  // finite: the tile's first key is at or before t
      msl[r] = tm * sl;
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float p = fast_exp2(fmaf(z[r][q], sl, -msl[r]));
        sum += p;
        pb[r][q >> 3][q & 7] = (__bf16)p;
      }
      L[r] = col_sum4(sum);  // >= 1: the maximum key contributes exp2(0)
    }
    f32x4 O[RT][DT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int n = 0; n < DT; ++n) O[r][n] = zero4();
    pv_tiles<D, RT>(Vs, pb, g4, r16, O);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (i + r >= cnt) break;  // uniform: a tile with an odd entry count
      const long row = en[r] >> 6;
      const int fs = en[r] & 63;
      float mx = 0.f;
#pragma unroll
      for (int n = 0; n < DT; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) mx = fmaxf(mx, fabsf(O[r][n][q]));
      const float inv = 1.0f / L[r];
      int ex = 0;
      (void)frexpf(col_max4(mx) * inv, &ex);  // = f 2^ex, f in [0.5, 1); 0 gives ex = 0
      ex = ex < -126 ? -126 : (ex > 127 ? 127 : ex);  // scale and 1 / scale both finite
      const float scale = ldexpf(1.f, ex);
      const float w = inv * ldexpf(1.f, -ex);  // exact power-of-two factor
      const long slot = ((row * a.Hkv + kvh) * a.FS + fs) * 16 + r16;
      // the lane's output quads of column tiles 2 p and 2 p + 1 in one 16-byte piece at
      // 32 p + 8 g4 of the row (the merge reads them back whole)
      _Float16* op = a.s_po + slot * D;
#pragma unroll
      for (int p2 = 0; p2 < DT / 2; ++p2) {
        h16x8 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = (_Float16)(O[r][2 * p2][q] * w);
          v[4 + q] = (_Float16)(O[r][2 * p2 + 1][q] * w);
        }
        *reinterpret_cast<h16x8*>(op + 32 * p2 + 8 * g4) = v;
      }
      if (g4 == 0) *reinterpret_cast<f32x4*>(a.s_ps + slot * 4) = f32x4{msl[r], L[r], scale, 0.f};
    }
  }
}

// ------------------------------------------------------------------ position-major part

// One wave per (position, KV group), kSelWaves consecutive positions of one group per workgroup:
// the group's heads form the 16 MFMA rows.  The forced blocks' tiles (block 0 and the local
// blocks) are common to the positions and staged in LDS once per workgroup (a tile occurring
// twice in a row counts twice); the position's other tiles arrive as the block-major partials,
// merged in slot order into the running (max, sum, output).  out += g1 * o_slc.
// Workgroups are dealt to the 8 XCDs round-robin; the linear index is remapped so that XCD x
// runs a contiguous 1/8 of the (sequence, group, position) range.
template <int D, int G>
__global__ __launch_bounds__(kSelWaves * 64, 1) void selected_kernel(PrefillArgs a) {
  constexpr int DT = D / 16;
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
  const SelShared sh = sel_shared(a, t0);

  int my_key0 = act ? sel_tile_key(a, b, kvh, t, lane) : -1;
  int shcnt[kSelShared];
  uint64_t shared_lanes = 0;
#pragma unroll
  for (int i = 0; i < kSelShared; ++i) {
    const uint64_t m = i < sh.n ? __ballot(my_key0 == sh.key(i)) : 0ull;
    shcnt[i] = (int)__popcll(m);
    shared_lanes |= m;
  }
  // the free tiles (the block-major entries of this row), in slot order
  const int nfree = (int)__popcll(__ballot(my_key0 >= 0) & ~shared_lanes);

  bf16x8 qf[D / 32];
  {
    const u16* qp = a.q + (prow(a, b, act ? t : a.q0) * Hq + head) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qf[c] = hlive ? load8(qp + 32 * c + 8 * g4) : zero8();
  }
  const int tmax = a.T - 1;
  if (threadIdx.x < 256) {  // the first four waves stage the shared tiles
    for (int i = 0; i < sh.n; ++i) {  // uniform
      KTileRegs<D, 256> sk;
      VTileRegs<D, 256> sv;
      sk.load(kb, sh.key(i), tmax);
      sv.load(vtb, a.TP, sh.key(i));
      sk.store(Ksh[i]);
      sv.store(Vsh[i]);
    }
  }
  __syncthreads();
  if (!act) return;  // after the workgroup's only barrier

  // the first block-major partial of the row: (max, sum, scale) of head r16 and the lane's 32
  // outputs, in flight while the shared tiles compute (slot 0 always exists in the layout, and
  // is unused when the row has no partial)
  const long pslot = ((long)(b * a.nq + (t - a.q0)) * a.Hkv + kvh) * a.FS;
  auto load_part = [&](int fs, float4& st, h16x8* ov) {
    const long slot = (pslot + fs) * 16 + r16;
    st = *reinterpret_cast<const float4*>(a.s_ps + slot * 4);
#pragma unroll
    for (int p2 = 0; p2 < DT / 2; ++p2)
      ov[p2] = *reinterpret_cast<const h16x8*>(a.s_po + slot * D + 32 * p2 + 8 * g4);
  };
  float4 st;
  h16x8 ov[DT / 2];
  load_part(0, st, ov);

  float mrun = kNegInf, lrun = 0.f;
  f32x4 O[DT];
#pragma unroll
  for (int n = 0; n < DT; ++n) O[n] = zero4();
  // shared tiles, from LDS: masking, online softmax (lazy rescale), P V
  for (int i = 0; i < sh.n; ++i)
    for (int c = 0; c < shcnt[i]; ++c) {
      float z[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 acc = score_subtile<D>(Ksh[i], qf, q >> 1, q & 1, g4, r16);
#pragma unroll
        for (int e = 0; e < 4; ++e) z[q * 4 + e] = acc[e];
      }
      const int k0 = sh.key(i);
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
      bf16x8 pb[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(fmaf(z[e], sl, -msl));
        sum += p;
        pb[e >> 3][e & 7] = (__bf16)p;
      }
      lrun += sum;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) pv_chunk<D>(Vsh[i], pb[kc], kc, g4, r16, O);
    }

  // the block-major partials of the row merged in slot order; the next slot's loads in flight
  // during this slot's merge
  float msl = mrun == kNegInf ? kNegInf : mrun * sl;
  float L = col_sum4(lrun);
  for (int fs = 0; fs < nfree; ++fs) {
    const float4 cs = st;
    h16x8 cv[DT / 2];
#pragma unroll
    for (int p2 = 0; p2 < DT / 2; ++p2) cv[p2] = ov[p2];
    load_part(fs + 1 < nfree ? fs + 1 : fs, st, ov);  // unconditional: the last re-fetches itself
    const float mn = fmaxf(msl, cs.x);
    const float a1 = msl == kNegInf ? 0.f : fast_exp2(msl - mn);
    const float a2 = fast_exp2(cs.x - mn);
    const float w2 = cs.y * cs.z * a2;
#pragma unroll
    for (int n = 0; n < DT; ++n)
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2)
        O[n][i2] = O[n][i2] * a1 + (float)cv[n >> 1][4 * (n & 1) + i2] * w2;
    L = L * a1 + cs.y * a2;
    msl = mn;
  }

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

// ------------------------------------------------------------------ launcher

template <int D, int G>
static void launch_selected_t(const PrefillArgs& a, hipStream_t s) {
  slc_count_kernel<<<dim3(a.SC, a.Hkv, a.B), kSlcCountThreads, a.NTK * sizeof(int), s>>>(a);
  slc_scan_kernel<<<1, 1024, 0, s>>>(a);
  const long nent = (long)a.B * a.nq * a.Hkv * a.FS;
  slc_fill_kernel<<<dim3((unsigned)((nent + 255) / 256)), 256, 0, s>>>(a);
  slc_block_kernel<D, G><<<dim3((unsigned)a.s_max_tiles), 256, 0, s>>>(a);
  const long nwg = (long)((a.nq + kSelWaves - 1) / kSelWaves) * a.Hkv * a.B;
  selected_kernel<D, G><<<dim3((unsigned)((nwg + 7) / 8 * 8)), kSelWaves * 64, 0, s>>>(a);
}

template <int D>
static void launch_selected_g(const PrefillArgs& a, hipStream_t s) {
  switch (a.G) {
    case 1: launch_selected_t<D, 1>(a, s); break;
    case 2: launch_selected_t<D, 2>(a, s); break;
    case 4: launch_selected_t<D, 4>(a, s); break;
    case 8: launch_selected_t<D, 8>(a, s); break;
    default: launch_selected_t<D, 16>(a, s); break;
  }
}

void launch_selected(const PrefillArgs& a0, hipStream_t s) {
  PrefillArgs a = a0;
  a.SC = slc_chunks(a.nq, a.NTK, a.top_n * (a.beta / 64));  // per (sequence, group) sub-lists
  if (a.D == 128) launch_selected_g<128>(a, s);
  else launch_selected_g<64>(a, s);
}

}  // namespace nsa
