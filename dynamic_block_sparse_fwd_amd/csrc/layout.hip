// Layout kernels: bf16 transpose (values with keys contiguous, compressor weights) and the
// block compression of K/V ("Native Sparse Attention" article, token compression: a learnable
// linear layer maps each l-token block, taken every d tokens, to one representative).
#include "dev_common.h"
#include "kernels.h"

namespace nsa {

// x [BH, rows, cols] -> xt [BH, cols, rows_pad]; one 64x64 tile per workgroup, 16-byte
// global loads and stores (cols and rows_pad multiples of 64, 16-byte aligned bases); rows past
// `rows` are written as zero.
constexpr int kTP = 72;  // LDS row pitch in bf16 (16-byte aligned rows)

// One 64 x 64 tile of x [bh][rows][cols] (row pitch `cols`, ld_rows rows per bh) into
// xt [bh][cols][rows_pad], rows past `rows` as zeros; 256 threads, through LDS.
__device__ __forceinline__ void transpose_tile(const u16* __restrict__ x, u16* __restrict__ xt,
                                               int rows, int cols, int rows_pad, int ld_rows,
                                               long bh, int r0, int c0, u16 (*tile)[kTP]) {
  const int tid = threadIdx.x;
  const int ch = tid & 7;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int r = (tid >> 3) + 32 * pass, row = r0 + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < rows)
      v = *reinterpret_cast<const u32x4*>(x + (bh * ld_rows + row) * cols + c0 + 8 * ch);
    *reinterpret_cast<u32x4*>(&tile[r][8 * ch]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int c = (tid >> 3) + 32 * pass;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[8 * ch + 2 * e][c] | ((uint32_t)tile[8 * ch + 2 * e + 1][c] << 16);
    *reinterpret_cast<u32x4*>(xt + (bh * cols + c0 + c) * rows_pad + r0 + 8 * ch) =
        u32x4{w[0], w[1], w[2], w[3]};
  }
}

__global__ __launch_bounds__(256) void transpose_kernel(const u16* __restrict__ x,
                                                        u16* __restrict__ xt, int rows,
                                                        int cols, int rows_pad, int ld_rows) {
  __shared__ __align__(16) u16 tile[64][kTP];
  transpose_tile(x, xt, rows, cols, rows_pad, ld_rows, blockIdx.z, blockIdx.x * 64,
                 blockIdx.y * 64, tile);
}

// The two compressor weights [l*D, D] transposed in one launch (blockIdx.z: keys, values) for
// an append of C tokens per sequence at the device-side lengths `seqlens`; when no sequence
// completes a compressed token (15 of 16 single-token steps) nothing reads them, and every
// workgroup leaves at once.
__global__ __launch_bounds__(256) void append_weights_kernel(
    const u16* __restrict__ wk, const u16* __restrict__ wv, u16* __restrict__ wkt,
    u16* __restrict__ wvt, int rows, int cols, const int32_t* __restrict__ seqlens, int B, int C,
    int l, int d, int ncap) {
  __shared__ __align__(16) u16 tile[64][kTP];
  int any = 0;
  for (int b = threadIdx.x; b < B; b += 256) {
    const int s0 = seqlens[b], s1 = s0 + C;
    int n0 = s0 >= l ? (s0 - l) / d + 1 : 0, n1 = s1 >= l ? (s1 - l) / d + 1 : 0;
    n0 = n0 < ncap ? n0 : ncap;
    n1 = n1 < ncap ? n1 : ncap;
    any |= n1 > n0;
  }
  if (!__syncthreads_or(any)) return;  // uniform
  const bool v = blockIdx.z == 1;
  transpose_tile(v ? wv : wk, v ? wvt : wkt, rows, cols, rows, rows, 0, blockIdx.x * 64,
                 blockIdx.y * 64, tile);
}

void launch_append_weights(const uint16_t* wk, const uint16_t* wv, uint16_t* wkt, uint16_t* wvt,
                           int rows, int cols, const int32_t* seqlens, int B, int C, int l,
                           int d, int ncap, hipStream_t s) {
  append_weights_kernel<<<dim3(rows / 64, cols / 64, 2), 256, 0, s>>>(wk, wv, wkt, wvt, rows,
                                                                        cols, seqlens, B, C, l,
                                                                        d, ncap);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float4* __restrict__ p, long n4) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

void launch_fill_zero(float* p, size_t n, hipStream_t s) {
  const long n4 = (long)(n / 4);
  if (n4 > 0) {
    const long want = (n4 + 255) / 256;
    fill_zero_kernel<<<(unsigned)(want < 8192 ? want : 8192), 256, 0, s>>>(
        reinterpret_cast<float4*>(p), n4);
  }
}

void launch_transpose(const uint16_t* x, uint16_t* xt, int BH, int rows, int cols, int rows_pad,
                      hipStream_t s, int ld_rows) {
  dim3 grid(rows_pad / 64, cols / 64, BH);
  transpose_kernel<<<grid, 256, 0, s>>>(x, xt, rows, cols, rows_pad, ld_rows < 0 ? rows : ld_rows);
}

// One thread per 16-byte octet of a new K row and of the matching V row.
__global__ __launch_bounds__(256) void append_rows_kernel(const u16* __restrict__ k_new,
                                                          const u16* __restrict__ v_new,
                                                          u16* __restrict__ kcache,
                                                          u16* __restrict__ vcache,
                                                          const int32_t* __restrict__ seqlens,
                                                          int Hkv, int C, int L, int D) {
  const long bh = blockIdx.y;
  const int oct = D / 8;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= C * oct) return;
  const int r = e / oct, c = (e % oct) * 8;
  const int pos = seqlens[bh / Hkv] + r;
  if (pos < 0 || pos >= L) return;
  const long src = (bh * C + r) * D + c, dst = (bh * L + pos) * D + c;
  *reinterpret_cast<u32x4*>(kcache + dst) = *reinterpret_cast<const u32x4*>(k_new + src);
  *reinterpret_cast<u32x4*>(vcache + dst) = *reinterpret_cast<const u32x4*>(v_new + src);
}

void launch_append_rows(const uint16_t* k_new, const uint16_t* v_new, uint16_t* kcache,
                        uint16_t* vcache, const int32_t* seqlens, int BH, int Hkv, int C, int L,
                        int D, hipStream_t s) {
  const int n = C * (D / 8);
  append_rows_kernel<<<dim3((n + 255) / 256, BH), 256, 0, s>>>(k_new, v_new, kcache, vcache,
                                                               seqlens, Hkv, C, L, D);
}

// One workgroup per 64-token tile of one (sequence, head): the tile's key rows are copied
// row-major, its value tile [D][64] lands in columns tile*64 .. tile*64+63 of [D, NCP].
__global__ __launch_bounds__(256) void cmp_cache_layout_kernel(
    const u16* __restrict__ kc, const u16* __restrict__ vtiles, u16* __restrict__ kco,
    u16* __restrict__ vcto, int D, int ncap, int ntcap, int ncmp, int NCP) {
  const int tile = blockIdx.x;
  const long bh = blockIdx.y;
  const int oct = D / 8;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int e = threadIdx.x; e < 64 * oct; e += 256) {
    const int i = tile * 64 + e / oct, c = (e % oct) * 8;
    u32x4 v = z;
    if (i < ncmp) v = *reinterpret_cast<const u32x4*>(kc + (bh * ncap + i) * D + c);
    *reinterpret_cast<u32x4*>(kco + (bh * NCP + i) * D + c) = v;
  }
  for (int e = threadIdx.x; e < D * 8; e += 256) {
    const int c = e / 8, i0 = tile * 64 + (e % 8) * 8;
    u32x4 v = z;
    if (i0 < ncmp) {
      v = *reinterpret_cast<const u32x4*>(vtiles + ((bh * ntcap + tile) * D + c) * 64 +
                                          (e % 8) * 8);
      // tokens past ncmp inside the last tile: zero, whatever the cache holds (NaN included)
      uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
      for (int h = 0; h < 8; ++h)
        if (i0 + h >= ncmp) w[h / 2] &= (h & 1) ? 0x0000FFFFu : 0xFFFF0000u;
      v = u32x4{w[0], w[1], w[2], w[3]};
    }
    *reinterpret_cast<u32x4*>(vcto + (bh * D + c) * (long)NCP + i0) = v;
  }
}

void launch_cmp_cache_layout(const uint16_t* kc, const uint16_t* vtiles, uint16_t* kco,
                             uint16_t* vcto, int BH, int D, int ncap, int ntcap, int ncmp,
                             int NCP, hipStream_t s) {
  if (NCP <= 0) return;
  cmp_cache_layout_kernel<<<dim3(NCP / 64, BH), 256, 0, s>>>(kc, vtiles, kco, vcto, D, ncap,
                                                              ntcap, ncmp, NCP);
}

// Computes the transposed tile  C^T[c][i] = sum_k Wt[c][k] * X_i[k]  where X_i is the l*D
// contiguous elements of x starting at token i*d (the l tokens of compressed token i), so the
// A operand is the weight and the B operand the token window, both staged in LDS.
// Workgroup: 64 compressed tokens x D features; wave w owns features [w*D/4, (w+1)*D/4).
// Half-width of the band around a bf16 rounding midpoint inside which an fp32 accumulation is
// re-done in fp64 (absolute below 1, relative above).  fp32 accumulation errors of these sums
// are around 1e-6 of the operand scale; 2^-16 leaves a wide margin and flags about 1% of outputs.
constexpr float kMidTol = 1.0f / 65536.0f;

// The fp64 dot product of the l*D elements at xp and wp (bf16; every product exact in fp64),
// summed by the whole wave, then its round-to-odd fp32 image (whose bf16 rounding equals the
// correctly rounded fp64 value).  Each lane sums elements 8 lane + 512 j in ascending j; the
// loads of eight j at a time are issued together, so one recomputation waits for one load
// round trip per 4096 elements instead of one per 512.
__device__ __forceinline__ float exact_dot_rto(const u16* xp, const u16* wp, int K, int lane) {
  double s = 0.0;
  for (int kb = 0; kb < K; kb += 4096) {
    bf16x8 xv[8], wv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int k = kb + 512 * j + 8 * lane;
      k = k < K ? k : 0;  // past the end: an in-bounds load whose products are skipped
      xv[j] = load8(xp + k);
      wv[j] = load8(wp + k);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (kb + 512 * j + 8 * lane < K)
#pragma unroll
        for (int q = 0; q < 8; ++q) s += (double)(float)xv[j][q] * (double)(float)wv[j][q];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  float f = __double2float_rz(s);
  if ((double)f != s) f = __uint_as_float(__float_as_uint(f) | 1u);  // round to odd
  return f;
}

template <int D>
__global__ __launch_bounds__(256) void compress_kernel(const u16* __restrict__ x,
                                                       const u16* __restrict__ wt,
                                                       u16* __restrict__ xc, u16* __restrict__ xct,
                                                       int T, int l, int d, int ncmp,
                                                       int rows_alloc, int ncp, int tiled,
                                                       const int32_t* __restrict__ seqlens,
                                                       int C, int Hkv, const u16* __restrict__ x2,
                                                       const u16* __restrict__ wt2,
                                                       u16* __restrict__ xc2,
                                                       u16* __restrict__ xct2) {
  constexpr int CT = D / 64;  // 16-wide feature tiles per wave
  if (blockIdx.z == 1) {  // the second operand set (values, when keys and values share a launch)
    x = x2;
    wt = wt2;
    xc = xc2;
    xct = xct2;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const long bh = blockIdx.y;
  // rows computed: [ilo, ihi); everything else is only zero-filled, and not at all in append
  // mode
  int ilo = 0, ihi = ncmp;
  const bool append = seqlens != nullptr;
  if (append) {
    const int s0 = seqlens[bh / Hkv], s1 = s0 + C;
    ilo = s0 >= l ? (s0 - l) / d + 1 : 0;
    ihi = s1 >= l ? (s1 - l) / d + 1 : 0;
    ihi = ihi < ncmp ? ihi : ncmp;
    if (ilo + (int)blockIdx.x * 64 >= ihi) return;  // uniform; nothing completed here
  }
  const int i0 = ilo + blockIdx.x * 64;
  const int K = l * D;
  const u16* xb = x + bh * (long)T * D;

  f32x4 acc[CT][4];
#pragma unroll
  for (int a = 0; a < CT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = zero4();

  if (ihi > 0) {  // uniform
    // A GEMM over k = l*D in 64-wide steps: the 64 token windows (each l*D contiguous elements
    // of x) and the weight rows are staged in LDS once per step for the four waves
    // (double-buffered, one barrier per step; 16-byte chunks swizzled by row so the 16 rows an
    // operand read touches fall on distinct banks).  The loads of the next NPF steps are in
    // flight in NPF register sets (a step's compute is far shorter than a load's latency, so
    // one set in flight left the loop waiting on every load).
    __shared__ __align__(16) u16 xs[2][64][64];
    __shared__ __align__(16) u16 ws[2][D][64];
    constexpr int XQ = 64 * 8 / 256, WQ = D * 8 / 256;  // 16-byte chunks per thread
    constexpr int NPF = 3;                               // register sets of steps in flight
    const int tid = threadIdx.x;
    const u16* xsrc[XQ];
    const u16* wsrc[WQ];
#pragma unroll
    for (int r = 0; r < XQ; ++r) {
      const int q = tid + 256 * r, tok = q / 8, ch = q % 8;
      int i = i0 + tok;
      i = i < ihi ? i : ihi - 1;  // clamp: rows past ihi are computed and discarded
      xsrc[r] = xb + (long)i * d * D + 8 * ch;
    }
#pragma unroll
    for (int r = 0; r < WQ; ++r) {
      const int q = tid + 256 * r;
      wsrc[r] = wt + (long)(q / 8) * K + 8 * (q % 8);
    }
    const int nks = K / 64;
    u32x4 px[NPF][XQ], pw[NPF][WQ];
    auto fetch = [&](int set, int step) {  // step clamped: past the end it reloads the last
      const int k0 = 64 * (step < nks ? step : nks - 1);
#pragma unroll
      for (int r = 0; r < XQ; ++r) px[set][r] = *reinterpret_cast<const u32x4*>(xsrc[r] + k0);
#pragma unroll
      for (int r = 0; r < WQ; ++r) pw[set][r] = *reinterpret_cast<const u32x4*>(wsrc[r] + k0);
    };
#pragma unroll
    for (int p = 0; p < NPF; ++p) fetch(p, p);
    for (int ks0 = 0; ks0 < nks; ks0 += NPF) {
#pragma unroll
      for (int p = 0; p < NPF; ++p) {
        const int ks = ks0 + p;
        if (ks >= nks) break;  // uniform
        const int buf = ks & 1;
#pragma unroll
        for (int r = 0; r < XQ; ++r) {
          const int q = tid + 256 * r, tok = q / 8, ch = q % 8;
          *reinterpret_cast<u32x4*>(&xs[buf][tok][8 * (ch ^ (tok & 7))]) = px[p][r];
        }
#pragma unroll
        for (int r = 0; r < WQ; ++r) {
          const int q = tid + 256 * r, f = q / 8, ch = q % 8;
          *reinterpret_cast<u32x4*>(&ws[buf][f][8 * (ch ^ (f & 7))]) = pw[p][r];
        }
        __syncthreads();  // step ks staged; step ks - 1's buffer is free again
        fetch(p, ks + NPF);
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const int ch = 8 * ((4 * kc + g4) ^ (r16 & 7));
          bf16x8 bx[4], aw[CT];
#pragma unroll
          for (int it = 0; it < 4; ++it) bx[it] = load8(&xs[buf][it * 16 + r16][ch]);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            aw[ct] = load8(&ws[buf][wave * (D / 4) + ct * 16 + r16][ch]);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int it = 0; it < 4; ++it)
              acc[ct][it] = mfma16x16x32(aw[ct], bx[it], acc[ct][it]);
        }
      }
    }
  }
  // lane holds C^T[c = base + 4*g4 + e][i = i0 + it*16 + r16]
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int c = wave * (D / 4) + ct * 16 + 4 * g4;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int i = i0 + it * 16 + r16;
      const bool live = i < ihi;
      u16 h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = live ? f32_to_bf16(acc[ct][it][e]) : (u16)0;
      if (xc != nullptr && i < rows_alloc && (live || !append)) {
        uint2 pk;
        pk.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        pk.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
        *reinterpret_cast<uint2*>(xc + (bh * rows_alloc + i) * D + c) = pk;
      }
      if (xct != nullptr && i < ncp && (live || !append)) {
        // feature-major [D, ncp], or in 64-token tiles [ncp / 64, D, 64]
        const long o = tiled ? ((bh * (ncp >> 6) + (i >> 6)) * D + c) * 64 + (i & 63)
                             : (bh * D + c) * (long)ncp + i;
        const long es = tiled ? 64 : ncp;
#pragma unroll
        for (int e = 0; e < 4; ++e) xct[o + e * es] = h[e];
      }
    }
  }
  // Exact rounding.  The fp32 sum of l*D products carries a small accumulation error; where
  // it lies within kMidTol of a bf16 rounding midpoint the rounding direction is not settled
  // by fp32, so the whole wave recomputes that element in fp64 (exact products, fp64 sum) and
  // its owner lane stores again the bf16 rounding of the round-to-odd fp32 image, which equals
  // the correctly rounded fp64 value.  Every other element already rounds like the exact sum.
  // The flags of the wave's CT x 16 accumulator slots go to LDS first, so the recomputation
  // loop below is not unrolled over the slots.
  if (ihi > 0) {  // uniform
    __shared__ uint64_t flags[4][CT * 16];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[ct][it][e];
          const float mid = __uint_as_float((__float_as_uint(v) & 0xFFFF0000u) | 0x8000u);
          const float tol = kMidTol * fmaxf(1.f, fabsf(v));
          const uint64_t m = __ballot(fabsf(v - mid) < tol && (i0 + it * 16 + r16) < ihi);
          if (lane == 0) flags[wave][(ct * 4 + it) * 4 + e] = m;
        }
    __asm__ volatile("" ::: "memory");  // the wave's own LDS writes come before its reads
    for (int slot = 0; slot < CT * 16; ++slot) {
      const uint64_t fl = flags[wave][slot];  // the same in every lane: made scalar
      uint64_t pending =
          ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(fl >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)fl);
      const int ct = slot >> 4, it = (slot >> 2) & 3, e = slot & 3;
      while (pending) {
        const int src = __builtin_ctzll(pending);
        pending &= pending - 1;
        const int c = wave * (D / 4) + ct * 16 + 4 * (src >> 4) + e;
        const int i = i0 + it * 16 + (src & 15);
        const float f = exact_dot_rto(xb + (long)i * d * D, wt + (long)c * K, K, lane);
        if (lane == src) {
          const u16 h = f32_to_bf16(f);
          if (xc != nullptr && i < rows_alloc) xc[(bh * rows_alloc + i) * D + c] = h;
          if (xct != nullptr && i < ncp)
            xct[tiled ? ((bh * (ncp >> 6) + (i >> 6)) * D + c) * 64 + (i & 63)
                      : (bh * D + c) * (long)ncp + i] = h;
        }
      }
    }
  }
}

// Append-time compression of the few tokens an append completes (at most `per` per
// sequence-head): a GEMM whose rows are the completed tokens gathered over all sequence-heads,
// so the weight is read once per 64 tokens instead of once per token.  Slot s = bh * per + q
// stands for token n_cmp(seqlens[b]) + q of sequence-head bh (b = bh / Hkv), live while below
// n_cmp(seqlens[b] + C).  The l*D reduction is split in `ks`-long pieces over blockIdx.y, each
// writing fp32 partials part[split][slot][D]; compress_finish_kernel sums them in split order
// and rounds like compress_kernel.  blockIdx.z: 0 keys, 1 values.
constexpr int kFewMaxSplits = 16;  // splits of the l*D reduction: few_splits gives at most 16

struct FewArgs {
  const u16* x[2];   // caches [BH, T, D]
  const u16* wt[2];  // transposed weights [D, l*D]
  u16* xc[2];        // [BH, rows_alloc, D] or null
  u16* xct[2];       // [BH, ncp / 64, D, 64] or null
  float* part;       // [2][nsplit][nslots][D]
  const int32_t* seqlens;
  int T, l, d, ncmp, rows_alloc, ncp, C, Hkv, per, nslots, ks, nsplit;
};

// Token of `slot` given its sequence's length s0 before the append (-1 when dead).
__device__ __forceinline__ int few_token_at(const FewArgs& a, int slot, int s0) {
  const int q = slot % a.per, s1 = s0 + a.C;
  const int ilo = s0 >= a.l ? (s0 - a.l) / a.d + 1 : 0;
  int ihi = s1 >= a.l ? (s1 - a.l) / a.d + 1 : 0;
  ihi = ihi < a.ncmp ? ihi : a.ncmp;
  return ilo + q < ihi ? ilo + q : -1;
}

__device__ __forceinline__ int few_token(const FewArgs& a, int slot, int* bh_out) {
  const int bh = slot / a.per, q = slot % a.per;
  const int s0 = a.seqlens[bh / a.Hkv], s1 = s0 + a.C;
  const int ilo = s0 >= a.l ? (s0 - a.l) / a.d + 1 : 0;
  int ihi = s1 >= a.l ? (s1 - a.l) / a.d + 1 : 0;
  ihi = ihi < a.ncmp ? ihi : a.ncmp;
  *bh_out = bh;
  return ilo + q < ihi ? ilo + q : -1;
}

template <int D>
__global__ __launch_bounds__(256) void compress_split_kernel(FewArgs a) {
  constexpr int CT = D / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int kv = blockIdx.z;
  const int g0 = blockIdx.x * 64, sp = blockIdx.y;
  const int K = a.l * D;
  const int k_lo = sp * a.ks, k_hi = k_lo + a.ks < K ? k_lo + a.ks : K;
  {  // every wave finds the same answer: a workgroup whose 64 slots are all dead leaves
    int bh;
    const int sl = g0 + lane < a.nslots ? g0 + lane : a.nslots - 1;
    const bool live = g0 + lane < a.nslots && few_token(a, sl, &bh) >= 0;
    if (__ballot(live) == 0ull) return;
  }
  long xrow[4];
  int s0v[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {  // the four length loads in flight together (slot clamped)
    const int slot = g0 + it * 16 + r16, sc = slot < a.nslots ? slot : a.nslots - 1;
    s0v[it] = a.seqlens[(sc / a.per) / a.Hkv];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int slot = g0 + it * 16 + r16, sc = slot < a.nslots ? slot : a.nslots - 1;
    int bh = sc / a.per;
    int i = few_token_at(a, sc, s0v[it]);
    if (slot >= a.nslots || i < 0) { bh = 0; i = 0; }  // dead: tokens 0 .. l-1 of head 0, discarded
    xrow[it] = ((long)bh * a.T + (long)i * a.d) * D;
  }
  const u16* xb = a.x[kv];
  const u16* wrow[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) wrow[ct] = a.wt[kv] + (long)(wave * (D / 4) + ct * 16 + r16) * K;
  f32x4 acc[CT][4];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int it = 0; it < 4; ++it) acc[ct][it] = zero4();
  // eight 32-wide k-steps at a time, their loads issued together (a split is a short chain of
  // steps, each with little to compute: one round trip per eight steps instead of per step)
  constexpr int KS = 8;
  for (int kb = k_lo; kb < k_hi; kb += KS * 32) {
    bf16x8 bx[KS][4], aw[KS][CT];
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      // past the split's end: an in-bounds load of its first step, its weight taken as zero
      // (the products are then exact zeros and the sums unchanged; no branch, so the loads of
      // all KS steps stay ahead of the products)
      const bool in = kb + 32 * st < k_hi;
      const int ko = (in ? kb + 32 * st : k_lo) + 8 * g4;
#pragma unroll
      for (int it = 0; it < 4; ++it) bx[st][it] = load8(xb + xrow[it] + ko);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const bf16x8 w = load8(wrow[ct] + ko);
        aw[st][ct] = in ? w : zero8();
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the scheduler keeps every load above the products
#pragma unroll
    for (int st = 0; st < KS; ++st) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int it = 0; it < 4; ++it)
          acc[ct][it] = mfma16x16x32(aw[st][ct], bx[st][it], acc[ct][it]);
    }
  }
  // lane holds C^T[c = base + 4*g4 + e][slot = g0 + it*16 + r16]
  float* pb = a.part + ((long)(kv * a.nsplit + sp) * a.nslots) * D;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int slot = g0 + it * 16 + r16;
    if (slot >= a.nslots) continue;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c = wave * (D / 4) + ct * 16 + 4 * g4;
      *reinterpret_cast<f32x4*>(pb + (long)slot * D + c) = acc[ct][it];
    }
  }
}

// One wave per (slot, 64 features): sum of the split partials in split order, then the exact
// rounding of compress_kernel (fp64 recomputation near a bf16 rounding midpoint).
template <int D>
__global__ __launch_bounds__(256) void compress_finish_kernel(FewArgs a) {
  const int kv = blockIdx.y;
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  const int slot = (int)(e / D), c = (int)(e % D);
  const int lane = threadIdx.x & 63;
  if (slot >= a.nslots) return;  // uniform per wave (D is a multiple of 64)
  int bh = 0;
  const int i = few_token(a, slot, &bh);
  if (i < 0) return;  // uniform per wave
  const float* pb = a.part + ((long)kv * a.nsplit * a.nslots + slot) * D + c;
  // every split's partial loaded at once (at most kFewMaxSplits), then summed in split order
  float pv[kFewMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kFewMaxSplits; ++sp)
    pv[sp] = pb[(long)(sp < a.nsplit ? sp : a.nsplit - 1) * a.nslots * D];
  float v = 0.f;
#pragma unroll
  for (int sp = 0; sp < kFewMaxSplits; ++sp)
    if (sp < a.nsplit) v += pv[sp];
  const int K = a.l * D;
  const u16* xp = a.x[kv] + ((long)bh * a.T + (long)i * a.d) * D;
  const float mid = __uint_as_float((__float_as_uint(v) & 0xFFFF0000u) | 0x8000u);
  uint64_t pending = __ballot(fabsf(v - mid) < kMidTol * fmaxf(1.f, fabsf(v)));
  while (pending) {  // rare: the whole wave recomputes one flagged feature in fp64
    const int src = __builtin_ctzll(pending);
    pending &= pending - 1;
    const u16* wp = a.wt[kv] + (long)(c - lane + src) * K;
    const float f = exact_dot_rto(xp, wp, K, lane);
    if (lane == src) v = f;
  }
  const u16 h = f32_to_bf16(v);
  if (a.xc[kv] != nullptr && i < a.rows_alloc) a.xc[kv][((long)bh * a.rows_alloc + i) * D + c] = h;
  if (a.xct[kv] != nullptr && i < a.ncp)
    a.xct[kv][(((long)bh * (a.ncp >> 6) + (i >> 6)) * D + c) * 64 + (i & 63)] = h;
}

int few_splits(int K, int* ks) {  // at most kFewMaxSplits
  int k = (K + 15) / 16;
  k = (k + 31) / 32 * 32;
  *ks = k;
  return (K + k - 1) / k;
}

size_t few_part_bytes(int BH, int D, int l, int per) {
  int ks;
  const int nsplit = few_splits(l * D, &ks);
  return (size_t)2 * nsplit * BH * per * D * sizeof(float);
}

void launch_compress_few(const uint16_t* const x[2], const uint16_t* const wt[2],
                         uint16_t* const xc[2],
                         uint16_t* const xct[2], float* part, int BH, int T, int D, int l, int d,
                         int ncmp, int rows_alloc, int ncp, const int32_t* seqlens, int C,
                         int Hkv, int per, hipStream_t s) {
  if (per <= 0 || ncmp <= 0) return;
  FewArgs a{};
  for (int j = 0; j < 2; ++j) {
    a.x[j] = x[j]; a.wt[j] = wt[j]; a.xc[j] = xc[j]; a.xct[j] = xct[j];
  }
  a.part = part; a.seqlens = seqlens;
  a.T = T; a.l = l; a.d = d; a.ncmp = ncmp; a.rows_alloc = rows_alloc; a.ncp = ncp;
  a.C = C; a.Hkv = Hkv; a.per = per; a.nslots = BH * per;
  a.nsplit = few_splits(l * D, &a.ks);
  const dim3 g1((a.nslots + 63) / 64, a.nsplit, 2);
  const dim3 g2((unsigned)(((long)a.nslots * D + 255) / 256), 2);
  if (D == 128) {
    compress_split_kernel<128><<<g1, 256, 0, s>>>(a);
    compress_finish_kernel<128><<<g2, 256, 0, s>>>(a);
  } else {
    compress_split_kernel<64><<<g1, 256, 0, s>>>(a);
    compress_finish_kernel<64><<<g2, 256, 0, s>>>(a);
  }
}

void launch_compress(const uint16_t* x, const uint16_t* wt, uint16_t* xc, uint16_t* xct, int BH,
                     int T, int D, int l, int d, int ncmp, int rows_alloc, int ncp, bool tiled,
                     hipStream_t s, const int32_t* seqlens, int C, int Hkv, const uint16_t* x2,
                     const uint16_t* wt2, uint16_t* xc2, uint16_t* xct2) {
  int rows = rows_alloc > ncp ? rows_alloc : ncp;
  // append mode: at most C / d + 1 tokens are completed per sequence
  if (seqlens != nullptr) rows = C / d + 1 < ncmp ? C / d + 1 : ncmp;
  if (rows <= 0) return;
  dim3 grid((rows + 63) / 64, BH, x2 != nullptr ? 2 : 1);
  if (D == 128)
    compress_kernel<128><<<grid, 256, 0, s>>>(x, wt, xc, xct, T, l, d, ncmp, rows_alloc, ncp,
                                              tiled ? 1 : 0, seqlens, C, Hkv, x2, wt2, xc2,
                                              xct2);
  else
    compress_kernel<64><<<grid, 256, 0, s>>>(x, wt, xc, xct, T, l, d, ncmp, rows_alloc, ncp,
                                             tiled ? 1 : 0, seqlens, C, Hkv, x2, wt2, xc2, xct2);
}

}  // namespace nsa
