/*
 * nsa_oracle.c -- plain, slow fp64 CPU oracle for the NSA and MoBA forward passes.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this file;
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark use it.  It shares
 * no code, header, table or helper with the GPU library.
 *
 * Sources (the pages are cited by title and section; see the method summary in each function):
 *   [P3] "Zhang Xiaojun podcast EP94 notes" -- section 5 (the three NSA branches), section 6
 *        (group-shared selection), sections 9-10 (MoBA), section 16 (parameter table).
 *   [P4] "Native Sparse Attention" popular article -- compression by a learnable linear layer,
 *        two-step selection (block importance from the compressed representatives, then top-K),
 *        the always-selected first block, the gate that mixes the three branches.
 *   [P1] podcast transcript "Late Talk #103" -- sliding window of the most recent tokens; MoBA
 *        always keeps the block the current token is in.
 *   [P5] news article on NSA/MoBA -- MoBA top-k gating without extra parameters.
 * Choices the pages leave open (all fixed here as plain readings):
 *   R1 compression is linear, no bias, one weight W[l, D, D] shared by all KV heads; a
 *      compressed token is rounded to bf16 once (it is a cache and a matrix operand);
 *   R2 compressed token i covers tokens [i*d, i*d+l) and is visible to query t once its whole
 *      span is in the past (i*d + l - 1 <= t); no visible token -> zero output, zero scores;
 *   R3 a block's importance is the compressed attention probability landing on it: each
 *      compressed probability is spread evenly over the l tokens it covers and summed per
 *      selection block;
 *   R4 group score = sum over the group's heads of the per-head normalised importances;
 *   R5 forced blocks = block 0 plus the n_local most recent blocks (b-n_local+1 .. b), counted
 *      inside top_n; the rest by (score desc, index asc); if every visible block fits, take all;
 *   R6 selected and window branches are causal (keys s <= t); the window holds the w most
 *      recent tokens including t;
 *   R7 gate values are given (already passed through a sigmoid), per (t, head, branch);
 *   R8 MoBA: block key = mean of the block's keys (fp64, no rounding); score = q . kbar;
 *      past blocks j < b ranked by (score desc, index asc); own block always added; one softmax
 *      over the union, causal.
 *   R9 adaptive top-p ([P4], closing remarks on adaptive sparsity: pick the most important
 *      first and stop once the picked share of the total score reaches p): the forced blocks
 *      of R5 are always kept and their importance counts as picked; free blocks are then taken
 *      in the R5 ranking while the importance picked so far is below p * M, M = sum of S_j over
 *      the visible blocks j <= b; top_n stays the cap on the whole set.  Applies whether or
 *      not every visible block would fit.
 * Inputs are bf16 bit patterns, converted exactly to fp64; all arithmetic is fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int B, T, Hkv, G, D;
  int cmp_len, cmp_stride;
  int sel_block, top_n, n_local;
  int window;
  double scale;
  double top_p; /* R9: 0 = fixed top_n; in (0, 1] = adaptive cut by cumulative importance */
} onsa_cfg;

typedef struct {
  int B, T, H, D;
  int block, top_k;
  double scale;
} omoba_cfg;

static double bf(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to the nearest bf16 (ties to even) in one step. */
static uint16_t round_bf16(double x) {
  if (x == 0.0) return signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  int e;
  frexp(a, &e);               /* a = m * 2^e, m in [0.5, 1) */
  int q = e - 8;              /* quantum exponent for 8 significant bits */
  if (q < -133) q = -133;     /* bf16 subnormal spacing 2^-133 */
  double r = rint(ldexp(a, -q)); /* default rounding mode: nearest, ties to even */
  double v = ldexp(r, q);
  float f = (float)v;         /* exact: <= 8 significant bits */
  if (v > 3.3895313892515355e38) f = INFINITY;
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t h = (uint16_t)(u >> 16);
  return x < 0 ? (uint16_t)(h | 0x8000) : h;
}

int onsa_n_cmp(int T, int l, int d) { return T >= l ? (T - l) / d + 1 : 0; }

/* R1: xc[b,h,i,:] = round_bf16( sum_{j<l} sum_{e<D} x[b,h,i*d+j,e] * w[j,e,:] ).
 * x: [B,H,T,D] bf16; w: [l,D,D] bf16; xc_bits: [B,H,n_cmp,D]; xc_exact (nullable): same, fp64. */
void onsa_compress(int B, int H, int T, int D, int l, int d, const uint16_t* x,
                   const uint16_t* w, uint16_t* xc_bits, double* xc_exact) {
  int n = onsa_n_cmp(T, l, d);
  long total = (long)B * H * n;
  /* the weight as fp64, converted once (exact) */
  double* wd = (double*)malloc(sizeof(double) * (size_t)l * D * D);
  for (long a = 0; a < (long)l * D * D; ++a) wd[a] = bf(w[a]);
#pragma omp parallel for schedule(dynamic, 4)
  for (long r = 0; r < total; ++r) {
    long bh = r / n;
    int i = (int)(r % n);
    double* acc = (double*)calloc((size_t)D, sizeof(double));
    for (int j = 0; j < l; ++j) {
      const uint16_t* xr = x + (bh * T + (long)i * d + j) * D;
      for (int e = 0; e < D; ++e) {
        double xv = bf(xr[e]);
        const double* wr = wd + ((long)j * D + e) * D;
        for (int c = 0; c < D; ++c) acc[c] += xv * wr[c];
      }
    }
    for (int c = 0; c < D; ++c) {
      if (xc_bits) xc_bits[r * D + c] = round_bf16(acc[c]);
      if (xc_exact) xc_exact[r * D + c] = acc[c];
    }
    free(acc);
  }
  free(wd);
}

/* softmax attention of one query over an explicit key list; writes o[D], returns lse.
 * keys: token positions into kbase/vbase (row stride D).  n == 0 -> o = 0, lse = -inf. */
static double attend(const double* q, int D, double scale, const uint16_t* kbase,
                     const uint16_t* vbase, const int* keys, int n, double* o, double* zbuf) {
  for (int c = 0; c < D; ++c) o[c] = 0.0;
  if (n == 0) return -INFINITY;
  double m = -INFINITY;
  for (int a = 0; a < n; ++a) {
    const uint16_t* kr = kbase + (long)keys[a] * D;
    double z = 0.0;
    for (int c = 0; c < D; ++c) z += q[c] * bf(kr[c]);
    z *= scale;
    zbuf[a] = z;
    if (z > m) m = z;
  }
  double s = 0.0;
  for (int a = 0; a < n; ++a) s += exp(zbuf[a] - m);
  double lse = m + log(s);
  for (int a = 0; a < n; ++a) {
    double p = exp(zbuf[a] - lse);
    const uint16_t* vr = vbase + (long)keys[a] * D;
    for (int c = 0; c < D; ++c) o[c] += p * bf(vr[c]);
  }
  return lse;
}

typedef struct { double s; int j; } cand;
static int cand_cmp(const void* a, const void* b) {
  const cand* x = (const cand*)a;
  const cand* y = (const cand*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return x->j < y->j ? -1 : (x->j > y->j);
}
static int int_cmp(const void* a, const void* b) {
  int x = *(const int*)a, y = *(const int*)b;
  return (x > y) - (x < y);
}

/*
 * One NSA query position t (all KV groups), shared by the prefill and decode oracles.
 *   qrow  [Hq, D]          bf16  the query vectors of position t
 *   kb/vb [Hkv, tstride, D] bf16 raw keys/values (positions 0..t valid)
 *   kcb/vcb [Hkv, cstride, D] bf16 compressed keys/values (first nvis rows used)
 *   grow  [Hq, 3]          fp32  gate values (cmp, slc, win)
 *   idx_in [Hkv, n] or NULL: replaces the selection step with these blocks (-1 = unused)
 * Outputs per row (any may be NULL except out and idx_out):
 *   out, o_cmp, o_slc, o_win [Hq, D]; lse_cmp [Hq]; scores [Hkv, nblk_cap] (block j <= b);
 *   idx_out [Hkv, n] ascending, -1 padded; gap [Hkv] = (S_(k) - S_(k+1)) / S_(k) of the free
 *   ranking at the number k of free blocks taken (INFINITY when no competitor is left out, 0 on
 *   an exact tie); under top-p also at most min_a |cum_a - p M| / M over the mass decisions.
 */
static void nsa_row(const onsa_cfg* cf, int t, const uint16_t* qrow, const uint16_t* kb,
                    const uint16_t* vb, long tstride, const uint16_t* kcb, const uint16_t* vcb,
                    long cstride, const float* grow, const int32_t* idx_in, int nblk_cap,
                    double* out, double* o_cmp, double* o_slc, double* o_win, double* lse_cmp,
                    double* scores, int32_t* idx_out, double* gap) {
  const int G = cf->G, D = cf->D, l = cf->cmp_len, d = cf->cmp_stride, beta = cf->sel_block;
  const int n = cf->top_n;
  int nvis = t >= l - 1 ? (t - l + 1) / d + 1 : 0; /* R2 */
  const int bcur = t / beta;                        /* block holding t */
  const int nb = bcur + 1;                          /* candidate blocks 0..bcur */
  int maxkeys = nvis > t + 1 ? nvis : t + 1;
  double* z = (double*)malloc(sizeof(double) * (size_t)(maxkeys + 1));
  int* keys = (int*)malloc(sizeof(int) * (size_t)(maxkeys + 1));
  int* wkeys = (int*)malloc(sizeof(int) * (size_t)(t + 1));
  double* S = (double*)calloc((size_t)nb, sizeof(double));
  double* qd = (double*)malloc(sizeof(double) * (size_t)D);
  double* oc = (double*)malloc(sizeof(double) * (size_t)D);
  double* os = (double*)malloc(sizeof(double) * (size_t)D);
  double* ow = (double*)malloc(sizeof(double) * (size_t)D);
  cand* cs = (cand*)malloc(sizeof(cand) * (size_t)nb);
  int* I = (int*)malloc(sizeof(int) * (size_t)(nb + n));
  char* forced = (char*)calloc((size_t)nb, 1);

  for (int g = 0; g < cf->Hkv; ++g) {
    const uint16_t* kg = kb + (long)g * tstride * D;
    const uint16_t* vg = vb + (long)g * tstride * D;
    const uint16_t* kcg = kcb + (long)g * cstride * D;
    const uint16_t* vcg = vcb + (long)g * cstride * D;
    for (int j = 0; j < nb; ++j) S[j] = 0.0;

    /* Branch 1 (compressed attention) and block importance, per head of the group. */
    for (int hh = 0; hh < G; ++hh) {
      int h = g * G + hh;
      for (int c = 0; c < D; ++c) qd[c] = bf(qrow[(long)h * D + c]);
      for (int i = 0; i < nvis; ++i) keys[i] = i;
      double lse = attend(qd, D, cf->scale, kcg, vcg, keys, nvis, oc, z);
      if (lse_cmp) lse_cmp[h] = lse;
      if (o_cmp) memcpy(o_cmp + (long)h * D, oc, sizeof(double) * (size_t)D);
      /* R3: probability p_i spread over tokens [i*d, i*d+l), summed per block. */
      for (int i = 0; i < nvis; ++i) {
        double p = exp(z[i] - lse);
        int s0 = i * d, s1 = i * d + l; /* half-open token span */
        for (int j = s0 / beta; j * beta < s1; ++j) {
          int lo = s0 > j * beta ? s0 : j * beta;
          int hi = s1 < (j + 1) * beta ? s1 : (j + 1) * beta;
          S[j] += p * (double)(hi - lo) / (double)l; /* R4: summed over the group */
        }
      }
      /* branch-1 output parked in out; the gate combination below reads it back */
      memcpy(out + (long)h * D, oc, sizeof(double) * (size_t)D);
    }
    if (scores) {
      for (int j = 0; j < nblk_cap; ++j) scores[(long)g * nblk_cap + j] = j < nb ? S[j] : 0.0;
    }

    /* Selection (R5). */
    int nI = 0;
    double gp = INFINITY;
    if (idx_in) {
      for (int a = 0; a < n; ++a) {
        int j = idx_in[(long)g * n + a];
        if (j >= 0) I[nI++] = j;
      }
    } else if (cf->top_p <= 0 && nb <= n) {
      for (int j = 0; j < nb; ++j) I[nI++] = j;
    } else {
      memset(forced, 0, (size_t)nb);
      forced[0] = 1;
      for (int j = bcur - cf->n_local + 1; j <= bcur; ++j)
        if (j >= 0) forced[j] = 1;
      int nf = 0, nc = 0;
      for (int j = 0; j < nb; ++j) {
        if (forced[j]) { I[nI++] = j; ++nf; }
        else { cs[nc].s = S[j]; cs[nc].j = j; ++nc; }
      }
      int k = n - nf;
      qsort(cs, (size_t)nc, sizeof(cand), cand_cmp);
      if (cf->top_p > 0) { /* R9 */
        double M = 0.0, cum = 0.0, close = INFINITY;
        for (int j = 0; j < nb; ++j) M += S[j];
        for (int j = 0; j < nb; ++j)
          if (forced[j]) cum += S[j];
        const double target = cf->top_p * M;
        int a = 0;
        for (; a < k && a < nc; ++a) {
          double dist = fabs(cum - target);
          if (dist < close) close = dist;
          if (!(cum < target)) break;
          I[nI++] = cs[a].j;
          cum += cs[a].s;
        }
        if (M > 0) gp = close / M;
        k = a; /* the ranking matters at the number actually taken */
      } else {
        for (int a = 0; a < k && a < nc; ++a) I[nI++] = cs[a].j;
      }
      if (k > 0 && k < nc) {
        double sk = cs[k - 1].s, sk1 = cs[k].s;
        double rg = sk == sk1 ? 0.0 : (sk > 0 ? (sk - sk1) / sk : INFINITY);
        if (rg < gp) gp = rg;
      }
    }
    qsort(I, (size_t)nI, sizeof(int), int_cmp);
    for (int a = 0; a < n; ++a) idx_out[(long)g * n + a] = a < nI ? I[a] : -1;
    if (gap) gap[g] = gp;

    /* Branches 2 (selected blocks) and 3 (window), per head; then the gate (R6, R7). */
    int nsel = 0;
    for (int a = 0; a < nI; ++a) {
      int j = I[a];
      for (int s = j * beta; s < (j + 1) * beta && s <= t; ++s) keys[nsel++] = s;
    }
    int w0 = t - cf->window + 1 > 0 ? t - cf->window + 1 : 0;
    for (int s = w0; s <= t; ++s) wkeys[s - w0] = s;
    for (int hh = 0; hh < G; ++hh) {
      int h = g * G + hh;
      for (int c = 0; c < D; ++c) qd[c] = bf(qrow[(long)h * D + c]);
      attend(qd, D, cf->scale, kg, vg, keys, nsel, os, z);
      attend(qd, D, cf->scale, kg, vg, wkeys, t - w0 + 1, ow, z);
      if (o_slc) memcpy(o_slc + (long)h * D, os, sizeof(double) * (size_t)D);
      if (o_win) memcpy(o_win + (long)h * D, ow, sizeof(double) * (size_t)D);
      double g0 = grow[h * 3 + 0], g1 = grow[h * 3 + 1], g2 = grow[h * 3 + 2];
      for (int c = 0; c < D; ++c) {
        double ocv = out[(long)h * D + c];
        out[(long)h * D + c] = g0 * ocv + g1 * os[c] + g2 * ow[c];
      }
    }
  }
  free(z); free(keys); free(S); free(qd); free(oc); free(os); free(ow); free(cs); free(I);
  free(forced); free(wkeys);
}

/*
 * NSA prefill, selected rows.  Row r is query position (row_b[r], row_t[r]) for every head.
 *   q [B,T,Hq,D], k/v [B,Hkv,T,D], kc/vc [B,Hkv,n_cmp,D] (from onsa_compress), gate [B,T,Hq,3].
 *   idx_in: NULL or [nrows, Hkv, top_n].
 * Outputs: out/o_cmp/o_slc/o_win [nrows,Hq,D], lse [nrows,Hq], scores [nrows,Hkv,ceil(T/beta)],
 *   idx_out [nrows,Hkv,top_n], gap [nrows,Hkv]; all but out and idx_out nullable.
 */
int onsa_prefill_rows(const onsa_cfg* cf, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const uint16_t* kc, const uint16_t* vc,
                      const float* gate, int nrows, const int32_t* row_b, const int32_t* row_t,
                      const int32_t* idx_in, double* out, double* o_cmp, double* o_slc,
                      double* o_win, double* lse, double* scores, int32_t* idx_out,
                      double* gap) {
  const int Hq = cf->Hkv * cf->G, D = cf->D, n = cf->top_n;
  const int ncmp = onsa_n_cmp(cf->T, cf->cmp_len, cf->cmp_stride);
  const int nblk = (cf->T + cf->sel_block - 1) / cf->sel_block;
  for (int r = 0; r < nrows; ++r)
    if (row_b[r] < 0 || row_b[r] >= cf->B || row_t[r] < 0 || row_t[r] >= cf->T) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nrows; ++r) {
    int b = row_b[r], t = row_t[r];
    long qo = ((long)b * cf->T + t) * Hq * D;
    long ko = (long)b * cf->Hkv * cf->T * D;
    long co = (long)b * cf->Hkv * ncmp * D;
    nsa_row(cf, t, q + qo, k + ko, v + ko, cf->T, kc + co, vc + co, ncmp,
            gate + ((long)b * cf->T + t) * Hq * 3, idx_in ? idx_in + (long)r * cf->Hkv * n : NULL,
            nblk, out + (long)r * Hq * D, o_cmp ? o_cmp + (long)r * Hq * D : NULL,
            o_slc ? o_slc + (long)r * Hq * D : NULL, o_win ? o_win + (long)r * Hq * D : NULL,
            lse ? lse + (long)r * Hq : NULL, scores ? scores + (long)r * cf->Hkv * nblk : NULL,
            idx_out + (long)r * cf->Hkv * n, gap ? gap + (long)r * cf->Hkv : NULL);
  }
  return 0;
}

/*
 * NSA decode: one new query per sequence at position t = seqlens[b] - 1 (the cache already
 * holds the new token).  cf->T is the cache capacity Lmax.
 *   q [B,Hq,D]; kcache/vcache [B,Hkv,Lmax,D]; kc/vc [B,Hkv,n_cmp(Lmax),D]; gate [B,Hq,3].
 * Outputs as in onsa_prefill_rows with one row per sequence.
 */
int onsa_decode(const onsa_cfg* cf, const uint16_t* q, const uint16_t* kcache,
                const uint16_t* vcache, const uint16_t* kc, const uint16_t* vc,
                const int32_t* seqlens, const float* gate, const int32_t* idx_in, double* out,
                double* o_cmp, double* o_slc, double* o_win, double* lse, double* scores,
                int32_t* idx_out, double* gap) {
  const int Hq = cf->Hkv * cf->G, D = cf->D, n = cf->top_n;
  const int ncmp = onsa_n_cmp(cf->T, cf->cmp_len, cf->cmp_stride);
  const int nblk = (cf->T + cf->sel_block - 1) / cf->sel_block;
  for (int b = 0; b < cf->B; ++b)
    if (seqlens[b] < 1 || seqlens[b] > cf->T) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int b = 0; b < cf->B; ++b) {
    int t = seqlens[b] - 1;
    long ko = (long)b * cf->Hkv * cf->T * D;
    long co = (long)b * cf->Hkv * ncmp * D;
    nsa_row(cf, t, q + (long)b * Hq * D, kcache + ko, vcache + ko, cf->T, kc + co, vc + co, ncmp,
            gate + (long)b * Hq * 3, idx_in ? idx_in + (long)b * cf->Hkv * n : NULL, nblk,
            out + (long)b * Hq * D, o_cmp ? o_cmp + (long)b * Hq * D : NULL,
            o_slc ? o_slc + (long)b * Hq * D : NULL, o_win ? o_win + (long)b * Hq * D : NULL,
            lse ? lse + (long)b * Hq : NULL, scores ? scores + (long)b * cf->Hkv * nblk : NULL,
            idx_out + (long)b * cf->Hkv * n, gap ? gap + (long)b * cf->Hkv : NULL);
  }
  return 0;
}

/* MoBA block keys (R8): kbar[b,h,j,:] = mean of keys j*block .. j*block+block-1 (full blocks). */
void omoba_pool(const omoba_cfg* cf, const uint16_t* k, double* kbar) {
  const int nb = cf->T / cf->block, D = cf->D;
  long total = (long)cf->B * cf->H * nb;
#pragma omp parallel for schedule(static)
  for (long r = 0; r < total; ++r) {
    long bh = r / nb;
    int j = (int)(r % nb);
    double* o = kbar + r * D;
    for (int c = 0; c < D; ++c) o[c] = 0.0;
    for (int s = j * cf->block; s < (j + 1) * cf->block; ++s) {
      const uint16_t* kr = k + (bh * cf->T + s) * D;
      for (int c = 0; c < D; ++c) o[c] += bf(kr[c]);
    }
    for (int c = 0; c < D; ++c) o[c] /= (double)cf->block;
  }
}

/*
 * MoBA prefill, selected rows (R8).  q [B,T,H,D]; k/v [B,H,T,D]; kbar from omoba_pool.
 *   idx_in: NULL or [nrows, H, top_k+1] (replaces the gating, -1 = unused).
 * Outputs: out [nrows,H,D]; idx_out [nrows,H,top_k+1] ascending incl. the own block, -1 padded;
 *   scores (nullable) [nrows,H,T/block] = q . kbar_j for j < b, 0 elsewhere;
 *   gap (nullable) [nrows,H] = (S_(k) - S_(k+1)) / (|q| * max_j |kbar_j|) over past blocks.
 */
int omoba_prefill_rows(const omoba_cfg* cf, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const double* kbar, int nrows, const int32_t* row_b,
                       const int32_t* row_t, const int32_t* idx_in, double* out,
                       int32_t* idx_out, double* scores, double* gap) {
  const int H = cf->H, D = cf->D, nbt = cf->T / cf->block, kk = cf->top_k + 1;
  for (int r = 0; r < nrows; ++r)
    if (row_b[r] < 0 || row_b[r] >= cf->B || row_t[r] < 0 || row_t[r] >= cf->T) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nrows; ++r) {
    int b = row_b[r], t = row_t[r];
    int bcur = t / cf->block;
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    double* z = (double*)malloc(sizeof(double) * (size_t)(t + 1));
    int* keys = (int*)malloc(sizeof(int) * (size_t)(t + 1));
    cand* cs = (cand*)malloc(sizeof(cand) * (size_t)(bcur + 1));
    int* I = (int*)malloc(sizeof(int) * (size_t)(bcur + 1 + kk));
    for (int h = 0; h < H; ++h) {
      const uint16_t* qr = q + (((long)b * cf->T + t) * H + h) * D;
      const uint16_t* kh = k + ((long)b * H + h) * cf->T * D;
      const uint16_t* vh = v + ((long)b * H + h) * cf->T * D;
      const double* kbh = kbar + ((long)b * H + h) * nbt * D;
      double qn = 0.0, kmax = 0.0;
      for (int c = 0; c < D; ++c) { qd[c] = bf(qr[c]); qn += qd[c] * qd[c]; }
      qn = sqrt(qn);
      for (int j = 0; j < bcur; ++j) {
        double s = 0.0, kn = 0.0;
        for (int c = 0; c < D; ++c) { s += qd[c] * kbh[(long)j * D + c]; kn += kbh[(long)j * D + c] * kbh[(long)j * D + c]; }
        cs[j].s = s;
        cs[j].j = j;
        if (sqrt(kn) > kmax) kmax = sqrt(kn);
      }
      if (scores) {
        double* sr = scores + ((long)r * H + h) * nbt;
        for (int j = 0; j < nbt; ++j) sr[j] = j < bcur ? cs[j].s : 0.0;
      }
      int nI = 0;
      double gp = INFINITY;
      if (idx_in) {
        for (int a = 0; a < kk; ++a) {
          int j = idx_in[((long)r * H + h) * kk + a];
          if (j >= 0) I[nI++] = j;
        }
      } else {
        if (bcur <= cf->top_k) {
          for (int j = 0; j < bcur; ++j) I[nI++] = j;
        } else {
          qsort(cs, (size_t)bcur, sizeof(cand), cand_cmp);
          for (int a = 0; a < cf->top_k; ++a) I[nI++] = cs[a].j;
          if (cf->top_k > 0) { /* top_k = 0: nothing ranked, no gap */
            double den = qn * kmax;
            double sk = cs[cf->top_k - 1].s, sk1 = cs[cf->top_k].s;
            gp = sk == sk1 ? 0.0 : (den > 0 ? (sk - sk1) / den : INFINITY);
          }
        }
        I[nI++] = bcur;
      }
      qsort(I, (size_t)nI, sizeof(int), int_cmp);
      for (int a = 0; a < kk; ++a) idx_out[((long)r * H + h) * kk + a] = a < nI ? I[a] : -1;
      if (gap) gap[(long)r * H + h] = gp;
      int nk = 0;
      for (int a = 0; a < nI; ++a)
        for (int s = I[a] * cf->block; s < (I[a] + 1) * cf->block && s <= t; ++s) keys[nk++] = s;
      attend(qd, D, cf->scale, kh, vh, keys, nk, out + ((long)r * H + h) * D, z);
    }
    free(qd); free(z); free(keys); free(cs); free(I);
  }
  return 0;
}

/* Threads the parallel loops above use (for reporting the CPU baseline). */
int onsa_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
