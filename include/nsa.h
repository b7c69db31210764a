/*
 * nsa.h -- C ABI of the MI355X (gfx950) Native Sparse Attention / MoBA forward library.
 *
 * The method (cited by page title and section):
 *   "Zhang Xiaojun podcast EP94 notes", section 5: an NSA layer runs three branches on every
 *   query -- attention over compressed block representatives of K/V, attention over the
 *   top-N selected 64-token blocks (chosen from the compressed branch's scores), and attention
 *   over a sliding window of recent tokens -- and a learned per-query gate mixes the three
 *   outputs.  Section 6: the heads of one GQA group sum their scores and share one selection.
 *   Sections 9-10: MoBA keeps only the selection branch, with mean-pooled block keys, top-k
 *   blocks per head, and (podcast transcript "Late Talk #103") always the query's own block.
 *   Section 16: NSA block 64 / top-16; MoBA block 512 / top-3.
 *   "Native Sparse Attention" article (lchairun): learnable linear compressor; importance from
 *   the compressed representatives and the query, then top-K; first block always selected;
 *   decode loads only the needed KV, saving HBM bandwidth rather than memory.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers, 16-byte aligned, densely packed (row-major) in the
 *     layouts stated below; bf16 tensors are IEEE bfloat16 bit patterns (uint16 storage).
 *   - Work is enqueued on `stream`; nothing synchronises the host.  The library allocates,
 *     frees and retains nothing: the caller owns every buffer, including the workspace, and
 *     may reuse it once the stream has passed the call.
 *   - All argument checks run on the host before any launch; on error nothing is enqueued and
 *     a negative status is returned.  Nothing is thrown across the ABI.
 *   - Calls that overlap on one workspace race; calls on distinct workspaces are independent.
 *
 * Readings of what the pages leave open (the same ones the CPU oracle takes):
 *   compression is linear with one weight W[l, D, D] shared by all KV heads,
 *     xc[i] = bf16_round( sum_{j<l} x[i*d + j] . W[j] ), i in [0, n_cmp), n_cmp = (T-l)/d + 1;
 *   compressed token i is visible to query t once i*d + l - 1 <= t;
 *   block importance = compressed attention probability spread evenly over the l tokens of
 *     each compressed token and summed per selection block, then summed over the group's heads;
 *   selection takes every visible block if they fit in top_n, else block 0, the n_local most
 *     recent blocks (b - n_local + 1 .. b, b = t / sel_block) and the best remaining blocks by
 *     (score desc, index asc); selected and window branches are causal (keys s <= t), the
 *     window being the `window` most recent tokens including t;
 *   out = gate[...,0] * o_cmp + gate[...,1] * o_slc + gate[...,2] * o_win (gates already
 *     passed through the sigmoid by the caller).
 */
#ifndef NSA_MI355X_H
#define NSA_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define NSA_OK 0
#define NSA_ERR_INVALID_ARG (-1) /* null pointer, misaligned pointer, non-positive size     */
#define NSA_ERR_UNSUPPORTED (-2) /* valid but outside what the kernels implement (see below) */
#define NSA_ERR_WORKSPACE (-3)   /* ws_bytes smaller than the *_workspace_bytes() figure     */
#define NSA_ERR_HIP (-4)         /* a HIP launch or runtime error                            */

/* One NSA layer call.  Hq = Hkv * G query heads; query head h reads KV head h / G. */
typedef struct nsa_config {
  int32_t B;          /* batch (sequences)                                            */
  int32_t T;          /* prefill: sequence length; decode: cache capacity Lmax         */
  int32_t Hkv;        /* KV heads                                                      */
  int32_t G;          /* query heads per KV head (GQA group): 1, 2, 4, 8 or 16         */
  int32_t D;          /* head dimension: 64 or 128                                     */
  int32_t cmp_len;    /* l, tokens per compressed token (32)                           */
  int32_t cmp_stride; /* d, stride between compressed tokens (16)                      */
  int32_t sel_block;  /* selection block size, a multiple of 64 (64)                   */
  int32_t top_n;      /* blocks selected per (query, group), forced ones included (16) */
  int32_t n_local;    /* most recent blocks always selected besides block 0 (2)        */
  int32_t window;     /* sliding-window length (512)                                   */
  float scale;        /* softmax scale applied to q.k (1/sqrt(D))                      */
  float top_p;        /* 0: top_n blocks per (query, group); in (0, 1]: adaptive cut, see
                       * below (top_n is then the cap)                                  */
} nsa_config;

/* One MoBA call (no GQA: H heads with their own K/V). */
typedef struct moba_config {
  int32_t B, T, H, D; /* D: 64 or 128; T a multiple of `block`                          */
  int32_t block;      /* block size, a multiple of 64 (512)                              */
  int32_t top_k;      /* past blocks chosen per (query, head), own block added (3)      */
  float scale;        /* softmax scale (1/sqrt(D))                                       */
} moba_config;

/* Human-readable text for a status code (static storage). */
const char* nsa_status_string(int status);

/*
 * Adaptive top-p block selection ("Native Sparse Attention" article, closing remarks on
 * adaptive sparsity: choose the most important blocks first and stop once their share of the
 * total importance reaches p).  With top_p > 0 the forced blocks (block 0 and the n_local most
 * recent) are kept as before and their importance counts as chosen; the free blocks are then
 * taken in rank order (importance descending, index ascending) while the importance chosen so
 * far is below top_p * G, G being the total importance of a position that sees at least one
 * compressed token (each of the group's heads spreads a probability mass of one), and 0 before
 * that.  top_n caps the whole set; the rule also applies when every block would fit.  Index
 * rows stay ascending with -1 padding.  top_p = 0 is the fixed top_n rule; NaN, negative or
 * > 1 is NSA_ERR_INVALID_ARG.
 */

/* Host-only checks; no device is touched.  NSA_ERR_UNSUPPORTED when: D not 64/128;
 * G not in {1,2,4,8,16}; sel_block not a positive multiple of 64; top_n < 1 + n_local or
 * top_n > 64; T > 2^20 (the prefill counts selected entries per 64-key tile in LDS);
 * top_n * sel_block / 64 > 64 (prefill tiles of a row); cmp_len < cmp_stride; and, when a
 * query tile's block scores outgrow LDS (the selection then streams) in a geometry other than
 * sel_block = 4 cmp_stride, cmp_len = 2 cmp_stride: (64 cmp_stride + 2 cmp_len) / sel_block
 * + 6 > 128. */
int nsa_validate(const nsa_config* cfg);
int moba_validate(const moba_config* cfg);

/* Workspace sizes in bytes for the calls below (0 on an invalid config). */
size_t nsa_compress_workspace_bytes(const nsa_config* cfg);
size_t nsa_prefill_workspace_bytes(const nsa_config* cfg);
size_t nsa_decode_workspace_bytes(const nsa_config* cfg);
size_t moba_prefill_workspace_bytes(const moba_config* cfg);

/* Number of compressed tokens for a length: (T - l) / d + 1, or 0 when T < l. */
int32_t nsa_num_compressed(int32_t T, int32_t cmp_len, int32_t cmp_stride);

/* Number of 64-token tiles of compressed tokens: ceil(nsa_num_compressed / 64). */
int32_t nsa_num_compressed_tiles(int32_t T, int32_t cmp_len, int32_t cmp_stride);

/*
 * Block compression (the compressed branch's learnable linear map; "Native Sparse Attention"
 * article, token compression), also the way to build the decode-time compressed cache.
 *   x  bf16 [B, Hkv, T, D]  keys or values
 *   w  bf16 [l, D, D]       W[j, e, c] maps input feature e of in-block token j to feature c
 *   xc bf16 [B, Hkv, n_cmp, D] output, n_cmp = nsa_num_compressed(T, l, d)
 *   ws at least nsa_compress_workspace_bytes(cfg) bytes (holds the transposed weight)
 * fp32 accumulation, one round-to-nearest-even to bf16.  Uses cfg B, T, Hkv, D, l, d only.
 */
int nsa_compress(const nsa_config* cfg, const void* x, const void* w, void* xc, void* ws,
                 size_t ws_bytes, hipStream_t stream);

/*
 * The same block compression written in 64-token tiles, each tile feature-major: the layout
 * nsa_decode takes for the compressed values (its probability-times-value product reads 64
 * consecutive compressed tokens of one feature at a time, and a tile is one contiguous 16 KB
 * (D = 128) read):
 *   xt bf16 [B, Hkv, nt, D, 64], nt = nsa_num_compressed_tiles(T, l, d);
 *      xt[.., i / 64, c, i % 64] is feature c of compressed token i; tokens n_cmp <= i < 64 * nt
 *      are written as zero
 * Values, rounding, workspace and errors as nsa_compress.
 */
int nsa_compress_tiles(const nsa_config* cfg, const void* x, const void* w, void* xt, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * NSA prefill (three branches + gate; podcast notes EP94 sections 5-6).
 *   q      bf16 [B, T, Hq, D]
 *   k, v   bf16 [B, Hkv, T, D]
 *   wk, wv bf16 [l, D, D]      compressor weights for K and V
 *   gate   fp32 [B, T, Hq, 3]  (cmp, slc, win) gate values
 *   out    fp32 [B, T, Hq, D]
 *   sel_idx int32 [B, T, Hkv, top_n] or NULL: selected blocks per (t, group), ascending,
 *           -1 padded
 *   ws     device workspace of at least nsa_prefill_workspace_bytes(cfg) bytes
 */
int nsa_prefill(const nsa_config* cfg, const void* q, const void* k, const void* v,
                const void* wk, const void* wv, const float* gate, float* out,
                int32_t* sel_idx, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The prefill branches one at a time (the kernels nsa_prefill runs, same code path), for
 * per-branch checks (podcast notes EP94 section 5: compressed, selected and sliding-window
 * branches, mixed by the gate).  `stages` ORs:
 *   NSA_STAGE_CMP_SELECT  compression of K and V, compressed attention, block importance, group
 *                         sum and top-n: out = g0 * o_cmp, selection written to sel_idx (or
 *                         kept in ws when sel_idx is NULL)
 *   NSA_STAGE_WINDOW      out (+)= g2 * o_win
 *   NSA_STAGE_SELECTED    out (+)= g1 * o_slc over the blocks in sel_idx; without
 *                         NSA_STAGE_CMP_SELECT sel_idx is an INPUT (required): per (t, group)
 *                         top_n block indices; entries outside [0, ceil(T/sel_block)) (e.g. the
 *                         -1 padding) are skipped, tiles past t are skipped
 * Without NSA_STAGE_CMP_SELECT out is cleared first.  With NSA_STAGE_CMP_SELECT and
 * NSA_STAGE_WINDOW together the window branch runs inside the compressed kernel on the same
 * query tile (out is written once), as in nsa_prefill, so NSA_STAGE_ALL reproduces nsa_prefill
 * bit for bit; separately computed stages add up to it to within the bf16 rounding of the
 * attention probabilities fed to the matrix core.  There is no
 * separate combine stage: each branch adds its gated output.  wk, wv may be NULL without
 * NSA_STAGE_CMP_SELECT.  Same workspace and errors as nsa_prefill; NSA_ERR_INVALID_ARG for an
 * empty or unknown stage mask.
 */
#define NSA_STAGE_CMP_SELECT 1u
#define NSA_STAGE_WINDOW 2u
#define NSA_STAGE_SELECTED 4u
#define NSA_STAGE_ALL 7u
int nsa_prefill_stages(const nsa_config* cfg, unsigned stages, const void* q, const void* k,
                       const void* v, const void* wk, const void* wv, const float* gate,
                       float* out, int32_t* sel_idx, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * nsa_prefill with two diagnostic outputs of the compressed branch and the selection (podcast
 * notes EP94 sections 5-6), for checking them against a reference:
 *   lse     fp32 [B, T, Hq] or NULL: ln of sum_i exp(scale q . kc_i) over the row's visible
 *           compressed tokens (-inf when none is visible)
 *   scores  fp32 [B, T, Hkv, ceil(T / sel_block)] or NULL: the group block scores the
 *           selection ranks (sum over the group's heads of each block's share of the
 *           compressed probabilities), 0 past the row's current block
 * Every other argument and result as nsa_prefill.  NSA_ERR_UNSUPPORTED when scores is given
 * and the sequence has more blocks than a query tile's scores can keep in LDS (2048, 1024 at
 * G = 1: the selection then streams and no score array exists).
 */
int nsa_prefill_diag(const nsa_config* cfg, const void* q, const void* k, const void* v,
                     const void* wk, const void* wv, const float* gate, float* out,
                     int32_t* sel_idx, float* lse, float* scores, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * Instrumented nsa_prefill: identical work, plus events[s] recorded on `stream` before stage s
 * and events[NSA_PREFILL_NSTAGES] after the last stage.  Stages: 0 layout (value and weight
 * transposes), 1 block compression of K and V, 2 compressed attention + sliding window + block
 * importance + selection, 3 (empty: the window runs inside stage 2), 4 selected blocks.  `events` holds NSA_PREFILL_NSTAGES + 1
 * caller-created events (hipEventCreate); for measurement only.
 */
#define NSA_PREFILL_NSTAGES 5
int nsa_prefill_timed(const nsa_config* cfg, const void* q, const void* k, const void* v,
                      const void* wk, const void* wv, const float* gate, float* out,
                      int32_t* sel_idx, void* ws, size_t ws_bytes, hipStream_t stream,
                      hipEvent_t* events);

/*
 * NSA decode: one new query per sequence; the caches already hold the new token, so query b
 * sits at position t = seqlens[b] - 1 (lchairun article: decode loads only the compressed,
 * selected and window KV).
 *   q              bf16 [B, Hq, D]
 *   kcache, vcache bf16 [B, Hkv, Lmax, D]    (Lmax = cfg->T)
 *   kcmp           bf16 [B, Hkv, n_cmp(Lmax), D]  compressed keys (nsa_compress of kcache)
 *   vcmp           bf16 [B, Hkv, nt(Lmax), D, 64]  compressed values in feature-major 64-token
 *                  tiles (nsa_compress_tiles of vcache; nt = nsa_num_compressed_tiles)
 *                  compressed token i must be valid in both when i*d + l <= seqlens[b]; the
 *                  rest (and the pad tokens of the last tile) may hold anything, NaN included
 *   seqlens        int32 [B], 1 <= seqlens[b] <= Lmax (device memory)
 *   gate           fp32 [B, Hq, 3];  out fp32 [B, Hq, D]
 *   sel_idx        int32 [B, Hkv, top_n] or NULL
 * Deterministic: the same inputs give the same output and indices bit for bit.  Captures into a
 * HIP graph (kernels only, no allocation, no memset).
 * Returns NSA_ERR_UNSUPPORTED when Lmax > 2^24, B or Hkv > 65535, when the per-slice
 * candidates outgrow the LDS that stages them, ceil(ceil(Lmax / sel_block) / S) *
 * max(1, top_n - 1 - n_local) > 16 * D (S = 256 selection blocks per slice for the default
 * geometry; about 10M tokens at D = 128, 5M at D = 64), or when a group's tile list outgrows
 * 256 entries: ceil(window / 64) + 1 + top_n * sel_block / 64 > 256.
 */
int nsa_decode(const nsa_config* cfg, const void* q, const void* kcache, const void* vcache,
               const void* kcmp, const void* vcmp, const int32_t* seqlens, const float* gate,
               float* out, int32_t* sel_idx, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * nsa_decode without a workspace argument, for callers that cannot allocate device memory
 * (code being captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc).  The workspace is a static array of the library, one copy per GPU, of
 * nsa_decode_noalloc_max_bytes() bytes (64 MiB), held until the process ends; nothing is
 * allocated or freed by the call.  Arguments, results and errors as nsa_decode, plus
 * NSA_ERR_WORKSPACE when the configuration needs more workspace than that
 * (nsa_decode_workspace_bytes(cfg) > nsa_decode_noalloc_max_bytes(); e.g. 64k tokens x batch
 * 32 x 4 KV heads needs about 15 MB) and NSA_ERR_HIP when the array's device address cannot be
 * resolved.  Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (concurrent streams or host threads) race.  The array is resolved on the device current at
 * the call, which must be the device of the pointers and the stream.
 */
size_t nsa_decode_noalloc_max_bytes(void);
int nsa_decode_noalloc(const nsa_config* cfg, const void* q, const void* kcache,
                       const void* vcache, const void* kcmp, const void* vcmp,
                       const int32_t* seqlens, const float* gate, float* out, int32_t* sel_idx,
                       hipStream_t stream);

/*
 * Instrumented nsa_decode: identical work, plus events[s] recorded before stage s and
 * events[NSA_DECODE_NSTAGES] after the last.  Stages: 0 compressed-cache stream, 1 block scores,
 * per-slice ranking and the compressed output, 2 top-n and the window's and selected tiles,
 * spread over several workgroups per group, 3 per group: merge of their partials and gate.
 * For measurement only.
 */
#define NSA_DECODE_NSTAGES 4
int nsa_decode_timed(const nsa_config* cfg, const void* q, const void* kcache,
                     const void* vcache, const void* kcmp, const void* vcmp,
                     const int32_t* seqlens, const float* gate, float* out, int32_t* sel_idx,
                     void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* events);

/*
 * Cache maintenance for generation ("Native Sparse Attention" article: the whole KV cache stays
 * in memory while decoding reads only the compressed, selected and window parts of it; its
 * token compression emits one compressed token per d tokens once all l of its tokens exist;
 * podcast notes EP94 section 3: long chains of thought are long decodes).  Appends C tokens to
 * every sequence and emits the compressed tokens those tokens complete.
 *   cfg            B, T = Lmax (cache capacity), Hkv, D, cmp_len l, cmp_stride d are used
 *   C              tokens appended per sequence, 1 <= C <= Lmax
 *   k_new, v_new   bf16 [B, Hkv, C, D]
 *   seqlens        int32 [B] (device memory): tokens each sequence holds BEFORE the append; the
 *                  new tokens go to positions seqlens[b] .. seqlens[b] + C - 1 (positions at or
 *                  past Lmax are not written: the caller keeps seqlens[b] + C <= Lmax).  Not
 *                  updated here.
 *   wk, wv         bf16 [l, D, D] compressor weights (as nsa_compress)
 *   kcache, vcache bf16 [B, Hkv, Lmax, D]           updated in place
 *   kcmp           bf16 [B, Hkv, n_cmp(Lmax), D]     compressed keys, updated in place
 *   vcmp           bf16 [B, Hkv, nt(Lmax), D, 64]    compressed values in tiles, updated in place
 *   ws             at least nsa_cache_append_workspace_bytes(cfg) bytes (transposed weights
 *                  and the fp32 partials of the split compressor, at most 64 MB of them;
 *                  appends completing more compressed tokens per sequence-head than those
 *                  partials hold use the tile compressor)
 * Exactly the compressed tokens i with n_cmp(seqlens[b]) <= i < n_cmp(seqlens[b] + C) are
 * written, each equal bit for bit to nsa_compress / nsa_compress_tiles of the full cache; no
 * other compressed token and no cache row outside the appended positions is touched.  With
 * n_cmp(Lmax) = 0, wk, wv, kcmp, vcmp and ws may be NULL.  Errors as nsa_compress, and
 * NSA_ERR_INVALID_ARG for C outside [1, Lmax].
 */
size_t nsa_cache_append_workspace_bytes(const nsa_config* cfg);
int nsa_cache_append(const nsa_config* cfg, int32_t C, const void* k_new, const void* v_new,
                     const int32_t* seqlens, const void* wk, const void* wv, void* kcache,
                     void* vcache, void* kcmp, void* vcmp, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * Chunked prefill from an existing cache: query positions P .. P + C - 1 of every sequence
 * (the same P and C for all), with keys 0 .. P + C - 1 read from the caches (podcast notes
 * EP94 sections 5-6, as nsa_prefill).  Row t of the outputs equals row t of an nsa_prefill of
 * the first P + C tokens.
 *   cfg            T = Lmax, the capacity of the caches; every other field as nsa_prefill
 *   P              first query position, a multiple of 64 (NSA_ERR_UNSUPPORTED otherwise)
 *   C              chunk length, P + C <= Lmax
 *   q              bf16 [B, C, Hq, D];  gate fp32 [B, C, Hq, 3];  out fp32 [B, C, Hq, D]
 *   kcache, vcache bf16 [B, Hkv, Lmax, D], positions 0 .. P + C - 1 valid (nsa_cache_append)
 *   kcmp, vcmp     compressed caches in the nsa_decode layouts; tokens i < n_cmp(P + C) valid,
 *                  the rest may hold anything
 *   sel_idx        int32 [B, C, Hkv, top_n] or NULL
 *   ws             at least nsa_prefill_chunk_workspace_bytes(cfg) bytes
 * Errors as nsa_prefill (validated at T = Lmax), NSA_ERR_INVALID_ARG for P < 0, C < 1 or
 * P + C > Lmax.
 */
size_t nsa_prefill_chunk_workspace_bytes(const nsa_config* cfg);
int nsa_prefill_chunk(const nsa_config* cfg, int32_t P, int32_t C, const void* q,
                      const void* kcache, const void* vcache, const void* kcmp,
                      const void* vcmp, const float* gate, float* out, int32_t* sel_idx,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward of the NSA prefill layer (podcast notes EP94 section 5: three attention branches and
 * a gate; "Native Sparse Attention" article: the layer is trained end to end, its compressor a
 * learnable linear map).  Gradients of sum(dout * out) for q, k, v, the compressor weights and
 * the gate, with the forward's block selection held fixed (a discrete choice: the
 * block-importance path carries no gradient) and the bf16 rounding of compressed tokens passed
 * through unchanged.
 *   q, k, v, wk, wv, gate  the nsa_prefill inputs (same shapes)
 *   sel_idx  int32 [B, T, Hkv, top_n]  the selection nsa_prefill returned, or any list in that
 *            format whose valid entries are distinct (a repeated block is not supported);
 *            entries outside [0, ceil(T / sel_block)) are skipped
 *   dout     fp32 [B, T, Hq, D]
 *   dq fp32 [B, T, Hq, D]; dk, dv fp32 [B, Hkv, T, D]; dwk, dwv fp32 [l, D, D];
 *   dgate fp32 [B, T, Hq, 3]   outputs, overwritten
 *   ws       at least nsa_backward_workspace_bytes(cfg) bytes
 * Matrix-core operands are bf16 (q, k, v, the compressed tokens as given; dout, the
 * probabilities and the score gradients rounded to bf16), accumulation fp32.  Checks as
 * nsa_prefill (every G it accepts).  Deterministic: no floating-point atomics; key gradients
 * that several position chunks contribute to are summed in a fixed chunk order, so two calls
 * on the same inputs give the same bits.  The workspace holds two fp32 [chunks, B, Hkv, T, D]
 * partial arrays (about 16 chunks) and a bitmap of the selection (one bit per position and
 * block): 4.3 GB at B = 1, T = 65536, Hkv = 4, D = 128.
 */
size_t nsa_backward_workspace_bytes(const nsa_config* cfg);
int nsa_backward(const nsa_config* cfg, const void* q, const void* k, const void* v,
                 const void* wk, const void* wv, const float* gate, const int32_t* sel_idx,
                 const float* dout, float* dq, float* dk, float* dv, float* dwk, float* dwv,
                 float* dgate, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Instrumented nsa_backward: events[s] recorded before stage s, events[NSA_BACKWARD_NSTAGES]
 * after the last.  Stages: 0 layout (key transpose, compression), 1 dout/q layouts, 2
 * query-major passes (dq, per-branch statistics, dgate), 3 key-major passes (dk, dv, compressed
 * partials), 4 compressor backward.  For measurement only.
 */
#define NSA_BACKWARD_NSTAGES 5
int nsa_backward_timed(const nsa_config* cfg, const void* q, const void* k, const void* v,
                       const void* wk, const void* wv, const float* gate,
                       const int32_t* sel_idx, const float* dout, float* dq, float* dk,
                       float* dv, float* dwk, float* dwv, float* dgate, void* ws,
                       size_t ws_bytes, hipStream_t stream, hipEvent_t* events);

/*
 * MoBA prefill (podcast notes EP94 sections 9-10): per head, block keys are the mean of the
 * block's keys, the query scores past blocks by q . kbar, keeps the top_k (ties to the lower
 * index) plus its own block, and attends causally over their union with one softmax.
 *   q bf16 [B, T, H, D]; k, v bf16 [B, H, T, D]; out fp32 [B, T, H, D]
 *   sel_idx int32 [B, T, H, top_k + 1] or NULL: chosen blocks incl. the own block,
 *           ascending, -1 padded
 * The heads run in passes of max(1, min(H, 2^24 / (B T))) heads (one pass up to 2^24 query
 * rows): the workspace holds one pass's per-(query, slot) partials, fp16, about
 * B T Hpass top_k (2 D + 16) bytes, plus the values transposed for one pass.
 * NSA_ERR_UNSUPPORTED (moba_validate) unless D is 64 or 128, block is a multiple of 64 that
 * divides T, top_k <= 8 and T <= 2^27.
 */
int moba_prefill(const moba_config* cfg, const void* q, const void* k, const void* v,
                 float* out, int32_t* sel_idx, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Instrumented moba_prefill: identical work, plus events[s] recorded before stage s and
 * events[NSA_MOBA_NSTAGES] after the last.  Stages: 0 value transpose, pooling and gating,
 * 1 per-block query lists, 2 block-major attention, 3 own block and merge.  With several head
 * passes, stages 1-3 are the last pass's and stage 0 also spans every earlier pass.
 */
#define NSA_MOBA_NSTAGES 4
int moba_prefill_timed(const moba_config* cfg, const void* q, const void* k, const void* v,
                       float* out, int32_t* sel_idx, void* ws, size_t ws_bytes,
                       hipStream_t stream, hipEvent_t* events);

#ifdef __cplusplus
}
#endif

#endif /* NSA_MI355X_H */
