// Internal launcher interface between the C-ABI layer (api.hip) and the kernel files.
// Every launcher only enqueues work on `stream`; shapes were validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

struct PrefillArgs {
  const uint16_t* q;    // [B, nq, Hq, D]
  const uint16_t* k;    // [B, Hkv, ldk, D]
  const uint16_t* vt;   // [B, Hkv, D, TP]  values, keys contiguous, zero past T
  const uint16_t* kc;   // [B, Hkv, NCP, D] compressed keys, zero rows past n_cmp
  const uint16_t* vct;  // [B, Hkv, D, NCP] compressed values (transposed), zero past n_cmp
  const float* gate;    // [B, nq, Hq, 3]
  float* out;           // [B, nq, Hq, D]
  int32_t* idx;         // [B, nq, Hkv, top_n]
  int B, T, Hkv, G, D;  // T: end of the query rows (keys 0 .. T-1 exist)
  int q0, nq;           // query rows processed: q0 .. q0+nq-1 (<= T-1)
  int ldq, qs;          // q/gate/out/idx hold row t of sequence b at b * ldq + t - qs
  int ldk;              // rows per (sequence, KV head) slab of k (T, or a cache's capacity)
  int l, d, beta, top_n, n_local, window;
  int ncmp, NCP, TP, nblk;
  float scale_log2;     // softmax scale * log2(e)
  float top_p;          // 0: fixed top_n; else the adaptive cut at top_p * G
  int fuse_window;      // cmp_select also runs the window branch and writes out once
  float* dlse;          // nullable [B, nq, Hq]: ln of the compressed branch's softmax sum
  float* dscores;       // nullable [B, nq, Hkv, nblk]: group block scores (block scores kept in
                        // LDS only)
  // Squared norms of the compressed keys as running maxima (workspace), from which the
  // compressed attention bounds a row's scores: kpmax[j] = max |k_i|^2 over the rows i <= j of
  // j's kNormRows-row chunk, kcmax[c] = the maximum over chunk c.
  float* kpmax;         // [B*Hkv, NCP]
  float* kcmax;         // [B*Hkv, NKB]
  int NKB;              // chunks of the visible compressed keys: ceil(ncmp / kNormRows)
  // Selected branch, block-major part (workspace).  An "entry" is one selected 64-key tile of one
  // (row, group) that is not among the tiles the selected kernel shares per eight positions;
  // row = b * nq + (t - q0), free slot fs = its rank among the row's such tiles (< FS).
  int32_t* s_rank;       // [B*nq, Hkv, FS] rank of the entry in its sub-list
  int32_t* s_kt;         // [B*nq, Hkv, FS] key tile of the entry, -1 past the row's entries
  int32_t* s_count;      // [SC, B*Hkv, NTK] entries per (T-chunk, sequence-group, key tile)
  int32_t* s_offset;     // [SC * B*Hkv * NTK + 1] sub-list offsets (after the scan)
  int32_t* s_tstart;     // [SC * B*Hkv * NTK] first work tile of each sub-list
  int32_t* s_ntiles;     // [1] work tiles in all
  int32_t* s_tile_entry; // [s_max_tiles] sub-list of each work tile
  int32_t* s_list;       // [B*nq*Hkv*FS] entries by sub-list: row << 6 | fs
  _Float16* s_po;        // [B*nq, Hkv, FS, 16, D] partial outputs / (sum * scale), fp16;
                         // the 8 values at 32 p + 8 g of a row are columns 32 p + 4 g ..
                         // + 3 and 32 p + 16 + 4 g .. + 3 (g < 4)
  float* s_ps;           // [B*nq, Hkv, FS, 16, 4] partial (max in log2 units, sum, scale, 0)
  int FS, NTK, s_max_tiles;
  int SC;  // T-chunks of the lists: slc_chunks(nq, NTK, top_n beta / 64), set at launch
};

constexpr int kNormRows = 256;  // compressed-key rows per chunk of the norm maxima
constexpr int kSlcChunks = 16;  // most T-chunks of the block-major lists (work tiles chunk-major)
constexpr int kSlcRows = 64;    // positions per block-major work tile
// T-chunks of the lists for nq query rows, ntk key tiles and `per` selected tiles per row: as
// many as keep a sub-list about one work tile long (nq per / (ntk kSlcRows) entries in all per
// key tile), a multiple of 4 in [4, kSlcChunks]
__host__ __device__ constexpr int slc_chunks(long nq, int ntk, int per) {
  const long c = nq * per / ((long)kSlcRows * (ntk > 0 ? ntk : 1));
  const long c4 = c / 4 * 4;
  return c4 < 4 ? 4 : (c4 > kSlcChunks ? kSlcChunks : (int)c4);
}

// Row of q/gate/out/idx holding query position t of sequence b.
__device__ __forceinline__ long prow(const PrefillArgs& a, int b, int t) {
  return (long)b * a.ldq + (t - a.qs);
}

struct DecodeArgs {
  const uint16_t* q;       // [B, Hq, D]
  const uint16_t* kcache;  // [B, Hkv, L, D]
  const uint16_t* vcache;  // [B, Hkv, L, D]
  const uint16_t* kc;      // [B, Hkv, ncmp, D]
  const uint16_t* vct;     // [B, Hkv, NT, D, 64] feature-major 64-token tiles
  const int32_t* seqlens;  // [B]
  const float* gate;       // [B, Hq, 3]
  float* out;              // [B, Hq, D]
  int32_t* idx;            // [B, Hkv, top_n]
  // workspace; 16 row slots (heads of a group) everywhere; every array holds at least one
  // chunk / tile per group, so clamped indices stay inside it when nothing is visible
  float* cm;    // [B*Hkv, NCH, 16] chunk max (scaled log2 units)
  float* cl;    // [B*Hkv, NCH, 16] sum of exp2(z - max)
  float* co;    // [B*Hkv, NCH, 16, D] unnormalised output
  float* tref;  // [B*Hkv, NT, 16] per 64-token tile: reference of its block masses (log2)
  float* cb;    // [B*Hkv, NT, NBT, 16] block masses of each tile, relative to exp2(tref)
  float* sS;        // [B*Hkv, NSL * SB] group block scores, written by the selection slices
  uint64_t* cand;   // [B*Hkv, NSL, KF] each slice's best free blocks (rank keys, 0 = none)
  float* ocmp;      // [B*Hkv, 16, D] compressed-branch output, normalised by the selection slices
  float* grec;      // [B*Hkv, NG, 2, 32 + 16 D] per tile workgroup and branch: 16 maxima (scaled
                    // log2), 16 sums, 16 x D outputs relative to the maxima
  int B, L, Hkv, G, D;
  int l, d, beta, top_n, n_local, window;
  int ncmp, nblk, NCH, NT, NBT;
  int SB, NSL;  // blocks per selection slice, slices per group
  int KF;       // free blocks per group: top_n - 1 - n_local (at least 1)
  int NG;       // tile workgroups per group
  int NGW;      // of them, the ones that take the window's and forced tiles
  float scale_log2;
  float top_p;  // 0: fixed top_n; else the adaptive cut at top_p * G
};

// ev: nullptr or NSA_DECODE_NSTAGES + 1 events recorded around the stages.
void launch_decode(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev);
int decode_chunk_tokens();
constexpr int kDecodeMaxList = 256;  // tiles of a group's tile list
// blocks per selection slice: at most 256, and few enough that the compressed-token tiles the
// slice's blocks touch fit the slice's 64-tile weight table
int decode_slice_blocks(int l, int d, int beta);
// candidates (slices x free blocks) a tile workgroup stages in LDS
__host__ __device__ constexpr int decode_max_candidates(int D) { return 4 * D * 64 * 2 / 8; }

// Backward of the prefill layer.
struct BwdArgs {
  const uint16_t* q;      // [B, T, Hq, D]
  const uint16_t* k;      // [B, Hkv, T, D]
  const uint16_t* v;      // [B, Hkv, T, D]
  const uint16_t* wk;     // [l, D, D]
  const uint16_t* wv;     // [l, D, D]
  const float* gate;      // [B, T, Hq, 3]
  const int32_t* idx;     // [B, T, Hkv, top_n] the forward's selection
  const float* dout;      // [B, T, Hq, D]
  // workspace
  const uint16_t* kt;     // [B*Hkv, D, TP] keys, transposed, zero past T
  const uint16_t* kc;     // [B*Hkv, NCP, D] compressed keys, zero past n_cmp
  const uint16_t* kct;    // [B*Hkv, D, NCP] compressed keys, transposed
  const uint16_t* vc;     // [B*Hkv, NCP, D] compressed values
  uint16_t* dob;          // [B, T, Hq, D] dout in bf16
  uint16_t* dot;          // [B, T, Hkv, D, 16] dout, the G heads contiguous per feature, then
                          // 16 - G zeros
  uint16_t* qt;           // [B, T, Hkv, D, 16] q, the same
  float* lse;             // [3, B, T, Hq] per branch: log2-sum-exp2 of the scaled scores
  float* dlt;             // [3, B, T, Hq] per branch: <dout, o_branch>
  float* pk;              // [NPC, B*Hkv, NCP, D] compressed-key gradient, per position chunk
  float* pv;              // [NPC, B*Hkv, NCP, D] compressed-value gradient, the same
  float* dkc;             // [B*Hkv, NCP, D]
  float* dvc;             // [B*Hkv, NCP, D]
  float* psk;             // [NPC, B*Hkv, T, D] selected-branch key gradient, per position chunk
  float* psv;             // [NPC, B*Hkv, T, D] selected-branch value gradient, the same
  uint32_t* selbits;      // [B*Hkv, nblk, SW] bit t of row (group, block): position t selected it
  // outputs
  float* dq;              // [B, T, Hq, D]
  float* dk;              // [B, Hkv, T, D]
  float* dv;              // [B, Hkv, T, D]
  float* dwk;             // [l, D, D]
  float* dwv;             // [l, D, D]
  float* dgate;           // [B, T, Hq, 3]
  int B, T, Hkv, G, D, l, d, beta, top_n, window;
  int ncmp, NCP, TP, nblk, PC, NPC;  // PC positions per chunk of the key-major passes
  int SW;                            // 32-bit words per bitmap row: ceil(T / 32)
  float scale, scale_log2;
};

// ev: nullptr or NSA_BACKWARD_NSTAGES + 1 events; ev[0] and ev[1] are recorded by the caller.
void launch_backward(const BwdArgs& a, hipStream_t s, hipEvent_t* ev);

constexpr int kMobaChunks = 8;  // T-chunks per head counted by separate workgroups
constexpr int kMobaCountBlocks = 16384;  // blocks per counting workgroup (64 KB of LDS)

// One pass over H of the caller's Hs heads; the workspace arrays (from vt on) hold this pass's
// heads only.
struct MobaArgs {
  const uint16_t* q;   // [B, T, Hs, D]
  const uint16_t* k;   // [B, Hs, T, D]
  const uint16_t* vt;  // [B*H, D, T] values, keys contiguous
  float* out;          // [B, T, Hs, D]
  int32_t* idx;        // [B, T, Hs, top_k + 1]
  uint16_t* kb_hi;     // [B*H, nb, D] block key mean, bf16 high part
  uint16_t* kb_lo;     // [B*H, nb, D] bf16 of the remainder
  int32_t* count;      // [B*H*nb, kMobaChunks] queries of each T-chunk that chose each block,
                       // turned into chunk offsets inside the block's list by the scan
  int32_t* rank;       // [B*H*T, top_k] position of each (query, slot) in its block's list
  int32_t* offset;     // [B*H*nb + 1] list offsets (exclusive prefix of the list lengths)
  int32_t* tstart;     // [B*H*nb] first 128-row tile of each list
  int32_t* ntiles;     // [1] total tiles
  int32_t* tile_entry; // [max_tiles] the list each 128-row tile belongs to
  int32_t* list;       // [B*T*H*top_k] (t << 4 | slot)
  _Float16* po;        // [B*T*H, top_k, D] partial outputs / (own sum * scale), fp16;
                       // values 32 p + 8 g .. + 7: columns 32 p + 4 g .. + 3, 32 p + 16 + 4 g .. + 3
  float* pml;          // [B*T*H, top_k, 4] partial (max in log2 units, sum, scale, 0)
  int B, T, H, D, block, top_k, nb, max_tiles;
  int Hs, h0;  // heads of the caller's q, k, out, idx; first head of this pass (H heads)
  float scale_log2;
};

// ev: nullptr or NSA_MOBA_NSTAGES + 1 events; ev[0] is recorded by the caller.
void launch_moba(const MobaArgs& a, hipStream_t s, hipEvent_t* ev);

// p[0 .. n) = 0 (n a multiple of 4, p 16-byte aligned); a kernel, so it may be captured.
void launch_fill_zero(float* p, size_t n, hipStream_t s);

// x [BH, ld_rows, cols] (first `rows` rows used) -> xt [BH, cols, rows_pad] (bf16),
// zero-filled for rows..rows_pad-1; cols and rows_pad multiples of 64, x and xt 16-byte
// aligned.  ld_rows < 0 means rows.
void launch_transpose(const uint16_t* x, uint16_t* xt, int BH, int rows, int cols, int rows_pad,
                      hipStream_t s, int ld_rows = -1);

// The compressor weights wk, wv [rows = l*D, cols = D] -> wkt, wvt [cols, rows] in one launch,
// skipped (every workgroup returns) when an append of C tokens at seqlens [B] completes no
// compressed token below the capacity ncap.
void launch_append_weights(const uint16_t* wk, const uint16_t* wv, uint16_t* wkt, uint16_t* wvt,
                           int rows, int cols, const int32_t* seqlens, int B, int C, int l,
                           int d, int ncap, hipStream_t s);

// Compressed tokens of x [BH, T, D] with the transposed weight wt [D, l*D]:
//   xc  (nullable) [BH, rows_alloc, D] row-major, rows n_cmp..rows_alloc-1 zero;
//   xct (nullable) [BH, D, ncp] transposed, or with `tiled` [BH, ncp / 64, D, 64] (64-token
//       tiles, each feature-major); columns n_cmp..ncp-1 zero.
// Append mode (seqlens non-null, Hkv heads per sequence): only the compressed tokens completed
// by appending C tokens to sequence b, i.e. n_cmp(seqlens[b]) <= i < n_cmp(seqlens[b] + C)
// (and i < ncmp), are computed and written; no other row is touched.
// With x2 non-null a second operand set (x2, wt2, xc2, xct2; same shapes) is compressed in the
// same launch (keys and values together: twice the workgroups in flight).
void launch_compress(const uint16_t* x, const uint16_t* wt, uint16_t* xc, uint16_t* xct, int BH,
                     int T, int D, int l, int d, int ncmp, int rows_alloc, int ncp, bool tiled,
                     hipStream_t s, const int32_t* seqlens = nullptr, int C = 0, int Hkv = 1,
                     const uint16_t* x2 = nullptr, const uint16_t* wt2 = nullptr,
                     uint16_t* xc2 = nullptr, uint16_t* xct2 = nullptr);

// Append mode for few tokens, keys and values in one go (index 0 keys, 1 values): the same
// tokens as launch_compress's append mode, at most `per` per sequence-head, gathered over all
// sequence-heads into one split-K GEMM; wt the transposed weights [D, l*D]; part a workspace
// of few_part_bytes(BH, D, l, per) bytes.
size_t few_part_bytes(int BH, int D, int l, int per);
void launch_compress_few(const uint16_t* const x[2], const uint16_t* const wt[2],
                         uint16_t* const xc[2],
                         uint16_t* const xct[2], float* part, int BH, int T, int D, int l, int d,
                         int ncmp, int rows_alloc, int ncp, const int32_t* seqlens, int C,
                         int Hkv, int per, hipStream_t s);

// Cache append: rows seqlens[b] .. seqlens[b]+C-1 of kc/vc [BH, L, D] <- k_new/v_new
// [BH, C, D] (rows at or past L are dropped).
void launch_append_rows(const uint16_t* k_new, const uint16_t* v_new, uint16_t* kcache,
                        uint16_t* vcache, const int32_t* seqlens, int BH, int Hkv, int C, int L,
                        int D, hipStream_t s);

// Compressed caches to the prefill layouts: keys [BH, ncap, D] -> kco [BH, NCP, D]; values in
// 64-token tiles [BH, ntcap, D, 64] -> vcto [BH, D, NCP]; tokens ncmp..NCP-1 written as zero
// (whatever the caches hold there).
void launch_cmp_cache_layout(const uint16_t* kc, const uint16_t* vtiles, uint16_t* kco,
                             uint16_t* vcto, int BH, int D, int ncap, int ntcap, int ncmp,
                             int NCP, hipStream_t s);

// Compressed attention (lse pass + probability pass), block importance, group selection;
// writes out = gate_cmp * o_cmp (+ gate_win * o_win when a.fuse_window) and idx.
void launch_cmp_select(const PrefillArgs& a, hipStream_t s);
// out += gate_win * o_win.
void launch_window(const PrefillArgs& a, hipStream_t s);
// out += gate_slc * o_slc over the blocks in idx.
void launch_selected(const PrefillArgs& a, hipStream_t s);

size_t cmp_select_lds_bytes(int G, int nblk);
// true when a query tile's block scores do not fit in LDS and the selection streams
bool cmp_select_streams(int G, int nblk);

}  // namespace nsa
