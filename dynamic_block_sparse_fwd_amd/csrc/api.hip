// C-ABI entry points: host-side validation, workspace planning and launch sequencing.
// Everything is enqueued on the caller's stream; no host synchronisation, no allocation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/nsa.h"
#include "kernels.h"

using namespace nsa;

namespace {


constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int round64(int x) { return (x + 63) / 64 * 64; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool g_ok(int G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

int check_nsa_base(const nsa_config* c) {
  if (c == nullptr) return NSA_ERR_INVALID_ARG;
  if (c->B <= 0 || c->T <= 0 || c->Hkv <= 0 || c->G <= 0 || c->D <= 0 || c->cmp_len <= 0 ||
      c->cmp_stride <= 0 || c->sel_block <= 0 || c->top_n <= 0 || c->n_local < 0 ||
      c->window <= 0 || !(c->scale > 0.f) || !std::isfinite(c->scale) ||
      !(c->top_p >= 0.f && c->top_p <= 1.f))
    return NSA_ERR_INVALID_ARG;
  if (c->D != 64 && c->D != 128) return NSA_ERR_UNSUPPORTED;
  if (!g_ok(c->G)) return NSA_ERR_UNSUPPORTED;
  if (c->sel_block % 64 != 0) return NSA_ERR_UNSUPPORTED;
  if (c->top_n < 1 + c->n_local || c->top_n > 64) return NSA_ERR_UNSUPPORTED;
  if (c->cmp_len < c->cmp_stride) return NSA_ERR_UNSUPPORTED;
  if ((long)c->B * c->Hkv * c->G > (1L << 30)) return NSA_ERR_UNSUPPORTED;
  return NSA_OK;
}

// Prefill lists a row's selected 64-key tiles one per lane and counts the selected branch's
// entries per 64-key tile in LDS (4 bytes per tile of the sequence, 64 KB at 2^20 tokens).  A
// query tile's block scores stay in LDS while they fit; longer sequences select on the fly,
// with the open block sums of the generic geometry in a ring of kCmpRing slots.
constexpr int kCmpRing = 128;

int check_nsa(const nsa_config* c) {
  int st = check_nsa_base(c);
  if (st != NSA_OK) return st;
  if (c->T > (1 << 20)) return NSA_ERR_UNSUPPORTED;
  const long nblk = ((long)c->T + c->sel_block - 1) / c->sel_block;
  const bool fast = c->sel_block == 4 * c->cmp_stride && c->cmp_len == 2 * c->cmp_stride;
  if (cmp_select_streams(c->G, (int)nblk) && !fast &&
      (64L * c->cmp_stride + 2L * c->cmp_len) / c->sel_block + 6 > kCmpRing)
    return NSA_ERR_UNSUPPORTED;
  if (c->top_n * (c->sel_block / 64) > 64) return NSA_ERR_UNSUPPORTED;  // one tile per lane
  if ((long)((c->T + 3) / 4) * c->B * c->Hkv > (1L << 31) - 8) return NSA_ERR_UNSUPPORTED;
  // block-major selected branch: entries are (row << 6 | slot) in 32 bits, work tiles in a 1-D
  // grid
  if ((long)c->B * c->T >= (1L << 25)) return NSA_ERR_UNSUPPORTED;
  if ((long)c->B * c->T * c->Hkv * c->top_n * (c->sel_block / 64) / kSlcRows >= (1L << 30))
    return NSA_ERR_UNSUPPORTED;
  return NSA_OK;
}

struct DecodeShape {
  int ncmp, nblk, NCH, NT, NBT;
  int SB, NSL, KF;
  int NG;     // tile workgroups per group of the last phase
  int NGW;    // of them, the ones that take the window's and forced tiles
  int ntile;  // most tiles a group's list can hold: window, forced and other selected blocks
};

DecodeShape decode_shape(const nsa_config* c) {
  DecodeShape p{};
  p.ncmp = nsa_num_compressed(c->T, c->cmp_len, c->cmp_stride);
  p.nblk = (c->T + c->sel_block - 1) / c->sel_block;
  const int chunk = decode_chunk_tokens();
  p.NCH = (p.ncmp + chunk - 1) / chunk;
  p.NT = (p.ncmp + 63) / 64;
  p.NBT = (63 * c->cmp_stride + c->cmp_len - 1) / c->sel_block + 2;
  const int per = c->sel_block / 64;
  p.SB = decode_slice_blocks(c->cmp_len, c->cmp_stride, c->sel_block);
  p.NSL = (p.nblk + p.SB - 1) / p.SB;
  p.KF = std::max(1, c->top_n - 1 - c->n_local);
  // about 512 tile workgroups in all, at least 2 and at most 8 per group (the merge's limit);
  // a quarter of them (at least one) take the tiles known before the selection
  p.NG = (int)std::min<long>(8, std::max<long>(2, (512 + (long)c->B * c->Hkv - 1) /
                                                      ((long)c->B * c->Hkv)));
  p.NGW = std::max(1, p.NG / 4);
  // the list: every tile when all blocks fit, else the window's and the selected blocks' tiles
  p.ntile = std::max(c->top_n * per, (c->window + 63) / 64 + 1 + c->top_n * per);
  return p;
}

// Decode addresses a cache row with 32-bit offsets, keeps a group's tile list in a 256-entry
// LDS table, stages a group's selection candidates in LDS and launches grids of (slot, KV head,
// sequence) or (KV head, sequence).
int check_nsa_decode(const nsa_config* c) {
  int st = check_nsa_base(c);
  if (st != NSA_OK) return st;
  if (c->T > (1 << 24)) return NSA_ERR_UNSUPPORTED;
  if (c->B > 65535 || c->Hkv > 65535) return NSA_ERR_UNSUPPORTED;
  const DecodeShape p = decode_shape(c);
  if (p.ntile > kDecodeMaxList) return NSA_ERR_UNSUPPORTED;
  if ((long)p.NSL * p.KF > decode_max_candidates(c->D)) return NSA_ERR_UNSUPPORTED;
  return NSA_OK;
}

int check_moba(const moba_config* c) {
  if (c == nullptr) return NSA_ERR_INVALID_ARG;
  if (c->B <= 0 || c->T <= 0 || c->H <= 0 || c->D <= 0 || c->block <= 0 || c->top_k < 0 ||
      !(c->scale > 0.f) || !std::isfinite(c->scale))
    return NSA_ERR_INVALID_ARG;
  if (c->D != 64 && c->D != 128) return NSA_ERR_UNSUPPORTED;
  if (c->block % 64 != 0 || c->T % c->block != 0) return NSA_ERR_UNSUPPORTED;
  if (c->top_k > 8) return NSA_ERR_UNSUPPORTED;
  if ((long)c->T > (1L << 27)) return NSA_ERR_UNSUPPORTED;  // list entries are t << 4 | slot
  if ((long)c->B * c->H * (c->T / 64) > (1L << 31) - 8) return NSA_ERR_UNSUPPORTED;  // 1-D grid
  return NSA_OK;
}

struct MobaPlan {
  size_t vt, hi, lo, count, rank, offset, tstart, ntiles, tile_entry, idx, list, po, pml, total;
  int nb, max_tiles;
  int Hc;  // heads per pass
};

// Heads per pass: all of them while a pass has at most 2^24 query rows (B T Hc), else fewer, so
// that the per-(query, slot) partials stay within 2^24 (top_k) entries.
int moba_heads_per_pass(const moba_config* c) {
  const long cap = (1L << 24) / ((long)c->B * c->T);
  return (int)std::min<long>(c->H, std::max<long>(1, cap));
}

MobaPlan plan_moba(const moba_config* c) {
  MobaPlan p{};
  p.Hc = moba_heads_per_pass(c);
  const size_t BH = (size_t)c->B * p.Hc, rows = BH * c->T;
  p.nb = c->T / c->block;
  const size_t entries = rows * c->top_k;
  p.max_tiles = (int)(entries / 128 + BH * p.nb + 1);
  size_t off = 0;
  p.vt = off;     off += align_up(BH * c->D * c->T * 2);
  p.hi = off;     off += align_up(BH * p.nb * c->D * 2);
  p.lo = off;     off += align_up(BH * p.nb * c->D * 2);
  p.count = off;  off += align_up(BH * p.nb * kMobaChunks * 4);
  p.rank = off;   off += align_up(entries * 4 + 4);
  p.offset = off; off += align_up((BH * p.nb + 1) * 4);
  p.tstart = off; off += align_up(BH * p.nb * 4);
  p.ntiles = off; off += align_up(4);
  p.tile_entry = off; off += align_up((size_t)p.max_tiles * 4);
  p.idx = off;    off += align_up((size_t)c->B * c->T * c->H * (c->top_k + 1) * 4);  // all heads
  p.list = off;   off += align_up(entries * 4 + 4);
  // one spare slot each: the merge loads slot 0 unconditionally, also when top_k = 0
  p.po = off;     off += align_up((entries + 1) * c->D * 2);  // fp16
  p.pml = off;    off += align_up((entries + 1) * 4 * 4);
  p.total = off;
  return p;
}

struct PrefillPlan {
  size_t vt, kc, vct, wkt, wvt, idx, total;
  size_t s_rank, s_kt, s_count, s_offset, s_tstart, s_ntiles, s_tile_entry, s_list, s_po, s_ps;
  size_t kpmax, kcmax;
  int ncmp, NCP, TP, nblk, FS, NTK, s_max_tiles;
};

PrefillPlan plan_prefill(const nsa_config* c) {
  PrefillPlan p{};
  const long BH = (long)c->B * c->Hkv;
  p.ncmp = nsa_num_compressed(c->T, c->cmp_len, c->cmp_stride);
  p.NCP = round64(p.ncmp);
  p.TP = round64(c->T);
  p.nblk = (c->T + c->sel_block - 1) / c->sel_block;
  size_t off = 0;
  p.vt = off;  off += align_up((size_t)BH * c->D * p.TP * 2);
  p.kc = off;  off += align_up((size_t)BH * p.NCP * c->D * 2);
  p.vct = off; off += align_up((size_t)BH * c->D * p.NCP * 2);
  p.wkt = off; off += align_up((size_t)c->cmp_len * c->D * c->D * 2);
  p.wvt = off; off += align_up((size_t)c->cmp_len * c->D * c->D * 2);
  p.idx = off; off += align_up((size_t)c->B * c->T * c->Hkv * c->top_n * 4);
  p.kpmax = off; off += align_up((size_t)BH * p.NCP * 4);
  p.kcmax = off; off += align_up((size_t)BH * ((p.ncmp + kNormRows - 1) / kNormRows + 1) * 4);
  // selected branch, block-major part: sized for query rows 0 .. T-1
  p.FS = c->top_n * (c->sel_block / 64);
  p.NTK = p.TP / 64;
  const size_t nent = (size_t)BH * c->T * p.FS;
  const size_t nsub = (size_t)kSlcChunks * BH * p.NTK;
  p.s_max_tiles = (int)(nent / kSlcRows + nsub + 1);
  p.s_rank = off;       off += align_up(nent * 4);
  p.s_kt = off;         off += align_up(nent * 4);
  p.s_count = off;      off += align_up(nsub * 4);
  p.s_offset = off;     off += align_up((nsub + 1) * 4);
  p.s_tstart = off;     off += align_up(nsub * 4);
  p.s_ntiles = off;     off += align_up(4);
  p.s_tile_entry = off; off += align_up((size_t)p.s_max_tiles * 4);
  p.s_list = off;       off += align_up(nent * 4);
  p.s_po = off;         off += align_up(nent * 16 * c->D * 2);
  p.s_ps = off;         off += align_up(nent * 16 * 4 * 4);
  p.total = off;
  return p;
}

void set_selected_ws(PrefillArgs& a, const PrefillPlan& p, char* base) {
  a.kpmax = reinterpret_cast<float*>(base + p.kpmax);
  a.kcmax = reinterpret_cast<float*>(base + p.kcmax);
  a.NKB = (a.ncmp + kNormRows - 1) / kNormRows;  // a.ncmp is set before this call
  a.s_rank = reinterpret_cast<int32_t*>(base + p.s_rank);
  a.s_kt = reinterpret_cast<int32_t*>(base + p.s_kt);
  a.s_count = reinterpret_cast<int32_t*>(base + p.s_count);
  a.s_offset = reinterpret_cast<int32_t*>(base + p.s_offset);
  a.s_tstart = reinterpret_cast<int32_t*>(base + p.s_tstart);
  a.s_ntiles = reinterpret_cast<int32_t*>(base + p.s_ntiles);
  a.s_tile_entry = reinterpret_cast<int32_t*>(base + p.s_tile_entry);
  a.s_list = reinterpret_cast<int32_t*>(base + p.s_list);
  a.s_po = reinterpret_cast<_Float16*>(base + p.s_po);
  a.s_ps = reinterpret_cast<float*>(base + p.s_ps);
  a.FS = p.FS;
  a.NTK = p.NTK;
  a.s_max_tiles = p.s_max_tiles;
}

struct BackwardPlan {
  size_t kt, kc, kct, vc, wkt, wvt, dob, dot, qt, lse, dlt, pk, pv, dkc, dvc, psk, psv, sbits;
  size_t total;
  int ncmp, NCP, TP, nblk, PC, NPC, SW;
};

BackwardPlan plan_backward(const nsa_config* c) {
  BackwardPlan p{};
  const size_t BH = (size_t)c->B * c->Hkv, rows = (size_t)c->B * c->T * c->Hkv * c->G;
  const size_t rows16 = (size_t)c->B * c->T * c->Hkv * 16;  // 16-row tiles per position
  p.ncmp = nsa_num_compressed(c->T, c->cmp_len, c->cmp_stride);
  p.NCP = round64(p.ncmp);
  p.TP = round64(c->T);
  p.nblk = (c->T + c->sel_block - 1) / c->sel_block;
  // positions per chunk of the compressed and selected key passes: about 16 chunks, at least
  // 256 positions
  p.PC = std::max(256, round64((c->T + 15) / 16));
  p.NPC = (c->T + p.PC - 1) / p.PC;
  const size_t cmpn = BH * (size_t)std::max(p.NCP, 64) * c->D;
  size_t off = 0;
  p.kt = off;  off += align_up(BH * c->D * p.TP * 2);
  p.kc = off;  off += align_up(cmpn * 2);
  p.kct = off; off += align_up(cmpn * 2);
  p.vc = off;  off += align_up(cmpn * 2);
  p.wkt = off; off += align_up((size_t)c->cmp_len * c->D * c->D * 2);
  p.wvt = off; off += align_up((size_t)c->cmp_len * c->D * c->D * 2);
  p.dob = off; off += align_up(rows * c->D * 2);
  p.dot = off; off += align_up(rows16 * c->D * 2);
  p.qt = off;  off += align_up(rows16 * c->D * 2);
  p.lse = off; off += align_up(3 * rows * 4);
  p.dlt = off; off += align_up(3 * rows * 4);
  p.pk = off;  off += align_up((size_t)p.NPC * cmpn * 4);
  p.pv = off;  off += align_up((size_t)p.NPC * cmpn * 4);
  p.dkc = off; off += align_up(cmpn * 4);
  p.dvc = off; off += align_up(cmpn * 4);
  p.psk = off; off += align_up((size_t)p.NPC * BH * c->T * c->D * 4);
  p.psv = off; off += align_up((size_t)p.NPC * BH * c->T * c->D * 4);
  p.SW = (c->T + 31) / 32;
  p.sbits = off; off += align_up(BH * p.nblk * p.SW * 4);
  p.total = off;
  return p;
}

struct DecodePlan {
  size_t cm, cl, co, tref, cb, sS, cand, ocmp, grec, idx, total;
  DecodeShape sh;
};

DecodePlan plan_decode(const nsa_config* c) {
  DecodePlan p{};
  p.sh = decode_shape(c);
  const DecodeShape& d = p.sh;
  const size_t BKV = (size_t)c->B * c->Hkv;
  const size_t F = sizeof(float);
  const size_t nch = d.NCH > 0 ? d.NCH : 1, nt = d.NT > 0 ? d.NT : 1;  // never empty
  size_t off = 0;
  p.cm = off;   off += align_up(BKV * nch * 16 * F);
  p.cl = off;   off += align_up(BKV * nch * 16 * F);
  p.co = off;   off += align_up(BKV * nch * 16 * c->D * F);
  p.tref = off; off += align_up(BKV * nt * 16 * F);
  p.cb = off;   off += align_up(BKV * nt * d.NBT * 16 * F);
  p.sS = off;   off += align_up(BKV * d.NSL * d.SB * F);
  p.cand = off; off += align_up(BKV * d.NSL * d.KF * sizeof(uint64_t));
  p.ocmp = off; off += align_up(BKV * 16 * c->D * F);
  p.grec = off; off += align_up(BKV * d.NG * 2 * (32 + 16 * (size_t)c->D) * F);
  p.idx = off;  off += align_up(BKV * c->top_n * 4);
  p.total = off;
  return p;
}

int hip_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NSA_OK : NSA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* nsa_status_string(int status) {
  switch (status) {
    case NSA_OK: return "ok";
    case NSA_ERR_INVALID_ARG: return "invalid argument (null/misaligned pointer or bad size)";
    case NSA_ERR_UNSUPPORTED: return "configuration not supported by the kernels";
    case NSA_ERR_WORKSPACE: return "workspace too small";
    case NSA_ERR_HIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

int32_t nsa_num_compressed(int32_t T, int32_t cmp_len, int32_t cmp_stride) {
  if (cmp_len <= 0 || cmp_stride <= 0 || T < cmp_len) return 0;
  return (T - cmp_len) / cmp_stride + 1;
}

int32_t nsa_num_compressed_tiles(int32_t T, int32_t cmp_len, int32_t cmp_stride) {
  return (nsa_num_compressed(T, cmp_len, cmp_stride) + 63) / 64;
}

int nsa_validate(const nsa_config* cfg) { return check_nsa(cfg); }
int moba_validate(const moba_config* cfg) { return check_moba(cfg); }

size_t nsa_prefill_workspace_bytes(const nsa_config* cfg) {
  if (check_nsa(cfg) != NSA_OK) return 0;
  return plan_prefill(cfg).total;
}

static int check_compress(const nsa_config* c) {
  if (c == nullptr) return NSA_ERR_INVALID_ARG;
  if (c->B <= 0 || c->T <= 0 || c->Hkv <= 0 || c->D <= 0 || c->cmp_len <= 0 ||
      c->cmp_stride <= 0)
    return NSA_ERR_INVALID_ARG;
  if (c->D != 64 && c->D != 128) return NSA_ERR_UNSUPPORTED;
  return NSA_OK;
}

size_t nsa_compress_workspace_bytes(const nsa_config* c) {
  if (check_compress(c) != NSA_OK) return 0;
  return align_up((size_t)c->cmp_len * c->D * c->D * 2);
}

static int compress_impl(const nsa_config* c, const void* x, const void* w, void* xc, void* xct,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_compress(c);
  if (st != NSA_OK) return st;
  const int ncmp = nsa_num_compressed(c->T, c->cmp_len, c->cmp_stride);
  void* dst = xc ? xc : xct;
  if (!x || !w || !ws || (!dst && ncmp > 0)) return NSA_ERR_INVALID_ARG;  // empty output may be null
  if (!aligned16(x) || !aligned16(w) || !aligned16(dst) || !aligned16(ws))
    return NSA_ERR_INVALID_ARG;
  if (ws_bytes < nsa_compress_workspace_bytes(c)) return NSA_ERR_WORKSPACE;
  if (ncmp == 0) return NSA_OK;
  const int LD = c->cmp_len * c->D;
  uint16_t* wt = static_cast<uint16_t*>(ws);
  const int ncp = xct ? 64 * ((ncmp + 63) / 64) : 0;
  (void)hipGetLastError();
  launch_transpose(static_cast<const uint16_t*>(w), wt, 1, LD, c->D, LD, stream);
  launch_compress(static_cast<const uint16_t*>(x), wt, static_cast<uint16_t*>(xc),
                  static_cast<uint16_t*>(xct), c->B * c->Hkv, c->T, c->D, c->cmp_len,
                  c->cmp_stride, ncmp, xc ? ncmp : 0, ncp, true, stream);
  return hip_status();
}

int nsa_compress(const nsa_config* c, const void* x, const void* w, void* xc, void* ws,
                 size_t ws_bytes, hipStream_t stream) {
  return compress_impl(c, x, w, xc, nullptr, ws, ws_bytes, stream);
}

int nsa_compress_tiles(const nsa_config* c, const void* x, const void* w, void* xct,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  return compress_impl(c, x, w, nullptr, xct, ws, ws_bytes, stream);
}

// Runs the requested prefill stages (NSA_STAGE_* bits) on the stream.  Without the compressed
// stage, `out` is cleared first and the window / selected stages add into it; the selected
// stage alone reads its block indices from `sel_idx`.
static int prefill_run(const nsa_config* c, unsigned stages, const void* q, const void* k,
                       const void* v, const void* wk, const void* wv, const float* gate,
                       float* out, int32_t* sel_idx, void* ws, size_t ws_bytes,
                       hipStream_t stream, hipEvent_t* ev, float* dlse = nullptr,
                       float* dscores = nullptr) {
  int st = check_nsa(c);
  if (st != NSA_OK) return st;
  if (dscores != nullptr &&
      cmp_select_streams(c->G, (c->T + c->sel_block - 1) / c->sel_block))
    return NSA_ERR_UNSUPPORTED;  // the selection streams: no block score array to export
  if (stages == 0 || (stages & ~(unsigned)NSA_STAGE_ALL) != 0) return NSA_ERR_INVALID_ARG;
  const bool s_cmp = stages & NSA_STAGE_CMP_SELECT, s_win = stages & NSA_STAGE_WINDOW;
  const bool s_slc = stages & NSA_STAGE_SELECTED;
  if (!q || !k || !v || !gate || !out || !ws) return NSA_ERR_INVALID_ARG;
  if (s_cmp && (!wk || !wv)) return NSA_ERR_INVALID_ARG;
  if (s_slc && !s_cmp && !sel_idx) return NSA_ERR_INVALID_ARG;  // indices are an input then
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (wk && !aligned16(wk)) ||
      (wv && !aligned16(wv)) || !aligned16(gate) || !aligned16(out) || !aligned16(ws) ||
      (sel_idx && !aligned16(sel_idx)))
    return NSA_ERR_INVALID_ARG;
  const PrefillPlan p = plan_prefill(c);
  if (ws_bytes < p.total) return NSA_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  uint16_t* vt = reinterpret_cast<uint16_t*>(base + p.vt);
  uint16_t* kcb = reinterpret_cast<uint16_t*>(base + p.kc);
  uint16_t* vct = reinterpret_cast<uint16_t*>(base + p.vct);
  uint16_t* wkt = reinterpret_cast<uint16_t*>(base + p.wkt);
  uint16_t* wvt = reinterpret_cast<uint16_t*>(base + p.wvt);
  int32_t* idx = sel_idx ? sel_idx : reinterpret_cast<int32_t*>(base + p.idx);
  const int BH = c->B * c->Hkv;
  const int LD = c->cmp_len * c->D;

  (void)hipGetLastError();
  auto mark = [&](int sidx) {
    if (ev != nullptr) (void)hipEventRecord(ev[sidx], stream);
  };
  mark(0);
  if (s_win || s_slc)
    launch_transpose(static_cast<const uint16_t*>(v), vt, BH, c->T, c->D, p.TP, stream);
  if (s_cmp && p.ncmp > 0) {
    launch_transpose(static_cast<const uint16_t*>(wk), wkt, 1, LD, c->D, LD, stream);
    launch_transpose(static_cast<const uint16_t*>(wv), wvt, 1, LD, c->D, LD, stream);
  }
  if (!s_cmp) launch_fill_zero(out, (size_t)c->B * c->T * c->Hkv * c->G * c->D, stream);
  mark(1);
  if (s_cmp && p.ncmp > 0) {
    launch_compress(static_cast<const uint16_t*>(k), wkt, kcb, nullptr, BH, c->T, c->D,
                    c->cmp_len, c->cmp_stride, p.ncmp, p.NCP, p.NCP, false, stream, nullptr, 0, 1,
                    static_cast<const uint16_t*>(v), wvt, nullptr, vct);
  }
  PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.vt = vt;
  a.kc = kcb;
  a.vct = vct;
  a.gate = gate;
  a.out = out;
  a.idx = idx;
  a.B = c->B; a.T = c->T; a.Hkv = c->Hkv; a.G = c->G; a.D = c->D;
  a.q0 = 0; a.nq = c->T; a.ldq = c->T; a.qs = 0; a.ldk = c->T;
  a.l = c->cmp_len; a.d = c->cmp_stride; a.beta = c->sel_block; a.top_n = c->top_n;
  a.n_local = c->n_local; a.window = c->window; a.top_p = c->top_p;
  a.ncmp = p.ncmp; a.NCP = p.NCP; a.TP = p.TP; a.nblk = p.nblk;
  a.scale_log2 = c->scale * 1.4426950408889634f;
  a.fuse_window = s_cmp && s_win;  // one query tile, out written once
  a.dlse = dlse;
  a.dscores = dscores;
  set_selected_ws(a, p, base);
  mark(2);
  if (s_cmp) launch_cmp_select(a, stream);
  mark(3);
  if (s_win && !s_cmp) launch_window(a, stream);
  mark(4);
  if (s_slc) launch_selected(a, stream);
  mark(5);
  return hip_status();
}

static int prefill_impl(const nsa_config* c, const void* q, const void* k, const void* v,
                        const void* wk, const void* wv, const float* gate, float* out,
                        int32_t* sel_idx, void* ws, size_t ws_bytes, hipStream_t stream,
                        hipEvent_t* ev) {
  return prefill_run(c, NSA_STAGE_ALL, q, k, v, wk, wv, gate, out, sel_idx, ws, ws_bytes,
                     stream, ev);
}

int nsa_prefill_stages(const nsa_config* c, unsigned stages, const void* q, const void* k,
                       const void* v, const void* wk, const void* wv, const float* gate,
                       float* out, int32_t* sel_idx, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  return prefill_run(c, stages, q, k, v, wk, wv, gate, out, sel_idx, ws, ws_bytes, stream,
                     nullptr);
}

int nsa_prefill(const nsa_config* c, const void* q, const void* k, const void* v, const void* wk,
                const void* wv, const float* gate, float* out, int32_t* sel_idx, void* ws,
                size_t ws_bytes, hipStream_t stream) {
  return prefill_impl(c, q, k, v, wk, wv, gate, out, sel_idx, ws, ws_bytes, stream, nullptr);
}

int nsa_prefill_diag(const nsa_config* c, const void* q, const void* k, const void* v,
                     const void* wk, const void* wv, const float* gate, float* out,
                     int32_t* sel_idx, float* lse, float* scores, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  if ((lse && !aligned16(lse)) || (scores && !aligned16(scores))) return NSA_ERR_INVALID_ARG;
  return prefill_run(c, NSA_STAGE_ALL, q, k, v, wk, wv, gate, out, sel_idx, ws, ws_bytes, stream,
                     nullptr, lse, scores);
}

int nsa_prefill_timed(const nsa_config* c, const void* q, const void* k, const void* v,
                      const void* wk, const void* wv, const float* gate, float* out,
                      int32_t* sel_idx, void* ws, size_t ws_bytes, hipStream_t stream,
                      hipEvent_t* events) {
  if (events == nullptr) return NSA_ERR_INVALID_ARG;
  for (int i = 0; i <= NSA_PREFILL_NSTAGES; ++i)
    if (events[i] == nullptr) return NSA_ERR_INVALID_ARG;
  return prefill_impl(c, q, k, v, wk, wv, gate, out, sel_idx, ws, ws_bytes, stream, events);
}

size_t nsa_prefill_chunk_workspace_bytes(const nsa_config* cfg) {
  return nsa_prefill_workspace_bytes(cfg);  // sized for a chunk ending at the capacity
}

int nsa_prefill_chunk(const nsa_config* c, int32_t P, int32_t C, const void* q,
                      const void* kcache, const void* vcache, const void* kcmp,
                      const void* vcmp, const float* gate, float* out, int32_t* sel_idx,
                      void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_nsa(c);
  if (st != NSA_OK) return st;
  if (P < 0 || C <= 0 || (long)P + C > c->T) return NSA_ERR_INVALID_ARG;
  if (P % 64 != 0) return NSA_ERR_UNSUPPORTED;
  const int Tend = P + C;
  const int ncmp = nsa_num_compressed(Tend, c->cmp_len, c->cmp_stride);
  if (!q || !kcache || !vcache || !gate || !out || !ws || (ncmp > 0 && (!kcmp || !vcmp)))
    return NSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(kcmp) ||
      !aligned16(vcmp) || !aligned16(gate) || !aligned16(out) || !aligned16(ws) ||
      (sel_idx && !aligned16(sel_idx)))
    return NSA_ERR_INVALID_ARG;
  const PrefillPlan p = plan_prefill(c);
  if (ws_bytes < p.total) return NSA_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  uint16_t* vt = reinterpret_cast<uint16_t*>(base + p.vt);
  uint16_t* kcb = reinterpret_cast<uint16_t*>(base + p.kc);
  uint16_t* vct = reinterpret_cast<uint16_t*>(base + p.vct);
  const int BH = c->B * c->Hkv;
  const int ncap = nsa_num_compressed(c->T, c->cmp_len, c->cmp_stride);
  PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(kcache);
  a.vt = vt;
  a.kc = kcb;
  a.vct = vct;
  a.gate = gate;
  a.out = out;
  a.idx = sel_idx ? sel_idx : reinterpret_cast<int32_t*>(base + p.idx);
  a.B = c->B; a.T = Tend; a.Hkv = c->Hkv; a.G = c->G; a.D = c->D;
  a.q0 = P; a.nq = C; a.ldq = C; a.qs = P; a.ldk = c->T;
  a.l = c->cmp_len; a.d = c->cmp_stride; a.beta = c->sel_block; a.top_n = c->top_n;
  a.n_local = c->n_local; a.window = c->window; a.top_p = c->top_p;
  a.ncmp = ncmp; a.NCP = round64(ncmp); a.TP = round64(Tend);
  a.nblk = (Tend + c->sel_block - 1) / c->sel_block;
  a.scale_log2 = c->scale * 1.4426950408889634f;
  a.fuse_window = 1;
  set_selected_ws(a, p, base);
  a.NTK = a.TP / 64;  // key tiles of this chunk's keys; the lists are sized for the capacity
  (void)hipGetLastError();
  launch_transpose(static_cast<const uint16_t*>(vcache), vt, BH, Tend, c->D, a.TP, stream, c->T);
  launch_cmp_cache_layout(static_cast<const uint16_t*>(kcmp), static_cast<const uint16_t*>(vcmp),
                          kcb, vct, BH, c->D, ncap, (ncap + 63) / 64, ncmp, a.NCP, stream);
  launch_cmp_select(a, stream);
  launch_selected(a, stream);
  return hip_status();
}

// Appends that complete at most split_tokens(cfg) compressed tokens per sequence-head compress
// with the split reduction (the completed tokens of all sequence-heads gathered into 64-row
// tiles, the l*D reduction split over workgroups, fp32 partials summed in split order): its
// partials take at most kSplitPartBytes of workspace, and at least kFewTokens tokens per
// sequence-head are allowed.  Longer appends use the 64-token tile compressor, whose long
// reduction per workgroup needs many workgroups to fill the GPU.
constexpr int kFewTokens = 4;
constexpr size_t kSplitPartBytes = (size_t)64 << 20;

static int split_tokens(const nsa_config* c) {
  const size_t one = few_part_bytes(c->B * c->Hkv, c->D, c->cmp_len, 1);
  const int ncap = nsa_num_compressed(c->T, c->cmp_len, c->cmp_stride);
  long n = one > 0 ? (long)(kSplitPartBytes / one) : kFewTokens;
  n = std::max<long>(n, kFewTokens);
  n = std::min<long>(n, std::max(ncap, kFewTokens));
  return (int)n;
}

size_t nsa_cache_append_workspace_bytes(const nsa_config* c) {
  if (check_compress(c) != NSA_OK) return 0;
  return 2 * align_up((size_t)c->cmp_len * c->D * c->D * 2) +
         align_up(few_part_bytes(c->B * c->Hkv, c->D, c->cmp_len, split_tokens(c)));
}

int nsa_cache_append(const nsa_config* c, int32_t C, const void* k_new, const void* v_new,
                     const int32_t* seqlens, const void* wk, const void* wv, void* kcache,
                     void* vcache, void* kcmp, void* vcmp, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  int st = check_compress(c);
  if (st != NSA_OK) return st;
  if (C <= 0 || C > c->T) return NSA_ERR_INVALID_ARG;
  const int ncap = nsa_num_compressed(c->T, c->cmp_len, c->cmp_stride);
  if (!k_new || !v_new || !seqlens || !kcache || !vcache ||
      (ncap > 0 && (!wk || !wv || !kcmp || !vcmp || !ws)))
    return NSA_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(seqlens) || !aligned16(kcache) ||
      !aligned16(vcache) || !aligned16(wk) || !aligned16(wv) || !aligned16(kcmp) ||
      !aligned16(vcmp) || !aligned16(ws))
    return NSA_ERR_INVALID_ARG;
  if (ncap > 0 && ws_bytes < nsa_cache_append_workspace_bytes(c)) return NSA_ERR_WORKSPACE;
  const int BH = c->B * c->Hkv, LD = c->cmp_len * c->D;
  uint16_t* kc16 = static_cast<uint16_t*>(kcache);
  uint16_t* vc16 = static_cast<uint16_t*>(vcache);
  (void)hipGetLastError();
  launch_append_rows(static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                     kc16, vc16, seqlens, BH, c->Hkv, C, c->T, c->D, stream);
  // at most C / d + 1 compressed tokens per sequence-head are completed
  const int per = C / c->cmp_stride + 1 < ncap ? C / c->cmp_stride + 1 : ncap;
  if (ncap > 0 && per <= split_tokens(c)) {
    char* base = static_cast<char*>(ws);
    uint16_t* wkt = reinterpret_cast<uint16_t*>(base);
    uint16_t* wvt = reinterpret_cast<uint16_t*>(base + align_up((size_t)LD * c->D * 2));
    float* part = reinterpret_cast<float*>(base + 2 * align_up((size_t)LD * c->D * 2));
    launch_append_weights(static_cast<const uint16_t*>(wk), static_cast<const uint16_t*>(wv),
                          wkt, wvt, LD, c->D, seqlens, c->B, C, c->cmp_len, c->cmp_stride, ncap,
                          stream);
    const uint16_t* xs[2] = {kc16, vc16};
    const uint16_t* wts[2] = {wkt, wvt};
    uint16_t* xcs[2] = {static_cast<uint16_t*>(kcmp), nullptr};
    uint16_t* xcts[2] = {nullptr, static_cast<uint16_t*>(vcmp)};
    launch_compress_few(xs, wts, xcs, xcts, part, BH, c->T, c->D, c->cmp_len,
                        c->cmp_stride, ncap, ncap, 64 * ((ncap + 63) / 64), seqlens, C, c->Hkv,
                        per, stream);
  } else if (ncap > 0) {
    uint16_t* wkt = static_cast<uint16_t*>(ws);
    uint16_t* wvt = wkt + align_up((size_t)LD * c->D * 2) / 2;
    launch_append_weights(static_cast<const uint16_t*>(wk), static_cast<const uint16_t*>(wv),
                          wkt, wvt, LD, c->D, seqlens, c->B, C, c->cmp_len, c->cmp_stride, ncap,
                          stream);
    // keys (row-major) and values (tiles) in one launch
    launch_compress(kc16, wkt, static_cast<uint16_t*>(kcmp), nullptr, BH, c->T, c->D,
                    c->cmp_len, c->cmp_stride, ncap, ncap, 64 * ((ncap + 63) / 64), true, stream,
                    seqlens, C, c->Hkv, vc16, wvt, nullptr, static_cast<uint16_t*>(vcmp));
  }
  return hip_status();
}

static int check_nsa_backward(const nsa_config* c) { return check_nsa(c); }

size_t nsa_backward_workspace_bytes(const nsa_config* cfg) {
  if (check_nsa_backward(cfg) != NSA_OK) return 0;
  return plan_backward(cfg).total;
}

static int backward_impl(const nsa_config* c, const void* q, const void* k, const void* v,
                         const void* wk, const void* wv, const float* gate,
                         const int32_t* sel_idx, const float* dout, float* dq, float* dk,
                         float* dv, float* dwk, float* dwv, float* dgate, void* ws,
                         size_t ws_bytes, hipStream_t stream, hipEvent_t* ev) {
  int st = check_nsa_backward(c);
  if (st != NSA_OK) return st;
  if (!q || !k || !v || !wk || !wv || !gate || !sel_idx || !dout || !dq || !dk || !dv || !dwk ||
      !dwv || !dgate || !ws)
    return NSA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, wk, wv, gate, sel_idx, dout, dq, dk, dv, dwk, dwv, dgate, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return NSA_ERR_INVALID_ARG;
  const BackwardPlan p = plan_backward(c);
  if (ws_bytes < p.total) return NSA_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  auto u16p = [&](size_t o) { return reinterpret_cast<uint16_t*>(base + o); };
  auto f32p = [&](size_t o) { return reinterpret_cast<float*>(base + o); };
  BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.wk = static_cast<const uint16_t*>(wk);
  a.wv = static_cast<const uint16_t*>(wv);
  a.gate = gate;
  a.idx = sel_idx;
  a.dout = dout;
  a.kt = u16p(p.kt); a.kc = u16p(p.kc); a.kct = u16p(p.kct); a.vc = u16p(p.vc);
  a.dob = u16p(p.dob); a.dot = u16p(p.dot); a.qt = u16p(p.qt);
  a.lse = f32p(p.lse); a.dlt = f32p(p.dlt); a.pk = f32p(p.pk); a.pv = f32p(p.pv);
  a.dkc = f32p(p.dkc); a.dvc = f32p(p.dvc); a.psk = f32p(p.psk); a.psv = f32p(p.psv);
  a.selbits = reinterpret_cast<uint32_t*>(base + p.sbits);
  a.SW = p.SW;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dwk = dwk; a.dwv = dwv; a.dgate = dgate;
  a.B = c->B; a.T = c->T; a.Hkv = c->Hkv; a.G = c->G; a.D = c->D;
  a.l = c->cmp_len; a.d = c->cmp_stride;
  a.beta = c->sel_block; a.top_n = c->top_n; a.window = c->window;
  a.ncmp = p.ncmp; a.NCP = p.NCP; a.TP = p.TP; a.nblk = p.nblk; a.PC = p.PC; a.NPC = p.NPC;
  a.scale = c->scale;
  a.scale_log2 = c->scale * 1.4426950408889634f;
  const int BH = c->B * c->Hkv, LD = c->cmp_len * c->D;
  (void)hipGetLastError();
  if (ev != nullptr) (void)hipEventRecord(ev[0], stream);
  launch_transpose(a.k, u16p(p.kt), BH, c->T, c->D, p.TP, stream);
  if (p.ncmp > 0) {
    launch_transpose(a.wk, u16p(p.wkt), 1, LD, c->D, LD, stream);
    launch_transpose(a.wv, u16p(p.wvt), 1, LD, c->D, LD, stream);
    launch_compress(a.k, u16p(p.wkt), u16p(p.kc), u16p(p.kct), BH, c->T, c->D, c->cmp_len,
                    c->cmp_stride, p.ncmp, p.NCP, p.NCP, false, stream, nullptr, 0, 1, a.v,
                    u16p(p.wvt), u16p(p.vc), nullptr);
  }
  if (ev != nullptr) (void)hipEventRecord(ev[1], stream);
  launch_backward(a, stream, ev);
  return hip_status();
}

int nsa_backward(const nsa_config* c, const void* q, const void* k, const void* v,
                 const void* wk, const void* wv, const float* gate, const int32_t* sel_idx,
                 const float* dout, float* dq, float* dk, float* dv, float* dwk, float* dwv,
                 float* dgate, void* ws, size_t ws_bytes, hipStream_t stream) {
  return backward_impl(c, q, k, v, wk, wv, gate, sel_idx, dout, dq, dk, dv, dwk, dwv, dgate, ws,
                       ws_bytes, stream, nullptr);
}

int nsa_backward_timed(const nsa_config* c, const void* q, const void* k, const void* v,
                       const void* wk, const void* wv, const float* gate,
                       const int32_t* sel_idx, const float* dout, float* dq, float* dk,
                       float* dv, float* dwk, float* dwv, float* dgate, void* ws,
                       size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
  if (events == nullptr) return NSA_ERR_INVALID_ARG;
  for (int i = 0; i <= NSA_BACKWARD_NSTAGES; ++i)
    if (events[i] == nullptr) return NSA_ERR_INVALID_ARG;
  return backward_impl(c, q, k, v, wk, wv, gate, sel_idx, dout, dq, dk, dv, dwk, dwv, dgate, ws,
                       ws_bytes, stream, events);
}

size_t nsa_decode_workspace_bytes(const nsa_config* cfg) {
  if (check_nsa_decode(cfg) != NSA_OK) return 0;
  return plan_decode(cfg).total;
}

static int decode_impl(const nsa_config* c, const void* q, const void* kcache,
                       const void* vcache, const void* kcmp, const void* vcmp,
                       const int32_t* seqlens, const float* gate, float* out, int32_t* sel_idx,
                       void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* ev) {
  int st = check_nsa_decode(c);
  if (st != NSA_OK) return st;
  const DecodePlan p = plan_decode(c);
  if (!q || !kcache || !vcache || !seqlens || !gate || !out || !ws ||
      (p.sh.ncmp > 0 && (!kcmp || !vcmp)))
    return NSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(kcmp) ||
      !aligned16(vcmp) || !aligned16(seqlens) || !aligned16(gate) || !aligned16(out) ||
      !aligned16(ws) || (sel_idx && !aligned16(sel_idx)))
    return NSA_ERR_INVALID_ARG;
  if (ws_bytes < p.total) return NSA_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kcache = static_cast<const uint16_t*>(kcache);
  a.vcache = static_cast<const uint16_t*>(vcache);
  a.kc = static_cast<const uint16_t*>(kcmp);
  a.vct = static_cast<const uint16_t*>(vcmp);
  a.seqlens = seqlens;
  a.gate = gate;
  a.out = out;
  a.idx = sel_idx ? sel_idx : reinterpret_cast<int32_t*>(base + p.idx);
  a.cm = reinterpret_cast<float*>(base + p.cm);
  a.cl = reinterpret_cast<float*>(base + p.cl);
  a.co = reinterpret_cast<float*>(base + p.co);
  a.tref = reinterpret_cast<float*>(base + p.tref);
  a.cb = reinterpret_cast<float*>(base + p.cb);
  a.sS = reinterpret_cast<float*>(base + p.sS);
  a.cand = reinterpret_cast<uint64_t*>(base + p.cand);
  a.ocmp = reinterpret_cast<float*>(base + p.ocmp);
  a.grec = reinterpret_cast<float*>(base + p.grec);
  a.B = c->B; a.L = c->T; a.Hkv = c->Hkv; a.G = c->G; a.D = c->D;
  a.l = c->cmp_len; a.d = c->cmp_stride; a.beta = c->sel_block; a.top_n = c->top_n;
  a.n_local = c->n_local; a.window = c->window; a.top_p = c->top_p;
  a.ncmp = p.sh.ncmp; a.nblk = p.sh.nblk; a.NCH = p.sh.NCH; a.NT = p.sh.NT; a.NBT = p.sh.NBT;
  a.SB = p.sh.SB; a.NSL = p.sh.NSL; a.KF = p.sh.KF; a.NG = p.sh.NG; a.NGW = p.sh.NGW;
  a.scale_log2 = c->scale * 1.4426950408889634f;
  (void)hipGetLastError();
  launch_decode(a, stream, ev);
  return hip_status();
}

int nsa_decode(const nsa_config* c, const void* q, const void* kcache, const void* vcache,
               const void* kcmp, const void* vcmp, const int32_t* seqlens, const float* gate,
               float* out, int32_t* sel_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(c, q, kcache, vcache, kcmp, vcmp, seqlens, gate, out, sel_idx, ws,
                     ws_bytes, stream, nullptr);
}

}  // extern "C"

// ---- allocation-free decode

namespace {

// The workspace of nsa_decode_noalloc: one copy per GPU, in the code object's device memory,
// held until the process ends.  In host code `scratch` names a host-side stand-in; the device
// address of each GPU's copy comes from hipGetSymbolAddress on that device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// This GPU's copy of the scratch array (resolved once per device, with that device current);
// null on failure.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t nsa_decode_noalloc_max_bytes(void) { return kScratchBytes; }

int nsa_decode_noalloc(const nsa_config* c, const void* q, const void* kcache, const void* vcache,
                       const void* kcmp, const void* vcmp, const int32_t* seqlens,
                       const float* gate, float* out, int32_t* sel_idx, hipStream_t stream) {
  int st = check_nsa_decode(c);
  if (st != NSA_OK) return st;
  if (plan_decode(c).total > kScratchBytes) return NSA_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return NSA_ERR_HIP;
  return decode_impl(c, q, kcache, vcache, kcmp, vcmp, seqlens, gate, out, sel_idx, ws,
                     kScratchBytes, stream, nullptr);
}

int nsa_decode_timed(const nsa_config* c, const void* q, const void* kcache, const void* vcache,
                     const void* kcmp, const void* vcmp, const int32_t* seqlens,
                     const float* gate, float* out, int32_t* sel_idx, void* ws, size_t ws_bytes,
                     hipStream_t stream, hipEvent_t* events) {
  if (events == nullptr) return NSA_ERR_INVALID_ARG;
  for (int i = 0; i <= NSA_DECODE_NSTAGES; ++i)
    if (events[i] == nullptr) return NSA_ERR_INVALID_ARG;
  return decode_impl(c, q, kcache, vcache, kcmp, vcmp, seqlens, gate, out, sel_idx, ws,
                     ws_bytes, stream, events);
}

}  // extern "C"

// ---- MoBA
extern "C" {

size_t moba_prefill_workspace_bytes(const moba_config* cfg) {
  if (check_moba(cfg) != NSA_OK) return 0;
  return plan_moba(cfg).total;
}

static int moba_impl(const moba_config* c, const void* q, const void* k, const void* v,
                     float* out, int32_t* sel_idx, void* ws, size_t ws_bytes,
                     hipStream_t stream, hipEvent_t* ev) {
  int st = check_moba(c);
  if (st != NSA_OK) return st;
  if (!q || !k || !v || !out || !ws) return NSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(ws) ||
      (sel_idx && !aligned16(sel_idx)))
    return NSA_ERR_INVALID_ARG;
  const MobaPlan p = plan_moba(c);
  if (ws_bytes < p.total) return NSA_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  MobaArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.vt = reinterpret_cast<const uint16_t*>(base + p.vt);
  a.out = out;
  a.kb_hi = reinterpret_cast<uint16_t*>(base + p.hi);
  a.kb_lo = reinterpret_cast<uint16_t*>(base + p.lo);
  a.count = reinterpret_cast<int32_t*>(base + p.count);
  a.rank = reinterpret_cast<int32_t*>(base + p.rank);
  a.offset = reinterpret_cast<int32_t*>(base + p.offset);
  a.tstart = reinterpret_cast<int32_t*>(base + p.tstart);
  a.ntiles = reinterpret_cast<int32_t*>(base + p.ntiles);
  a.tile_entry = reinterpret_cast<int32_t*>(base + p.tile_entry);
  a.list = reinterpret_cast<int32_t*>(base + p.list);
  a.po = reinterpret_cast<_Float16*>(base + p.po);
  a.pml = reinterpret_cast<float*>(base + p.pml);
  a.idx = sel_idx ? sel_idx : reinterpret_cast<int32_t*>(base + p.idx);
  a.B = c->B; a.T = c->T; a.D = c->D; a.block = c->block; a.top_k = c->top_k;
  a.nb = p.nb; a.max_tiles = p.max_tiles; a.Hs = c->H;
  a.scale_log2 = c->scale * 1.4426950408889634f;
  (void)hipGetLastError();
  if (ev != nullptr) (void)hipEventRecord(ev[0], stream);
  // heads in passes of Hc; with events, the stage marks are those of the last pass
  for (int h0 = 0; h0 < c->H; h0 += p.Hc) {
    a.h0 = h0;
    a.H = std::min(p.Hc, c->H - h0);
    const size_t head = (size_t)c->T * c->D;  // elements of one (sequence, head) of v
    for (int b = 0; b < c->B; ++b)
      launch_transpose(static_cast<const uint16_t*>(v) + ((size_t)b * c->H + h0) * head,
                       reinterpret_cast<uint16_t*>(base + p.vt) + (size_t)b * a.H * head, a.H,
                       c->T, c->D, c->T, stream);
    launch_moba(a, stream, ev);
  }
  return hip_status();
}

int moba_prefill(const moba_config* c, const void* q, const void* k, const void* v, float* out,
                 int32_t* sel_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  return moba_impl(c, q, k, v, out, sel_idx, ws, ws_bytes, stream, nullptr);
}

int moba_prefill_timed(const moba_config* c, const void* q, const void* k, const void* v,
                       float* out, int32_t* sel_idx, void* ws, size_t ws_bytes,
                       hipStream_t stream, hipEvent_t* events) {
  if (events == nullptr) return NSA_ERR_INVALID_ARG;
  for (int i = 0; i <= NSA_MOBA_NSTAGES; ++i)
    if (events[i] == nullptr) return NSA_ERR_INVALID_ARG;
  return moba_impl(c, q, k, v, out, sel_idx, ws, ws_bytes, stream, events);
}

}  // extern "C"
