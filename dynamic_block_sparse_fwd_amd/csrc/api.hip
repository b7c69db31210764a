// C-ABI entry points: host-side validation, workspace planning and launch sequencing.
// Everything is enqueued on the caller's stream; no host synchronisation, no allocation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/nsa.h"
#include "kernels.h"

using namespace nsa;

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kMaxDynLds = 64 * 1024;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int round64(int x) { return (x + 63) / 64 * 64; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool g_ok(int G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

int check_nsa(const nsa_config* c) {
  if (c == nullptr) return NSA_ERR_INVALID_ARG;
  if (c->B <= 0 || c->T <= 0 || c->Hkv <= 0 || c->G <= 0 || c->D <= 0 || c->cmp_len <= 0 ||
      c->cmp_stride <= 0 || c->sel_block <= 0 || c->top_n <= 0 || c->n_local < 0 ||
      c->window <= 0 || !(c->scale > 0.f) || !std::isfinite(c->scale))
    return NSA_ERR_INVALID_ARG;
  if (c->D != 64 && c->D != 128) return NSA_ERR_UNSUPPORTED;
  if (!g_ok(c->G)) return NSA_ERR_UNSUPPORTED;
  if (c->sel_block % 64 != 0) return NSA_ERR_UNSUPPORTED;
  if (c->top_n < 1 + c->n_local || c->top_n > 64) return NSA_ERR_UNSUPPORTED;
  if (c->cmp_len < c->cmp_stride) return NSA_ERR_UNSUPPORTED;
  const long nblk = ((long)c->T + c->sel_block - 1) / c->sel_block;
  if (nblk > 2048) return NSA_ERR_UNSUPPORTED;
  if (cmp_select_lds_bytes(c->G, (int)nblk) > kMaxDynLds) return NSA_ERR_UNSUPPORTED;
  if ((long)c->B * c->Hkv * c->G > (1L << 30)) return NSA_ERR_UNSUPPORTED;
  return NSA_OK;
}

int check_moba(const moba_config* c) {
  if (c == nullptr) return NSA_ERR_INVALID_ARG;
  if (c->B <= 0 || c->T <= 0 || c->H <= 0 || c->D <= 0 || c->block <= 0 || c->top_k < 0 ||
      !(c->scale > 0.f) || !std::isfinite(c->scale))
    return NSA_ERR_INVALID_ARG;
  if (c->D != 64 && c->D != 128) return NSA_ERR_UNSUPPORTED;
  if (c->block % 64 != 0 || c->T % c->block != 0) return NSA_ERR_UNSUPPORTED;
  if (c->top_k > 15) return NSA_ERR_UNSUPPORTED;
  return NSA_OK;
}

struct PrefillPlan {
  size_t vt, kc, vct, wkt, wvt, idx, total;
  int ncmp, NCP, TP, nblk;
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

int nsa_compress(const nsa_config* c, const void* x, const void* w, void* xc, void* ws,
                 size_t ws_bytes, hipStream_t stream) {
  int st = check_compress(c);
  if (st != NSA_OK) return st;
  const int ncmp = nsa_num_compressed(c->T, c->cmp_len, c->cmp_stride);
  if (!x || !w || !ws || (!xc && ncmp > 0)) return NSA_ERR_INVALID_ARG;  // empty output may be null
  if (!aligned16(x) || !aligned16(w) || !aligned16(xc) || !aligned16(ws))
    return NSA_ERR_INVALID_ARG;
  if (ws_bytes < nsa_compress_workspace_bytes(c)) return NSA_ERR_WORKSPACE;
  if (ncmp == 0) return NSA_OK;
  const int LD = c->cmp_len * c->D;
  uint16_t* wt = static_cast<uint16_t*>(ws);
  (void)hipGetLastError();
  launch_transpose(static_cast<const uint16_t*>(w), wt, 1, LD, c->D, LD, stream);
  launch_compress(static_cast<const uint16_t*>(x), wt, static_cast<uint16_t*>(xc), nullptr,
                  c->B * c->Hkv, c->T, c->D, c->cmp_len, c->cmp_stride, ncmp, ncmp, 0, stream);
  return hip_status();
}

static int prefill_impl(const nsa_config* c, const void* q, const void* k, const void* v,
                        const void* wk, const void* wv, const float* gate, float* out,
                        int32_t* sel_idx, void* ws, size_t ws_bytes, hipStream_t stream,
                        hipEvent_t* ev) {
  int st = check_nsa(c);
  if (st != NSA_OK) return st;
  if (!q || !k || !v || !wk || !wv || !gate || !out || !ws) return NSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(wk) || !aligned16(wv) ||
      !aligned16(gate) || !aligned16(out) || !aligned16(ws) ||
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
  launch_transpose(static_cast<const uint16_t*>(v), vt, BH, c->T, c->D, p.TP, stream);
  if (p.ncmp > 0) {
    launch_transpose(static_cast<const uint16_t*>(wk), wkt, 1, LD, c->D, LD, stream);
    launch_transpose(static_cast<const uint16_t*>(wv), wvt, 1, LD, c->D, LD, stream);
  }
  mark(1);
  if (p.ncmp > 0) {
    launch_compress(static_cast<const uint16_t*>(k), wkt, kcb, nullptr, BH, c->T, c->D,
                    c->cmp_len, c->cmp_stride, p.ncmp, p.NCP, p.NCP, stream);
    launch_compress(static_cast<const uint16_t*>(v), wvt, nullptr, vct, BH, c->T, c->D,
                    c->cmp_len, c->cmp_stride, p.ncmp, p.NCP, p.NCP, stream);
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
  a.l = c->cmp_len; a.d = c->cmp_stride; a.beta = c->sel_block; a.top_n = c->top_n;
  a.n_local = c->n_local; a.window = c->window;
  a.ncmp = p.ncmp; a.NCP = p.NCP; a.TP = p.TP; a.nblk = p.nblk;
  a.scale_log2 = c->scale * 1.4426950408889634f;
  mark(2);
  launch_cmp_select(a, stream);
  mark(3);
  launch_window(a, stream);
  mark(4);
  launch_selected(a, stream);
  mark(5);
  return hip_status();
}

int nsa_prefill(const nsa_config* c, const void* q, const void* k, const void* v, const void* wk,
                const void* wv, const float* gate, float* out, int32_t* sel_idx, void* ws,
                size_t ws_bytes, hipStream_t stream) {
  return prefill_impl(c, q, k, v, wk, wv, gate, out, sel_idx, ws, ws_bytes, stream, nullptr);
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

}  // extern "C"

// ---- decode and MoBA: kernels land in decode.hip / moba.hip
extern "C" {
size_t nsa_decode_workspace_bytes(const nsa_config* cfg) {
  if (check_nsa(cfg) != NSA_OK) return 0;
  return 0;
}
int nsa_decode(const nsa_config* c, const void*, const void*, const void*, const void*,
               const void*, const int32_t*, const float*, float*, int32_t*, void*, size_t,
               hipStream_t) {
  int st = check_nsa(c);
  return st != NSA_OK ? st : NSA_ERR_UNSUPPORTED;
}
size_t moba_prefill_workspace_bytes(const moba_config* cfg) {
  if (check_moba(cfg) != NSA_OK) return 0;
  return 0;
}
int moba_prefill(const moba_config* c, const void* q, const void* k, const void* v, float* out,
                 int32_t*, void* ws, size_t, hipStream_t) {
  int st = check_moba(c);
  if (st != NSA_OK) return st;
  if (!q || !k || !v || !out || !ws) return NSA_ERR_INVALID_ARG;
  return NSA_ERR_UNSUPPORTED;
}
}
