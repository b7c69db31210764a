"""Thin ctypes binding of libnsa.so, the gfx950 NSA / MoBA forward library.

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
torch provides device memory and the current stream; tensors are passed by data_ptr().
bf16 tensors may be torch.bfloat16 or int16/uint16 holding bf16 bit patterns.

There is no fallback: if libnsa.so is missing the import of the binding fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
# NSA_LIBRARY: another build of the library (the host-side sanitizer run of the tests)
LIB_PATH = os.environ.get("NSA_LIBRARY") or os.path.join(_PKG, "libnsa.so")

NSA_OK = 0
NSA_ERR_INVALID_ARG = -1
NSA_ERR_UNSUPPORTED = -2
NSA_ERR_WORKSPACE = -3
NSA_ERR_HIP = -4

_lib = None


class NsaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, status_string(status), status))


class nsa_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "T", "Hkv", "G", "D", "cmp_len", "cmp_stride",
                                               "sel_block", "top_n", "n_local", "window")] + \
               [("scale", ctypes.c_float), ("top_p", ctypes.c_float)]


class moba_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "T", "H", "D", "block", "top_k")] + \
               [("scale", ctypes.c_float)]


EXPORTS = {
    # name: (restype, argtypes)
    "nsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "nsa_validate": (ctypes.c_int, [ctypes.c_void_p]),
    "moba_validate": (ctypes.c_int, [ctypes.c_void_p]),
    "nsa_num_compressed": (ctypes.c_int32, [ctypes.c_int32] * 3),
    "nsa_num_compressed_tiles": (ctypes.c_int32, [ctypes.c_int32] * 3),
    "nsa_compress_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "nsa_prefill_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "nsa_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "moba_prefill_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "nsa_compress": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p]),
    "nsa_compress_tiles": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p]),
    "nsa_prefill": (ctypes.c_int, [ctypes.c_void_p] * 10 + [ctypes.c_size_t, ctypes.c_void_p]),
    "nsa_prefill_stages": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint] + [ctypes.c_void_p] * 9
                           + [ctypes.c_size_t, ctypes.c_void_p]),
    "nsa_prefill_diag": (ctypes.c_int, [ctypes.c_void_p] * 12 + [ctypes.c_size_t,
                                                                 ctypes.c_void_p]),
    "nsa_prefill_timed": (ctypes.c_int,
                          [ctypes.c_void_p] * 10 + [ctypes.c_size_t, ctypes.c_void_p,
                                                     ctypes.c_void_p]),
    "nsa_decode": (ctypes.c_int, [ctypes.c_void_p] * 11 + [ctypes.c_size_t, ctypes.c_void_p]),
    "nsa_decode_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 11),
    "nsa_decode_noalloc_max_bytes": (ctypes.c_size_t, []),
    "nsa_decode_timed": (ctypes.c_int, [ctypes.c_void_p] * 11 + [ctypes.c_size_t, ctypes.c_void_p,
                                                                 ctypes.c_void_p]),
    "nsa_cache_append_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "nsa_cache_append": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32] + [ctypes.c_void_p] * 10
                         + [ctypes.c_size_t, ctypes.c_void_p]),
    "nsa_prefill_chunk_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "nsa_prefill_chunk": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
                          + [ctypes.c_void_p] * 9 + [ctypes.c_size_t, ctypes.c_void_p]),
    "nsa_backward_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "nsa_backward": (ctypes.c_int, [ctypes.c_void_p] * 16 + [ctypes.c_size_t, ctypes.c_void_p]),
    "nsa_backward_timed": (ctypes.c_int, [ctypes.c_void_p] * 16 + [ctypes.c_size_t,
                                                                   ctypes.c_void_p,
                                                                   ctypes.c_void_p]),
    "moba_prefill": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_size_t, ctypes.c_void_p]),
    "moba_prefill_timed": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_size_t, ctypes.c_void_p,
                                                                  ctypes.c_void_p]),
}


def load_library(path: str = LIB_PATH):
    """Load libnsa.so; raises OSError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise OSError("libnsa.so not built (%s); run __graft_entry__.build()" % path)
        lib = ctypes.CDLL(path)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().nsa_status_string(status).decode()


@dataclass
class NsaConfig:
    B: int
    T: int
    Hkv: int
    G: int
    D: int
    cmp_len: int = 32
    cmp_stride: int = 16
    sel_block: int = 64
    top_n: int = 16
    n_local: int = 2
    window: int = 512
    scale: float = None
    top_p: float = 0.0  # 0: fixed top_n; in (0, 1]: adaptive cut by cumulative importance

    @property
    def Hq(self):
        return self.Hkv * self.G

    @property
    def ncmp(self):
        return (self.T - self.cmp_len) // self.cmp_stride + 1 if self.T >= self.cmp_len else 0

    @property
    def ncmp_tiles(self):
        """64-token tiles of compressed tokens: ceil(ncmp / 64)."""
        return (self.ncmp + 63) // 64

    def c(self):
        s = self.scale if self.scale is not None else self.D ** -0.5
        return nsa_config(self.B, self.T, self.Hkv, self.G, self.D, self.cmp_len,
                          self.cmp_stride, self.sel_block, self.top_n, self.n_local,
                          self.window, s, self.top_p)


@dataclass
class MobaConfig:
    B: int
    T: int
    H: int
    D: int
    block: int = 512
    top_k: int = 3
    scale: float = None

    def c(self):
        s = self.scale if self.scale is not None else self.D ** -0.5
        return moba_config(self.B, self.T, self.H, self.D, self.block, self.top_k, s)


# ---------------------------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _dev(x, name, dtypes, shape=None):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not x.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if x.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, x.dtype, dtypes))
    if shape is not None and tuple(x.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(x.shape), tuple(shape)))
    return ctypes.c_void_p(x.data_ptr())


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes, device, ws=None):
    torch = _torch()
    if ws is None:
        ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    if ws.numel() < nbytes:
        raise ValueError("workspace of %d bytes, need %d" % (ws.numel(), nbytes))
    return ws


def _check(st, what):
    if st != NSA_OK:
        raise NsaError(st, what)


def compress_workspace_bytes(cfg: NsaConfig) -> int:
    return load_library().nsa_compress_workspace_bytes(ctypes.byref(cfg.c()))


def prefill_workspace_bytes(cfg: NsaConfig) -> int:
    return load_library().nsa_prefill_workspace_bytes(ctypes.byref(cfg.c()))


def cache_append_workspace_bytes(cfg: NsaConfig) -> int:
    return load_library().nsa_cache_append_workspace_bytes(ctypes.byref(cfg.c()))


def decode_workspace_bytes(cfg: NsaConfig) -> int:
    return load_library().nsa_decode_workspace_bytes(ctypes.byref(cfg.c()))


def moba_workspace_bytes(cfg: MobaConfig) -> int:
    return load_library().moba_prefill_workspace_bytes(ctypes.byref(cfg.c()))


def nsa_compress(cfg: NsaConfig, x, w, out=None, ws=None, stream=None):
    """x bf16 [B, Hkv, T, D], w bf16 [l, D, D] -> compressed bf16 bits [B, Hkv, n_cmp, D]."""
    torch = _torch()
    lib = load_library()
    c = cfg.c()
    if out is None:
        out = torch.empty((cfg.B, cfg.Hkv, cfg.ncmp, cfg.D), dtype=torch.int16, device=x.device)
    ws = _workspace(lib.nsa_compress_workspace_bytes(ctypes.byref(c)), x.device, ws)
    bt = _bf16_types()
    st = lib.nsa_compress(ctypes.byref(c), _dev(x, "x", bt, (cfg.B, cfg.Hkv, cfg.T, cfg.D)),
                          _dev(w, "w", bt, (cfg.cmp_len, cfg.D, cfg.D)),
                          _dev(out, "out", bt, (cfg.B, cfg.Hkv, cfg.ncmp, cfg.D)),
                          ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream))
    _check(st, "nsa_compress")
    return out


def nsa_compress_tiles(cfg: NsaConfig, x, w, out=None, ws=None, stream=None):
    """x bf16 [B, Hkv, T, D], w bf16 [l, D, D] -> compressed bf16 bits in feature-major 64-token
    tiles [B, Hkv, ncmp_tiles, D, 64] (tokens past n_cmp zero); the compressed-value layout of
    nsa_decode."""
    torch = _torch()
    lib = load_library()
    c = cfg.c()
    shape = (cfg.B, cfg.Hkv, cfg.ncmp_tiles, cfg.D, 64)
    if out is None:
        out = torch.empty(shape, dtype=torch.int16, device=x.device)
    ws = _workspace(lib.nsa_compress_workspace_bytes(ctypes.byref(c)), x.device, ws)
    bt = _bf16_types()
    st = lib.nsa_compress_tiles(
        ctypes.byref(c), _dev(x, "x", bt, (cfg.B, cfg.Hkv, cfg.T, cfg.D)),
        _dev(w, "w", bt, (cfg.cmp_len, cfg.D, cfg.D)), _dev(out, "out", bt, shape),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream))
    _check(st, "nsa_compress_tiles")
    return out


PREFILL_STAGES = ("layout", "compress", "cmp_select", "window", "selected")


def nsa_prefill(cfg: NsaConfig, q, k, v, wk, wv, gate, out=None, sel_idx=None, ws=None,
                want_idx=True, stream=None, events=None):
    """Returns (out fp32 [B,T,Hq,D], sel_idx int32 [B,T,Hkv,top_n] or None).
    events: optional ctypes array of len(PREFILL_STAGES) + 1 hipEvent_t handles, recorded
    around every stage (nsa_prefill_timed)."""
    torch = _torch()
    lib = load_library()
    c = cfg.c()
    B, T, Hkv, Hq, D = cfg.B, cfg.T, cfg.Hkv, cfg.Hq, cfg.D
    dev = q.device
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    if want_idx and sel_idx is None:
        sel_idx = torch.empty((B, T, Hkv, cfg.top_n), dtype=torch.int32, device=dev)
    ws = _workspace(lib.nsa_prefill_workspace_bytes(ctypes.byref(c)), dev, ws)
    bt = _bf16_types()
    fn = lib.nsa_prefill if events is None else lib.nsa_prefill_timed
    extra = () if events is None else (ctypes.cast(events, ctypes.c_void_p),)
    st = fn(
        ctypes.byref(c), _dev(q, "q", bt, (B, T, Hq, D)), _dev(k, "k", bt, (B, Hkv, T, D)),
        _dev(v, "v", bt, (B, Hkv, T, D)), _dev(wk, "wk", bt, (cfg.cmp_len, D, D)),
        _dev(wv, "wv", bt, (cfg.cmp_len, D, D)),
        _dev(gate, "gate", (torch.float32,), (B, T, Hq, 3)),
        _dev(out, "out", (torch.float32,), (B, T, Hq, D)),
        None if sel_idx is None else _dev(sel_idx, "sel_idx", (torch.int32,), (B, T, Hkv, cfg.top_n)),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream), *extra)
    _check(st, "nsa_prefill")
    return out, sel_idx


def nsa_prefill_diag(cfg: NsaConfig, q, k, v, wk, wv, gate, want_scores=True, ws=None,
                     stream=None):
    """nsa_prefill plus its diagnostics: returns (out, sel_idx, lse fp32 [B,T,Hq], scores fp32
    [B,T,Hkv,nblk] or None).  lse: ln of the compressed branch's softmax sum (-inf with no
    visible compressed token); scores: the group block scores the selection ranks."""
    torch = _torch()
    lib = load_library()
    c = cfg.c()
    B, T, Hkv, Hq, D = cfg.B, cfg.T, cfg.Hkv, cfg.Hq, cfg.D
    nblk = (T + cfg.sel_block - 1) // cfg.sel_block
    dev = q.device
    f32 = (torch.float32,)
    out = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    sel_idx = torch.empty((B, T, Hkv, cfg.top_n), dtype=torch.int32, device=dev)
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=dev)
    scores = torch.empty((B, T, Hkv, nblk), dtype=torch.float32, device=dev) if want_scores \
        else None
    ws = _workspace(lib.nsa_prefill_workspace_bytes(ctypes.byref(c)), dev, ws)
    bt = _bf16_types()
    st = lib.nsa_prefill_diag(
        ctypes.byref(c), _dev(q, "q", bt, (B, T, Hq, D)), _dev(k, "k", bt, (B, Hkv, T, D)),
        _dev(v, "v", bt, (B, Hkv, T, D)), _dev(wk, "wk", bt, (cfg.cmp_len, D, D)),
        _dev(wv, "wv", bt, (cfg.cmp_len, D, D)), _dev(gate, "gate", f32, (B, T, Hq, 3)),
        _dev(out, "out", f32, (B, T, Hq, D)),
        _dev(sel_idx, "sel_idx", (torch.int32,), (B, T, Hkv, cfg.top_n)),
        _dev(lse, "lse", f32, (B, T, Hq)),
        None if scores is None else _dev(scores, "scores", f32, (B, T, Hkv, nblk)),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream))
    _check(st, "nsa_prefill_diag")
    return out, sel_idx, lse, scores


STAGE_CMP_SELECT, STAGE_WINDOW, STAGE_SELECTED = 1, 2, 4
STAGE_ALL = STAGE_CMP_SELECT | STAGE_WINDOW | STAGE_SELECTED


def nsa_prefill_stages(cfg: NsaConfig, stages: int, q, k, v, wk, wv, gate, out=None,
                       sel_idx=None, ws=None, stream=None):
    """The prefill branches selected by `stages` (STAGE_* bits), same kernels as nsa_prefill.
    With STAGE_SELECTED but not STAGE_CMP_SELECT, sel_idx is the input selection.  wk, wv may be
    None without STAGE_CMP_SELECT.  Returns (out, sel_idx)."""
    torch = _torch()
    lib = load_library()
    c = cfg.c()
    B, T, Hkv, Hq, D = cfg.B, cfg.T, cfg.Hkv, cfg.Hq, cfg.D
    dev = q.device
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    if sel_idx is None and stages & STAGE_CMP_SELECT:
        sel_idx = torch.empty((B, T, Hkv, cfg.top_n), dtype=torch.int32, device=dev)
    ws = _workspace(lib.nsa_prefill_workspace_bytes(ctypes.byref(c)), dev, ws)
    bt = _bf16_types()
    st = lib.nsa_prefill_stages(
        ctypes.byref(c), int(stages), _dev(q, "q", bt, (B, T, Hq, D)),
        _dev(k, "k", bt, (B, Hkv, T, D)), _dev(v, "v", bt, (B, Hkv, T, D)),
        None if wk is None else _dev(wk, "wk", bt, (cfg.cmp_len, D, D)),
        None if wv is None else _dev(wv, "wv", bt, (cfg.cmp_len, D, D)),
        _dev(gate, "gate", (torch.float32,), (B, T, Hq, 3)),
        _dev(out, "out", (torch.float32,), (B, T, Hq, D)),
        None if sel_idx is None else _dev(sel_idx, "sel_idx", (torch.int32,), (B, T, Hkv, cfg.top_n)),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream))
    _check(st, "nsa_prefill_stages")
    return out, sel_idx


DECODE_STAGES = ("cmp_stream", "select", "tiles", "merge")


def nsa_decode(cfg: NsaConfig, q, kcache, vcache, kcmp, vcmp, seqlens, gate, out=None,
               sel_idx=None, ws=None, want_idx=True, stream=None, events=None):
    """cfg.T is the cache capacity; kcmp is [B,Hkv,ncmp,D] (nsa_compress), vcmp is
    [B,Hkv,ncmp_tiles,D,64] (nsa_compress_tiles).  Returns (out fp32 [B,Hq,D], sel_idx
    [B,Hkv,top_n]).
    events: optional ctypes array of len(DECODE_STAGES) + 1 hipEvent_t (nsa_decode_timed)."""
    torch = _torch()
    lib = load_library()
    c = cfg.c()
    B, L, Hkv, Hq, D = cfg.B, cfg.T, cfg.Hkv, cfg.Hq, cfg.D
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    if want_idx and sel_idx is None:
        sel_idx = torch.empty((B, Hkv, cfg.top_n), dtype=torch.int32, device=dev)
    ws = _workspace(lib.nsa_decode_workspace_bytes(ctypes.byref(c)), dev, ws)
    bt = _bf16_types()
    fn = lib.nsa_decode if events is None else lib.nsa_decode_timed
    extra = () if events is None else (ctypes.cast(events, ctypes.c_void_p),)
    st = fn(
        ctypes.byref(c), _dev(q, "q", bt, (B, Hq, D)), _dev(kcache, "kcache", bt, (B, Hkv, L, D)),
        _dev(vcache, "vcache", bt, (B, Hkv, L, D)), _dev(kcmp, "kcmp", bt, (B, Hkv, cfg.ncmp, D)),
        _dev(vcmp, "vcmp", bt, (B, Hkv, cfg.ncmp_tiles, D, 64)),
        _dev(seqlens, "seqlens", (torch.int32,), (B,)),
        _dev(gate, "gate", (torch.float32,), (B, Hq, 3)),
        _dev(out, "out", (torch.float32,), (B, Hq, D)),
        None if sel_idx is None else _dev(sel_idx, "sel_idx", (torch.int32,), (B, Hkv, cfg.top_n)),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream), *extra)
    _check(st, "nsa_decode")
    return out, sel_idx


def nsa_decode_noalloc(cfg: NsaConfig, q, kcache, vcache, kcmp, vcmp, seqlens, gate, out,
                       sel_idx=None, stream=None):
    """nsa_decode on the library's static per-GPU workspace (no workspace argument; neither the
    library nor this binding allocates).  out (fp32 [B,Hq,D]) must be given; sel_idx
    ([B,Hkv,top_n] int32) is optional.  Returns (out, sel_idx)."""
    torch = _torch()
    lib = load_library()
    c = cfg.c()
    B, L, Hkv, Hq, D = cfg.B, cfg.T, cfg.Hkv, cfg.Hq, cfg.D
    bt = _bf16_types()
    st = lib.nsa_decode_noalloc(
        ctypes.byref(c), _dev(q, "q", bt, (B, Hq, D)), _dev(kcache, "kcache", bt, (B, Hkv, L, D)),
        _dev(vcache, "vcache", bt, (B, Hkv, L, D)), _dev(kcmp, "kcmp", bt, (B, Hkv, cfg.ncmp, D)),
        _dev(vcmp, "vcmp", bt, (B, Hkv, cfg.ncmp_tiles, D, 64)),
        _dev(seqlens, "seqlens", (torch.int32,), (B,)),
        _dev(gate, "gate", (torch.float32,), (B, Hq, 3)),
        _dev(out, "out", (torch.float32,), (B, Hq, D)),
        None if sel_idx is None else _dev(sel_idx, "sel_idx", (torch.int32,), (B, Hkv, cfg.top_n)),
        _stream(stream))
    _check(st, "nsa_decode_noalloc")
    return out, sel_idx


def decode_noalloc_max_bytes() -> int:
    return int(load_library().nsa_decode_noalloc_max_bytes())


def nsa_cache_append(cfg: NsaConfig, k_new, v_new, seqlens, wk, wv, kcache, vcache, kcmp,
                     vcmp, ws=None, stream=None):
    """Append k_new/v_new [B,Hkv,C,D] at positions seqlens[b] .. seqlens[b]+C-1 (seqlens: the
    lengths BEFORE the append, not updated) and emit the compressed tokens they complete into
    kcmp [B,Hkv,ncmp,D] and vcmp [B,Hkv,ncmp_tiles,D,64].  cfg.T is the cache capacity."""
    torch = _torch()
    lib = load_library()
    c = cfg.c()
    B, L, Hkv, D = cfg.B, cfg.T, cfg.Hkv, cfg.D
    if k_new.dim() != 4:
        raise ValueError("k_new must be [B, Hkv, C, D]")
    C = int(k_new.shape[2])
    bt = _bf16_types()
    ws = _workspace(lib.nsa_cache_append_workspace_bytes(ctypes.byref(c)), k_new.device, ws)
    st = lib.nsa_cache_append(
        ctypes.byref(c), C, _dev(k_new, "k_new", bt, (B, Hkv, C, D)),
        _dev(v_new, "v_new", bt, (B, Hkv, C, D)), _dev(seqlens, "seqlens", (torch.int32,), (B,)),
        _dev(wk, "wk", bt, (cfg.cmp_len, D, D)), _dev(wv, "wv", bt, (cfg.cmp_len, D, D)),
        _dev(kcache, "kcache", bt, (B, Hkv, L, D)), _dev(vcache, "vcache", bt, (B, Hkv, L, D)),
        _dev(kcmp, "kcmp", bt, (B, Hkv, cfg.ncmp, D)),
        _dev(vcmp, "vcmp", bt, (B, Hkv, cfg.ncmp_tiles, D, 64)),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream))
    _check(st, "nsa_cache_append")


def nsa_prefill_chunk(cfg: NsaConfig, P: int, q, kcache, vcache, kcmp, vcmp, gate, out=None,
                      sel_idx=None, ws=None, want_idx=True, stream=None):
    """Query positions P .. P+C-1 (C = q.shape[1]) against the caches (cfg.T = capacity).
    Returns (out fp32 [B,C,Hq,D], sel_idx int32 [B,C,Hkv,top_n])."""
    torch = _torch()
    lib = load_library()
    c = cfg.c()
    B, L, Hkv, Hq, D = cfg.B, cfg.T, cfg.Hkv, cfg.Hq, cfg.D
    if q.dim() != 4:
        raise ValueError("q must be [B, C, Hq, D]")
    C = int(q.shape[1])
    dev = q.device
    if out is None:
        out = torch.empty((B, C, Hq, D), dtype=torch.float32, device=dev)
    if want_idx and sel_idx is None:
        sel_idx = torch.empty((B, C, Hkv, cfg.top_n), dtype=torch.int32, device=dev)
    ws = _workspace(lib.nsa_prefill_chunk_workspace_bytes(ctypes.byref(c)), dev, ws)
    bt = _bf16_types()
    st = lib.nsa_prefill_chunk(
        ctypes.byref(c), int(P), C, _dev(q, "q", bt, (B, C, Hq, D)),
        _dev(kcache, "kcache", bt, (B, Hkv, L, D)), _dev(vcache, "vcache", bt, (B, Hkv, L, D)),
        _dev(kcmp, "kcmp", bt, (B, Hkv, cfg.ncmp, D)),
        _dev(vcmp, "vcmp", bt, (B, Hkv, cfg.ncmp_tiles, D, 64)),
        _dev(gate, "gate", (torch.float32,), (B, C, Hq, 3)),
        _dev(out, "out", (torch.float32,), (B, C, Hq, D)),
        None if sel_idx is None else _dev(sel_idx, "sel_idx", (torch.int32,),
                                          (B, C, Hkv, cfg.top_n)),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream))
    _check(st, "nsa_prefill_chunk")
    return out, sel_idx


BACKWARD_STAGES = ("layout", "prep", "query_major", "key_major", "compressor")


def backward_workspace_bytes(cfg: NsaConfig) -> int:
    return load_library().nsa_backward_workspace_bytes(ctypes.byref(cfg.c()))


def nsa_backward(cfg: NsaConfig, q, k, v, wk, wv, gate, sel_idx, dout, grads=None, ws=None,
                 stream=None, events=None):
    """Gradients of sum(dout * nsa_prefill(...)) with the selection sel_idx held fixed.
    Returns dict(dq, dk, dv, dwk, dwv, dgate) (fp32; `grads` may supply the tensors).
    events: optional ctypes array of len(BACKWARD_STAGES) + 1 hipEvent_t."""
    torch = _torch()
    lib = load_library()
    c = cfg.c()
    B, T, Hkv, Hq, D, l = cfg.B, cfg.T, cfg.Hkv, cfg.Hq, cfg.D, cfg.cmp_len
    dev = q.device
    shapes = dict(dq=(B, T, Hq, D), dk=(B, Hkv, T, D), dv=(B, Hkv, T, D), dwk=(l, D, D),
                  dwv=(l, D, D), dgate=(B, T, Hq, 3))
    if grads is None:
        grads = {n: torch.empty(s, dtype=torch.float32, device=dev) for n, s in shapes.items()}
    ws = _workspace(lib.nsa_backward_workspace_bytes(ctypes.byref(c)), dev, ws)
    bt = _bf16_types()
    f32 = (torch.float32,)
    fn = lib.nsa_backward if events is None else lib.nsa_backward_timed
    extra = () if events is None else (ctypes.cast(events, ctypes.c_void_p),)
    st = fn(
        ctypes.byref(c), _dev(q, "q", bt, (B, T, Hq, D)), _dev(k, "k", bt, (B, Hkv, T, D)),
        _dev(v, "v", bt, (B, Hkv, T, D)), _dev(wk, "wk", bt, (l, D, D)),
        _dev(wv, "wv", bt, (l, D, D)), _dev(gate, "gate", f32, (B, T, Hq, 3)),
        _dev(sel_idx, "sel_idx", (torch.int32,), (B, T, Hkv, cfg.top_n)),
        _dev(dout, "dout", f32, (B, T, Hq, D)),
        *[_dev(grads[n], n, f32, shapes[n]) for n in ("dq", "dk", "dv", "dwk", "dwv", "dgate")],
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream), *extra)
    _check(st, "nsa_backward")
    return grads


MOBA_STAGES = ("pool_gate", "lists", "block_attn", "own_merge")


def moba_prefill(cfg: MobaConfig, q, k, v, out=None, sel_idx=None, ws=None, want_idx=True,
                 stream=None, events=None):
    """Returns (out fp32 [B,T,H,D], sel_idx int32 [B,T,H,top_k+1]).
    events: optional ctypes array of len(MOBA_STAGES) + 1 hipEvent_t (moba_prefill_timed)."""
    torch = _torch()
    lib = load_library()
    c = cfg.c()
    B, T, H, D = cfg.B, cfg.T, cfg.H, cfg.D
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, D), dtype=torch.float32, device=dev)
    if want_idx and sel_idx is None:
        sel_idx = torch.empty((B, T, H, cfg.top_k + 1), dtype=torch.int32, device=dev)
    ws = _workspace(lib.moba_prefill_workspace_bytes(ctypes.byref(c)), dev, ws)
    bt = _bf16_types()
    fn = lib.moba_prefill if events is None else lib.moba_prefill_timed
    extra = () if events is None else (ctypes.cast(events, ctypes.c_void_p),)
    st = fn(
        ctypes.byref(c), _dev(q, "q", bt, (B, T, H, D)), _dev(k, "k", bt, (B, H, T, D)),
        _dev(v, "v", bt, (B, H, T, D)), _dev(out, "out", (torch.float32,), (B, T, H, D)),
        None if sel_idx is None else _dev(sel_idx, "sel_idx", (torch.int32,), (B, T, H, cfg.top_k + 1)),
        ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream), *extra)
    _check(st, "moba_prefill")
    return out, sel_idx
