"""ctypes front end of the fp64 CPU oracle (nsa_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the CPU-baseline leg of
bench.py.  The product path never imports this package.  The oracle shares no code with the
GPU library; its only common ground with the GPU side is the seeded input generator.

Arrays in and out are numpy: bf16 tensors are uint16 bit patterns, gates fp32, results fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "nsa_oracle.c")
_LIB = os.path.join(_DIR, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile nsa_oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-D_DEFAULT_SOURCE", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _NsaCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "T", "Hkv", "G", "D", "cmp_len", "cmp_stride",
                                             "sel_block", "top_n", "n_local", "window")] + \
               [("scale", ctypes.c_double), ("top_p", ctypes.c_double)]


class _MobaCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "T", "H", "D", "block", "top_k")] + \
               [("scale", ctypes.c_double)]


def _load():
    global _lib
    if _lib is None:
        alt = os.environ.get("NSA_ORACLE_LIB")  # another build of nsa_oracle.c (sanitizer runs)
        if alt:
            _lib = ctypes.CDLL(alt)
        else:
            build(force=False)
            _lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        _lib.onsa_compress.argtypes = [ctypes.c_int] * 6 + [P, P, P, P]
        _lib.onsa_compress.restype = None
        _lib.onsa_prefill_rows.argtypes = [P] * 7 + [ctypes.c_int] + [P] * 11
        _lib.onsa_prefill_rows.restype = ctypes.c_int
        _lib.onsa_decode.argtypes = [P] * 17
        _lib.onsa_decode.restype = ctypes.c_int
        _lib.omoba_pool.argtypes = [P, P, P]
        _lib.omoba_pool.restype = None
        _lib.omoba_prefill_rows.argtypes = [P] * 5 + [ctypes.c_int] + [P] * 7
        _lib.omoba_prefill_rows.restype = ctypes.c_int
        _lib.onsa_threads.argtypes = []
        _lib.onsa_threads.restype = ctypes.c_int
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops run on."""
    return int(_load().onsa_threads())


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def n_cmp(T, l, d):
    return (T - l) // d + 1 if T >= l else 0


class NsaCfg:
    """Hyper-parameters of one NSA layer call (notation of the pages: block 64, top-16 ...)."""

    def __init__(self, B, T, Hkv, G, D, cmp_len=32, cmp_stride=16, sel_block=64, top_n=16,
                 n_local=2, window=512, scale=None, top_p=0.0):
        self.B, self.T, self.Hkv, self.G, self.D = B, T, Hkv, G, D
        self.cmp_len, self.cmp_stride = cmp_len, cmp_stride
        self.sel_block, self.top_n, self.n_local, self.window = sel_block, top_n, n_local, window
        self.scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
        self.top_p = float(top_p)  # 0: fixed top_n; in (0, 1]: adaptive cut (R9)

    @property
    def Hq(self):
        return self.Hkv * self.G

    @property
    def ncmp(self):
        return n_cmp(self.T, self.cmp_len, self.cmp_stride)

    @property
    def nblk(self):
        return -(-self.T // self.sel_block)

    def c(self):
        return _NsaCfg(self.B, self.T, self.Hkv, self.G, self.D, self.cmp_len, self.cmp_stride,
                       self.sel_block, self.top_n, self.n_local, self.window, self.scale,
                       self.top_p)


class MobaCfg:
    def __init__(self, B, T, H, D, block=512, top_k=3, scale=None):
        self.B, self.T, self.H, self.D, self.block, self.top_k = B, T, H, D, block, top_k
        self.scale = 1.0 / np.sqrt(D) if scale is None else float(scale)

    @property
    def nblk(self):
        return self.T // self.block

    def c(self):
        return _MobaCfg(self.B, self.T, self.H, self.D, self.block, self.top_k, self.scale)


def compress(x, w, l, d, exact=False):
    """x: bf16 bits [B, H, T, D]; w: [l, D, D].  Returns bf16 bits [B, H, n_cmp, D]
    (and the unrounded fp64 values when exact=True)."""
    lib = _load()
    x = _u16(x)
    w = _u16(w)
    B, H, T, D = x.shape
    n = n_cmp(T, l, d)
    bits = np.empty((B, H, n, D), dtype=np.uint16)
    ex = np.empty((B, H, n, D), dtype=np.float64) if exact else None
    lib.onsa_compress(B, H, T, D, l, d, _p(x), _p(w), _p(bits), _p(ex))
    return (bits, ex) if exact else bits


def nsa_prefill_rows(cfg: NsaCfg, q, k, v, kc, vc, gate, rows_b, rows_t, idx_in=None,
                     branches=False, want_scores=False):
    """Oracle NSA prefill at query positions (rows_b[r], rows_t[r]).  Returns a dict with
    out [R,Hq,D], idx [R,Hkv,n], gap [R,Hkv] and, on request, o_cmp/o_slc/o_win/lse/scores."""
    lib = _load()
    rb = np.ascontiguousarray(rows_b, dtype=np.int32)
    rt = np.ascontiguousarray(rows_t, dtype=np.int32)
    R = len(rb)
    Hq, D, n = cfg.Hq, cfg.D, cfg.top_n
    res = dict(out=np.empty((R, Hq, D)), idx=np.empty((R, cfg.Hkv, n), dtype=np.int32),
               gap=np.empty((R, cfg.Hkv)))
    if branches:
        for nm in ("o_cmp", "o_slc", "o_win"):
            res[nm] = np.empty((R, Hq, D))
        res["lse"] = np.empty((R, Hq))
    if want_scores:
        res["scores"] = np.empty((R, cfg.Hkv, cfg.nblk))
    ii = None if idx_in is None else np.ascontiguousarray(idx_in, dtype=np.int32)
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    rc = lib.onsa_prefill_rows(ctypes.byref(cfg.c()), _p(_u16(q)), _p(_u16(k)), _p(_u16(v)),
                               _p(_u16(kc)), _p(_u16(vc)), _p(gate), R, _p(rb), _p(rt), _p(ii),
                               _p(res["out"]), _p(res.get("o_cmp")), _p(res.get("o_slc")),
                               _p(res.get("o_win")), _p(res.get("lse")), _p(res.get("scores")),
                               _p(res["idx"]), _p(res["gap"]))
    if rc != 0:
        raise ValueError("oracle: row out of range")
    return res


def nsa_decode(cfg: NsaCfg, q, kcache, vcache, kc, vc, seqlens, gate, idx_in=None,
               branches=False, want_scores=False):
    """Oracle NSA decode; cfg.T is the cache capacity.  One row per sequence."""
    lib = _load()
    B, Hq, D, n = cfg.B, cfg.Hq, cfg.D, cfg.top_n
    res = dict(out=np.empty((B, Hq, D)), idx=np.empty((B, cfg.Hkv, n), dtype=np.int32),
               gap=np.empty((B, cfg.Hkv)))
    if branches:
        for nm in ("o_cmp", "o_slc", "o_win"):
            res[nm] = np.empty((B, Hq, D))
        res["lse"] = np.empty((B, Hq))
    if want_scores:
        res["scores"] = np.empty((B, cfg.Hkv, cfg.nblk))
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    ii = None if idx_in is None else np.ascontiguousarray(idx_in, dtype=np.int32)
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    rc = lib.onsa_decode(ctypes.byref(cfg.c()), _p(_u16(q)), _p(_u16(kcache)), _p(_u16(vcache)),
                         _p(_u16(kc)), _p(_u16(vc)), _p(sl), _p(gate), _p(ii), _p(res["out"]),
                         _p(res.get("o_cmp")), _p(res.get("o_slc")), _p(res.get("o_win")),
                         _p(res.get("lse")), _p(res.get("scores")), _p(res["idx"]),
                         _p(res["gap"]))
    if rc != 0:
        raise ValueError("oracle: bad seqlens")
    return res


def moba_pool(cfg: MobaCfg, k):
    lib = _load()
    kbar = np.empty((cfg.B, cfg.H, cfg.nblk, cfg.D))
    lib.omoba_pool(ctypes.byref(cfg.c()), _p(_u16(k)), _p(kbar))
    return kbar


def moba_prefill_rows(cfg: MobaCfg, q, k, v, rows_b, rows_t, kbar=None, idx_in=None,
                      want_scores=False):
    """Oracle MoBA prefill at the given query positions.  Returns out [R,H,D],
    idx [R,H,top_k+1] (own block included), gap [R,H] and optionally scores [R,H,T/block]."""
    lib = _load()
    if kbar is None:
        kbar = moba_pool(cfg, k)
    rb = np.ascontiguousarray(rows_b, dtype=np.int32)
    rt = np.ascontiguousarray(rows_t, dtype=np.int32)
    R = len(rb)
    kk = cfg.top_k + 1
    res = dict(out=np.empty((R, cfg.H, cfg.D)), idx=np.empty((R, cfg.H, kk), dtype=np.int32),
               gap=np.empty((R, cfg.H)))
    if want_scores:
        res["scores"] = np.empty((R, cfg.H, cfg.nblk))
    ii = None if idx_in is None else np.ascontiguousarray(idx_in, dtype=np.int32)
    rc = lib.omoba_prefill_rows(ctypes.byref(cfg.c()), _p(_u16(q)), _p(_u16(k)), _p(_u16(v)),
                                _p(np.ascontiguousarray(kbar, dtype=np.float64)), R, _p(rb),
                                _p(rt), _p(ii), _p(res["out"]), _p(res["idx"]),
                                _p(res.get("scores")), _p(res["gap"]))
    if rc != 0:
        raise ValueError("oracle: row out of range")
    return res
