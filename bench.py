#!/usr/bin/env python3
"""Benchmark of the NSA forward hot path on one MI355X.

Headline workload: NSA prefill, B=1, T=65536, 4 KV heads x group 16 (64 query heads),
head_dim 128, compression l=32 / d=16, selection block 64, top-16 (block 0 + 2 local blocks
forced), window 512; bf16 inputs ~ N(0,1), random compressor weights and gates (seeded,
synthetic).  One step = one nsa_prefill call over the whole sequence (every stage: layout,
compression, compressed attention + importance + selection, window, selected blocks, gate).

Prints ONE JSON line.  `value` = prefill tokens/s; `roofline` = the dominant kernel's
algorithmic TFLOP/s against the bf16 MFMA peak, measured with HIP events recorded around each
stage on the stream the kernels run on; `cpu_baseline` = the fp64 oracle timed on a bounded,
stratified sample of the same workload on this host.  Decode and MoBA workloads are reported in
extra fields when their entry points are available.
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NSA prefill tok/s @64k (MFMA % peak); decode tok/s + KV GB/s @64k (HBM % peak)"
MFMA_PEAK_BF16 = 2.5e15   # dense bf16 matrix peak, FLOP/s
HBM_PEAK = 8.0e12         # bytes/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "dynamic_block_sparse_fwd_amd", "csrc")
# the sources a kernel's code object depends on (its translation unit, shared headers, flags)
_HDRS = ["attn_tile.h", "dev_common.h", "kernels.h", "../build.py"]
KERNEL_SOURCES = {
    "cmp_select_kernel": ["prefill.hip"] + _HDRS,
    "slc_block_kernel": ["selected.hip"] + _HDRS,
    "selected_kernel": ["selected.hip"] + _HDRS,
    "dec_cmp_kernel": ["decode.hip"] + _HDRS,
    "moba_block_kernel": ["moba.hip"] + _HDRS,
    "moba_own_kernel": ["moba.hip"] + _HDRS,
}


def source_digest(kernel):
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each divided by what the same counter reads per byte of a
    plain copy of known size.  None when there is no summary or the kernel's sources changed
    since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        k = tr["kernels"][kernel]
        cal = tr["copy_calibration"]
    except (OSError, KeyError, ValueError):
        return None
    if k.get("source_sha256") != source_digest(kernel):
        return None
    fetch = k["fetch_kib_per_dispatch"] * 1024.0 / cal["fetch_counter_bytes_per_byte"]
    write = k["write_kib_per_dispatch"] * 1024.0 / cal["write_counter_bytes_per_byte"]
    return int(round(fetch + write))


def copy_calibration():
    """A plain device copy of known size (256 MiB read + 256 MiB written per dispatch, three
    dispatches) for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    x = torch.ones(1 << 26, dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_dispatch": x.numel() * 4}), flush=True)


# ----------------------------------------------------------------------------- HIP events

class HipEvents:
    def __init__(self, n):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            rc = self.lib.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError("hipEventCreate failed (%d)" % rc)
            self.ev[i] = h

    def record(self, i, stream):
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        rc = self.lib.hipEventRecord(self.ev[i], stream)
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def group(self, start, count):
        return ctypes.cast(ctypes.byref(self.ev, start * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.POINTER(ctypes.c_void_p))

    def elapsed_ms(self, i, j):
        self.lib.hipEventSynchronize(self.ev[j])
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value


# ----------------------------------------------------------------------------- work counts

def selected_traffic(stage_ms):
    """HBM bytes of the selected stage's two heavy launches (block-major tiles and the merge)
    from the committed counters, over the stage's time: the bound of the block-major design,
    whose q reads and partials are traffic of the design rather than of the method.  None while
    the counters are stale."""
    t1, t2 = measured_traffic("slc_block_kernel"), measured_traffic("selected_kernel")
    if t1 is None or t2 is None or stage_ms <= 0:
        return {"bytes": None, "gbs": None, "hbm_frac": None}
    gbs = (t1 + t2) / (stage_ms * 1e-3)
    return {"bytes": t1 + t2, "gbs": round(gbs / 1e9, 1), "hbm_frac": round(gbs / HBM_PEAK, 4),
            "kernels": ["slc_block_kernel", "selected_kernel"]}


def prefill_pairs(T, l=32, d=16, beta=64, n=16, n_local=2, w=512):
    """Query-key pairs per head performed by each branch (the method's algorithmic work)."""
    t = np.arange(T, dtype=np.int64)
    ncmp = (T - l) // d + 1 if T >= l else 0
    vis = np.where(t >= l - 1, np.minimum((t - l + 1) // d + 1, ncmp), 0)
    b = t // beta
    slc = np.where(b + 1 <= n, t + 1, (n - 1) * beta + (t - b * beta + 1))
    win = np.minimum(t + 1, w)
    return int(vis.sum()), int(slc.sum()), int(win.sum())


def selected_keys(idx, beta=64):
    """Causal keys of the selected blocks, summed over (sequence, position, KV group), from a
    prefill index tensor [B, T, Hkv, n] (-1 = unused)."""
    import torch

    T = idx.shape[1]
    t = torch.arange(T, device=idx.device).view(1, T, 1, 1)
    k = (t + 1 - idx.long() * beta).clamp(0, beta)
    return int(torch.where(idx >= 0, k, torch.zeros_like(k)).sum())


def prefill_flops(B, T, Hkv, G, D, l=32, d=16, slc_keys=None):
    """slc_keys: selected keys summed over (sequence, position, KV group) when the selection
    is adaptive; None = the fixed top-16 count."""
    cmp_, slc, win = prefill_pairs(T, l, d)
    if slc_keys is not None:
        slc = slc_keys / (B * Hkv)
    Hq = Hkv * G
    ncmp = (T - l) // d + 1
    per = {
        "compress": 2.0 * 2 * ncmp * l * D * D * Hkv * B,
        "cmp_select": 4.0 * D * Hq * cmp_ * B,
        "window": 4.0 * D * Hq * win * B,
        "selected": 4.0 * D * Hq * slc * B,
        "layout": 0.0,
    }
    return per


def cmp_select_performed_flops(B, T, Hkv, G, D, l=32, d=16, window=512):
    """Matrix-core FLOPs the compressed-attention kernel issues (fused window, G = 16: query
    tiles of 8 positions x 16 heads): per tile, two score passes and one P V product over the
    64-key tiles of the compressed tokens the tile's last position sees, and score + P V over
    the 64-key tiles that cover the tile's windows.  Masked keys inside a tile count: the
    matrix core computes them."""
    TQ = 8
    rows = TQ * G
    ncmp = (T - l) // d + 1 if T >= l else 0
    t0 = np.arange(0, T, TQ, dtype=np.int64)
    tl = np.minimum(t0 + TQ - 1, T - 1)
    nvis = np.where(tl >= l - 1, np.minimum((tl - l) // d + 1, ncmp), 0)
    nkt = (nvis + 63) // 64
    kw0 = np.maximum(t0 - window + 1, 0) // 64
    nwt = tl // 64 - kw0 + 1
    tile = 2.0 * rows * 64 * D  # one 64-key product of the tile's rows
    return float(B * Hkv * tile * (3 * nkt + 2 * nwt).sum())


# ----------------------------------------------------------------------------- prefill

def bench_prefill(args):
    import torch

    import dynamic_block_sparse_fwd_amd as nsa
    import synth_inputs as S

    nsa.load_library()
    B, T, Hkv, G, D = 1, args.seq, 4, 16, 128
    cfg = nsa.NsaConfig(B, T, Hkv, G, D, top_p=args.top_p)
    t0 = time.time()
    x = S.nsa_prefill_inputs(2, B, T, Hkv, G, D)
    print("[bench] prefill inputs generated in %.1fs" % (time.time() - t0), file=sys.stderr,
          flush=True)
    dev = torch.device("cuda:0")
    d = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).to(dev)
         for k, v in x.items()}
    out = torch.empty((B, T, Hkv * G, D), dtype=torch.float32, device=dev)
    idx = torch.empty((B, T, Hkv, cfg.top_n), dtype=torch.int32, device=dev)
    ws = torch.empty(nsa.prefill_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    nst = len(nsa.PREFILL_STAGES)

    def step(events=None):
        nsa.nsa_prefill(cfg, d["q"], d["k"], d["v"], d["wk"], d["wv"], d["gate"], out=out,
                        sel_idx=idx, ws=ws, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: the production call, bracketed by device synchronisations
    t_start = time.perf_counter()
    for s in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    # per-stage times from the instrumented call (the same kernels, events between them)
    ev = HipEvents(args.steps * (nst + 1))
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(ev.group(s * (nst + 1), nst + 1))
    torch.cuda.synchronize()
    stage_ms = {nm: 0.0 for nm in nsa.PREFILL_STAGES}
    total_ev = 0.0
    for s in range(args.steps):
        base = s * (nst + 1)
        for i, nm in enumerate(nsa.PREFILL_STAGES):
            stage_ms[nm] += ev.elapsed_ms(base + i, base + i + 1) / args.steps
        total_ev += ev.elapsed_ms(base, base + nst) / args.steps
    ms = wall * 1e3 / args.steps
    slc_keys = selected_keys(idx) if args.top_p > 0 else None
    blocks_per_row = float((idx >= 0).sum(-1).float().mean())
    flops = prefill_flops(B, T, Hkv, G, D, slc_keys=slc_keys)
    F = sum(flops.values())
    # nsa_prefill runs the window branch inside the compressed-attention kernel (same query
    # tile, output written once): its stage interval is empty and its work counts there
    flops["cmp_select"] += flops["window"]
    flops["window"] = 0.0
    dom = max(stage_ms, key=lambda k: stage_ms[k])
    stages = {nm: {"ms": round(stage_ms[nm], 4),
                   "tflops": round(flops[nm] / (stage_ms[nm] * 1e-3) / 1e12, 2)
                   if flops.get(nm, 0) > 0 and stage_ms[nm] > 0 else None}
              for nm in nsa.PREFILL_STAGES}
    stages["window"]["fused_into"] = "cmp_select"
    res = dict(
        ms_per_step=ms, events_ms_per_step=total_ev, tok_s=B * T / (ms * 1e-3),
        algorithmic_tflop=F / 1e12, mfma_frac=F / (ms * 1e-3) / MFMA_PEAK_BF16, stages=stages,
        # the dominant single kernel: the compressed-attention kernel (with the fused window and
        # the selection) is one launch; the selected stage is five (lists, block-major tiles,
        # merge), each shorter
        roofline={"bound": "mfma", "kernel": "cmp_select_kernel",
                  "achieved": flops["cmp_select"] / (stage_ms["cmp_select"] * 1e-3) / 1e12,
                  "peak": MFMA_PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                  "frac": flops["cmp_select"] / (stage_ms["cmp_select"] * 1e-3) / MFMA_PEAK_BF16,
                  "traffic": measured_traffic("cmp_select_kernel")},
        longest_stage=dom,
        cmp_select_performed={
            "tflop": cmp_select_performed_flops(B, T, Hkv, G, D) / 1e12,
            "mfma_frac": cmp_select_performed_flops(B, T, Hkv, G, D)
                         / (stage_ms["cmp_select"] * 1e-3) / MFMA_PEAK_BF16},
        # the selected branch is bound by HBM: its counted bytes over the stage's time
        selected_traffic=selected_traffic(stage_ms["selected"]),
        blocks_per_row=blocks_per_row,
    )
    del d, out, idx, ws
    torch.cuda.empty_cache()
    return res, x


def cpu_baseline_prefill(x, T, rows=1024):
    """fp64 oracle on a stratified sample: full compression + `rows` evenly spaced positions
    (all heads), scaled to the whole sequence."""
    import oracle as O

    cfg = O.NsaCfg(1, T, 4, 16, 128)
    t0 = time.perf_counter()
    kc = O.compress(x["k"], x["wk"], 32, 16)
    vc = O.compress(x["v"], x["wv"], 32, 16)
    t_cmp = time.perf_counter() - t0
    step = max(1, T // rows)
    rt = np.arange(step // 2, T, step, dtype=np.int32)
    rb = np.zeros_like(rt)
    t0 = time.perf_counter()
    O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], rb, rt)
    t_rows = time.perf_counter() - t0
    est = t_cmp + t_rows * T / len(rt)
    return {"value": T / est, "unit": "tok/s", "cores": O.threads(), "kind": "oracle",
            "sample": "fp64 oracle: full K/V compression (%.1fs) + %d positions every %d-th of "
                      "the 64k prefill, all 64 heads (%.1fs), scaled to 65536 positions"
                      % (t_cmp, len(rt), step, t_rows)}


# ----------------------------------------------------------------------------- decode

def decode_kv_bytes(idx, seqlens, L, D, l=32, d=16, beta=64, w=512, n_local=2, fixed=False):
    """Unique K+V bytes one decode step must read: every visible compressed token, and the
    union of the selected blocks' and the window's tokens (causal), per (sequence, KV group).
    fixed=True also returns the bytes of the window's and the forced blocks' tokens (block 0 and
    the n_local most recent), which do not depend on the selection."""
    B, Hkv, _ = idx.shape
    cmp_b = 0
    tok_b = 0
    fix_b = 0
    for b in range(B):
        t = int(seqlens[b]) - 1
        nvis = (t - l + 1) // d + 1 if t >= l - 1 else 0
        bcur = t // beta
        for h in range(Hkv):
            toks = set(range(max(0, t - w + 1), t + 1))
            for j in {0} | set(range(max(0, bcur - n_local + 1), bcur + 1)):
                toks.update(range(j * beta, min((j + 1) * beta, t + 1)))
            fix_b += len(toks)
            for j in idx[b, h]:
                if j >= 0:
                    toks.update(range(j * beta, min((j + 1) * beta, t + 1)))
            tok_b += len(toks)
            cmp_b += nvis
    per_tok = 2 * D * 2  # K and V, bf16
    if fixed:
        return cmp_b * per_tok, tok_b * per_tok, fix_b * per_tok
    return cmp_b * per_tok, tok_b * per_tok


def time_decode(nsa, cfg, d, kc, vc, out, idx, ws, calls, flush):
    """Median per-call time of nsa_decode (ms) with one event pair around each call, and the
    median of each stage from the instrumented twin; 1 GiB is READ between calls to evict the
    256 MB Infinity Cache (a write sweep would leave dirty lines whose write-back competes with
    the call)."""
    nst = len(nsa.DECODE_STAGES)

    def call(events=None):
        nsa.nsa_decode(cfg, d["q"], d["kcache"], d["vcache"], kc, vc, d["seqlens"], d["gate"],
                       out=out, sel_idx=idx, ws=ws, events=events)

    for _ in range(3):
        call()
    import torch
    ev = HipEvents(calls * (nst + 1))
    torch.cuda.synchronize()
    for c in range(calls):
        flush.sum()
        call(ev.group(c * (nst + 1), nst + 1))
    torch.cuda.synchronize()
    per_call = []
    stage_ms = {nm: [] for nm in nsa.DECODE_STAGES}
    for c in range(calls):
        base = c * (nst + 1)
        per_call.append(ev.elapsed_ms(base, base + nst))
        for i, nm in enumerate(nsa.DECODE_STAGES):
            stage_ms[nm].append(ev.elapsed_ms(base + i, base + i + 1))
    # the whole call without the per-stage events (one event pair around it)
    stream = torch.cuda.current_stream().cuda_stream
    ev2 = HipEvents(2 * calls)
    for c in range(calls):
        flush.sum()
        ev2.record(2 * c, stream)
        call()
        ev2.record(2 * c + 1, stream)
    torch.cuda.synchronize()
    plain = [ev2.elapsed_ms(2 * c, 2 * c + 1) for c in range(calls)]
    med = {nm: float(np.median(v)) for nm, v in stage_ms.items()}
    return float(np.median(plain)), float(np.median(per_call)), med


def decode_result(workload, B, ms, ms_ev, med, idx, seqlens, L, D, calls):
    cmp_bytes, tok_bytes = decode_kv_bytes(idx, seqlens, L, D)
    kv = cmp_bytes + tok_bytes
    first = next(iter(med))  # the compressed-cache stream
    return {
        "workload": workload,
        "blocks_per_row": round(float((idx >= 0).sum(-1).mean()), 3),
        "us_per_step": round(ms * 1e3, 2),
        "us_per_step_with_stage_events": round(ms_ev * 1e3, 2),
        "tok_s": round(B / (ms * 1e-3), 1),
        "kv_bytes": kv,
        "kv_gbs": round(kv / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(kv / (ms * 1e-3) / HBM_PEAK, 4),
        "stages_us": {nm: round(v * 1e3, 2) for nm, v in med.items()},
        # the whole call is the unit of the decode roofline: every kernel streams HBM, and the
        # bytes are the unique K/V the step must read (compressed cache + selected and window
        # tokens), over the call's event-timed duration
        "roofline": {"bound": "hbm", "kernel": "nsa_decode (whole call)",
                     "achieved": round(kv / (ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(kv / (ms * 1e-3) / HBM_PEAK, 4),
                     "traffic": None},
        "compressed_stream": {"bytes": cmp_bytes,
                              "gbs": round(cmp_bytes / (med[first] * 1e-3) / 1e9, 1),
                              "traffic": measured_traffic("dec_cmp_kernel")},
        "timing": "median of %d calls, HIP events around each call, 1 GiB read between "
                  "calls to evict the Infinity Cache" % calls,
    }


def bench_decode(args, B=32, L=65536, Hkv=4, G=16, D=128, seed=3, calls=20):
    import torch

    import dynamic_block_sparse_fwd_amd as nsa
    import synth_inputs as S

    cfg = nsa.NsaConfig(B, L, Hkv, G, D, top_p=args.top_p)
    t0 = time.time()
    x = S.nsa_decode_inputs(seed, B, L, Hkv, G, D)
    print("[bench] decode inputs generated in %.1fs" % (time.time() - t0), file=sys.stderr,
          flush=True)
    dev = torch.device("cuda:0")
    d = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).to(dev)
         for k, v in x.items()}
    kc = nsa.nsa_compress(cfg, d["kcache"], d["wk"])
    vc = nsa.nsa_compress_tiles(cfg, d["vcache"], d["wv"])
    out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, cfg.top_n), dtype=torch.int32, device=dev)
    ws = torch.empty(nsa.decode_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    flush = torch.zeros(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB
    ms, ms_ev, med = time_decode(nsa, cfg, d, kc, vc, out, idx, ws, calls, flush)

    def call():
        nsa.nsa_decode(cfg, d["q"], d["kcache"], d["vcache"], kc, vc, d["seqlens"], d["gate"],
                       out=out, sel_idx=idx, ws=ws)

    stream = torch.cuda.current_stream().cuda_stream
    # a generation step: nsa_cache_append of the newest token (here the last cached one,
    # rewritten with its own values at position L-1, which also completes compressed token
    # n_cmp(L) - 1: the 1-in-16 steps that emit one), then the decode
    k_last = d["kcache"][:, :, L - 1:L].contiguous()
    v_last = d["vcache"][:, :, L - 1:L].contiguous()
    before = (d["seqlens"] - 1).contiguous()
    aws = torch.empty(nsa.cache_append_workspace_bytes(cfg), dtype=torch.uint8, device=dev)

    def app():
        nsa.nsa_cache_append(cfg, k_last, v_last, before, d["wk"], d["wv"], d["kcache"],
                             d["vcache"], kc, vc, ws=aws)

    ev3 = HipEvents(3 * calls)
    for c in range(calls):
        flush.sum()
        ev3.record(3 * c, stream)
        app()
        ev3.record(3 * c + 1, stream)
        call()
        ev3.record(3 * c + 2, stream)
    torch.cuda.synchronize()
    app_ms = float(np.median([ev3.elapsed_ms(3 * c, 3 * c + 1) for c in range(calls)]))
    gen_ms = float(np.median([ev3.elapsed_ms(3 * c, 3 * c + 2) for c in range(calls)]))
    # the other 15 of 16 steps: the token at L-2 (rewritten with its own values) completes no
    # compressed token
    k_prev = d["kcache"][:, :, L - 2:L - 1].contiguous()
    v_prev = d["vcache"][:, :, L - 2:L - 1].contiguous()
    before2 = (d["seqlens"] - 2).contiguous()
    ev4 = HipEvents(2 * calls)
    for c in range(calls):
        flush.sum()
        ev4.record(2 * c, stream)
        nsa.nsa_cache_append(cfg, k_prev, v_prev, before2, d["wk"], d["wv"], d["kcache"],
                             d["vcache"], kc, vc, ws=aws)
        ev4.record(2 * c + 1, stream)
    torch.cuda.synchronize()
    app0_ms = float(np.median([ev4.elapsed_ms(2 * c, 2 * c + 1) for c in range(calls)]))
    res = decode_result("nsa_decode B=%d L=%d Hkv=%d G=%d D=%d top16 window512%s" % (
        B, L, Hkv, G, D, " top_p=%g" % args.top_p if args.top_p > 0 else ""),
        B, ms, ms_ev, med, idx.cpu().numpy(), x["seqlens"], L, D, calls)
    res["append_us"] = round(app_ms * 1e3, 2)
    res["append_us_no_emission"] = round(app0_ms * 1e3, 2)
    res["generation_step_us"] = round(gen_ms * 1e3, 2)
    del d, kc, vc, out, idx, ws, flush, aws
    torch.cuda.empty_cache()
    return res, x


def planted_decode_inputs_device(seed, B, L, Hkv, G, D, n_plant=16, shift=2.0, beta=64):
    """The long-context planted decode inputs drawn on the device (a host draw of 2 x 1G bf16
    values takes about a minute): q, K/V caches ~ N(0,1) bf16 from a seeded torch generator;
    per KV head, n_plant distinct blocks from [1, nblk - 3] (a seeded CPU permutation) whose 64
    keys get + shift * unit(sum of the group's queries), re-rounded to bf16; gates sigmoid(N(0,1)).
    Returns the device tensors and the planted block ids [B, Hkv, n_plant] (sorted)."""
    import torch

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    Hq = Hkv * G
    q = torch.randn((B, Hq, D), generator=g, device=dev).to(torch.bfloat16)
    kc = torch.empty((B, Hkv, L, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    for b in range(B):  # per sequence: bounds the fp32 temporary
        kc[b] = torch.randn((Hkv, L, D), generator=g, device=dev).to(torch.bfloat16)
        vc[b] = torch.randn((Hkv, L, D), generator=g, device=dev).to(torch.bfloat16)
    gate = torch.sigmoid(torch.randn((B, Hq, 3), generator=g, device=dev))
    nblk = L // beta
    gc = torch.Generator()
    gc.manual_seed(seed)
    planted = np.empty((B, Hkv, n_plant), dtype=np.int64)
    dirn = q.float().view(B, Hkv, G, D).sum(2)
    dirn = dirn / dirn.norm(dim=-1, keepdim=True)
    for b in range(B):
        for h in range(Hkv):
            blocks = torch.sort(1 + torch.randperm(nblk - 3, generator=gc)[:n_plant]).values
            planted[b, h] = blocks.numpy()
            rows = (blocks.view(-1, 1) * beta + torch.arange(beta).view(1, -1)).reshape(-1)
            rows = rows.to(dev)
            kc[b, h, rows] = (kc[b, h, rows].float() + shift * dirn[b, h]).to(torch.bfloat16)
    seqlens = torch.full((B,), L, dtype=torch.int32, device=dev)
    return dict(q=q, kcache=kc, vcache=vc, gate=gate, seqlens=seqlens), planted


def bench_decode_planted(args, B=1, L=1 << 20, Hkv=8, G=8, D=128, seed=5, calls=20):
    """Long-context decode with planted structure: batch 1, 1M cached tokens, 8 KV heads x
    group 8, mean-pooled compressor (a random one would hide the plant), top-16, window 512."""
    import torch

    import dynamic_block_sparse_fwd_amd as nsa
    import synth_inputs as S

    cfg = nsa.NsaConfig(B, L, Hkv, G, D, top_p=args.top_p)
    t0 = time.time()
    d, planted = planted_decode_inputs_device(seed, B, L, Hkv, G, D)
    dev = d["q"].device
    mp = torch.from_numpy(S.mean_pool_weights(32, D).view(np.int16)).to(dev)
    kc = nsa.nsa_compress(cfg, d["kcache"], mp)
    vc = nsa.nsa_compress_tiles(cfg, d["vcache"], mp)
    torch.cuda.synchronize()
    print("[bench] planted 1M decode inputs drawn on the device in %.1fs" % (time.time() - t0),
          file=sys.stderr, flush=True)
    out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, cfg.top_n), dtype=torch.int32, device=dev)
    ws = torch.empty(nsa.decode_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    flush = torch.zeros(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB
    ms, ms_ev, med = time_decode(nsa, cfg, d, kc, vc, out, idx, ws, calls, flush)
    gidx = idx.cpu().numpy()
    nblk = L // 64
    hits = total = 0
    for b in range(B):
        for h in range(Hkv):
            free = [int(j) for j in gidx[b, h] if j >= 0 and j not in (0, nblk - 2, nblk - 1)]
            hits += len(set(free) & set(planted[b, h].tolist()))
            total += len(free)
    res = decode_result("nsa_decode planted B=%d L=%d Hkv=%d G=%d D=%d top16 window512, "
                        "mean-pool compressor" % (B, L, Hkv, G, D),
                        B, ms, ms_ev, med, gidx, [L] * B, L, D, calls)
    res["planted_recall"] = round(hits / max(total, 1), 4)
    res["inputs"] = ("q, K/V caches ~ N(0,1) bf16 drawn on the device (seeded torch generator); "
                     "16 planted blocks per KV head shifted +2 sigma toward the group's query "
                     "direction")
    host = None
    if not args.no_cpu_baseline:
        host = {k: v.cpu() for k, v in d.items()}
    del d, kc, vc, out, idx, ws, flush
    torch.cuda.empty_cache()
    return res, host


def cpu_baseline_decode_planted(host, L=1 << 20, Hkv=8, G=8, D=128, reps=3):
    """fp64 oracle decode of the planted 1M-token step on the same inputs (copied from the
    device; the compressed caches built by the oracle's own compression, untimed)."""
    import oracle as O
    import synth_inputs as S

    def bits(t):
        import torch
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
            else t.numpy()

    q, kcache, vcache = bits(host["q"]), bits(host["kcache"]), bits(host["vcache"])
    gate = host["gate"].numpy()
    mp = S.mean_pool_weights(32, D)
    t0 = time.perf_counter()
    kc = O.compress(kcache, mp, 32, 16)
    vc = O.compress(vcache, mp, 32, 16)
    t_cmp = time.perf_counter() - t0
    cfg = O.NsaCfg(1, L, Hkv, G, D)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        O.nsa_decode(cfg, q, kcache, vcache, kc, vc, [L], gate)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return {"value": 1 / dt, "unit": "tok/s", "cores": O.threads(), "kind": "oracle",
            "sample": "fp64 oracle decode of the whole step (batch 1, all 64 heads), median of "
                      "%d runs; its compressed caches built by the oracle's compression first "
                      "(%.1fs, untimed)" % (reps, t_cmp)}


def backward_flops(B, T, Hkv, G, D, l=32, d=16):
    """Algorithmic work of the backward: per (row, key) pair of a branch, the scores, dP, dq, dK
    and dV products (5 x 2 D flop); per compressed token the two products of the compressor
    backward (dX and dW) for K and V."""
    cmp_, slc, win = prefill_pairs(T, l, d)
    ncmp = (T - l) // d + 1
    attn = 10.0 * D * Hkv * G * (cmp_ + slc + win) * B
    comp = 2 * 2 * (2.0 * ncmp * l * D * D * Hkv * B)
    return attn, comp


def bench_backward(args, B=1, Hkv=4, G=16, D=128):
    """nsa_backward at the 64k prefill shape: gradients for q, k, v, the compressor weights
    and the gate, the selection taken from nsa_prefill on the same inputs."""
    import torch

    import dynamic_block_sparse_fwd_amd as nsa
    import synth_inputs as S

    T = args.seq
    cfg = nsa.NsaConfig(B, T, Hkv, G, D)
    x = S.nsa_prefill_inputs(2, B, T, Hkv, G, D)
    dev = torch.device("cuda:0")
    d = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).to(dev)
         for k, v in x.items()}
    del x
    dout = torch.from_numpy(S.upstream_grad(6, (B, T, Hkv * G, D))).to(dev)
    _, idx = nsa.nsa_prefill(cfg, d["q"], d["k"], d["v"], d["wk"], d["wv"], d["gate"])
    ws = torch.empty(nsa.backward_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    grads = None
    nst = len(nsa.BACKWARD_STAGES)

    def step(events=None):
        nonlocal grads
        grads = nsa.nsa_backward(cfg, d["q"], d["k"], d["v"], d["wk"], d["wv"], d["gate"], idx,
                                 dout, grads=grads, ws=ws, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents(args.steps * (nst + 1))
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev.group(s * (nst + 1), nst + 1))
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    stage = {nm: 0.0 for nm in nsa.BACKWARD_STAGES}
    for s in range(args.steps):
        b0 = s * (nst + 1)
        for i, nm in enumerate(nsa.BACKWARD_STAGES):
            stage[nm] += ev.elapsed_ms(b0 + i, b0 + i + 1) / args.steps
    attn, comp = backward_flops(B, T, Hkv, G, D)
    F = attn + comp
    return {
        "workload": "nsa backward B=%d T=%d Hkv=%d G=%d D=%d top16 window512" % (B, T, Hkv, G, D),
        "ms_per_step": round(wall * 1e3, 3),
        "tok_s": round(B * T / wall, 1),
        "algorithmic_tflop": round(F / 1e12, 3),
        "tflops": round(F / wall / 1e12, 1),
        "mfma_frac": round(F / wall / MFMA_PEAK_BF16, 4),
        "stages_ms": {k: round(v, 3) for k, v in stage.items()},
    }


def bench_chunked(args, B=1, Hkv=4, G=16, D=128):
    """The 64k prefill run as a sequence of chunks from the caches: per chunk,
    nsa_cache_append of its K/V (cache rows and the compressed tokens they complete) and
    nsa_prefill_chunk of its query rows."""
    import torch

    import dynamic_block_sparse_fwd_amd as nsa
    import synth_inputs as S

    T, C = args.seq, args.chunk
    cfg = nsa.NsaConfig(B, T, Hkv, G, D, top_p=args.top_p)
    x = S.nsa_prefill_inputs(2, B, T, Hkv, G, D)
    dev = torch.device("cuda:0")
    d = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).to(dev)
         for k, v in x.items()}
    del x
    kcache = torch.zeros((B, Hkv, T, D), dtype=torch.int16, device=dev)
    vcache = torch.zeros_like(kcache)
    kc = torch.zeros((B, Hkv, cfg.ncmp, D), dtype=torch.int16, device=dev)
    vc = torch.zeros((B, Hkv, cfg.ncmp_tiles, D, 64), dtype=torch.int16, device=dev)
    starts = list(range(0, T, C))
    kn = [d["k"][:, :, P:P + C].contiguous() for P in starts]
    vn = [d["v"][:, :, P:P + C].contiguous() for P in starts]
    qn = [d["q"][:, P:P + C].contiguous() for P in starts]
    gn = [d["gate"][:, P:P + C].contiguous() for P in starts]
    sl = [torch.full((B,), P, dtype=torch.int32, device=dev) for P in starts]
    out = [torch.empty((B, q.shape[1], Hkv * G, D), dtype=torch.float32, device=dev) for q in qn]
    idx = [torch.empty((B, q.shape[1], Hkv, cfg.top_n), dtype=torch.int32, device=dev)
           for q in qn]
    aws = torch.empty(nsa.cache_append_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    pws = torch.empty(nsa.prefill_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    n = len(starts)

    def step(ev=None, base=0):
        for i, P in enumerate(starts):
            if ev is not None:
                ev.record(base + 2 * i, stream)
            nsa.nsa_cache_append(cfg, kn[i], vn[i], sl[i], d["wk"], d["wv"], kcache, vcache, kc,
                                 vc, ws=aws)
            if ev is not None:
                ev.record(base + 2 * i + 1, stream)
            nsa.nsa_prefill_chunk(cfg, P, qn[i], kcache, vcache, kc, vc, gn[i], out=out[i],
                                  sel_idx=idx[i], ws=pws)
        if ev is not None:
            ev.record(base + 2 * n, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents(args.steps * (2 * n + 1))
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev, s * (2 * n + 1))
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    app = [0.0] * n
    pre = [0.0] * n
    tot = 0.0
    for s in range(args.steps):
        b0 = s * (2 * n + 1)
        tot += ev.elapsed_ms(b0, b0 + 2 * n) / args.steps
        for i in range(n):
            app[i] += ev.elapsed_ms(b0 + 2 * i, b0 + 2 * i + 1) / args.steps
            pre[i] += ev.elapsed_ms(b0 + 2 * i + 1, b0 + 2 * i + 2) / args.steps
    return {
        "workload": "nsa chunked prefill B=%d T=%d Hkv=%d G=%d D=%d, chunks of %d%s" % (
            B, T, Hkv, G, D, C, " top_p=%g" % args.top_p if args.top_p > 0 else ""),
        "ms_per_step": round(wall * 1e3, 3),
        "events_ms_per_step": round(tot, 3),
        "tok_s": round(B * T / wall, 1),
        "append_ms": [round(v, 3) for v in app],
        "prefill_chunk_ms": [round(v, 3) for v in pre],
    }


def cpu_baseline_decode(x, B=32, L=65536, Hkv=4, G=16, D=128, nseq=4, reps=15):
    """fp64 oracle decode of `nseq` of the B sequences (their compressed caches built by the
    oracle, not timed: the decode call takes them as inputs), scaled to tokens/s."""
    import oracle as O

    sub = {k: (v[:nseq] if k in ("q", "kcache", "vcache", "gate", "seqlens") else v)
           for k, v in x.items()}
    kc = O.compress(sub["kcache"], x["wk"], 32, 16)
    vc = O.compress(sub["vcache"], x["wv"], 32, 16)
    cfg = O.NsaCfg(nseq, L, Hkv, G, D)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        O.nsa_decode(cfg, sub["q"], sub["kcache"], sub["vcache"], kc, vc, sub["seqlens"],
                     sub["gate"])
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return {"value": nseq / dt, "unit": "tok/s", "cores": O.threads(),
            "kind": "oracle", "sample": "fp64 oracle decode of %d of the %d sequences, median of "
                                        "%d runs (compressed caches precomputed, untimed)"
                                        % (nseq, B, reps)}


# ----------------------------------------------------------------------------- MoBA

def moba_work(T, H, D, block=512, top_k=3):
    t = np.arange(T, dtype=np.int64)
    b = t // block
    pairs = (t - b * block + 1) + block * np.minimum(b, top_k)
    gate = np.where(b > top_k, b, 0)
    return 4.0 * D * H * pairs.sum(), 2.0 * D * H * gate.sum(), int(pairs.sum())


def bench_moba(args, B=1, T=131072, H=32, D=128, seed=4, calls=5):
    """MoBA prefill at T tokens.  Up to 128k the inputs come from synth_inputs (shared with the
    oracle baseline); beyond, N(0,1) bf16 values are drawn on the device with a seeded torch
    generator (the host generator would take minutes and tens of GB at 1M x 32 heads)."""
    import torch

    import dynamic_block_sparse_fwd_amd as nsa
    import synth_inputs as S

    cfg = nsa.MobaConfig(B, T, H, D, block=512, top_k=3)
    t0 = time.time()
    dev = torch.device("cuda:0")
    if T <= 131072:
        x = S.moba_inputs(seed, B, T, H, D)
        d = {k: torch.from_numpy(v.view(np.int16)).to(dev) for k, v in x.items()}
    else:
        x = None
        shapes = {"q": (B, T, H, D), "k": (B, H, T, D), "v": (B, H, T, D)}
        d = {k: S.normal_bf16_device(seed, k, sh, dev) for k, sh in shapes.items()}
    print("[bench] MoBA inputs generated in %.1fs" % (time.time() - t0), file=sys.stderr,
          flush=True)
    out = torch.empty((B, T, H, D), dtype=torch.float32, device=dev)
    idx = torch.empty((B, T, H, cfg.top_k + 1), dtype=torch.int32, device=dev)
    ws = torch.empty(nsa.moba_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    nst = len(nsa.MOBA_STAGES)

    def call(events=None):
        nsa.moba_prefill(cfg, d["q"], d["k"], d["v"], out=out, sel_idx=idx, ws=ws, events=events)

    call()
    ev = HipEvents(calls * (nst + 1))
    torch.cuda.synchronize()
    for c in range(calls):
        call(ev.group(c * (nst + 1), nst + 1))
    torch.cuda.synchronize()
    tot = [ev.elapsed_ms(c * (nst + 1), c * (nst + 1) + nst) for c in range(calls)]
    stg = {nm: float(np.median([ev.elapsed_ms(c * (nst + 1) + i, c * (nst + 1) + i + 1)
                                for c in range(calls)]))
           for i, nm in enumerate(nsa.MOBA_STAGES)}
    ms = float(np.median(tot))
    f_att, f_gate, pairs = moba_work(T, H, D)
    passes = -(-H // max(1, min(H, (1 << 24) // (B * T))))
    res = {
        "workload": "moba_prefill B=%d T=%d H=%d D=%d block 512 top-3 + own" % (B, T, H, D),
        "ms_per_step": round(ms, 4),
        "tok_s": round(B * T / (ms * 1e-3), 1),
        "algorithmic_tflop": round((f_att + f_gate) / 1e12, 4),
        "mfma_frac_total": round((f_att + f_gate) / (ms * 1e-3) / MFMA_PEAK_BF16, 4),
        "head_passes": passes,
    }
    traffic = {"moba_block_kernel": measured_traffic("moba_block_kernel"),
               "moba_own_kernel": measured_traffic("moba_own_kernel")}
    if passes == 1:
        att_ms = stg["block_attn"] + stg["own_merge"]
        res["stages_ms"] = {k: round(v, 4) for k, v in stg.items()}
        res["roofline"] = {"bound": "mfma", "kernel": "block_attn + own_merge (attention)",
                           "achieved": round(f_att / (att_ms * 1e-3) / 1e12, 2),
                           "peak": MFMA_PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                           "frac": round(f_att / (att_ms * 1e-3) / MFMA_PEAK_BF16, 4),
                           "traffic": traffic}
    else:
        # the heads run in several passes and the stage events of a call mark only the last
        # pass (stage 0 spans the earlier ones): the roofline is the whole call's
        res["stages_ms_last_pass"] = {k: round(v, 4) for k, v in stg.items() if k != "pool_gate"}
        res["roofline"] = {"bound": "mfma", "kernel": "moba_prefill (whole call: gate and "
                                                      "attention, %d head passes)" % passes,
                           "achieved": round((f_att + f_gate) / (ms * 1e-3) / 1e12, 2),
                           "peak": MFMA_PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                           "frac": round((f_att + f_gate) / (ms * 1e-3) / MFMA_PEAK_BF16, 4),
                           "traffic": None}
    res["timing"] = "median of %d calls, HIP events around each stage" % calls
    del d, out, idx, ws
    torch.cuda.empty_cache()
    return res, x


def cpu_baseline_moba(x, T=131072, H=32, D=128, rows=24576):
    import oracle as O

    cfg = O.MobaCfg(1, T, H, D, block=512, top_k=3)
    t0 = time.perf_counter()
    kbar = O.moba_pool(cfg, x["k"])
    t_pool = time.perf_counter() - t0
    step = T // rows
    rt = np.arange(step // 2, T, step, dtype=np.int32)
    t0 = time.perf_counter()
    O.moba_prefill_rows(cfg, x["q"], x["k"], x["v"], np.zeros_like(rt), rt, kbar=kbar)
    t_rows = time.perf_counter() - t0
    est = t_pool + t_rows * T / len(rt)
    return {"value": T / est, "unit": "tok/s", "cores": O.threads(),
            "kind": "oracle", "sample": "fp64 oracle: block-key pooling (%.1fs) + %d positions "
                                        "every %d-th, all 32 heads (%.1fs), scaled to %d"
                                        % (t_pool, len(rt), step, t_rows, T)}


# ----------------------------------------------------------------------------- main

def host_info():
    """What the numbers were measured with: the host CPU model and thread count (the oracle
    baseline runs there), the library's source digest and, when the tree is a git checkout, its
    commit."""
    import hashlib
    import subprocess

    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    digest = h.hexdigest()[:16]
    try:
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                             text=True, timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        sha = None
    sha_from = "git" if sha else None
    if sha is None:  # a copy of the tree without .git: the commit recorded at build time
        try:
            with open(os.path.join(ROOT, "dynamic_block_sparse_fwd_amd",
                                   "libnsa.buildinfo.json")) as fh:
                info = json.load(fh)
            if info.get("library_source_sha256") == digest and info.get("git_sha"):
                sha = info["git_sha"]
                sha_from = ("build record, sources modified since that commit"
                            if info.get("csrc_modified_since_commit") else "build record")
        except (OSError, ValueError):
            pass
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "git_sha": sha,
            "git_sha_source": sha_from, "library_source_sha256": digest}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seq", type=int, default=65536)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-decode-1m", action="store_true",
                    help="skip the planted 1M-token decode workload")
    ap.add_argument("--no-moba", action="store_true")
    ap.add_argument("--moba-seq", type=int, default=131072,
                    help="MoBA sequence length for --only moba (beyond 128k: device-drawn inputs)")
    ap.add_argument("--moba-heads", type=int, default=32, help="MoBA heads for --only moba")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the rows beyond the headline workloads (MoBA at 10M tokens, the "
                         "backward, the chunked prefill)")
    ap.add_argument("--chunk", type=int, default=8192,
                    help="chunk length for --only chunked (a multiple of 64)")
    ap.add_argument("--only", choices=("prefill", "decode", "decode_1m", "moba", "chunked",
                                       "backward"),
                    help="run one workload and print its result alone (for profiling runs)")
    ap.add_argument("--top-p", type=float, default=0.0,
                    help="adaptive top-p block selection for the NSA workloads (0: fixed top-16)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run the plain copy used to scale the traffic counters, then exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs the NSA/MoBA forward on a single "
              "MI355X (multi-GPU sharding is a design note, not implemented); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.only == "decode":
        dec, _ = bench_decode(args)
        print(json.dumps({"decode": dec}), flush=True)
        return
    if args.only == "decode_1m":
        dec, host = bench_decode_planted(args)
        if host is not None:
            dec["cpu_baseline"] = cpu_baseline_decode_planted(host)
        print(json.dumps({"decode_1m": dec}), flush=True)
        return
    if args.only == "backward":
        print(json.dumps({"backward": bench_backward(args)}), flush=True)
        return
    if args.only == "chunked":
        print(json.dumps({"chunked": bench_chunked(args)}), flush=True)
        return
    if args.only == "moba":
        mo, _ = bench_moba(args, T=args.moba_seq, H=args.moba_heads)
        print(json.dumps({"moba": mo}), flush=True)
        return
    pre, x = bench_prefill(args)
    line = {
        "metric": METRIC,
        "value": round(pre["tok_s"], 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, random compressor weights and sigmoid gates)",
        "config": {"workload": "nsa_prefill", "B": 1, "T": args.seq, "Hkv": 4, "G": 16, "D": 128,
                   "cmp_len": 32, "cmp_stride": 16, "sel_block": 64, "top_n": 16, "n_local": 2,
                   "window": 512, "parallelism": "single GPU"},
        "roofline": {k: (round(v, 4) if isinstance(v, float) else v)
                     for k, v in pre["roofline"].items()},
        "prefill": {"mfma_frac_total": round(pre["mfma_frac"], 4),
                    "algorithmic_tflop": round(pre["algorithmic_tflop"], 4),
                    "instrumented_ms_per_step": round(pre["events_ms_per_step"], 4),
                    "stages": pre["stages"],
                    "selected_traffic": pre["selected_traffic"],
                    "blocks_per_row": round(pre["blocks_per_row"], 3),
                    "longest_stage": pre["longest_stage"],
                    "cmp_select_performed": {k: round(v, 4) for k, v in
                                             pre["cmp_select_performed"].items()}},
    }
    if args.top_p > 0:
        line["config"]["top_p"] = args.top_p
    line["host"] = host_info()
    if args.only == "prefill":
        print(json.dumps(line), flush=True)
        return
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(x, args.seq, args.cpu_rows)
    del x
    if not args.no_decode:
        dec, xd = bench_decode(args)
        if not args.no_cpu_baseline:
            dec["cpu_baseline"] = cpu_baseline_decode(xd)
        del xd
        line["decode"] = dec
    if not args.no_decode_1m:
        dec, host = bench_decode_planted(args)
        if host is not None:
            dec["cpu_baseline"] = cpu_baseline_decode_planted(host)
        del host
        line["decode_1m"] = dec
    if not args.no_moba:
        mo, xm = bench_moba(args)
        if not args.no_cpu_baseline:
            mo["cpu_baseline"] = cpu_baseline_moba(xm)
        del xm
        line["moba"] = mo
    if not args.no_next:
        # rows beyond the headline workloads, timed in the same run
        nxt = {"moba_10m": bench_moba(args, T=10 * (1 << 20), H=4, seed=10, calls=3)[0]}
        nxt["backward_64k"] = bench_backward(args)
        nxt["chunked_prefill_64k"] = bench_chunked(args)
        line["next_rows"] = nxt
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
