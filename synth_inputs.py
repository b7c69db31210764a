"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module only draws random numbers and stores them as bfloat16 bit patterns; it holds
none of the attention arithmetic.  Every tensor gets its own PCG64 substream
(seed * 16 + slot) so any tensor can be regenerated alone, in chunks, with identical bits.

Value recipe (the pages measure on activations of trained models, which are not available;
these i.i.d. draws stand in for them):
  * Q, K, V, KV caches ~ N(0, 1), rounded to bf16 (round to nearest even);
  * compressor weights ~ N(0, std = 1/sqrt(l * D)), rounded to bf16;
  * gates = sigmoid(N(0, 1)) as fp32 (the gate network itself is outside the layer);
  * planted long-context decode: per KV head, 16 distinct blocks drawn from [1, nblk - 3];
    every key of those blocks gets + 2 * unit(sum of the group's query vectors), re-rounded.
"""
from __future__ import annotations

import numpy as np

SLOT = {"q": 0, "k": 1, "v": 2, "wk": 3, "wv": 4, "gate": 5, "plant": 6, "seqlen": 7,
        "dout": 8}


def _gen(seed: int, slot: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed * 16 + SLOT[slot]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even. Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: int, slot: str, shape, std: float = 1.0, chunk: int = 1 << 26) -> np.ndarray:
    """N(0, std^2) draws in fp32, rounded to bf16 bits.  Drawn in chunks to bound host memory;
    chunked draws from one PCG64 stream equal a single draw."""
    g = _gen(seed, slot)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = g.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = f32_to_bf16_bits(x)
    return out.reshape(shape)


def normal_bf16_device(seed: int, slot: str, shape, device, chunk: int = 1 << 28):
    """N(0, 1) bf16 drawn on a torch device with its Philox generator seeded seed * 16 + slot,
    in chunks of `chunk` fp32 draws rounded to bf16 (round to nearest even) -- for inputs too
    large to draw on the host (tens of GB).  Not the same values as normal_bf16."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed * 16 + SLOT[slot])
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        flat[s:e] = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
    return out


def upstream_grad(seed: int, shape) -> np.ndarray:
    """Gradient of the loss with respect to the layer output: N(0, 1) in fp32."""
    g = _gen(seed, "dout")
    return g.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)


def block_selection(B: int, T: int, Hkv: int, top_n: int = 16, beta: int = 64,
                    n_local: int = 2) -> np.ndarray:
    """A deterministic, valid block-index list [B, T, Hkv, top_n] (ascending, -1 padded) for
    inputs of the backward: block 0, the n_local most recent blocks, and top_n - 1 - n_local
    distinct other blocks spread by a fixed stride (all blocks while they fit).  No scores are
    involved: any selection is a legal input of the backward."""
    t = np.arange(T, dtype=np.int64)
    b = t // beta
    out = np.full((B, T, Hkv, top_n), -1, dtype=np.int32)
    kfree = top_n - 1 - n_local
    for g in range(Hkv):
        for bb in range(B):
            rows = np.full((T, top_n), -1, dtype=np.int64)
            fit = b + 1 <= top_n
            ar = np.arange(top_n)
            rows[fit] = np.where(ar[None, :] <= b[fit, None], ar[None, :], -1)
            nf = ~fit
            bn = b[nf]
            span = bn - n_local  # free candidates 1 .. bn - n_local
            off = (t[nf] * 7919 + g * 31 + bb * 17) % span
            free = 1 + (off[:, None] + np.arange(kfree)[None, :] * 104729) % span[:, None]
            local = bn[:, None] - np.arange(n_local)[None, :]
            sel = np.concatenate([np.zeros((nf.sum(), 1), np.int64), free, local], axis=1)
            rows[nf] = np.sort(sel, axis=1)
            out[bb, :, g] = rows
    return out


def gates(seed: int, shape) -> np.ndarray:
    g = _gen(seed, "gate")
    x = g.standard_normal(int(np.prod(shape)), dtype=np.float32).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32).reshape(shape)


def nsa_prefill_inputs(seed: int, B: int, T: int, Hkv: int, G: int, D: int, l: int = 32):
    Hq = Hkv * G
    wstd = 1.0 / np.sqrt(l * D)
    return dict(
        q=normal_bf16(seed, "q", (B, T, Hq, D)),
        k=normal_bf16(seed, "k", (B, Hkv, T, D)),
        v=normal_bf16(seed, "v", (B, Hkv, T, D)),
        wk=normal_bf16(seed, "wk", (l, D, D), std=wstd),
        wv=normal_bf16(seed, "wv", (l, D, D), std=wstd),
        gate=gates(seed, (B, T, Hq, 3)),
    )


def nsa_decode_inputs(seed: int, B: int, L: int, Hkv: int, G: int, D: int, l: int = 32,
                      seqlens=None):
    """Decode inputs: one query per sequence, a K/V cache of capacity L (all positions filled),
    compressor weights for building the compressed cache, gates.  seqlens defaults to L."""
    Hq = Hkv * G
    wstd = 1.0 / np.sqrt(l * D)
    if seqlens is None:
        seqlens = np.full(B, L, dtype=np.int32)
    return dict(
        q=normal_bf16(seed, "q", (B, Hq, D)),
        kcache=normal_bf16(seed, "k", (B, Hkv, L, D)),
        vcache=normal_bf16(seed, "v", (B, Hkv, L, D)),
        wk=normal_bf16(seed, "wk", (l, D, D), std=wstd),
        wv=normal_bf16(seed, "wv", (l, D, D), std=wstd),
        gate=gates(seed, (B, Hq, 3)),
        seqlens=np.asarray(seqlens, dtype=np.int32),
    )


def mean_pool_weights(l: int, D: int) -> np.ndarray:
    """W[j] = I / l as bf16 bits (1/l is a power of two for l = 32, so exact)."""
    w = np.zeros((l, D, D), dtype=np.float32)
    for j in range(l):
        w[j] = np.eye(D, dtype=np.float32) / l
    return f32_to_bf16_bits(w)


def plant_blocks(seed: int, kcache: np.ndarray, q: np.ndarray, G: int, sel_block: int = 64,
                 n_plant: int = 16, shift: float = 2.0):
    """Shift every key of n_plant random blocks per KV head toward the group's query direction.

    kcache: bf16 bits [B, Hkv, L, D] (modified in place); q: bf16 bits [B, Hq, D].
    Returns the planted block ids, int64 [B, Hkv, n_plant] (sorted)."""
    B, Hkv, L, D = kcache.shape
    nblk = L // sel_block
    g = _gen(seed, "plant")
    planted = np.empty((B, Hkv, n_plant), dtype=np.int64)
    qf = bf16_bits_to_f32(q).reshape(B, Hkv, G, D).astype(np.float64)
    for b in range(B):
        for h in range(Hkv):
            blocks = np.sort(g.choice(np.arange(1, nblk - 2), size=n_plant, replace=False))
            planted[b, h] = blocks
            dirn = qf[b, h].sum(axis=0)
            dirn /= np.linalg.norm(dirn)
            for j in blocks:
                s = slice(j * sel_block, (j + 1) * sel_block)
                kk = bf16_bits_to_f32(kcache[b, h, s]).astype(np.float64) + shift * dirn
                kcache[b, h, s] = f32_to_bf16_bits(kk.astype(np.float32))
    return planted


def moba_inputs(seed: int, B: int, T: int, H: int, D: int):
    return dict(
        q=normal_bf16(seed, "q", (B, T, H, D)),
        k=normal_bf16(seed, "k", (B, H, T, D)),
        v=normal_bf16(seed, "v", (B, H, T, D)),
    )
