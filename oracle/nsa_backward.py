"""fp64 backward of the NSA prefill layer, for the parity tests of nsa_backward.

TEST INFRASTRUCTURE ONLY: imported by tests/ (and nothing on the product path).  Plain numpy,
one (sequence, KV group, position) at a time, vectorised over the group's heads and the
position's keys.  It shares no code with the GPU library.

Method ([Notes] "Zhang Xiaojun podcast EP94" notes, section 5: the three branches and the gate;
section 8 and the "Native Sparse Attention" article: the layer is trained end to end, the
compressor being a learnable linear map):
  out = g_cmp * o_cmp + g_slc * o_slc + g_win * o_win, each o an attention
  o = softmax(scale * q . K_set) V_set over its key set: the visible compressed tokens, the
  tokens (<= t) of the selected blocks, the w most recent tokens.
Readings:
  B1 the block selection is a discrete choice: its indices are held fixed (taken from the
     forward) and the block-importance path carries no gradient;
  B2 the bf16 rounding of a compressed token is treated as the identity in the backward
     (straight-through); the forward values use the rounded tokens, like the forward oracle
     (round_cmp=False drops the rounding, for finite-difference checks);
  B3 gates are inputs of the layer: d gate[t, h, br] = <d out[t, h], o_br[t, h]>.
Gradients of one branch, with P the probabilities, dO_br = g_br * d out:
  dV_set += P^T dO_br;  dP = dO_br V_set^T;  dS = P * (dP - rowsum(P * dP));
  dq += scale * dS K_set;  dK_set += scale * dS^T q;
and through the compressor Kc[i] = sum_j K[i d + j] W[j]:
  dK[i d + j] += dKc[i] W[j]^T,  dW[j] += K[i d + j]^T dKc[i] (summed over sequences, heads).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def round_bf16(x):
    """fp64 -> nearest bf16 value (ties to even), via fp32 with round-to-odd so the double
    rounding is exact."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    back = f.astype(np.float64)
    u = f.view(np.uint32).copy()
    inexact = back != x
    # round-to-odd fp32: if the fp32 rounding was inexact, force the last bit to 1 after
    # truncating toward zero
    trunc = np.where(np.abs(back) > np.abs(x), np.nextafter(f, np.float32(0)), f)
    ut = trunc.view(np.uint32) | np.uint32(1)
    u = np.where(inexact, ut, u)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    b = ((u + r) >> 16).astype(np.uint16)
    return bf16_to_f64(b)


def n_cmp(T, l, d):
    return (T - l) // d + 1 if T >= l else 0


def compress_f64(x, w, l, d, round_cmp=True):
    """x [T, D] fp64, w [l, D, D] -> [n_cmp, D]: token i = sum_j x[i d + j] @ w[j]."""
    T, D = x.shape
    n = n_cmp(T, l, d)
    out = np.zeros((n, D))
    for j in range(l):
        out += x[j:j + d * (n - 1) + 1:d] @ w[j]
    return round_bf16(out) if round_cmp else out


def _key_sets(t, nvis, idx_row, beta, window):
    sel = [s for j in idx_row if j >= 0 for s in range(j * beta, min((j + 1) * beta, t + 1))]
    win = list(range(max(0, t - window + 1), t + 1))
    return np.arange(nvis), np.array(sel, dtype=np.int64), np.array(win, dtype=np.int64)


def _attend(qh, K, V, scale):
    S = scale * qh @ K.T
    S -= S.max(axis=1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(axis=1, keepdims=True)
    return P, P @ V


def forward(cfg, q, k, v, wk, wv, gate, idx, round_cmp=True):
    """fp64 forward with the selection fixed to idx [B, T, Hkv, n].
    q [B,T,Hq,D], k/v [B,Hkv,T,D], wk/wv [l,D,D], gate [B,T,Hq,3], all fp64.
    Returns out [B,T,Hq,D]."""
    B, T, Hq, D = q.shape
    G, l, d = cfg.G, cfg.cmp_len, cfg.cmp_stride
    out = np.zeros((B, T, Hq, D))
    for b in range(B):
        for g in range(cfg.Hkv):
            kc = compress_f64(k[b, g], wk, l, d, round_cmp)
            vc = compress_f64(v[b, g], wv, l, d, round_cmp)
            hs = slice(g * G, (g + 1) * G)
            for t in range(T):
                nvis = n_cmp(t + 1, l, d)
                c_keys, s_keys, w_keys = _key_sets(t, nvis, idx[b, t, g], cfg.sel_block,
                                                   cfg.window)
                qh = q[b, t, hs]
                o = np.zeros((G, D))
                if nvis > 0:
                    o += gate[b, t, hs, 0:1] * _attend(qh, kc[c_keys], vc[c_keys], cfg.scale)[1]
                o += gate[b, t, hs, 1:2] * _attend(qh, k[b, g, s_keys], v[b, g, s_keys],
                                                   cfg.scale)[1]
                o += gate[b, t, hs, 2:3] * _attend(qh, k[b, g, w_keys], v[b, g, w_keys],
                                                   cfg.scale)[1]
                out[b, t, hs] = o
    return out


def backward(cfg, q, k, v, wk, wv, gate, idx, dout, round_cmp=True, rows=None):
    """Gradients of sum(dout * out) for the inputs of forward(): dict with dq, dk, dv, dwk, dwv,
    dgate (same shapes as the inputs).  rows: None, or the positions whose terms are summed (the
    others count as dout = 0): dq and dgate are then exact on those rows, and dk, dv on keys
    that only they can see (keys s with every position >= s in rows)."""
    B, T, Hq, D = q.shape
    G, l, d, sc = cfg.G, cfg.cmp_len, cfg.cmp_stride, cfg.scale
    # fp64 results whatever the input dtype (bf16 inputs may come as exact fp32 arrays)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    dwk = np.zeros(wk.shape)
    dwv = np.zeros(wv.shape)
    dgate = np.zeros(gate.shape)
    for b in range(B):
        for g in range(cfg.Hkv):
            kc = compress_f64(k[b, g].astype(np.float64), wk, l, d, round_cmp)
            vc = compress_f64(v[b, g].astype(np.float64), wv, l, d, round_cmp)
            dkc = np.zeros_like(kc)
            dvc = np.zeros_like(vc)
            hs = slice(g * G, (g + 1) * G)
            for t in (range(T) if rows is None else rows):
                nvis = n_cmp(t + 1, l, d)
                c_keys, s_keys, w_keys = _key_sets(t, nvis, idx[b, t, g], cfg.sel_block,
                                                   cfg.window)
                qh = q[b, t, hs]
                do = dout[b, t, hs]
                branches = [(kc, vc, dkc, dvc, c_keys), (k[b, g], v[b, g], dk[b, g], dv[b, g],
                                                         s_keys),
                            (k[b, g], v[b, g], dk[b, g], dv[b, g], w_keys)]
                for br, (Ks, Vs, dKs, dVs, keys) in enumerate(branches):
                    if len(keys) == 0:
                        continue  # no visible compressed token: the branch output is zero
                    K_, V_ = Ks[keys], Vs[keys]
                    P, O = _attend(qh, K_, V_, sc)
                    dgate[b, t, hs, br] = np.sum(do * O, axis=1)
                    dob = gate[b, t, hs, br][:, None] * do
                    np.add.at(dVs, keys, P.T @ dob)
                    dP = dob @ V_.T
                    dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
                    dq[b, t, hs] += sc * dS @ K_
                    np.add.at(dKs, keys, sc * dS.T @ qh)
            # through the compressor (the rounding passes the gradient unchanged, B2)
            n = kc.shape[0]
            for j in range(l):
                toks = slice(j, j + d * (n - 1) + 1, d)
                if n == 0:
                    continue
                dk[b, g, toks] += dkc @ wk[j].T
                dv[b, g, toks] += dvc @ wv[j].T
                dwk[j] += k[b, g, toks].T @ dkc
                dwv[j] += v[b, g, toks].T @ dvc
    return dict(dq=dq, dk=dk, dv=dv, dwk=dwk, dwv=dwv, dgate=dgate)


def inputs_f64(x):
    """The seeded bf16 inputs (and fp32 gates) as fp64 arrays."""
    return dict(q=bf16_to_f64(x["q"]), k=bf16_to_f64(x["k"]), v=bf16_to_f64(x["v"]),
                wk=bf16_to_f64(x["wk"]), wv=bf16_to_f64(x["wv"]),
                gate=np.asarray(x["gate"], dtype=np.float64))
