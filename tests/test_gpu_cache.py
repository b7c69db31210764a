"""GPU checks of generation-time cache maintenance (nsa_cache_append) and of chunked prefill
from the caches (nsa_prefill_chunk), through the C ABI.

  * appended rows land bit for bit; the compressed tokens emitted by the appends equal the
    oracle's compression of the whole sequence bit for bit; compressed tokens not yet complete
    keep the NaN they were poisoned with;
  * chunked prefill rows equal the one-shot nsa_prefill rows bit for bit, and the oracle's rows
    under the parity rules (indices bit-exact with the near-tie rule, outputs 1e-2 / 1e-3);
  * a generation loop (chunked prefill, then append-one-token + decode) matches the oracle at
    every step."""
import numpy as np
import pytest

import oracle as O
import synth_inputs as S
from tests.parity import check_close, check_nsa_idx

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

BF16_NAN = 0x7FC0


def _nsa():
    import dynamic_block_sparse_fwd_amd as nsa
    nsa.load_library()
    return nsa


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits(t):
    return t.cpu().numpy().view(np.uint16)


def empty_caches(B, L, Hkv, D, ncmp, nt):
    """Caches full of NaN: anything read before it is written shows up."""
    kc = torch.full((B, Hkv, L, D), BF16_NAN, dtype=torch.int16).cuda()
    vc = torch.full((B, Hkv, L, D), BF16_NAN, dtype=torch.int16).cuda()
    kcmp = torch.full((B, Hkv, max(ncmp, 1), D), BF16_NAN, dtype=torch.int16).cuda()[:, :, :ncmp]
    vcmp = torch.full((B, Hkv, nt, D, 64), BF16_NAN, dtype=torch.int16).cuda()
    return kc, vc, kcmp.contiguous(), vcmp


def append(nsa, cfg, x, caches, start, C):
    """Append tokens start[b] .. start[b]+C-1 of every sequence's full K/V."""
    kc, vc, kcmp, vcmp = caches
    idx = np.asarray(start)[:, None] + np.arange(C)[None, :]  # [B, C]
    bsel = np.arange(cfg.B)[:, None]
    k_new = np.ascontiguousarray(x["k"][bsel, :, idx].transpose(0, 2, 1, 3))  # [B,Hkv,C,D]
    v_new = np.ascontiguousarray(x["v"][bsel, :, idx].transpose(0, 2, 1, 3))
    nsa.nsa_cache_append(cfg, to_dev(k_new), to_dev(v_new), to_dev(np.asarray(start, np.int32)),
                         to_dev(x["wk"]), to_dev(x["wv"]), kc, vc, kcmp, vcmp)


@pytest.mark.parametrize("D", [64, 128])
def test_cache_append_bit_exact(D):
    nsa = _nsa()
    B, L, Hkv, G = 3, 1100, 2, 4
    print("case append D=%d" % D, flush=True)
    cfg = nsa.NsaConfig(B, L, Hkv, G, D)
    x = S.nsa_prefill_inputs(61 + D, B, L, Hkv, G, D)
    caches = empty_caches(B, L, Hkv, D, cfg.ncmp, cfg.ncmp_tiles)
    cur = np.array([0, 37, 300])
    # sequences 1 and 2 start from a host-filled prefix whose compressed tokens the host fills
    kc_full = O.compress(x["k"], x["wk"], 32, 16)
    vc_full = O.compress(x["v"], x["wv"], 32, 16)
    kc, vc, kcmp, vcmp = caches
    for b in (1, 2):
        kc[b, :, :cur[b]] = to_dev(x["k"][b, :, :cur[b]])
        vc[b, :, :cur[b]] = to_dev(x["v"][b, :, :cur[b]])
        n = O.n_cmp(int(cur[b]), 32, 16)
        kcmp[b, :, :n] = to_dev(kc_full[b, :, :n])
        vt = vc_full[b, :, :n].transpose(0, 2, 1)  # [Hkv, D, n]
        for i0 in range(0, n, 64):
            w = min(64, n - i0)
            vcmp[b, :, i0 // 64, :, :w] = to_dev(np.ascontiguousarray(vt[:, :, i0:i0 + w]))
    for C in [1, 1, 15, 16, 17, 64, 100, 1, 31, 33, 200, 3, 16, 16, 1]:
        append(nsa, cfg, x, caches, cur, C)
        cur = cur + C
    torch.cuda.synchronize()
    assert cur.max() <= L
    kcb, vcb, kcmpb, vcmpb = (bits(t) for t in caches)
    for b in range(B):
        n = O.n_cmp(int(cur[b]), 32, 16)
        assert np.array_equal(kcb[b, :, :cur[b]], x["k"][b, :, :cur[b]])
        assert np.array_equal(vcb[b, :, :cur[b]], x["v"][b, :, :cur[b]])
        assert (kcb[b, :, cur[b]:] == BF16_NAN).all()
        assert np.array_equal(kcmpb[b, :, :n], kc_full[b, :, :n]), "compressed keys, seq %d" % b
        assert (kcmpb[b, :, n:] == BF16_NAN).all(), "compressed keys written past n_cmp"
        vflat = vcmpb[b].transpose(0, 1, 3, 2).reshape(Hkv, -1, D)  # [Hkv, nt*64, D]
        assert np.array_equal(vflat[:, :n], vc_full[b, :, :n]), "compressed values, seq %d" % b
        assert (vflat[:, n:] == BF16_NAN).all(), "compressed values written past n_cmp"
    print("append D=%d: lengths %s bit-exact" % (D, cur.tolist()), flush=True)


CHUNK_CASES = [
    # name, B, L, Hkv, G, D, chunk boundaries, extra
    ("G4_D64", 1, 2048, 1, 4, 64, [0, 512, 1536, 2000], {}),
    ("G16_D128_B2", 2, 1700, 2, 16, 128, [0, 64, 1088, 1600, 1700], {}),
    ("G8_D128_topp", 1, 1500, 2, 8, 128, [0, 320, 1500], dict(top_p=0.5)),
    ("G2_D64_block128", 1, 1300, 2, 2, 64, [0, 640, 1300], dict(sel_block=128, top_n=6,
                                                             window=200)),
]


@pytest.mark.parametrize("name,B,L,Hkv,G,D,bounds,extra", CHUNK_CASES,
                         ids=[c[0] for c in CHUNK_CASES])
def test_prefill_chunks(name, B, L, Hkv, G, D, bounds, extra):
    nsa = _nsa()
    print("case chunk", name, flush=True)
    cfg = nsa.NsaConfig(B, L, Hkv, G, D, **extra)
    ocfg = O.NsaCfg(B, L, Hkv, G, D, **extra)
    x = S.nsa_prefill_inputs(71 + len(name), B, L, Hkv, G, D)
    d = {k: to_dev(v) for k, v in x.items()}
    one_out, one_idx = nsa.nsa_prefill(cfg, d["q"], d["k"], d["v"], d["wk"], d["wv"], d["gate"])
    caches = empty_caches(B, L, Hkv, D, cfg.ncmp, cfg.ncmp_tiles)
    kc = O.compress(x["k"], x["wk"], 32, 16)
    vc = O.compress(x["v"], x["wv"], 32, 16)
    for P, E in zip(bounds[:-1], bounds[1:]):
        C = E - P
        append(nsa, cfg, x, caches, [P] * B, C)
        out, idx = nsa.nsa_prefill_chunk(cfg, P, d["q"][:, P:E].contiguous(), *caches,
                                         d["gate"][:, P:E].contiguous())
        torch.cuda.synchronize()
        out, idx = out.cpu().numpy(), idx.cpu().numpy()
        assert np.array_equal(idx, one_idx[:, P:E].cpu().numpy()), "chunk [%d,%d) idx" % (P, E)
        assert np.array_equal(out, one_out[:, P:E].cpu().numpy()), "chunk [%d,%d) out" % (P, E)
        # oracle rows of the chunk (all of them for short chunks, else a spread sample)
        rt = np.arange(P, E) if C <= 600 else np.unique(np.r_[np.arange(P, P + 64),
                                                              np.linspace(P, E - 1, 300).astype(int),
                                                              np.arange(E - 64, E)])
        rb = np.repeat(np.arange(B), len(rt)).astype(np.int32)
        rt = np.tile(rt, B).astype(np.int32)
        ora = O.nsa_prefill_rows(ocfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], rb, rt,
                                 want_scores=True)
        gi = idx[rb, rt - P]
        rerun, acc = check_nsa_idx(gi, ora, rt, ocfg.sel_block, ocfg.top_n, ocfg.n_local,
                                   ocfg.top_p)
        ref = ora["out"].copy()
        if rerun:
            rr = np.array(rerun)
            ref[rr] = O.nsa_prefill_rows(ocfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], rb[rr],
                                         rt[rr], idx_in=gi[rr])["out"]
        mx, mean = check_close(out[rb, rt - P], ref, "%s chunk [%d,%d)" % (name, P, E))
        print("%s chunk [%d,%d): one-shot bit-exact, oracle max-abs %.2e mean-abs %.2e "
              "near-ties %d" % (name, P, E, mx, mean, acc), flush=True)


def test_prefill_chunk_1m_tail():
    """Chunked prefill at the largest capacity, 2^20 tokens (1 KV head x group 16, D = 128):
    the last 2048 positions from full caches, 16384 selection blocks (the selection streams).
    The compressed caches are the oracle's compression; queries and gates are drawn for the
    chunk's positions only (the oracle reads the rows it is asked for).  Sampled rows against
    the oracle, selection bit-exact under the near-tie rule."""
    nsa = _nsa()
    B, L, Hkv, G, D = 1, 1 << 20, 1, 16, 128
    P, C = L - 2048, 2048
    Hq = Hkv * G
    print("case chunk 1M tail", flush=True)
    cfg = nsa.NsaConfig(B, L, Hkv, G, D)
    ocfg = O.NsaCfg(B, L, Hkv, G, D)
    wstd = 1.0 / np.sqrt(32 * D)
    k = S.normal_bf16(61, "k", (B, Hkv, L, D))
    v = S.normal_bf16(61, "v", (B, Hkv, L, D))
    wk = S.normal_bf16(61, "wk", (32, D, D), std=wstd)
    wv = S.normal_bf16(61, "wv", (32, D, D), std=wstd)
    qc = S.normal_bf16(61, "q", (B, C, Hq, D))
    gc = S.gates(61, (B, C, Hq, 3))
    kc = O.compress(k, wk, 32, 16)
    vc = O.compress(v, wv, 32, 16)
    n = kc.shape[2]
    assert n == cfg.ncmp
    nt = cfg.ncmp_tiles
    vt = np.zeros((B, Hkv, nt * 64, D), dtype=np.uint16)
    vt[:, :, :n] = vc
    vt = np.ascontiguousarray(vt.reshape(B, Hkv, nt, 64, D).transpose(0, 1, 2, 4, 3))
    out, idx = nsa.nsa_prefill_chunk(cfg, P, to_dev(qc), to_dev(k), to_dev(v), to_dev(kc),
                                     to_dev(vt), to_dev(gc))
    torch.cuda.synchronize()
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    q = np.zeros((B, L, Hq, D), dtype=np.uint16)
    q[:, P:] = qc
    gate = np.zeros((B, L, Hq, 3), dtype=np.float32)
    gate[:, P:] = gc
    rng = np.random.default_rng(61)
    rt = np.unique(np.r_[np.arange(P, P + 32), rng.choice(np.arange(P, L), 96, replace=False),
                         np.arange(L - 32, L)]).astype(np.int32)
    rb = np.zeros_like(rt)
    ora = O.nsa_prefill_rows(ocfg, q, k, v, kc, vc, gate, rb, rt, want_scores=True)
    gi = idx[0, rt - P]
    rerun, acc = check_nsa_idx(gi, ora, rt, ocfg.sel_block, ocfg.top_n, ocfg.n_local,
                               ocfg.top_p)
    ref = ora["out"].copy()
    if rerun:
        rr = np.array(rerun)
        ref[rr] = O.nsa_prefill_rows(ocfg, q, k, v, kc, vc, gate, rb[rr], rt[rr],
                                     idx_in=gi[rr])["out"]
    mx, mean = check_close(out[0, rt - P], ref, "chunk 1M tail")
    print("chunk 1M tail: %d rows, max-abs %.2e mean-abs %.2e near-ties %d" % (
        len(rt), mx, mean, acc), flush=True)


def test_generation_loop():
    """Chunked prefill of 1024 tokens for two sequences, then 24 decode steps in which each
    sequence appends its newest token and decodes it; the second sequence starts 40 tokens
    behind, so compressed tokens are completed at different steps."""
    nsa = _nsa()
    B, L, Hkv, G, D = 2, 1200, 2, 16, 128
    cfg = nsa.NsaConfig(B, L, Hkv, G, D)
    ocfg = O.NsaCfg(B, L, Hkv, G, D)
    x = S.nsa_prefill_inputs(81, B, L, Hkv, G, D)
    kc = O.compress(x["k"], x["wk"], 32, 16)
    vc = O.compress(x["v"], x["wv"], 32, 16)
    d = {k: to_dev(v) for k, v in x.items()}
    caches = empty_caches(B, L, Hkv, D, cfg.ncmp, cfg.ncmp_tiles)
    append(nsa, cfg, x, caches, [0, 0], 1024)
    nsa.nsa_prefill_chunk(cfg, 0, d["q"][:, :1024].contiguous(), *caches,
                          d["gate"][:, :1024].contiguous())
    # the second sequence rolls back to 984 tokens (its cache rows past that are simply
    # overwritten by the next appends)
    cur = np.array([1024, 984])
    outs, rows_b, rows_t, idxs = [], [], [], []
    for step in range(24):
        append(nsa, cfg, x, caches, cur, 1)
        cur = cur + 1
        t = cur - 1
        q = torch.stack([d["q"][b, t[b]] for b in range(B)]).contiguous()
        g = torch.stack([d["gate"][b, t[b]] for b in range(B)]).contiguous()
        out, idx = nsa.nsa_decode(cfg, q, caches[0], caches[1], caches[2], caches[3],
                                  to_dev(cur.astype(np.int32)), g)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        idxs.append(idx.cpu().numpy())
        rows_b += list(range(B))
        rows_t += t.tolist()
    gout = np.concatenate(outs)
    gidx = np.concatenate(idxs)
    rb = np.array(rows_b, np.int32)
    rt = np.array(rows_t, np.int32)
    ora = O.nsa_prefill_rows(ocfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], rb, rt,
                             want_scores=True)
    rerun, acc = check_nsa_idx(gidx, ora, rt, 64, 16, 2)
    ref = ora["out"].copy()
    if rerun:
        rr = np.array(rerun)
        ref[rr] = O.nsa_prefill_rows(ocfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], rb[rr],
                                     rt[rr], idx_in=gidx[rr])["out"]
    mx, mean = check_close(gout, ref, "generation loop")
    print("generation loop: %d decode rows, max-abs %.2e mean-abs %.2e near-ties %d" % (
        len(rt), mx, mean, acc), flush=True)
