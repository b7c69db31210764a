"""GPU parity of nsa_decode (through the C ABI) against the fp64 oracle.

The compressed caches fed to both sides are the oracle's compression of the KV cache (the
decode call takes them as inputs; the GPU gets the values in feature-major 64-token tiles, as
nsa_decode wants); nsa_compress and nsa_compress_tiles are checked bit-exact elsewhere.  Every
compressed token a sequence may not see, and the pad tokens of the last value tile, hold NaN on
the GPU side: the kernels must never let them into a result."""
import numpy as np
import pytest

import oracle as O
import synth_inputs as S
from tests.parity import check_close, check_nsa_idx

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


BF16_NAN = np.uint16(0x7FC0)


def poisoned_caches(cfg, kc, vc, seqlens):
    """kc [B,Hkv,ncmp,D] and vc in feature-major 64-token tiles [B,Hkv,nt,D,64], with NaN in
    every compressed token that the sequence's query may not see (i*d + l > seqlen) and in the
    pad tokens of the last tile."""
    B, Hkv, ncmp, D = kc.shape
    nt = (ncmp + 63) // 64
    kp = kc.copy()
    vp = np.full((B, Hkv, nt * 64, D), BF16_NAN, dtype=np.uint16)
    vp[:, :, :ncmp] = vc
    for b, L in enumerate(seqlens):
        nvis = (L - cfg.cmp_len) // cfg.cmp_stride + 1 if L >= cfg.cmp_len else 0
        kp[b, :, nvis:] = BF16_NAN
        vp[b, :, nvis:] = BF16_NAN
    vt = np.ascontiguousarray(vp.reshape(B, Hkv, nt, 64, D).transpose(0, 1, 2, 4, 3))
    return kp, vt


def gpu_decode(cfg, x, kc, vc, seqlens, repeat=False):
    """nsa_decode on the device; repeat: call it a second time on the same buffers and require
    the same output and indices bit for bit (decode is deterministic)."""
    import dynamic_block_sparse_fwd_amd as nsa
    nsa.load_library()
    c = nsa.NsaConfig(cfg.B, cfg.T, cfg.Hkv, cfg.G, cfg.D, cfg.cmp_len, cfg.cmp_stride,
                      cfg.sel_block, cfg.top_n, cfg.n_local, cfg.window, cfg.scale,
                      cfg.top_p)
    kp, vt = poisoned_caches(cfg, kc, vc, seqlens)
    args = (to_dev(x["q"]), to_dev(x["kcache"]), to_dev(x["vcache"]), to_dev(kp), to_dev(vt),
            to_dev(np.asarray(seqlens, np.int32)), to_dev(x["gate"]))
    out, idx = nsa.nsa_decode(c, *args)
    if repeat:
        out2, idx2 = nsa.nsa_decode(c, *args)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx2), "decode indices differ between two calls"
        assert torch.equal(out, out2), "decode output differs between two calls"
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


def check_decode(cfg, x, kc, vc, seqlens, what, repeat=False):
    gout, gidx = gpu_decode(cfg, x, kc, vc, seqlens, repeat)
    ora = O.nsa_decode(cfg, x["q"], x["kcache"], x["vcache"], kc, vc, seqlens, x["gate"],
                       want_scores=True)
    rows_t = np.asarray(seqlens) - 1
    rerun, acc = check_nsa_idx(gidx, ora, rows_t, cfg.sel_block, cfg.top_n, cfg.n_local,
                               cfg.top_p)
    ref = ora["out"].copy()
    if rerun:
        idx_in = ora["idx"].copy()
        idx_in[rerun] = gidx[rerun]
        ref = O.nsa_decode(cfg, x["q"], x["kcache"], x["vcache"], kc, vc, seqlens, x["gate"],
                           idx_in=idx_in)["out"]
    mx, mean = check_close(gout, ref, what)
    print("%s: max-abs %.2e mean-abs %.2e near-ties %d" % (what, mx, mean, acc), flush=True)
    return gout, gidx, ora


DECODE_CASES = [
    # name, B, L, Hkv, G, D, seqlens, extra
    ("G16_D128", 4, 2000, 2, 16, 128, [2000, 1500, 777, 64], {}),
    ("G8_D128_short", 6, 700, 1, 8, 128, [1, 31, 32, 33, 65, 700], {}),
    ("G4_D64", 3, 3000, 3, 4, 64, [3000, 2999, 1025], {}),
    ("G1_D64_block128", 2, 2500, 2, 1, 64, [2500, 1300], dict(sel_block=128, top_n=6, window=200)),
    ("G2_D128_top5", 2, 4100, 1, 2, 128, [4100, 4096], dict(top_n=5, n_local=1, window=64)),
    # 128 compressed tokens fill two tiles exactly; the last block's only visible token is the
    # carry out of the last tile
    ("G4_D128_tile_edge", 2, 2064, 1, 4, 128, [2064, 2063], {}),
    # adaptive top-p, also on sequences short enough for every block to fit
    ("topp0.3_G16_D128", 4, 2000, 2, 16, 128, [2000, 1500, 777, 64], dict(top_p=0.3)),
    ("topp0.5_G8_D128_short", 6, 700, 1, 8, 128, [1, 31, 32, 33, 65, 700], dict(top_p=0.5)),
    ("topp0.9_G4_D64", 3, 3000, 3, 4, 64, [3000, 2999, 1025], dict(top_p=0.9)),
    ("topp0.5_G2_D128_top5", 2, 4100, 1, 2, 128, [4100, 4096],
     dict(top_p=0.5, top_n=5, n_local=1, window=64)),
    ("topp1_G1_D64_block128", 2, 2500, 2, 1, 64, [2500, 1300],
     dict(top_p=1.0, sel_block=128, top_n=6, window=200)),
    ("topp_tiny_G16_D128", 3, 3000, 2, 16, 128, [3000, 1000, 40], dict(top_p=1e-6)),
    # other compression geometries (the generic block-mass path)
    ("cmp16x16_G4_D64", 2, 2100, 2, 4, 64, [2100, 1100], dict(cmp_len=16, cmp_stride=16)),
    ("cmp48x16_G16_D128", 2, 2000, 1, 16, 128, [2000, 47], dict(cmp_len=48, cmp_stride=16)),
    ("cmp64x32_G8_D128", 2, 3000, 2, 8, 128, [3000, 1500], dict(cmp_len=64, cmp_stride=32)),
]


@pytest.mark.parametrize("name,B,L,Hkv,G,D,seqlens,extra", DECODE_CASES,
                         ids=[c[0] for c in DECODE_CASES])
def test_decode_parity(name, B, L, Hkv, G, D, seqlens, extra):
    print("case", name, flush=True)
    cfg = O.NsaCfg(B, L, Hkv, G, D, **extra)
    x = S.nsa_decode_inputs(30 + len(name), B, L, Hkv, G, D, l=cfg.cmp_len)
    kc = O.compress(x["kcache"], x["wk"], cfg.cmp_len, cfg.cmp_stride)
    vc = O.compress(x["vcache"], x["wv"], cfg.cmp_len, cfg.cmp_stride)
    check_decode(cfg, x, kc, vc, seqlens, name, repeat=True)


def test_decode_equals_prefill_last_row_on_gpu():
    """Cross path: decode of position L-1 equals row L-1 of a prefill on the same data."""
    import dynamic_block_sparse_fwd_amd as nsa
    B, L, Hkv, G, D = 1, 1500, 2, 16, 128
    x = S.nsa_prefill_inputs(33, B, L, Hkv, G, D)
    c = nsa.NsaConfig(B, L, Hkv, G, D)
    d = {k: to_dev(v) for k, v in x.items()}
    pout, pidx = nsa.nsa_prefill(c, d["q"], d["k"], d["v"], d["wk"], d["wv"], d["gate"])
    kc = nsa.nsa_compress(c, d["k"], d["wk"])
    vc = nsa.nsa_compress_tiles(c, d["v"], d["wv"])
    dout, didx = nsa.nsa_decode(c, d["q"][:, L - 1].contiguous(), d["k"], d["v"], kc, vc,
                                torch.tensor([L], dtype=torch.int32, device="cuda"),
                                d["gate"][:, L - 1].contiguous())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(didx.cpu().numpy(), pidx[:, L - 1].cpu().numpy())
    check_close(dout.cpu().numpy(), pout[:, L - 1].cpu().numpy(), "decode vs prefill row")


def test_decode_64k_batch32_all_rows():
    """The 64k decode workload: batch 32, 4 KV heads x group 16, D=128, every sequence full;
    two calls on the same buffers give the same result bit for bit."""
    B, L, Hkv, G, D = 32, 65536, 4, 16, 128
    cfg = O.NsaCfg(B, L, Hkv, G, D)
    x = S.nsa_decode_inputs(3, B, L, Hkv, G, D)
    kc = O.compress(x["kcache"], x["wk"], 32, 16)
    vc = O.compress(x["vcache"], x["wv"], 32, 16)
    check_decode(cfg, x, kc, vc, [L] * B, "decode 64k x 32", repeat=True)


def test_decode_1m_planted_recall():
    """1M-token decode, 8 KV heads x group 8: 16 planted blocks per KV head, keys shifted +2
    sigma toward the group's query direction; with mean-pooled compression every free pick must
    be a planted block, and the output must match the oracle."""
    B, L, Hkv, G, D = 1, 1 << 20, 8, 8, 128
    cfg = O.NsaCfg(B, L, Hkv, G, D)
    x = S.nsa_decode_inputs(5, B, L, Hkv, G, D)
    planted = S.plant_blocks(5, x["kcache"], x["q"], G)
    mp = S.mean_pool_weights(32, D)
    kc = O.compress(x["kcache"], mp, 32, 16)
    vc = O.compress(x["vcache"], mp, 32, 16)
    gout, gidx, ora = check_decode(cfg, x, kc, vc, [L], "decode 1M planted")
    nblk = L // 64
    for h in range(Hkv):
        free = [j for j in gidx[0, h] if j not in (0, nblk - 2, nblk - 1)]
        assert len(free) == 13
        assert set(free) <= set(planted[0, h].tolist()), (h, free, planted[0, h])
