"""GPU parity of moba_prefill (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

import oracle as O
import synth_inputs as S
from tests.parity import check_close, check_moba_idx

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def to_dev(a):
    return torch.from_numpy(a.view(np.int16)).cuda()


def gpu_moba(cfg, x):
    import dynamic_block_sparse_fwd_amd as nsa
    nsa.load_library()
    c = nsa.MobaConfig(cfg.B, cfg.T, cfg.H, cfg.D, cfg.block, cfg.top_k, cfg.scale)
    out, idx = nsa.moba_prefill(c, to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]))
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


def check_moba(cfg, x, rows_b, rows_t, gout, gidx, what):
    """gout [R, H, D] and gidx [R, H, top_k + 1]: the GPU's rows (rows_b, rows_t)."""
    kbar = O.moba_pool(cfg, x["k"])
    ora = O.moba_prefill_rows(cfg, x["q"], x["k"], x["v"], rows_b, rows_t, kbar=kbar,
                              want_scores=True)
    qf = S.bf16_bits_to_f32(x["q"][rows_b, rows_t]).astype(np.float64)  # [R, H, D]
    qn = np.linalg.norm(qf, axis=-1)
    kn = np.linalg.norm(kbar, axis=-1)  # [B, H, nb]
    den = np.zeros_like(qn)
    for r, (b, t) in enumerate(zip(rows_b, rows_t)):
        bq = t // cfg.block
        if bq > 0:
            den[r] = qn[r] * kn[b, :, :bq].max(axis=-1)
    gi = gidx
    rerun, acc = check_moba_idx(gi, ora, rows_t, cfg.block, cfg.top_k, den)
    ref = ora["out"].copy()
    if rerun:
        rr = np.array(rerun)
        ref[rr] = O.moba_prefill_rows(cfg, x["q"], x["k"], x["v"], rows_b[rr], rows_t[rr],
                                      kbar=kbar, idx_in=gi[rr])["out"]
    mx, mean = check_close(gout, ref, what)
    print("%s: rows=%d max-abs %.2e mean-abs %.2e near-ties %d" % (what, len(rows_t), mx, mean,
                                                                    acc), flush=True)


CASES = [
    ("T2048_H2_D64_blk128", 1, 2048, 2, 64, 128, 3),
    ("T4096_H4_D128_blk512", 1, 4096, 4, 128, 512, 3),
    ("B2_T3072_H3_D128_blk256_top2", 2, 3072, 3, 128, 256, 2),
    ("T2560_H2_D64_blk64_top8", 1, 2560, 2, 64, 64, 8),
    ("T1024_H2_D64_blk128_top0", 1, 1024, 2, 64, 128, 0),
]


@pytest.mark.parametrize("name,B,T,H,D,block,top_k", CASES, ids=[c[0] for c in CASES])
def test_moba_parity_all_rows(name, B, T, H, D, block, top_k):
    print("case", name, flush=True)
    cfg = O.MobaCfg(B, T, H, D, block=block, top_k=top_k)
    x = S.moba_inputs(40 + T // 64 + top_k, B, T, H, D)
    gout, gidx = gpu_moba(cfg, x)
    b, t = np.meshgrid(np.arange(B), np.arange(T), indexing="ij")
    rb, rt = b.ravel().astype(np.int32), t.ravel().astype(np.int32)
    check_moba(cfg, x, rb, rt, gout[rb, rt], gidx[rb, rt], name)


def test_moba_full_coverage_is_causal_attention():
    """top_k >= number of past blocks: MoBA is full causal attention (GPU vs oracle vs SDPA)."""
    cfg = O.MobaCfg(1, 1024, 2, 64, block=128, top_k=8)
    x = S.moba_inputs(49, 1, 1024, 2, 64)
    gout, gidx = gpu_moba(cfg, x)
    f = lambda a: S.bf16_bits_to_f32(a).astype(np.float64)
    q = torch.from_numpy(f(x["q"][0]).transpose(1, 0, 2).copy())
    k = torch.from_numpy(f(x["k"][0]).copy())
    v = torch.from_numpy(f(x["v"][0]).copy())
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).numpy()
    check_close(gout[0], ref.transpose(1, 0, 2), "moba full coverage")


def test_moba_128k_sampled_rows():
    """The 128k MoBA workload (32 heads, D=128, block 512, top-3 + own): every row of the
    first 4 blocks, the last 64 rows, and a seeded random remainder (4096 rows in all)."""
    B, T, H, D = 1, 131072, 32, 128
    cfg = O.MobaCfg(B, T, H, D, block=512, top_k=3)
    x = S.moba_inputs(4, B, T, H, D)
    gout, gidx = gpu_moba(cfg, x)
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([np.arange(2048), np.arange(T - 64, T),
                                     rng.choice(np.arange(2048, T - 64), 4096 - 2048 - 64,
                                                replace=False)])).astype(np.int32)
    check_moba(cfg, x, np.zeros_like(rows), rows, gout[0, rows], gidx[0, rows], "moba 128k")


def test_moba_1m_sampled_rows():
    """MoBA at 1M tokens (the next row after the 128k workload: 2048 blocks of 512 per head), 4
    heads, D=128, top-3 + own: every row of the first 4 blocks, the last 64 rows and a seeded
    random remainder (3072 rows in all)."""
    B, T, H, D = 1, 1 << 20, 4, 128
    cfg = O.MobaCfg(B, T, H, D, block=512, top_k=3)
    x = S.moba_inputs(6, B, T, H, D)
    gout, gidx = gpu_moba(cfg, x)
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([np.arange(2048), np.arange(T - 64, T),
                                     rng.choice(np.arange(2048, T - 64), 3072 - 2048 - 64,
                                                replace=False)])).astype(np.int32)
    check_moba(cfg, x, np.zeros_like(rows), rows, gout[0, rows], gidx[0, rows], "moba 1M")


def test_moba_10m_sampled_rows():
    """MoBA at 10M tokens (10 x 2^20 = 20480 blocks of 512 per head), 4 heads, D=128, top-3 +
    own; the heads run in passes of one.  Inputs are drawn on the device (32 GB); the oracle
    gets the keys and values whole and the queries of the checked rows: every row of the first
    4 blocks, the last 64 rows and a seeded random remainder (2560 rows in all)."""
    import dynamic_block_sparse_fwd_amd as nsa
    nsa.load_library()
    B, T, H, D = 1, 10 * (1 << 20), 4, 128
    print("case moba 10M", flush=True)
    cfg = O.MobaCfg(B, T, H, D, block=512, top_k=3)
    c = nsa.MobaConfig(B, T, H, D, 512, 3, cfg.scale)
    dev = torch.device("cuda")
    d = {"q": S.normal_bf16_device(10, "q", (B, T, H, D), dev),
         "k": S.normal_bf16_device(10, "k", (B, H, T, D), dev),
         "v": S.normal_bf16_device(10, "v", (B, H, T, D), dev)}
    out, idx = nsa.moba_prefill(c, d["q"], d["k"], d["v"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(10)
    rows = np.unique(np.concatenate([np.arange(2048), np.arange(T - 64, T),
                                     rng.choice(np.arange(2048, T - 64), 448,
                                                replace=False)])).astype(np.int32)
    ri = torch.from_numpy(rows.astype(np.int64)).to(dev)
    gout = out[0].index_select(0, ri).cpu().numpy()
    gidx = idx[0].index_select(0, ri).cpu().numpy()
    qrows = d["q"][0].index_select(0, ri).cpu().view(torch.int16).numpy().view(np.uint16)
    host = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
    k, v = host(d["k"]), host(d["v"])
    del d, out, idx
    torch.cuda.empty_cache()
    q = np.zeros((B, T, H, D), dtype=np.uint16)  # only the checked rows are read (and touched)
    q[0, rows] = qrows
    print("moba 10M: GPU done, oracle on %d rows" % len(rows), flush=True)
    check_moba(cfg, dict(q=q, k=k, v=v), np.zeros_like(rows), rows, gout, gidx, "moba 10M")


def test_moba_head_passes_two_sequences():
    """B = 2, T = 2^22, H = 3 (D = 64): more than 2^24 query rows, so the heads run in passes of
    2 and 1, with each sequence's values transposed per pass.  Sampled rows of both sequences:
    the first 2 blocks, the last 64 and a seeded random remainder."""
    import dynamic_block_sparse_fwd_amd as nsa
    nsa.load_library()
    B, T, H, D = 2, 1 << 22, 3, 64
    print("case moba head passes", flush=True)
    cfg = O.MobaCfg(B, T, H, D, block=512, top_k=3)
    c = nsa.MobaConfig(B, T, H, D, 512, 3, cfg.scale)
    dev = torch.device("cuda")
    d = {"q": S.normal_bf16_device(11, "q", (B, T, H, D), dev),
         "k": S.normal_bf16_device(11, "k", (B, H, T, D), dev),
         "v": S.normal_bf16_device(11, "v", (B, H, T, D), dev)}
    out, idx = nsa.moba_prefill(c, d["q"], d["k"], d["v"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rt1 = np.unique(np.concatenate([np.arange(1024), np.arange(T - 64, T),
                                    rng.choice(np.arange(1024, T - 64), 256, replace=False)]))
    rb = np.repeat(np.arange(B), len(rt1)).astype(np.int32)
    rt = np.tile(rt1, B).astype(np.int32)
    flat = torch.from_numpy((rb.astype(np.int64) * T + rt)).to(dev)
    gout = out.view(B * T, H, D).index_select(0, flat).cpu().numpy()
    gidx = idx.view(B * T, H, -1).index_select(0, flat).cpu().numpy()
    host = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
    x = {n: host(t) for n, t in d.items()}
    del d, out, idx
    torch.cuda.empty_cache()
    check_moba(cfg, x, rb, rt, gout, gidx, "moba head passes")


def scaled_bits(bits, e):
    """bf16 bit patterns times 2**e, exactly (a power of two moves only the exponent, which
    stays in range here)."""
    f = S.bf16_bits_to_f32(bits).astype(np.float64) * (2.0 ** e)
    return S.f32_to_bf16_bits(f.astype(np.float32))


@pytest.mark.parametrize("e", [20, -20])
def test_moba_value_range(e):
    """Values far outside fp16's range (x 2^20: up to ~4e6) or deep below its normal range
    (x 2^-20: ~1e-6): the partial outputs the block-major kernel stores in fp16 carry a
    power-of-two scale, so the output equals 2^e times the unscaled oracle output."""
    B, T, H, D, block, top_k = 1, 2048, 2, 128, 256, 3
    cfg = O.MobaCfg(B, T, H, D, block=block, top_k=top_k)
    x = S.moba_inputs(77, B, T, H, D)
    xs = dict(x, v=scaled_bits(x["v"], e))
    gout, gidx = gpu_moba(cfg, xs)
    assert np.isfinite(gout).all()
    rb, rt = np.zeros(T, np.int32), np.arange(T, dtype=np.int32)
    check_moba(cfg, x, rb, rt, gout[rb, rt] * (2.0 ** -e), gidx[rb, rt], "moba v x 2^%d" % e)


def test_moba_deterministic():
    """Two calls on the same inputs give the same output and indices bit for bit: the block
    lists are filled in an order that LDS atomics decide, but each (query, slot) partial is
    computed on its own and the partials are merged in slot order."""
    B, T, H, D = 2, 8192, 4, 128
    cfg = O.MobaCfg(B, T, H, D, block=512, top_k=3)
    x = S.moba_inputs(78, B, T, H, D)
    out1, idx1 = gpu_moba(cfg, x)
    out2, idx2 = gpu_moba(cfg, x)
    np.testing.assert_array_equal(idx1, idx2)
    assert np.array_equal(out1.view(np.uint32), out2.view(np.uint32))
