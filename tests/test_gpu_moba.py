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
    kbar = O.moba_pool(cfg, x["k"])
    ora = O.moba_prefill_rows(cfg, x["q"], x["k"], x["v"], rows_b, rows_t, kbar=kbar,
                              want_scores=True)
    qf = S.bf16_bits_to_f32(x["q"]).astype(np.float64)[rows_b, rows_t]  # [R, H, D]
    qn = np.linalg.norm(qf, axis=-1)
    kn = np.linalg.norm(kbar, axis=-1)  # [B, H, nb]
    den = np.zeros_like(qn)
    for r, (b, t) in enumerate(zip(rows_b, rows_t)):
        bq = t // cfg.block
        if bq > 0:
            den[r] = qn[r] * kn[b, :, :bq].max(axis=-1)
    gi = gidx[rows_b, rows_t]
    rerun, acc = check_moba_idx(gi, ora, rows_t, cfg.block, cfg.top_k, den)
    ref = ora["out"].copy()
    if rerun:
        rr = np.array(rerun)
        ref[rr] = O.moba_prefill_rows(cfg, x["q"], x["k"], x["v"], rows_b[rr], rows_t[rr],
                                      kbar=kbar, idx_in=gi[rr])["out"]
    mx, mean = check_close(gout[rows_b, rows_t], ref, what)
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
    check_moba(cfg, x, b.ravel().astype(np.int32), t.ravel().astype(np.int32), gout, gidx, name)


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
    check_moba(cfg, x, np.zeros_like(rows), rows, gout, gidx, "moba 128k")


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
    check_moba(cfg, x, np.zeros_like(rows), rows, gout, gidx, "moba 1M")


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
    check_moba(cfg, x, rb, rt, gout * (2.0 ** -e), gidx, "moba v x 2^%d" % e)
