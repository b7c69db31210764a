"""GPU parity of nsa_prefill (through the C ABI) against the fp64 oracle on the same seeded
inputs: selected indices bit-exact (near-tie rule), outputs within 1e-2 max / 1e-3 mean."""
import zlib

import numpy as np
import pytest

import oracle as O
import synth_inputs as S
from tests.parity import check_close, check_nsa_idx

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _nsa():
    import dynamic_block_sparse_fwd_amd as nsa
    nsa.load_library()
    return nsa


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gpu_prefill(cfg, x):
    nsa = _nsa()
    c = nsa.NsaConfig(cfg.B, cfg.T, cfg.Hkv, cfg.G, cfg.D, cfg.cmp_len, cfg.cmp_stride,
                      cfg.sel_block, cfg.top_n, cfg.n_local, cfg.window, cfg.scale,
                      cfg.top_p)
    d = {k: to_dev(v) for k, v in x.items()}
    out, idx = nsa.nsa_prefill(c, d["q"], d["k"], d["v"], d["wk"], d["wv"], d["gate"])
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


def compare_prefill(cfg, x, rows_b, rows_t, gout, gidx, what):
    kc = O.compress(x["k"], x["wk"], cfg.cmp_len, cfg.cmp_stride)
    vc = O.compress(x["v"], x["wv"], cfg.cmp_len, cfg.cmp_stride)
    ora = O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], rows_b, rows_t,
                             want_scores=True)
    gi = gidx[rows_b, rows_t]
    rerun, accepted = check_nsa_idx(gi, ora, rows_t, cfg.sel_block, cfg.top_n, cfg.n_local,
                                    cfg.top_p)
    ref = ora["out"].copy()
    if rerun:
        rr = np.array(rerun)
        ora2 = O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], rows_b[rr],
                                  rows_t[rr], idx_in=gi[rr])
        ref[rr] = ora2["out"]
    mx, mean = check_close(gout[rows_b, rows_t], ref, what)
    print("%s: rows=%d max-abs %.2e mean-abs %.2e near-ties accepted %d" % (
        what, len(rows_t), mx, mean, accepted), flush=True)


def all_rows(cfg):
    b, t = np.meshgrid(np.arange(cfg.B), np.arange(cfg.T), indexing="ij")
    return b.ravel().astype(np.int32), t.ravel().astype(np.int32)


CASES = [
    # name, B, T, Hkv, G, D, extra
    ("tiny_prefill_T2048_G4_D64", 1, 2048, 1, 4, 64, {}),  # the tiny workload, every row
    ("ragged_G16_D128", 2, 777, 2, 16, 128, {}),
    ("G8_D128_T1500", 1, 1500, 2, 8, 128, {}),
    ("G2_D64_top5", 1, 1100, 3, 2, 64, dict(top_n=5, n_local=1)),
    ("G1_D64_nolocal", 2, 700, 2, 1, 64, dict(top_n=4, n_local=0, window=100)),
    ("G16_D64_block128", 1, 1300, 1, 16, 64, dict(sel_block=128, top_n=6, window=200)),
    # adaptive top-p: the number of blocks taken varies from the forced three to the cap
    ("topp0.3_G4_D64", 1, 2048, 1, 4, 64, dict(top_p=0.3)),
    ("topp0.5_G16_D128", 2, 1300, 2, 16, 128, dict(top_p=0.5)),
    ("topp0.9_G8_D128", 1, 1500, 2, 8, 128, dict(top_p=0.9)),
    ("topp0.5_G2_D64_block128", 1, 1500, 2, 2, 64, dict(top_p=0.5, sel_block=128, top_n=6,
                                                        window=200)),
    ("topp1_G1_D64_nolocal", 2, 700, 2, 1, 64, dict(top_p=1.0, top_n=4, n_local=0, window=100)),
    # p below any forced mass: only block 0 and the local blocks are kept
    ("topp_tiny_G4_D128", 1, 1300, 2, 4, 128, dict(top_p=1e-6)),
    # other compression geometries (the generic importance path): l = d, l = 3 d, and l = 2 d
    # with a selection block of only two strides
    ("cmp16x16_G4_D64", 1, 1500, 2, 4, 64, dict(cmp_len=16, cmp_stride=16)),
    ("cmp48x16_G16_D128", 1, 1300, 1, 16, 128, dict(cmp_len=48, cmp_stride=16)),
    ("cmp64x32_G8_D64", 1, 2100, 2, 8, 64, dict(cmp_len=64, cmp_stride=32)),
]


@pytest.mark.parametrize("name,B,T,Hkv,G,D,extra", CASES, ids=[c[0] for c in CASES])
def test_prefill_parity_all_rows(name, B, T, Hkv, G, D, extra):
    print("case", name, flush=True)
    cfg = O.NsaCfg(B, T, Hkv, G, D, **extra)
    seed = 1 if name == CASES[0][0] else zlib.crc32(name.encode()) % 1000 + 10
    x = S.nsa_prefill_inputs(seed, B, T, Hkv, G, D, l=cfg.cmp_len)
    gout, gidx = run_gpu_prefill(cfg, x)
    rb, rt = all_rows(cfg)
    compare_prefill(cfg, x, rb, rt, gout, gidx, name)


@pytest.mark.parametrize("T", [1, 31, 32, 33, 64, 65, 130])
def test_prefill_short_sequences(T):
    """Edge cases: no compressed token yet (T < 32), exactly one, a single block."""
    cfg = O.NsaCfg(1, T, 2, 4, 64)
    x = S.nsa_prefill_inputs(100 + T, 1, T, 2, 4, 64)
    gout, gidx = run_gpu_prefill(cfg, x)
    rb, rt = all_rows(cfg)
    compare_prefill(cfg, x, rb, rt, gout, gidx, "T=%d" % T)


def test_prefill_branches_one_hot_gates():
    """Gate = e_k isolates branch k: compare each branch output separately."""
    cfg = O.NsaCfg(1, 1000, 2, 16, 128)
    x = S.nsa_prefill_inputs(7, 1, 1000, 2, 16, 128)
    kc = O.compress(x["k"], x["wk"], 32, 16)
    vc = O.compress(x["v"], x["wv"], 32, 16)
    rb, rt = all_rows(cfg)
    ora = O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], rb, rt,
                             branches=True, want_scores=True)
    for kb, nm in enumerate(("o_cmp", "o_slc", "o_win")):
        x2 = dict(x)
        g = np.zeros_like(x["gate"])
        g[..., kb] = 1.0
        x2["gate"] = g
        gout, gidx = run_gpu_prefill(cfg, x2)
        if nm == "o_slc":
            rerun, _ = check_nsa_idx(gidx[rb, rt], ora, rt, 64, 16, 2)
            assert not rerun
        check_close(gout[0], ora[nm], nm)


def test_prefill_zero_query_ties_bit_exact():
    """Q = 0 makes every full block tie; the GPU must break ties toward the lower index
    exactly like the oracle (no near-tie allowance needed: the scores tie exactly)."""
    cfg = O.NsaCfg(1, 2048, 1, 16, 64)
    x = S.nsa_prefill_inputs(8, 1, 2048, 1, 16, 64)
    x["q"] = np.zeros_like(x["q"])
    gout, gidx = run_gpu_prefill(cfg, x)
    rb, rt = all_rows(cfg)
    kc = O.compress(x["k"], x["wk"], 32, 16)
    vc = O.compress(x["v"], x["wv"], 32, 16)
    ora = O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], rb, rt)
    np.testing.assert_array_equal(gidx[0], ora["idx"])
    check_close(gout[0], ora["out"], "zero-q")


@pytest.mark.parametrize("G,D", [(16, 128), (4, 64)])
def test_prefill_loose_score_bound(G, D):
    """Keys 512 .. 639 scaled by 16 (exact in bf16): a query tile that sees their compressed
    tokens bounds its scores by |q| times their norm, more than 60 (log2 units) above its actual
    maximum, so the compressed attention's first pass takes its running-maximum form there,
    while the tiles before them keep the bounded form.  Every row against the oracle."""
    T = 1500
    print("case loose bound G%d D%d" % (G, D), flush=True)
    cfg = O.NsaCfg(1, T, 2, G, D)
    x = S.nsa_prefill_inputs(21 + G, 1, T, 2, G, D)
    k = S.bf16_bits_to_f32(x["k"]).astype(np.float64)
    k[:, :, 512:640] *= 16.0
    x["k"] = S.f32_to_bf16_bits(k.astype(np.float32))
    gout, gidx = run_gpu_prefill(cfg, x)
    rb, rt = all_rows(cfg)
    compare_prefill(cfg, x, rb, rt, gout, gidx, "loose bound G%d D%d" % (G, D))


def test_prefill_deterministic():
    cfg = O.NsaCfg(1, 3000, 2, 16, 128)
    x = S.nsa_prefill_inputs(9, 1, 3000, 2, 16, 128)
    o1, i1 = run_gpu_prefill(cfg, x)
    o2, i2 = run_gpu_prefill(cfg, x)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_array_equal(o1, o2)


def test_prefill_64k_sampled_rows():
    """The 64k prefill workload (B=1, T=65536, 4 KV heads x group 16, D=128), run exactly as
    bench.py runs it; checked on 4096 positions: all t < 1024 (every visible block selected),
    the last 64, and a seeded random remainder."""
    B, T, Hkv, G, D = 1, 65536, 4, 16, 128
    cfg = O.NsaCfg(B, T, Hkv, G, D)
    x = S.nsa_prefill_inputs(2, B, T, Hkv, G, D)
    gout, gidx = run_gpu_prefill(cfg, x)
    rng = np.random.default_rng(2)
    rest = rng.choice(np.arange(1024, T - 64), 4096 - 1024 - 64, replace=False)
    rt = np.unique(np.concatenate([np.arange(1024), np.arange(T - 64, T), rest])).astype(np.int32)
    compare_prefill(cfg, x, np.zeros_like(rt), rt, gout, gidx, "prefill 64k")


DIAG_CASES = [
    # name, B, T, Hkv, G, D, extra
    ("G4_D64", 1, 2048, 1, 4, 64, {}),
    ("G16_D128_B2", 2, 1500, 2, 16, 128, {}),
    ("G1_D64_cmp48x16", 1, 1800, 2, 1, 64, dict(cmp_len=48, cmp_stride=16)),
    ("G8_D128_block128", 1, 2100, 1, 8, 128, dict(sel_block=128, top_n=6)),
]


def check_diag(cfg, x, rb, rt, glse, gsc, what):
    """lse within 1e-5 relative (absolute below 1), block scores within 1e-5 of the group's
    total importance G, on rows (rb, rt)."""
    kc = O.compress(x["k"], x["wk"], cfg.cmp_len, cfg.cmp_stride)
    vc = O.compress(x["v"], x["wv"], cfg.cmp_len, cfg.cmp_stride)
    ora = O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], rb, rt,
                             branches=True, want_scores=True)
    ol, os_ = ora["lse"], ora["scores"]
    none = np.isneginf(ol)
    assert np.array_equal(np.isneginf(glse), none), "%s: rows without a visible token" % what
    el = np.abs(glse[~none] - ol[~none]) / np.maximum(1.0, np.abs(ol[~none]))
    es = np.abs(gsc - os_)
    assert el.max(initial=0.0) <= 1e-5, "%s: lse rel err %.3g" % (what, el.max())
    assert es.max() <= 1e-5 * cfg.G, "%s: block score err %.3g" % (what, es.max())
    print("%s: %d rows, lse max rel err %.2e, block score max err %.2e (G = %d)" % (
        what, len(rt), el.max(initial=0.0), es.max(), cfg.G), flush=True)


@pytest.mark.parametrize("name,B,T,Hkv,G,D,extra", DIAG_CASES, ids=[c[0] for c in DIAG_CASES])
def test_prefill_diagnostics_lse_and_scores(name, B, T, Hkv, G, D, extra):
    """The compressed branch's log-sum-exp and the group block scores the selection ranks,
    exported by nsa_prefill_diag, against the oracle's on every row; the output and indices
    equal nsa_prefill's bit for bit."""
    nsa = _nsa()
    print("case diag", name, flush=True)
    cfg = O.NsaCfg(B, T, Hkv, G, D, **extra)
    x = S.nsa_prefill_inputs(60 + len(name), B, T, Hkv, G, D, l=cfg.cmp_len)
    c = nsa.NsaConfig(B, T, Hkv, G, D, cfg.cmp_len, cfg.cmp_stride, cfg.sel_block, cfg.top_n,
                      cfg.n_local, cfg.window, cfg.scale, cfg.top_p)
    d = {k: to_dev(v) for k, v in x.items()}
    out, idx, lse, sc = nsa.nsa_prefill_diag(c, d["q"], d["k"], d["v"], d["wk"], d["wv"],
                                              d["gate"])
    out2, idx2 = nsa.nsa_prefill(c, d["q"], d["k"], d["v"], d["wk"], d["wv"], d["gate"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(idx, idx2)
    b, t = np.meshgrid(np.arange(B), np.arange(T), indexing="ij")
    rb, rt = b.ravel().astype(np.int32), t.ravel().astype(np.int32)
    check_diag(cfg, x, rb, rt, lse.cpu().numpy()[rb, rt], sc.cpu().numpy()[rb, rt], name)


def test_prefill_diagnostics_64k_sampled_rows():
    """The 64k prefill workload's lse and block scores on 1024 sampled rows."""
    nsa = _nsa()
    B, T, Hkv, G, D = 1, 65536, 4, 16, 128
    cfg = O.NsaCfg(B, T, Hkv, G, D)
    x = S.nsa_prefill_inputs(2, B, T, Hkv, G, D)
    c = nsa.NsaConfig(B, T, Hkv, G, D)
    d = {k: to_dev(v) for k, v in x.items()}
    _, _, lse, sc = nsa.nsa_prefill_diag(c, d["q"], d["k"], d["v"], d["wk"], d["wv"], d["gate"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rt = np.unique(np.concatenate([np.arange(48), rng.choice(np.arange(48, T), 976,
                                                             replace=False)])).astype(np.int32)
    ri = torch.from_numpy(rt.astype(np.int64)).cuda()
    glse = lse[0].index_select(0, ri).cpu().numpy()
    gsc = sc[0].index_select(0, ri).cpu().numpy()
    del d, lse, sc
    check_diag(cfg, x, np.zeros_like(rt), rt, glse, gsc, "diag 64k")


STREAM_CASES = [
    # name, T, Hkv, G, D, extra: more selection blocks than a query tile's block scores can
    # keep in LDS (64 KB / 4 bytes / positions per tile: 2048 blocks for G >= 4, 1024 for
    # G = 1), so the selection streams
    ("G16_T140000_D128", 140000, 1, 16, 128, {}),
    ("G16_T140000_D64_topp0.5", 140000, 1, 16, 64, dict(top_p=0.5)),
    ("G1_T70000_Hkv2_D64", 70000, 2, 1, 64, {}),
    ("G4_T140000_cmp48x16_D64", 140000, 1, 4, 64, dict(cmp_len=48, cmp_stride=16)),
    ("G8_T140000_cmp64x32_topp0.3", 140000, 1, 8, 128,
     dict(cmp_len=64, cmp_stride=32, top_p=0.3)),
]


@pytest.mark.parametrize("name,T,Hkv,G,D,extra", STREAM_CASES, ids=[c[0] for c in STREAM_CASES])
def test_prefill_streaming_selection(name, T, Hkv, G, D, extra):
    """Long sequences: the top list of every position is built while the compressed keys are
    walked; checked on the first 64 positions, the positions around block edges where the
    forced set moves, a seeded random sample and the last 64."""
    print("case stream", name, flush=True)
    cfg = O.NsaCfg(1, T, Hkv, G, D, **extra)
    x = S.nsa_prefill_inputs(50 + len(name), 1, T, Hkv, G, D, l=cfg.cmp_len)
    gout, gidx = run_gpu_prefill(cfg, x)
    rng = np.random.default_rng(len(name))
    edges = np.array([1023, 1024, 1087, 4095, 4096, 65535, 65536, 65600, 131071, 131072])
    rt = np.unique(np.concatenate([np.arange(64), edges[edges < T],
                                   rng.choice(np.arange(64, T - 64), 240, replace=False),
                                   np.arange(T - 64, T)])).astype(np.int32)
    compare_prefill(cfg, x, np.zeros_like(rt), rt, gout, gidx, name)


def _stage_inputs(cfg, x):
    nsa = _nsa()
    c = nsa.NsaConfig(cfg.B, cfg.T, cfg.Hkv, cfg.G, cfg.D, cfg.cmp_len, cfg.cmp_stride,
                      cfg.sel_block, cfg.top_n, cfg.n_local, cfg.window, cfg.scale)
    return nsa, c, {k: to_dev(v) for k, v in x.items()}


def test_prefill_stages_compose_bit_exact():
    """nsa_prefill_stages runs the same kernels: all stages at once equal nsa_prefill bit for
    bit; the three stages run separately (the window then in its own kernel, not fused into the
    compressed one) add up to it within the bf16 rounding of the probabilities that feed the
    matrix core."""
    cfg = O.NsaCfg(2, 1300, 2, 16, 128)
    x = S.nsa_prefill_inputs(11, 2, 1300, 2, 16, 128)
    nsa, c, d = _stage_inputs(cfg, x)
    full, fidx = nsa.nsa_prefill(c, d["q"], d["k"], d["v"], d["wk"], d["wv"], d["gate"])
    allst, aidx = nsa.nsa_prefill_stages(c, nsa.STAGE_ALL, d["q"], d["k"], d["v"], d["wk"],
                                         d["wv"], d["gate"])
    o_c, cidx = nsa.nsa_prefill_stages(c, nsa.STAGE_CMP_SELECT, d["q"], d["k"], d["v"], d["wk"],
                                       d["wv"], d["gate"])
    o_w, _ = nsa.nsa_prefill_stages(c, nsa.STAGE_WINDOW, d["q"], d["k"], d["v"], None, None,
                                    d["gate"])
    o_s, _ = nsa.nsa_prefill_stages(c, nsa.STAGE_SELECTED, d["q"], d["k"], d["v"], None, None,
                                    d["gate"], sel_idx=cidx)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(allst.cpu().numpy(), full.cpu().numpy())
    np.testing.assert_array_equal(aidx.cpu().numpy(), fidx.cpu().numpy())
    np.testing.assert_array_equal(cidx.cpu().numpy(), fidx.cpu().numpy())
    summed = (o_c + o_w) + o_s
    np.testing.assert_allclose(summed.cpu().numpy(), full.cpu().numpy(), rtol=0, atol=2e-3)


def test_prefill_window_and_selected_stages_against_oracle():
    """Window stage = g2 * o_win; selected stage with the ORACLE's indices (no near-tie
    question) = g1 * o_slc; then the same with an index list holding -1 holes in the middle,
    an out-of-range block and a repeated block, which the oracle treats identically."""
    cfg = O.NsaCfg(1, 1500, 2, 8, 128, top_n=6, n_local=1, window=300)
    x = S.nsa_prefill_inputs(12, 1, 1500, 2, 8, 128)
    kc = O.compress(x["k"], x["wk"], 32, 16)
    vc = O.compress(x["v"], x["wv"], 32, 16)
    rb, rt = all_rows(cfg)
    ora = O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], rb, rt,
                             branches=True)
    nsa, c, d = _stage_inputs(cfg, x)
    g = x["gate"][0]
    o_w, _ = nsa.nsa_prefill_stages(c, nsa.STAGE_WINDOW, d["q"], d["k"], d["v"], None, None,
                                    d["gate"])
    check_close(o_w.cpu().numpy()[0], g[..., 2:3] * ora["o_win"], "window stage")
    idx = ora["idx"].reshape(1, cfg.T, cfg.Hkv, cfg.top_n).astype(np.int32)
    o_s, _ = nsa.nsa_prefill_stages(c, nsa.STAGE_SELECTED, d["q"], d["k"], d["v"], None, None,
                                    d["gate"], sel_idx=to_dev(idx))
    check_close(o_s.cpu().numpy()[0], g[..., 1:2] * ora["o_slc"], "selected stage")
    # holes, an out-of-range block and a repeat
    rng = np.random.default_rng(12)
    idx2 = idx.copy()
    holes = rng.random(idx2.shape) < 0.2
    idx2[holes] = -1
    idx2[..., 0] = np.where(rng.random(idx2.shape[:-1]) < 0.1, cfg.nblk + 3, idx2[..., 0])
    idx2[..., 1] = np.where(rng.random(idx2.shape[:-1]) < 0.1, idx2[..., 2], idx2[..., 1])
    ora2 = O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], rb, rt,
                              idx_in=idx2[0], branches=True)
    o_s2, _ = nsa.nsa_prefill_stages(c, nsa.STAGE_SELECTED, d["q"], d["k"], d["v"], None, None,
                                     d["gate"], sel_idx=to_dev(idx2))
    check_close(o_s2.cpu().numpy()[0], g[..., 1:2] * ora2["o_slc"], "selected stage, holes")


@pytest.mark.parametrize("e", [20, -20])
def test_prefill_value_range(e):
    """Values far outside fp16's range (x 2^20) or deep below its normal range (x 2^-20): the
    selected branch's block-major partials are stored in fp16 with a power-of-two scale per
    head, so every branch (compression is linear and the scaling exact) and the output equal
    2^e times the unscaled run, whose oracle output they are compared with."""
    B, T, Hkv, G, D = 1, 2048, 2, 16, 128
    cfg = O.NsaCfg(B, T, Hkv, G, D)
    x = S.nsa_prefill_inputs(78, B, T, Hkv, G, D)
    f = S.bf16_bits_to_f32(x["v"]).astype(np.float64) * (2.0 ** e)
    xs = dict(x, v=S.f32_to_bf16_bits(f.astype(np.float32)))
    gout, gidx = run_gpu_prefill(cfg, xs)
    assert np.isfinite(gout).all()
    rb, rt = all_rows(cfg)
    compare_prefill(cfg, x, rb, rt, gout * (2.0 ** -e), gidx, "prefill v x 2^%d" % e)
