"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics (CPU only).

Each pin reaches the oracle's result through a different route than the oracle itself:
a library routine on a special case (torch SDPA, numpy mean), a closed form derived by hand,
a token-level expansion, a brute-force enumeration, or an invariant (causality, linearity,
mass conservation).  A dropped term, a wrong sign or index, or a transposed operand in the
oracle fails at least one of them.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle as O
import synth_inputs as S

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def f64(bits):
    return S.bf16_bits_to_f32(bits).astype(np.float64)


def bf16_round_f64(x):
    """Independent fp64 -> bf16 (nearest, ties to even) by integer manipulation of the fp64
    bit pattern.  Normal-range values only."""
    x = np.asarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    sign = (u >> np.uint64(63)).astype(np.uint32)
    mag = u & np.uint64(0x7FFFFFFFFFFFFFFF)
    # keep 1 + 7 significand bits: drop the low 45 bits of the 52-bit fraction
    drop = np.uint64(45)
    low = mag & ((np.uint64(1) << drop) - np.uint64(1))
    half = np.uint64(1) << (drop - np.uint64(1))
    kept = mag >> drop
    up = (low > half) | ((low == half) & ((kept & np.uint64(1)) == np.uint64(1)))
    kept = kept + up.astype(np.uint64)
    # kept now holds the fp64 exponent (11 bits) and 7 fraction bits; rebias 1023 -> 127
    exp64 = (kept >> np.uint64(7)).astype(np.int64)
    frac = (kept & np.uint64(0x7F)).astype(np.uint32)
    exp32 = exp64 - 1023 + 127
    out = (sign << 15) | (exp32.astype(np.uint32) << 7) | frac
    out = np.where(x == 0, sign << 15, out)
    return out.astype(np.uint16)


def sdpa_causal(q, k, v, scale=None):
    """q [T,H,D], k/v [T,H,D] fp64 -> causal attention output [T,H,D] via torch (fp64 CPU)."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.numpy().transpose(1, 0, 2)


def small_nsa(seed=11, T=256, Hkv=2, G=4, D=32, **kw):
    cfg = O.NsaCfg(1, T, Hkv, G, D, **kw)
    x = S.nsa_prefill_inputs(seed, 1, T, Hkv, G, D, l=cfg.cmp_len)
    return cfg, x


def run_rows(cfg, x, rows=None, wk=None, wv=None, **kw):
    wk = x["wk"] if wk is None else wk
    wv = x["wv"] if wv is None else wv
    kc = O.compress(x["k"], wk, cfg.cmp_len, cfg.cmp_stride)
    vc = O.compress(x["v"], wv, cfg.cmp_len, cfg.cmp_stride)
    if rows is None:
        rows = np.arange(cfg.T)
    return O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"],
                              np.zeros(len(rows), np.int32), rows, **kw)


# ---------------------------------------------------------------- compression (branch 1 input)

def test_compress_mean_pool_is_numpy_mean():
    """W[j] = I/l turns the linear compressor into the block mean (numpy), rounded once."""
    T, D, l, d = 300, 64, 32, 16
    k = S.normal_bf16(3, "k", (1, 2, T, D))
    bits, ex = O.compress(k, S.mean_pool_weights(l, D), l, d, exact=True)
    kf = f64(k)
    n = O.n_cmp(T, l, d)
    ref = np.stack([kf[:, :, i * d:i * d + l].mean(axis=2) for i in range(n)], axis=2)
    np.testing.assert_allclose(ex, ref, rtol=0, atol=1e-15)
    assert np.array_equal(bits, bf16_round_f64(ref))


def test_compress_single_weight_picks_one_element():
    """W with a single 1 at (j0, a, c0): Kc[i, c0] = K[i*d + j0, a], every other column 0.
    Fails on a transposed W, a wrong stride or a wrong in-block offset."""
    T, D, l, d = 200, 16, 32, 16
    k = S.normal_bf16(4, "k", (1, 1, T, D))
    kf = f64(k)[0, 0]
    for (j0, a, c0) in [(0, 0, 0), (5, 3, 11), (31, 15, 2), (17, 9, 9)]:
        w = np.zeros((l, D, D), dtype=np.float32)
        w[j0, a, c0] = 1.0
        bits = O.compress(k, S.f32_to_bf16_bits(w), l, d)[0, 0]
        got = f64(bits)
        n = O.n_cmp(T, l, d)
        assert got.shape == (n, D)
        np.testing.assert_array_equal(got[:, c0], kf[np.arange(n) * d + j0, a])
        mask = np.ones(D, bool)
        mask[c0] = False
        assert not got[:, mask].any()


def test_compress_identity_and_rounding():
    """l = d = 1 with W = I reproduces K bit for bit; a 3-term sum rounds like an independent
    integer-based round-to-nearest-even."""
    T, D = 40, 8
    k = S.normal_bf16(5, "k", (1, 1, T, D))
    eye = S.f32_to_bf16_bits(np.eye(D, dtype=np.float32)[None])
    assert np.array_equal(O.compress(k, eye, 1, 1), k)
    w = np.zeros((3, D, D), dtype=np.float32)
    for j in range(3):
        w[j] = np.eye(D) * [1.0, 0.5, 0.25][j]
    bits, ex = O.compress(k, S.f32_to_bf16_bits(w), 3, 1, exact=True)
    assert np.array_equal(bits, bf16_round_f64(ex))


def test_compress_linear_before_rounding():
    T, D, l, d = 96, 16, 32, 16
    k = S.normal_bf16(6, "k", (1, 1, T, D))
    w1 = S.normal_bf16(7, "wk", (l, D, D), std=0.05)
    w2 = S.normal_bf16(8, "wk", (l, D, D), std=0.05)
    w12 = S.f32_to_bf16_bits(S.bf16_bits_to_f32(w1) * 2)  # exact doubling
    _, e1 = O.compress(k, w1, l, d, exact=True)
    _, e12 = O.compress(k, w12, l, d, exact=True)
    np.testing.assert_allclose(e12, 2 * e1, rtol=1e-14, atol=1e-14)
    _, e2 = O.compress(k, w2, l, d, exact=True)
    _, es = O.compress(k, S.f32_to_bf16_bits(S.bf16_bits_to_f32(w1) + S.bf16_bits_to_f32(w2)),
                       l, d, exact=True)
    ws = S.bf16_bits_to_f32(w1).astype(np.float64) + S.bf16_bits_to_f32(w2)
    if np.array_equal(S.bf16_bits_to_f32(S.f32_to_bf16_bits(ws.astype(np.float32))), ws):
        np.testing.assert_allclose(es, e1 + e2, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- branches vs full attention

def gqa_expand(kv, G):
    """[1,Hkv,T,D] -> [T, Hkv*G, D] with head h reading KV head h // G."""
    a = kv[0].transpose(1, 0, 2)
    return np.repeat(a, G, axis=1)


def test_selected_branch_is_full_attention_when_top_n_covers_all():
    cfg, x = small_nsa(T=256, top_n=16)  # 4 blocks <= 16
    r = run_rows(cfg, x, branches=True)
    ref = sdpa_causal(f64(x["q"][0]), gqa_expand(f64(x["k"]), cfg.G), gqa_expand(f64(x["v"]), cfg.G))
    np.testing.assert_allclose(r["o_slc"], ref, rtol=0, atol=1e-12)
    assert (r["idx"][:, :, 0] == 0).all()


def test_window_branch_is_full_attention_when_window_covers_all():
    cfg, x = small_nsa(T=200, window=4096)
    r = run_rows(cfg, x, branches=True)
    ref = sdpa_causal(f64(x["q"][0]), gqa_expand(f64(x["k"]), cfg.G), gqa_expand(f64(x["v"]), cfg.G))
    np.testing.assert_allclose(r["o_win"], ref, rtol=0, atol=1e-12)


def test_window_of_one_returns_own_value():
    cfg, x = small_nsa(T=130, window=1)
    r = run_rows(cfg, x, branches=True)
    vf = gqa_expand(f64(x["v"]), cfg.G)
    np.testing.assert_allclose(r["o_win"], vf, rtol=0, atol=1e-15)


def test_window_is_a_band_of_w_tokens():
    """Window w vs full attention restricted by an explicit band mask (SDPA with attn_mask)."""
    cfg, x = small_nsa(T=160, window=37, D=16)
    r = run_rows(cfg, x, branches=True)
    q = f64(x["q"][0]).transpose(1, 0, 2)
    k = gqa_expand(f64(x["k"]), cfg.G).transpose(1, 0, 2)
    v = gqa_expand(f64(x["v"]), cfg.G).transpose(1, 0, 2)
    t = np.arange(cfg.T)
    band = (t[None, :] <= t[:, None]) & (t[None, :] > t[:, None] - 37)
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(band)).numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(r["o_win"], o, rtol=0, atol=1e-12)


def test_compressed_branch_is_full_attention_for_unit_blocks():
    """l = d = 1, W = I: every token is its own compressed token, visible once s <= t."""
    cfg, x = small_nsa(T=96, cmp_len=1, cmp_stride=1, D=16)
    eye = S.f32_to_bf16_bits(np.eye(cfg.D, dtype=np.float32)[None])
    r = run_rows(cfg, x, wk=eye, wv=eye, branches=True)
    ref = sdpa_causal(f64(x["q"][0]), gqa_expand(f64(x["k"]), cfg.G), gqa_expand(f64(x["v"]), cfg.G))
    np.testing.assert_allclose(r["o_cmp"], ref, rtol=0, atol=1e-12)


def test_branch_rows_sum_to_one():
    """V = 1 everywhere (and a mean-pool Wv, so Vc = 1): each branch returns exactly 1 once it
    has keys, i.e. every softmax row sums to one.  Rows with no visible compressed token give 0."""
    cfg, x = small_nsa(T=300, D=16)
    x = dict(x)
    x["v"] = S.f32_to_bf16_bits(np.ones(x["v"].shape, np.float32))
    r = run_rows(cfg, x, wv=S.mean_pool_weights(cfg.cmp_len, cfg.D), branches=True)
    np.testing.assert_allclose(r["o_slc"], 1.0, atol=1e-13)
    np.testing.assert_allclose(r["o_win"], 1.0, atol=1e-13)
    t = np.arange(cfg.T)
    vis = t >= cfg.cmp_len - 1
    np.testing.assert_allclose(r["o_cmp"][vis], 1.0, atol=1e-13)
    assert not r["o_cmp"][~vis].any()


# ---------------------------------------------------------------- block importance and selection

def test_block_scores_equal_attention_onto_block_indicator_values():
    """Independent route to the block scores: give token s the value one-hot(block of s) and
    use a mean-pool Wv, so compressed value i is its overlap fraction with each block.  Then the
    compressed branch output of head h *is* that head's block importance, and the group sum of
    those outputs must equal the oracle's group score S[j]."""
    cfg, x = small_nsa(T=512, G=4, D=16)  # 8 blocks <= D
    x = dict(x)
    onehot = np.zeros((cfg.T, cfg.D), np.float32)
    onehot[np.arange(cfg.T), np.arange(cfg.T) // cfg.sel_block] = 1.0
    x["v"] = np.broadcast_to(S.f32_to_bf16_bits(onehot), x["v"].shape).copy()
    r = run_rows(cfg, x, wv=S.mean_pool_weights(cfg.cmp_len, cfg.D), branches=True,
                 want_scores=True)
    oc = r["o_cmp"].reshape(cfg.T, cfg.Hkv, cfg.G, cfg.D).sum(axis=2)[:, :, :cfg.nblk]
    np.testing.assert_allclose(r["scores"], oc, rtol=0, atol=1e-12)


def test_uniform_query_scores_closed_form():
    """Q = 0: every visible compressed token gets probability 1/nvis.  Counting, per token, the
    visible spans that cover it (each token is covered by l/d = 2 spans, the first 16 tokens by
    one) gives S[j] = G * sum_{s in block j} cover(s) / (l * nvis); in particular an interior
    fully covered block scores 4G/nvis and block 0 scores 3.5G/nvis (l=32, d=16, beta=64)."""
    cfg, x = small_nsa(T=1100, Hkv=1, G=4, D=16)
    x = dict(x)
    x["q"] = np.zeros_like(x["q"])
    rows = np.array([31, 47, 100, 255, 256, 700, 1099])
    r = run_rows(cfg, x, rows=rows, want_scores=True)
    l, d, beta, G = cfg.cmp_len, cfg.cmp_stride, cfg.sel_block, cfg.G
    for a, t in enumerate(rows):
        nvis = (t - l + 1) // d + 1
        cover = np.zeros(cfg.T)
        for s in range(cfg.T):
            cover[s] = sum(1 for i in range(nvis) if i * d <= s < i * d + l)
        ref = np.array([cover[j * beta:(j + 1) * beta].sum() for j in range(cfg.nblk)])
        ref = G * ref / (l * nvis)
        np.testing.assert_allclose(r["scores"][a, 0], ref, rtol=0, atol=1e-13)
        assert abs(r["scores"][a, 0].sum() - G) < 1e-12  # mass conservation
        full_end = (16 * (nvis - 1) + 32) // beta  # blocks entirely inside covered tokens
        if full_end > 2:
            assert abs(r["scores"][a, 0, 1] - 4 * G / nvis) < 1e-13
            assert abs(r["scores"][a, 0, 0] - 3.5 * G / nvis) < 1e-13


def test_uniform_query_ties_go_to_lower_index():
    """Q = 0 at t = 1099 (b = 17): the free blocks 1..14 tie at the top score; with block 0 and
    the local blocks 16, 17 forced, the 13 free picks are blocks 1..13."""
    cfg, x = small_nsa(T=1100, Hkv=1, G=4, D=16)
    x = dict(x)
    x["q"] = np.zeros_like(x["q"])
    r = run_rows(cfg, x, rows=np.array([1099]))
    assert r["idx"][0, 0].tolist() == list(range(0, 14)) + [16, 17]
    assert r["gap"][0, 0] == 0.0


def test_no_visible_compressed_token():
    cfg, x = small_nsa(T=64, Hkv=1, G=2, D=16)
    r = run_rows(cfg, x, rows=np.arange(31), branches=True, want_scores=True)
    assert not r["o_cmp"].any() and not r["scores"].any()
    assert (r["idx"][:, 0, 0] == 0).all() and (r["idx"][:, 0, 1:] == -1).all()


def brute_force_selection(S_row, b, n, n_local):
    forced = {0} | {j for j in range(b - n_local + 1, b + 1) if j >= 0}
    if b + 1 <= n:
        return list(range(b + 1))
    free = [j for j in range(b + 1) if j not in forced]
    best = None
    for comb in itertools.combinations(free, n - len(forced)):
        sc = sum(S_row[j] for j in comb)
        key = (-sc, sorted(comb))
        if best is None or key < best[0]:
            best = (key, comb)
    return sorted(forced | set(best[1]))


@pytest.mark.parametrize("n_local", [0, 1, 2])
def test_selection_matches_brute_force_enumeration(n_local):
    """Every size-n subset containing the forced blocks is enumerated; the max-sum subset with
    the lexicographically smallest index list must be the oracle's choice."""
    cfg, x = small_nsa(seed=21, T=576, Hkv=2, G=2, D=16, top_n=5, n_local=n_local)
    rows = np.array([63, 64, 300, 383, 500, 575])
    r = run_rows(cfg, x, rows=rows, want_scores=True)
    for a, t in enumerate(rows):
        b = t // cfg.sel_block
        for g in range(cfg.Hkv):
            ref = brute_force_selection(r["scores"][a, g], b, cfg.top_n, n_local)
            got = [j for j in r["idx"][a, g] if j >= 0]
            assert got == ref, (t, g, got, ref)


def test_selection_with_integer_score_ties_brute_force():
    """Integer-valued construction: Q = 0 makes blocks tie; brute force agrees on tie order."""
    cfg, x = small_nsa(seed=22, T=640, Hkv=1, G=2, D=16, top_n=4, n_local=1)
    x = dict(x)
    x["q"] = np.zeros_like(x["q"])
    rows = np.array([639, 500])
    r = run_rows(cfg, x, rows=rows, want_scores=True)
    for a, t in enumerate(rows):
        ref = brute_force_selection(r["scores"][a, 0], t // 64, 4, 1)
        assert [j for j in r["idx"][a, 0] if j >= 0] == ref


def brute_force_top_p(S_row, b, n, n_local, p):
    """Adaptive cut by enumeration: among the sets of free blocks (at most n - |forced|) whose
    importance together with the forced blocks' reaches p * M (M = total importance), the
    smallest size wins, then the largest sum, then the smallest index list; when no set
    reaches p * M, the cap-sized best set is taken."""
    forced = {0} | {j for j in range(b - n_local + 1, b + 1) if j >= 0}
    free = [j for j in range(b + 1) if j not in forced]
    M = sum(S_row[:b + 1])
    fm = sum(S_row[j] for j in forced)
    cap = min(n - len(forced), len(free))
    for size in range(cap + 1):
        best = None
        for comb in itertools.combinations(free, size):
            sc = sum(S_row[j] for j in comb)
            key = (-sc, sorted(comb))
            if best is None or key < best[0]:
                best = (key, comb)
        if fm - best[0][0] >= p * M or size == cap:
            return sorted(forced | set(best[1]))


@pytest.mark.parametrize("p", [0.3, 0.6, 0.9, 1.0])
def test_top_p_matches_brute_force_enumeration(p):
    """Top-p selection against the enumeration of every candidate set (rows with few blocks,
    so also the rows where every block would fit under the fixed rule)."""
    cfg, x = small_nsa(seed=25, T=640, Hkv=2, G=2, D=16, top_n=6, n_local=1, top_p=p)
    rows = np.array([63, 64, 200, 383, 450, 575, 639])
    r = run_rows(cfg, x, rows=rows, want_scores=True)
    for a, t in enumerate(rows):
        b = t // cfg.sel_block
        for g in range(cfg.Hkv):
            ref = brute_force_top_p(r["scores"][a, g], b, cfg.top_n, cfg.n_local, p)
            got = [j for j in r["idx"][a, g] if j >= 0]
            assert got == ref, (p, t, g, got, ref)
            assert (r["idx"][a, g, len(got):] == -1).all()


def test_top_p_one_equals_fixed_top_n_and_sets_are_nested():
    """p = 1 keeps taking blocks until the cap (every free block carries mass here), so it
    equals the fixed top-n rule on rows with more blocks than top_n; the selected sets grow
    with p; a tiny p keeps only the forced blocks."""
    cfg0, x = small_nsa(seed=26, T=2000, Hkv=2, G=4, D=16)
    rows = np.array([700, 1100, 1500, 1999])
    fixed = run_rows(cfg0, x, rows=rows, want_scores=True)
    prev = None
    for p in [1e-9, 0.2, 0.5, 0.8, 0.95, 1.0]:
        cfg = O.NsaCfg(1, cfg0.T, cfg0.Hkv, cfg0.G, cfg0.D, top_p=p)
        r = run_rows(cfg, x, rows=rows)
        sets = [[set(j for j in r["idx"][a, g] if j >= 0) for g in range(cfg.Hkv)]
                for a in range(len(rows))]
        if p == 1e-9:
            for a, t in enumerate(rows):
                b = t // 64
                for g in range(cfg.Hkv):
                    assert sets[a][g] == {0, b - 1, b}
        if p == 1.0:
            assert (fixed["scores"][:, :, :] >= 0).all()
            assert np.array_equal(r["idx"], fixed["idx"])
        if prev is not None:
            for a in range(len(rows)):
                for g in range(cfg.Hkv):
                    assert prev[a][g] <= sets[a][g], (p, a, g)
        prev = sets


def test_top_p_concentrated_attention_takes_one_free_block():
    """Compressed keys all zero except one whose span lies inside free block 5, which every
    head's query matches strongly: nearly all importance lands on block 5, so p = 0.5 takes
    exactly the forced blocks plus block 5, and the fixed rule still takes top_n blocks."""
    T, D, G = 1500, 16, 2
    cfg, x = small_nsa(seed=27, T=T, Hkv=1, G=G, D=D, top_p=0.5)
    x = dict(x)
    x["k"] = np.zeros_like(x["k"])
    # compressed token i = 21 covers tokens 336..367, inside block 5 (320..383); a mean-pool
    # compressor turns keys of value 8 on those tokens into a compressed key of 8 at i = 21
    # (its neighbours i = 20, 22 overlap it by half and get 4)
    kk = np.zeros((T, D), np.float32)
    kk[336:368, 0] = 8.0
    x["k"] = np.broadcast_to(S.f32_to_bf16_bits(kk), x["k"].shape).copy()
    q = np.zeros((T, G, D), np.float32)
    q[:, :, 0] = 8.0
    x["q"] = S.f32_to_bf16_bits(q).reshape(x["q"].shape)
    rows = np.array([1400, 1499])
    wk = S.mean_pool_weights(cfg.cmp_len, D)
    r = run_rows(cfg, x, rows=rows, wk=wk, want_scores=True)
    for a, t in enumerate(rows):
        b = t // 64
        assert r["scores"][a, 0, 5] > 0.9 * G
        assert [j for j in r["idx"][a, 0] if j >= 0] == [0, 5, b - 1, b]
    cfg_fixed = O.NsaCfg(1, T, 1, G, D)
    rf = run_rows(cfg_fixed, x, rows=rows, wk=wk)
    assert (rf["idx"] >= 0).all()


def test_head_permutation_inside_group_keeps_scores():
    cfg, x = small_nsa(seed=23, T=512, Hkv=2, G=4, D=16)
    r1 = run_rows(cfg, x, rows=np.array([511, 300]), want_scores=True)
    x2 = dict(x)
    q = x["q"].reshape(1, cfg.T, cfg.Hkv, cfg.G, cfg.D)
    x2["q"] = q[:, :, :, ::-1].reshape(x["q"].shape).copy()
    r2 = run_rows(cfg, x2, rows=np.array([511, 300]), want_scores=True)
    np.testing.assert_allclose(r1["scores"], r2["scores"], rtol=1e-13, atol=0)
    assert np.array_equal(r1["idx"], r2["idx"])


def test_idx_override_reproduces_selection():
    cfg, x = small_nsa(seed=24, T=1500, Hkv=1, G=4, D=16)
    rows = np.array([1400, 1499])
    r1 = run_rows(cfg, x, rows=rows)
    r2 = run_rows(cfg, x, rows=rows, idx_in=r1["idx"])
    np.testing.assert_array_equal(r1["out"], r2["out"])


# ---------------------------------------------------------------- gate, causality, decode

def test_gate_one_hot_returns_each_branch_and_is_linear():
    cfg, x = small_nsa(seed=25, T=700, D=16)
    base = run_rows(cfg, x, rows=np.array([699, 350, 40]), branches=True)
    for kb, nm in enumerate(("o_cmp", "o_slc", "o_win")):
        x2 = dict(x)
        g = np.zeros_like(x["gate"])
        g[..., kb] = 1.0
        x2["gate"] = g
        r = run_rows(cfg, x2, rows=np.array([699, 350, 40]))
        np.testing.assert_allclose(r["out"], base[nm], rtol=0, atol=0)
    gt = x["gate"][0, [699, 350, 40]].astype(np.float64)
    comb = (gt[..., 0:1] * base["o_cmp"] + gt[..., 1:2] * base["o_slc"] + gt[..., 2:3] * base["o_win"])
    np.testing.assert_allclose(base["out"], comb, rtol=1e-14, atol=1e-14)


def test_causality_future_changes_do_not_leak():
    cfg, x = small_nsa(seed=26, T=900, Hkv=2, G=2, D=16)
    t0 = 700
    rows = np.array([t0, 699, 500, 64])
    r1 = run_rows(cfg, x, rows=rows)
    x2 = dict(x)
    for nm, shape in (("k", None), ("v", None)):
        a = x[nm].copy()
        a[:, :, t0 + 1:] = S.normal_bf16(99, nm, a[:, :, t0 + 1:].shape)
        x2[nm] = a
    qq = x["q"].copy()
    qq[:, t0 + 1:] = 0
    x2["q"] = qq
    r2 = run_rows(cfg, x2, rows=rows)
    np.testing.assert_array_equal(r1["out"], r2["out"])
    np.testing.assert_array_equal(r1["idx"], r2["idx"])


def test_decode_equals_prefill_last_row():
    cfg, x = small_nsa(seed=27, T=1200, Hkv=2, G=4, D=32)
    kc = O.compress(x["k"], x["wk"], 32, 16)
    vc = O.compress(x["v"], x["wv"], 32, 16)
    for L in (1200, 777, 64, 1):
        rp = O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"], [0], [L - 1],
                                branches=True)
        rd = O.nsa_decode(cfg, x["q"][:, L - 1], x["k"], x["v"], kc, vc, [L], x["gate"][:, L - 1],
                          branches=True)
        np.testing.assert_array_equal(rp["out"], rd["out"])
        np.testing.assert_array_equal(rp["idx"], rd["idx"])


# ---------------------------------------------------------------- MoBA

def test_moba_block_keys_are_numpy_means():
    cfg = O.MobaCfg(1, 2048, 3, 32, block=512)
    x = S.moba_inputs(31, 1, 2048, 3, 32)
    kbar = O.moba_pool(cfg, x["k"])
    ref = f64(x["k"]).reshape(1, 3, 4, 512, 32).mean(axis=3)
    np.testing.assert_allclose(kbar, ref, rtol=0, atol=1e-15)


def test_moba_full_coverage_is_causal_attention():
    cfg = O.MobaCfg(1, 1024, 2, 16, block=128, top_k=8)
    x = S.moba_inputs(32, 1, 1024, 2, 16)
    r = O.moba_prefill_rows(cfg, x["q"], x["k"], x["v"], np.zeros(1024, np.int32), np.arange(1024))
    ref = sdpa_causal(f64(x["q"][0]), f64(x["k"][0]).transpose(1, 0, 2),
                      f64(x["v"][0]).transpose(1, 0, 2))
    np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-12)


def test_moba_selection_brute_force_and_own_block():
    cfg = O.MobaCfg(1, 2048, 2, 16, block=128, top_k=3)
    x = S.moba_inputs(33, 1, 2048, 2, 16)
    rows = np.array([0, 127, 128, 511, 512, 1000, 2047])
    r = O.moba_prefill_rows(cfg, x["q"], x["k"], x["v"], np.zeros(len(rows), np.int32), rows,
                            want_scores=True)
    kbar = O.moba_pool(cfg, x["k"])
    qf = f64(x["q"][0])
    for a, t in enumerate(rows):
        b = t // 128
        for h in range(2):
            sc = r["scores"][a, h]
            # scores are the plain dot products with the pooled keys (numpy matvec)
            np.testing.assert_allclose(sc[:b], kbar[0, h, :b] @ qf[t, h], rtol=1e-13, atol=1e-13)
            if b <= 3:
                ref = list(range(b + 1))
            else:
                best = max(itertools.combinations(range(b), 3),
                           key=lambda c: (sum(sc[j] for j in c), [-j for j in c]))
                ref = sorted(set(best) | {b})
            assert [j for j in r["idx"][a, h] if j >= 0] == ref


def test_moba_causality():
    cfg = O.MobaCfg(1, 1024, 2, 16, block=128, top_k=2)
    x = S.moba_inputs(34, 1, 1024, 2, 16)
    rows = np.array([600, 300])
    r1 = O.moba_prefill_rows(cfg, x["q"], x["k"], x["v"], np.zeros(2, np.int32), rows)
    x2 = {k: v.copy() for k, v in x.items()}
    x2["k"][:, :, 601:] = 0
    x2["v"][:, :, 601:] = 0
    r2 = O.moba_prefill_rows(cfg, x2["q"], x2["k"], x2["v"], np.zeros(2, np.int32), rows)
    np.testing.assert_array_equal(r1["out"], r2["out"])
    np.testing.assert_array_equal(r1["idx"], r2["idx"])
