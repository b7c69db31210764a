"""The near-tie rules of the GPU parity checks, exercised on the CPU against the oracle's own
choices (always accepted) and against planted wrong choices (always rejected)."""
import numpy as np
import pytest

import oracle as O
import synth_inputs as S
from tests.parity import check_nsa_idx, check_top_p_choice


def oracle_rows(p, seed=41, T=1500, Hkv=2, G=4, D=32):
    cfg = O.NsaCfg(1, T, Hkv, G, D, top_p=p)
    x = S.nsa_prefill_inputs(seed, 1, T, Hkv, G, D)
    kc = O.compress(x["k"], x["wk"], cfg.cmp_len, cfg.cmp_stride)
    vc = O.compress(x["v"], x["wv"], cfg.cmp_len, cfg.cmp_stride)
    rows = np.arange(200, T, 97).astype(np.int32)
    r = O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"],
                           np.zeros(len(rows), np.int32), rows, want_scores=True)
    return cfg, rows, r


@pytest.mark.parametrize("p", [0.2, 0.5, 0.9])
def test_top_p_checker_accepts_the_oracle_choice(p):
    cfg, rows, r = oracle_rows(p)
    assert check_nsa_idx(r["idx"], r, rows, 64, cfg.top_n, cfg.n_local, p) == ([], 0)
    for a, t in enumerate(rows):
        for g in range(cfg.Hkv):
            chosen = [int(j) for j in r["idx"][a, g] if j >= 0]
            check_top_p_choice(chosen, r["scores"][a, g], int(t), 64, cfg.top_n, cfg.n_local, p,
                               "oracle")


def test_top_p_checker_rejects_planted_mistakes():
    """One block more, one block fewer, or a free block swapped for a worse one: each breaks
    a rule of the checker (rows whose oracle choice is clear of the boundary)."""
    p = 0.5
    cfg, rows, r = oracle_rows(p)
    tried = 0
    for a, t in enumerate(rows):
        t = int(t)
        b = t // 64
        for g in range(cfg.Hkv):
            if r["gap"][a, g] < 1e-2:
                continue
            s = r["scores"][a, g]
            chosen = [int(j) for j in r["idx"][a, g] if j >= 0]
            forced = {0, b - 1, b}
            free_in = [j for j in chosen if j not in forced]
            free_out = sorted((j for j in range(b + 1) if j not in forced and j not in chosen),
                              key=lambda j: -s[j])
            bad = []
            if free_out and len(chosen) < cfg.top_n:
                bad.append(sorted(chosen + [free_out[0]]))        # one more than needed
            if free_in:
                worst = min(free_in, key=lambda j: s[j])
                bad.append(sorted(set(chosen) - {worst}))          # one fewer
                if free_out and s[free_out[-1]] < s[worst] * (1 - 1e-3):
                    bad.append(sorted((set(chosen) - {worst}) | {free_out[-1]}))  # weaker
            for c in bad:
                with pytest.raises(AssertionError):
                    check_top_p_choice(c, s, t, 64, cfg.top_n, cfg.n_local, p, "planted")
                tried += 1
    assert tried >= 10
