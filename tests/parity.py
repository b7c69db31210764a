"""Parity rules shared by the GPU tests (test support module, not a test file).

  * selected block indices must match the oracle bit for bit;
  * a (row, group) whose oracle top-n score gap is below 1e-4 (relative) is a near tie: the
    GPU's choice is accepted when every free block it picked scores at least
    S_(k) * (1 - 1e-4) in the oracle, and the oracle is then re-run with the GPU's indices
    before outputs are compared;
  * under adaptive top-p the oracle's gap also covers the mass decisions (|cum - p M| / M);
    a near-tie choice is accepted when, in the oracle's scores, its free blocks outrank the
    rest within the same tolerance, the last one taken was still needed (mass before it below
    p M + tol M) and it stopped only at the cap, with no block left, or with p M - tol M reached;
  * fp32 outputs within max-abs 1e-2 and mean-abs 1e-3 of the fp64 oracle.
"""
import numpy as np

GAP_TOL = 1e-4
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def free_kth_score(scores_row, t, beta, n, n_local):
    """S_(k): the k-th best free score of one (row, group) (forced blocks excluded)."""
    b = t // beta
    forced = {0} | set(range(max(0, b - n_local + 1), b + 1))
    free = sorted((scores_row[j] for j in range(b + 1) if j not in forced), reverse=True)
    k = n - len(forced)
    return free[k - 1] if 0 < k <= len(free) else None


def check_top_p_choice(chosen, scores_row, t, beta, n, n_local, top_p, msg):
    """Validity of one adaptive top-p index list against the oracle's fp64 scores."""
    b = t // beta
    forced = {0} | set(j for j in range(b - n_local + 1, b + 1) if j >= 0)
    assert forced <= set(chosen), "forced block missing: " + msg
    assert len(set(chosen)) == len(chosen) <= n, "bad index list: " + msg
    assert sorted(chosen) == chosen, "indices not ascending: " + msg
    s = scores_row
    M = float(s[:b + 1].sum())
    tol = GAP_TOL * M
    free_in = sorted((s[j] for j in chosen if j not in forced), reverse=True)
    free_out = [s[j] for j in range(b + 1) if j not in forced and j not in chosen]
    if free_in and free_out:
        assert free_in[-1] >= max(free_out) * (1 - GAP_TOL), "weak pick: " + msg
    fm = float(sum(s[j] for j in forced))
    total = fm + float(sum(free_in))
    if free_in:
        assert total - free_in[-1] < top_p * M + tol, "pick not needed: " + msg
    if free_out and len(chosen) < n:
        assert total >= top_p * M - tol, "stopped short of p: " + msg


def check_nsa_idx(gpu_idx, ora, rows_t, beta, n, n_local, top_p=0.0):
    """Compare GPU indices with the oracle's.  Returns (rows needing an oracle re-run with the
    GPU indices, number of near-tie rows accepted).  Raises AssertionError on a real mismatch."""
    gpu_idx = np.asarray(gpu_idx)
    rerun = []
    accepted = 0
    for r in range(gpu_idx.shape[0]):
        bad_groups = np.nonzero((gpu_idx[r] != ora["idx"][r]).any(axis=-1))[0]
        if len(bad_groups) == 0:
            continue
        t = int(rows_t[r])
        for g in bad_groups:
            gap = ora["gap"][r, g]
            msg = "row t=%d group %d: gpu %s oracle %s gap %.3g" % (
                t, g, gpu_idx[r, g].tolist(), ora["idx"][r, g].tolist(), gap)
            assert gap < GAP_TOL, "index mismatch outside near-tie: " + msg
            if top_p > 0:
                chosen = [int(j) for j in gpu_idx[r, g] if j >= 0]
                assert (gpu_idx[r, g, len(chosen):] == -1).all(), "bad padding: " + msg
                check_top_p_choice(chosen, ora["scores"][r, g], t, beta, n, n_local, top_p, msg)
                accepted += 1
                continue
            sk = free_kth_score(ora["scores"][r, g], t, beta, n, n_local)
            assert sk is not None, msg
            b = t // beta
            forced = {0} | set(range(max(0, b - n_local + 1), b + 1))
            chosen = [j for j in gpu_idx[r, g] if j >= 0]
            assert forced <= set(chosen), "forced block missing: " + msg
            assert len(set(chosen)) == len(chosen) == min(n, b + 1), "bad index list: " + msg
            assert sorted(chosen) == chosen, "indices not ascending: " + msg
            for j in chosen:
                if j not in forced:
                    assert ora["scores"][r, g, j] >= sk * (1 - GAP_TOL), "weak pick: " + msg
            accepted += 1
        rerun.append(r)
    return rerun, accepted


def check_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), what + ": non-finite GPU output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert mx <= MAX_ABS, "%s: max-abs error %.3g > %g at %s" % (
        what, mx, MAX_ABS, np.unravel_index(int(err.argmax()), err.shape))
    assert mean <= MEAN_ABS, "%s: mean-abs error %.3g > %g" % (what, mean, MEAN_ABS)
    return mx, mean


def check_moba_idx(gpu_idx, ora, rows_t, block, top_k, den):
    """MoBA indices: bit-exact, except near ties (oracle gap < 1e-4, the gap being normalised
    by den = |q| * max_j |kbar_j| of the row/head) where every GPU-chosen past block must score
    within 1e-4 * den of the oracle's k-th score.  Returns rows to re-run with GPU indices."""
    gpu_idx = np.asarray(gpu_idx)
    rerun, accepted = [], 0
    for r in range(gpu_idx.shape[0]):
        bad = np.nonzero((gpu_idx[r] != ora["idx"][r]).any(axis=-1))[0]
        if len(bad) == 0:
            continue
        t = int(rows_t[r])
        b = t // block
        for h in bad:
            msg = "row t=%d head %d: gpu %s oracle %s gap %.3g" % (
                t, h, gpu_idx[r, h].tolist(), ora["idx"][r, h].tolist(), ora["gap"][r, h])
            assert ora["gap"][r, h] < GAP_TOL, "index mismatch outside near-tie: " + msg
            sc = ora["scores"][r, h, :b]
            sk = np.sort(sc)[::-1][top_k - 1]
            chosen = [j for j in gpu_idx[r, h] if j >= 0]
            assert chosen[-1] == b and chosen == sorted(chosen) and len(chosen) == top_k + 1, msg
            for j in chosen[:-1]:
                assert sc[j] >= sk - GAP_TOL * den[r, h], "weak pick: " + msg
            accepted += 1
        rerun.append(r)
    return rerun, accepted
