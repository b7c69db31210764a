"""Host logic of bench.py, on the CPU: the work counts that its rates divide by, checked against
the key sets the oracle actually attends over, the one-GPU rule, the counter-traffic and
commit records and when they are reported."""
import os
import subprocess
import sys

import numpy as np

import bench
import oracle as O
import synth_inputs as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def causal_block_keys(t, j, block):
    """Keys of block j at or before position t, counted one by one."""
    return sum(1 for s in range(j * block, (j + 1) * block) if s <= t)


def test_prefill_pairs_match_the_oracle_selection():
    """prefill_pairs gives, per head, the (query, key) pairs of each NSA branch: compressed
    tokens whose span has ended, keys of the selected blocks (block 0, the local blocks and the
    ranked ones, as the oracle selects them here) and the 512-token window."""
    B, T, Hkv, G, D = 1, 1300, 2, 4, 64
    cfg = O.NsaCfg(B, T, Hkv, G, D)
    x = S.nsa_prefill_inputs(5, B, T, Hkv, G, D)
    kc = O.compress(x["k"], x["wk"], cfg.cmp_len, cfg.cmp_stride)
    vc = O.compress(x["v"], x["wv"], cfg.cmp_len, cfg.cmp_stride)
    rt = np.arange(T, dtype=np.int32)
    ora = O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"],
                             np.zeros(T, dtype=np.int32), rt)
    idx = ora["idx"]  # [T, Hkv, n]
    slc = sum(causal_block_keys(t, int(j), cfg.sel_block)
              for t in range(T) for g in range(Hkv) for j in idx[t, g] if j >= 0)
    vis = sum(1 for t in range(T) for i in range(O.n_cmp(T, cfg.cmp_len, cfg.cmp_stride))
              if i * cfg.cmp_stride + cfg.cmp_len - 1 <= t)
    win = sum(1 for t in range(T) for s in range(T) if t - cfg.window < s <= t)
    cmp_b, slc_b, win_b = bench.prefill_pairs(T)
    assert slc == slc_b * Hkv
    assert vis == cmp_b
    assert win == win_b
    # the torch helper used for adaptive selections counts the same keys from the index tensor
    import torch
    assert bench.selected_keys(torch.from_numpy(idx[None])) == slc


def test_moba_work_matches_the_oracle_selection():
    """moba_work counts, per head, the causal keys of each query's own block and its top-k
    past blocks (all past blocks while there are at most k)."""
    B, T, H, D, block, top_k = 1, 2048, 2, 64, 128, 3
    cfg = O.MobaCfg(B, T, H, D, block=block, top_k=top_k)
    x = S.moba_inputs(6, B, T, H, D)
    rt = np.arange(T, dtype=np.int32)
    ora = O.moba_prefill_rows(cfg, x["q"], x["k"], x["v"], np.zeros(T, dtype=np.int32), rt)
    keys = sum(causal_block_keys(t, int(j), block)
               for t in range(T) for h in range(H) for j in ora["idx"][t, h] if j >= 0)
    flops, _, pairs = bench.moba_work(T, H, D, block, top_k)
    assert keys == pairs * H
    assert flops == 4.0 * D * keys


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    """measured_traffic scales the committed counters by the copy calibration while the
    kernel's source digest matches, and reports nothing once it does not; the selected stage's
    rate follows the same rule."""
    import json

    tr = {"copy_calibration": {"fetch_counter_bytes_per_byte": 0.5,
                               "write_counter_bytes_per_byte": 1.0},
          "kernels": {k: {"fetch_kib_per_dispatch": 1000.0, "write_kib_per_dispatch": 500.0,
                          "source_sha256": bench.source_digest(k)}
                      for k in ("slc_block_kernel", "selected_kernel")}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(tr))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    expect = int(round(1000.0 * 1024 / 0.5 + 500.0 * 1024))
    assert bench.measured_traffic("slc_block_kernel") == expect
    sel = bench.selected_traffic(2.0)
    assert sel["bytes"] == 2 * expect
    assert abs(sel["gbs"] - 2 * expect / 2e-3 / 1e9) < 0.1
    tr["kernels"]["selected_kernel"]["source_sha256"] = "0" * 64
    path.write_text(json.dumps(tr))
    assert bench.measured_traffic("selected_kernel") is None
    assert bench.selected_traffic(2.0)["bytes"] is None


def test_host_info_names_the_commit_from_the_build_record(tmp_path, monkeypatch):
    """Outside a git checkout the bench takes the commit from the record the build wrote beside
    the library, and only while the record's source digest equals the sources'."""
    import json
    import shutil

    pkg = tmp_path / "dynamic_block_sparse_fwd_amd"
    shutil.copytree(bench.CSRC, pkg / "csrc")
    digest = bench.host_info()["library_source_sha256"]
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))  # no .git there
    monkeypatch.setattr(bench, "CSRC", str(pkg / "csrc"))
    rec = pkg / "libnsa.buildinfo.json"
    rec.write_text(json.dumps({"git_sha": "abc123", "csrc_modified_since_commit": False,
                               "library_source_sha256": digest}))
    info = bench.host_info()
    assert info["git_sha"] == "abc123" and info["git_sha_source"] == "build record"
    rec.write_text(json.dumps({"git_sha": "abc123", "csrc_modified_since_commit": False,
                               "library_source_sha256": "stale"}))
    assert bench.host_info()["git_sha"] is None
