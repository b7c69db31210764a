"""The decode step (nsa_cache_append of the newest token, then nsa_decode) captured in a HIP
graph and replayed: every replay, with new inputs copied into the captured buffers and eager
work between the replays, must reproduce the eager calls bit for bit (decode is deterministic:
two eager runs are compared too).  The
library launches only kernels (it clears memory with a kernel, never with a memset node) and
allocates nothing, so a serving loop can capture it."""
import numpy as np
import pytest

import synth_inputs as S

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_decode_step_graph_replays_match_eager():
    import dynamic_block_sparse_fwd_amd as nsa
    nsa.load_library()
    B, L, Hkv, G, D = 4, 4096, 2, 16, 128
    cfg = nsa.NsaConfig(B, L, Hkv, G, D)
    x = S.nsa_prefill_inputs(101, B, L, Hkv, G, D)
    d = {k: to_dev(v) for k, v in x.items()}
    start = np.array([3000, 2047, 1024, 97], np.int32)  # lengths before the steps
    steps = 5

    def fresh_caches():
        kc = d["k"].clone()
        vc = d["v"].clone()
        kcmp = nsa.nsa_compress(cfg, kc, d["wk"])
        vcmp = nsa.nsa_compress_tiles(cfg, vc, d["wv"])
        return kc, vc, kcmp, vcmp

    def step_inputs(i):
        pos = torch.from_numpy(start + i).long().cuda()
        bidx = torch.arange(B, device="cuda")
        k_new = d["k"][bidx, :, pos].unsqueeze(2).contiguous()  # [B, Hkv, 1, D]
        v_new = d["v"][bidx, :, pos].unsqueeze(2).contiguous()
        q = d["q"][bidx, pos].contiguous()  # [B, Hq, D]
        g = d["gate"][bidx, pos].contiguous()
        return k_new, v_new, q, g

    aws = torch.empty(nsa.cache_append_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    dws = torch.empty(nsa.decode_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")

    # eager reference, twice: the run-to-run spread of the output
    refs = []
    for _ in range(2):
        caches = fresh_caches()
        ref = []
        for i in range(steps):
            k_new, v_new, q, g = step_inputs(i)
            before = torch.from_numpy(start + i).cuda()
            nsa.nsa_cache_append(cfg, k_new, v_new, before, d["wk"], d["wv"], *caches, ws=aws)
            out, idx = nsa.nsa_decode(cfg, q, *caches[:2], caches[2], caches[3], before + 1, g,
                                      ws=dws)
            ref.append((out.clone(), idx.clone()))
        refs.append(ref)
    torch.cuda.synchronize()
    ref = refs[0]
    spread = max(float((a[0] - b[0]).abs().max()) for a, b in zip(refs[0], refs[1]))
    tol = 0.0

    # captured: static input buffers, one graph for append + decode
    caches = fresh_caches()
    s_k, s_v, s_q, s_g = (t.clone() for t in step_inputs(0))
    s_before = torch.from_numpy(start).cuda()
    s_after = s_before + 1
    s_out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device="cuda")
    s_idx = torch.empty((B, Hkv, cfg.top_n), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            nsa.nsa_cache_append(cfg, s_k, s_v, s_before, d["wk"], d["wv"], *caches, ws=aws)
            nsa.nsa_decode(cfg, s_q, *caches[:2], caches[2], caches[3], s_after, s_g,
                           out=s_out, sel_idx=s_idx, ws=dws)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    worst = 0.0
    for i in range(steps):
        k_new, v_new, q, g = step_inputs(i)
        s_k.copy_(k_new)
        s_v.copy_(v_new)
        s_q.copy_(q)
        s_g.copy_(g)
        s_before.copy_(torch.from_numpy(start + i).cuda())
        s_after.copy_(s_before + 1)
        graph.replay()
        torch.cuda.synchronize()
        _ = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(s_idx, ref[i][1]), "replay %d: indices" % i
        err = float((s_out - ref[i][0]).abs().max())
        assert err <= tol, "replay %d: output differs by %.3g" % (i, err)
        worst = max(worst, err)
    assert spread <= tol, "eager runs differ by %.3g" % spread
    print("graph: %d replays of append + decode match the eager calls: max diff %.2e (eager "
          "run-to-run %.2e)" % (steps, worst, spread), flush=True)
