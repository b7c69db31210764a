"""nsa_decode_noalloc (the decode on the library's static per-GPU workspace) against nsa_decode
with a caller-owned workspace, through the C ABI.  Both run the same kernels, so outputs and
indices must agree bit for bit; two calls in a row, the second on a smaller problem, so the
second reads a scratch array that still holds the first call's contents."""
import numpy as np
import pytest

import synth_inputs as S

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


CASES = [
    # B, L, Hkv, G, D, seqlens, extra -- the second smaller than the first
    (4, 4100, 2, 16, 128, [4100, 3000, 777, 64], {}),
    (2, 700, 1, 8, 64, [700, 33], dict(top_p=0.5)),
]


def test_noalloc_decode_matches_workspace_decode():
    import dynamic_block_sparse_fwd_amd as nsa
    nsa.load_library()
    for i, (B, L, Hkv, G, D, seqlens, extra) in enumerate(CASES):
        print("noalloc case", i, (B, L, Hkv, G, D, seqlens, extra), flush=True)
        cfg = nsa.NsaConfig(B, L, Hkv, G, D, **extra)
        assert nsa.decode_workspace_bytes(cfg) <= nsa.decode_noalloc_max_bytes()
        x = S.nsa_decode_inputs(70 + i, B, L, Hkv, G, D, seqlens=seqlens)
        d = {k: to_dev(v) for k, v in x.items()}
        kc = nsa.nsa_compress(cfg, d["kcache"], d["wk"])
        vc = nsa.nsa_compress_tiles(cfg, d["vcache"], d["wv"])
        args = (d["q"], d["kcache"], d["vcache"], kc, vc, d["seqlens"], d["gate"])
        ref_out, ref_idx = nsa.nsa_decode(cfg, *args)
        out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device="cuda")
        idx = torch.empty((B, Hkv, cfg.top_n), dtype=torch.int32, device="cuda")
        nsa.nsa_decode_noalloc(cfg, *args, out, idx)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        assert torch.equal(idx, ref_idx), "indices differ from nsa_decode (case %d)" % i
        assert torch.equal(out, ref_out), "output differs from nsa_decode (case %d)" % i


def test_noalloc_rejects_too_large_before_launch():
    """A configuration whose workspace exceeds the static array is refused on the host."""
    import dynamic_block_sparse_fwd_amd as nsa
    lib = nsa.load_library()
    import ctypes
    cfg = nsa.NsaConfig(1024, 65536, 4, 16, 128)
    assert nsa.decode_workspace_bytes(cfg) > nsa.decode_noalloc_max_bytes()
    st = lib.nsa_decode_noalloc(ctypes.byref(cfg.c()), *([None] * 9), None)
    assert st == nsa.NSA_ERR_WORKSPACE
