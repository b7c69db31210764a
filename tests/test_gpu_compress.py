"""nsa_compress on the GPU reproduces the oracle's compressed tokens bit for bit (both round
the exact sum to the nearest bf16; the kernel re-does near-midpoint sums in fp64), and
nsa_compress_tiles writes the same values in feature-major 64-token tiles, zero past n_cmp."""
import numpy as np
import pytest

import oracle as O
import synth_inputs as S

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


SHAPES = [(1, 2048, 1, 64, 32, 16), (1, 4096, 4, 128, 32, 16), (2, 1000, 3, 128, 32, 16),
          (1, 777, 2, 64, 48, 16), (1, 300, 1, 128, 16, 16), (1, 20, 1, 64, 32, 16)]


@pytest.mark.parametrize("B,T,H,D,l,d", SHAPES)
def test_compress_bit_exact(B, T, H, D, l, d):
    import dynamic_block_sparse_fwd_amd as nsa
    nsa.load_library()
    seed = 40 + T + D
    x = S.normal_bf16(seed, "k", (B, H, T, D))
    w = S.normal_bf16(seed, "wk", (l, D, D), std=1.0 / np.sqrt(l * D))
    ref = O.compress(x, w, l, d)
    cfg = nsa.NsaConfig(B, T, H, 1, D, cmp_len=l, cmp_stride=d)
    got = nsa.nsa_compress(cfg, torch.from_numpy(x.view(np.int16)).cuda(),
                           torch.from_numpy(w.view(np.int16)).cuda())
    got = got.cpu().numpy().view(np.uint16)
    assert got.shape == ref.shape
    diff = np.nonzero(got != ref)
    assert len(diff[0]) == 0, "%d of %d compressed values differ, first at %s" % (
        len(diff[0]), ref.size, [int(a[0]) for a in diff])


@pytest.mark.parametrize("B,T,H,D,l,d", SHAPES)
def test_compress_tiles_bit_exact(B, T, H, D, l, d):
    import dynamic_block_sparse_fwd_amd as nsa
    nsa.load_library()
    seed = 50 + T + D
    x = S.normal_bf16(seed, "v", (B, H, T, D))
    w = S.normal_bf16(seed, "wv", (l, D, D), std=1.0 / np.sqrt(l * D))
    ref = O.compress(x, w, l, d)
    cfg = nsa.NsaConfig(B, T, H, 1, D, cmp_len=l, cmp_stride=d)
    n = ref.shape[2]
    nt = (n + 63) // 64
    assert cfg.ncmp_tiles == nt == nsa.load_library().nsa_num_compressed_tiles(T, l, d)
    out = torch.full((B, H, nt, D, 64), 0x3F80, dtype=torch.int16, device="cuda")  # 1.0, not 0
    got = nsa.nsa_compress_tiles(cfg, torch.from_numpy(x.view(np.int16)).cuda(),
                                 torch.from_numpy(w.view(np.int16)).cuda(), out=out)
    got = got.cpu().numpy().view(np.uint16)
    flat = got.transpose(0, 1, 3, 2, 4).reshape(B, H, D, nt * 64)  # [.., c, i]
    np.testing.assert_array_equal(flat[:, :, :, :n], ref.transpose(0, 1, 3, 2))
    assert not flat[:, :, :, n:].any(), "tokens past n_cmp must be zero"
