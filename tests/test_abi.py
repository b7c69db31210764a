"""The C-ABI library loads, exports every declared entry point, and rejects bad arguments on the
host before touching a device (CPU only: no compute call reaches a kernel here)."""
import ctypes
import os
import re

import pytest

import dynamic_block_sparse_fwd_amd as nsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "nsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                                 src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return nsa.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert {"nsa_prefill", "nsa_decode", "moba_prefill", "nsa_compress"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(nsa.EXPORTS), "binding and header disagree"


def cfgB():
    return nsa.NsaConfig(1, 65536, 4, 16, 128)


def test_validate_accepts_the_workloads(lib):
    for c in (nsa.NsaConfig(1, 2048, 1, 4, 64), cfgB(), nsa.NsaConfig(32, 65536, 4, 16, 128),
              nsa.NsaConfig(1, 1 << 20, 8, 8, 128)):
        assert lib.nsa_validate(ctypes.byref(c.c())) == nsa.NSA_OK
    assert lib.moba_validate(ctypes.byref(nsa.MobaConfig(1, 131072, 32, 128).c())) == nsa.NSA_OK
    for p in (0.0, 1e-6, 0.5, 1.0):
        c = cfgB()
        c.top_p = p
        assert lib.nsa_validate(ctypes.byref(c.c())) == nsa.NSA_OK


@pytest.mark.parametrize("field,value,code", [
    ("D", 96, nsa.NSA_ERR_UNSUPPORTED), ("G", 3, nsa.NSA_ERR_UNSUPPORTED),
    ("G", 0, nsa.NSA_ERR_INVALID_ARG), ("T", 0, nsa.NSA_ERR_INVALID_ARG),
    ("sel_block", 48, nsa.NSA_ERR_UNSUPPORTED), ("top_n", 2, nsa.NSA_ERR_UNSUPPORTED),
    ("top_n", 65, nsa.NSA_ERR_UNSUPPORTED), ("window", 0, nsa.NSA_ERR_INVALID_ARG),
    ("cmp_stride", 64, nsa.NSA_ERR_UNSUPPORTED), ("scale", -1.0, nsa.NSA_ERR_INVALID_ARG),
    ("T", (1 << 20) + 1, nsa.NSA_ERR_UNSUPPORTED), ("top_p", -0.1, nsa.NSA_ERR_INVALID_ARG),
    ("top_p", 1.5, nsa.NSA_ERR_INVALID_ARG), ("top_p", float("nan"), nsa.NSA_ERR_INVALID_ARG),
])
def test_validate_rejects(lib, field, value, code):
    c = cfgB()
    setattr(c, field, value)
    assert lib.nsa_validate(ctypes.byref(c.c())) == code
    assert lib.nsa_prefill_workspace_bytes(ctypes.byref(c.c())) == 0


def test_moba_validate_rejects(lib):
    for kw, code in ((dict(D=80), nsa.NSA_ERR_UNSUPPORTED), (dict(block=100), nsa.NSA_ERR_UNSUPPORTED),
                     (dict(T=1000), nsa.NSA_ERR_UNSUPPORTED), (dict(H=0), nsa.NSA_ERR_INVALID_ARG)):
        c = nsa.MobaConfig(1, 131072, 32, 128)
        for k, v in kw.items():
            setattr(c, k, v)
        assert lib.moba_validate(ctypes.byref(c.c())) == code


def test_null_config_and_status_strings(lib):
    assert lib.nsa_validate(None) == nsa.NSA_ERR_INVALID_ARG
    assert lib.nsa_prefill_workspace_bytes(None) == 0
    for code in (0, -1, -2, -3, -4, 7):
        assert len(nsa.status_string(code)) > 0


def test_workspace_sizes_are_plausible(lib):
    c = cfgB()
    ws = lib.nsa_prefill_workspace_bytes(ctypes.byref(c.c()))
    # the selected branch's block-major partials, one per (row, group, slot): 16 heads x D fp16
    # outputs + 16 x 4 fp32 statistics; besides them transposed V (64 MiB), compressed caches,
    # weights, indices and the entry lists, well under 1 GiB
    partials = c.B * c.T * c.Hkv * c.top_n * (c.sel_block // 64) * (16 * c.D * 2 + 16 * 16)
    assert partials + (64 << 20) < ws < partials + (1 << 30)
    assert lib.nsa_num_compressed(65536, 32, 16) == 4095
    assert lib.nsa_num_compressed(31, 32, 16) == 0
    assert lib.nsa_num_compressed_tiles(65536, 32, 16) == 64
    assert lib.nsa_num_compressed_tiles(32 + 16 * 64, 32, 16) == 2  # 65 tokens
    assert lib.nsa_num_compressed_tiles(31, 32, 16) == 0
    assert lib.nsa_compress_workspace_bytes(ctypes.byref(c.c())) >= 32 * 128 * 128 * 2


def test_entry_points_reject_before_any_launch(lib):
    c = nsa.NsaConfig(1, 2048, 1, 4, 64).c()
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: the calls must fail on host checks first
    # null tensor pointers
    assert lib.nsa_prefill(ctypes.byref(c), None, fake, fake, fake, fake, fake, fake, None, fake,
                           1 << 30, None) == nsa.NSA_ERR_INVALID_ARG
    # workspace too small
    assert lib.nsa_prefill(ctypes.byref(c), fake, fake, fake, fake, fake, fake, fake, None, fake,
                           16, None) == nsa.NSA_ERR_WORKSPACE
    # misaligned pointer
    assert lib.nsa_prefill(ctypes.byref(c), P(0x1001), fake, fake, fake, fake, fake, fake, None,
                           fake, 1 << 40, None) == nsa.NSA_ERR_INVALID_ARG
    assert lib.nsa_compress(ctypes.byref(c), None, fake, fake, fake, 1 << 20, None) == \
        nsa.NSA_ERR_INVALID_ARG
    assert lib.nsa_compress(ctypes.byref(c), fake, fake, fake, fake, 8, None) == nsa.NSA_ERR_WORKSPACE
    assert lib.nsa_compress_tiles(ctypes.byref(c), fake, fake, None, fake, 1 << 20,
                                  None) == nsa.NSA_ERR_INVALID_ARG
    assert lib.nsa_compress_tiles(ctypes.byref(c), fake, fake, fake, fake, 8,
                                  None) == nsa.NSA_ERR_WORKSPACE
    bad = nsa.NsaConfig(1, 2048, 1, 3, 64).c()
    assert lib.nsa_decode(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, fake, fake, None,
                          fake, 1 << 30, None) == nsa.NSA_ERR_UNSUPPORTED
    m = nsa.MobaConfig(1, 1024, 2, 64, block=128).c()
    assert lib.moba_prefill(ctypes.byref(m), None, fake, fake, fake, None, fake, 1 << 30, None) == \
        nsa.NSA_ERR_INVALID_ARG


def test_prefill_stages_reject_before_any_launch(lib):
    c = nsa.NsaConfig(1, 2048, 1, 4, 64).c()
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced
    ws = 1 << 40
    # empty and unknown stage masks
    for mask in (0, 8, 15):
        assert lib.nsa_prefill_stages(ctypes.byref(c), mask, fake, fake, fake, fake, fake, fake,
                                      fake, fake, fake, ws, None) == nsa.NSA_ERR_INVALID_ARG
    # the selected stage alone needs the index list as input
    assert lib.nsa_prefill_stages(ctypes.byref(c), nsa.STAGE_SELECTED, fake, fake, fake, None,
                                  None, fake, fake, None, fake, ws, None) == nsa.NSA_ERR_INVALID_ARG
    # the compressed stage needs the compressor weights
    assert lib.nsa_prefill_stages(ctypes.byref(c), nsa.STAGE_CMP_SELECT, fake, fake, fake, None,
                                  fake, fake, fake, fake, fake, ws, None) == nsa.NSA_ERR_INVALID_ARG
    # workspace too small
    assert lib.nsa_prefill_stages(ctypes.byref(c), nsa.STAGE_WINDOW, fake, fake, fake, None, None,
                                  fake, fake, None, fake, 16, None) == nsa.NSA_ERR_WORKSPACE


def test_product_path_does_not_touch_the_oracle():
    """The binding and kernels never import or link the CPU oracle."""
    pkg = os.path.join(ROOT, "dynamic_block_sparse_fwd_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt.lower().replace("oracles", ""), f


def test_cache_append_and_chunk_reject_before_any_launch(lib):
    c = nsa.NsaConfig(2, 4096, 2, 4, 64).c()
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced
    ws = 1 << 40
    wsb = lib.nsa_cache_append_workspace_bytes(ctypes.byref(c))
    assert wsb >= 2 * 32 * 64 * 64 * 2
    assert lib.nsa_prefill_chunk_workspace_bytes(ctypes.byref(c)) == \
        lib.nsa_prefill_workspace_bytes(ctypes.byref(c))
    args = [fake] * 10
    # C outside [1, Lmax]
    for C in (0, -3, 4097):
        assert lib.nsa_cache_append(ctypes.byref(c), C, *args, ws, None) == nsa.NSA_ERR_INVALID_ARG
    # null new rows, null seqlens, small workspace, misaligned cache
    for i in (0, 2):
        a = list(args)
        a[i] = None
        assert lib.nsa_cache_append(ctypes.byref(c), 1, *a, ws, None) == nsa.NSA_ERR_INVALID_ARG
    assert lib.nsa_cache_append(ctypes.byref(c), 1, *args, wsb - 1, None) == nsa.NSA_ERR_WORKSPACE
    a = list(args)
    a[5] = P(0x1008)
    assert lib.nsa_cache_append(ctypes.byref(c), 1, *a, ws, None) == nsa.NSA_ERR_INVALID_ARG
    cargs = [fake] * 9
    # chunk start not a multiple of 64; negative start; empty chunk; past the capacity
    assert lib.nsa_prefill_chunk(ctypes.byref(c), 32, 64, *cargs, ws, None) == \
        nsa.NSA_ERR_UNSUPPORTED
    for (p0, C) in ((-64, 64), (0, 0), (4032, 128)):
        assert lib.nsa_prefill_chunk(ctypes.byref(c), p0, C, *cargs, ws, None) == \
            nsa.NSA_ERR_INVALID_ARG
    a = list(cargs)
    a[0] = None
    assert lib.nsa_prefill_chunk(ctypes.byref(c), 0, 64, *a, ws, None) == nsa.NSA_ERR_INVALID_ARG
    assert lib.nsa_prefill_chunk(ctypes.byref(c), 0, 64, *cargs, 16, None) == \
        nsa.NSA_ERR_WORKSPACE
    bad = nsa.NsaConfig(2, 4096, 2, 3, 64).c()
    assert lib.nsa_prefill_chunk(ctypes.byref(bad), 0, 64, *cargs, ws, None) == \
        nsa.NSA_ERR_UNSUPPORTED


def test_backward_rejects_before_any_launch(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced
    c = nsa.NsaConfig(1, 2048, 2, 16, 128).c()
    assert lib.nsa_backward_workspace_bytes(ctypes.byref(c)) > 0
    args = [fake] * 15
    # every group size the forward takes; an unsupported one is rejected
    for G in (1, 2, 4, 8):
        assert lib.nsa_backward_workspace_bytes(ctypes.byref(nsa.NsaConfig(1, 2048, 2, G, 64).c()))
    bad = nsa.NsaConfig(1, 2048, 2, 3, 128).c()
    assert lib.nsa_backward_workspace_bytes(ctypes.byref(bad)) == 0
    assert lib.nsa_backward(ctypes.byref(bad), *args, 1 << 40, None) == nsa.NSA_ERR_UNSUPPORTED
    # a null input or output, a misaligned pointer, a small workspace
    for i in (0, 6, 7, 13):
        a = list(args)
        a[i] = None
        assert lib.nsa_backward(ctypes.byref(c), *a, 1 << 40, None) == nsa.NSA_ERR_INVALID_ARG
    a = list(args)
    a[8] = P(0x1004)
    assert lib.nsa_backward(ctypes.byref(c), *a, 1 << 40, None) == nsa.NSA_ERR_INVALID_ARG
    assert lib.nsa_backward(ctypes.byref(c), *args, 16, None) == nsa.NSA_ERR_WORKSPACE


def test_prefill_diag_rejects_before_any_launch(lib):
    """nsa_prefill_diag: the block scores exist only while a query tile's scores stay in LDS
    (here 140000 tokens: 2188 blocks, the selection streams), and the diagnostic outputs must be
    16-byte aligned; both are refused on the host."""
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced
    args = [fake] * 8
    long_cfg = nsa.NsaConfig(1, 140000, 1, 16, 128).c()
    assert lib.nsa_prefill_diag(ctypes.byref(long_cfg), *args, fake, fake, fake, 1 << 40,
                                None) == nsa.NSA_ERR_UNSUPPORTED
    c = nsa.NsaConfig(1, 2048, 1, 4, 64).c()
    assert lib.nsa_prefill_diag(ctypes.byref(c), *args, P(0x1004), None, fake, 1 << 40,
                                None) == nsa.NSA_ERR_INVALID_ARG
