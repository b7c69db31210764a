"""GPU parity of nsa_backward (through the C ABI) against the fp64 backward oracle.

Both sides take the same seeded inputs and the same block selection, the C oracle forward's
(the selection is an input of the backward).  The matrix core sees bf16 operands (dout, the
probabilities and the score gradients rounded to bf16) with fp32 accumulation.  Rounding dout
alone gives every term of every gradient a relative error of up to 2^-9 (about 2e-3), and
sums of such terms keep that relative size, so each gradient is held to an error relative to
its own scale: mean |err| <= 4e-3 * mean |ref| (2^-8) and max |err| <= 1e-2 * max |ref|
(per tensor).  Two calls on the same inputs must give the same bits (no atomics)."""
import numpy as np
import pytest

import oracle as O
import synth_inputs as S
from oracle import nsa_backward as NB

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

MAX_REL = 1e-2
MEAN_REL = 4e-3


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_grad(name, got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), "%s %s: non-finite" % (what, name)
    err = np.abs(got - ref)
    scale_max = float(np.abs(ref).max())
    scale_mean = float(np.abs(ref).mean())
    if scale_max == 0.0:
        assert float(err.max()) == 0.0, "%s %s: expected zeros" % (what, name)
        return 0.0, 0.0
    mx, mean = float(err.max()) / scale_max, float(err.mean()) / scale_mean
    assert mx <= MAX_REL, "%s %s: max err %.3g of max |ref| at %s" % (
        what, name, mx, np.unravel_index(int(err.argmax()), err.shape))
    assert mean <= MEAN_REL, "%s %s: mean err %.3g of mean |ref|" % (what, name, mean)
    return mx, mean


CASES = [
    # name, B, T, Hkv, D, extra (G = 16 unless given)
    ("T700_Hkv2_D64", 1, 700, 2, 64, {}),
    # smaller groups: rows G .. 15 of each 16-row tile are padding
    ("G8_T650_Hkv2_D128", 1, 650, 2, 128, dict(G=8)),
    ("G4_B2_T700_D64", 2, 700, 1, 64, dict(G=4, top_p=0.5)),
    ("G1_T500_Hkv3_D64", 1, 500, 3, 64, dict(G=1)),
    ("G2_T520_D128_block128", 1, 520, 2, 128, dict(G=2, sel_block=128, top_n=5, window=100)),
    ("B2_T530_D128", 2, 530, 1, 128, {}),
    ("block128_top6_win200_D64", 1, 900, 1, 64, dict(sel_block=128, top_n=6, window=200)),
    ("top5_local1_win100_D128", 1, 1100, 1, 128, dict(top_n=5, n_local=1, window=100)),
    ("short_T40", 1, 40, 2, 64, {}),
    ("no_compressed_T20", 1, 20, 1, 128, {}),
    # an adaptive top-p selection: index rows of varying length, -1 padded
    ("topp0.4_T800_D128", 1, 800, 2, 128, dict(top_p=0.4)),
    # values with a large common part: dP' = dO . v sits near its mean <dO, o> for every key,
    # so dS = p (dP' - <dO, o>) is a small difference of large terms
    ("v_offset4_T600_D128", 1, 600, 1, 128, dict(v_offset=4.0)),
    # peaked attention (queries scaled by 4): the running maxima move often and p is nearly
    # one-hot
    ("peaked_q4_T600_D64", 1, 600, 2, 64, dict(q_scale=4.0)),
    # compressor geometries other than l = 2 d (the generic importance and compression paths)
    ("cmp16x16_G4_T600_D64", 1, 600, 2, 64, dict(G=4, cmp_len=16, cmp_stride=16)),
    ("cmp48x16_T650_D128", 1, 650, 1, 128, dict(cmp_len=48, cmp_stride=16)),
    ("cmp64x32_G8_T700_D64", 1, 700, 2, 64, dict(G=8, cmp_len=64, cmp_stride=32)),
]


def shifted_bf16(bits, scale=1.0, offset=0.0):
    """bf16 bits of scale * x + offset, rounded to bf16 (an input transform)."""
    return S.f32_to_bf16_bits(S.bf16_bits_to_f32(bits) * np.float32(scale) + np.float32(offset))


@pytest.mark.parametrize("name,B,T,Hkv,D,extra", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(name, B, T, Hkv, D, extra):
    import dynamic_block_sparse_fwd_amd as nsa
    nsa.load_library()
    print("case backward", name, flush=True)
    extra = dict(extra)
    G = extra.pop("G", 16)
    v_offset, q_scale = extra.pop("v_offset", 0.0), extra.pop("q_scale", 1.0)
    ocfg = O.NsaCfg(B, T, Hkv, G, D, **extra)
    x = S.nsa_prefill_inputs(91 + len(name), B, T, Hkv, G, D, l=ocfg.cmp_len)
    if v_offset:
        x["v"] = shifted_bf16(x["v"], offset=v_offset)
    if q_scale != 1.0:
        x["q"] = shifted_bf16(x["q"], scale=q_scale)
    dout = S.upstream_grad(92 + len(name), (B, T, Hkv * G, D))
    kc = O.compress(x["k"], x["wk"], ocfg.cmp_len, ocfg.cmp_stride)
    vc = O.compress(x["v"], x["wv"], ocfg.cmp_len, ocfg.cmp_stride)
    rb, rt = np.meshgrid(np.arange(B), np.arange(T), indexing="ij")
    ora = O.nsa_prefill_rows(ocfg, x["q"], x["k"], x["v"], kc, vc, x["gate"],
                             rb.ravel().astype(np.int32), rt.ravel().astype(np.int32))
    idx = ora["idx"].reshape(B, T, Hkv, ocfg.top_n)
    f = NB.inputs_f64(x)
    ref = NB.backward(ocfg, f["q"], f["k"], f["v"], f["wk"], f["wv"], f["gate"], idx,
                      dout.astype(np.float64))
    cfg = nsa.NsaConfig(B, T, Hkv, G, D, ocfg.cmp_len, ocfg.cmp_stride, ocfg.sel_block,
                        ocfg.top_n, ocfg.n_local, ocfg.window, ocfg.scale)
    d = {k_: to_dev(v_) for k_, v_ in x.items()}
    args = (cfg, d["q"], d["k"], d["v"], d["wk"], d["wv"], d["gate"], to_dev(idx), to_dev(dout))
    got = nsa.nsa_backward(*args)
    again = nsa.nsa_backward(*args)  # deterministic: the same bits on a second call
    torch.cuda.synchronize()
    for n in got:
        assert torch.equal(got[n], again[n]), "%s: %s differs between two calls" % (name, n)
    msg = []
    for n in ("dq", "dk", "dv", "dwk", "dwv", "dgate"):
        mx, mean = check_grad(n, got[n].cpu().numpy(), ref[n], name)
        msg.append("%s %.1e/%.1e" % (n, mx, mean))
    print("%s: %s (max/mean error relative to the gradient's scale)" % (name, ", ".join(msg)),
          flush=True)


def test_backward_64k_sampled_rows():
    """The 64k prefill shape (1 x 65536, 4 KV heads x 16, D = 128) with a synthetic selection:
    dq and dgate on 60 sampled positions (the first rows, block edges, random ones) and dk, dv
    on the last 128 keys, which only the last 128 positions can see, against the oracle summed
    over exactly those positions."""
    import dynamic_block_sparse_fwd_amd as nsa
    nsa.load_library()
    B, T, Hkv, G, D = 1, 65536, 4, 16, 128
    print("case backward 64k", flush=True)
    ocfg = O.NsaCfg(B, T, Hkv, G, D)
    x = S.nsa_prefill_inputs(2, B, T, Hkv, G, D)
    dout = S.upstream_grad(7, (B, T, Hkv * G, D))
    idx = S.block_selection(B, T, Hkv)
    cfg = nsa.NsaConfig(B, T, Hkv, G, D)
    d = {k_: to_dev(v_) for k_, v_ in x.items()}
    got = nsa.nsa_backward(cfg, d["q"], d["k"], d["v"], d["wk"], d["wv"], d["gate"], to_dev(idx),
                           to_dev(dout))
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    sample = sorted(set([0, 1, 31, 32, 63, 64, 511, 512, 1023, 1024, 4095, 4096]) |
                    set(rng.integers(1025, T - 128, 48).tolist()))
    tail = list(range(T - 128, T))
    rows = sample + tail
    ri = torch.tensor(rows, device="cuda")
    gdq = got["dq"][:, ri].cpu().numpy()
    gdg = got["dgate"][:, ri].cpu().numpy()
    gdk = got["dk"][:, :, T - 128:].cpu().numpy()
    gdv = got["dv"][:, :, T - 128:].cpu().numpy()
    del got, d
    f = dict(q=S.bf16_bits_to_f32(x["q"]), k=NB.bf16_to_f64(x["k"]), v=NB.bf16_to_f64(x["v"]),
             wk=NB.bf16_to_f64(x["wk"]), wv=NB.bf16_to_f64(x["wv"]), gate=x["gate"])
    ref = NB.backward(ocfg, f["q"], f["k"], f["v"], f["wk"], f["wv"], f["gate"], idx, dout,
                      rows=rows)
    msg = []
    for n, gv, rv in (("dq", gdq, ref["dq"][:, rows]), ("dgate", gdg, ref["dgate"][:, rows]),
                      ("dk", gdk, ref["dk"][:, :, T - 128:]), ("dv", gdv, ref["dv"][:, :, T - 128:])):
        mx, mean = check_grad(n, gv, rv, "64k")
        msg.append("%s %.1e/%.1e" % (n, mx, mean))
    print("backward 64k sampled: %s" % ", ".join(msg), flush=True)
