"""Pins of the fp64 backward oracle (oracle/nsa_backward.py), CPU only.

  * its forward, on the seeded bf16 inputs, equals the C oracle's forward (two independent
    implementations of the same readings);
  * every gradient equals a central finite difference of that forward along a random
    direction (selection held fixed, compressed rounding off);
  * special cases that reduce to full causal attention (the selected branch with every block
    selected, the window branch with w >= T, the compressed branch with l = d = 1 and W = I)
    match torch's fp64 autograd of scaled_dot_product_attention.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth_inputs as S
from oracle import nsa_backward as NB


def setup(seed=51, B=1, T=200, Hkv=2, G=2, D=16, **kw):
    cfg = O.NsaCfg(B, T, Hkv, G, D, **kw)
    x = S.nsa_prefill_inputs(seed, B, T, Hkv, G, D, l=cfg.cmp_len)
    kc = O.compress(x["k"], x["wk"], cfg.cmp_len, cfg.cmp_stride)
    vc = O.compress(x["v"], x["wv"], cfg.cmp_len, cfg.cmp_stride)
    rb, rt = np.meshgrid(np.arange(B), np.arange(T), indexing="ij")
    ora = O.nsa_prefill_rows(cfg, x["q"], x["k"], x["v"], kc, vc, x["gate"],
                             rb.ravel().astype(np.int32), rt.ravel().astype(np.int32))
    idx = ora["idx"].reshape(B, T, Hkv, cfg.top_n)
    return cfg, x, idx, ora["out"].reshape(B, T, cfg.Hq, D)


def test_forward_equals_c_oracle():
    for kw in ({}, dict(top_n=4, n_local=1, window=50), dict(sel_block=128, top_n=3),
               dict(cmp_len=16, cmp_stride=16), dict(cmp_len=48, cmp_stride=16),
               dict(cmp_len=64, cmp_stride=32)):
        cfg, x, idx, ref = setup(T=300, **kw)
        f = NB.inputs_f64(x)
        out = NB.forward(cfg, f["q"], f["k"], f["v"], f["wk"], f["wv"], f["gate"], idx)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["q", "k", "v", "wk", "wv", "gate"])
def test_gradients_match_finite_differences(name):
    cfg, x, idx, _ = setup(T=170, G=2, D=16, top_n=4, n_local=1, window=40)
    f = NB.inputs_f64(x)
    dout = S.upstream_grad(52, f["q"].shape).astype(np.float64)
    g = NB.backward(cfg, f["q"], f["k"], f["v"], f["wk"], f["wv"], f["gate"], idx, dout,
                    round_cmp=False)["d" + name]
    u = np.random.default_rng(53).standard_normal(f[name].shape)
    eps = 1e-5

    def loss(delta):
        ff = dict(f)
        ff[name] = f[name] + delta * u
        return float(np.sum(dout * NB.forward(cfg, ff["q"], ff["k"], ff["v"], ff["wk"], ff["wv"],
                                              ff["gate"], idx, round_cmp=False)))

    fd = (loss(eps) - loss(-eps)) / (2 * eps)
    an = float(np.sum(g * u))
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.parametrize("l,d", [(16, 16), (48, 16), (64, 32)])
def test_generic_compressor_gradients_match_finite_differences(l, d):
    """Compressor geometries other than l = 2 d (l = d, l = 3 d, l = 2 d with d = 32): every
    gradient against a central finite difference along a random direction, as above."""
    cfg, x, idx, _ = setup(seed=54 + l + d, T=160, G=2, D=16, top_n=4, n_local=1, window=40,
                           cmp_len=l, cmp_stride=d)
    f = NB.inputs_f64(x)
    dout = S.upstream_grad(55, f["q"].shape).astype(np.float64)
    grads = NB.backward(cfg, f["q"], f["k"], f["v"], f["wk"], f["wv"], f["gate"], idx, dout,
                        round_cmp=False)
    for i, name in enumerate(["q", "k", "v", "wk", "wv", "gate"]):
        u = np.random.default_rng(56 + i).standard_normal(f[name].shape)
        eps = 1e-5

        def loss(delta):
            ff = dict(f)
            ff[name] = f[name] + delta * u
            return float(np.sum(dout * NB.forward(cfg, ff["q"], ff["k"], ff["v"], ff["wk"],
                                                  ff["wv"], ff["gate"], idx, round_cmp=False)))

        fd = (loss(eps) - loss(-eps)) / (2 * eps)
        an = float(np.sum(grads["d" + name] * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (l, d, name, fd, an)


def sdpa_grads(q, k, v, dout, scale, window=None):
    """q [T,H,D] (H query heads sharing one K/V [T,D]), causal (optionally banded)."""
    T, H, D = q.shape
    qt = torch.tensor(q.transpose(1, 0, 2), requires_grad=True)
    kt = torch.tensor(np.broadcast_to(k, (H, T, D)).copy())
    vt = torch.tensor(np.broadcast_to(v, (H, T, D)).copy())
    kt.requires_grad_(True)
    vt.requires_grad_(True)
    mask = None
    if window is not None:
        i = torch.arange(T)
        mask = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - window)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, is_causal=mask is None, scale=scale)
    o.backward(torch.tensor(dout.transpose(1, 0, 2)))
    return (qt.grad.numpy().transpose(1, 0, 2), kt.grad.numpy().sum(0), vt.grad.numpy().sum(0))


@pytest.mark.parametrize("branch", ["selected", "window", "compressed"])
def test_special_cases_equal_sdpa_autograd(branch):
    T, G, D = 150, 3, 16
    kw = dict(selected=dict(top_n=3, sel_block=64), window=dict(window=40),
              compressed=dict(cmp_len=1, cmp_stride=1))[branch]
    cfg, x, idx, _ = setup(T=T, Hkv=1, G=G, D=D, **kw)
    f = NB.inputs_f64(x)
    br = dict(compressed=0, selected=1, window=2)[branch]
    f["gate"] = np.zeros_like(f["gate"])
    f["gate"][..., br] = 1.0
    if branch == "compressed":
        f["wk"] = np.eye(D)[None].copy()
        f["wv"] = np.eye(D)[None].copy()
    dout = S.upstream_grad(54, f["q"].shape).astype(np.float64)
    g = NB.backward(cfg, f["q"], f["k"], f["v"], f["wk"], f["wv"], f["gate"], idx, dout)
    rq, rk, rv = sdpa_grads(f["q"][0], f["k"][0, 0], f["v"][0, 0], dout[0], cfg.scale,
                            window=40 if branch == "window" else None)
    np.testing.assert_allclose(g["dq"][0], rq, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dk"][0, 0], rk, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dv"][0, 0], rv, rtol=0, atol=1e-11)
    if branch != "compressed":
        assert not g["dwk"].any() and not g["dwv"].any()


def test_row_restricted_backward_is_exact_where_claimed():
    """rows=[...]: dq and dgate on those rows, and dk/dv on keys only those rows see, equal the
    full backward's."""
    cfg, x, idx, _ = setup(T=260, G=2, D=16, window=40)
    f = NB.inputs_f64(x)
    dout = S.upstream_grad(55, f["q"].shape).astype(np.float64)
    full = NB.backward(cfg, f["q"], f["k"], f["v"], f["wk"], f["wv"], f["gate"], idx, dout)
    rows = [3, 77, 150] + list(range(200, 260))
    part = NB.backward(cfg, f["q"], f["k"], f["v"], f["wk"], f["wv"], f["gate"], idx, dout,
                       rows=rows)
    np.testing.assert_allclose(part["dq"][:, rows], full["dq"][:, rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(part["dgate"][:, rows], full["dgate"][:, rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(part["dk"][:, :, 200:], full["dk"][:, :, 200:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(part["dv"][:, :, 200:], full["dv"][:, :, 200:], rtol=0, atol=1e-12)
