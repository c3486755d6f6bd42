"""Pins of the fp64 oracle of the block (LayerNorm, GeLU, SWA, PTB forward and
backward) against facts that do not come from the oracle itself: closed forms,
invariants, brute force on tiny inputs, torch library routines and central
finite differences.  CPU only."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ptb
import torch_layer

MICRO = dict(batch=2, seq=8, hidden=16, n_heads=2, head_dim=8, ffn=32, window=3,
             add_residual=1, ln_eps=1e-5)


def micro_inputs(dims, seed=0, wstd=0.3):
    rng = np.random.default_rng(seed)
    T, h = dims["batch"] * dims["seq"], dims["hidden"]
    A = dims["n_heads"] * dims["head_dim"]
    F_ = dims["ffn"]
    return dict(x=rng.standard_normal((T, h)),
                gamma=1.0 + 0.2 * rng.standard_normal(h),
                beta=0.2 * rng.standard_normal(h),
                w_in=wstd * rng.standard_normal((3 * A + F_, h)),
                w_out=wstd * rng.standard_normal((A + F_, h)),
                dy=rng.standard_normal((T, h)))


# ---------------------------------------------------------------- LayerNorm
def test_layernorm_unit_affine_invariants():
    rng = np.random.default_rng(1)
    x = 3.0 + 2.0 * rng.standard_normal((7, 33))
    eps = 1e-5
    xn, xhat, mean, rstd = ptb.layernorm(x, np.ones(33), np.zeros(33), eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(xn.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose(xn.var(axis=1), var / (var + eps), rtol=1e-12)
    np.testing.assert_allclose(mean, x.mean(axis=1), rtol=1e-14)
    np.testing.assert_allclose(rstd, 1 / np.sqrt(var + eps), rtol=1e-14)


def test_layernorm_matches_torch():
    rng = np.random.default_rng(2)
    x, g, b = rng.standard_normal((5, 20)), rng.standard_normal(20), rng.standard_normal(20)
    xn, _, _, _ = ptb.layernorm(x, g, b, 1e-5)
    ref = F.layer_norm(torch.tensor(x), (20,), torch.tensor(g), torch.tensor(b), 1e-5).numpy()
    np.testing.assert_allclose(xn, ref, rtol=1e-12, atol=1e-12)


def test_layernorm_constant_row():
    x = np.full((1, 8), 2.5)
    xn, xhat, mean, rstd = ptb.layernorm(x, np.ones(8), np.full(8, 0.75), 1e-5)
    np.testing.assert_allclose(xn, 0.75)
    assert rstd[0] == pytest.approx(1 / math.sqrt(1e-5))


# ---------------------------------------------------------------- GeLU
def test_gelu_closed_forms():
    # GeLU(1) = Phi(1); GeLU(x) - GeLU(-x) = x because Phi(x) + Phi(-x) = 1.
    assert ptb.gelu(np.array([1.0]))[0] == pytest.approx(0.8413447460685429, rel=1e-15)
    assert ptb.gelu(np.array([0.0]))[0] == 0.0
    x = np.linspace(-6, 6, 101)
    np.testing.assert_allclose(ptb.gelu(x) - ptb.gelu(-x), x, atol=1e-14)
    ref = F.gelu(torch.tensor(x), approximate="none").numpy()
    np.testing.assert_allclose(ptb.gelu(x), ref, rtol=1e-13, atol=1e-15)


def test_gelu_grad_finite_difference():
    x = np.linspace(-5, 5, 41)
    hstep = 1e-6
    fd = (ptb.gelu(x + hstep) - ptb.gelu(x - hstep)) / (2 * hstep)
    np.testing.assert_allclose(ptb.gelu_grad(x), fd, rtol=1e-7, atol=1e-9)
    # d/dx at 0 is Phi(0) = 1/2
    assert ptb.gelu_grad(np.array([0.0]))[0] == pytest.approx(0.5, rel=1e-15)


# ---------------------------------------------------------------- SWA
def _sdpa(q, k, v, mask=None, causal=False):
    t = lambda a: torch.tensor(a)[None, None]
    return F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=None if mask is None else mask,
                                          is_causal=causal)[0, 0].numpy()


@pytest.mark.parametrize("s,d,w", [(16, 8, 16), (16, 8, 40), (33, 4, 33)])
def test_swa_window_ge_seq_is_causal(s, d, w):
    rng = np.random.default_rng(s + w)
    q, k, v = (rng.standard_normal((s, d)) for _ in range(3))
    o, p, lse = ptb.swa_head(q, k, v, w)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal=True), rtol=1e-12, atol=1e-12)


def test_swa_window_one_returns_v():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((12, 5)) for _ in range(3))
    o, p, lse = ptb.swa_head(q, k, v, 1)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, (q * k).sum(1) / math.sqrt(5), rtol=1e-14)


@pytest.mark.parametrize("w", [2, 3, 5])
def test_swa_band_mask_matches_sdpa(w):
    rng = np.random.default_rng(w)
    s, d = 14, 6
    q, k, v = (rng.standard_normal((s, d)) for _ in range(3))
    o, p, lse = ptb.swa_head(q, k, v, w)
    mask = torch.tensor(ptb.swa_visible(s, w))
    np.testing.assert_allclose(o, _sdpa(q, k, v, mask=mask), rtol=1e-12, atol=1e-12)
    # every row of P sums to one and is zero outside the window
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=1e-14)
    assert np.all(p[~ptb.swa_visible(s, w)] == 0)


def test_swa_brute_force_loops():
    """Triple loop with explicit window bounds, plain Python floats."""
    rng = np.random.default_rng(9)
    s, d, w = 7, 3, 3
    q, k, v = (rng.standard_normal((s, d)) for _ in range(3))
    o, _, lse = ptb.swa_head(q, k, v, w)
    for i in range(s):
        keys = range(max(0, i - w + 1), i + 1)
        sc = {j: sum(q[i, c] * k[j, c] for c in range(d)) / math.sqrt(d) for j in keys}
        z = sum(math.exp(sc[j]) for j in keys)
        assert lse[i] == pytest.approx(math.log(z), rel=1e-12)
        for c in range(d):
            ref = sum(math.exp(sc[j]) / z * v[j, c] for j in keys)
            assert o[i, c] == pytest.approx(ref, rel=1e-11, abs=1e-13)


def test_swa_backward_vs_autograd():
    rng = np.random.default_rng(4)
    s, d, w = 11, 4, 4
    q, k, v, do = (rng.standard_normal((s, d)) for _ in range(4))
    o, p, _ = ptb.swa_head(q, k, v, w)
    dq, dk, dv = ptb.swa_head_backward(q, k, v, p, do)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    out = F.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None],
                                         attn_mask=torch.tensor(ptb.swa_visible(s, w)))[0, 0]
    (out * torch.tensor(do)).sum().backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- PTB forward
def test_ptb_fused_equals_formula_terms():
    inp = micro_inputs(MICRO)
    y, _ = ptb.ptb_forward(MICRO, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    y2 = ptb.ptb_forward_branches(MICRO, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)


def test_ptb_forward_matches_torch_library_layer():
    inp = micro_inputs(MICRO)
    y, _ = ptb.ptb_forward(MICRO, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    yt, _ = torch_layer.layer_with_grads(MICRO, inp)
    np.testing.assert_allclose(y, yt, rtol=1e-11, atol=1e-11)


def test_ptb_single_branch_special_cases():
    """Zeroing one branch's output columns leaves x + the other branch,
    each computed here from torch library routines."""
    d = MICRO
    A = d["n_heads"] * d["head_dim"]
    inp = micro_inputs(d, seed=5)
    xn = F.layer_norm(torch.tensor(inp["x"]), (d["hidden"],), torch.tensor(inp["gamma"]),
                      torch.tensor(inp["beta"]), d["ln_eps"])
    w_in = torch.tensor(inp["w_in"])
    # MLP only
    w_out = inp["w_out"].copy()
    w_out[:A] = 0
    y, _ = ptb.ptb_forward(d, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], w_out)
    mlp = F.linear(F.gelu(F.linear(xn, w_in[3 * A:])), torch.tensor(w_out[A:].T)).numpy()
    np.testing.assert_allclose(y, inp["x"] + mlp, rtol=1e-11, atol=1e-12)
    # attention only
    w_out = inp["w_out"].copy()
    w_out[A:] = 0
    y, _ = ptb.ptb_forward(d, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], w_out)
    b, s, H, hd = d["batch"], d["seq"], d["n_heads"], d["head_dim"]
    heads = lambda t: t.reshape(b, s, H, hd).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(heads(F.linear(xn, w_in[:A])), heads(F.linear(xn, w_in[A:2 * A])),
                                       heads(F.linear(xn, w_in[2 * A:3 * A])),
                                       attn_mask=torch_layer.band_mask(s, d["window"]))
    att = F.linear(o.permute(0, 2, 1, 3).reshape(b * s, A), torch.tensor(w_out[:A].T)).numpy()
    np.testing.assert_allclose(y, inp["x"] + att, rtol=1e-11, atol=1e-12)


def test_ptb_differs_from_serial_block():
    inp = micro_inputs(MICRO, seed=6)
    y, _ = ptb.ptb_forward(MICRO, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    ys = ptb.serial_forward(MICRO, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    assert np.max(np.abs(y - ys)) > 1e-2


def test_no_residual_is_pure_partial():
    d0 = dict(MICRO, add_residual=0)
    inp = micro_inputs(MICRO, seed=7)
    y1, _ = ptb.ptb_forward(MICRO, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    y0, _ = ptb.ptb_forward(d0, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    np.testing.assert_allclose(y1 - y0, inp["x"], rtol=1e-12, atol=1e-12)


def test_sequences_in_a_batch_are_independent():
    inp = micro_inputs(MICRO, seed=8)
    y, _ = ptb.ptb_forward(MICRO, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    s = MICRO["seq"]
    one = dict(MICRO, batch=1)
    for bi in range(2):
        rows = slice(bi * s, (bi + 1) * s)
        yb, _ = ptb.ptb_forward(one, inp["x"][rows], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
        np.testing.assert_allclose(y[rows], yb, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- backward
def _loss(dims, inp, **over):
    a = dict(inp, **over)
    y, _ = ptb.ptb_forward(dims, a["x"], a["gamma"], a["beta"], a["w_in"], a["w_out"])
    return float(np.sum(y * inp["dy"]))


@pytest.mark.parametrize("add_residual", [1, 0])
def test_ptb_backward_finite_differences(add_residual):
    """Central differences on every element of every input and parameter."""
    dims = dict(MICRO, add_residual=add_residual)
    inp = micro_inputs(dims, seed=11)
    _, saved = ptb.ptb_forward(dims, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    g = ptb.ptb_backward(dims, inp["x"], inp["gamma"], inp["w_in"], inp["w_out"], saved, inp["dy"])
    names = dict(x="dx", gamma="dgamma", beta="dbeta", w_in="dw_in", w_out="dw_out")
    hstep = 1e-5
    for name, gname in names.items():
        base = inp[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += hstep
            minus[idx] -= hstep
            fd[idx] = (_loss(dims, inp, **{name: plus}) - _loss(dims, inp, **{name: minus})) / (2 * hstep)
        err = np.max(np.abs(fd - g[gname])) / np.max(np.abs(fd))
        assert err < 1e-6, (name, err)


def test_ptb_backward_matches_autograd_tiny_shape():
    dims = dict(batch=1, seq=64, hidden=64, n_heads=2, head_dim=16, ffn=96, window=9,
                add_residual=1, ln_eps=1e-5)
    inp = micro_inputs(dims, seed=12, wstd=0.1)
    y, saved = ptb.ptb_forward(dims, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    g = ptb.ptb_backward(dims, inp["x"], inp["gamma"], inp["w_in"], inp["w_out"], saved, inp["dy"])
    yt, gt = torch_layer.layer_with_grads(dims, inp)
    np.testing.assert_allclose(y, yt, rtol=1e-11, atol=1e-11)
    for k in ("x", "gamma", "beta", "w_in", "w_out"):
        np.testing.assert_allclose(g["d" + k], gt[k], rtol=1e-9, atol=1e-10)


# ---------------------------------------------------------------- TP shard semantics
def test_tensor_parallel_shards_sum_to_full_layer():
    """A full layer with 8 heads and FFN 64 split into 4 shards (row blocks of
    both weights):
    the shard outputs (residual only on shard 0) sum to the full layer, and so
    do dx, dgamma, dbeta; each shard's weight gradient is a slice of the full one."""
    n_shards, H_full, d, F_full, h = 4, 8, 4, 64, 24
    full = dict(batch=1, seq=10, hidden=h, n_heads=H_full, head_dim=d, ffn=F_full, window=4,
                add_residual=1, ln_eps=1e-5)
    inp = micro_inputs(full, seed=13, wstd=0.2)
    A, Hs, Fs = H_full * d, H_full // n_shards, F_full // n_shards
    As = Hs * d
    y, sv = ptb.ptb_forward(full, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    gf = ptb.ptb_backward(full, inp["x"], inp["gamma"], inp["w_in"], inp["w_out"], sv, inp["dy"])
    ysum = 0
    gsum = dict(dx=0, dgamma=0, dbeta=0)
    for r in range(n_shards):
        attn_rows = lambda base: np.arange(base + r * As, base + (r + 1) * As)
        rows = np.concatenate([attn_rows(0), attn_rows(A), attn_rows(2 * A),
                               3 * A + np.arange(r * Fs, (r + 1) * Fs)])
        out_rows = np.concatenate([np.arange(r * As, (r + 1) * As), A + np.arange(r * Fs, (r + 1) * Fs)])
        sd = dict(full, n_heads=Hs, ffn=Fs, add_residual=int(r == 0))
        w_in_s, w_out_s = inp["w_in"][rows], inp["w_out"][out_rows]
        ys, ss = ptb.ptb_forward(sd, inp["x"], inp["gamma"], inp["beta"], w_in_s, w_out_s)
        gs = ptb.ptb_backward(sd, inp["x"], inp["gamma"], w_in_s, w_out_s, ss, inp["dy"])
        ysum = ysum + ys
        for k in gsum:
            gsum[k] = gsum[k] + gs[k]
        np.testing.assert_allclose(gs["dw_in"], gf["dw_in"][rows], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(gs["dw_out"], gf["dw_out"][out_rows], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ysum, y, rtol=1e-11, atol=1e-11)
    for k in gsum:
        np.testing.assert_allclose(gsum[k], gf[k], rtol=1e-10, atol=1e-11)
