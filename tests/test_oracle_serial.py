"""Pins of the oracle's serial pre-LN block (h = x + Attention(LN1(x)),
y = h + MLP(LN2(h))), the arrangement the PTB replaces: central finite
differences, torch library routines with autograd, and the special cases that
reduce it to one sub-layer.  CPU only."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ptb
import torch_layer

MICRO = dict(batch=2, seq=8, hidden=16, n_heads=2, head_dim=8, ffn=32, window=3,
             add_residual=1, ln_eps=1e-5)
NAMES = ("x", "gamma1", "beta1", "gamma2", "beta2", "w_in", "w_out")


def serial_inputs(dims, seed=0, wstd=0.3):
    rng = np.random.default_rng(seed)
    T, h = dims["batch"] * dims["seq"], dims["hidden"]
    A = dims["n_heads"] * dims["head_dim"]
    F_ = dims["ffn"]
    return dict(x=rng.standard_normal((T, h)),
                gamma1=1.0 + 0.2 * rng.standard_normal(h), beta1=0.2 * rng.standard_normal(h),
                gamma2=1.0 + 0.2 * rng.standard_normal(h), beta2=0.2 * rng.standard_normal(h),
                w_in=wstd * rng.standard_normal((3 * A + F_, h)),
                w_out=wstd * rng.standard_normal((A + F_, h)),
                dy=rng.standard_normal((T, h)))


def _fwd(dims, a):
    return ptb.serial_block_forward(dims, *(a[k] for k in NAMES))


def test_serial_forward_matches_torch_library_layer():
    inp = serial_inputs(MICRO, seed=1)
    y, _ = _fwd(MICRO, inp)
    yt, _ = torch_layer.serial_layer_with_grads(MICRO, inp)
    np.testing.assert_allclose(y, yt, rtol=1e-11, atol=1e-11)


def test_serial_single_sublayer_special_cases():
    """Zero attention-out rows: h = x, y = x + MLP(LN2(x)).  Zero FC2 rows:
    y = h = x + Attention(LN1(x)).  Each side computed with torch routines."""
    d = MICRO
    A = d["n_heads"] * d["head_dim"]
    inp = serial_inputs(d, seed=2)
    x = torch.tensor(inp["x"])
    w_in = torch.tensor(inp["w_in"])
    w_out = inp["w_out"].copy()
    w_out[:A] = 0
    y, _ = _fwd(d, dict(inp, w_out=w_out))
    xn2 = F.layer_norm(x, (d["hidden"],), torch.tensor(inp["gamma2"]), torch.tensor(inp["beta2"]),
                       d["ln_eps"])
    ref = x + F.gelu(F.linear(xn2, w_in[3 * A:])) @ torch.tensor(w_out[A:])
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-11, atol=1e-12)
    w_out = inp["w_out"].copy()
    w_out[A:] = 0
    y, saved = _fwd(d, dict(inp, w_out=w_out))
    np.testing.assert_allclose(y, saved["h"], rtol=0, atol=0)
    b, s, H, hd = d["batch"], d["seq"], d["n_heads"], d["head_dim"]
    xn1 = F.layer_norm(x, (d["hidden"],), torch.tensor(inp["gamma1"]), torch.tensor(inp["beta1"]),
                       d["ln_eps"])
    heads = lambda t: t.reshape(b, s, H, hd).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(heads(F.linear(xn1, w_in[:A])), heads(F.linear(xn1, w_in[A:2 * A])),
                                       heads(F.linear(xn1, w_in[2 * A:3 * A])),
                                       attn_mask=torch_layer.band_mask(s, d["window"]))
    ref = x + o.permute(0, 2, 1, 3).reshape(b * s, A) @ torch.tensor(w_out[:A])
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_serial_shares_ln_params_with_old_helper():
    inp = serial_inputs(MICRO, seed=3)
    y, _ = _fwd(MICRO, dict(inp, gamma2=inp["gamma1"], beta2=inp["beta1"]))
    y2 = ptb.serial_forward(MICRO, inp["x"], inp["gamma1"], inp["beta1"], inp["w_in"], inp["w_out"])
    np.testing.assert_allclose(y, y2, rtol=0, atol=0)


def _loss(dims, inp, **over):
    y, _ = _fwd(dims, dict(inp, **over))
    return float(np.sum(y * inp["dy"]))


def test_serial_backward_finite_differences():
    """Central differences on every element of every input and parameter."""
    inp = serial_inputs(MICRO, seed=11)
    _, saved = _fwd(MICRO, inp)
    g = ptb.serial_block_backward(MICRO, inp["gamma1"], inp["gamma2"], inp["w_in"], inp["w_out"],
                                  saved, inp["dy"])
    hstep = 1e-5
    for name in NAMES:
        base = inp[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += hstep
            minus[idx] -= hstep
            fd[idx] = (_loss(MICRO, inp, **{name: plus}) - _loss(MICRO, inp, **{name: minus})) / (2 * hstep)
        err = np.max(np.abs(fd - g["d" + name])) / np.max(np.abs(fd))
        assert err < 1e-6, (name, err)


def test_serial_backward_matches_autograd_tiny_shape():
    dims = dict(batch=1, seq=64, hidden=64, n_heads=2, head_dim=16, ffn=96, window=9,
                add_residual=1, ln_eps=1e-5)
    inp = serial_inputs(dims, seed=12, wstd=0.1)
    y, saved = _fwd(dims, inp)
    g = ptb.serial_block_backward(dims, inp["gamma1"], inp["gamma2"], inp["w_in"], inp["w_out"],
                                  saved, inp["dy"])
    yt, gt = torch_layer.serial_layer_with_grads(dims, inp)
    np.testing.assert_allclose(y, yt, rtol=1e-11, atol=1e-11)
    for k in NAMES:
        np.testing.assert_allclose(g["d" + k], gt[k], rtol=1e-9, atol=1e-10)
