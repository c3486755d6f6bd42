"""fp64 oracle of the parallel transformer block (PTB) with causal
sliding-window attention (SWA), forward and backward.

Test infrastructure only (see the package docstring).

What is computed (MegaScale study guide, ch.2 §2.2 = paper §3.1, table of the
three algorithmic changes):
  * PTB row: the block output is the input plus an MLP branch and an attention
    branch that both read the SAME LayerNorm of the input, so one LN feeds
    both branches and their outputs are summed onto the residual.
  * SWA row: every token attends only to a fixed window of w tokens, cost
    O(s*w) instead of O(s*s).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * one LN with one (gamma, beta); biased variance; eps inside the square root;
  * no biases, no dropout;
  * exact erf GeLU;
  * causal window: key j is visible to query i iff 0 <= i - j < w, so exactly
    w keys including the query itself (fewer at the start of a sequence) and
    w >= s is plain causal attention;
  * softmax scale 1/sqrt(d);
  * w_in [3*H*d + F, hidden] rows are Q | K | V | FC1 (each of Q, K, V
    head-major); w_out [H*d + F, hidden] rows are the attention output
    projection (head-major) | FC2, so y = [O | GeLU(f)] @ w_out;
  * tensor parallel shard: the shard returns x + its partial sum when
    add_residual is set, else the pure partial sum.

Everything is float64 numpy.  Arrays are token-major: x is [T, hidden] with
T = batch * seq and the tokens of one sequence contiguous.
"""
from __future__ import annotations

import math
import numpy as np
from scipy.special import erf


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# LayerNorm (the one shared pre-LN of the PTB formula)
# --------------------------------------------------------------------------
def layernorm(x, gamma, beta, eps):
    """Row-wise LayerNorm: xn = (x - mean) / sqrt(var + eps) * gamma + beta.

    var is the biased (population) variance of the row.  Returns
    (xn, xhat, mean, rstd) where xhat = (x - mean) * rstd.
    """
    x = _f64(x)
    mean = x.mean(axis=1)
    centred = x - mean[:, None]
    var = (centred * centred).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = centred * rstd[:, None]
    xn = xhat * _f64(gamma)[None, :] + _f64(beta)[None, :]
    return xn, xhat, mean, rstd


def layernorm_backward(dxn, xhat, rstd, gamma):
    """Chain rule through the LayerNorm above.

    With dxhat = dxn * gamma and n the row width,
      dx = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat)),
      dgamma = sum over tokens of dxn * xhat,  dbeta = sum over tokens of dxn.
    """
    dxn = _f64(dxn)
    dgamma = (dxn * xhat).sum(axis=0)
    dbeta = dxn.sum(axis=0)
    dxhat = dxn * _f64(gamma)[None, :]
    m1 = dxhat.mean(axis=1, keepdims=True)
    m2 = (dxhat * xhat).mean(axis=1, keepdims=True)
    dx = rstd[:, None] * (dxhat - m1 - xhat * m2)
    return dx, dgamma, dbeta


# --------------------------------------------------------------------------
# GeLU (exact, erf form)
# --------------------------------------------------------------------------
def gelu(f):
    """GeLU(f) = f * Phi(f) with Phi the standard normal CDF."""
    f = _f64(f)
    return 0.5 * f * (1.0 + erf(f / math.sqrt(2.0)))


def gelu_grad(f):
    """d GeLU / df = Phi(f) + f * phi(f)."""
    f = _f64(f)
    cdf = 0.5 * (1.0 + erf(f / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * f * f) / math.sqrt(2.0 * math.pi)
    return cdf + f * pdf


# --------------------------------------------------------------------------
# Sliding-window attention, one sequence and one head
# --------------------------------------------------------------------------
def swa_visible(s, window):
    """Boolean [s, s]: key j visible to query i iff 0 <= i - j < window."""
    i = np.arange(s)[:, None]
    j = np.arange(s)[None, :]
    return (i - j >= 0) & (i - j < window)


def swa_head(q, k, v, window):
    """O = softmax(mask(q k^T / sqrt(d))) v for one sequence and one head.

    q, k, v: [s, d].  Returns (O [s, d], P [s, s], lse [s]) where lse is the
    natural log of the softmax normaliser of each query row (the log-sum-exp
    of its visible scaled scores).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    s, d = q.shape
    scores = (q @ k.T) / math.sqrt(d)
    vis = swa_visible(s, window)
    scores = np.where(vis, scores, -np.inf)
    rowmax = scores.max(axis=1, keepdims=True)      # finite: the diagonal is visible
    e = np.exp(scores - rowmax)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    lse = (rowmax + np.log(z))[:, 0]
    return p @ v, p, lse


def swa_head_backward(q, k, v, p, d_o):
    """Chain rule through swa_head given its probabilities P.

    dP = dO v^T; dV = P^T dO; softmax Jacobian per row:
    dS = P * (dP - sum_j P dP); scores were scaled by 1/sqrt(d), so
    dQ = dS k / sqrt(d) and dK = dS^T q / sqrt(d).  Masked entries have P = 0
    and so get no gradient.
    """
    q, k, v, d_o = _f64(q), _f64(k), _f64(v), _f64(d_o)
    d = q.shape[1]
    dp = d_o @ v.T
    dv = p.T @ d_o
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = ds @ k / math.sqrt(d)
    dk = ds.T @ q / math.sqrt(d)
    return dq, dk, dv


# --------------------------------------------------------------------------
# The block
# --------------------------------------------------------------------------
def _split(dims):
    b, s, H, d = dims["batch"], dims["seq"], dims["n_heads"], dims["head_dim"]
    A = H * d
    return b, s, H, d, A, dims["ffn"]


def attention(dims, q, k, v):
    """Multi-head SWA over token-major q, k, v [T, A]; returns O [T, A], P, lse.

    P is a dict (batch, head) -> [s, s]; lse is [batch, H, s].
    """
    b, s, H, d, A, _ = _split(dims)
    out = np.zeros((b * s, A))
    probs = {}
    lse = np.zeros((b, H, s))
    for bi in range(b):
        rows = slice(bi * s, (bi + 1) * s)
        for h in range(H):
            cols = slice(h * d, (h + 1) * d)
            o, p, l = swa_head(q[rows, cols], k[rows, cols], v[rows, cols], dims["window"])
            out[rows, cols] = o
            probs[(bi, h)] = p
            lse[bi, h] = l
    return out, probs, lse


def attn_branch(dims, xn, w_in, w_out):
    """Attention(LN(x)) of the PTB formula: heads of SWA, then the output projection."""
    _, _, _, _, A, _ = _split(dims)
    w_in, w_out = _f64(w_in), _f64(w_out)
    q = xn @ w_in[0:A].T
    k = xn @ w_in[A:2 * A].T
    v = xn @ w_in[2 * A:3 * A].T
    o, _, _ = attention(dims, q, k, v)
    return o @ w_out[:A]


def mlp_branch(dims, xn, w_in, w_out):
    """MLP(LN(x)) of the PTB formula: FC1, GeLU, FC2."""
    _, _, _, _, A, _ = _split(dims)
    w_in, w_out = _f64(w_in), _f64(w_out)
    f = xn @ w_in[3 * A:].T
    return gelu(f) @ w_out[A:]


def ptb_forward(dims, x, gamma, beta, w_in, w_out):
    """y = [x] + MLP(LN(x)) + Attention(LN(x)), written as the fused shard.

    The two branches are computed as one input projection [q|k|v|f] and one
    output projection over [O | GeLU(f)], which is the same sum.  Returns y
    and a dict of intermediates used by the backward and by tests.
    """
    _, _, _, _, A, _ = _split(dims)
    x, w_in, w_out = _f64(x), _f64(w_in), _f64(w_out)
    xn, xhat, mean, rstd = layernorm(x, gamma, beta, dims["ln_eps"])
    z = xn @ w_in.T
    q, k, v, f = z[:, :A], z[:, A:2 * A], z[:, 2 * A:3 * A], z[:, 3 * A:]
    o, probs, lse = attention(dims, q, k, v)
    g = gelu(f)
    cat = np.concatenate([o, g], axis=1)
    y = cat @ w_out
    if dims["add_residual"]:
        y = y + x
    saved = dict(xn=xn, xhat=xhat, mean=mean, rstd=rstd, q=q, k=k, v=v, f=f,
                 o=o, g=g, cat=cat, probs=probs, lse=lse)
    return y, saved


def ptb_forward_branches(dims, x, gamma, beta, w_in, w_out):
    """The PTB formula term by term: x + MLP(LN(x)) + Attention(LN(x))."""
    xn, _, _, _ = layernorm(x, gamma, beta, dims["ln_eps"])
    y = mlp_branch(dims, xn, w_in, w_out) + attn_branch(dims, xn, w_in, w_out)
    if dims["add_residual"]:
        y = y + _f64(x)
    return y


def serial_forward(dims, x, gamma, beta, w_in, w_out, gamma2=None, beta2=None):
    """The serial pre-LN block the PTB replaces, for contrast in tests:
    h = x + Attention(LN1(x)); y = h + MLP(LN2(h))."""
    g2 = gamma if gamma2 is None else gamma2
    b2 = beta if beta2 is None else beta2
    y, _ = serial_block_forward(dims, x, gamma, beta, g2, b2, w_in, w_out)
    return y


# --------------------------------------------------------------------------
# The serial pre-LN block (the arrangement the PTB row replaces)
# --------------------------------------------------------------------------
# The page writes the serial block as y = x + MLP(LN(x + Attention(LN(x)))),
# which drops the residual around the attention sub-layer; the block the PTB
# row contrasts with is the usual pre-LN transformer layer, read here as
#   h = x + Attention(LN1(x)),   y = h + MLP(LN2(h)),
# with its own (gamma, beta) per LayerNorm and the same projections as the
# PTB: w_in rows Q | K | V | FC1, w_out rows attention-out | FC2.  Both
# residuals are always present (LN2 needs the whole h, so the serial block is
# not a sum of per-branch partials).
def serial_block_forward(dims, x, gamma1, beta1, gamma2, beta2, w_in, w_out):
    """Returns y and the intermediates its backward uses."""
    _, _, _, _, A, _ = _split(dims)
    x, w_in, w_out = _f64(x), _f64(w_in), _f64(w_out)
    xn1, xhat1, _, rstd1 = layernorm(x, gamma1, beta1, dims["ln_eps"])
    q = xn1 @ w_in[0:A].T
    k = xn1 @ w_in[A:2 * A].T
    v = xn1 @ w_in[2 * A:3 * A].T
    o, probs, lse = attention(dims, q, k, v)
    hid = x + o @ w_out[:A]
    xn2, xhat2, _, rstd2 = layernorm(hid, gamma2, beta2, dims["ln_eps"])
    f = xn2 @ w_in[3 * A:].T
    g = gelu(f)
    y = hid + g @ w_out[A:]
    saved = dict(xn1=xn1, xhat1=xhat1, rstd1=rstd1, q=q, k=k, v=v, o=o, probs=probs, lse=lse,
                 h=hid, xn2=xn2, xhat2=xhat2, rstd2=rstd2, f=f, g=g)
    return y, saved


def serial_block_backward(dims, gamma1, gamma2, w_in, w_out, saved, dy):
    """Gradients of sum(y * dy) through the serial block, sub-layer by
    sub-layer in reverse: FC2, GeLU, FC1, LN2 (plus the residual into h),
    the attention output projection, SWA, the Q/K/V projection, LN1 (plus
    the residual into x)."""
    b, s, H, d, A, _ = _split(dims)
    w_in, w_out, dy = _f64(w_in), _f64(w_out), _f64(dy)
    dw_fc2 = saved["g"].T @ dy
    df = (dy @ w_out[A:].T) * gelu_grad(saved["f"])
    dw_fc1 = df.T @ saved["xn2"]
    dxn2 = df @ w_in[3 * A:]
    dh_ln, dgamma2, dbeta2 = layernorm_backward(dxn2, saved["xhat2"], saved["rstd2"], gamma2)
    dh = dy + dh_ln
    dw_o = saved["o"].T @ dh
    d_o = dh @ w_out[:A].T
    dq = np.zeros_like(d_o)
    dk = np.zeros_like(d_o)
    dv = np.zeros_like(d_o)
    for bi in range(b):
        rows = slice(bi * s, (bi + 1) * s)
        for hh in range(H):
            cols = slice(hh * d, (hh + 1) * d)
            dq[rows, cols], dk[rows, cols], dv[rows, cols] = swa_head_backward(
                saved["q"][rows, cols], saved["k"][rows, cols], saved["v"][rows, cols],
                saved["probs"][(bi, hh)], d_o[rows, cols])
    dqkv = np.concatenate([dq, dk, dv], axis=1)
    dw_qkv = dqkv.T @ saved["xn1"]
    dxn1 = dqkv @ w_in[:3 * A]
    dx_ln, dgamma1, dbeta1 = layernorm_backward(dxn1, saved["xhat1"], saved["rstd1"], gamma1)
    return dict(dx=dh + dx_ln, dgamma1=dgamma1, dbeta1=dbeta1, dgamma2=dgamma2, dbeta2=dbeta2,
                dw_in=np.concatenate([dw_qkv, dw_fc1], axis=0),
                dw_out=np.concatenate([dw_o, dw_fc2], axis=0), dh=dh, d_o=d_o)


def ptb_backward(dims, x, gamma, w_in, w_out, saved, dy):
    """Gradients of sum(y * dy) w.r.t. x, gamma, beta, w_in, w_out."""
    b, s, H, d, A, _ = _split(dims)
    w_in, w_out, dy = _f64(w_in), _f64(w_out), _f64(dy)
    cat = saved["cat"]
    dw_out = cat.T @ dy
    dcat = dy @ w_out.T
    d_o, dg = dcat[:, :A], dcat[:, A:]
    df = dg * gelu_grad(saved["f"])
    dq = np.zeros_like(d_o)
    dk = np.zeros_like(d_o)
    dv = np.zeros_like(d_o)
    for bi in range(b):
        rows = slice(bi * s, (bi + 1) * s)
        for h in range(H):
            cols = slice(h * d, (h + 1) * d)
            dq[rows, cols], dk[rows, cols], dv[rows, cols] = swa_head_backward(
                saved["q"][rows, cols], saved["k"][rows, cols], saved["v"][rows, cols],
                saved["probs"][(bi, h)], d_o[rows, cols])
    dz = np.concatenate([dq, dk, dv, df], axis=1)
    dw_in = dz.T @ saved["xn"]
    dxn = dz @ w_in
    dx, dgamma, dbeta = layernorm_backward(dxn, saved["xhat"], saved["rstd"], gamma)
    if dims["add_residual"]:
        dx = dx + dy
    return dict(dx=dx, dgamma=dgamma, dbeta=dbeta, dw_in=dw_in, dw_out=dw_out,
                dz=dz, dcat=dcat, dxn=dxn)


def dims_of(cfg) -> dict:
    """A plain dict of layer dimensions from any object with those attributes."""
    keys = ("batch", "seq", "hidden", "n_heads", "head_dim", "ffn", "window",
            "add_residual", "ln_eps")
    if isinstance(cfg, dict):
        return {k: cfg[k] for k in keys}
    return {k: getattr(cfg, k) for k in keys}
