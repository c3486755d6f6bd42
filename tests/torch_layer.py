"""An independent fp64 CPU implementation of the block written with torch
library routines (layer_norm, linear, scaled_dot_product_attention with a
boolean band mask, gelu) and differentiated by torch.autograd.

It is a second, library-based construction of the same maths used only to pin
the hand-written oracle; it shares no code with the oracle or the HIP path.
"""
import torch
import torch.nn.functional as F


def band_mask(s, window):
    i = torch.arange(s)[:, None]
    j = torch.arange(s)[None, :]
    return (i >= j) & (i - j < window)


def layer(dims, x, gamma, beta, w_in, w_out):
    b, s, H, d = dims["batch"], dims["seq"], dims["n_heads"], dims["head_dim"]
    A = H * d
    xn = F.layer_norm(x, (x.shape[1],), gamma, beta, dims["ln_eps"])
    z = F.linear(xn, w_in)
    q, k, v, f = z[:, :A], z[:, A:2 * A], z[:, 2 * A:3 * A], z[:, 3 * A:]

    def heads(t):
        return t.reshape(b, s, H, d).permute(0, 2, 1, 3)

    o = F.scaled_dot_product_attention(heads(q), heads(k), heads(v),
                                       attn_mask=band_mask(s, dims["window"]))
    o = o.permute(0, 2, 1, 3).reshape(b * s, A)
    attn = o @ w_out[:A]
    mlp = F.gelu(f) @ w_out[A:]
    y = attn + mlp
    if dims["add_residual"]:
        y = y + x
    return y


def layer_with_grads(dims, inputs):
    """Returns y and the gradients of sum(y * dy) (all fp64, CPU)."""
    names = ("x", "gamma", "beta", "w_in", "w_out")
    leaves = {k: torch.tensor(inputs[k], dtype=torch.float64, requires_grad=True) for k in names}
    y = layer(dims, *(leaves[k] for k in names))
    dy = torch.tensor(inputs["dy"], dtype=torch.float64)
    (y * dy).sum().backward()
    return y.detach().numpy(), {k: leaves[k].grad.numpy() for k in names}


def serial_layer(dims, x, gamma1, beta1, gamma2, beta2, w_in, w_out):
    """The serial pre-LN block: h = x + Attention(LN1(x)); y = h + MLP(LN2(h))."""
    b, s, H, d = dims["batch"], dims["seq"], dims["n_heads"], dims["head_dim"]
    A = H * d
    xn1 = F.layer_norm(x, (x.shape[1],), gamma1, beta1, dims["ln_eps"])

    def heads(t):
        return t.reshape(b, s, H, d).permute(0, 2, 1, 3)

    o = F.scaled_dot_product_attention(heads(F.linear(xn1, w_in[:A])),
                                       heads(F.linear(xn1, w_in[A:2 * A])),
                                       heads(F.linear(xn1, w_in[2 * A:3 * A])),
                                       attn_mask=band_mask(s, dims["window"]))
    hid = x + o.permute(0, 2, 1, 3).reshape(b * s, A) @ w_out[:A]
    xn2 = F.layer_norm(hid, (hid.shape[1],), gamma2, beta2, dims["ln_eps"])
    return hid + F.gelu(F.linear(xn2, w_in[3 * A:])) @ w_out[A:]


def serial_layer_with_grads(dims, inputs):
    names = ("x", "gamma1", "beta1", "gamma2", "beta2", "w_in", "w_out")
    leaves = {k: torch.tensor(inputs[k], dtype=torch.float64, requires_grad=True) for k in names}
    y = serial_layer(dims, *(leaves[k] for k in names))
    dy = torch.tensor(inputs["dy"], dtype=torch.float64)
    (y * dy).sum().backward()
    return y.detach().numpy(), {k: leaves[k].grad.numpy() for k in names}
