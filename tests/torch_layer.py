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
