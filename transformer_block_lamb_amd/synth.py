"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and rounds them to the storage type; it
holds none of the layer's or the optimizer's arithmetic.  The oracle never
imports it; the tests and the bench feed its arrays to both the oracle and the
HIP library.

Recipe (one numpy PCG64 stream per tensor, spawned from one seed in a fixed
order x, gamma, beta, w_in, w_out, dy):
  x, dy        ~ N(0, 1)
  w_in, w_out  ~ N(0, 0.02)          (sigma is the standard deviation)
  gamma = 1, beta = 0                (or N(1, 0.1) / N(0, 0.1) when
                                      ``ln_affine="random"``, used by parity
                                      tests so that a gamma/beta mix-up shows)
For bf16 runs every value is drawn in fp32 and rounded once to bf16
(round-to-nearest-even); both sides then consume those same bf16 values.

The shapes are one tensor-parallel shard (TP=8) of the 175B and 530B layer
configurations of MegaScale (Table 1 on the MegaScale study-guide page), plus a
tiny and a small layer.  Weight layouts:
  w_in  [3*H*d + F, hidden]  rows: Q (head-major) | K | V | FC1
  w_out [H*d + F, hidden]    rows: attention output projection (head-major) | FC2
"""
from __future__ import annotations

import dataclasses
import numpy as np

SEED = 1234


@dataclasses.dataclass(frozen=True)
class PtbConfig:
    name: str
    batch: int
    seq: int
    hidden: int
    n_heads: int
    head_dim: int
    ffn: int
    window: int
    dtype: str = "bf16"          # "bf16" or "f32"
    add_residual: int = 1
    ln_eps: float = 1e-5

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def attn_width(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def n_in(self) -> int:
        return 3 * self.attn_width + self.ffn

    @property
    def k_out(self) -> int:
        return self.attn_width + self.ffn

    def replace(self, **kw) -> "PtbConfig":
        return dataclasses.replace(self, **kw)


# Named workloads.  "tiny" is the fp32 case the oracle finishes instantly; the
# 175B shard at window 512 is the headline workload.
CONFIGS = {
    "tiny": PtbConfig("tiny", 1, 128, 256, 4, 64, 1024, 32, "f32"),
    "small": PtbConfig("small", 4, 2048, 2048, 16, 128, 8192, 512, "bf16"),
    "175b_w512": PtbConfig("175b_w512", 1, 2048, 12288, 16, 96, 6144, 512, "bf16"),
    "175b_w2048": PtbConfig("175b_w2048", 1, 2048, 12288, 16, 96, 6144, 2048, "bf16"),
    "530b_w512": PtbConfig("530b_w512", 1, 2048, 20480, 20, 128, 10240, 512, "bf16"),
}

# The parameter tensors of one 175B TP=8 layer shard, in optimizer order.
LAMB_175B_TENSORS = (
    ("w_qkv", 3 * 1536 * 12288),
    ("w_fc1", 6144 * 12288),
    ("w_o", 1536 * 12288),
    ("w_fc2", 12288 * 6144),
    ("ln_gamma", 12288),
    ("ln_beta", 12288),
)
LAMB_HPARAMS = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-6, weight_decay=0.01)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return fp32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # finite inputs only: the carry never leaves 32 bits below the NaN range
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of values that are already bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal(rng, shape, std, mean=0.0):
    out = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    if mean != 0.0:
        out += np.float32(mean)
    return out


def ptb_inputs(cfg: PtbConfig, seed: int = SEED, ln_affine: str = "unit",
               weight_std: float = 0.02) -> dict:
    """fp32 arrays (bf16-exact when cfg.dtype == "bf16") for one layer call."""
    T, h = cfg.tokens, cfg.hidden
    r = _streams(seed, 6)
    x = _normal(r[0], (T, h), 1.0)
    if ln_affine == "unit":
        gamma = np.ones(h, np.float32)
        beta = np.zeros(h, np.float32)
    elif ln_affine == "random":
        gamma = _normal(r[1], (h,), 0.1, 1.0)
        beta = _normal(r[2], (h,), 0.1)
    else:
        raise ValueError(ln_affine)
    w_in = _normal(r[3], (cfg.n_in, h), weight_std)
    w_out = _normal(r[4], (cfg.k_out, h), weight_std)
    dy = _normal(r[5], (T, h), 1.0)
    out = dict(x=x, gamma=gamma, beta=beta, w_in=w_in, w_out=w_out, dy=dy)
    if cfg.dtype == "bf16":
        # gamma/beta stay fp32 (LN parameters are kept in fp32 on both sides).
        for k in ("x", "w_in", "w_out", "dy"):
            out[k] = bf16_round(out[k])
    return out


def second_ln_params(cfg: PtbConfig, seed: int = SEED + 2, ln_affine: str = "unit"):
    """(gamma2, beta2) fp32 for the serial block's second LayerNorm."""
    h = cfg.hidden
    if ln_affine == "unit":
        return np.ones(h, np.float32), np.zeros(h, np.float32)
    r = _streams(seed, 2)
    return _normal(r[0], (h,), 0.1, 1.0), _normal(r[1], (h,), 0.1)


def lamb_inputs(sizes, seed: int = SEED + 1, grad_std: float = 1e-3,
                grad_dtype: str = "bf16", gamma_beta_tail: bool = True) -> list:
    """Per tensor: fp32 master w, bf16-exact (or fp32) gradient g, m = v = 0.

    Matrices ~ N(0, 0.02); when ``gamma_beta_tail`` the last two tensors are a
    LayerNorm gamma (ones) and beta (zeros), as in one layer shard.
    """
    r = _streams(seed, 2 * len(sizes))
    out = []
    for i, n in enumerate(sizes):
        if gamma_beta_tail and i == len(sizes) - 2:
            w = np.ones(n, np.float32)
        elif gamma_beta_tail and i == len(sizes) - 1:
            w = np.zeros(n, np.float32)
        else:
            w = _normal(r[2 * i], (n,), 0.02)
        g = _normal(r[2 * i + 1], (n,), grad_std)
        if grad_dtype == "bf16":
            g = bf16_round(g)
        out.append(dict(w=w, g=g, m=np.zeros(n, np.float32), v=np.zeros(n, np.float32)))
    return out


def lamb_grads(sizes, step: int, seed: int = SEED + 2, grad_std: float = 1e-3,
               grad_dtype: str = "bf16") -> list:
    """Fresh gradients for a later optimizer step (one stream per tensor and step)."""
    r = _streams(seed * 1000 + step, len(sizes))
    out = []
    for i, n in enumerate(sizes):
        g = _normal(r[i], (n,), grad_std)
        out.append(bf16_round(g) if grad_dtype == "bf16" else g)
    return out
