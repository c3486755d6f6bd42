"""Parity of the whole shard (ptb_forward + ptb_backward through the C ABI)
against the fp64 oracle, elementwise on every output, from ragged shapes up
to the full 175B and 530B TP=8 shard shapes."""
import numpy as np
import pytest
import torch

from oracle import ptb as O
from parity import check, errors, half_ulp, TOL
from transformer_block_lamb_amd.device import PtbShard
from transformer_block_lamb_amd.synth import CONFIGS, PtbConfig, ptb_inputs

pytestmark = pytest.mark.gpu

RAGGED = [
    PtbConfig("ragged_a", 2, 200, 264, 3, 64, 328, 50, "bf16", 1),
    PtbConfig("ragged_b", 1, 333, 512, 2, 96, 520, 77, "bf16", 0),
    PtbConfig("ragged_c", 3, 97, 136, 2, 128, 264, 1000, "bf16", 1),
    PtbConfig("ragged_w1", 1, 130, 256, 2, 64, 256, 1, "bf16", 1),
    PtbConfig("tiny_bf16", 1, 128, 256, 4, 64, 1024, 32, "bf16", 1),
    PtbConfig("ragged_f32", 2, 77, 72, 2, 64, 40, 20, "f32", 1),
    # input projections with two-pass (q, k) tiles under the split-K
    # schedules on 256 CUs: single-pass tiles whole, then the two-pass ones
    # split (1800 tokens: 8 M-tiles, the last ragged); all tiles split
    # (1000 tokens, K = 1000 not a multiple of the 64-wide K tile)
    PtbConfig("sk_lf_ragged", 1, 1800, 1024, 3, 128, 7096, 300, "bf16", 1),
    PtbConfig("sk_pure_ragged", 1, 1000, 1000, 3, 128, 8000, 100, "bf16", 1),
    # the same light-first schedule with a 2560-wide input (40 K tiles), so
    # each two-pass tile splits across about three workers
    PtbConfig("sk_lf_k2560", 1, 1800, 2560, 3, 128, 7096, 300, "bf16", 1),
]


def run_case(cfg, ln_affine="random"):
    print(f"ptb case {cfg}", flush=True)
    inp = ptb_inputs(cfg, ln_affine=ln_affine)
    shard = PtbShard(cfg, inp)
    shard.forward()
    shard.backward()
    torch.cuda.synchronize()
    got = shard.outputs()
    d = O.dims_of(cfg)
    y, saved = O.ptb_forward(d, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    g = O.ptb_backward(d, inp["x"], inp["gamma"], inp["w_in"], inp["w_out"], saved, inp["dy"])
    res = {"y": errors(got["y"], y)}
    if cfg.add_residual:
        # the partial sum y - x, allowing for the rounding of y to its storage type
        res["y-x"] = errors(got["y"] - inp["x"], y - inp["x"], half_ulp(y, cfg.dtype))
    for k in ("dx", "dgamma", "dbeta", "dw_in", "dw_out"):
        res[k] = errors(got[k], g[k])
    print({k: f"{v[0]:.2e}/{v[1]:.2e}" for k, v in res.items()}, flush=True)
    tmax, tmean = TOL[cfg.dtype]
    bad = {k: v for k, v in res.items() if not (v[0] <= tmax and v[1] <= tmean)}
    assert not bad, f"over tolerance {tmax}/{tmean}: {bad}"
    for k in ("y", "dx", "dw_in", "dw_out"):
        assert np.all(np.isfinite(got[k])), k
    return shard


def test_tiny_fp32():
    run_case(CONFIGS["tiny"])


@pytest.mark.parametrize("cfg", RAGGED, ids=lambda c: c.name)
def test_ragged(cfg):
    run_case(cfg)


def test_deterministic_bitwise():
    cfg = RAGGED[0]
    shard = run_case(cfg)
    first = {k: v.clone() for k, v in (("y", shard.y), ("dx", shard.dx), ("dw_in", shard.dw_in),
                                       ("dw_out", shard.dw_out), ("dgamma", shard.dgamma))}
    shard.forward()
    shard.backward()
    torch.cuda.synchronize()
    for k, v in first.items():
        assert torch.equal(v, getattr(shard, k)), k


@pytest.mark.parametrize("name", ["175b_w512", "175b_w2048", "small", "530b_w512"])
def test_full_size(name):
    run_case(CONFIGS[name], ln_affine="unit")
