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


def run_case(cfg, ln_affine="random", use_scratch=True):
    print(f"ptb case {cfg} scratch={use_scratch}", flush=True)
    inp = ptb_inputs(cfg, ln_affine=ln_affine)
    shard = PtbShard(cfg, inp)
    shard.forward(use_scratch=use_scratch)
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
    run_case(CONFIGS[name], ln_affine="random")


def test_forward_without_scratch():
    """ptb_forward with no scratch runs every GEMM on whole-tile schedules;
    the shape is one whose input projection otherwise splits."""
    run_case(RAGGED[6], use_scratch=False)


@pytest.mark.parametrize("cfg", [RAGGED[0], RAGGED[5]], ids=lambda c: c.name)
def test_window_beyond_seq_is_causal_bitwise(cfg):
    """Any window >= seq is plain causal attention: window = 2^31 - 1 gives
    bit for bit the outputs of window = seq (bf16 and fp32)."""
    print(f"window beyond seq {cfg.name}", flush=True)
    inp = ptb_inputs(cfg, ln_affine="random")
    outs = []
    for w in (cfg.seq, 2 ** 31 - 1):
        shard = PtbShard(cfg.replace(window=w), inp)
        shard.forward()
        shard.backward()
        torch.cuda.synchronize()
        outs.append({k: getattr(shard, k).clone() for k in ("y", "dx", "dgamma", "dbeta", "dw_in",
                                                            "dw_out")})
    for k in outs[0]:
        assert torch.equal(outs[0][k], outs[1][k]), k


def test_tensor_parallel_shards_sum_to_full_layer():
    """A full layer of 16 heads x 64 and FFN 1088 split into 8 tensor-parallel
    shards (row blocks of w_in and w_out), each run through ptb_forward /
    ptb_backward with the residual on shard 0 only: the shards' y, dx,
    dgamma, dbeta summed on the device match the oracle's unsharded layer,
    and each shard's weight gradients match the rows of the full ones."""
    n, Hf, d, Ff = 8, 16, 64, 1088
    full = PtbConfig("tp_full", 2, 200, 264, Hf, d, Ff, 50, "bf16", 1)
    print(f"tp shards {full}", flush=True)
    inp = ptb_inputs(full, ln_affine="random")
    A, Hs, Fs = Hf * d, Hf // n, Ff // n
    As = Hs * d
    dm = O.dims_of(full)
    y, saved = O.ptb_forward(dm, inp["x"], inp["gamma"], inp["beta"], inp["w_in"], inp["w_out"])
    g = O.ptb_backward(dm, inp["x"], inp["gamma"], inp["w_in"], inp["w_out"], saved, inp["dy"])
    sums = {k: None for k in ("y", "dx", "dgamma", "dbeta")}
    allow = 0.0  # each shard's y is rounded to bf16 before the sum
    for r in range(n):
        blk = lambda base: np.arange(base + r * As, base + (r + 1) * As)
        rows = np.concatenate([blk(0), blk(A), blk(2 * A), 3 * A + np.arange(r * Fs, (r + 1) * Fs)])
        out_rows = np.concatenate([blk(0), A + np.arange(r * Fs, (r + 1) * Fs)])
        cfg = full.replace(name=f"tp{r}", n_heads=Hs, ffn=Fs, add_residual=int(r == 0))
        shard = PtbShard(cfg, dict(inp, w_in=inp["w_in"][rows], w_out=inp["w_out"][out_rows]))
        shard.forward()
        shard.backward()
        for k in sums:
            t = getattr(shard, k).float()
            sums[k] = t if sums[k] is None else sums[k] + t
        torch.cuda.synchronize()
        got = shard.outputs()
        allow = allow + half_ulp(got["y"], "bf16")
        check(f"dw_in[{r}]", got["dw_in"], g["dw_in"][rows], "bf16")
        check(f"dw_out[{r}]", got["dw_out"], g["dw_out"][out_rows], "bf16")
    host = {k: v.cpu().numpy().astype(np.float64) for k, v in sums.items()}
    check("sum y", host["y"], y, "bf16")
    check("sum y - x", host["y"] - inp["x"], y - inp["x"], "bf16", allow)
    for k in ("dx", "dgamma", "dbeta"):
        check(f"sum {k}", host[k], g[k], "bf16")
