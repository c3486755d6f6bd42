"""Parity of lamb_step (through the C ABI) against the fp64 oracle: updated
weights compared as the update dw = w' - w, moments m and v, per-tensor
trust ratios; the norm invariant ||w' - w|| = lr ||w||; resume from saved
state; the full 175B TP=8 layer shard (226.5M parameters); the ZeRO-2
sharded halves (lamb_shard_norms / lamb_shard_apply) against lamb_step and
the oracle."""
import numpy as np
import pytest
import torch

from oracle import lamb as OL
from parity import check, half_ulp
from transformer_block_lamb_amd.device import LambState, ShardedLamb
from transformer_block_lamb_amd.synth import LAMB_175B_TENSORS, LAMB_HPARAMS, lamb_grads, lamb_inputs

pytestmark = pytest.mark.gpu
HP = LAMB_HPARAMS
SMALL = [1, 3, 4097, 8192 * 3 + 5, 4096, 264, 264]


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def _oracle_steps(tensors, grads_per_step, first_step):
    state = [dict(w=t["w"].astype(np.float64), m=t["m"].astype(np.float64),
                  v=t["v"].astype(np.float64), weight_decay=t.get("weight_decay", HP["weight_decay"]))
             for t in tensors]
    ratios = None
    for s, grads in enumerate(grads_per_step, start=first_step):
        ins = [dict(st, g=g) for st, g in zip(state, grads)]
        out = OL.lamb_step(ins, s, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
        ratios = [o["ratio"] for o in out]
        state = [dict(w=o["w"], m=o["m"], v=o["v"], weight_decay=st["weight_decay"]) for o, st in zip(out, state)]
    return state, ratios


def _compare(dev, w0, ref_state, ref_ratios, tol_dtype="f32", ratios=None):
    for i, (p, ref) in enumerate(zip(dev.params, ref_state)):
        # the update w' - w, allowing for the rounding of w' to fp32
        check(f"dw[{i}]", _host(p["w"]) - w0[i], ref["w"] - w0[i], tol_dtype,
              allowance=2 * half_ulp(ref["w"], "f32"))
        check(f"m[{i}]", _host(p["m"]), ref["m"], tol_dtype)
        check(f"v[{i}]", _host(p["v"]), ref["v"], tol_dtype)
    np.testing.assert_allclose(_host(dev.ratios if ratios is None else ratios), ref_ratios,
                               rtol=1e-4)


@pytest.mark.parametrize("grad_dtype", ["bf16", "f32"])
def test_lamb_small_step1(grad_dtype):
    print(f"lamb small step1 {grad_dtype}", flush=True)
    ts = lamb_inputs(SMALL, grad_dtype=grad_dtype)
    ts[2]["weight_decay"] = 0.0
    dev = LambState(ts, grad_dtype)
    w0 = [t["w"].astype(np.float64) for t in ts]
    dev.step(1, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"])
    torch.cuda.synchronize()
    ref, ratios = _oracle_steps(ts, [[t["g"] for t in ts]], 1)
    _compare(dev, w0, ref, ratios)
    # the trust-ratio invariant on every tensor with nonzero norms
    for i, p in enumerate(dev.params):
        if np.linalg.norm(w0[i]) > 0:
            dn = np.linalg.norm(_host(p["w"]) - w0[i])
            assert dn == pytest.approx(HP["lr"] * np.linalg.norm(w0[i]), rel=1e-3), i


def test_lamb_step10_after_oracle_replay():
    """State after 9 oracle steps is loaded into the device; step 10 compared."""
    print("lamb step10", flush=True)
    ts = lamb_inputs(SMALL)
    grads = [lamb_grads(SMALL, s) for s in range(1, 10)]
    st9, _ = _oracle_steps(ts, grads, 1)
    ts9 = [dict(w=s["w"].astype(np.float32), m=s["m"].astype(np.float32), v=s["v"].astype(np.float32),
                g=g) for s, g in zip(st9, lamb_grads(SMALL, 10))]
    dev = LambState(ts9, "bf16")
    w0 = [t["w"].astype(np.float64) for t in ts9]
    dev.step(10, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"])
    torch.cuda.synchronize()
    ref, ratios = _oracle_steps(ts9, [[t["g"] for t in ts9]], 10)
    _compare(dev, w0, ref, ratios)


def test_lamb_resume_equals_uninterrupted():
    print("lamb resume", flush=True)
    ts = lamb_inputs(SMALL)
    a = LambState(ts, "bf16")
    for s in range(1, 4):
        a.set_grads(lamb_grads(SMALL, s))
        a.step(s, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"])
    torch.cuda.synchronize()
    saved = [{k: _host(p[k]).astype(np.float32) for k in ("w", "m", "v")} for p in a.params]
    b = LambState([dict(s, g=g) for s, g in zip(saved, lamb_grads(SMALL, 4))], "bf16")
    a.set_grads(lamb_grads(SMALL, 4))
    a.step(4, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"])
    b.step(4, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"])
    torch.cuda.synchronize()
    for pa, pb in zip(a.params, b.params):
        for k in ("w", "m", "v"):
            assert torch.equal(pa[k], pb[k]), k


def test_lamb_zero_norms():
    ts = [dict(w=np.zeros(100, np.float32), g=np.ones(100, np.float32), m=np.zeros(100, np.float32),
               v=np.zeros(100, np.float32)),
          dict(w=np.ones(20, np.float32), g=np.zeros(20, np.float32), m=np.zeros(20, np.float32),
               v=np.zeros(20, np.float32), weight_decay=0.0)]
    dev = LambState(ts, ["f32", "bf16"])
    dev.step(1, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(dev.ratios), [1.0, 1.0])
    np.testing.assert_allclose(_host(dev.params[0]["w"]), -HP["lr"] / (1 + HP["eps"]), rtol=1e-6)
    np.testing.assert_array_equal(_host(dev.params[1]["w"]), 1.0)


def test_lamb_mixed_grad_dtypes_and_bf16_copy():
    """Matrices with bf16 gradients and LN vectors with fp32 gradients in one
    call; the bf16 copy of each new w equals the new fp32 w rounded to bf16."""
    print("lamb mixed dtypes + bf16 copy", flush=True)
    sizes = [5000, 264, 264]
    ts = lamb_inputs(sizes, grad_dtype="f32")
    from transformer_block_lamb_amd.synth import bf16_round
    ts[0]["g"] = bf16_round(ts[0]["g"])
    dev = LambState(ts, ["bf16", "f32", "f32"], bf16_copy=True)
    w0 = [t["w"].astype(np.float64) for t in ts]
    dev.step(1, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"])
    torch.cuda.synchronize()
    ref, ratios = _oracle_steps(ts, [[t["g"] for t in ts]], 1)
    _compare(dev, w0, ref, ratios)
    for p in dev.params:
        assert torch.equal(p["w_bf16"], p["w"].to(torch.bfloat16))


def test_lamb_full_175b_shard():
    sizes = [n for _, n in LAMB_175B_TENSORS]
    print(f"lamb full 175B shard {sum(sizes)} params", flush=True)
    ts = lamb_inputs(sizes)
    dev = LambState(ts, "bf16")
    w0 = [t["w"].astype(np.float64) for t in ts]
    dev.step(1, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"])
    torch.cuda.synchronize()
    ref, ratios = _oracle_steps(ts, [[t["g"] for t in ts]], 1)
    _compare(dev, w0, ref, ratios)


def _sharded_vs_full(sizes, n_shards, steps, oracle=False):
    ts = lamb_inputs(sizes)
    full = LambState(ts, "bf16", bf16_copy=True)
    sharded_state = LambState(ts, "bf16", bf16_copy=True)
    sh = ShardedLamb(sharded_state.params, n_shards)
    w0 = [t["w"].astype(np.float64) for t in ts]
    # largest |w| each element reaches over the steps (the scale of its rounding)
    wmax = [np.abs(w) for w in w0]
    for s in range(1, steps + 1):
        if s > 1:
            g = lamb_grads(sizes, s)
            full.set_grads(g)
            sharded_state.set_grads(g)
        full.step(s, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"])
        sh.step(s, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"])
        wmax = [np.maximum(m, np.abs(_host(p["w"]))) for m, p in zip(wmax, full.params)]
    torch.cuda.synchronize()
    for i, (pa, pb) in enumerate(zip(full.params, sharded_state.params)):
        # pass A is elementwise: the moments match bit for bit
        assert torch.equal(pa["m"], pb["m"]), i
        assert torch.equal(pa["v"], pb["v"]), i
        # the norms are added in another order (fp64), which can move each
        # step's fp32 ratio by an ulp, and a step starts from the previous
        # step's (slightly different) w: w within 3 ulps per step of the
        # largest magnitude the element reached (w - lr r u can cancel to far
        # below the magnitudes it was rounded at)
        a, b = _host(pa["w"]), _host(pb["w"])
        mag = wmax[i].astype(np.float32)
        ulps = np.abs(a - b) / np.spacing(mag)
        assert np.all(ulps <= 3 * steps), (i, float(ulps.max()))
        assert torch.equal(pb["w_bf16"], pb["w"].to(torch.bfloat16)), i
    np.testing.assert_allclose(_host(sh.ratios), _host(full.ratios), rtol=1e-6)
    if oracle:
        ref, ratios = _oracle_steps(ts, [[t["g"] for t in ts]], 1)
        _compare(sharded_state, w0, ref, ratios, ratios=sh.ratios)


@pytest.mark.parametrize("n_shards", [2, 3, 8])
def test_lamb_sharded_equals_unsharded(n_shards):
    """Ragged ranges; the smallest tensors do not reach every rank."""
    print(f"lamb sharded x{n_shards}", flush=True)
    _sharded_vs_full(SMALL, n_shards, 1, oracle=True)
    _sharded_vs_full(SMALL, n_shards, 3)




MANY = [1, 3, 4097, 5000, 12, 264, 8192 * 3 + 5, 7, 4096, 100, 2, 999, 16384, 31, 64, 520, 3000,
        8, 1]


def test_lamb_more_tensors_than_one_launch():
    """19 tensors of mixed sizes: more than one kernel-argument table (16), so
    the step runs as two batches of launches whose partials, ratios and
    norms sit at offsets into the scratch and the outputs."""
    print(f"lamb {len(MANY)} tensors", flush=True)
    ts = lamb_inputs(MANY)
    ts[5]["weight_decay"] = 0.0
    ts[17]["weight_decay"] = 0.1
    dev = LambState(ts, "bf16")
    w0 = [t["w"].astype(np.float64) for t in ts]
    dev.step(1, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"])
    torch.cuda.synchronize()
    ref, ratios = _oracle_steps(ts, [[t["g"] for t in ts]], 1)
    _compare(dev, w0, ref, ratios)


@pytest.mark.parametrize("n_shards", [2, 3])
def test_lamb_sharded_more_tensors_than_one_launch(n_shards):
    print(f"lamb sharded {len(MANY)} tensors x{n_shards}", flush=True)
    _sharded_vs_full(MANY, n_shards, 1, oracle=True)
    _sharded_vs_full(MANY, n_shards, 2)


def test_lamb_full_175b_shard_step10():
    """Step 10 (bias corrections 1 - 0.9^10 and 1 - 0.999^10) on the whole
    226.5M-parameter shard, from a synthetic mid-training state: moments of
    the size a few steps of N(0, 1e-3) gradients leave."""
    sizes = [n for _, n in LAMB_175B_TENSORS]
    print(f"lamb full 175B shard step 10 {sum(sizes)} params", flush=True)
    ts = lamb_inputs(sizes)
    rng = np.random.default_rng(10)
    for t in ts:
        n = t["w"].size
        t["m"] = (3e-4 * rng.standard_normal(n)).astype(np.float32)
        t["v"] = (1e-6 * rng.standard_normal(n) ** 2 + 1e-8).astype(np.float32)
    dev = LambState(ts, "bf16")
    w0 = [t["w"].astype(np.float64) for t in ts]
    dev.step(10, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"])
    torch.cuda.synchronize()
    print("device step done; oracle step", flush=True)
    ref, ratios = _oracle_steps(ts, [[t["g"] for t in ts]], 10)
    _compare(dev, w0, ref, ratios)


def test_lamb_sharded_175b_dp8_vs_oracle():
    """ZeRO-2 at DP = 8 over the whole shard, against the oracle (and the
    unsharded step)."""
    sizes = [n for _, n in LAMB_175B_TENSORS]
    print(f"lamb sharded 175B x8 vs oracle {sum(sizes)} params", flush=True)
    _sharded_vs_full(sizes, 8, 1, oracle=True)
