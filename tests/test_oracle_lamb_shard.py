"""Pins of the oracle's ZeRO-2 sharded LAMB step: for any split of every
tensor into contiguous slices, norms summed over the slices then applied
per slice give the unsharded oracle step (itself pinned in
test_oracle_lamb_flops.py); and the same over two processes whose norms
meet in a gloo all-reduce."""
import os
import socket

import numpy as np
import pytest
import torch
import torch.distributed as dist
import torch.multiprocessing as mp

from oracle import lamb as OL

HP = dict(lr=2e-3, beta1=0.9, beta2=0.999, eps=1e-6, weight_decay=0.01)


def _tensors(sizes, seed=3):
    rng = np.random.default_rng(seed)
    return [dict(w=rng.normal(0, 0.02, n), g=rng.normal(0, 1e-3, n), m=rng.normal(0, 1e-4, n),
                 v=np.abs(rng.normal(0, 1e-7, n))) for n in sizes]


def _sharded(ts, cuts_per_tensor, step):
    """Runs the sharded step with the given slice boundaries; returns per
    tensor (w, m, v, ratio)."""
    out = []
    for t, cuts in zip(ts, cuts_per_tensor):
        edges = [0] + list(cuts) + [len(t["w"])]
        halves = [OL.lamb_shard_norms(t["w"][a:b], t["g"][a:b], t["m"][a:b], t["v"][a:b], step,
                                      HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
                  for a, b in zip(edges[:-1], edges[1:])]
        W = sum(h[2] for h in halves)
        U = sum(h[3] for h in halves)
        ws, ratios = [], []
        for (a, b), h in zip(zip(edges[:-1], edges[1:]), halves):
            w_new, r = OL.lamb_shard_apply(t["w"][a:b], h[0], h[1], W, U, step, HP["lr"],
                                           HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
            ws.append(w_new)
            ratios.append(r)
        assert len(set(ratios)) == 1
        out.append((np.concatenate(ws), np.concatenate([h[0] for h in halves]),
                    np.concatenate([h[1] for h in halves]), ratios[0]))
    return out


@pytest.mark.parametrize("step", [1, 7])
def test_any_split_equals_unsharded(step):
    sizes = [1000, 37, 4096]
    ts = _tensors(sizes)
    full = OL.lamb_step([dict(t) for t in ts], step, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                        HP["weight_decay"])
    for cuts in ([[500], [1], [8, 4000]], [[0, 1000], [37], [1024, 2048, 3072]],
                 [[123, 124, 999], [20], [4095]]):
        got = _sharded(ts, cuts, step)
        for (w, m, v, r), ref in zip(got, full):
            np.testing.assert_allclose(w, ref["w"], rtol=1e-13, atol=1e-16)
            np.testing.assert_array_equal(m, ref["m"])
            np.testing.assert_array_equal(v, ref["v"])
            assert r == pytest.approx(ref["ratio"], rel=1e-13)


def test_zero_norm_shards_keep_the_unit_ratio():
    """A zero tensor split over ranks: every slice's w^2 sum is 0, so the
    ratio is 1 on every rank, as in the unsharded step."""
    ts = [dict(w=np.zeros(64), g=np.ones(64), m=np.zeros(64), v=np.zeros(64))]
    got = _sharded(ts, [[16, 40]], 1)
    assert got[0][3] == 1.0
    np.testing.assert_allclose(got[0][0], -HP["lr"] / (1 + HP["eps"]), rtol=1e-12)


def _rank_main(rank, world, port, sizes, result_path):
    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=world)
    ts = _tensors(sizes)
    mine, norms = [], []
    for t in ts:
        n = len(t["w"])
        a, b = rank * n // world, (rank + 1) * n // world
        h = OL.lamb_shard_norms(t["w"][a:b], t["g"][a:b], t["m"][a:b], t["v"][a:b], 2,
                                HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
        mine.append((a, b, h))
        norms += [h[2], h[3]]
    total = torch.tensor(norms, dtype=torch.float64)
    dist.all_reduce(total)
    out = []
    for i, (a, b, h) in enumerate(mine):
        w_new, r = OL.lamb_shard_apply(ts[i]["w"][a:b], h[0], h[1], float(total[2 * i]),
                                       float(total[2 * i + 1]), 2, HP["lr"], HP["beta1"],
                                       HP["beta2"], HP["eps"], HP["weight_decay"])
        out.append(w_new)
    gathered = [None] * world
    dist.all_gather_object(gathered, out)
    if rank == 0:
        np.savez(result_path, *[np.concatenate([g[i] for g in gathered]) for i in range(len(ts))])
    dist.destroy_process_group()


def test_two_ranks_over_gloo(tmp_path):
    sizes = [999, 64, 3]
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        port = s.getsockname()[1]
    path = str(tmp_path / "w.npz")
    mp.spawn(_rank_main, args=(2, port, sizes, path), nprocs=2, join=True)
    got = np.load(path)
    full = OL.lamb_step(_tensors(sizes), 2, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                        HP["weight_decay"])
    for i, ref in enumerate(full):
        np.testing.assert_allclose(got[f"arr_{i}"], ref["w"], rtol=1e-13, atol=1e-16)
