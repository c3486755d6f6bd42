"""Pipeline-bubble and batch-size arithmetic behind the LAMB motivation
(MegaScale study guide, ch.2 §2.2: the interleaved 1F1B bubble term
(p - 1) / (v m) and LAMB's larger batch; §2.5 ablation table, "+LAMB (BS x3)"
row).  Host-side analytics: no GPU and no part of the block's kernels.

Notation: p pipeline stages (devices), v model chunks per device
(interleaving), m micro-batches per step, t = the time of one micro-batch's
forward + backward through one device's layers.  A step of interleaved 1F1B
keeps every device busy m t and idle (p - 1) t / v, so

    bubble fraction = (p - 1) / (v m)          (idle / busy)

`simulate_1f1b` replays the schedule event by event to check that closed
form; `lamb_batch_comparison` sets out the pages' comparison of one step at
k-times the batch against k steps at 1x, under each reading the pages offer.
"""
from __future__ import annotations


def bubble_fraction(p: int, m: int, v: int = 1) -> float:
    """Idle time over busy time of one interleaved-1F1B step."""
    if p < 1 or m < 1 or v < 1:
        raise ValueError("p, m, v must be >= 1")
    return (p - 1) / (v * m)


def bubble_time(p: int, v: int = 1, t: float = 1.0) -> float:
    """Idle time of one device in one step (independent of m)."""
    return (p - 1) * t / v


def _schedule(p: int, m: int, v: int, d: int):
    """Operation order of device d: ("F"|"B", chunk, micro-batch).  Forward
    micro-batches go in groups of p through chunk 0, then chunk 1, ...;
    backwards in the same groups through the chunks in reverse; a warm-up of
    p - d - 1 forwards (2 (p - d - 1) + (v - 1) p when interleaved), then one
    forward and one backward alternately, then the remaining backwards."""
    n = m * v

    def fwd(k):
        return (k // p) % v, (k // (p * v)) * p + k % p

    def bwd(k):
        return v - 1 - (k // p) % v, (k // (p * v)) * p + k % p

    warm = min(n, (p - d - 1) if v == 1 else 2 * (p - d - 1) + (v - 1) * p)
    ops, nf, nb = [], 0, 0
    for _ in range(warm):
        ops.append(("F",) + fwd(nf)); nf += 1
    while nf < n:
        ops.append(("F",) + fwd(nf)); nf += 1
        ops.append(("B",) + bwd(nb)); nb += 1
    while nb < n:
        ops.append(("B",) + bwd(nb)); nb += 1
    return ops


def simulate_1f1b(p: int, m: int, v: int = 1, f: float = 1.0, b: float = 2.0) -> dict:
    """Event-by-event replay of (interleaved) 1F1B.  Device d holds model
    stages c p + d for chunks c = 0..v-1; a chunk's forward takes f / v and
    its backward b / v.  Forward of stage s needs stage s-1's forward of the
    same micro-batch, backward of s needs stage s+1's backward (the last
    stage: its own forward).  Returns the makespan and each device's idle
    time (makespan - m (f + b))."""
    if v > 1 and m % p:
        raise ValueError("interleaving needs m to be a multiple of p")
    S = p * v
    done = {}                       # (kind, stage, mb) -> finish time
    queues = [_schedule(p, m, v, d) for d in range(p)]
    pos = [0] * p
    free = [0.0] * p
    remaining = sum(len(q) for q in queues)
    while remaining:
        progressed = False
        for d in range(p):
            while pos[d] < len(queues[d]):
                kind, c, mb = queues[d][pos[d]]
                s = c * p + d
                if kind == "F":
                    dep = [("F", s - 1, mb)] if s > 0 else []
                else:
                    dep = [("B", s + 1, mb)] if s < S - 1 else [("F", s, mb)]
                    dep.append(("F", s, mb))
                if any(x not in done for x in dep):
                    break
                start = max([free[d]] + [done[x] for x in dep])
                free[d] = start + (f if kind == "F" else b) / v
                done[(kind, s, mb)] = free[d]
                pos[d] += 1
                remaining -= 1
                progressed = True
        if not progressed:
            raise RuntimeError("schedule deadlocks")
    span = max(free)
    return {"makespan": span, "idle": [span - m * (f + b)] * p}


def lamb_batch_comparison(p: int, v: int, m: int, k: int) -> dict:
    """k steps at batch m against one step at batch k m (the same tokens).

    same_tokens_time   : total idle time, one big step / k small steps = 1/k
    fraction           : bubble fraction, big / small = 1/k
    literal_page       : the pages' printed pair, k (p-1)/(v m) against
                         (p-1)/(v k m), = 1/k^2 (for k = 4: 1/16, 93.75 % less)
    The pages' "87.5 % fewer bubbles" (1/8) matches none of these; for the
    production batch of 3x the literal pair gives 1/9 (88.9 % less)."""
    small = bubble_fraction(p, m, v)
    big = bubble_fraction(p, k * m, v)
    return {
        "same_tokens_time": bubble_time(p, v) / (k * bubble_time(p, v)),
        "fraction": big / small,
        "literal_page": big / (k * small),
        "literal_page_reduction": 1.0 - big / (k * small),
    }
