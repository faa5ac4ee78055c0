"""CPU checks of the pair counts behind bench.py's throughput figures.

bench.py reports causal-adjusted TFLOP/s = 4 d FLOP per visible (query, key)
pair per query head.  The pairs come from `causal_pairs` over the launches of
`step_plan` (one ZigZag ring device: step 0 causal over its own chunks, steps
1..rank its queries against the source's front chunk, later steps its back
queries against both source chunks -- the twinkle ZigZag section).  These
tests pin those counts against brute force and against a count made from the
positions alone, with no ring schedule.
"""
import numpy as np
import pytest

import bench


def brute_pairs(q_pos, k_pos):
    return sum(1 for p in q_pos for k in k_pos if k <= p)


@pytest.mark.parametrize("seed", range(5))
def test_causal_pairs_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 60, size=rng.integers(0, 40))
    k = rng.integers(0, 60, size=rng.integers(0, 40))
    assert bench.causal_pairs(q, k) == brute_pairs(q, k)


def test_runs_positions():
    assert list(bench.runs_positions([(3, 2), (10, 3)])) == [3, 4, 10, 11, 12]
    assert len(bench.runs_positions([])) == 0


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8])
def test_step_plan_covers_each_visible_pair_once(W):
    N = 2 * W * 6  # chunks of 6 tokens
    c = N // (2 * W)
    for rank in range(W):
        plan = bench.step_plan(N, W, rank, c)
        assert len(plan) == W
        seen = {}
        for q_runs, k_runs in plan:
            for p in bench.runs_positions(q_runs):
                for k in bench.runs_positions(k_runs):
                    if k <= p:
                        seen[(p, k)] = seen.get((p, k), 0) + 1
        shard = [r * c + i for r in (rank, 2 * W - 1 - rank) for i in range(c)]
        want = {(p, k) for p in shard for k in range(N) if k <= p}
        assert set(seen) == want
        assert all(n == 1 for n in seen.values())


def test_ring_share_pair_count():
    # the ring share that bench.py times: 131072 tokens, 8 devices, rank 2,
    # ZigZag chunks {2, 13} of 8192 -- each query at position p sees p + 1 keys
    N, W, rank = 131072, 8, 2
    c = N // (2 * W)
    plan = bench.step_plan(N, W, rank, c)
    pairs = sum(bench.causal_pairs(bench.runs_positions(q), bench.runs_positions(k))
                for q, k in plan)
    pos = np.concatenate([np.arange(rank * c, (rank + 1) * c),
                          np.arange((2 * W - 1 - rank) * c, (2 * W - rank) * c)])
    assert pairs == int((pos + 1).sum()) == 1_073_750_016


def test_tile_efficiency_bounds():
    # full square causal: visible N(N+1)/2 of the computed tiles' pairs
    qp = np.arange(512)
    eff = bench.tile_efficiency([(qp, qp)])
    assert 0.5 < eff <= 1.0
    # a non-causal step (all keys before all queries) computes only visible pairs
    assert bench.tile_efficiency([(np.arange(1000, 1256), np.arange(0, 640))]) == 1.0
