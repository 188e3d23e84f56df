"""The stale-plan baseline's load split (bench.py ``stale_rank_loads``):
a hand-worked case, and the identity that a plan applied to the counts it
was made from gives back its own rank loads."""
import numpy as np
import torch

import bench
import oracle
import pins


def test_hand_worked_split():
    # E=4, R=2 (N=2), S=1, slots per rank: two natives then one spare.
    # Old plan: e0 keeps 4 at home and 2 on rank 1's spare; e1 saw nothing.
    se = torch.tensor([[0, 1, -1, 2, 3, 0]])
    sc = torch.tensor([[4, 0, 0, 1, 1, 2]])
    new = torch.tensor([[3, 2, 0, 1]])
    # e0: 3 split 4:2 -> 2 and 1; e1 whole on its native slot; e3 -> 1
    got = bench.stale_rank_loads(se, sc, new, 2, 3, 2)
    assert got.tolist() == [[4.0, 2.0]]


def test_same_counts_give_the_plan_loads():
    rng = np.random.default_rng(17)
    for _ in range(40):
        R = int(rng.integers(1, 9))
        N = int(rng.integers(1, 5))
        S = int(rng.integers(0, 3))
        E = R * N
        routing = pins.random_routing(rng, int(rng.integers(1, 3000)), E,
                                      int(rng.integers(1, min(E, 4) + 1)),
                                      float(rng.uniform(0, 2.5)))
        counts, _ = oracle.load(routing[None], E)
        pl = oracle.plan(counts[0], R, S)
        got = bench.stale_rank_loads(torch.from_numpy(pl["slot_expert"])[None],
                                     torch.from_numpy(pl["slot_cap"])[None],
                                     torch.from_numpy(counts), N, N + S, R)
        np.testing.assert_allclose(got[0].numpy(), pl["load_after"],
                                   rtol=0, atol=1e-9)
        # the split conserves the new total
        other = counts[0][::-1].copy()
        got2 = bench.stale_rank_loads(torch.from_numpy(pl["slot_expert"])[None],
                                      torch.from_numpy(pl["slot_cap"])[None],
                                      torch.from_numpy(other)[None], N, N + S, R)
        assert abs(float(got2.sum()) - float(other.sum())) < 1e-6
