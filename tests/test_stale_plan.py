"""The stale-plan split (periodic, historical-load balancing applied to new
counts; UltraEP abstract, news write-up section on the problem UltraEP
solves) in the oracle: hand-worked cases, the closed form that a plan
applied to the counts it was made from gives back its own rank loads, and
conservation of the new total."""
import numpy as np

import oracle
import pins


def hand_plan():
    # E=4, R=2 (N=2), S=1: slots per rank two natives then one spare
    # (p0 p1 p2 | p3 p4 p5). Old plan: e0 keeps 4 at home (p0) and has 2 on
    # rank 1's spare (p5); e1 saw no tokens; e2 and e3 kept 1 each.
    return dict(E=4, R=2, N=2, S=1,
                rep_off=np.array([0, 2, 3, 4, 5], np.int32),
                rep_slot=np.array([0, 5, 1, 3, 4, -1], np.int32),
                rep_cap=np.array([4, 2, 0, 1, 1, 0], np.int32))


def test_hand_worked_split():
    pl = hand_plan()
    # new [3,2,0,1]: e0 3 over caps 4:2 -> floor(3*4/6) = 2 at p0, the other
    # 1 at p5; e1 (no old tokens) whole on its master p1; e3 1 at p4;
    # r0 = 2 + 2, r1 = 1 + 1
    assert oracle.stale_loads(pl, [3, 2, 0, 1]).tolist() == [4, 2]
    # new [5,0,2,1]: e0 5 -> floor(5*4/6) = 3 at p0, 5 - 3 = 2 at p5; e2 2
    # at p3; e3 1 at p4; r0 = 3, r1 = 2 + 2 + 1
    assert oracle.stale_loads(pl, [5, 0, 2, 1]).tolist() == [3, 5]
    # nothing new: nothing anywhere
    assert oracle.stale_loads(pl, [0, 0, 0, 0]).tolist() == [0, 0]


def test_same_counts_give_the_plan_loads():
    """floor(c * prefix / c) = prefix: applied to its own counts a plan's
    replicas take exactly their capacities, so the rank loads are the
    plan's load_after; any new counts keep their total."""
    rng = np.random.default_rng(17)
    for it in range(60):
        R = int(rng.integers(1, 9))
        N = int(rng.integers(1, 5))
        S = int(rng.integers(0, 3))
        E = R * N
        routing = pins.random_routing(rng, int(rng.integers(1, 3000)), E,
                                      int(rng.integers(1, min(E, 4) + 1)),
                                      float(rng.uniform(0, 2.5)))
        counts, _ = oracle.load(routing[None], E)
        for policy, quota_mode in pins_rules():
            pl = oracle.plan(counts[0], R, S, policy, quota_mode)
            got = oracle.stale_loads(pl, counts[0])
            assert np.array_equal(got, pl["load_after"]), (it, policy)
            other = rng.permutation(counts[0])
            got2 = oracle.stale_loads(pl, other)
            assert int(got2.sum()) == int(other.sum())
            assert np.all(got2 >= 0)


def pins_rules():
    return [(0, 0), (1, 0), (0, 1), (1, 1)]


def test_unplanned_expert_stays_native():
    """An expert with no old tokens keeps all of its new ones on its home
    rank, whatever the plan did for the others."""
    pl = oracle.plan(np.array([9, 0, 0, 0, 0, 0], np.int32), 3, 1)
    # e0 was spread; e1..e5 saw nothing: they stay on ranks e // 2
    new = np.array([0, 7, 5, 3, 2, 1], np.int64)
    assert oracle.stale_loads(pl, new).tolist() == [7, 8, 3]
