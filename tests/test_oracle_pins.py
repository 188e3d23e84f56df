"""The CPU oracle checked against hand-worked cases, closed forms, library
routines and brute force (see ``pins.py``)."""
import numpy as np
import pytest

import pins


@pytest.mark.parametrize("case", pins.golden_cases(), ids=lambda g: g["name"])
def test_golden(case):
    pins.check_golden(case)


RULES = [(0, 0), (1, 0), (0, 1), (1, 1), (2, 0), (2, 1), (3, 0), (3, 1)]
RULE_IDS = ["least_loaded", "best_fit", "least_loaded_search",
            "best_fit_search", "cover", "cover_search", "ascending",
            "ascending_search"]


@pytest.mark.parametrize("policy,quota_mode", RULES, ids=RULE_IDS)
def test_invariants_random(policy, quota_mode):
    rng = np.random.default_rng(20260602 + quota_mode)
    for _ in range(1500 if quota_mode == 0 else 600):
        pins.check_instance(*pins.random_instance(rng), policy=policy,
                            quota_mode=quota_mode)


@pytest.mark.parametrize("policy,quota_mode", RULES, ids=RULE_IDS)
def test_invariants_larger(policy, quota_mode):
    rng = np.random.default_rng(7)
    for _ in range(40):
        routing, E, R, S = pins.random_instance(
            rng, max_ranks=32, max_native=8, max_spare=3, max_tokens=2000,
            max_k=8)
        pins.check_instance(routing, E, R, S, policy=policy,
                            quota_mode=quota_mode)


def test_quota_search_large_quota():
    """Quotas in the thousands (steps of ceil(Q0/256) > 1): the kept quota
    is on the grid and every lower step exhausts, for every rule."""
    rng = np.random.default_rng(8)
    for it in range(12):
        R = int(rng.choice([4, 8, 16]))
        N = int(rng.integers(1, 5))
        E = R * N
        k = int(min(E, 4))
        routing = pins.random_routing(rng, 6000, E, k, float(rng.uniform(0.8, 2)))
        for policy in (0, 1, 2, 3):
            pl = pins.check_instance(routing, E, R, 1, policy=policy,
                                     quota_mode=1)
            assert pl["quota"] >= 256     # the step is above one token here


def test_no_spares():
    pins.check_no_spares(np.random.default_rng(1))


def test_one_rank():
    pins.check_one_rank(np.random.default_rng(2))


def test_balanced():
    pins.check_balanced()


def test_single_hot_expert():
    pins.check_single_hot()


def test_invalid_ids():
    pins.check_invalid_ids()


@pytest.mark.parametrize("policy,quota_mode", RULES, ids=RULE_IDS)
def test_brute_force_optimum(policy, quota_mode):
    """Exhaustive optimum on tiny instances: greedy == optimum == Q whenever
    slots suffice; otherwise the optimum never exceeds greedy. The worst
    observed greedy/optimum ratio is reported."""
    rng = np.random.default_rng(3)
    worst = 1.0
    n_exhausted = 0
    for _ in range(60):
        R = int(rng.integers(2, 4))
        N = int(rng.integers(1, 3))
        S = int(rng.integers(1, 3 if R == 2 else 2))
        E = R * N
        counts = rng.integers(0, 9, size=E).astype(np.int32)
        counts[rng.integers(0, E)] += int(rng.integers(0, 12))
        ratio = pins.check_against_optimum(counts, R, S, policy, quota_mode)
        worst = max(worst, ratio)
        n_exhausted += ratio > 1.0
    print(f"policy {policy} quota {quota_mode}: greedy/optimum worst {worst:.3f}; above optimum in "
          f"{n_exhausted}/60")
    assert worst <= 2.0
