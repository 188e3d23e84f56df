"""HIP path (through the C ABI) against the CPU oracle, bit-exact: expert
counts, the whole placement block, physical routing, per-rank counts, the
dispatch permutation and its inverse."""
import numpy as np
import pytest
import torch

import moe_expert_load_ue_amd as ue
import oracle
import pins
from gpu_helpers import compare_with_oracle, gpu_rebalance, say
from moe_expert_load_ue_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def make_ctx(E, R, S, k, T, L=1, policy=ue.PLAN_LEAST_LOADED,
             quota_mode=ue.QUOTA_FIXED):
    return ue.Context(E, R, S, k, max(T, 1), L, device=DEV,
                      plan_policy=policy, quota_mode=quota_mode)


# (destination rule, quota mode): the default, best fit, best fit in
# covering order and in ascending order, each also with the quota search
RULES = [(0, 0), (1, 0), (0, 1), (1, 1), (2, 0), (2, 1), (3, 0), (3, 1)]
RULE_IDS = ["least_loaded", "best_fit", "least_loaded_search",
            "best_fit_search", "cover", "cover_search", "ascending",
            "ascending_search"]


@pytest.mark.parametrize("case", [g for g in pins.golden_cases()
                                  if "routing" in g and "kind" not in g],
                         ids=lambda g: g["name"])
def test_golden_cases(case):
    say("golden", case["name"])
    routing = np.asarray(case["routing"], np.int32)[None]
    ctx = make_ctx(case["E"], case["R"], case["S"], case["k"], case["T"],
                   policy=case.get("policy", 0),
                   quota_mode=case.get("quota_mode", 0))
    res = gpu_rebalance(ctx, torch.from_numpy(routing))
    for key in ("phys", "perm", "inv_perm", "rank_counts"):
        assert res[key].reshape(-1).tolist() == case[key], key
    compare_with_oracle(res, routing, case["E"], case["R"], case["S"])


@pytest.mark.parametrize("case", [g for g in pins.golden_cases()
                                  if g.get("kind") == "faults"],
                         ids=lambda g: g["name"])
def test_golden_faults(case):
    """The hand-worked fault case through ue_load, ue_plan (on the counts
    the plan was made from) and ue_reroute: faulted assignments get phys =
    inv_perm = -1 and no position, rank_counts leave them out, and perm
    positions nothing fills keep the value the caller put there."""
    say("golden faults", case["name"])
    fill = pins.PERM_FILL
    routing = torch.tensor(case["routing"], dtype=torch.int32,
                           device=DEV)[None]
    ctx = make_ctx(case["E"], case["R"], case["S"], case["k"], case["T"])
    invalid = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    counts = ue.ue_load(ctx, routing, invalid=invalid)
    plan_counts = torch.tensor(case["plan_counts"], dtype=torch.int32,
                               device=DEV)[None]
    placement = ue.ue_plan(ctx, plan_counts)
    perm = torch.full((1, case["T"] * case["k"]), fill, dtype=torch.int32,
                      device=DEV)
    out = ue.ue_reroute(ctx, routing, placement, perm=perm)
    torch.cuda.synchronize()
    assert counts[0].tolist() == case["routing_counts"]
    assert int(invalid[0]) == case["invalid"]
    assert int(out["faults"][0]) == case["faults"]
    for key in ("phys", "inv_perm", "rank_counts"):
        assert out[key].reshape(-1).tolist() == case[key], key
    assert perm[0].tolist() == [fill if v is None else v for v in case["perm"]]


def test_golden_planner_only():
    for case in pins.golden_cases():
        if case.get("kind") == "faults":
            continue
        say("golden plan", case["name"])
        ctx = make_ctx(case["E"], case["R"], case["S"], 1, 1,
                       policy=case.get("policy", 0),
                       quota_mode=case.get("quota_mode", 0))
        counts = torch.tensor(case["counts"], dtype=torch.int32,
                              device=DEV)[None]
        f = ctx.placement_fields(ue.ue_plan(ctx, counts))
        for key in ("quota", "exhausted", "residual", "n_rep"):
            assert int(f[key][0]) == case[key], key
        for key in ("load_before", "load_after", "rep_off", "slot_expert",
                    "slot_cap", "slot_off"):
            assert f[key][0].tolist() == case[key], key
        n = case["n_rep"]
        assert f["rep_slot"][0, :n].tolist() == case["rep_slot"]
        assert f["rep_cap"][0, :n].tolist() == case["rep_cap"]


@pytest.mark.parametrize("policy,quota_mode", RULES, ids=RULE_IDS)
def test_random_instances(policy, quota_mode):
    """Seeded random shapes: tiny to several tiles with ragged tails, skew
    from uniform to extreme, S = 0..3, one to four layers."""
    rng = np.random.default_rng(99 + policy + 2 * quota_mode)
    for it in range(60):
        R = int(rng.integers(1, 17))
        N = int(rng.integers(1, 9))
        E = R * N
        if E > 1024:
            continue
        S = int(rng.integers(0, 4))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([0, 1, 7, 100, 511, 2048, 3001, 9000]))
        L = int(rng.integers(1, 5))
        skew = float(rng.uniform(0, 3))
        routing = np.stack([pins.random_routing(rng, T, E, k, skew)
                            for _ in range(L)])
        say(f"random {it}: E={E} R={R} S={S} k={k} T={T} L={L} "
            f"policy={policy} quota_mode={quota_mode}")
        ctx = make_ctx(E, R, S, k, T, L, policy, quota_mode)
        res = gpu_rebalance(ctx, torch.from_numpy(routing))
        compare_with_oracle(res, routing, E, R, S)


@pytest.mark.parametrize("policy,quota_mode", RULES, ids=RULE_IDS)
def test_many_spares_and_ranks(policy, quota_mode):
    """Several spare slots per rank (destinations that take more than one
    chunk and stay eligible), ranks beyond one wave's lanes (R > 64), and
    skew strong enough to exhaust the slots: the planner's held-rank path
    against the oracle."""
    rng = np.random.default_rng(1234 + policy + 2 * quota_mode)
    shapes = [(128, 128, 3), (256, 128, 2), (96, 32, 8), (64, 16, 16),
              (512, 256, 4), (200, 100, 5), (1024, 1024, 1), (1024, 64, 12)]
    for it, (E, R, S) in enumerate(shapes):
        if R * (E // R + S) > 4096:
            continue
        k = int(rng.integers(1, 9))
        T = int(rng.choice([3000, 9000, 20000]))
        L = 2
        routing = np.stack([pins.random_routing(rng, T, E, k,
                                                float(rng.uniform(0.8, 2.5)))
                            for _ in range(L)])
        say(f"spares {it}: E={E} R={R} S={S} k={k} T={T} policy={policy} "
            f"quota_mode={quota_mode}")
        ctx = make_ctx(E, R, S, k, T, L, policy, quota_mode)
        for fused in (False, True):
            res = gpu_rebalance(ctx, torch.from_numpy(routing), fused=fused)
            compare_with_oracle(res, routing, E, R, S)


@pytest.mark.parametrize("policy,quota_mode", RULES, ids=RULE_IDS)
def test_one_spare_slot_up_to_256_ranks(policy, quota_mode):
    """One spare slot per rank, ranks from 1 to 256: the planner's
    one-ballot path up to 64 ranks and its general loop above, with skew
    from none to extreme (plans that run out of slots, best-fit placements
    out of list order, no receiving rank at all), several layers per
    call."""
    rng = np.random.default_rng(777 + policy + 2 * quota_mode)
    for it in range(32):
        R = int(rng.choice([1, 2, 3, 7, 16, 31, 32, 33, 63, 64, 65, 100,
                            128, 129, 200, 256]))
        N = int(rng.integers(1, min(8, 1024 // R) + 1))
        E = R * N
        if E > 1024:
            continue
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([0, 5, 700, 4096, 9001]))
        L = int(rng.integers(1, 4))
        routing = np.stack([pins.random_routing(rng, T, E, k,
                                                float(rng.uniform(0, 3.5)))
                            for _ in range(L)])
        say(f"one slot {it}: E={E} R={R} k={k} T={T} L={L} policy={policy} "
            f"quota_mode={quota_mode}")
        ctx = make_ctx(E, R, 1, k, T, L, policy, quota_mode)
        res = gpu_rebalance(ctx, torch.from_numpy(routing), fused=True)
        compare_with_oracle(res, routing, E, R, 1)


def test_many_layers_ragged_load_groups():
    """130 layers of 63 tiles each, the last one ragged: 130 x 8 load groups
    of 8 tiles, with a partial last group (7 tiles) and a partial last tile
    in every layer."""
    rng = np.random.default_rng(4321)
    E, R, S, k, T, L = 64, 8, 2, 8, 16001, 130
    routing = np.stack([pins.random_routing(rng, T, E, k,
                                            float(rng.uniform(0.5, 2.0)))
                        for _ in range(L)])
    say(f"ragged load groups: E={E} R={R} S={S} k={k} T={T} L={L}")
    ctx = make_ctx(E, R, S, k, T, L)
    for fused in (False, True):
        res = gpu_rebalance(ctx, torch.from_numpy(routing), fused=fused)
        compare_with_oracle(res, routing, E, R, S)


@pytest.mark.parametrize("policy,quota_mode", RULES, ids=RULE_IDS)
@pytest.mark.parametrize("fused", [False, True], ids=["calls", "fused"])
@pytest.mark.parametrize("name", ["tiny", "large_ep", "pipeline", "dsv3"])
def test_configs_full_size(name, fused, policy, quota_mode):
    """Every routing workload at its full size, every layer, bit-exact, as
    three calls and as one ue_rebalance call, under every planner rule."""
    cfg = W.CONFIGS[name]
    say("full size", name, "fused" if fused else "calls", "policy", policy,
        "quota_mode", quota_mode)
    routing = W.make_routing(cfg, device=DEV)
    ctx = make_ctx(cfg.experts, cfg.ranks, cfg.spare, cfg.topk, cfg.tokens,
                   cfg.layers, policy, quota_mode)
    res = gpu_rebalance(ctx, routing, fused=fused)
    compare_with_oracle(res, routing.cpu().numpy(), cfg.experts, cfg.ranks,
                        cfg.spare)


def test_fused_equals_calls_random():
    """ue_rebalance gives the same bits as ue_load + ue_plan + ue_reroute on
    random shapes (ragged tails, k not dividing the tile, repeated calls
    with changing sizes on one context), and matches the oracle."""
    rng = np.random.default_rng(17)
    ctx = make_ctx(96, 8, 2, 8, 9000, 3)
    for it in range(12):
        T = int(rng.choice([0, 1, 100, 4095, 4096, 4097, 9000]))
        L = int(rng.integers(1, 4))
        k = 8
        routing = np.stack([pins.random_routing(rng, T, 96, k,
                                                float(rng.uniform(0, 2.5)))
                            for _ in range(L)])
        say(f"fused vs calls {it}: T={T} L={L}")
        a = gpu_rebalance(ctx, torch.from_numpy(routing), fused=True)
        b = gpu_rebalance(ctx, torch.from_numpy(routing), fused=False)
        for key in ("counts", "invalid", "placement", "phys", "perm",
                    "inv_perm", "rank_counts", "faults"):
            assert np.array_equal(a[key], b[key]), key
        compare_with_oracle(a, routing, 96, 8, 2)


def test_duplicate_expert_in_token():
    """Top-k never repeats an expert within a token, but the path must stay
    exact if a token does (those tiles rank by matching lanes)."""
    rng = np.random.default_rng(21)
    E, R, S, k, T = 64, 8, 2, 8, 5000
    routing = pins.random_routing(rng, T, E, k, 1.2)
    routing[10, 3] = routing[10, 5]
    routing[4500, 0] = routing[4500, 7]
    say("duplicates")
    ctx = make_ctx(E, R, S, k, T)
    for fused in (False, True):
        res = gpu_rebalance(ctx, torch.from_numpy(routing[None]), fused=fused)
        compare_with_oracle(res, routing[None], E, R, S)


@pytest.mark.parametrize("k", [8, 4, 3])
def test_expert_in_every_token(k):
    """One expert in every token: its rank within a tile reaches the tile's
    last token, the largest per-word popcount prefix (one byte per word at
    k = 8, 16 bits at k = 4 and k = 3, which does not divide the tile)."""
    rng = np.random.default_rng(31 + k)
    E, R, S, T = 64, 8, 2, 7000
    routing = np.empty((T, k), np.int32)
    for t in range(T):
        routing[t] = np.concatenate(
            [[5], rng.choice(np.delete(np.arange(E), 5), k - 1, replace=False)])
        rng.shuffle(routing[t])
    say(f"expert in every token: k={k}")
    ctx = make_ctx(E, R, S, k, T)
    for fused in (False, True):
        res = gpu_rebalance(ctx, torch.from_numpy(routing[None]), fused=fused)
        compare_with_oracle(res, routing[None], E, R, S)


def test_kernel_times():
    cfg = W.CONFIGS["tiny"]
    routing = W.make_routing(cfg, device=DEV)
    ctx = make_ctx(cfg.experts, cfg.ranks, cfg.spare, cfg.topk, cfg.tokens)
    say("kernel times")
    with pytest.raises(ue.UEError):
        ue.ue_kernel_times(ctx)
    ue.ue_set_timing(ctx, True)
    ue.ue_rebalance(ctx, routing)
    t = ue.ue_kernel_times(ctx)
    assert len(t) == 3 and all(v > 0 for v in t)
    ue.ue_load(ctx, routing)
    assert len(ue.ue_kernel_times(ctx)) == 2     # count, scan
    ue.ue_set_timing(ctx, False)


def test_invalid_ids_and_faults():
    rng = np.random.default_rng(5)
    E, R, S, k, T = 32, 4, 2, 4, 3000
    routing = pins.random_routing(rng, T, E, k, 1.0)
    routing[0, 0] = -1
    routing[17, 3] = E
    routing[2999, 1] = 12345
    say("invalid ids")
    ctx = make_ctx(E, R, S, k, T)
    res = gpu_rebalance(ctx, torch.from_numpy(routing[None]))
    assert int(res["invalid"][0]) == 3
    assert int(res["faults"][0]) == 3
    compare_with_oracle(res, routing[None], E, R, S)


def test_plan_from_other_counts_faults():
    """A plan made for fewer tokens than routed: the overflow is reported,
    never written out of bounds."""
    rng = np.random.default_rng(6)
    E, R, S, k, T = 16, 4, 1, 2, 500
    routing = torch.from_numpy(pins.random_routing(rng, T, E, k, 1.5)[None])
    half = routing[:, : T // 2].contiguous()
    say("plan from other counts")
    ctx = make_ctx(E, R, S, k, T)
    counts = ue.ue_load(ctx, half.to(DEV))
    pl = ue.ue_plan(ctx, counts)
    out = ue.ue_reroute(ctx, routing.to(DEV), pl)
    torch.cuda.synchronize()
    assert int(out["faults"][0]) == T * k - (T // 2) * k


@pytest.mark.parametrize("E,k", [(256, 8), (512, 8), (256, 7)],
                         ids=["top8_instance", "top8_over_256_experts",
                              "general_instance"])
def test_top8_and_general_reroute_instances(E, k):
    """The reroute has an instance for top-8 routing with at most 256
    experts (constant bitmap shape, one expert per thread) and a general
    one. Each, as three calls and fused: ids out of range, a token that
    repeats an expert (its tile ranks by matching), a ragged last tile;
    then a plan made from the first half of the tokens applied to all of
    them through the standalone reroute, so that assignments past the
    plan's capacities and positions are faults, against the oracle's
    reroute of the oracle's plan of the same half."""
    rng = np.random.default_rng(8000 + E + k)
    R, S, T, L = 64, 1, 9001, 2
    routing = np.stack([pins.random_routing(rng, T, E, k, 1.3)
                        for _ in range(L)])
    routing[0, 17, 2] = E + 3
    routing[1, 4000, 0] = -5
    routing[1, 8999, 1] = routing[1, 8999, 4]
    say(f"reroute instances: E={E} k={k}")
    ctx = make_ctx(E, R, S, k, T, L)
    for fused in (False, True):
        res = gpu_rebalance(ctx, torch.from_numpy(routing), fused=fused)
        compare_with_oracle(res, routing, E, R, S)
    half = np.ascontiguousarray(routing[:, : T // 2])
    counts = ue.ue_load(ctx, torch.from_numpy(half).to(DEV))
    placement = ue.ue_plan(ctx, counts)
    fill = pins.PERM_FILL
    perm = torch.full((L, T * k), fill, dtype=torch.int32, device=DEV)
    out = ue.ue_reroute(ctx, torch.from_numpy(routing).to(DEV), placement,
                        perm=perm)
    torch.cuda.synchronize()
    half_counts, _ = oracle.load(half, E)
    for layer in range(L):
        pl = oracle.plan(half_counts[layer], R, S)
        rr = oracle.reroute(routing[layer].reshape(-1), pl, perm_fill=fill)
        assert rr["faults"] > 0
        assert int(out["faults"][layer]) == rr["faults"], layer
        for key in ("phys", "inv_perm", "rank_counts"):
            assert np.array_equal(out[key][layer].cpu().numpy().reshape(-1),
                                  rr[key].reshape(-1)), (layer, key)
        assert np.array_equal(perm[layer].cpu().numpy(), rr["perm"]), layer


@pytest.mark.parametrize("E,R,k,T", [(250, 25, 8, 70001), (1024, 64, 8, 40001),
                                     (64, 8, 8, 300000)],
                         ids=["E250_35_groups", "E1024_20_groups",
                              "E64_147_groups"])
def test_scan_of_many_load_groups(E, R, k, T):
    """Layers whose load groups are too many for one batch of the scan's
    loads per thread: the scan then takes the experts in pairs (one 32-bit
    load per pair and group), with ragged last groups, threads whose chunk
    is empty, and at E = 1024 two threads per pair; counts, bases (through
    the reroute) and plans against the oracle, standalone and fused."""
    rng = np.random.default_rng(9000 + E)
    S, L = 1, 2
    routing = np.stack([pins.random_routing(rng, T, E, k, 1.1)
                        for _ in range(L)])
    say(f"many load groups: E={E} R={R} k={k} T={T}")
    ctx = make_ctx(E, R, S, k, T, L)
    for fused in (False, True):
        res = gpu_rebalance(ctx, torch.from_numpy(routing), fused=fused)
        compare_with_oracle(res, routing, E, R, S)


def test_deterministic_repeats():
    cfg = W.CONFIGS["large_ep"]
    routing = W.make_routing(cfg, device=DEV)
    ctx = make_ctx(cfg.experts, cfg.ranks, cfg.spare, cfg.topk, cfg.tokens)
    say("repeats large_ep")
    first = gpu_rebalance(ctx, routing)
    for _ in range(10):
        again = gpu_rebalance(ctx, routing)
        for key in ("counts", "placement", "phys", "perm", "inv_perm",
                    "rank_counts"):
            assert np.array_equal(first[key], again[key]), key


def test_batched_equals_single_layers():
    cfg = W.CONFIGS["dsv3"]
    routing = W.make_routing(cfg, device=DEV, layers=8)
    ctx = make_ctx(cfg.experts, cfg.ranks, cfg.spare, cfg.topk, cfg.tokens, 8)
    say("batched vs single dsv3 x8")
    batched = gpu_rebalance(ctx, routing)
    for layer in range(8):
        one = gpu_rebalance(ctx, routing[layer:layer + 1].contiguous())
        for key in ("counts", "placement", "phys", "perm", "inv_perm",
                    "rank_counts"):
            assert np.array_equal(batched[key][layer], one[key][0]), key


def test_refusals_leave_outputs_untouched():
    E, R, S, k, T = 64, 8, 2, 8, 1000
    ctx = make_ctx(E, R, S, k, T, 2)
    routing = torch.zeros((1, T, k), dtype=torch.int32, device=DEV)
    sentinel = torch.full((1, E), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    counts = sentinel.clone()
    lib = ue.library()
    import ctypes
    say("refusals")
    # too many tokens, too many layers, null counts, misaligned pointer
    assert lib.ue_load(ctx._h, ctypes.c_void_p(routing.data_ptr()), 1, T + 1,
                       ctypes.c_void_p(counts.data_ptr()), None,
                       None) == -2
    assert lib.ue_load(ctx._h, ctypes.c_void_p(routing.data_ptr()), 3, T,
                       ctypes.c_void_p(counts.data_ptr()), None, None) == -2
    assert lib.ue_load(ctx._h, ctypes.c_void_p(routing.data_ptr()), 1, T,
                       None, None, None) == -1
    assert lib.ue_load(ctx._h, ctypes.c_void_p(routing.data_ptr() + 2), 1, T,
                       ctypes.c_void_p(counts.data_ptr()), None, None) == -1
    assert "aligned" in ue.ue_last_error(ctx)
    placement = torch.full((1, ctx.placement_words), 77, dtype=torch.int32,
                           device=DEV)
    assert lib.ue_plan(ctx._h, None, 1, ctypes.c_void_p(placement.data_ptr()),
                       None) == -1
    assert lib.ue_plan(ctx._h, ctypes.c_void_p(counts.data_ptr()), 0,
                       ctypes.c_void_p(placement.data_ptr()), None) == -2
    phys = torch.full((1, T, k), 9, dtype=torch.int32, device=DEV)
    assert lib.ue_reroute(ctx._h, ctypes.c_void_p(routing.data_ptr()),
                          ctypes.c_void_p(placement.data_ptr()), 1, T,
                          ctypes.c_void_p(phys.data_ptr()), None, None, None,
                          None, None) == -1
    assert lib.ue_weight_sync(ctx._h, None, None, 1, None) == -6
    torch.cuda.synchronize()
    assert torch.equal(counts, sentinel)
    assert bool((placement == 77).all()) and bool((phys == 9).all())
    # unsupported configurations are refused at creation
    for bad in ((63, 8, 1, 8), (2048, 8, 1, 8), (64, 8, 100, 8), (64, 8, 1, 65)):
        with pytest.raises(ue.UEError):
            ue.Context(*bad, 100, 1, device=DEV)
    with pytest.raises(ue.UEError):
        ue.Context(64, 8, 1, 8, 100, 1, device=DEV, plan_policy=4)
    with pytest.raises(ue.UEError):
        ue.Context(64, 8, 1, 8, 100, 1, device=DEV, quota_mode=2)


def _layer_from_loads(rng, loads):
    """k = 1 routing whose expert e (one per rank) gets loads[e] tokens,
    in random token order."""
    ids = np.repeat(np.arange(len(loads), dtype=np.int32), loads)
    rng.shuffle(ids)
    return ids.reshape(-1, 1)


@pytest.mark.parametrize("policy", [0, 1, 2, 3],
                         ids=["least_loaded", "best_fit", "cover", "ascending"])
@pytest.mark.parametrize("L", [3, 20])
def test_spread_search_late_and_no_quota(policy, L):
    """The quota search with more than 64 ranks, spread over several
    workgroups per layer (16 each for a few layers: 64 quotas at once; 4
    each for up to 64 layers: 16 quotas, then rounds in the last one).
    Layers built so that the first quota that works is step 18 (88 ranks
    just above it, 20 far above, 20 empty), or none of the 64 does (100
    ranks above the highest quota tried, 28 empty: more sources than spare
    slots), or random skew; bit-exact against the oracle."""
    rng = np.random.default_rng(55 + L + 7 * policy)
    R = 128
    late = np.array([1070] * 88 + [1690] * 20 + [0] * 20)
    T = int(late.sum())
    none = np.array([T // 100] * 100 + [0] * 28)
    none[0] += T - int(none.sum())
    layers = []
    for i in range(L):
        kind = i % 3
        if kind == 0:
            loads = rng.permutation(late)
        elif kind == 1:
            loads = rng.permutation(none)
        else:
            r = pins.random_routing(rng, T, R, 1, float(rng.uniform(0.5, 3)))
            loads = np.bincount(r.reshape(-1), minlength=R)
        layers.append(_layer_from_loads(rng, loads))
    routing = np.stack(layers)
    # the cases are what they claim (checked on the oracle first)
    for i in range(min(L, 2)):
        c = np.bincount(routing[i].reshape(-1), minlength=R).astype(np.int32)
        pl = oracle.plan(c, R, 1, policy, 1)
        Q0 = -(-int(c.sum()) // R)
        if i % 3 == 0:
            assert pl["quota"] == Q0 + 18 * (-(-Q0 // 256))
            assert not pl["exhausted"]
        else:
            assert pl["exhausted"] and pl["quota"] == Q0
    say(f"spread search: R={R} L={L} T={T} policy={policy}")
    ctx = make_ctx(R, R, 1, 1, T, L, policy, ue.QUOTA_SEARCH)
    for fused in (True, False):
        res = gpu_rebalance(ctx, torch.from_numpy(routing), fused=fused)
        compare_with_oracle(res, routing, R, R, 1)
