"""The stale-plan split on the device (ue_stale_loads) against the oracle,
bit-exact, on the two workloads whose numbers the benchmark reports: plans
of the previous microbatch and of the summed earlier microbatches applied
under the pipeline workload's drift, and each dsv3 layer's plan applied one
step later (same distribution, fresh tokens). The oracle computes its own
counts and plans from the same routing; nothing on its side comes from the
device."""
import numpy as np
import pytest
import torch

import moe_expert_load_ue_amd as ue
import oracle
from gpu_helpers import say
from moe_expert_load_ue_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

RULES = [(0, 0), (1, 1), (2, 1), (3, 1)]
RULE_IDS = ["least_loaded", "best_fit_search", "cover_search",
            "ascending_search"]


def oracle_plans(counts, cfg, policy, quota_mode):
    return [oracle.plan(c, cfg.ranks, cfg.spare, policy, quota_mode)
            for c in counts]


@pytest.mark.parametrize("policy,quota_mode", RULES, ids=RULE_IDS)
def test_pipeline_drift(policy, quota_mode):
    cfg = W.CONFIGS["pipeline"]
    say("stale pipeline", policy, quota_mode)
    routing = W.make_routing(cfg, device=DEV)
    ctx = ue.Context(cfg.experts, cfg.ranks, cfg.spare, cfg.topk, cfg.tokens,
                     cfg.layers, device=DEV, plan_policy=policy,
                     quota_mode=quota_mode)
    out = ue.ue_rebalance(ctx, routing)
    counts = out["counts"]
    prev = ue.ue_stale_loads(ctx, out["placement"][:-1].contiguous(),
                             counts[1:].contiguous())
    cum = torch.cumsum(counts, 0, dtype=torch.int32)[:-1].contiguous()
    hist_pl = ue.ue_plan(ctx, cum)
    summed = ue.ue_stale_loads(ctx, hist_pl, counts[1:].contiguous())
    torch.cuda.synchronize()

    r = routing.cpu().numpy()
    want_counts, _ = oracle.load(r, cfg.experts)
    pls = oracle_plans(want_counts, cfg, policy, quota_mode)
    hist = oracle_plans(np.cumsum(want_counts, axis=0, dtype=np.int64)[:-1]
                        .astype(np.int32), cfg, policy, quota_mode)
    prev = prev.cpu().numpy()
    summed = summed.cpu().numpy()
    for m in range(1, cfg.layers):
        want = oracle.stale_loads(pls[m - 1], want_counts[m])
        assert np.array_equal(prev[m - 1], want), f"microbatch {m} previous"
        want = oracle.stale_loads(hist[m - 1], want_counts[m])
        assert np.array_equal(summed[m - 1], want), f"microbatch {m} summed"
    ctx.close()


@pytest.mark.parametrize("policy,quota_mode", RULES, ids=RULE_IDS)
def test_dsv3_next_step(policy, quota_mode):
    cfg = W.CONFIGS["dsv3"]
    say("stale dsv3", policy, quota_mode)
    r0 = W.make_routing(cfg, device=DEV)
    r1 = W.make_routing(cfg, device=DEV, step=1)
    ctx = ue.Context(cfg.experts, cfg.ranks, cfg.spare, cfg.topk, cfg.tokens,
                     cfg.layers, device=DEV, plan_policy=policy,
                     quota_mode=quota_mode)
    old = ue.ue_plan(ctx, ue.ue_load(ctx, r0))
    c1 = ue.ue_load(ctx, r1)
    got = ue.ue_stale_loads(ctx, old, c1).cpu().numpy()
    c0_want, _ = oracle.load(r0.cpu().numpy(), cfg.experts)
    c1_want, _ = oracle.load(r1.cpu().numpy(), cfg.experts)
    for layer in range(cfg.layers):
        pl = oracle.plan(c0_want[layer], cfg.ranks, cfg.spare, policy,
                         quota_mode)
        want = oracle.stale_loads(pl, c1_want[layer])
        assert np.array_equal(got[layer], want), f"layer {layer}"
    ctx.close()


def test_stale_refusals():
    ctx = ue.Context(8, 4, 1, 2, 16, 2, device=DEV)
    pl = ctx.new_placement(2)
    counts = torch.zeros((3, 8), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        ue.ue_stale_loads(ctx, pl, counts)       # 3 layers, 2 blocks
    rc = ue.library().ue_stale_loads(ctx._h, None, None, 1, None, None)
    assert rc == -1                             # UE_EINVAL
    ctx.close()
