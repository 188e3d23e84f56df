"""Error paths forced from the host, with every kernel still ending
normally: bounded waits of the standalone reroute that give up (a wait
limit of 0) mark their layer poisoned in faults, the calls that do not wait
stay exact, and the context works again afterwards; counts the planner
cannot plan give an empty, marked block whose reroute faults every
assignment."""
import numpy as np
import pytest
import torch

import moe_expert_load_ue_amd as ue
import oracle
from gpu_helpers import compare_with_oracle, gpu_rebalance, say
from moe_expert_load_ue_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_waits_that_give_up_are_reported():
    """ue_reroute's tiles wait on each other (lookback); with a wait limit
    of 0 every wait gives up and every layer of more than one tile is
    marked in faults. ue_load and ue_rebalance wait on nothing, so the same
    limit leaves them exact. Back at the default limit the context works
    as before."""
    cfg = W.CONFIGS["dsv3"]
    routing = W.make_routing(cfg, device=DEV, layers=3)
    ctx = ue.Context(cfg.experts, cfg.ranks, cfg.spare, cfg.topk, cfg.tokens,
                     3, device=DEV)
    say("wait limit 0: three calls")
    ue.ue_set_wait_limit(ctx, 0)
    invalid = torch.zeros(3, dtype=torch.int32, device=DEV)
    counts = ue.ue_load(ctx, routing, invalid=invalid)
    pl = ue.ue_plan(ctx, counts)
    rr = ue.ue_reroute(ctx, routing, pl)
    torch.cuda.synchronize()
    assert not np.any(invalid.cpu().numpy() & ue.POISONED)
    assert np.all(rr["faults"].cpu().numpy() & ue.POISONED)
    say("wait limit 0: fused, which does not wait")
    res = gpu_rebalance(ctx, routing.cpu(), fused=True)
    compare_with_oracle(res, routing.cpu().numpy(), cfg.experts, cfg.ranks,
                        cfg.spare)
    say("default wait limit again: clean and exact")
    ue.ue_set_wait_limit(ctx, 1 << 22)
    for fused in (True, False):
        res = gpu_rebalance(ctx, routing.cpu(), fused=fused)
        assert not np.any(res["invalid"] & ue.POISONED)
        assert not np.any(res["faults"] & ue.POISONED)
        compare_with_oracle(res, routing.cpu().numpy(), cfg.experts,
                            cfg.ranks, cfg.spare)
    ctx.close()


def test_single_group_layer_has_no_wait():
    """A layer of one tile never waits on another workgroup, so even a wait
    limit of 0 leaves it exact."""
    rng = np.random.default_rng(5)
    routing = torch.from_numpy(
        rng.integers(0, 16, size=(1, 300, 2)).astype(np.int32))
    ctx = ue.Context(16, 4, 1, 2, 300, 1, device=DEV)
    ue.ue_set_wait_limit(ctx, 0)
    say("wait limit 0: one tile")
    for fused in (True, False):
        res = gpu_rebalance(ctx, routing, fused=fused)
        compare_with_oracle(res, routing.numpy(), 16, 4, 1)
    ctx.close()


@pytest.mark.parametrize("bad", ["negative", "sum_too_large"])
def test_plan_refuses_counts_it_cannot_plan(bad):
    E, R, S, k, T = 8, 4, 1, 2, 40
    ctx = ue.Context(E, R, S, k, T, 2, device=DEV)
    counts = np.array([[10, 5, 5, 0, 20, 0, 0, 0],
                       [10, 5, 5, 0, 20, 0, 0, 0]], np.int32)
    if bad == "negative":
        counts[1, 3] = -1
    else:
        counts[1, :4] = (1 << 28)
    say("plan refuses", bad)
    pl = ue.ue_plan(ctx, torch.from_numpy(counts).to(DEV))
    f = ctx.placement_fields(pl)
    assert int(f["exhausted"][1]) == -1 and int(f["n_rep"][1]) == 0
    assert f["rep_off"][1].tolist() == [0] * (E + 1)
    assert np.all(f["rep_slot"][1].cpu().numpy() == -1)
    # the good layer is planned as usual
    want = oracle.plan(counts[0], R, S)
    assert int(f["exhausted"][0]) == want["exhausted"]
    assert f["rep_slot"][0].tolist() == want["rep_slot"].tolist()
    # rerouting the bad layer faults every assignment
    routing = torch.from_numpy(
        np.random.default_rng(1).integers(0, E, size=(2, T, k)).astype(np.int32)
    ).to(DEV)
    rr = ue.ue_reroute(ctx, routing, pl)
    torch.cuda.synchronize()
    assert int(rr["faults"][1]) == T * k
    assert np.all(rr["phys"][1].cpu().numpy() == -1)
    ctx.close()
